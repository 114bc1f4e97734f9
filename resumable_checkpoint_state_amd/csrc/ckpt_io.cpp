// ckpt_io.cpp -- host side of the on-disk step file: atomic write, read,
// newest-valid lookup, rotation, and the SIGTERM / SIGUSR1 flags.
//
// Sources (pages named by title, then section):
//   * grow_a_language_model_checkpoints, "SIGTERM & SIGUSR1": on SIGTERM the
//     engine finishes the current step, writes step_NNNNNN.bin and exits; on
//     SIGUSR1 it finishes the step, writes the file and carries on. Recovery
//     needs only the newest .bin.
//   * Phase 19 lesson 80 (checkpoint-sharded-resume), "atomic write": write
//     to a temporary path, fsync, then rename; a crash before the rename
//     leaves the previous checkpoint intact. Production keeps the last K
//     checkpoints and deletes older ones.
// The handlers only set flags; the training loop polls them after each
// completed update (the resume lesson saves after a complete optimizer step),
// which is also how the polish-pivot sequence lands its checkpoint on a step
// boundary.

#include <dirent.h>
#include <errno.h>
#include <fcntl.h>
#include <signal.h>
#include <stdio.h>
#include <string.h>
#include <sys/stat.h>
#include <sys/types.h>
#include <unistd.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "rcs.h"

namespace {

volatile sig_atomic_t g_sigusr1 = 0;
volatile sig_atomic_t g_sigterm = 0;

void on_signal(int sig) {
    if (sig == SIGUSR1) g_sigusr1 = 1;
    if (sig == SIGTERM) g_sigterm = 1;
}

int32_t le32(const unsigned char *p) {
    uint32_t u = 0;
    for (int k = 0; k < 4; ++k) u |= (uint32_t)p[k] << (8 * k);
    return (int32_t)u;
}

// Header consistency of a whole step file image of `size` bytes.
int check_header(const unsigned char *h, int64_t size, int32_t *step, int32_t *n) {
    if (size < 8) return RCS_ESIZE;
    *step = le32(h);
    *n = le32(h + 4);
    if (*n <= 0 || *step < 0) return RCS_EHEADER;
    if (size != 8 + 12 * (int64_t)*n) return RCS_ESIZE;
    return RCS_OK;
}

std::string step_name(int32_t step) {
    char b[32];
    snprintf(b, sizeof b, "step_%06d.bin", (int)step);
    return b;
}

int write_all(int fd, const unsigned char *p, int64_t len) {
    while (len > 0) {
        const size_t chunk = (size_t)std::min<int64_t>(len, (int64_t)1 << 30);
        const ssize_t k = write(fd, p, chunk);
        if (k < 0) {
            if (errno == EINTR) continue;
            return RCS_EIO;
        }
        p += k;
        len -= k;
    }
    return RCS_OK;
}

int read_all(int fd, unsigned char *p, int64_t len) {
    while (len > 0) {
        const size_t chunk = (size_t)std::min<int64_t>(len, (int64_t)1 << 30);
        const ssize_t k = read(fd, p, chunk);
        if (k < 0) {
            if (errno == EINTR) continue;
            return RCS_EIO;
        }
        if (k == 0) return RCS_ESIZE;
        p += k;
        len -= k;
    }
    return RCS_OK;
}

int copy_path(const std::string &s, char *out, int64_t cap) {
    if (out == nullptr) return RCS_OK;
    if (cap < (int64_t)s.size() + 1) return RCS_EINVAL;
    memcpy(out, s.c_str(), s.size() + 1);
    return RCS_OK;
}

// Reads the header of a file and checks it against the file's size.
int probe_file(const std::string &path, int32_t *step, int32_t *n) {
    struct stat st;
    if (stat(path.c_str(), &st) != 0 || !S_ISREG(st.st_mode)) return RCS_ENOENT;
    const int fd = open(path.c_str(), O_RDONLY | O_CLOEXEC);
    if (fd < 0) return RCS_EIO;
    unsigned char h[8];
    const int rc = read_all(fd, h, st.st_size < 8 ? st.st_size : 8);
    close(fd);
    if (rc != RCS_OK) return rc;
    return check_header(h, st.st_size, step, n);
}

struct Found {
    int32_t step;
    std::string name;
};

// Valid step files in dir (name step_<digits>.bin, header consistent with the
// size, header step equal to the step in the name), newest first.
std::vector<Found> list_valid(const std::string &dir) {
    std::vector<Found> out;
    DIR *d = opendir(dir.c_str());
    if (!d) return out;
    while (dirent *e = readdir(d)) {
        const std::string nm = e->d_name;
        if (nm.size() < 10 || nm.compare(0, 5, "step_") != 0 ||
            nm.compare(nm.size() - 4, 4, ".bin") != 0)
            continue;
        const std::string digits = nm.substr(5, nm.size() - 9);
        if (digits.empty() || digits.size() > 10 ||
            digits.find_first_not_of("0123456789") != std::string::npos)
            continue;
        int32_t step = 0, n = 0;
        if (probe_file(dir + "/" + nm, &step, &n) != RCS_OK) continue;
        if (std::to_string(step) != std::to_string(std::stoll(digits))) continue;
        out.push_back({step, nm});
    }
    closedir(d);
    std::sort(out.begin(), out.end(), [](const Found &a, const Found &b) { return a.step > b.step; });
    return out;
}

// <path>.tmp, fsync, rename to <path>, fsync the directory.
int atomic_write(const std::string &final_path, const unsigned char *b, int64_t len) {
    const std::string tmp_path = final_path + ".tmp";
    const int fd = open(tmp_path.c_str(), O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644);
    if (fd < 0) return RCS_EIO;
    int rc = write_all(fd, b, len);
    if (rc == RCS_OK && fsync(fd) != 0) rc = RCS_EIO;
    if (close(fd) != 0 && rc == RCS_OK) rc = RCS_EIO;
    if (rc != RCS_OK) {
        unlink(tmp_path.c_str());
        return rc;
    }
    if (rename(tmp_path.c_str(), final_path.c_str()) != 0) {
        unlink(tmp_path.c_str());
        return RCS_EIO;
    }
    const size_t slash = final_path.find_last_of('/');
    const std::string d = slash == std::string::npos ? "." : final_path.substr(0, slash + 1);
    const int dfd = open(d.c_str(), O_RDONLY | O_DIRECTORY | O_CLOEXEC);
    if (dfd >= 0) {
        (void)fsync(dfd);  // make the rename itself durable
        close(dfd);
    }
    return RCS_OK;
}

}  // namespace

extern "C" {

int ckpt_file_write(const char *dir, const void *host_buf, int64_t buf_bytes, char *path_out,
                    int64_t path_cap) {
    if (dir == nullptr || host_buf == nullptr) return RCS_EINVAL;
    const unsigned char *b = static_cast<const unsigned char *>(host_buf);
    int32_t step = 0, n = 0;
    int rc = check_header(b, buf_bytes, &step, &n);
    if (rc != RCS_OK) return rc;
    const std::string final_path = std::string(dir) + "/" + step_name(step);
    // a path_out too small for the path is refused before anything is written
    if (path_out != nullptr && path_cap < (int64_t)final_path.size() + 1) return RCS_EINVAL;
    if ((rc = atomic_write(final_path, b, buf_bytes)) != RCS_OK) return rc;
    return copy_path(final_path, path_out, path_cap);
}

int ckpt_file_write_path(const char *path, const void *host_buf, int64_t buf_bytes) {
    if (path == nullptr || host_buf == nullptr) return RCS_EINVAL;
    const unsigned char *b = static_cast<const unsigned char *>(host_buf);
    int32_t step = 0, n = 0;
    const int rc = check_header(b, buf_bytes, &step, &n);
    if (rc != RCS_OK) return rc;
    return atomic_write(path, b, buf_bytes);
}

int rcs_file_write_atomic(const char *path, const void *data, int64_t len) {
    if (path == nullptr || (data == nullptr && len > 0) || len < 0) return RCS_EINVAL;
    return atomic_write(path, static_cast<const unsigned char *>(data), len);
}

int64_t ckpt_file_size(const char *path) {
    if (path == nullptr) return RCS_EINVAL;
    struct stat st;
    if (stat(path, &st) != 0 || !S_ISREG(st.st_mode)) return RCS_ENOENT;
    return (int64_t)st.st_size;
}

int ckpt_file_read(const char *path, void *host_buf, int64_t buf_bytes) {
    if (path == nullptr || host_buf == nullptr) return RCS_EINVAL;
    const int64_t size = ckpt_file_size(path);
    if (size < 0) return (int)size;
    if (size != buf_bytes) return RCS_ESIZE;
    const int fd = open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return RCS_EIO;
    unsigned char *b = static_cast<unsigned char *>(host_buf);
    int rc = read_all(fd, b, buf_bytes);
    close(fd);
    if (rc != RCS_OK) return rc;
    int32_t step = 0, n = 0;
    return check_header(b, buf_bytes, &step, &n);
}

int ckpt_file_latest(const char *dir, int32_t *step_out, char *path_out, int64_t path_cap) {
    if (dir == nullptr || step_out == nullptr) return RCS_EINVAL;
    const std::vector<Found> v = list_valid(dir);
    if (v.empty()) return RCS_ENOENT;
    const int rc = copy_path(std::string(dir) + "/" + v[0].name, path_out, path_cap);
    if (rc != RCS_OK) return rc;
    *step_out = v[0].step;
    return RCS_OK;
}

int ckpt_file_rotate(const char *dir, int keep) {
    if (dir == nullptr || keep < 1) return RCS_EINVAL;
    const std::string d = dir;
    const std::vector<Found> v = list_valid(d);
    int removed = 0;
    for (size_t i = (size_t)keep; i < v.size(); ++i)
        if (unlink((d + "/" + v[i].name).c_str()) == 0) ++removed;
    // leftovers of interrupted writes
    if (DIR *dd = opendir(d.c_str())) {
        std::vector<std::string> tmps;
        while (dirent *e = readdir(dd)) {
            const std::string nm = e->d_name;
            if (nm.compare(0, 5, "step_") == 0 && nm.size() > 8 &&
                nm.compare(nm.size() - 8, 8, ".bin.tmp") == 0)
                tmps.push_back(nm);
        }
        closedir(dd);
        for (const auto &nm : tmps)
            if (unlink((d + "/" + nm).c_str()) == 0) ++removed;
    }
    return removed;
}

int rcs_signals_install(void) {
    struct sigaction sa;
    memset(&sa, 0, sizeof sa);
    sa.sa_handler = on_signal;
    sigemptyset(&sa.sa_mask);
    sa.sa_flags = SA_RESTART;
    if (sigaction(SIGTERM, &sa, nullptr) != 0 || sigaction(SIGUSR1, &sa, nullptr) != 0)
        return RCS_EINVAL;
    return RCS_OK;
}

int rcs_signals_poll(void) {
    int r = 0;
    if (g_sigusr1) {
        g_sigusr1 = 0;
        r |= RCS_SIG_WRITE_CONTINUE;
    }
    if (g_sigterm) {
        g_sigterm = 0;
        r |= RCS_SIG_WRITE_EXIT;
    }
    return r;
}

}  // extern "C"

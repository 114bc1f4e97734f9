// Host-only driver of ckpt_io.cpp, built with AddressSanitizer and UBSan by
// the test suite (no device code is involved): atomic write, read, newest
// lookup over malformed files, rotation, signal flags.
#include <signal.h>
#include <stdio.h>
#include <string.h>
#include <unistd.h>

#include <string>
#include <vector>

#include "rcs.h"

#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            return 1;                                                 \
        }                                                             \
    } while (0)

static std::vector<unsigned char> packed(int32_t step, int32_t n) {
    std::vector<unsigned char> b(8 + 12 * (size_t)n);
    for (int k = 0; k < 4; ++k) {
        b[k] = (unsigned char)((uint32_t)step >> (8 * k));
        b[4 + k] = (unsigned char)((uint32_t)n >> (8 * k));
    }
    for (size_t i = 8; i < b.size(); ++i) b[i] = (unsigned char)(i * 31u);
    return b;
}

int main(int argc, char **argv) {
    if (argc != 2) return 2;
    const std::string d = argv[1];
    char path[4096];
    for (int s : {10, 20, 30, 40}) {
        auto b = packed(s, 100 + s);
        EXPECT(ckpt_file_write(d.c_str(), b.data(), (int64_t)b.size(), path, sizeof path) == RCS_OK);
    }
    char small[8];
    auto b = packed(50, 7);
    EXPECT(ckpt_file_write(d.c_str(), b.data(), (int64_t)b.size(), small, sizeof small) ==
           RCS_EINVAL);  // path does not fit: refused before anything is written
    EXPECT(ckpt_file_size((d + "/step_000050.bin").c_str()) == RCS_ENOENT);
    EXPECT(ckpt_file_write(d.c_str(), b.data(), (int64_t)b.size(), nullptr, 0) == RCS_OK);
    b.pop_back();
    EXPECT(ckpt_file_write(d.c_str(), b.data(), (int64_t)b.size(), nullptr, 0) == RCS_ESIZE);
    FILE *f = fopen((d + "/step_000060.bin").c_str(), "wb");  // truncated newer file
    EXPECT(f != nullptr);
    fwrite(b.data(), 1, 20, f);
    fclose(f);
    f = fopen((d + "/step_000070.bin.tmp").c_str(), "wb");
    fwrite(b.data(), 1, b.size(), f);
    fclose(f);
    int32_t step = -1;
    EXPECT(ckpt_file_latest(d.c_str(), &step, path, sizeof path) == RCS_OK);
    EXPECT(step == 50);
    const int64_t sz = ckpt_file_size(path);
    EXPECT(sz == 8 + 12 * 7);
    std::vector<unsigned char> back((size_t)sz);
    EXPECT(ckpt_file_read(path, back.data(), sz) == RCS_OK);
    EXPECT(ckpt_file_read(path, back.data(), sz - 1) == RCS_ESIZE);
    EXPECT(ckpt_file_rotate(d.c_str(), 2) == 4);  // 10, 20, 30 and the .tmp
    EXPECT(ckpt_file_latest(d.c_str(), &step, nullptr, 0) == RCS_OK && step == 50);
    const char msg[] = "{\"manifest\": 1}";
    EXPECT(rcs_file_write_atomic((d + "/manifest.json").c_str(), msg, sizeof msg - 1) == RCS_OK);
    EXPECT(rcs_signals_install() == RCS_OK);
    raise(SIGUSR1);
    raise(SIGTERM);
    EXPECT(rcs_signals_poll() == (RCS_SIG_WRITE_CONTINUE | RCS_SIG_WRITE_EXIT));
    EXPECT(rcs_signals_poll() == 0);
    printf("ckpt_io driver ok\n");
    return 0;
}

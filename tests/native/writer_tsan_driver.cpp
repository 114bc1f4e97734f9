// Host-only driver for csrc/ckpt_writer.cpp under ThreadSanitizer: the
// writer's worker thread, its mutex and condition variable, and concurrent
// submit / wait calls, with the device side replaced by plain host stand-ins
// (no GPU, no HIP runtime linked). The stand-ins keep the contract the writer
// relies on: ckpt_pack_async takes the state at the call (after the previous
// copy out of the same snapshot has landed, as the library orders its snapshot
// kernel on the device) and lands it in the host buffer later, on another
// thread; ckpt_pack_wait blocks until the newest such copy has landed.
// The file side is the real csrc/ckpt_io.cpp.
//
// usage: writer_tsan_driver DIR     prints "writer tsan driver ok" on success
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "rcs.h"
#include "rcs_internal.h"

// ---------------------------------------------------------------- HIP stand-ins
extern "C" {
hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipMalloc(void **p, size_t n) {
    *p = std::malloc(n);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *p) {
    std::free(p);
    return hipSuccess;
}
hipError_t hipHostMalloc(void **p, size_t n, unsigned int) { return hipMalloc(p, n); }
hipError_t hipHostFree(void *p) { return hipFree(p); }
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned int) {
    static int dummy;
    *s = reinterpret_cast<hipStream_t>(&dummy);
    return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
}

// ---------------------------------------------------------------- pack stand-ins
namespace {
// One "copy" out of a snapshot: a thread that lands the payload later, and a
// flag set when it has.
struct CopyDone {
    std::mutex mu;
    std::condition_variable cv;
    bool done = false;
};
struct SnapState {
    std::vector<std::thread> threads;
    std::shared_ptr<CopyDone> last;  // the newest copy out of the snapshot
};
std::mutex g_mu;
std::map<const void *, SnapState> g_snaps;

void wait_done(const std::shared_ptr<CopyDone> &d) {
    if (!d) return;
    std::unique_lock<std::mutex> lk(d->mu);
    d->cv.wait(lk, [&] { return d->done; });
}

void put_le32(unsigned char *p, int32_t x) {
    const uint32_t u = (uint32_t)x;
    for (int k = 0; k < 4; ++k) p[k] = (unsigned char)(u >> (8 * k));
}
}  // namespace

void rcs_snapshot_forget(int, const void *snapshot) {
    std::vector<std::thread> ts;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_snaps.find(snapshot);
        if (it == g_snaps.end()) return;
        ts.swap(it->second.threads);
        g_snaps.erase(it);
    }
    for (auto &t : ts) t.join();
}

extern "C" {
int64_t ckpt_bytes(int64_t n) { return n >= 1 && n <= RCS_MAX_N ? 8 + 12 * n : -1; }
int64_t ckpt_snapshot_bytes(int64_t n) { return n >= 1 && n <= RCS_MAX_N ? 12 * n : -1; }

int ckpt_pack_async(int32_t step, int64_t n, const float *w, const float *m, const float *v,
                    float *snapshot, int64_t snapshot_bytes, void *host_buf, int64_t buf_bytes,
                    hipStream_t, hipStream_t) {
    if (snapshot_bytes != 12 * n || buf_bytes != 8 + 12 * n) return RCS_ESIZE;
    std::shared_ptr<CopyDone> prev;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        prev = g_snaps[snapshot].last;
    }
    // the library orders the snapshot kernel after the previous copy out of it
    wait_done(prev);
    // the "snapshot kernel": the state at the call
    std::memcpy(snapshot, w, 4 * n);
    std::memcpy(snapshot + n, m, 4 * n);
    std::memcpy(snapshot + 2 * n, v, 4 * n);
    unsigned char *b = static_cast<unsigned char *>(host_buf);
    put_le32(b, step);
    put_le32(b + 4, (int32_t)n);
    // the "copy stream": lands the payload a little later, on another thread
    auto d = std::make_shared<CopyDone>();
    std::thread copy([=] {
        std::this_thread::sleep_for(std::chrono::milliseconds(2));
        std::memcpy(b + 8, snapshot, 12 * n);
        {
            std::lock_guard<std::mutex> lk(d->mu);
            d->done = true;
        }
        d->cv.notify_all();
    });
    std::lock_guard<std::mutex> lk(g_mu);
    SnapState &st = g_snaps[snapshot];
    st.threads.push_back(std::move(copy));
    st.last = d;
    return RCS_OK;
}

// Blocks until the newest copy out of the snapshot has landed.
int ckpt_pack_wait(const float *snapshot) {
    std::shared_ptr<CopyDone> d;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_snaps.find(snapshot);
        if (it == g_snaps.end()) return RCS_OK;
        d = it->second.last;
    }
    wait_done(d);
    return RCS_OK;
}
}

// ---------------------------------------------------------------- driver
#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c); \
            return 1;                                                 \
        }                                                             \
    } while (0)

static std::vector<unsigned char> read_file(const std::string &p) {
    std::vector<unsigned char> out;
    FILE *f = std::fopen(p.c_str(), "rb");
    if (!f) return out;
    unsigned char buf[4096];
    size_t k;
    while ((k = std::fread(buf, 1, sizeof buf, f)) > 0) out.insert(out.end(), buf, buf + k);
    std::fclose(f);
    return out;
}

int main(int argc, char **argv) {
    CHECK(argc == 2);
    const std::string dir = argv[1];
    const int64_t n = 1000;
    std::vector<float> w(n), m(n), v(n);
    rcs_ckpt_writer *wr = nullptr;
    CHECK(rcs_ckpt_writer_create(dir.c_str(), n, 2, &wr) == RCS_OK);

    // a second thread waits while the first submits
    std::atomic<bool> done{false};
    std::atomic<int> waited{0};
    std::thread waiter([&] {
        char path[4096];
        while (!done.load()) {
            if (rcs_ckpt_writer_wait(wr, path, sizeof path) == RCS_OK) waited++;
            std::this_thread::yield();
        }
    });
    std::vector<std::vector<unsigned char>> expect(22);
    for (int step = 1; step <= 21; ++step) {
        if (step == 21) {  // the concurrent waiter has stopped
            done = true;
            waiter.join();
        }
        for (int64_t i = 0; i < n; ++i) {
            w[i] = (float)(step * 1000 + i);
            m[i] = (float)(step + 0.5 * i);
            v[i] = (float)(step * 0.25 + i);
        }
        std::vector<unsigned char> e(8 + 12 * n);
        put_le32(e.data(), step);
        put_le32(e.data() + 4, (int32_t)n);
        std::memcpy(e.data() + 8, w.data(), 4 * n);
        std::memcpy(e.data() + 8 + 4 * n, m.data(), 4 * n);
        std::memcpy(e.data() + 8 + 8 * n, v.data(), 4 * n);
        expect[step] = e;
        CHECK(rcs_ckpt_writer_submit(wr, step, w.data(), m.data(), v.data(), nullptr) == RCS_OK);
        // the caller may change the state at once; the file must hold the state at submit
        for (int64_t i = 0; i < n; ++i) w[i] = -1.0f;
    }
    // a path buffer too small for the path reports nothing; the next wait does
    char path[4096], small[4];
    CHECK(rcs_ckpt_writer_wait(wr, small, sizeof small) == RCS_EINVAL);
    CHECK(rcs_ckpt_writer_wait(wr, path, sizeof path) == RCS_OK);
    CHECK(std::strstr(path, "step_000021.bin") != nullptr);
    CHECK(rcs_ckpt_writer_wait(wr, path, sizeof path) == RCS_OK && path[0] == '\0');
    CHECK(rcs_ckpt_writer_destroy(wr) == RCS_OK);
    for (int step = 20; step <= 21; ++step) {
        char name[64];
        std::snprintf(name, sizeof name, "/step_%06d.bin", step);
        CHECK(read_file(dir + name) == expect[step]);
    }
    char old[64];
    std::snprintf(old, sizeof old, "/step_%06d.bin", 19);
    CHECK(read_file(dir + old).empty());  // rotated away (keep = 2)

    // a failed write is reported by wait
    CHECK(rcs_ckpt_writer_create((dir + "/missing").c_str(), n, 1, &wr) == RCS_OK);
    CHECK(rcs_ckpt_writer_submit(wr, 1, w.data(), m.data(), v.data(), nullptr) == RCS_OK);
    CHECK(rcs_ckpt_writer_wait(wr, path, sizeof path) == RCS_EIO);
    CHECK(rcs_ckpt_writer_wait(wr, path, sizeof path) == RCS_OK && path[0] == '\0');
    CHECK(rcs_ckpt_writer_destroy(wr) == RCS_OK);
    std::printf("writer tsan driver ok (%d concurrent waits returned)\n", waited.load());
    return 0;
}

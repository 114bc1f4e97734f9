// ckpt_writer.cpp -- asynchronous step-file writer: device snapshot, copy to
// pinned host memory on its own stream, atomic file write and rotation on a
// worker thread, so the training stream and the training loop run on during
// both the host-link copy and the disk write.
//
// Sources (pages named by title, then section):
//   * Phase 19 lesson 80 (checkpoint-sharded-resume), production patterns:
//     write the checkpoint asynchronously so training does not stall, write it
//     atomically (temporary file, fsync, rename), keep the newest K.
//   * grow_a_language_model_checkpoints, "SIGTERM & SIGUSR1": a save requested
//     by a signal lands on a completed step; on SIGTERM the caller waits for
//     the write before exiting (rcs_ckpt_writer_wait).
//
// One job at a time: a submit first waits for the previous write to finish,
// because the snapshot and the host buffer are reused.

#include <hip/hip_runtime_api.h>

#include <condition_variable>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <thread>

#include "rcs.h"
#include "rcs_internal.h"

struct rcs_ckpt_writer {
    std::string dir;
    int64_t n = 0;
    int keep = 1;
    int device = 0;
    float *snapshot = nullptr;      // device, 12 n bytes
    unsigned char *host = nullptr;  // pinned, 8 + 12 n bytes
    hipStream_t copy = nullptr;

    std::mutex submit_mu;  // one submit at a time
    std::mutex mu;         // guards the job state below
    std::condition_variable cv;
    bool pending = false;  // a job is queued or running
    bool stop = false;
    int status = RCS_OK;   // of the last finished job, until rcs_ckpt_writer_wait reports it
    std::string path;      // file written by the last finished job
    std::thread worker;

    void run() {
        (void)hipSetDevice(device);
        std::unique_lock<std::mutex> lk(mu);
        for (;;) {
            cv.wait(lk, [this] { return pending || stop; });
            if (!pending) return;  // stop with nothing queued
            lk.unlock();
            char out[4096];
            out[0] = '\0';
            int rc = ckpt_pack_wait(snapshot);
            if (rc == RCS_OK) rc = ckpt_file_write(dir.c_str(), host, ckpt_bytes(n), out, sizeof out);
            if (rc == RCS_OK) {
                const int removed = ckpt_file_rotate(dir.c_str(), keep);
                if (removed < 0) rc = removed;
            }
            lk.lock();
            status = rc;
            path = out;
            pending = false;
            cv.notify_all();
        }
    }
};

namespace {

void release(rcs_ckpt_writer *wr) {
    if (wr->snapshot) {
        rcs_snapshot_forget(wr->device, wr->snapshot);
        (void)hipFree(wr->snapshot);
    }
    if (wr->host) (void)hipHostFree(wr->host);
    if (wr->copy) (void)hipStreamDestroy(wr->copy);
    delete wr;
}

}  // namespace

extern "C" {

int rcs_ckpt_writer_create(const char *dir, int64_t n, int keep, rcs_ckpt_writer **out) {
    if (dir == nullptr || out == nullptr || keep < 1 || ckpt_bytes(n) < 0) return RCS_EINVAL;
    *out = nullptr;
    rcs_ckpt_writer *wr = new (std::nothrow) rcs_ckpt_writer;
    if (wr == nullptr) return RCS_ENOMEM;
    wr->dir = dir;
    wr->n = n;
    wr->keep = keep;
    if (hipGetDevice(&wr->device) != hipSuccess) {
        release(wr);
        return RCS_EHIP;
    }
    if (hipMalloc(&wr->snapshot, (size_t)ckpt_snapshot_bytes(n)) != hipSuccess ||
        hipHostMalloc(&wr->host, (size_t)ckpt_bytes(n), hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        release(wr);
        return RCS_ENOMEM;
    }
    if (hipStreamCreateWithFlags(&wr->copy, hipStreamNonBlocking) != hipSuccess) {
        (void)hipGetLastError();
        release(wr);
        return RCS_EHIP;
    }
    try {
        wr->worker = std::thread([wr] { wr->run(); });
    } catch (...) {
        release(wr);
        return RCS_ENOMEM;
    }
    *out = wr;
    return RCS_OK;
}

int rcs_ckpt_writer_submit(rcs_ckpt_writer *wr, int32_t step, const float *w, const float *m,
                           const float *v, hipStream_t compute_stream) {
    if (wr == nullptr) return RCS_EINVAL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != wr->device) return RCS_EINVAL;
    std::lock_guard<std::mutex> one(wr->submit_mu);
    {
        std::unique_lock<std::mutex> lk(wr->mu);
        wr->cv.wait(lk, [wr] { return !wr->pending; });
        if (wr->status != RCS_OK) {  // the previous write failed: report it first
            const int rc = wr->status;
            wr->status = RCS_OK;
            return rc;
        }
    }
    const int rc = ckpt_pack_async(step, wr->n, w, m, v, wr->snapshot, ckpt_snapshot_bytes(wr->n),
                                   wr->host, ckpt_bytes(wr->n), compute_stream, wr->copy);
    if (rc != RCS_OK) return rc;
    {
        std::lock_guard<std::mutex> lk(wr->mu);
        wr->pending = true;
        wr->path.clear();
    }
    wr->cv.notify_all();
    return RCS_OK;
}

int rcs_ckpt_writer_wait(rcs_ckpt_writer *wr, char *path_out, int64_t path_cap) {
    if (wr == nullptr) return RCS_EINVAL;
    std::unique_lock<std::mutex> lk(wr->mu);
    wr->cv.wait(lk, [wr] { return !wr->pending; });
    // a path_out too small for the path reports nothing and leaves both pending
    if (path_out != nullptr && path_cap < (int64_t)wr->path.size() + 1) return RCS_EINVAL;
    const int rc = wr->status;
    wr->status = RCS_OK;
    std::string path;
    path.swap(wr->path);  // reported once, like the status
    if (path_out != nullptr) memcpy(path_out, path.c_str(), path.size() + 1);
    return rc;
}

int rcs_ckpt_writer_destroy(rcs_ckpt_writer *wr) {
    if (wr == nullptr) return RCS_OK;
    int rc;
    {
        std::unique_lock<std::mutex> lk(wr->mu);
        wr->cv.wait(lk, [wr] { return !wr->pending; });
        rc = wr->status;
        wr->stop = true;
    }
    wr->cv.notify_all();
    wr->worker.join();
    release(wr);
    return rc;
}

}  // extern "C"

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
// Two pinned host images: a submit copies into one while the worker may still
// be writing the other to disk, so a submit waits only while the image it is
// about to reuse is still being written (the save two submits back); the
// device snapshot is shared, and the library's asynchronous pack orders each
// new snapshot after the previous copy out of it, on the device.

#include <hip/hip_runtime_api.h>

#include <condition_variable>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>
#include <string>
#include <thread>

#include "rcs.h"
#include "rcs_internal.h"

struct rcs_ckpt_writer {
    static constexpr int kSlots = 2;
    std::string dir;
    int64_t n = 0;
    int keep = 1;
    int device = 0;
    float *snapshot = nullptr;               // device, 12 n bytes
    unsigned char *host[kSlots] = {};        // pinned, 8 + 12 n bytes each
    hipStream_t copy = nullptr;

    std::mutex submit_mu;  // one submit at a time
    std::mutex mu;         // guards the job state below
    std::condition_variable cv;
    bool busy[kSlots] = {};  // a copy into this image or its file write is under way
    std::deque<int> queue;   // images waiting for (or in) their file write, in submit order
    int next = 0;            // the image the next submit uses
    bool stop = false;
    int status = RCS_OK;   // first failure not yet reported by submit or wait
    std::string path;      // file written by the last finished job
    std::thread worker;

    bool idle() const { return queue.empty(); }

    void run() {
        (void)hipSetDevice(device);
        std::unique_lock<std::mutex> lk(mu);
        for (;;) {
            cv.wait(lk, [this] { return !queue.empty() || stop; });
            if (queue.empty()) return;  // stop with nothing queued
            const int slot = queue.front();
            lk.unlock();
            char out[4096];
            out[0] = '\0';
            // waits for the newest copy out of the snapshot; copies run in
            // submit order on the one copy stream, so this image's has landed
            int rc = ckpt_pack_wait(snapshot);
            if (rc == RCS_OK)
                rc = ckpt_file_write(dir.c_str(), host[slot], ckpt_bytes(n), out, sizeof out);
            if (rc == RCS_OK) {
                const int removed = ckpt_file_rotate(dir.c_str(), keep);
                if (removed < 0) rc = removed;
            }
            lk.lock();
            if (rc != RCS_OK && status == RCS_OK) status = rc;
            if (rc == RCS_OK) path = out;
            busy[slot] = false;
            queue.pop_front();
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
    for (unsigned char *h : wr->host)
        if (h) (void)hipHostFree(h);
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
    bool ok = hipMalloc(&wr->snapshot, (size_t)ckpt_snapshot_bytes(n)) == hipSuccess;
    for (int k = 0; ok && k < rcs_ckpt_writer::kSlots; ++k)
        ok = hipHostMalloc(reinterpret_cast<void **>(&wr->host[k]), (size_t)ckpt_bytes(n),
                           hipHostMallocDefault) == hipSuccess;
    if (!ok) {
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
    int slot;
    {
        std::unique_lock<std::mutex> lk(wr->mu);
        slot = wr->next;
        wr->cv.wait(lk, [wr, slot] { return !wr->busy[slot]; });
        if (wr->status != RCS_OK) {  // an earlier write failed: report it first
            const int rc = wr->status;
            wr->status = RCS_OK;
            return rc;
        }
        wr->busy[slot] = true;  // no worker touches a free image
    }
    const int rc = ckpt_pack_async(step, wr->n, w, m, v, wr->snapshot, ckpt_snapshot_bytes(wr->n),
                                   wr->host[slot], ckpt_bytes(wr->n), compute_stream, wr->copy);
    {
        std::lock_guard<std::mutex> lk(wr->mu);
        if (rc != RCS_OK) {
            wr->busy[slot] = false;
            return rc;
        }
        wr->queue.push_back(slot);
        wr->next = (slot + 1) % rcs_ckpt_writer::kSlots;
    }
    wr->cv.notify_all();
    return RCS_OK;
}

int rcs_ckpt_writer_wait(rcs_ckpt_writer *wr, char *path_out, int64_t path_cap) {
    if (wr == nullptr) return RCS_EINVAL;
    std::unique_lock<std::mutex> lk(wr->mu);
    wr->cv.wait(lk, [wr] { return wr->idle(); });
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
        wr->cv.wait(lk, [wr] { return wr->idle(); });
        rc = wr->status;
        wr->stop = true;
    }
    wr->cv.notify_all();
    wr->worker.join();
    release(wr);
    return rc;
}

}  // extern "C"

/*
 * rcs.h -- C ABI of the MI355X (gfx950) library for one clipped AdamW update
 * over a flat float32 parameter vector and for the step_NNNNNN.bin state.
 *
 * All entry points are extern "C", take plain pointers and sizes, and only
 * enqueue work on the given HIP stream (0 = the null stream of the current
 * device). Every array argument is caller-owned; the library never frees or
 * retains it. Device pointers and the stream must belong to the current
 * device. Results are valid once the stream reaches the enqueued work; the
 * caller must not touch the arrays or host buffers before then.
 *
 * The only device memory the library owns is a per-(device, stream)
 * workspace of about 2.3 KiB (256 per-block float64 partial sums and the clip
 * scalars). It is allocated by rcs_init or on the first call that needs it,
 * never inside a later call, and lives until the process ends. Under
 * hipStreamPerThread, which is a different stream in every host thread, each
 * calling thread gets its own workspace (rcs_init from that thread). (The
 * asynchronous pack also keeps two HIP events per snapshot buffer, and the
 * instrumentation its events while enabled. An rcs_ckpt_writer, created and
 * destroyed explicitly, owns its snapshot, host buffer, stream and thread.)
 *
 * Every call validates its arguments on the host before enqueuing anything and
 * returns one of the status codes below; a negative return means nothing was
 * enqueued (except RCS_EHIP, which reports a failed launch or copy).
 *
 * What the device-array checks can see: each array must be device (or
 * managed) memory of the current device, and [p, p + 4 n) must lie inside the
 * allocation the runtime reports for p (RCS_ESIZE otherwise). That is the
 * allocation as the HIP runtime made it: a caller's sub-allocator (PyTorch's
 * caching allocator, an arena) carves many arrays out of one allocation, and an
 * array too short for n that still ends inside that allocation cannot be told
 * from a long enough one, so the call would read and write past it. Memory for
 * which the runtime reports no range (e.g. some virtual-memory mappings) is
 * accepted without the length check. Callers that carve arrays out of larger
 * blocks must pass the true n.
 */
#ifndef RCS_H
#define RCS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum rcs_status {
    RCS_OK = 0,
    RCS_EINVAL = -1,  /* null pointer, bad size, bad scalar, not device memory */
    RCS_ESIZE = -2,   /* buffer length differs from 8 + 12 n, or an array is too short */
    RCS_EHEADER = -3, /* step file header inconsistent (n <= 0, step < 0, n mismatch) */
    RCS_EHIP = -4,    /* a HIP launch, copy or allocation failed */
    RCS_ENOMEM = -5,  /* workspace allocation failed */
    RCS_EIO = -6,     /* a file could not be written, read or renamed */
    RCS_ENOENT = -7   /* no such file, or no valid step file in the directory */
};

/* Largest n the step file's int32 header can describe. */
#define RCS_MAX_N 2147483647LL

/* Human-readable text for a status code (static storage). */
const char *rcs_strerror(int status);

/* Allocates the workspace of (device, stream) ahead of time so that no later
 * call allocates, and looks up the device's copy of the static array that
 * adamw_clip_step_noalloc uses. Optional; needed before capturing
 * adamw_clip_step (or the norm and clip calls) on that stream into a graph:
 * the capture then holds only the kernels, with t and the hyper-parameters
 * fixed at capture. */
int rcs_init(int device, hipStream_t stream);

/*
 * One training update: global L2 gradient-norm clip, then decoupled-weight-
 * decay AdamW with bias correction, in place on w, m, v.
 *
 * Follows "Training as a Recoverable State Transition", section "The Exact
 * Targets of Clipping and AdamW": g is one vector; if ||g||_2 > clip it is
 * scaled by clip/||g||, otherwise left alone; beta1 = 0.9, beta2 = 0.999,
 * eps = 1e-8, m_hat = m/(1-beta1^t), v_hat = v/(1-beta2^t); parameters are
 * first multiplied by (1 - lr*wd), then lr*m_hat/(sqrt(v_hat)+eps) is
 * subtracted; decay applies to every element. The three-kernel clip split
 * (per-block partial sums, one final reduction, one scale) is the one the
 * backprop lesson of grow_a_language_model names in its pairing-rule table;
 * here the scale is applied in registers inside the update and g is not
 * written.
 *
 *   w, m, v  device float32[n], read and written.
 *   g        device float32[n], read only. Must not overlap w, m or v.
 *   n        1 .. RCS_MAX_N.
 *   t        1-based index of this update (a fresh run starts at 1; after
 *            ckpt_unpack returned step k, continue with t = k + 1).
 *   lr, wd   finite; clip > 0 (+inf means never clip).
 *
 * Arithmetic (float32, each op rounded to nearest-even, no contraction,
 * subnormals kept): norm = sqrt(sum of float64 squares) in float64;
 * s = (float)(clip/norm) if norm > clip else 1; per element gp = g*s,
 * m = 0.9f*m + 0.1f*gp, v = 0.999f*v + 0.001f*(gp*gp), mh = m/bc1,
 * vh = v/bc2, w = w*decay - (lr*mh)/(sqrtf(vh) + 1e-8f), where
 * bc1 = (float)(1-0.9^t), bc2 = (float)(1-0.999^t) and
 * decay = (float)(1 - (double)lr*(double)wd) are computed on the host.
 * If the norm is not finite the update is skipped on the device (w, m, v are
 * left untouched); read the norm with last_grad_norm.
 * The reduction order depends only on n and on g's address modulo 256
 * bytes, so results are deterministic for a given buffer.
 * The update kernel streams the arrays in 16-byte vectors from the next
 * 256-byte boundary of an anchor array on and takes the 0-63 elements before
 * it separately (with fewer than 4 elements after that boundary: from the next
 * 16-byte one). The anchor is w or m, whichever shares its 128-byte line
 * phase with more of w, m, v (m only when v lies at m's 16-byte phase; w on
 * a tie); arrays at the anchor's 16-byte phase take aligned vectors, the
 * others aligned vectors shifted across neighbouring lanes (so every array
 * is still read and written 16 bytes at a time), and the lines that two
 * waves share when an array's span does not start on a line are read and
 * written with cache-retaining accesses. Up to n = 8,388,608 the update
 * kernel also does the final reduction itself, in grad_norm_final's order
 * (two launches instead of three; the same norm bits as grad_global_norm).
 * Arrays too short for a head and one vector take partial, final and a
 * scalar update kernel with the same arithmetic.
 */
int adamw_clip_step(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                    float lr, float wd, float clip, hipStream_t stream);

/*
 * adamw_clip_step for a gradient accumulated over micro-batches: g holds the
 * sum of n_micro micro-batch gradients (backward passes add into one buffer)
 * and grad_scale = 1/n_micro. Each element is first multiplied by grad_scale
 * in float32 (the averaging step the backprop lesson runs before the optimizer
 * step, under "accumulation over micro-batches"), then norm, clip and update
 * proceed exactly as in adamw_clip_step on that averaged gradient. The scale
 * is applied in registers in both kernels; g is not written. grad_scale must
 * be finite and > 0; adamw_clip_step is this call with grad_scale = 1.
 */
int adamw_clip_step_accum(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                          float lr, float wd, float clip, float grad_scale, hipStream_t stream);

/*
 * adamw_clip_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as adamw_clip_step (bit for bit), but
 * the norm pass's partial sums and the clip record live in a static device
 * array of 4 KiB compiled into the library (one per GPU, held until the
 * process ends) instead of the per-(device, stream) workspace, and the call
 * makes no allocation of any kind. The array's device address is looked up
 * once per GPU, by rcs_init or else by the first call on that GPU. Every n
 * from 1 to RCS_MAX_N fits in it (the norm pass never has more than 256
 * blocks); a larger n is RCS_EINVAL as for adamw_clip_step.
 * norm_out (may be NULL): pinned host or current-device memory that receives
 * the float64 pre-clip norm in stream order (this call does not update what
 * last_grad_norm reports).
 * All calls on one GPU share the array: two calls whose work overlaps on the
 * device (different streams without ordering between them) race on it and may
 * corrupt each other's norm; order them, or use adamw_clip_step. Nothing in
 * the array needs clearing: every call writes the partials and the record
 * before reading them.
 */
int adamw_clip_step_noalloc(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                            float lr, float wd, float clip, double *norm_out,
                            hipStream_t stream);

/*
 * The pre-clip global norm alone: sqrt(sum_i (double)g[i]^2), same kernels and
 * order as adamw_clip_step (the per-block partial sums and the final reduction
 * of the backprop lesson's pairing-rule table, without the scale). The resume
 * page ("Task and Prerequisites") records this norm before clipping, to spot
 * numerical faults. norm_out is device memory or pinned host memory and
 * receives one float64 once the stream reaches this call.
 */
int grad_global_norm(const float *g, int64_t n, double *norm_out, hipStream_t stream);

/*
 * The global clip on its own, in place: the norm kernels as in
 * adamw_clip_step, then the pages' third clip kernel (the grad_scale of the
 * backprop lesson's pairing-rule table; up to n = 8,388,608 it does the final
 * reduction itself, as the update kernel does): g[i] = g[i] * s in float32 with
 * s = (float)(clip/norm) if norm > clip, else 1. If the norm is not finite,
 * g is left untouched. For callers that need the clipped gradient itself
 * (adamw_clip_step never writes g). g: device float32[n]; clip > 0 (+inf
 * never clips). 12 bytes of HBM traffic per element (norm read, scale read
 * and write). The pre-clip norm is then available from last_grad_norm.
 */
int grad_clip_inplace(float *g, int64_t n, float clip, hipStream_t stream);

/*
 * Sets g[0..n) to +0.0f: the reset of the gradient buffer after the
 * optimizer step in the backprop lesson's accumulation loop (under
 * "accumulation over micro-batches": backward adds into one buffer with +=,
 * so it must be cleared before the next step's first micro-batch; the
 * resume page's update order likewise starts with zeroing the gradients).
 * g: device float32[n], n 1 .. RCS_MAX_N; 4 bytes written per element, with
 * 16-byte stores (256-lane blocks) from g's next 256-byte boundary on. A
 * kernel, not a memset, so it may be captured into a graph. Asynchronous on
 * stream.
 */
int grad_zero(float *g, int64_t n, hipStream_t stream);

/*
 * Copies the pre-clip norm computed by the most recent adamw_clip_step,
 * adamw_clip_step_accum, grad_clip_inplace or grad_global_norm on this stream
 * into norm_out (device or pinned host float64), in stream order. The resume
 * lesson records this norm before the clip to detect numerical faults.
 * RCS_EINVAL if nothing ran on the stream.
 */
int last_grad_norm(hipStream_t stream, double *norm_out);

/*
 * Size of a step file for n parameters: 8 + 12 n, or -1 if n <= 0 or
 * n > RCS_MAX_N. Layout from grow_a_language_model_checkpoints, sections
 * "Format" and "Total size": [int32 step][int32 n][n f32 w][n f32 m][n f32 v].
 */
int64_t ckpt_bytes(int64_t n);

/*
 * Packs the state into host_buf (buf_bytes must equal ckpt_bytes(n)):
 * little-endian int32 step and n at offsets 0 and 4 (written by the host
 * before returning), then w, m, v copied device-to-host at offsets 8, 8+4n,
 * 8+8n in stream order. step is the number of completed updates (>= 0); the
 * resume lesson saves after a complete optimizer step. host_buf should be
 * pinned (hipHostMalloc) for the copies to be asynchronous.
 */
int ckpt_pack(int32_t step, int64_t n, const float *w, const float *m, const float *v,
              void *host_buf, int64_t buf_bytes, hipStream_t stream);

/*
 * Validates a packed state and copies it host-to-device. The header is read
 * on the host before returning, so host_buf must already hold the bytes.
 * Rejected (nothing copied, outputs untouched): buf_bytes < 8 (RCS_ESIZE),
 * header n <= 0 or step < 0 or n != n_expected (RCS_EHEADER), buf_bytes !=
 * 8 + 12 n (RCS_ESIZE). On success *step_out = step and w, m, v (device
 * float32[n_expected]) receive the arrays in stream order; continue training
 * with t = step + 1. The checks follow the sharded-resume lesson's rule that
 * a bad checkpoint must fail loudly rather than load silently.
 */
int ckpt_unpack(const void *host_buf, int64_t buf_bytes, int64_t n_expected, int32_t *step_out,
                float *w, float *m, float *v, hipStream_t stream);

/*
 * Asynchronous pack, so the training stream does not stall for the host
 * link (the sharded-resume lesson's "async write" production pattern):
 *   1. on compute_stream, in order after the updates already enqueued there,
 *      a kernel copies w, m, v into `snapshot` (device float32[3n], the file
 *      payload [w | m | v]): 24 B per parameter at HBM speed;
 *   2. copy_stream waits for that kernel, then copies the snapshot to
 *      host_buf + 8; the header is written by the host before returning.
 * Updates enqueued on compute_stream afterwards may change w, m, v at once;
 * the packed bytes are those of the state at the call. A later
 * ckpt_pack_async on the same snapshot makes compute_stream wait until the
 * earlier copy out of it has finished. host_buf must not be read or reused
 * until ckpt_pack_wait(snapshot) returns (or copy_stream is synchronized).
 * Sizes: snapshot_bytes == ckpt_snapshot_bytes(n) == 12 n, buf_bytes ==
 * ckpt_bytes(n). The snapshot must not overlap w, m or v (they may sit next
 * to it in one allocation). The snapshot kernel writes each part in aligned
 * 16-byte vectors and reads its source in aligned 16-byte vectors at any
 * 4-byte phase (n >= 4, 4-byte aligned pointers; otherwise a 4-byte copy).
 */
int64_t ckpt_snapshot_bytes(int64_t n);
int ckpt_pack_async(int32_t step, int64_t n, const float *w, const float *m, const float *v,
                    float *snapshot, int64_t snapshot_bytes, void *host_buf, int64_t buf_bytes,
                    hipStream_t compute_stream, hipStream_t copy_stream);
/* Blocks until the last ckpt_pack_async out of `snapshot` has landed in its
 * host buffer (RCS_OK at once if there is none). */
int ckpt_pack_wait(const float *snapshot);

/*
 * On-disk step files (grow_a_language_model_checkpoints, "SIGTERM &
 * SIGUSR1"; the sharded-resume lesson's atomic write). All host-only; none
 * touches the device.
 *
 * ckpt_file_write: host_buf holds a packed state (as ckpt_pack leaves it,
 * after its copies have completed); its header must be consistent with
 * buf_bytes. Writes <dir>/step_%06d.bin.tmp, fsyncs it, renames it to
 * <dir>/step_%06d.bin (atomic on POSIX) and fsyncs the directory, so a crash
 * leaves either the old set of files or the new complete file. The final path
 * is copied to path_out (if not NULL; RCS_EINVAL, before anything is
 * written, if path_cap is too small).
 * ckpt_file_size: size in bytes of a regular file, or RCS_ENOENT.
 * ckpt_file_read: reads a whole file into host_buf; its size must equal
 * buf_bytes (RCS_ESIZE) and its header must be consistent (RCS_EHEADER).
 * ckpt_file_latest: the valid step file with the highest step in dir (name
 * step_<digits>.bin matching the header's step, header consistent with the
 * size); temporaries and malformed files are skipped; RCS_ENOENT if none.
 * ckpt_file_rotate: keeps the `keep` newest valid step files, deletes the
 * older ones and any step_*.bin.tmp leftovers (so no other writer may be
 * writing into dir at the time); returns how many were removed.
 */
int ckpt_file_write(const char *dir, const void *host_buf, int64_t buf_bytes, char *path_out,
                    int64_t path_cap);
/* Same atomic write (tmp, fsync, rename, fsync dir) of a packed state to an
 * explicit path, e.g. one rank's shard file of a sharded checkpoint. */
int ckpt_file_write_path(const char *path, const void *host_buf, int64_t buf_bytes);
/* Atomic write of arbitrary bytes (a shard manifest, written last so that a
 * crash never leaves a manifest pointing at missing or partial shards). */
int rcs_file_write_atomic(const char *path, const void *data, int64_t len);
int64_t ckpt_file_size(const char *path);
int ckpt_file_read(const char *path, void *host_buf, int64_t buf_bytes);
int ckpt_file_latest(const char *dir, int32_t *step_out, char *path_out, int64_t path_cap);
int ckpt_file_rotate(const char *dir, int keep);

/*
 * SIGTERM / SIGUSR1 (grow_a_language_model_checkpoints, "SIGTERM & SIGUSR1"):
 * rcs_signals_install sets handlers that only raise flags; the training loop
 * calls rcs_signals_poll after each completed update and gets a bit mask
 * (cleared by the call): RCS_SIG_WRITE_CONTINUE (SIGUSR1: write the step file
 * and carry on), RCS_SIG_WRITE_EXIT (SIGTERM: write the step file and exit).
 */
#define RCS_SIG_WRITE_CONTINUE 1
#define RCS_SIG_WRITE_EXIT 2
int rcs_signals_install(void);
int rcs_signals_poll(void);

/*
 * Asynchronous step-file writer (the sharded-resume lesson's production
 * patterns: asynchronous, atomic, keep the newest K; the checkpoints page's
 * SIGTERM save, after which the caller waits and exits). The writer owns a
 * device snapshot (12 n bytes), two pinned host images (8 + 12 n bytes
 * each), a copy stream and one worker thread, all made by
 * rcs_ckpt_writer_create on the current device and freed by
 * rcs_ckpt_writer_destroy. dir must exist (as
 * for ckpt_file_write); a missing or unwritable one makes each write fail
 * with RCS_EIO.
 *
 * The writer has two pinned host images of 8 + 12 n bytes each, so that one
 * can receive a copy while the other is being written to disk.
 * rcs_ckpt_writer_submit: waits while the host image it will use is still
 * being written (the save two submits back); if an earlier write failed,
 * returns that status and submits nothing; then enqueues ckpt_pack_async of
 * (step, w, m, v) -- a snapshot kernel on compute_stream, the device-to-host
 * copy into the image on the writer's copy stream -- and returns; the worker
 * waits for the copy, writes <dir>/step_%06d.bin atomically (ckpt_file_write)
 * and keeps the `keep` newest files (ckpt_file_rotate), one job at a time in
 * submit order. w, m, v may be updated by later work on compute_stream right
 * away. Must be called with the writer's device current; submits are
 * serialized.
 * rcs_ckpt_writer_wait: blocks until no write is in flight and returns the
 * first failure not yet reported (else RCS_OK); path_out (optional, path_cap
 * bytes) receives the newest path written since the last wait. Both are
 * reported once: a second wait returns RCS_OK and "". A path_cap too small
 * for the path returns RCS_EINVAL and leaves the status and path to the next
 * wait.
 * rcs_ckpt_writer_destroy: waits, stops the worker, frees everything; returns
 * the status of the last write not yet reported. NULL is a no-op.
 */
typedef struct rcs_ckpt_writer rcs_ckpt_writer;
int rcs_ckpt_writer_create(const char *dir, int64_t n, int keep, rcs_ckpt_writer **out);
int rcs_ckpt_writer_submit(rcs_ckpt_writer *writer, int32_t step, const float *w, const float *m,
                           const float *v, hipStream_t compute_stream);
int rcs_ckpt_writer_wait(rcs_ckpt_writer *writer, char *path_out, int64_t path_cap);
int rcs_ckpt_writer_destroy(rcs_ckpt_writer *writer);

/*
 * Instrumentation: while enabled, adamw_clip_step has its kernel dispatches
 * stamp HIP events (start of grad_norm_partial, end of the last norm kernel
 * -- grad_norm_partial itself when the update kernel does the final
 * reduction --, start and end of the update kernel) on one call in `every`
 * (the first call after enabling is recorded), up to max_records recorded
 * calls. rcs_profile_read synchronizes those events and returns the summed
 * milliseconds and the number of recorded calls. Enabling (or
 * disabling) discards earlier records. Events are created here, not in the
 * recorded calls.
 */
int rcs_profile_enable(int on, int max_records, int every);
int rcs_profile_read(double *norm_ms_total, double *update_ms_total, int64_t *steps);

#ifdef __cplusplus
}
#endif

#endif /* RCS_H */

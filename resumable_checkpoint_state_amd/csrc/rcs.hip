// rcs.hip -- gfx950 kernels and the C ABI for one clipped AdamW update over a
// flat float32 parameter vector, plus the step_NNNNNN.bin pack/unpack.
//
// Method sources (pages named by title, then section):
//   * "Training as a Recoverable State Transition", section "The Exact Targets
//     of Clipping and AdamW": global L2 clip to threshold c; AdamW with
//     beta1 = 0.9, beta2 = 0.999, eps = 1e-8, bias correction by
//     1 - beta^t, decay (1 - lr*wd) applied to every parameter first.
//   * grow_a_language_model_backprop, section on the pairing rule: the clip
//     is split into a per-block partial-sum kernel, a final-reduction kernel
//     and a scale kernel. Here the scale is folded into the update so g is
//     read once more and never written.
//   * grow_a_language_model_checkpoints, sections "Format", "Region by
//     region" and "Total size": [int32 step][int32 n][w][m][v], 8 + 12 n bytes.
//
// Hardware mapping (MI355X, CDNA4, 64-wide waves, 256 CUs):
//   * grad_norm_partial: a grid fixed by n alone (at most 256 blocks of 512
//     lanes) streams g with 16-byte loads, squares in float64 (exact for
//     float32 inputs) into four independent accumulators per lane, reduces
//     each wave with DPP row permutes plus two cross-row swizzles, and
//     combines the block's waves through LDS in wave order: one float64
//     partial per block. The last 320 MB of g are read with cache-allocating
//     loads so that the part of g still in the 256 MB last-level cache serves
//     the update's second read; the rest streams.
//   * grad_norm_final: one wave sums the <= 256 partials in a fixed tree
//     (4 per lane, then the wave butterfly), takes the float64 square root and
//     writes {norm, clip factor, apply flag}. No float atomics anywhere, so
//     the result depends only on n and the data. (A single kernel whose last
//     block does this step needs a device-scope release per block, which on
//     this chip costs an L2 write-back per block and measured slower.)
//   * adamw_update_vec: one wave per block, one 16-byte vector of w, g, m, v
//     per lane (16 B read + 12 B written per element) with streaming loads
//     and stores; the clip factor comes from device memory, so the host never
//     waits between kernels. Each XCD streams its own contiguous eighth of the
//     vectors (block b works in region b % 8, blocks being dispatched
//     round-robin over the 8 XCDs), which evens out DRAM contention between
//     the seven streams.
//   * adamw_update_vec_fold: for n up to 8,388,608, where the step is bound
//     by launch cost, every wave does grad_norm_final's reduction itself (the
//     same bits) and the step is two launches instead of three.
//   * Arrays that start off a 16-byte boundary (views into a flat buffer)
//     keep the vector kernels: block 0 takes the 0-63 elements before w's
//     next 256-byte boundary one per lane, and the waves stream whole cache
//     lines from there; g, m or v at another 16-byte phase than w take four
//     4-byte accesses per lane (adamw_update_mixed).
// No MFMA: nothing here is a contraction.
//
// Floating-point contract: built with -ffp-contract=off (and the pragma
// below), correctly rounded float32 divide and square root (HIP's default),
// and without denormal flushing, so every float32 op is one IEEE
// round-to-nearest-even operation, matching the sequence documented in rcs.h.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "rcs.h"

#pragma clang fp contract(off)

// Launch-shape knobs (overridable at build time for sweeps).
// Contiguous regions of the vectors the update streams at once: block b
// works in region b % k. Blocks are dispatched round-robin over the chip's 8
// XCDs, so with k = 8 each XCD streams its own contiguous eighth of w, g, m, v.
// With one-wave blocks, over 14 buffer placements on one box the step took
// 605.0-619.3 us (mean 611.0) with k = 8 against 612.9-631.1 (617.5) with
// k = 4 (6 placements on another box: means 609.9 and 608.0; k = 2, 1, 16
// and 32 were slower).
#ifndef RCS_UPD_REGIONS
#define RCS_UPD_REGIONS 8
#endif
#ifndef RCS_UPD_NT
#define RCS_UPD_NT 1
#endif
// Largest n whose step folds the final norm reduction into the update kernel
// (measured: folding saves 1.7-2.4 us per step up to 8,388,608 elements and
// costs 4.8 us at 16,777,216 and 23 us at 124,356,864).
#ifndef RCS_FOLD_MAX_N
#define RCS_FOLD_MAX_N 8388608
#endif
// Bytes at the end of g that the norm pass reads with ordinary (cache-
// allocating) loads so that the update, which reads g again right after,
// finds them in the last-level cache; the rest is read with streaming loads.
// A negative value reads all of g with ordinary loads.
#ifndef RCS_NORM_CACHED_TAIL_BYTES
#define RCS_NORM_CACHED_TAIL_BYTES (320LL << 20)
#endif

namespace {

constexpr int kWave = 64;
// Norm pass: at most 256 blocks of 512 lanes, 4 loads of 16 B in flight per
// lane (measured best of 256-1024 lanes x 2-8 loads with 256 blocks, and
// faster per step than 2048 blocks x 256 lanes followed by a final kernel).
constexpr int kNormThreads = 512;
constexpr int kNormUnroll = 4;
constexpr int64_t kNormChunk = (int64_t)kNormThreads * kNormUnroll;  // vectors per block-iteration
constexpr int kNormMaxBlocks = 256;
// At most this many partials reach the final reduction.
constexpr int kParts = kNormMaxBlocks;
// Lanes per block of the update and in-place scale kernels, one 16-byte
// vector of each array per lane; the final reduction (in those kernels and in
// grad_norm_final) runs on blocks of the same size, lane i summing partials
// i, i + L, i + 2L, ... in that order, so all three give the same bits.
// One wave per block measured fastest: the update takes 529.7 us at the
// ANDREA-120M size against 546.1 us with 256 lanes (same process).
#ifndef RCS_UPD_THREADS
#define RCS_UPD_THREADS 64
#endif
constexpr int kUpdThreads = RCS_UPD_THREADS;
static_assert(kUpdThreads == 64 || kUpdThreads == 128 || kUpdThreads == 256, "lanes per block");
constexpr int kPartsPerLane = kParts / kUpdThreads;

// Native 16-byte vector (the nontemporal builtins need a clang vector type).
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ClipScalars {
    double norm;    // pre-clip global L2 norm
    float scale;    // clip factor s
    int32_t apply;  // 1 when the norm is finite, else the update is skipped
};

struct StepScalars {
    float lr, bc1, bc2, decay;
    float gscale;  // micro-batch averaging factor applied to g first (1 = none)
};

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ double as_double(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
    return as_double((uint32_t)lo, (uint32_t)hi);
}

// Sum over the 64 lanes; every lane ends with the same value (each step adds
// a value to its mirror partner, and a + b == b + a exactly).
__device__ __forceinline__ double wave_sum(double x) {
    x += dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]: pairs
    x += dpp_f64<0x4E>(x);   // quad_perm [2,3,0,1]: quads
    x += dpp_f64<0x141>(x);  // row_half_mirror: 8 lanes
    x += dpp_f64<0x140>(x);  // row_mirror: 16-lane row
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

// Block sum in wave order; the result is valid in thread 0 only.
template <int THREADS>
__device__ __forceinline__ double block_sum(double x, double *lds) {
    x = wave_sum(x);
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    if (lane == 0) lds[wid] = x;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
        r = lds[0];
#pragma unroll
        for (int i = 1; i < THREADS / kWave; ++i) r += lds[i];
    }
    return r;
}

// Square, in float64, of the gradient after the float32 micro-batch scale
// (x * gscale is one float32 rounding; gscale = 1 leaves x unchanged).
__device__ __forceinline__ double sq(float x, float gscale) {
    const double d = (double)(x * gscale);
    return d * d;
}

// a1: per-block float64 partial sums of squares. head >= 0 (at most 63):
// g + head is 16-byte aligned; its vectors are read with 16-byte loads (the first
// nt_limit4 streaming, the rest cache-allocating), block 0 adds the head
// elements before it and the n % 4 after it. head < 0: scalar loads only.
__global__ __launch_bounds__(kNormThreads) void grad_norm_partial(const float *__restrict__ g,
                                                                  int64_t n, int head,
                                                                  int64_t nt_limit4, float gscale,
                                                                  double *__restrict__ partials) {
    __shared__ double lds[kNormThreads / kWave];
    double acc[kNormUnroll];
#pragma unroll
    for (int j = 0; j < kNormUnroll; ++j) acc[j] = 0.0;
    const int64_t nblk = gridDim.x;
    if (head >= 0) {
        if (blockIdx.x == 0 && (int)threadIdx.x < head) acc[1] += sq(g[threadIdx.x], gscale);
        g += head;
        n -= head;
        const f32x4 *__restrict__ g4 = reinterpret_cast<const f32x4 *>(g);
        const int64_t n4 = n >> 2;
        for (int64_t base = (int64_t)blockIdx.x * kNormChunk; base < n4; base += nblk * kNormChunk) {
            f32x4 x[kNormUnroll];
            if (base < nt_limit4) {
#pragma unroll
                for (int j = 0; j < kNormUnroll; ++j) {
                    const int64_t i = base + (int64_t)j * kNormThreads + threadIdx.x;
                    x[j] = (i < n4) ? __builtin_nontemporal_load(g4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else {
#pragma unroll
                for (int j = 0; j < kNormUnroll; ++j) {
                    const int64_t i = base + (int64_t)j * kNormThreads + threadIdx.x;
                    x[j] = (i < n4) ? g4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int j = 0; j < kNormUnroll; ++j) {
                acc[j] += sq(x[j].x, gscale);
                acc[j] += sq(x[j].y, gscale);
                acc[j] += sq(x[j].z, gscale);
                acc[j] += sq(x[j].w, gscale);
            }
        }
        const int rem = (int)(n & 3);
        if (blockIdx.x == 0 && (int)threadIdx.x < rem) acc[0] += sq(g[(n4 << 2) + threadIdx.x], gscale);
    } else {
        for (int64_t i = (int64_t)blockIdx.x * kNormThreads + threadIdx.x; i < n;
             i += nblk * kNormThreads)
            acc[0] += sq(g[i], gscale);
    }
    const double t = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const double b = block_sum<kNormThreads>(t, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = b;
}

// a2, first half: lane i of a kUpdThreads-lane block loads partials i, i + L,
// i + 2L, ... (L = kUpdThreads). Every load is issued (lanes past nparts
// re-read the last partial; final_reduce drops them), so that a caller can
// issue its own loads behind these and still wait for these alone.
__device__ __forceinline__ void load_partials(const double *__restrict__ partials, int nparts,
                                              double (&x)[kPartsPerLane]) {
#pragma unroll
    for (int k = 0; k < kPartsPerLane; ++k) {
        const int j = (int)threadIdx.x + k * kUpdThreads;
        x[k] = partials[j < nparts ? j : nparts - 1];
    }
}

// a2, second half: each lane sums its partials in index order (0 beyond
// nparts), the block sums the lanes in the fixed wave/LDS tree, then the
// float64 square root and the clip factor. The result is valid in every lane.
__device__ __forceinline__ ClipScalars final_reduce(const double (&x)[kPartsPerLane], int nparts,
                                                    float clip, double *lds) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kPartsPerLane; ++k)
        acc += ((int)threadIdx.x + k * kUpdThreads < nparts) ? x[k] : 0.0;
    double S;
    if constexpr (kUpdThreads == kWave) {
        S = wave_sum(acc);  // the same bits in every lane
    } else {
        const double b = block_sum<kUpdThreads>(acc, lds);
        if (threadIdx.x == 0) lds[0] = b;  // block_sum's reads of lds are done by now
        __syncthreads();
        S = lds[0];
    }
    ClipScalars r;
    r.norm = sqrt(S);
    r.apply = isfinite(r.norm) ? 1 : 0;
    r.scale = (r.norm > (double)clip) ? (float)((double)clip / r.norm) : 1.0f;
    return r;
}

// a2 as its own kernel (the norm alone, and the unaligned / n < 4 paths):
// one kUpdThreads-lane block writes {norm, clip factor, apply flag}.
__global__ __launch_bounds__(kUpdThreads) void grad_norm_final(const double *__restrict__ partials,
                                                               int nparts, float clip,
                                                               ClipScalars *__restrict__ out) {
    __shared__ double lds[kUpdThreads / kWave];
    double x[kPartsPerLane];
    load_partials(partials, nparts, x);
    const ClipScalars r = final_reduce(x, nparts, clip, lds);
    if (threadIdx.x == 0) *out = r;
}

// ---------------------------------------------------------------- update

// The float32 op sequence of one element; every line is one rounding.
__device__ __forceinline__ void adamw_elem(float &w, float g, float &m, float &v, float s,
                                           const StepScalars &h) {
    const float ga = g * h.gscale;
    const float gp = ga * s;
    const float mi = 0.9f * m + 0.1f * gp;
    const float vi = 0.999f * v + 0.001f * (gp * gp);
    const float mh = mi / h.bc1;
    const float vh = vi / h.bc2;
    const float den = __builtin_sqrtf(vh) + 1e-8f;
    w = w * h.decay - (h.lr * mh) / den;
    m = mi;
    v = vi;
}

__device__ __forceinline__ void adamw_vec4(f32x4 &w, f32x4 g, f32x4 &m, f32x4 &v, float s,
                                           const StepScalars &h) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float ww = w[k], mm = m[k], vv = v[k];
        adamw_elem(ww, g[k], mm, vv, s, h);
        w[k] = ww;
        m[k] = mm;
        v[k] = vv;
    }
}

template <typename T>
__device__ __forceinline__ T ld_stream(const T *p) {
#if RCS_UPD_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void st_stream(T *p, T x) {
#if RCS_UPD_NT
    __builtin_nontemporal_store(x, p);
#else
    *p = x;
#endif
}

// Four consecutive floats of a lane: one 16-byte access when the array shares
// w's 16-byte phase (VEC), else four 4-byte accesses (still streaming).
template <bool VEC>
__device__ __forceinline__ f32x4 ld4(const float *p) {
    if constexpr (VEC) return ld_stream(reinterpret_cast<const f32x4 *>(p));
    else return f32x4{ld_stream(p), ld_stream(p + 1), ld_stream(p + 2), ld_stream(p + 3)};
}

template <bool VEC>
__device__ __forceinline__ void st4(float *p, f32x4 x) {
    if constexpr (VEC) {
        st_stream(reinterpret_cast<f32x4 *>(p), x);
    } else {
        st_stream(p, x.x);
        st_stream(p + 1, x.y);
        st_stream(p + 2, x.z);
        st_stream(p + 3, x.w);
    }
}

// a3: clip factor and AdamW on one 16-byte vector of w, g, m, v per lane, with
// streaming loads and stores; block b works in contiguous region b % 8 (one
// region per XCD). Every load is unconditional (lanes past the end re-read the
// last vector and discard it; the host guarantees n >= 4; a discarded re-read
// may overlap the owner lane's store, and its value is never used).
// FOLD = false: the clip record comes from grad_norm_final, launched before.
// FOLD = true: every block first does grad_norm_final's reduction itself (same
// order, same bits; block 0 stores the record), saving a launch, which pays
// only while launches are the cost; the partial loads go out first so that
// waiting for them leaves the element loads in flight. At large n the
// per-wave float64 square root and division cost more than the launch (one
// wave per block: 529.7 against 552.2 us for the update at the ANDREA-120M
// size, measured in one process).
// w's body is 16-byte aligned (the head is w's); GV, MV, VV say whether g, m
// and v share w's 16-byte phase and so take one 16-byte access per lane, or
// lie at another and take four 4-byte accesses (ld4 / st4).
template <bool FOLD, bool GV, bool MV, bool VV>
__device__ __forceinline__ void update_body(f32x4 *__restrict__ w, const float *__restrict__ gf,
                                            float *__restrict__ mf, float *__restrict__ vf,
                                            int64_t n, int head,
                                            const double *__restrict__ partials, int nparts,
                                            float clip, ClipScalars *__restrict__ sc,
                                            const StepScalars &h, double *lds) {
    const int64_t n4 = n >> 2;
    int64_t c = blockIdx.x;
    if (RCS_UPD_REGIONS > 1) {  // bijection of [0, nblk): region b % k, position b / k
        const int64_t nblk = gridDim.x;
        const int64_t k = RCS_UPD_REGIONS, q = nblk / k, r = nblk % k, x = c % k, j = c / k;
        c = (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
    }
    const int64_t i = c * kUpdThreads + threadIdx.x;
    double xp[kPartsPerLane];
    if constexpr (FOLD) load_partials(partials, nparts, xp);
    const int64_t ic = i < n4 ? i : n4 - 1;
    f32x4 gr = ld4<GV>(gf + 4 * ic);
    f32x4 wr = ld_stream(w + ic);
    f32x4 mr = ld4<MV>(mf + 4 * ic);
    f32x4 vr = ld4<VV>(vf + 4 * ic);
    ClipScalars cs;
    if constexpr (FOLD) {
        cs = final_reduce(xp, nparts, clip, lds);
        if (blockIdx.x == 0 && threadIdx.x == 0) *sc = cs;
    } else {
        cs = *sc;
    }
    if (!cs.apply) return;
    const float s = cs.scale;
    if (i < n4) {
        adamw_vec4(wr, gr, mr, vr, s, h);
        st_stream(w + i, wr);
        st4<MV>(mf + 4 * i, mr);
        st4<VV>(vf + 4 * i, vr);
    }
    // block 0: the head elements before the body (indices -head .. -1);
    // the last block: the n % 4 after the last vector
    float *wf = reinterpret_cast<float *>(w);
    if (blockIdx.x == 0 && (int)threadIdx.x < head) {
        const int64_t k = (int64_t)threadIdx.x - head;
        float ww = wf[k], mm = mf[k], vv = vf[k];
        adamw_elem(ww, gf[k], mm, vv, s, h);
        wf[k] = ww;
        mf[k] = mm;
        vf[k] = vv;
    }
    if (blockIdx.x == gridDim.x - 1 && (int)threadIdx.x < (int)(n & 3)) {
        const int64_t k = (n4 << 2) + threadIdx.x;
        float ww = wf[k], mm = mf[k], vv = vf[k];
        adamw_elem(ww, gf[k], mm, vv, s, h);
        wf[k] = ww;
        mf[k] = mm;
        vf[k] = vv;
    }
}

// a3 after grad_norm_final. w, g, m, v point `head` (0-63) elements past the
// arrays' starts, at 16-byte boundaries; n counts from there.
__global__ __launch_bounds__(kUpdThreads) void adamw_update_vec(
    f32x4 *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, const ClipScalars *__restrict__ sc,
    StepScalars h) {
    update_body<false, true, true, true>(w, g, m, v, n, head, nullptr, 0, 0.0f,
                                         const_cast<ClipScalars *>(sc), h, nullptr);
}

// a2 + a3 in one kernel (small n).
__global__ __launch_bounds__(kUpdThreads) void adamw_update_vec_fold(
    f32x4 *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, const double *__restrict__ partials, int nparts,
    float clip, ClipScalars *__restrict__ sc_out, StepScalars h) {
    __shared__ double lds[kUpdThreads / kWave];
    update_body<true, true, true, true>(w, g, m, v, n, head, partials, nparts, clip, sc_out, h,
                                        lds);
}

// The same two kernels when some of g, m, v lie at another 16-byte phase than
// w (e.g. w a view into a flat parameter buffer at an odd offset, m and v
// fresh allocations): w and the arrays at its phase keep 16-byte vectors, the
// others take four 4-byte accesses per lane.
template <bool GV, bool MV, bool VV>
__global__ __launch_bounds__(kUpdThreads) void adamw_update_mixed(
    f32x4 *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, const ClipScalars *__restrict__ sc,
    StepScalars h) {
    update_body<false, GV, MV, VV>(w, g, m, v, n, head, nullptr, 0, 0.0f,
                                   const_cast<ClipScalars *>(sc), h, nullptr);
}

template <bool GV, bool MV, bool VV>
__global__ __launch_bounds__(kUpdThreads) void adamw_update_mixed_fold(
    f32x4 *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, const double *__restrict__ partials, int nparts,
    float clip, ClipScalars *__restrict__ sc_out, StepScalars h) {
    __shared__ double lds[kUpdThreads / kWave];
    update_body<true, GV, MV, VV>(w, g, m, v, n, head, partials, nparts, clip, sc_out, h, lds);
}

// a3 for arrays that are not 4-byte aligned or too short for a head and one
// vector: same arithmetic per element.
__global__ __launch_bounds__(kUpdThreads) void adamw_update_scalar(
    float *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, const ClipScalars *__restrict__ sc, StepScalars h) {
    if (!sc->apply) return;
    const float s = sc->scale;
    const int64_t stride = (int64_t)gridDim.x * kUpdThreads;
    for (int64_t i = (int64_t)blockIdx.x * kUpdThreads + threadIdx.x; i < n; i += stride) {
        float ww = w[i], mm = m[i], vv = v[i];
        adamw_elem(ww, g[i], mm, vv, s, h);
        w[i] = ww;
        m[i] = mm;
        v[i] = vv;
    }
}

__global__ __launch_bounds__(256) void fp32_div_sqrt_probe(const float *__restrict__ a,
                                                           const float *__restrict__ b,
                                                           float *__restrict__ q,
                                                           float *__restrict__ r, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        q[i] = a[i] / b[i];
        r[i] = __builtin_sqrtf(a[i]);
    }
}

// The pages' third clip kernel on its own, for callers that need the clipped
// gradient itself: g *= s in place (skipped when the norm is not finite). Same
// float32 product as the update's g * s. g points `head` (0-63) elements past
// the array's start, at a 16-byte boundary, and n counts from there. Lanes past the end re-read the last vector and discard it (the host
// guarantees n >= 4); block 0 also scales the head elements and the last
// block the n % 4 trailing ones. FOLD as in update_body: the record from
// grad_norm_final, or the final reduction at the head of every block.
template <bool FOLD>
__device__ __forceinline__ void scale_body(f32x4 *__restrict__ g, int64_t n, int head,
                                           const double *__restrict__ partials, int nparts,
                                           float clip, ClipScalars *__restrict__ sc, double *lds) {
    const int64_t n4 = n >> 2;
    const int64_t i = (int64_t)blockIdx.x * kUpdThreads + threadIdx.x;
    double xp[kPartsPerLane];
    if constexpr (FOLD) load_partials(partials, nparts, xp);
    f32x4 x = __builtin_nontemporal_load(g + (i < n4 ? i : n4 - 1));
    ClipScalars cs;
    if constexpr (FOLD) {
        cs = final_reduce(xp, nparts, clip, lds);
        if (blockIdx.x == 0 && threadIdx.x == 0) *sc = cs;
    } else {
        cs = *sc;
    }
    if (!cs.apply) return;
    const float s = cs.scale;
    if (i < n4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = x[k] * s;
        __builtin_nontemporal_store(x, g + i);
    }
    float *gf = reinterpret_cast<float *>(g);
    if (blockIdx.x == 0 && (int)threadIdx.x < head) {  // indices -head .. -1
        const int64_t k = (int64_t)threadIdx.x - head;
        gf[k] = gf[k] * s;
    }
    if (blockIdx.x == gridDim.x - 1 && (int)threadIdx.x < (int)(n & 3)) {
        const int64_t k = (n4 << 2) + threadIdx.x;
        gf[k] = gf[k] * s;
    }
}

__global__ __launch_bounds__(kUpdThreads) void grad_scale_vec(f32x4 *__restrict__ g, int64_t n,
                                                              int head,
                                                              const ClipScalars *__restrict__ sc) {
    scale_body<false>(g, n, head, nullptr, 0, 0.0f, const_cast<ClipScalars *>(sc), nullptr);
}

__global__ __launch_bounds__(kUpdThreads) void grad_scale_vec_fold(
    f32x4 *__restrict__ g, int64_t n, int head, const double *__restrict__ partials, int nparts,
    float clip, ClipScalars *__restrict__ sc_out) {
    __shared__ double lds[kUpdThreads / kWave];
    scale_body<true>(g, n, head, partials, nparts, clip, sc_out, lds);
}

// Clears the gradient buffer for the next step's micro-batches (the backprop
// lesson's accumulation loop: backward adds into one buffer, the optimizer
// step reads it, then it is reset to zero). g points `head` (0-63) elements
// past the array's start, at a 16-byte boundary; one 16-byte store per lane,
// block 0 also clears the head elements, the last block the n % 4 trailing
// ones. A pure write stream wants more lanes per block than the update: at
// the ANDREA-120M size 256-lane blocks fill at 6.6-6.8 TB/s against 4.7 with
// one-wave blocks (128: 6.1, 512: 6.2, 1024: 5.9; 2 vectors per lane or a
// grid-stride loop slower still), and ordinary stores edge out streaming
// ones (73-74 against 75-77 us). A kernel rather than a memset, so that it
// can sit in a captured graph.
constexpr int kZeroThreads = 256;
__global__ __launch_bounds__(kZeroThreads) void grad_zero_vec(f32x4 *__restrict__ g, int64_t n,
                                                              int head) {
    const int64_t n4 = n >> 2;
    const int64_t i = (int64_t)blockIdx.x * kZeroThreads + threadIdx.x;
    if (i < n4) g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float *gf = reinterpret_cast<float *>(g);
    if (blockIdx.x == 0 && (int)threadIdx.x < head) gf[(int64_t)threadIdx.x - head] = 0.0f;
    if (blockIdx.x == gridDim.x - 1 && (int)threadIdx.x < (int)(n & 3))
        gf[(n4 << 2) + threadIdx.x] = 0.0f;
}

__global__ __launch_bounds__(256) void grad_zero_scalar(float *__restrict__ g, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) g[i] = 0.0f;
}

__global__ __launch_bounds__(256) void grad_scale_scalar(float *__restrict__ g, int64_t n,
                                                         const ClipScalars *__restrict__ sc) {
    if (!sc->apply) return;
    const float s = sc->scale;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        g[i] = g[i] * s;
}

// a4 (asynchronous form): copy w, m, v into one device snapshot laid out like
// the step file's payload [w | m | v], so that the training stream can keep
// updating w, m, v while the snapshot drains to the host on a copy stream.
// Vector path: n % 4 == 0 and all pointers 16-byte aligned; lane i copies
// snapshot vector i, taken from w, m or v by which third it falls in.
// One wave per block here too: 452-463 us against 466-483 us with 256 lanes
// for the 1.49 GB snapshot at the ANDREA-120M size.
#ifndef RCS_SNAP_THREADS
#define RCS_SNAP_THREADS 64
#endif
constexpr int kSnapThreads = RCS_SNAP_THREADS;
__global__ __launch_bounds__(kSnapThreads) void ckpt_snapshot_vec(const f32x4 *__restrict__ w,
                                                                  const f32x4 *__restrict__ m,
                                                                  const f32x4 *__restrict__ v,
                                                                  f32x4 *__restrict__ snap,
                                                                  int64_t n4) {
    const int64_t total = 3 * n4;
    const int64_t stride = (int64_t)gridDim.x * kSnapThreads;
    for (int64_t i = (int64_t)blockIdx.x * kSnapThreads + threadIdx.x; i < total; i += stride) {
        const f32x4 *src = (i < n4) ? w + i : (i < 2 * n4) ? m + (i - n4) : v + (i - 2 * n4);
        __builtin_nontemporal_store(__builtin_nontemporal_load(src), snap + i);
    }
}

__global__ __launch_bounds__(256) void ckpt_snapshot_scalar(const float *__restrict__ w,
                                                            const float *__restrict__ m,
                                                            const float *__restrict__ v,
                                                            float *__restrict__ snap, int64_t n) {
    const int64_t total = 3 * n;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const float *src = (i < n) ? w + i : (i < 2 * n) ? m + (i - n) : v + (i - 2 * n);
        snap[i] = *src;
    }
}

// ---------------------------------------------------------------- host side

}  // namespace

#include <thread>
#include <tuple>

#include "rcs_internal.h"

namespace {

struct Workspace {
    double *partials = nullptr;      // kNormMaxBlocks float64
    ClipScalars *scalars = nullptr;  // one record
    std::atomic<bool> has_norm{false};
};

std::mutex g_mu;
// Keyed by device and stream; hipStreamPerThread names a different stream in
// every host thread, so under that handle the thread is part of the key.
using WsKey = std::tuple<int, hipStream_t, std::thread::id>;
std::map<WsKey, Workspace> g_ws;

// Per snapshot buffer: `ready` is recorded on the compute stream after the
// snapshot kernel, `copied` on the copy stream after the device-to-host copy.
struct SnapshotSync {
    hipEvent_t ready = nullptr;
    hipEvent_t copied = nullptr;
    bool pending = false;  // a copy out of this snapshot has been enqueued
};
std::map<std::pair<int, const void *>, SnapshotSync> g_snap;

struct Profile {
    bool on = false;
    int max_records = 0;
    int every = 1;       // record one step in `every`
    int64_t calls = 0;   // adamw_clip_step calls since enabling
    int next = 0;
    // 4 per recorded step: start of grad_norm_partial, end of grad_norm_final,
    // start and end of the update kernel, stamped by the dispatches themselves
    std::vector<hipEvent_t> ev;
} g_prof;

int get_workspace(hipStream_t stream, Workspace **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RCS_EHIP;
    const WsKey key(dev, stream,
                    stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id());
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_ws.find(key);
    if (it == g_ws.end()) {
        void *p = nullptr;
        const size_t bytes = (size_t)kNormMaxBlocks * sizeof(double) + 256;
        if (hipMalloc(&p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return RCS_ENOMEM;
        }
        char *base = static_cast<char *>(p);
        it = g_ws.try_emplace(key).first;
        it->second.partials = reinterpret_cast<double *>(base);
        it->second.scalars =
            reinterpret_cast<ClipScalars *>(base + (size_t)kNormMaxBlocks * sizeof(double));
    }
    *out = &it->second;
    return RCS_OK;
}

// p must be device (or managed) memory of the current device and the range
// [p, p + bytes) must lie inside one allocation. Memory the runtime cannot
// report a range for (e.g. virtual-memory mappings) is accepted without the
// length check.
int check_device_range(const void *p, int64_t bytes) {
    if (p == nullptr) return RCS_EINVAL;
    int dev = -1;
    hipPointerAttribute_t pa;
    if (hipGetDevice(&dev) != hipSuccess || hipPointerGetAttributes(&pa, p) != hipSuccess) {
        (void)hipGetLastError();
        return RCS_EINVAL;
    }
    if (pa.type != hipMemoryTypeDevice && pa.type != hipMemoryTypeManaged) return RCS_EINVAL;
    if (pa.type == hipMemoryTypeDevice && pa.device != dev) return RCS_EINVAL;  // another GPU's
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) == hipSuccess && base) {
        const char *lo = static_cast<const char *>(base);
        const char *q = static_cast<const char *>(p);
        if (q < lo || q + bytes > lo + size) return RCS_ESIZE;
        return RCS_OK;
    }
    (void)hipGetLastError();
    return RCS_OK;  // device memory without a reportable range: accepted, length unchecked
}

bool overlaps(const void *a, const void *b, int64_t bytes) {
    const char *x = static_cast<const char *>(a);
    const char *y = static_cast<const char *>(b);
    return x < y + bytes && y < x + bytes;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int norm_blocks(int64_t n) {
    const int64_t per_block = kNormChunk * 4;  // floats per block-iteration
    int64_t b = (n + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > kNormMaxBlocks) b = kNormMaxBlocks;
    return (int)b;
}

// First vector index the norm pass reads with cache-allocating loads.
int64_t norm_nt_limit4(int64_t n) {
    const int64_t n4 = n >> 2;
    if (RCS_NORM_CACHED_TAIL_BYTES < 0) return 0;
    const int64_t tail4 = (int64_t)RCS_NORM_CACHED_TAIL_BYTES / 16;
    return n4 > tail4 ? n4 - tail4 : 0;
}

// Elements before the body the vector kernels take: up to the next 256-byte
// boundary of p (0-63), so that the body's waves cover whole cache lines;
// when fewer than 4 elements would follow it, up to the next 16-byte boundary
// (0-3). -1 when p is not 4-byte aligned or neither leaves 4 elements: the
// vector kernels then do not apply.
int head_of(const void *p, int64_t n) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p) & 255u;
    if (a & 3u) return -1;
    const int h = (int)((256u - a) & 255u) / 4;
    if (n - h >= 4) return h;
    const int h16 = h & 3;
    return n - h16 >= 4 ? h16 : -1;
}

// a1 alone. ev0 / ev1 (optional, profiling) take the kernel's start / end.
void launch_partial(const float *g, int64_t n, float gscale, Workspace *ws, hipStream_t stream,
                    hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    const int head = head_of(g, n);
    hipExtLaunchKernelGGL(grad_norm_partial, dim3(norm_blocks(n)), dim3(kNormThreads), 0, stream,
                          ev0, ev1, 0, g, n, head, norm_nt_limit4(head >= 0 ? n - head : n),
                          gscale, ws->partials);
}

// a1 + a2. ev (optional, profiling): ev[0] takes the partial kernel's start,
// ev[1] the final kernel's end.
int launch_norm(const float *g, int64_t n, float gscale, float clip, Workspace *ws,
                hipStream_t stream, hipEvent_t *ev = nullptr) {
    launch_partial(g, n, gscale, ws, stream, ev ? ev[0] : nullptr);
    hipExtLaunchKernelGGL(grad_norm_final, dim3(1), dim3(kUpdThreads), 0, stream, nullptr,
                          ev ? ev[1] : nullptr, 0, (const double *)ws->partials, norm_blocks(n),
                          clip, ws->scalars);
    return hipGetLastError() == hipSuccess ? RCS_OK : RCS_EHIP;
}

// Whether the vector kernels do the final reduction themselves (two launches)
// rather than after grad_norm_final (three): only while the launch it saves
// costs more than the reduction at the head of every wave.
bool fold_final(int64_t n) { return n <= (int64_t)RCS_FOLD_MAX_N; }

// Arguments of the update kernels after the norm kernels.
struct UpdateLaunch {
    dim3 grid;
    f32x4 *w;
    const float *g;
    float *m, *v;
    int64_t nb;
    int head;
    bool fold;
    const double *partials;
    int nparts;
    float clip;
    ClipScalars *sc;
    StepScalars h;
    hipStream_t stream;
    hipEvent_t e2, e3;
};

template <bool GV, bool MV, bool VV>
void launch_update(const UpdateLaunch &a) {
    const dim3 block(kUpdThreads);
    if constexpr (GV && MV && VV) {
        if (a.fold)
            hipExtLaunchKernelGGL(adamw_update_vec_fold, a.grid, block, 0, a.stream, a.e2, a.e3, 0,
                                  a.w, a.g, a.m, a.v, a.nb, a.head, a.partials, a.nparts, a.clip,
                                  a.sc, a.h);
        else
            hipExtLaunchKernelGGL(adamw_update_vec, a.grid, block, 0, a.stream, a.e2, a.e3, 0, a.w,
                                  a.g, a.m, a.v, a.nb, a.head, (const ClipScalars *)a.sc, a.h);
    } else {
        if (a.fold)
            hipExtLaunchKernelGGL(adamw_update_mixed_fold<GV, MV, VV>, a.grid, block, 0, a.stream,
                                  a.e2, a.e3, 0, a.w, a.g, a.m, a.v, a.nb, a.head, a.partials,
                                  a.nparts, a.clip, a.sc, a.h);
        else
            hipExtLaunchKernelGGL(adamw_update_mixed<GV, MV, VV>, a.grid, block, 0, a.stream, a.e2,
                                  a.e3, 0, a.w, a.g, a.m, a.v, a.nb, a.head,
                                  (const ClipScalars *)a.sc, a.h);
    }
}

// The whole step a1..a3. Vector form (all four arrays 4-byte aligned, at
// least 4 elements past w's head): the partial kernel, [grad_norm_final,] the
// update kernel on w's aligned body, which also takes the head elements; g, m
// and v at w's 16-byte phase are accessed as 16-byte vectors, the others four
// floats per lane. Otherwise: partial, final, scalar update.
// ev (optional, profiling): ev[0] / ev[1] take the start of the partial kernel
// and the end of the last norm kernel, ev[2] / ev[3] the update's start / end.
int launch_step(float *w, const float *g, float *m, float *v, int64_t n, float clip,
                const StepScalars &h, Workspace *ws, hipStream_t stream, hipEvent_t *ev) {
    hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
    const uintptr_t wa = reinterpret_cast<uintptr_t>(w), ga = reinterpret_cast<uintptr_t>(g);
    const uintptr_t ma = reinterpret_cast<uintptr_t>(m), va = reinterpret_cast<uintptr_t>(v);
    const int head = ((ga | ma | va) & 3u) == 0 ? head_of(w, n) : -1;
    if (head >= 0) {
        const bool fold = fold_final(n);
        if (fold) {
            launch_partial(g, n, h.gscale, ws, stream, ev ? ev[0] : nullptr,
                           ev ? ev[1] : nullptr);
        } else {
            const int rc = launch_norm(g, n, h.gscale, clip, ws, stream, ev);
            if (rc != RCS_OK) return rc;
        }
        UpdateLaunch a;
        a.nb = n - head;  // elements from w's boundary on
        a.grid = dim3((unsigned)(((a.nb >> 2) + kUpdThreads - 1) / kUpdThreads));
        a.w = reinterpret_cast<f32x4 *>(w + head);
        a.g = g + head;
        a.m = m + head;
        a.v = v + head;
        a.head = head;
        a.fold = fold;
        a.partials = ws->partials;
        a.nparts = norm_blocks(n);
        a.clip = clip;
        a.sc = ws->scalars;
        a.h = h;
        a.stream = stream;
        a.e2 = e2;
        a.e3 = e3;
        const uintptr_t ph = wa & 15u;
        const int mask = ((ga & 15u) == ph ? 4 : 0) | ((ma & 15u) == ph ? 2 : 0) |
                         ((va & 15u) == ph ? 1 : 0);
        switch (mask) {
            case 7: launch_update<true, true, true>(a); break;
            case 6: launch_update<true, true, false>(a); break;
            case 5: launch_update<true, false, true>(a); break;
            case 4: launch_update<true, false, false>(a); break;
            case 3: launch_update<false, true, true>(a); break;
            case 2: launch_update<false, true, false>(a); break;
            case 1: launch_update<false, false, true>(a); break;
            default: launch_update<false, false, false>(a); break;
        }
    } else {
        const int rc = launch_norm(g, n, h.gscale, clip, ws, stream, ev);
        if (rc != RCS_OK) return rc;
        int64_t blocks = (n + kUpdThreads - 1) / kUpdThreads;
        if (blocks > 65536) blocks = 65536;
        hipExtLaunchKernelGGL(adamw_update_scalar, dim3((unsigned)blocks), dim3(kUpdThreads), 0,
                              stream, e2, e3, 0, w, g, m, v, n, (const ClipScalars *)ws->scalars,
                              h);
    }
    return hipGetLastError() == hipSuccess ? RCS_OK : RCS_EHIP;
}

void put_le32(unsigned char *p, int32_t x) {
    const uint32_t u = (uint32_t)x;
    for (int k = 0; k < 4; ++k) p[k] = (unsigned char)((u >> (8 * k)) & 0xffu);
}

int32_t get_le32(const unsigned char *p) {
    uint32_t u = 0;
    for (int k = 0; k < 4; ++k) u |= (uint32_t)p[k] << (8 * k);
    return (int32_t)u;
}

bool valid_n(int64_t n) { return n >= 1 && n <= RCS_MAX_N; }

}  // namespace

void rcs_snapshot_forget(int dev, const void *snapshot) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_snap.find(std::make_pair(dev, snapshot));
    if (it == g_snap.end()) return;
    (void)hipEventDestroy(it->second.ready);
    (void)hipEventDestroy(it->second.copied);
    g_snap.erase(it);
}

// ---------------------------------------------------------------- C ABI

extern "C" {

const char *rcs_strerror(int status) {
    switch (status) {
        case RCS_OK: return "ok";
        case RCS_EINVAL: return "invalid argument (null pointer, bad size or scalar, or not device memory)";
        case RCS_ESIZE: return "size mismatch (buffer is not 8 + 12 n bytes, or an array is shorter than n)";
        case RCS_EHEADER: return "step file header rejected (n <= 0, step < 0 or n differs from the expected n)";
        case RCS_EHIP: return "HIP launch, copy or allocation failed";
        case RCS_ENOMEM: return "workspace allocation failed";
        case RCS_EIO: return "file write, read or rename failed";
        case RCS_ENOENT: return "no such file, or no valid step file in the directory";
        default: return "unknown status";
    }
}

int rcs_init(int device, hipStream_t stream) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return RCS_EHIP;
    if (hipSetDevice(device) != hipSuccess) {
        (void)hipGetLastError();
        return RCS_EINVAL;
    }
    Workspace *ws = nullptr;
    const int rc = get_workspace(stream, &ws);
    (void)hipSetDevice(prev);
    return rc;
}

int adamw_clip_step(float *w, const float *g, float *m, float *v, int64_t n, int32_t t, float lr,
                    float wd, float clip, hipStream_t stream) {
    return adamw_clip_step_accum(w, g, m, v, n, t, lr, wd, clip, 1.0f, stream);
}

int adamw_clip_step_accum(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                          float lr, float wd, float clip, float grad_scale, hipStream_t stream) {
    if (!valid_n(n) || t < 1) return RCS_EINVAL;
    if (!std::isfinite(grad_scale) || !(grad_scale > 0.0f)) return RCS_EINVAL;
    if (!std::isfinite(lr) || !std::isfinite(wd) || std::isnan(clip) || !(clip > 0.0f))
        return RCS_EINVAL;
    const int64_t bytes = 4 * n;
    int rc;
    if ((rc = check_device_range(w, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(g, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(m, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(v, bytes)) != RCS_OK) return rc;
    if (overlaps(w, g, bytes) || overlaps(w, m, bytes) || overlaps(w, v, bytes) ||
        overlaps(g, m, bytes) || overlaps(g, v, bytes) || overlaps(m, v, bytes))
        return RCS_EINVAL;
    Workspace *ws = nullptr;
    if ((rc = get_workspace(stream, &ws)) != RCS_OK) return rc;

    // a0: host scalars, float64 then one rounding each.
    StepScalars h;
    h.lr = lr;
    h.bc1 = (float)(1.0 - std::pow(0.9, (double)t));
    h.bc2 = (float)(1.0 - std::pow(0.999, (double)t));
    h.decay = (float)(1.0 - (double)lr * (double)wd);
    h.gscale = grad_scale;

    hipEvent_t *ev = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (g_prof.on && (g_prof.calls++ % g_prof.every) == 0 && g_prof.next < g_prof.max_records)
            ev = &g_prof.ev[4 * g_prof.next++];
    }
    rc = launch_step(w, g, m, v, n, clip, h, ws, stream, ev);
    if (rc == RCS_OK) ws->has_norm = true;
    return rc;
}

int grad_global_norm(const float *g, int64_t n, double *norm_out, hipStream_t stream) {
    if (!valid_n(n) || norm_out == nullptr) return RCS_EINVAL;
    int rc;
    if ((rc = check_device_range(g, 4 * n)) != RCS_OK) return rc;
    Workspace *ws = nullptr;
    if ((rc = get_workspace(stream, &ws)) != RCS_OK) return rc;
    if ((rc = launch_norm(g, n, 1.0f, INFINITY, ws, stream)) != RCS_OK) return rc;
    ws->has_norm = true;
    if (hipMemcpyAsync(norm_out, &ws->scalars->norm, sizeof(double), hipMemcpyDefault, stream) !=
        hipSuccess)
        return RCS_EHIP;
    return RCS_OK;
}

int grad_clip_inplace(float *g, int64_t n, float clip, hipStream_t stream) {
    if (!valid_n(n)) return RCS_EINVAL;
    if (std::isnan(clip) || !(clip > 0.0f)) return RCS_EINVAL;
    int rc;
    if ((rc = check_device_range(g, 4 * n)) != RCS_OK) return rc;
    Workspace *ws = nullptr;
    if ((rc = get_workspace(stream, &ws)) != RCS_OK) return rc;
    const int head = head_of(g, n);
    if (head >= 0) {  // partial, [final,] the vector scale kernel on the aligned body
        const int64_t nb = n - head;
        const dim3 grid((unsigned)(((nb >> 2) + kUpdThreads - 1) / kUpdThreads));
        f32x4 *g4 = reinterpret_cast<f32x4 *>(g + head);
        if (fold_final(n)) {
            launch_partial(g, n, 1.0f, ws, stream);
            hipLaunchKernelGGL(grad_scale_vec_fold, grid, dim3(kUpdThreads), 0, stream, g4, nb,
                               head, (const double *)ws->partials, norm_blocks(n), clip,
                               ws->scalars);
        } else {
            if ((rc = launch_norm(g, n, 1.0f, clip, ws, stream)) != RCS_OK) return rc;
            hipLaunchKernelGGL(grad_scale_vec, grid, dim3(kUpdThreads), 0, stream, g4, nb, head,
                               (const ClipScalars *)ws->scalars);
        }
    } else {  // g not 4-byte aligned or too short: partial, final, scalar scale
        if ((rc = launch_norm(g, n, 1.0f, clip, ws, stream)) != RCS_OK) return rc;
        int64_t blocks = (n + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(grad_scale_scalar, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                           n, (const ClipScalars *)ws->scalars);
    }
    if (hipGetLastError() != hipSuccess) return RCS_EHIP;
    ws->has_norm = true;
    return RCS_OK;
}

int grad_zero(float *g, int64_t n, hipStream_t stream) {
    if (!valid_n(n)) return RCS_EINVAL;
    int rc;
    if ((rc = check_device_range(g, 4 * n)) != RCS_OK) return rc;
    const int head = head_of(g, n);
    if (head >= 0) {
        const int64_t nb = n - head;
        const dim3 grid((unsigned)(((nb >> 2) + kZeroThreads - 1) / kZeroThreads));
        hipLaunchKernelGGL(grad_zero_vec, grid, dim3(kZeroThreads), 0, stream,
                           reinterpret_cast<f32x4 *>(g + head), nb, head);
    } else {
        int64_t blocks = (n + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(grad_zero_scalar, dim3((unsigned)blocks), dim3(256), 0, stream, g, n);
    }
    return hipGetLastError() == hipSuccess ? RCS_OK : RCS_EHIP;
}

int last_grad_norm(hipStream_t stream, double *norm_out) {
    if (norm_out == nullptr) return RCS_EINVAL;
    Workspace *ws = nullptr;
    int rc;
    if ((rc = get_workspace(stream, &ws)) != RCS_OK) return rc;
    if (!ws->has_norm) return RCS_EINVAL;
    if (hipMemcpyAsync(norm_out, &ws->scalars->norm, sizeof(double), hipMemcpyDefault, stream) !=
        hipSuccess)
        return RCS_EHIP;
    return RCS_OK;
}

int64_t ckpt_bytes(int64_t n) { return valid_n(n) ? 8 + 12 * n : -1; }

int ckpt_pack(int32_t step, int64_t n, const float *w, const float *m, const float *v,
              void *host_buf, int64_t buf_bytes, hipStream_t stream) {
    if (!valid_n(n) || step < 0 || host_buf == nullptr) return RCS_EINVAL;
    if (buf_bytes != ckpt_bytes(n)) return RCS_ESIZE;
    const int64_t bytes = 4 * n;
    int rc;
    if ((rc = check_device_range(w, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(m, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(v, bytes)) != RCS_OK) return rc;
    unsigned char *b = static_cast<unsigned char *>(host_buf);
    put_le32(b, step);
    put_le32(b + 4, (int32_t)n);
    if (hipMemcpyAsync(b + 8, w, bytes, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(b + 8 + bytes, m, bytes, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(b + 8 + 2 * bytes, v, bytes, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return RCS_EHIP;
    return RCS_OK;
}

int ckpt_unpack(const void *host_buf, int64_t buf_bytes, int64_t n_expected, int32_t *step_out,
                float *w, float *m, float *v, hipStream_t stream) {
    if (host_buf == nullptr || step_out == nullptr || !valid_n(n_expected)) return RCS_EINVAL;
    if (buf_bytes < 8) return RCS_ESIZE;
    const unsigned char *b = static_cast<const unsigned char *>(host_buf);
    const int32_t step = get_le32(b);
    const int32_t n = get_le32(b + 4);
    if (n <= 0 || step < 0) return RCS_EHEADER;
    if ((int64_t)n != n_expected) return RCS_EHEADER;
    if (buf_bytes != 8 + 12 * (int64_t)n) return RCS_ESIZE;
    const int64_t bytes = 4 * (int64_t)n;
    int rc;
    if ((rc = check_device_range(w, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(m, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(v, bytes)) != RCS_OK) return rc;
    if (hipMemcpyAsync(w, b + 8, bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipMemcpyAsync(m, b + 8 + bytes, bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipMemcpyAsync(v, b + 8 + 2 * bytes, bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
        return RCS_EHIP;
    *step_out = step;
    return RCS_OK;
}

int64_t ckpt_snapshot_bytes(int64_t n) { return valid_n(n) ? 12 * n : -1; }

int ckpt_pack_async(int32_t step, int64_t n, const float *w, const float *m, const float *v,
                    float *snapshot, int64_t snapshot_bytes, void *host_buf, int64_t buf_bytes,
                    hipStream_t compute_stream, hipStream_t copy_stream) {
    if (!valid_n(n) || step < 0 || host_buf == nullptr) return RCS_EINVAL;
    if (buf_bytes != ckpt_bytes(n) || snapshot_bytes != 12 * n) return RCS_ESIZE;
    const int64_t bytes = 4 * n;
    int rc;
    if ((rc = check_device_range(w, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(m, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(v, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(snapshot, 3 * bytes)) != RCS_OK) return rc;
    if (overlaps(snapshot, w, 3 * bytes) || overlaps(snapshot, m, 3 * bytes) ||
        overlaps(snapshot, v, 3 * bytes) || overlaps(w, snapshot, bytes) ||
        overlaps(m, snapshot, bytes) || overlaps(v, snapshot, bytes))
        return RCS_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RCS_EHIP;
    SnapshotSync *ss = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        SnapshotSync &e = g_snap[std::make_pair(dev, (const void *)snapshot)];
        if (e.ready == nullptr) {
            if (hipEventCreateWithFlags(&e.ready, hipEventDisableTiming) != hipSuccess ||
                hipEventCreateWithFlags(&e.copied, hipEventDisableTiming) != hipSuccess) {
                (void)hipGetLastError();
                return RCS_EHIP;
            }
        }
        ss = &e;
    }
    // the snapshot must not be overwritten while an earlier copy still reads it
    bool pending = false;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        pending = ss->pending;
    }
    if (pending && hipStreamWaitEvent(compute_stream, ss->copied, 0) != hipSuccess)
        return RCS_EHIP;
    if (n % 4 == 0 && aligned16(w) && aligned16(m) && aligned16(v) && aligned16(snapshot)) {
        const int64_t total = 3 * (n >> 2);
        const int64_t blocks = (total + kSnapThreads - 1) / kSnapThreads;  // one vector per lane
        hipLaunchKernelGGL(ckpt_snapshot_vec, dim3((unsigned)blocks), dim3(kSnapThreads), 0,
                           compute_stream,
                           reinterpret_cast<const f32x4 *>(w), reinterpret_cast<const f32x4 *>(m),
                           reinterpret_cast<const f32x4 *>(v), reinterpret_cast<f32x4 *>(snapshot),
                           n >> 2);
    } else {
        int64_t blocks = (3 * n + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(ckpt_snapshot_scalar, dim3((unsigned)blocks), dim3(256), 0,
                           compute_stream, w, m, v, snapshot, n);
    }
    if (hipGetLastError() != hipSuccess) return RCS_EHIP;
    if (hipEventRecord(ss->ready, compute_stream) != hipSuccess ||
        hipStreamWaitEvent(copy_stream, ss->ready, 0) != hipSuccess)
        return RCS_EHIP;
    unsigned char *b = static_cast<unsigned char *>(host_buf);
    put_le32(b, step);
    put_le32(b + 4, (int32_t)n);
    if (hipMemcpyAsync(b + 8, snapshot, 3 * bytes, hipMemcpyDeviceToHost, copy_stream) !=
            hipSuccess ||
        hipEventRecord(ss->copied, copy_stream) != hipSuccess)
        return RCS_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    ss->pending = true;
    return RCS_OK;
}

int ckpt_pack_wait(const float *snapshot) {
    if (snapshot == nullptr) return RCS_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RCS_EHIP;
    hipEvent_t e = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_snap.find(std::make_pair(dev, (const void *)snapshot));
        if (it == g_snap.end() || !it->second.pending) return RCS_OK;
        e = it->second.copied;
    }
    return hipEventSynchronize(e) == hipSuccess ? RCS_OK : RCS_EHIP;
}

int rcs_profile_enable(int on, int max_records, int every) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.on = false;
    g_prof.next = 0;
    g_prof.calls = 0;
    g_prof.max_records = 0;
    if (!on) return RCS_OK;
    if (max_records < 1 || max_records > (1 << 20) || every < 1) return RCS_EINVAL;
    g_prof.every = every;
    g_prof.ev.resize((size_t)4 * max_records);
    for (auto &e : g_prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            (void)hipGetLastError();
            return RCS_EHIP;
        }
    }
    g_prof.max_records = max_records;
    g_prof.on = true;
    return RCS_OK;
}

int rcs_profile_read(double *norm_ms_total, double *update_ms_total, int64_t *steps) {
    if (!norm_ms_total || !update_ms_total || !steps) return RCS_EINVAL;
    std::vector<hipEvent_t> ev;
    {  // copy the handles; wait on them without holding the library lock
        std::lock_guard<std::mutex> lk(g_mu);
        ev.assign(g_prof.ev.begin(), g_prof.ev.begin() + 4 * (size_t)g_prof.next);
    }
    double a = 0.0, b = 0.0;
    for (size_t i = 0; i + 3 < ev.size(); i += 4) {
        if (hipEventSynchronize(ev[i + 3]) != hipSuccess) return RCS_EHIP;
        float x = 0.f, y = 0.f;
        if (hipEventElapsedTime(&x, ev[i], ev[i + 1]) != hipSuccess ||
            hipEventElapsedTime(&y, ev[i + 2], ev[i + 3]) != hipSuccess)
            return RCS_EHIP;
        a += x;
        b += y;
    }
    *norm_ms_total = a;
    *update_ms_total = b;
    *steps = (int64_t)(ev.size() / 4);
    return RCS_OK;
}

int rcs_fp32_div_sqrt_probe(const float *a, const float *b, float *q, float *r, int64_t n,
                            hipStream_t stream) {
    if (n < 1 || n > RCS_MAX_N) return RCS_EINVAL;
    const int64_t bytes = 4 * n;
    int rc;
    if ((rc = check_device_range(a, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(b, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(q, bytes)) != RCS_OK) return rc;
    if ((rc = check_device_range(r, bytes)) != RCS_OK) return rc;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fp32_div_sqrt_probe, dim3((unsigned)blocks), dim3(256), 0, stream, a, b, q,
                       r, n);
    return hipGetLastError() == hipSuccess ? RCS_OK : RCS_EHIP;
}

}  // extern "C"

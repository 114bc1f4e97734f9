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
//     keep the vector kernels: block 0 takes the 0-63 elements before the
//     anchor array's next 256-byte boundary one per lane (the anchor is w or
//     m, whichever shares its line phase with more of the written arrays),
//     and the waves stream whole cache lines from there; an array at another
//     16-byte phase is still read and written in aligned 16-byte vectors,
//     shifted by whole floats across neighbouring lanes (adamw_update_mixed).
//     The lines a wave shares with its neighbour (an array whose span does not
//     start on a line) are read and written with cache-retaining accesses.
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

namespace {

constexpr int kWave = 64;
// Contiguous regions of the vectors the update streams at once: block b
// works in region b % kRegions. Blocks are dispatched round-robin over the
// chip's 8 XCDs, so with 8 regions each XCD streams its own contiguous eighth
// of w, g, m, v. With one-wave blocks, over 14 buffer placements on one box
// the step took 605.0-619.3 us (mean 611.0) with 8 regions against
// 612.9-631.1 (617.5) with 4 (6 placements on another box: means 609.9 and
// 608.0; 2, 1, 16 and 32 regions were slower).
constexpr int64_t kRegions = 8;
// Largest n whose step folds the final norm reduction into the update kernel
// (measured: folding saves 1.7-2.4 us per step up to 8,388,608 elements and
// costs 4.8 us at 16,777,216 and 23 us at 124,356,864).
constexpr int64_t kFoldMaxN = 8388608;
// Bytes at the end of g that the norm pass reads with ordinary (cache-
// allocating) loads so that the update, which reads g again right after,
// finds them in the last-level cache; the rest is read with streaming loads.
constexpr int64_t kNormCachedTailBytes = 320LL << 20;
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
constexpr int kUpdThreads = 64;
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
    return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void st_stream(T *p, T x) {
    __builtin_nontemporal_store(x, p);
}

// Cache-retaining accesses for the 128-byte lines a wave shares with a
// neighbouring wave. A wave's span of one array is 1 KiB from the vector its
// lane 0 handles; when that array's span does not start on a line boundary,
// its first and last lines are read and written by two waves. Streaming
// accesses there make each wave fetch the whole line and write its part of
// it on its own; these loads and stores (relaxed workgroup-scope atomics of 8
// or 4 bytes, which the compiler emits as ordinary loads and stores with the
// sc0 cache policy, no ordering implied) keep the line in L2, so the second
// wave's read hits it and the two parts meet there. The neighbouring waves
// run on the same XCD (one region per XCD). Measured at the ANDREA-120M size,
// same buffers, one process: w 16 bytes past the others (so g, m and v
// 112 bytes into a line) 721 us/step streaming, 627 with these and the anchor
// chosen by line phase; v alone 16 bytes off 641 against 625; a 616-621 us
// aligned step.
__device__ __forceinline__ f32x4 ld_keep(const f32x4 *p) {
    uint64_t *q = reinterpret_cast<uint64_t *>(const_cast<f32x4 *>(p));
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                 __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

__device__ __forceinline__ float ld_keep1(const float *p) {
    uint32_t *q = reinterpret_cast<uint32_t *>(const_cast<float *>(p));
    return __uint_as_float(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

__device__ __forceinline__ void st_keep(f32x4 *p, f32x4 x) {
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    const uint64_t a = (uint64_t)__float_as_uint(x.x) | ((uint64_t)__float_as_uint(x.y) << 32);
    const uint64_t b = (uint64_t)__float_as_uint(x.z) | ((uint64_t)__float_as_uint(x.w) << 32);
    __hip_atomic_store(q, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(q + 1, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Whether the 16-byte vector at p lies in a line its wave shares with a
// neighbouring wave. a0: the vector the wave's lane 0 handles in the same
// array. split: the array is read in shifted vectors, so the vector at a0 is
// split between two waves whatever its line phase.
__device__ __forceinline__ bool shared_line(const void *p, const void *a0, bool split) {
    const uintptr_t l = reinterpret_cast<uintptr_t>(p) >> 7;
    const uintptr_t s = reinterpret_cast<uintptr_t>(a0);
    return (split || (s & 127u) != 0) && (l == (s >> 7) || l == ((s + 1024u) >> 7));
}

// An array at another 16-byte phase than the anchor (the array whose body
// starts on the 256-byte boundary): its body xb (the element matching the
// anchor's first body element) lies q = 1-3 floats past a 16-byte boundary,
// so lane i's four elements xb[4i .. 4i+3] straddle two aligned
// vectors of the array. Every access stays a 16-byte aligned one: each lane
// loads the aligned vector holding its first element (its positions q..3 are
// the lane's first 4 - q elements) and takes the rest (positions 0..q-1 of the
// next aligned vector) from the next lane's load through a cross-lane shift;
// stores work the other way round, each lane writing the aligned vector that
// holds its first element from the previous lane's last q elements and its
// own first 4 - q. At the wave's edges, where the neighbouring lane is in
// another wave, and at the ends of the body, the missing elements are loaded
// or stored one by one (`own`, `lane0`, `first`). Any element a lane uses was
// read by itself or by the next lane of its own wave before that wave's
// stores; other waves only ever write positions this lane discards.

template <bool KEEP>
__device__ __forceinline__ float ld_edge1(const float *p) {
    if constexpr (KEEP) return ld_keep1(p);
    else return ld_stream(p);
}

// xb[4i .. 4i+3] for vector ic (i clamped to the body). first: ic is vector 0
// and the aligned vector holding xb[0] starts before the array (head < q):
// the lane's elements of it are read one by one. own: the next lane does not
// hold the next aligned vector (this is the wave's last lane or the body's
// last vector): positions 0..q-1 of it are read one by one. KEEP: the lines
// shared with the neighbouring wave (always two: the vector at the wave's
// start is split between the waves) are read with cache-retaining loads,
// for the update, whose neighbouring waves run on one XCD; the snapshot
// kernel, whose neighbouring blocks do not, streams them. Every lane of the
// wave must call this (cross-lane shifts).
template <bool KEEP>
__device__ __forceinline__ f32x4 ld_shifted(const float *__restrict__ xb, int q, int64_t ic,
                                            bool first, bool own) {
    f32x4 a;
    if (first) {
        a = f32x4{0.f, 0.f, 0.f, 0.f};
        a.w = ld_edge1<KEEP>(xb + 3 - q);
        if (q <= 2) a.z = ld_edge1<KEEP>(xb + 2 - q);
        if (q == 1) a.y = ld_edge1<KEEP>(xb);
    } else {
        const f32x4 *base = reinterpret_cast<const f32x4 *>(xb - q);
        const int64_t i0 = ic - (int64_t)(threadIdx.x & (kWave - 1));
        a = KEEP && shared_line(base + ic, base + i0, true) ? ld_keep(base + ic)
                                                            : ld_stream(base + ic);
    }
    float b0 = __shfl_down(a.x, 1, kWave);
    float b1 = __shfl_down(a.y, 1, kWave);
    float b2 = __shfl_down(a.z, 1, kWave);
    if (own) {
        const float *p = xb + 4 * ic + 4 - q;
        b0 = ld_edge1<KEEP>(p);
        if (q >= 2) b1 = ld_edge1<KEEP>(p + 1);
        if (q == 3) b2 = ld_edge1<KEEP>(p + 2);
    }
    return q == 1 ? f32x4{a.y, a.z, a.w, b0} : q == 2 ? f32x4{a.z, a.w, b0, b1}
                                                     : f32x4{a.w, b0, b1, b2};
}

// Writes r to xb[4i .. 4i+3] when active (i < n4). lane0: the wave's first
// lane, whose previous lane is in another wave: its first 4 - q elements are
// written one by one. own: as for ld_shifted, its last q elements are written
// one by one. Those one-by-one writes fill part of a 16-byte vector that a
// neighbouring wave fills the rest of; they are plain (cache-retained) stores
// so that the two halves meet in the L2 cache rather than reaching memory as
// partial writes (measured at the ANDREA-120M size with only v off w's phase:
// 633-636 us/step against 650-656 with streaming stores there, 614-620 with v
// at w's phase). Every lane of the wave must call this (cross-lane shifts).
__device__ __forceinline__ void st_shifted(float *__restrict__ xb, int q, int64_t i, f32x4 r,
                                           bool active, bool lane0, bool own) {
    const float p1 = __shfl_up(r.y, 1, kWave);
    const float p2 = __shfl_up(r.z, 1, kWave);
    const float p3 = __shfl_up(r.w, 1, kWave);
    if (!active) return;
    float *p = xb + 4 * i;
    if (!lane0) {
        const f32x4 x = q == 1 ? f32x4{p3, r.x, r.y, r.z}
                               : q == 2 ? f32x4{p2, p3, r.x, r.y} : f32x4{p1, p2, p3, r.x};
        st_stream(reinterpret_cast<f32x4 *>(xb - q) + i, x);
    } else {
        p[0] = r.x;
        if (q <= 2) p[1] = r.y;
        if (q == 1) p[2] = r.z;
    }
    if (own) {
        if (q == 3) {
            p[1] = r.y;
            p[2] = r.z;
        } else if (q == 2) {
            p[2] = r.z;
        }
        p[3] = r.w;
    }
}

// The chunk of the vectors block blockIdx.x works on: a bijection of
// [0, gridDim.x) that puts block b in contiguous region b % kRegions, at
// position b / kRegions. Blocks are dispatched round-robin over the XCDs, so
// each XCD streams its own regions, and neighbouring chunks (which share a
// cache line at their common edge when an array is off the body's phase) run
// on the same XCD and its L2.
__device__ __forceinline__ int64_t chunk_of_block() {
    const int64_t nblk = gridDim.x, b = blockIdx.x;
    const int64_t k = kRegions, q = nblk / k, r = nblk % k, x = b % k, j = b / k;
    return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// Phases of w, g, m, v relative to the 16-byte aligned body, in floats
// (0 = at the body's phase).
struct Phases {
    int w, g, m, v;
};

// Four elements of an array's body per lane: an aligned vector (VEC: the
// array is at the body's 16-byte phase) or a shifted one.
// LINES: some array's span may not start on a line (shared_line is checked);
// false when every array's body starts on a line boundary.
template <bool VEC, bool LINES>
__device__ __forceinline__ f32x4 load4(const float *__restrict__ xb, int q, int64_t ic,
                                       int head, bool own) {
    if constexpr (VEC) {
        const f32x4 *x4 = reinterpret_cast<const f32x4 *>(xb);
        if constexpr (!LINES) return ld_stream(x4 + ic);
        const int64_t i0 = ic - (int64_t)(threadIdx.x & (kWave - 1));
        return shared_line(x4 + ic, x4 + i0, false) ? ld_keep(x4 + ic) : ld_stream(x4 + ic);
    } else {
        return ld_shifted<true>(xb, q, ic, ic == 0 && head < q, own);
    }
}

template <bool VEC, bool LINES>
__device__ __forceinline__ void store4(float *__restrict__ xb, int q, int64_t i, f32x4 r,
                                       bool active, bool lane0, bool own) {
    if constexpr (VEC) {
        if (active) {
            f32x4 *x4 = reinterpret_cast<f32x4 *>(xb);
            const int64_t i0 = i - (int64_t)(threadIdx.x & (kWave - 1));
            if (LINES && shared_line(x4 + i, x4 + i0, false)) st_keep(x4 + i, r);
            else st_stream(x4 + i, r);
        }
    } else {
        st_shifted(xb, q, i, r, active, lane0, own);
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
// w, g, m, v point `head` (0-63) elements past the arrays' starts, where the
// body begins; the anchor array (w or m, the host's choice) has its body on a
// 16-byte (normally 256-byte) boundary, and WV, GV, MV, VV say which
// arrays share its 16-byte phase (aligned vectors) rather than lying ph.*
// floats past it (shifted vectors; kUpdThreads is one wave). LINES as for
// load4 (always true when an array is shifted).
template <bool FOLD, bool LINES, bool WV, bool GV, bool MV, bool VV>
__device__ __forceinline__ void update_body(float *__restrict__ wf, const float *__restrict__ gf,
                                            float *__restrict__ mf, float *__restrict__ vf,
                                            int64_t n, int head, Phases ph,
                                            const double *__restrict__ partials, int nparts,
                                            float clip, ClipScalars *__restrict__ sc,
                                            const StepScalars &h, double *lds) {
    const int64_t n4 = n >> 2;
    const int64_t i = chunk_of_block() * kUpdThreads + threadIdx.x;
    double xp[kPartsPerLane];
    if constexpr (FOLD) load_partials(partials, nparts, xp);
    const int64_t ic = i < n4 ? i : n4 - 1;
    const int lane = (int)threadIdx.x & (kWave - 1);
    const bool own = lane == kWave - 1 || ic == n4 - 1;
    f32x4 gr = load4<GV, LINES>(gf, ph.g, ic, head, own);
    f32x4 wr = load4<WV, LINES>(wf, ph.w, ic, head, own);
    f32x4 mr = load4<MV, LINES>(mf, ph.m, ic, head, own);
    f32x4 vr = load4<VV, LINES>(vf, ph.v, ic, head, own);
    ClipScalars cs;
    if constexpr (FOLD) {
        cs = final_reduce(xp, nparts, clip, lds);
        if (blockIdx.x == 0 && threadIdx.x == 0) *sc = cs;
    } else {
        cs = *sc;
    }
    if (!cs.apply) return;
    const float s = cs.scale;
    const bool active = i < n4;
    if (active) adamw_vec4(wr, gr, mr, vr, s, h);
    const bool lane0 = lane == 0;
    store4<WV, LINES>(wf, ph.w, i, wr, active, lane0, own);
    store4<MV, LINES>(mf, ph.m, i, mr, active, lane0, own);
    store4<VV, LINES>(vf, ph.v, i, vr, active, lane0, own);
    // block 0: the head elements before the body (indices -head .. -1);
    // the last block: the n % 4 after the last vector
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

// a3 after grad_norm_final, all four arrays at one 16-byte phase. w, g, m, v
// point `head` (0-63) elements past the arrays' starts, at 16-byte
// boundaries; n counts from there. LINES: some array's body is not on a
// 128-byte line boundary.
template <bool LINES>
__global__ __launch_bounds__(kUpdThreads) void adamw_update_vec(
    float *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, const ClipScalars *__restrict__ sc,
    StepScalars h) {
    update_body<false, LINES, true, true, true, true>(w, g, m, v, n, head, Phases{0, 0, 0, 0},
                                                      nullptr, 0, 0.0f,
                                                      const_cast<ClipScalars *>(sc), h, nullptr);
}

// a2 + a3 in one kernel (small n).
template <bool LINES>
__global__ __launch_bounds__(kUpdThreads) void adamw_update_vec_fold(
    float *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, const double *__restrict__ partials, int nparts,
    float clip, ClipScalars *__restrict__ sc_out, StepScalars h) {
    __shared__ double lds[kUpdThreads / kWave];
    update_body<true, LINES, true, true, true, true>(w, g, m, v, n, head, Phases{0, 0, 0, 0},
                                                     partials, nparts, clip, sc_out, h, lds);
}

// The same two kernels when the arrays lie at more than one 16-byte phase
// (e.g. w a view into a flat parameter buffer at an odd offset, m and v fresh
// allocations): the arrays at the anchor's phase take aligned 16-byte
// vectors, the others shifted ones.
template <bool WV, bool GV, bool MV, bool VV>
__global__ __launch_bounds__(kUpdThreads) void adamw_update_mixed(
    float *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, Phases ph, const ClipScalars *__restrict__ sc,
    StepScalars h) {
    update_body<false, true, WV, GV, MV, VV>(w, g, m, v, n, head, ph, nullptr, 0, 0.0f,
                                             const_cast<ClipScalars *>(sc), h, nullptr);
}

template <bool WV, bool GV, bool MV, bool VV>
__global__ __launch_bounds__(kUpdThreads) void adamw_update_mixed_fold(
    float *__restrict__ w, const float *__restrict__ g, float *__restrict__ m,
    float *__restrict__ v, int64_t n, int head, Phases ph, const double *__restrict__ partials,
    int nparts, float clip, ClipScalars *__restrict__ sc_out, StepScalars h) {
    __shared__ double lds[kUpdThreads / kWave];
    update_body<true, true, WV, GV, MV, VV>(w, g, m, v, n, head, ph, partials, nparts, clip,
                                            sc_out, h, lds);
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

// The pages' third clip kernel on its own, for callers that need the clipped
// gradient itself: g *= s in place (skipped when the norm is not finite). Same
// float32 product as the update's g * s. g points `head` (0-63) elements past
// the array's start, at a 16-byte boundary, and n counts from there. Lanes
// past the end re-read the last vector and discard it (the host guarantees
// n >= 4); block 0 also scales the head elements and the last block the n % 4
// trailing ones. FOLD as in update_body: the record from
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
// blockIdx.y picks the array (w, m, v) and its place snap + y n. Each part is
// written in aligned 16-byte vectors from its next 256-byte boundary on
// (ph.h*: the 0-63 elements before it, or 0-3 to the next 16-byte boundary
// when fewer than 4 would follow; block 0 copies those one per lane, and the
// 0-3 after the last vector), so its waves write whole cache lines (with the
// snapshot buffer one float off a 16-byte boundary: 507-509 us at the
// ANDREA-120M size, against 534 with 16-byte heads). A source at another
// 16-byte phase than its destination (an n not divisible by 4 puts the m and
// v parts there, and so can a view) is read in aligned 16-byte vectors
// shifted across lanes, as the update reads arrays off the anchor's phase
// (ld_shifted); ph.q* is that phase in floats. One vector per lane, one wave
// per block (452-463 us against 466-483 us with 256 lanes for the 1.49 GB
// snapshot at the ANDREA-120M size), blocks in address order (the update's
// XCD region mapping measured no better here). The host guarantees a head
// for every part and 4-byte aligned pointers.
constexpr int kSnapThreads = 64;
static_assert(kSnapThreads == kWave, "the shifted loads and the 0-63 element heads assume one wave");
struct SnapPhases {
    int qw, qm, qv;  // source phase relative to the destination's body, floats
    int hw, hm, hv;  // elements before the destination's body
};
__global__ __launch_bounds__(kSnapThreads) void ckpt_snapshot_vec(const float *__restrict__ w,
                                                                  const float *__restrict__ m,
                                                                  const float *__restrict__ v,
                                                                  float *__restrict__ snap,
                                                                  int64_t n, SnapPhases ph) {
    const int y = blockIdx.y;
    const float *src = y == 0 ? w : y == 1 ? m : v;
    float *dst = snap + (int64_t)y * n;
    const int q = y == 0 ? ph.qw : y == 1 ? ph.qm : ph.qv;
    const int head = y == 0 ? ph.hw : y == 1 ? ph.hm : ph.hv;
    const int64_t nb = n - head;
    const int64_t nb4 = nb >> 2;
    const int64_t i = (int64_t)blockIdx.x * kSnapThreads + threadIdx.x;
    if (nb4 > 0 && (int64_t)blockIdx.x * kSnapThreads < nb4) {  // uniform per block
        const int64_t ic = i < nb4 ? i : nb4 - 1;
        const float *sb = src + head;
        f32x4 x;
        if (q == 0)
            x = ld_stream(reinterpret_cast<const f32x4 *>(sb) + ic);
        else
            x = ld_shifted<false>(sb, q, ic, ic == 0 && head < q,
                                  threadIdx.x == kWave - 1 || ic == nb4 - 1);
        if (i < nb4) st_stream(reinterpret_cast<f32x4 *>(dst + head) + i, x);
    }
    if (blockIdx.x == 0) {  // each part's head and tail
        if ((int)threadIdx.x < head) dst[threadIdx.x] = src[threadIdx.x];
        if ((int)threadIdx.x < (int)(nb & 3)) {
            const int64_t k = head + (nb4 << 2) + threadIdx.x;
            dst[k] = src[k];
        }
    }
}

// The same copy for pointers off a 4-byte boundary, or parts too short for
// a head and one vector.
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

// Device scratch of adamw_clip_step_noalloc, for callers that cannot allocate:
// the norm pass's per-block float64 partial sums (at most kNormMaxBlocks of
// them, 2 KiB, whatever n is) followed by the clip record. Each GPU holds one
// copy until the process ends. Host code never passes this name to a kernel
// (on the host it only stands in for the symbol): it takes the copy's device
// address once per device with hipGetSymbolAddress and passes that.
constexpr size_t kScratchBytes = 4096;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

#include <thread>
#include <tuple>

#include "rcs_internal.h"

namespace {

// Device memory the norm kernels write: the per-block partial sums and the
// clip record the update reads.
struct NormBuffers {
    double *partials = nullptr;      // kNormMaxBlocks float64
    ClipScalars *scalars = nullptr;  // one record
};

struct Workspace : NormBuffers {
    std::atomic<bool> has_norm{false};
};

std::mutex g_mu;
// Keyed by device and stream; hipStreamPerThread names a different stream in
// every host thread, so under that handle the thread is part of the key.
using WsKey = std::tuple<int, hipStream_t, std::thread::id>;
std::map<WsKey, Workspace> g_ws;

// Device address of each GPU's copy of `scratch` (null until looked up).
constexpr int kMaxDevices = 256;
std::atomic<char *> g_scratch_addr[kMaxDevices];
constexpr size_t kScratchRecordOffset = (size_t)kNormMaxBlocks * sizeof(double);
static_assert(kScratchRecordOffset % alignof(ClipScalars) == 0, "record alignment");
static_assert(kScratchRecordOffset + sizeof(ClipScalars) <= kScratchBytes, "scratch size");

// The address of device dev's copy of `scratch`; dev must be the current
// device. Looked up once per device (rcs_init, else the first
// adamw_clip_step_noalloc on it); no allocation.
int scratch_address(int dev, char **out) {
    if (dev < 0 || dev >= kMaxDevices) return RCS_EINVAL;
    char *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lk(g_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void *q = nullptr;
            if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
                (void)hipGetLastError();
                return RCS_EHIP;
            }
            p = static_cast<char *>(q);
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RCS_OK;
}

// Per snapshot buffer: `ready` is recorded on the compute stream after the
// snapshot kernel, `copied` on the copy stream after the device-to-host copy.
struct SnapshotSync {
    hipEvent_t ready = nullptr;
    hipEvent_t copied = nullptr;
    bool pending = false;  // a copy out of this snapshot has been enqueued
};
std::map<std::pair<int, const void *>, SnapshotSync> g_snap;

// Read without the lock on every step; the records themselves are guarded.
std::atomic<bool> g_prof_on{false};
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

// The last (device, stream) a host thread used and its workspace; workspaces
// live until the process ends, so the pointer stays valid. Saves the map
// lookup under the library lock on every step of a training loop.
struct WsCache {
    int dev = -1;
    hipStream_t stream = nullptr;
    Workspace *ws = nullptr;
};
thread_local WsCache t_ws;

int get_workspace(hipStream_t stream, Workspace **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RCS_EHIP;
    if (t_ws.ws != nullptr && t_ws.dev == dev && t_ws.stream == stream) {
        *out = t_ws.ws;
        return RCS_OK;
    }
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
    t_ws.dev = dev;
    t_ws.stream = stream;
    t_ws.ws = &it->second;
    return RCS_OK;
}

// p must be device (or managed) memory of the current device and the range
// [p, p + bytes) must lie inside the allocation the runtime reports for p.
// That allocation is the runtime's own: an array carved by a sub-allocator out
// of a larger block passes as long as it ends inside that block, whatever its
// true length. Memory the runtime cannot report a range for (e.g. virtual-
// memory mappings) is accepted without the length check.
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

// Whether [a, a + a_bytes) and [b, b + b_bytes) share a byte.
bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes) {
    const char *x = static_cast<const char *>(a);
    const char *y = static_cast<const char *>(b);
    return x < y + b_bytes && y < x + a_bytes;
}

bool overlaps(const void *a, const void *b, int64_t bytes) { return overlaps(a, bytes, b, bytes); }

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

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
    const int64_t tail4 = kNormCachedTailBytes / 16;
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
void launch_partial(const float *g, int64_t n, float gscale, const NormBuffers *ws,
                    hipStream_t stream, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    const int head = head_of(g, n);
    hipExtLaunchKernelGGL(grad_norm_partial, dim3(norm_blocks(n)), dim3(kNormThreads), 0, stream,
                          ev0, ev1, 0, g, n, head, norm_nt_limit4(head >= 0 ? n - head : n),
                          gscale, ws->partials);
}

// a1 + a2. ev (optional, profiling): ev[0] takes the partial kernel's start,
// ev[1] the final kernel's end.
int launch_norm(const float *g, int64_t n, float gscale, float clip, const NormBuffers *ws,
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
bool fold_final(int64_t n) { return n <= kFoldMaxN; }

// Arguments of the update kernels after the norm kernels.
struct UpdateLaunch {
    dim3 grid;
    float *w;
    const float *g;
    float *m, *v;
    int64_t nb;
    int head;
    Phases ph;
    bool fold;
    bool lines;  // some array's body does not start on a 128-byte line
    const double *partials;
    int nparts;
    float clip;
    ClipScalars *sc;
    StepScalars h;
    hipStream_t stream;
    hipEvent_t e2, e3;
};

template <bool WV, bool GV, bool MV, bool VV>
void launch_update(const UpdateLaunch &a) {
    const dim3 block(kUpdThreads);
    if constexpr (WV && GV && MV && VV) {
        if (a.fold && a.lines)
            hipExtLaunchKernelGGL(adamw_update_vec_fold<true>, a.grid, block, 0, a.stream, a.e2,
                                  a.e3, 0, a.w, a.g, a.m, a.v, a.nb, a.head, a.partials, a.nparts,
                                  a.clip, a.sc, a.h);
        else if (a.fold)
            hipExtLaunchKernelGGL(adamw_update_vec_fold<false>, a.grid, block, 0, a.stream, a.e2,
                                  a.e3, 0, a.w, a.g, a.m, a.v, a.nb, a.head, a.partials, a.nparts,
                                  a.clip, a.sc, a.h);
        else if (a.lines)
            hipExtLaunchKernelGGL(adamw_update_vec<true>, a.grid, block, 0, a.stream, a.e2, a.e3,
                                  0, a.w, a.g, a.m, a.v, a.nb, a.head, (const ClipScalars *)a.sc,
                                  a.h);
        else
            hipExtLaunchKernelGGL(adamw_update_vec<false>, a.grid, block, 0, a.stream, a.e2, a.e3,
                                  0, a.w, a.g, a.m, a.v, a.nb, a.head, (const ClipScalars *)a.sc,
                                  a.h);
    } else {
        if (a.fold)
            hipExtLaunchKernelGGL(adamw_update_mixed_fold<WV, GV, MV, VV>, a.grid, block, 0,
                                  a.stream, a.e2, a.e3, 0, a.w, a.g, a.m, a.v, a.nb, a.head, a.ph,
                                  a.partials, a.nparts, a.clip, a.sc, a.h);
        else
            hipExtLaunchKernelGGL(adamw_update_mixed<WV, GV, MV, VV>, a.grid, block, 0, a.stream,
                                  a.e2, a.e3, 0, a.w, a.g, a.m, a.v, a.nb, a.head, a.ph,
                                  (const ClipScalars *)a.sc, a.h);
    }
}

// The anchor of the update's body among the written arrays w and m: each
// scores 2 for every written array (w, m, v) at its 128-byte line phase and 1
// for every one at its 16-byte phase, and the higher score wins (w on a tie).
// Arrays at the anchor's line phase stream whole lines; at its 16-byte phase
// only, they take aligned vectors with shared edge lines; otherwise shifted
// vectors. m wins only when v shares its 16-byte phase (its score can exceed
// w's only through v), so the anchor's phase always holds w, or m and v.
// 0 = w, 1 = m.
int anchor_of(uintptr_t wa, uintptr_t ma, uintptr_t va) {
    const uintptr_t o[3] = {wa & 127u, ma & 127u, va & 127u};
    int best = 0, best_score = -1;
    for (int a = 0; a < 2; ++a) {
        int score = 0;
        for (int x = 0; x < 3; ++x)
            score += (o[x] == o[a] ? 2 : 0) + ((o[x] & 15u) == (o[a] & 15u) ? 1 : 0);
        if (score > best_score) {
            best = a;
            best_score = score;
        }
    }
    return best;
}

// The whole step a1..a3. Vector form (all four arrays 4-byte aligned, at
// least 4 elements past the anchor's head): the partial kernel,
// [grad_norm_final,] the update kernel on the body from the anchor's next
// 256-byte boundary on, which also takes the head elements; arrays at the
// anchor's 16-byte phase are accessed as aligned 16-byte vectors, the others
// as shifted ones. Otherwise: partial, final, scalar update.
// ev (optional, profiling): ev[0] / ev[1] take the start of the partial kernel
// and the end of the last norm kernel, ev[2] / ev[3] the update's start / end.
int launch_step(float *w, const float *g, float *m, float *v, int64_t n, float clip,
                const StepScalars &h, const NormBuffers *ws, hipStream_t stream, hipEvent_t *ev) {
    hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
    const uintptr_t wa = reinterpret_cast<uintptr_t>(w), ga = reinterpret_cast<uintptr_t>(g);
    const uintptr_t ma = reinterpret_cast<uintptr_t>(m), va = reinterpret_cast<uintptr_t>(v);
    const int anchor = anchor_of(wa, ma, va);
    const float *anchor_ptr = anchor == 0 ? w : m;
    const int head = ((wa | ga | ma | va) & 3u) == 0 ? head_of(anchor_ptr, n) : -1;
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
        a.nb = n - head;  // elements from the body's boundary on
        a.grid = dim3((unsigned)(((a.nb >> 2) + kUpdThreads - 1) / kUpdThreads));
        a.w = w + head;
        a.g = g + head;
        a.m = m + head;
        a.v = v + head;
        a.head = head;
        a.fold = fold;
        a.lines = (((uintptr_t)a.w | (uintptr_t)a.g | (uintptr_t)a.m | (uintptr_t)a.v) & 127u) != 0;
        a.partials = ws->partials;
        a.nparts = norm_blocks(n);
        a.clip = clip;
        a.sc = ws->scalars;
        a.h = h;
        a.stream = stream;
        a.e2 = e2;
        a.e3 = e3;
        // each array's phase in floats past the 16-byte boundary where the body starts
        const uintptr_t hb = 4u * (uintptr_t)head;
        a.ph.w = (int)(((wa + hb) & 15u) >> 2);
        a.ph.g = (int)(((ga + hb) & 15u) >> 2);
        a.ph.m = (int)(((ma + hb) & 15u) >> 2);
        a.ph.v = (int)(((va + hb) & 15u) >> 2);
        const int mask = (a.ph.w == 0 ? 8 : 0) | (a.ph.g == 0 ? 4 : 0) | (a.ph.m == 0 ? 2 : 0) |
                         (a.ph.v == 0 ? 1 : 0);
        // the anchor is at phase 0: w (bit 8), or m together with v (bits 2 and 1)
        switch (mask) {
            case 15: launch_update<true, true, true, true>(a); break;
            case 14: launch_update<true, true, true, false>(a); break;
            case 13: launch_update<true, true, false, true>(a); break;
            case 12: launch_update<true, true, false, false>(a); break;
            case 11: launch_update<true, false, true, true>(a); break;
            case 10: launch_update<true, false, true, false>(a); break;
            case 9: launch_update<true, false, false, true>(a); break;
            case 8: launch_update<true, false, false, false>(a); break;
            case 7: launch_update<false, true, true, true>(a); break;
            case 3: launch_update<false, false, true, true>(a); break;
            default: return RCS_EINVAL;  // unreachable, as above
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

bool valid_n(int64_t n) { return n >= 1 && n <= RCS_MAX_N; }

// Host-side checks shared by the update entry points: sizes, scalars, every
// array inside one device allocation of the current device, g apart from
// w, m, v and those apart from each other.
int validate_step(float *w, const float *g, float *m, float *v, int64_t n, int32_t t, float lr,
                  float wd, float clip, float grad_scale) {
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
    return RCS_OK;
}

// a0: bias corrections and decay in float64, each rounded once to float32.
StepScalars host_scalars(int32_t t, float lr, float wd, float grad_scale) {
    StepScalars h;
    h.lr = lr;
    h.bc1 = (float)(1.0 - std::pow(0.9, (double)t));
    h.bc2 = (float)(1.0 - std::pow(0.999, (double)t));
    h.decay = (float)(1.0 - (double)lr * (double)wd);
    h.gscale = grad_scale;
    return h;
}

// A norm destination: pinned host memory, or 8 bytes of device memory of
// device dev.
int check_norm_out(const double *p, int dev) {
    hipPointerAttribute_t pa;
    if (hipPointerGetAttributes(&pa, p) != hipSuccess) {
        (void)hipGetLastError();
        return RCS_EINVAL;
    }
    if (pa.type == hipMemoryTypeHost) return RCS_OK;
    if (pa.type == hipMemoryTypeDevice && pa.device != dev) return RCS_EINVAL;
    return check_device_range(p, sizeof(double));
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
    int rc = get_workspace(stream, &ws);
    char *scr = nullptr;
    if (rc == RCS_OK) rc = scratch_address(device, &scr);
    (void)hipSetDevice(prev);
    return rc;
}

int adamw_clip_step(float *w, const float *g, float *m, float *v, int64_t n, int32_t t, float lr,
                    float wd, float clip, hipStream_t stream) {
    return adamw_clip_step_accum(w, g, m, v, n, t, lr, wd, clip, 1.0f, stream);
}

int adamw_clip_step_accum(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                          float lr, float wd, float clip, float grad_scale, hipStream_t stream) {
    int rc;
    if ((rc = validate_step(w, g, m, v, n, t, lr, wd, clip, grad_scale)) != RCS_OK) return rc;
    Workspace *ws = nullptr;
    if ((rc = get_workspace(stream, &ws)) != RCS_OK) return rc;
    const StepScalars h = host_scalars(t, lr, wd, grad_scale);
    hipEvent_t *ev = nullptr;
    if (g_prof_on.load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lk(g_mu);
        if (g_prof.on && (g_prof.calls++ % g_prof.every) == 0 && g_prof.next < g_prof.max_records)
            ev = &g_prof.ev[4 * g_prof.next++];
    }
    rc = launch_step(w, g, m, v, n, clip, h, ws, stream, ev);
    if (rc == RCS_OK) ws->has_norm = true;
    return rc;
}

int adamw_clip_step_noalloc(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                            float lr, float wd, float clip, double *norm_out,
                            hipStream_t stream) {
    int rc;
    if ((rc = validate_step(w, g, m, v, n, t, lr, wd, clip, 1.0f)) != RCS_OK) return rc;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RCS_EHIP;
    if (norm_out != nullptr && (rc = check_norm_out(norm_out, dev)) != RCS_OK) return rc;
    // every valid n fits: the norm pass never has more than kNormMaxBlocks blocks
    if ((size_t)norm_blocks(n) * sizeof(double) > kScratchRecordOffset) return RCS_ESIZE;
    char *base = nullptr;
    if ((rc = scratch_address(dev, &base)) != RCS_OK) return rc;
    NormBuffers nb;
    nb.partials = reinterpret_cast<double *>(base);
    nb.scalars = reinterpret_cast<ClipScalars *>(base + kScratchRecordOffset);
    if ((rc = launch_step(w, g, m, v, n, clip, host_scalars(t, lr, wd, 1.0f), &nb, stream,
                          nullptr)) != RCS_OK)
        return rc;
    if (norm_out != nullptr &&
        hipMemcpyAsync(norm_out, &nb.scalars->norm, sizeof(double), hipMemcpyDefault, stream) !=
            hipSuccess)
        return RCS_EHIP;
    return RCS_OK;
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
    if (overlaps(snapshot, 3 * bytes, w, bytes) || overlaps(snapshot, 3 * bytes, m, bytes) ||
        overlaps(snapshot, 3 * bytes, v, bytes))
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
    // each part's head (to its destination's next 256-byte boundary, or
    // 16-byte one when fewer than 4 elements would follow) and its source's
    // phase relative to the destination's body; the vector kernel needs a
    // head for every part and 4-byte aligned sources
    SnapPhases ph;
    const float *src[3] = {w, m, v};
    int *q[3] = {&ph.qw, &ph.qm, &ph.qv};
    int *hd[3] = {&ph.hw, &ph.hm, &ph.hv};
    bool vec = aligned4(w) && aligned4(m) && aligned4(v);
    for (int k = 0; vec && k < 3; ++k) {
        const int h = head_of(snapshot + (int64_t)k * n, n);
        vec = h >= 0;
        *hd[k] = h;
        *q[k] = (int)(((reinterpret_cast<uintptr_t>(src[k]) + 4u * (uintptr_t)h) & 15u) >> 2);
    }
    if (vec) {
        const int64_t blocks = ((n >> 2) + kSnapThreads - 1) / kSnapThreads;  // one vector per lane
        hipLaunchKernelGGL(ckpt_snapshot_vec, dim3((unsigned)blocks, 3), dim3(kSnapThreads), 0,
                           compute_stream, w, m, v, snapshot, n, ph);
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
    g_prof_on.store(false, std::memory_order_release);
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
    g_prof_on.store(true, std::memory_order_release);
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

}  // extern "C"

// ceilings.hip -- streaming reference kernels that bench.py times beside the
// update, to show how close the update's memory pattern runs to what the
// chip's HBM gives that pattern. Not part of the library's C ABI and not on
// the training path: they compute nothing of the method.
//
// Over float32 arrays of n4 16-byte vectors:
//   read:  reads g in the norm pass's shape (at most 256 blocks of 512 lanes,
//          4 streaming 16-byte loads in flight per lane, grid-stride); each
//          block writes one float (the sum of everything it read, so no load
//          is dropped or narrowed): 16 B/vector.
// and in the update's launch shape (one wave per block, one 16-byte vector of
// each array per lane, streaming loads and stores, block b working in
// contiguous region b % 8 of the vectors):
//   copy:  m = w: 32 B/vector.
//   4r3w:  reads w, g, m, v and writes w, m, v with one add per element
//          (w += g, m += g, v += g): the update's 28 B per 4 elements with
//          trivial arithmetic.
//   4r3w_keep: the same, but vectors in a 128-byte line the wave shares with
//          a neighbouring wave (an array whose span does not start on a
//          line) are loaded and stored with the sc0 cache policy (relaxed
//          workgroup-scope atomics), as the update does for views; with every
//          array on a line it is 4r3w.
// rcs_ceiling_time launches one of them `reps` times, each launch stamped
// with its own start and stop events (the stamps of the launch itself, as
// the library's instrumented updates take them), and returns the average
// duration: at large n the rate HBM gives the pattern, at small n the
// per-launch floor of the shape. Pointers must be 16-byte aligned device
// memory holding n4 vectors (the read's `out`: one float per block,
// rcs_ceiling_blocks of them).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

namespace {

constexpr int kLanes = 64;
constexpr int64_t kRegions = 8;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The update's block-to-chunk bijection: region b % 8, position b / 8.
__device__ __forceinline__ int64_t chunk_of_block() {
    const int64_t nblk = gridDim.x, c = blockIdx.x;
    const int64_t q = nblk / kRegions, r = nblk % kRegions, x = c % kRegions, j = c / kRegions;
    return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

constexpr int kReadLanes = 512;
constexpr int kReadUnroll = 4;
constexpr int kReadMaxBlocks = 256;

__global__ __launch_bounds__(kReadLanes) void ceiling_read(const f32x4 *__restrict__ a, int64_t n4,
                                                           float *__restrict__ out) {
    __shared__ float lds[kReadLanes / 64];
    float x = 0.0f;
    const int64_t chunk = (int64_t)kReadLanes * kReadUnroll;
    for (int64_t base = (int64_t)blockIdx.x * chunk; base < n4; base += (int64_t)gridDim.x * chunk) {
        f32x4 v[kReadUnroll];
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) {
            const int64_t i = base + (int64_t)j * kReadLanes + threadIdx.x;
            v[j] = (i < n4) ? __builtin_nontemporal_load(a + i) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) x += (v[j].x + v[j].y) + (v[j].z + v[j].w);
    }
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x / 64] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int k = 0; k < kReadLanes / 64; ++k) t += lds[k];
        out[blockIdx.x] = t;
    }
}

int64_t read_blocks(int64_t n4) {
    const int64_t b = (n4 + (int64_t)kReadLanes * kReadUnroll - 1) / ((int64_t)kReadLanes * kReadUnroll);
    return b < kReadMaxBlocks ? b : kReadMaxBlocks;
}

__global__ __launch_bounds__(kLanes) void ceiling_copy(const f32x4 *__restrict__ a,
                                                       f32x4 *__restrict__ b, int64_t n4) {
    const int64_t i = chunk_of_block() * kLanes + threadIdx.x;
    if (i < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

__global__ __launch_bounds__(kLanes) void ceiling_4r3w(f32x4 *__restrict__ w,
                                                       const f32x4 *__restrict__ g,
                                                       f32x4 *__restrict__ m,
                                                       f32x4 *__restrict__ v, int64_t n4) {
    const int64_t i = chunk_of_block() * kLanes + threadIdx.x;
    if (i < n4) {
        const f32x4 gg = __builtin_nontemporal_load(g + i);
        const f32x4 ww = __builtin_nontemporal_load(w + i);
        const f32x4 mm = __builtin_nontemporal_load(m + i);
        const f32x4 vv = __builtin_nontemporal_load(v + i);
        __builtin_nontemporal_store(ww + gg, w + i);
        __builtin_nontemporal_store(mm + gg, m + i);
        __builtin_nontemporal_store(vv + gg, v + i);
    }
}

// Whether the vector at p lies in a line the wave shares with a neighbour;
// a0 is the vector of the wave's lane 0 in the same array.
__device__ __forceinline__ bool shared_line(const void *p, const void *a0) {
    const uintptr_t l = reinterpret_cast<uintptr_t>(p) >> 7;
    const uintptr_t s = reinterpret_cast<uintptr_t>(a0);
    return (s & 127u) != 0 && (l == (s >> 7) || l == ((s + 1024u) >> 7));
}

__device__ __forceinline__ f32x4 ld_line(const f32x4 *p, const f32x4 *a0) {
    if (!shared_line(p, a0)) return __builtin_nontemporal_load(p);
    uint64_t *q = reinterpret_cast<uint64_t *>(const_cast<f32x4 *>(p));
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                 __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

__device__ __forceinline__ void st_line(f32x4 *p, const f32x4 *a0, f32x4 x) {
    if (!shared_line(p, a0)) {
        __builtin_nontemporal_store(x, p);
        return;
    }
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    __hip_atomic_store(q, (uint64_t)__float_as_uint(x.x) | ((uint64_t)__float_as_uint(x.y) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(q + 1, (uint64_t)__float_as_uint(x.z) | ((uint64_t)__float_as_uint(x.w) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__global__ __launch_bounds__(kLanes) void ceiling_4r3w_keep(f32x4 *__restrict__ w,
                                                            const f32x4 *__restrict__ g,
                                                            f32x4 *__restrict__ m,
                                                            f32x4 *__restrict__ v, int64_t n4) {
    const int64_t c = chunk_of_block() * kLanes;
    const int64_t i = c + threadIdx.x;
    if (i < n4) {
        const f32x4 gg = ld_line(g + i, g + c);
        const f32x4 ww = ld_line(w + i, w + c);
        const f32x4 mm = ld_line(m + i, m + c);
        const f32x4 vv = ld_line(v + i, v + c);
        st_line(w + i, w + c, ww + gg);
        st_line(m + i, m + c, mm + gg);
        st_line(v + i, v + c, vv + gg);
    }
}

bool ok16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dim3 grid_of(int64_t n4) { return dim3((unsigned)((n4 + kLanes - 1) / kLanes)); }

int launched() { return hipGetLastError() == hipSuccess ? 0 : -4; }

bool ok_n4(int64_t n4) { return n4 >= 1 && n4 <= ((int64_t)1 << 36); }

// One launch of ceiling `kind` (0 read, 1 copy, 2 4r3w, 3 4r3w_keep) between
// the events start and stop (either may be null).
void launch_kind(int kind, f32x4 *w, const f32x4 *g, f32x4 *m, f32x4 *v, int64_t n4, float *out,
                 hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (kind == 0)
        hipExtLaunchKernelGGL(ceiling_read, dim3((unsigned)read_blocks(n4)), dim3(kReadLanes), 0,
                              stream, start, stop, 0, g, n4, out);
    else if (kind == 1)
        hipExtLaunchKernelGGL(ceiling_copy, grid_of(n4), dim3(kLanes), 0, stream, start, stop, 0,
                              static_cast<const f32x4 *>(w), m, n4);
    else if (kind == 2)
        hipExtLaunchKernelGGL(ceiling_4r3w, grid_of(n4), dim3(kLanes), 0, stream, start, stop, 0,
                              w, g, m, v, n4);
    else
        hipExtLaunchKernelGGL(ceiling_4r3w_keep, grid_of(n4), dim3(kLanes), 0, stream, start, stop,
                              0, w, g, m, v, n4);
}

}  // namespace

extern "C" {

// Blocks of the read ceiling (and so floats of its output) for n4 vectors.
int64_t rcs_ceiling_blocks(int64_t n4) { return n4 < 1 ? 0 : read_blocks(n4); }

// Average duration in microseconds of `reps` stamped launches of ceiling
// `kind` over w, g, m, v (kind 0 reads g into out; kind 1 copies w to m;
// kind 2 is the 4-read/3-write pattern, kind 3 the same with cache-retaining
// accesses on shared lines), after two unstamped ones. Blocks until they are
// done. Returns 0, -1 for bad arguments, -4 on a HIP error.
int rcs_ceiling_time(int kind, float *w, const float *g, float *m, float *v, int64_t n4,
                     float *out, int reps, hipStream_t stream, double *avg_us) {
    if (kind < 0 || kind > 3 || !ok_n4(n4) || reps < 1 || reps > 1000 || avg_us == nullptr)
        return -1;
    if (kind == 0 && (!ok16(g) || out == nullptr)) return -1;
    if (kind == 1 && (!ok16(w) || !ok16(m))) return -1;
    if (kind >= 2 && (!ok16(w) || !ok16(g) || !ok16(m) || !ok16(v))) return -1;
    f32x4 *w4 = reinterpret_cast<f32x4 *>(w), *m4 = reinterpret_cast<f32x4 *>(m);
    f32x4 *v4 = reinterpret_cast<f32x4 *>(v);
    const f32x4 *g4 = reinterpret_cast<const f32x4 *>(g);
    std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
    int rc = 0;
    for (auto &e : ev)
        if (hipEventCreate(&e) != hipSuccess) rc = -4;
    if (rc == 0) {
        for (int k = 0; k < 2; ++k) launch_kind(kind, w4, g4, m4, v4, n4, out, stream, nullptr, nullptr);
        for (int k = 0; k < reps; ++k)
            launch_kind(kind, w4, g4, m4, v4, n4, out, stream, ev[2 * k], ev[2 * k + 1]);
        rc = launched();
    }
    double sum_ms = 0.0;
    if (rc == 0 && hipEventSynchronize(ev[2 * (size_t)reps - 1]) != hipSuccess) rc = -4;
    for (int k = 0; rc == 0 && k < reps; ++k) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]) != hipSuccess) rc = -4;
        sum_ms += ms;
    }
    for (auto &e : ev)
        if (e != nullptr) (void)hipEventDestroy(e);
    if (rc == 0) *avg_us = sum_ms / reps * 1e3;
    (void)hipGetLastError();
    return rc;
}

}  // extern "C"

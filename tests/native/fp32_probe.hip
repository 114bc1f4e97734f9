// fp32_probe.hip -- test helper, not part of the library: the device's float32
// divide and square root (HIP defaults: correctly rounded, subnormals kept, no
// contraction), for comparison with the host's IEEE results. The update's
// float32 sequence relies on both being correctly rounded.
#include <hip/hip_runtime.h>

#include <cstdint>

#pragma clang fp contract(off)

__global__ __launch_bounds__(256) void fp32_div_sqrt(const float *__restrict__ a,
                                                     const float *__restrict__ b,
                                                     float *__restrict__ q, float *__restrict__ r,
                                                     int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        q[i] = a[i] / b[i];
        r[i] = __builtin_sqrtf(a[i]);
    }
}

// q = a / b and r = sqrtf(a) elementwise over device float32 arrays of n
// elements; 0 on a successful launch, -1 on bad arguments, -4 on a failed one.
extern "C" int fp32_div_sqrt_probe(const float *a, const float *b, float *q, float *r, int64_t n,
                                   hipStream_t stream) {
    if (!a || !b || !q || !r || n < 1 || n > ((int64_t)1 << 30)) return -1;
    hipLaunchKernelGGL(fp32_div_sqrt, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a,
                       b, q, r, n);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

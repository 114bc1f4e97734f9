/* Exact-size hipMalloc buffers handed to the C ABI with an n longer than one
 * of them: every entry point that takes device arrays refuses with RCS_ESIZE
 * before enqueuing anything, and no array changes (each holds a byte pattern
 * that any launched kernel or copy would overwrite). No Python in the process.
 *
 * usage: abi_short_buffers      prints "abi short buffers ok" on success */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rcs.h"

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            return 1;                                                 \
        }                                                             \
    } while (0)

enum { N = 4096, SHORT = N / 2, NBUF = 7 };

int main(void) {
    /* w, g, m, v of N floats; a short g, a short w (N / 2 floats); a snapshot
     * of half the 12 N bytes the asynchronous pack needs */
    const size_t sizes[NBUF] = {4 * N, 4 * N, 4 * N, 4 * N, 4 * SHORT, 4 * SHORT, 6 * N};
    void *d[NBUF];
    for (int k = 0; k < NBUF; ++k) {
        CHECK(hipMalloc(&d[k], sizes[k]) == hipSuccess);
        CHECK(hipMemset(d[k], 0x5A, sizes[k]) == hipSuccess);
    }
    CHECK(hipDeviceSynchronize() == hipSuccess);
    float *w = d[0], *g = d[1], *m = d[2], *v = d[3], *gs = d[4], *ws = d[5], *snap = d[6];
    double *norm = NULL;
    CHECK(hipMalloc((void **)&norm, sizeof(double)) == hipSuccess);
    unsigned char *host = NULL;
    CHECK(hipHostMalloc((void **)&host, (size_t)ckpt_bytes(N), 0) == hipSuccess);
    memset(host, 0, (size_t)ckpt_bytes(N));
    hipStream_t s = 0;

    CHECK(adamw_clip_step(w, gs, m, v, N, 1, 1e-3f, 0.0f, 1.0f, s) == RCS_ESIZE);
    CHECK(adamw_clip_step(ws, g, m, v, N, 1, 1e-3f, 0.0f, 1.0f, s) == RCS_ESIZE);
    CHECK(adamw_clip_step(w, g, ws, v, N, 1, 1e-3f, 0.0f, 1.0f, s) == RCS_ESIZE);
    CHECK(adamw_clip_step_accum(w, gs, m, v, N, 1, 1e-3f, 0.0f, 1.0f, 0.5f, s) == RCS_ESIZE);
    CHECK(adamw_clip_step_noalloc(w, g, m, ws, N, 1, 1e-3f, 0.0f, 1.0f, NULL, s) == RCS_ESIZE);
    CHECK(grad_global_norm(gs, N, norm, s) == RCS_ESIZE);
    CHECK(grad_clip_inplace(gs, N, 1.0f, s) == RCS_ESIZE);
    CHECK(grad_zero(gs, N, s) == RCS_ESIZE);
    CHECK(ckpt_pack(1, N, ws, m, v, host, ckpt_bytes(N), s) == RCS_ESIZE);
    /* a valid image of N parameters unpacked into a short array */
    CHECK(ckpt_pack(1, N, w, m, v, host, ckpt_bytes(N), s) == RCS_OK);
    CHECK(hipDeviceSynchronize() == hipSuccess);
    int32_t step = -1;
    CHECK(hipMemset(w, 0x5A, 4 * N) == hipSuccess);
    CHECK(ckpt_unpack(host, ckpt_bytes(N), N, &step, w, ws, v, s) == RCS_ESIZE && step == -1);
    CHECK(ckpt_pack_async(1, N, w, m, v, snap, ckpt_snapshot_bytes(N), host, ckpt_bytes(N), s,
                          s) == RCS_ESIZE);
    CHECK(hipDeviceSynchronize() == hipSuccess);

    unsigned char *back = (unsigned char *)malloc(6 * N);
    CHECK(back != NULL);
    for (int k = 0; k < NBUF; ++k) {
        CHECK(hipMemcpy(back, d[k], sizes[k], hipMemcpyDeviceToHost) == hipSuccess);
        for (size_t i = 0; i < sizes[k]; ++i) CHECK(back[i] == 0x5A);
    }
    free(back);
    for (int k = 0; k < NBUF; ++k) CHECK(hipFree(d[k]) == hipSuccess);
    CHECK(hipFree(norm) == hipSuccess);
    CHECK(hipHostFree(host) == hipSuccess);
    printf("abi short buffers ok\n");
    return 0;
}

/* A plain C training loop over the library, without Python or PyTorch: reads
 * the initial weights and one gradient per update from a file, runs
 * adamw_clip_step on the GPU for each, prints every pre-clip norm, packs the
 * final state and writes it with ckpt_file_write, then saves the same state
 * once more through the asynchronous writer into a second directory.
 *
 * usage: c_step_driver INPUT N STEPS LR WD CLIP OUT_DIR WRITER_DIR
 * INPUT: float32 w0[N], then g_1[N] ... g_STEPS[N] (little-endian).
 * Output lines: "norm <t> <%.17g>", "file <path>", "writer <path>". */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "rcs.h"

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            return 1;                                                 \
        }                                                             \
    } while (0)

static int read_floats(FILE *f, float *dst, int64_t n) {
    return fread(dst, sizeof(float), (size_t)n, f) == (size_t)n;
}

int main(int argc, char **argv) {
    CHECK(argc == 9);
    const int64_t n = atoll(argv[2]);
    const int steps = atoi(argv[3]);
    const float lr = (float)atof(argv[4]), wd = (float)atof(argv[5]), clip = (float)atof(argv[6]);
    CHECK(n > 0 && steps > 0);
    const size_t bytes = (size_t)n * sizeof(float);

    FILE *in = fopen(argv[1], "rb");
    CHECK(in != NULL);
    float *host = (float *)malloc(bytes);
    CHECK(host != NULL);

    float *w = NULL, *g = NULL, *m = NULL, *v = NULL;
    CHECK(hipMalloc((void **)&w, bytes) == hipSuccess);
    CHECK(hipMalloc((void **)&g, bytes) == hipSuccess);
    CHECK(hipMalloc((void **)&m, bytes) == hipSuccess);
    CHECK(hipMalloc((void **)&v, bytes) == hipSuccess);
    CHECK(hipMemset(m, 0, bytes) == hipSuccess);
    CHECK(hipMemset(v, 0, bytes) == hipSuccess);
    CHECK(read_floats(in, host, n));
    CHECK(hipMemcpy(w, host, bytes, hipMemcpyHostToDevice) == hipSuccess);

    hipStream_t s;
    CHECK(hipStreamCreate(&s) == hipSuccess);
    CHECK(rcs_init(0, s) == RCS_OK);
    double *norm = NULL;
    CHECK(hipHostMalloc((void **)&norm, sizeof(double), hipHostMallocDefault) == hipSuccess);

    for (int t = 1; t <= steps; ++t) {
        CHECK(read_floats(in, host, n));
        /* the previous update must be done with g before it is overwritten */
        CHECK(hipStreamSynchronize(s) == hipSuccess);
        CHECK(hipMemcpy(g, host, bytes, hipMemcpyHostToDevice) == hipSuccess);
        CHECK(adamw_clip_step(w, g, m, v, n, t, lr, wd, clip, s) == RCS_OK);
        CHECK(last_grad_norm(s, norm) == RCS_OK);
        CHECK(hipStreamSynchronize(s) == hipSuccess);
        printf("norm %d %.17g\n", t, *norm);
    }
    fclose(in);

    const int64_t nb = ckpt_bytes(n);
    void *buf = NULL;
    CHECK(hipHostMalloc(&buf, (size_t)nb, hipHostMallocDefault) == hipSuccess);
    CHECK(ckpt_pack(steps, n, w, m, v, buf, nb, s) == RCS_OK);
    CHECK(hipStreamSynchronize(s) == hipSuccess);
    char path[4096];
    CHECK(ckpt_file_write(argv[7], buf, nb, path, sizeof path) == RCS_OK);
    printf("file %s\n", path);

    rcs_ckpt_writer *wr = NULL;
    CHECK(rcs_ckpt_writer_create(argv[8], n, 2, &wr) == RCS_OK);
    CHECK(rcs_ckpt_writer_submit(wr, steps, w, m, v, s) == RCS_OK);
    CHECK(rcs_ckpt_writer_wait(wr, path, sizeof path) == RCS_OK);
    printf("writer %s\n", path);
    CHECK(rcs_ckpt_writer_destroy(wr) == RCS_OK);

    CHECK(hipHostFree(buf) == hipSuccess);
    CHECK(hipHostFree(norm) == hipSuccess);
    CHECK(hipStreamDestroy(s) == hipSuccess);
    CHECK(hipFree(w) == hipSuccess && hipFree(g) == hipSuccess);
    CHECK(hipFree(m) == hipSuccess && hipFree(v) == hipSuccess);
    free(host);
    printf("c step driver ok\n");
    return 0;
}

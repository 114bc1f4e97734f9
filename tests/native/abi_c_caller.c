/* A plain C caller of the library: include/rcs.h must compile as C, link
 * against librcs.so, and reject bad arguments on the host without a GPU. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rcs.h"

#define EXPECT(cond)                                              \
    do {                                                          \
        if (!(cond)) {                                            \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            return 1;                                             \
        }                                                         \
    } while (0)

int main(void) {
    unsigned char buf[8 + 12 * 4];
    int32_t step = -7;
    EXPECT(ckpt_bytes(4) == 8 + 12 * 4);
    EXPECT(ckpt_bytes(0) == -1);
    EXPECT(ckpt_bytes(RCS_MAX_N) == 8 + 12 * RCS_MAX_N);
    EXPECT(ckpt_snapshot_bytes(4) == 48);
    EXPECT(adamw_clip_step(NULL, NULL, NULL, NULL, 16, 1, 1e-3f, 0.0f, 1.0f, 0) == RCS_EINVAL);
    EXPECT(adamw_clip_step_accum(NULL, NULL, NULL, NULL, 16, 1, 1e-3f, 0.0f, 1.0f, 0.5f, 0) ==
           RCS_EINVAL);
    EXPECT(adamw_clip_step_noalloc(NULL, NULL, NULL, NULL, 16, 1, 1e-3f, 0.0f, 1.0f, NULL, 0) ==
           RCS_EINVAL);
    EXPECT(adamw_clip_step_noalloc((float *)0x1000, (float *)0x1000, (float *)0x1000,
                                   (float *)0x1000, RCS_MAX_N + 1, 1, 1e-3f, 0.0f, 1.0f, NULL,
                                   0) == RCS_EINVAL);
    EXPECT(grad_zero(NULL, 16, 0) == RCS_EINVAL);
    EXPECT(grad_zero((float *)0x1000, 0, 0) == RCS_EINVAL);
    memset(buf, 0, sizeof buf);
    buf[0] = 5;  /* step 5 */
    buf[4] = 3;  /* n = 3, but the buffer holds 4 */
    EXPECT(ckpt_unpack(buf, sizeof buf, 4, &step, (float *)0x1000, (float *)0x1000,
                       (float *)0x1000, 0) == RCS_EHEADER);
    buf[4] = 4;
    EXPECT(ckpt_unpack(buf, sizeof buf - 1, 4, &step, (float *)0x1000, (float *)0x1000,
                       (float *)0x1000, 0) == RCS_ESIZE);
    EXPECT(step == -7);
    EXPECT(strlen(rcs_strerror(RCS_EIO)) > 0);
    EXPECT(rcs_signals_poll() == 0);
    printf("c caller ok\n");
    return 0;
}

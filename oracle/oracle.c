/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for one clipped AdamW
 * update over a flat float32 parameter vector, and for the step_NNNNNN.bin
 * checkpoint layout.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file's library. The
 * product library (resumable_checkpoint_state_amd) shares no code, header,
 * table or constant with it, and must never route through it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64 SSE arithmetic: every float op is rounded to nearest-even on its
 * own, no fused multiply-add, subnormals kept; no -march flags).
 *
 * What each function follows (pages named by title, then section):
 *   - global clip: "Training as a Recoverable State Transition",
 *     section "The Exact Targets of Clipping and AdamW" (first paragraph):
 *     all gradients form one vector g; if its L2 norm exceeds the threshold
 *     c the whole vector is multiplied by c/||g||, else it is left alone.
 *     The same page's Example 1 code applies no epsilon and skips a zero
 *     gradient.
 *   - AdamW: same page and section (second paragraph): beta1=0.9,
 *     beta2=0.999, eps=1e-8, m and v start at zero, t counts updates from
 *     the beginning, m_hat=m/(1-beta1^t), v_hat=v/(1-beta2^t), parameters are
 *     first multiplied by (1-lr*wd), then lr*m_hat/(sqrt(v_hat)+eps) is
 *     subtracted; decay applies to every parameter.
 *   - update order: same page, section "Task and Prerequisites": record the
 *     pre-clip norm, clip globally, then step.
 *   - state layout: grow_a_language_model_checkpoints (Georgian and Spanish
 *     editions), sections "Format", "Region by region", "Total size":
 *     [int32 step][int32 n_params][n x f32 weights][n x f32 m][n x f32 v],
 *     8 + 12 n bytes.
 *   - step meaning: "Training as a Recoverable State Transition", section
 *     "The Checkpoint Contract and a Real Recovery Test": the file is written
 *     after a complete optimizer step and the step count is the number of
 *     updates performed, so a resume continues with t = step + 1.
 *
 * Readings where the pages leave the arithmetic open (one line each):
 *   R1 norm: squares in float64 (exact for float32 inputs), summed in index
 *      order with Neumaier compensation, float64 square root.
 *   R2 clip scale s = (float)((double)c / norm) when norm > c, else 1.0f;
 *      no epsilon; norm == 0 gives s = 1.
 *   R3 non-finite norm: the update is skipped (w, m, v untouched) and the
 *      norm is reported.
 *   R4 the state is float32 (the file stores float32), so the per-element
 *      update is a fixed float32 sequence, each op rounded separately:
 *        gp = g*s; m = 0.9f*m + 0.1f*gp; v = 0.999f*v + 0.001f*(gp*gp);
 *        mh = m/bc1; vh = v/bc2; den = sqrtf(vh) + 1e-8f;
 *        w = w*decay - (lr*mh)/den
 *      with bc1 = (float)(1 - 0.9^t), bc2 = (float)(1 - 0.999^t) and
 *      decay = (float)(1 - (double)lr*(double)wd), each computed in float64
 *      and rounded once.
 *   R5 header integers are little-endian signed int32; n <= 0, step < 0 and
 *      any buffer length other than 8 + 12 n are rejected before anything
 *      is copied.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_SKIPPED 1
#define ORACLE_EINVAL (-1)
#define ORACLE_ESIZE (-2)
#define ORACLE_EHEADER (-3)

/* ---- R1: float64 sum of squares, index order, Neumaier compensation ---- */

/* state[0] = running sum, state[1] = running compensation.  Chunks may be fed
 * one after another in index order; the result is the same as one call over
 * the concatenation. */
void oracle_sumsq_accum(double state[2], const float *g, int64_t n) {
    double sum = state[0], comp = state[1];
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)g[i] * (double)g[i]; /* exact: 24x24 bits < 53 */
        double t = sum + x;
        if (fabs(sum) >= fabs(x))
            comp += (sum - t) + x;
        else
            comp += (x - t) + sum;
        sum = t;
    }
    state[0] = sum;
    state[1] = comp;
}

/* A non-finite running sum (an infinite or NaN square) is returned as is: the
 * compensation term is then meaningless (inf - inf), and the plain definition
 * of the norm of a vector holding +-inf is +inf, of one holding NaN, NaN. */
double oracle_sumsq_finish(const double state[2]) {
    if (!isfinite(state[0])) return state[0];
    return state[0] + state[1];
}

double oracle_grad_norm(const float *g, int64_t n) {
    double st[2] = {0.0, 0.0};
    oracle_sumsq_accum(st, g, n);
    return sqrt(oracle_sumsq_finish(st));
}

/* ---- R2: the single global clip factor ---- */
float oracle_clip_scale(double norm, float clip) {
    if (norm > (double)clip) return (float)((double)clip / norm);
    return 1.0f;
}

/* ---- R4: host scalars, float64 then one rounding each ---- */
void oracle_scalars(int32_t t, float lr, float wd, float *bc1, float *bc2, float *decay) {
    *bc1 = (float)(1.0 - pow(0.9, (double)t));
    *bc2 = (float)(1.0 - pow(0.999, (double)t));
    *decay = (float)(1.0 - (double)lr * (double)wd);
}

/* ---- R4: per-element float32 AdamW with the clip factor applied to g ---- */
void oracle_adamw_elems(float *w, const float *g, float *m, float *v, int64_t n, float s,
                        float bc1, float bc2, float decay, float lr) {
    for (int64_t i = 0; i < n; ++i) {
        float gp = g[i] * s;
        float m_old = 0.9f * m[i];
        float m_new_part = 0.1f * gp;
        float mi = m_old + m_new_part;
        float gsq = gp * gp;
        float v_old = 0.999f * v[i];
        float v_new_part = 0.001f * gsq;
        float vi = v_old + v_new_part;
        float mh = mi / bc1;
        float vh = vi / bc2;
        float root = sqrtf(vh);
        float den = root + 1e-8f;
        float decayed = w[i] * decay;
        float num = lr * mh;
        float stepv = num / den;
        w[i] = decayed - stepv;
        m[i] = mi;
        v[i] = vi;
    }
}

/* The averaging step of gradient accumulation, grow_a_language_model_backprop,
 * section on accumulation over micro-batches: backward passes add into one
 * gradient buffer, then every element is multiplied by 1/n_micro (a float32
 * multiply) before the optimizer step. */
void oracle_scale_grads(float *g, int64_t n, float scale) {
    for (int64_t i = 0; i < n; ++i) g[i] = g[i] * scale;
}

/* The global clip alone, in place (R1-R3): g[i] = g[i] * s, skipped when the
 * norm is not finite. Returns ORACLE_OK or ORACLE_SKIPPED. */
int oracle_clip_grads(float *g, int64_t n, float clip, double *norm_out) {
    double norm = oracle_grad_norm(g, n);
    if (norm_out) *norm_out = norm;
    if (!isfinite(norm)) return ORACLE_SKIPPED;
    float s = oracle_clip_scale(norm, clip);
    for (int64_t i = 0; i < n; ++i) g[i] = g[i] * s;
    return ORACLE_OK;
}

/* One full update: norm, clip factor, scalars, elementwise step.
 * Returns ORACLE_OK, ORACLE_SKIPPED (non-finite norm, R3) or ORACLE_EINVAL. */
int oracle_adamw_clip_step(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                           float lr, float wd, float clip, double *norm_out) {
    if (!w || !g || !m || !v || n <= 0 || t < 1) return ORACLE_EINVAL;
    if (!isfinite(lr) || !isfinite(wd) || isnan(clip) || !(clip > 0.0f)) return ORACLE_EINVAL;
    double norm = oracle_grad_norm(g, n);
    if (norm_out) *norm_out = norm;
    if (!isfinite(norm)) return ORACLE_SKIPPED;
    float s = oracle_clip_scale(norm, clip);
    float bc1, bc2, decay;
    oracle_scalars(t, lr, wd, &bc1, &bc2, &decay);
    oracle_adamw_elems(w, g, m, v, n, s, bc1, bc2, decay, lr);
    return ORACLE_OK;
}

/* The definition of the clipped AdamW update ("Training as a Recoverable State
 * Transition", section "The Exact Targets of Clipping and AdamW") evaluated in
 * float64 from start to end, over a vector: one global L2 clip of g to norm
 * <= clip (no epsilon), then for the 1-based update index t the moving
 * averages m = beta1 m + (1 - beta1) g' and v = beta2 v + (1 - beta2) g'^2,
 * their bias corrections by 1 - beta^t, and every parameter decayed by
 * (1 - lr wd) before the Adam step lr m_hat / (sqrt(v_hat) + eps) is taken
 * off it. The page's worked example (Example 1) prints float64 figures; this
 * function is what they pin, and it in turn bounds the float32 sequence
 * above. ORACLE_SKIPPED (w, m, v untouched) for a non-finite norm. */
int oracle_adamw_clip_step_f64(double *w, const double *g, double *m, double *v, int64_t n,
                               int32_t t, double lr, double wd, double clip, double *norm_out) {
    const double beta1 = 0.9, beta2 = 0.999, eps = 1e-8;
    if (!w || !g || !m || !v || n <= 0 || t < 1 || !(clip > 0.0)) return ORACLE_EINVAL;
    double sumsq = 0.0;
    for (int64_t i = 0; i < n; ++i) sumsq += g[i] * g[i];
    const double norm = sqrt(sumsq);
    if (norm_out) *norm_out = norm;
    if (!isfinite(norm)) return ORACLE_SKIPPED;
    const double scale = (norm > clip) ? clip / norm : 1.0;
    const double corr1 = 1.0 - pow(beta1, (double)t);
    const double corr2 = 1.0 - pow(beta2, (double)t);
    const double keep = 1.0 - lr * wd;
    for (int64_t i = 0; i < n; ++i) {
        const double gi = g[i] * scale;
        m[i] = beta1 * m[i] + (1.0 - beta1) * gi;
        v[i] = beta2 * v[i] + (1.0 - beta2) * (gi * gi);
        const double m_hat = m[i] / corr1;
        const double v_hat = v[i] / corr2;
        w[i] = keep * w[i] - lr * m_hat / (sqrt(v_hat) + eps);
    }
    return ORACLE_OK;
}

/* ---- state layout ---- */

int64_t oracle_ckpt_bytes(int64_t n) {
    if (n <= 0 || n > 2147483647LL) return -1;
    return 8 + 12 * n;
}

static void put_i32_le(uint8_t *p, int32_t x) {
    uint32_t u = (uint32_t)x;
    p[0] = (uint8_t)(u & 0xffu);
    p[1] = (uint8_t)((u >> 8) & 0xffu);
    p[2] = (uint8_t)((u >> 16) & 0xffu);
    p[3] = (uint8_t)((u >> 24) & 0xffu);
}

static int32_t get_i32_le(const uint8_t *p) {
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                 ((uint32_t)p[3] << 24);
    return (int32_t)u;
}

/* float32 bit pattern written byte by byte, little-endian */
static void put_f32_le(uint8_t *p, float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    put_i32_le(p, (int32_t)u);
}

static float get_f32_le(const uint8_t *p) {
    uint32_t u = (uint32_t)get_i32_le(p);
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int oracle_ckpt_pack(int32_t step, int64_t n, const float *w, const float *m, const float *v,
                     uint8_t *buf, int64_t len) {
    if (!w || !m || !v || !buf || step < 0) return ORACLE_EINVAL;
    int64_t need = oracle_ckpt_bytes(n);
    if (need < 0) return ORACLE_EINVAL;
    if (len != need) return ORACLE_ESIZE;
    put_i32_le(buf + 0, step);
    put_i32_le(buf + 4, (int32_t)n);
    uint8_t *pw = buf + 8, *pm = buf + 8 + 4 * n, *pv = buf + 8 + 8 * n;
    for (int64_t i = 0; i < n; ++i) {
        put_f32_le(pw + 4 * i, w[i]);
        put_f32_le(pm + 4 * i, m[i]);
        put_f32_le(pv + 4 * i, v[i]);
    }
    return ORACLE_OK;
}

/* Reads the header only. Returns ORACLE_OK and fills step/n, or an error. */
int oracle_ckpt_header(const uint8_t *buf, int64_t len, int32_t *step, int32_t *n) {
    if (!buf || len < 8) return ORACLE_ESIZE;
    *step = get_i32_le(buf);
    *n = get_i32_le(buf + 4);
    return ORACLE_OK;
}

int oracle_ckpt_unpack(const uint8_t *buf, int64_t len, int64_t n_expected, int32_t *step_out,
                       float *w, float *m, float *v) {
    if (!buf || !step_out || !w || !m || !v) return ORACLE_EINVAL;
    if (len < 8) return ORACLE_ESIZE;
    int32_t step = get_i32_le(buf);
    int32_t n = get_i32_le(buf + 4);
    if (n <= 0 || step < 0) return ORACLE_EHEADER;
    if (n_expected > 0 && (int64_t)n != n_expected) return ORACLE_EHEADER;
    if (len != 8 + 12 * (int64_t)n) return ORACLE_ESIZE;
    const uint8_t *pw = buf + 8, *pm = buf + 8 + 4 * (int64_t)n, *pv = buf + 8 + 8 * (int64_t)n;
    for (int64_t i = 0; i < n; ++i) {
        w[i] = get_f32_le(pw + 4 * i);
        m[i] = get_f32_le(pm + 4 * i);
        v[i] = get_f32_le(pv + 4 * i);
    }
    *step_out = step;
    return ORACLE_OK;
}

/* 1 if float32 subnormals survive arithmetic in this process (no FTZ/DAZ). */
int oracle_subnormals_kept(void) {
    volatile float tiny = 1.17549435e-38f; /* FLT_MIN */
    volatile float half = 0.5f;
    float r = tiny * half;
    return r != 0.0f;
}

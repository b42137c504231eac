/*
 * attnres_oracle.c -- plain fp64 CPU oracle for the Kimi-K3 attention-residual
 * (AttnRes) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the GPU library.
 *
 * Sources of the definition (the pages, cited by title and section):
 *  [ASC]  vllm-ascend PR #14840 "[Performance][Ops] Add Kimi K3 attention
 *         residual fusion", author's "Implementation walkthrough": for each
 *         token the bank rows in use are taken, the current prefix sum joins
 *         them as the last candidate, each candidate's RMS is normalised in
 *         fp32 and scored against the product of the two weight vectors, the
 *         scores become softmax weights over exactly those candidates, and
 *         the weighted sum of the candidates is converted to the model's
 *         dtype; the bank's slot dimension is its capacity, not the number
 *         in use, and slots beyond that number take no part.
 *  [P1]   prhub digest of vLLM PR #54261 (native CUDA Kimi-K3 AttnRes made the
 *         default on SM100), "Implementation breakdown" items 1-3 and the
 *         kernel snippet under "Key source snippets": optional delta added
 *         into the prefix row which is then stored back to the layer residual,
 *         block_write_idx (-1 = none) storing that same row into the block
 *         bank, optional output RMSNorm applied to the fp32 accumulator and
 *         multiplied by its weight, bf16 output.
 *  [P2]   prhub digest of vLLM PR #50185 (AttnRes latency), "Implementation
 *         breakdown" item 2: the fused query q_cache = rms_w * res_w.
 *
 * Readings taken where the pages are silent (each is applied once, here):
 *  R1 the softmax weights the RAW source rows (the sum is over the residual
 *     streams themselves); the normalised rows only produce the logits.
 *  R2 the current-layer source is cur = bf16_RNE(prefix + delta) (the row the
 *     kernel stores back), or prefix when there is no delta.
 *  R3 with a delta, prefix is overwritten with cur; without one it is left
 *     untouched.
 *  R4 the row written to blocks[t, block_write_idx] is cur.
 *  R5 every read sees the state before the call: a written slot that is also
 *     a source contributes its old value.
 *  R6 source order: bank slots 0..nb-1, then cur.
 *  R7 RMSNorm(x) = x / sqrt(mean_h(x^2) + eps) * w (eps inside the root,
 *     mean over the hidden size, plain weight).
 *  R8 no temperature or bias on the logits.
 *  R10 the output norm acts on the unrounded mixture; one final rounding to
 *     bf16, ties to even.
 *
 * Precision: every arithmetic step is IEEE double, evaluated sequentially in
 * the order written; the only bf16 roundings are those the definition states
 * (cur, and the final output).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double, exact (bf16 is the top half of an fp32). */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16 value, ties to even (IEEE 754
 * roundTiesToEven at 8 significant bits, fp32 exponent range).  Normal bf16
 * numbers have an 8-bit significand, so the quantum at binary exponent e
 * (x = m * 2^e, 0.5 <= |m| < 1) is 2^(e-8); below the smallest normal
 * 2^-126 the quantum stays at the subnormal step 2^-133.  nearbyint() in the
 * default rounding mode is round-half-to-even.  Results at or beyond 2^128
 * overflow to infinity.
 */
static double round_to_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    int e;
    (void)frexp(x, &e);
    int qexp = e - 8;
    if (qexp < -133)
        qexp = -133;
    double y = ldexp(nearbyint(ldexp(x, -qexp)), qexp);
    if (fabs(y) >= ldexp(1.0, 128))
        return copysign(INFINITY, x);
    return y;
}

/* A double that is exactly a bf16 value (or +-inf / NaN) -> its bit pattern. */
static uint16_t bf16_value_to_bits(double v)
{
    if (isnan(v))
        return (uint16_t)0x7FC0u;
    float f = (float)v; /* exact for bf16-representable values */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Exported rounding helper for the tests: out[i] = bits(RNE_bf16(x[i])). */
void oracle_round_bf16(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_value_to_bits(round_to_bf16(x[i]));
}

/* Exported widening helper for the tests. */
void oracle_bf16_to_double(const uint16_t *b, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_bits_to_double(b[i]);
}

/*
 * RMS-normalise one row: xhat[h] = x[h] / sqrt(mean(x^2) + eps)   (R7, without
 * the weight; the weight is applied by the caller where the definition puts
 * it).
 */
static void rms_normalise(const double *x, int64_t H, double eps, double *xhat)
{
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h)
        ss += x[h] * x[h];
    double denom = sqrt(ss / (double)H + eps);
    for (int64_t h = 0; h < H; ++h)
        xhat[h] = x[h] / denom;
}

/*
 * The AttnRes forward over T tokens, in place on prefix and blocks exactly as
 * the op's contract states, plus the fp64 output before its final rounding.
 *
 *   prefix  [T, H] bf16 bits, row stride H; overwritten with cur when delta
 *           is given (R3).
 *   delta   [T, H] bf16 bits, row stride H, or NULL.
 *   blocks  element (t, i, h) at blocks[t*token_stride + i*slot_stride + h];
 *           slots 0..nb-1 are sources; slot widx (if >= 0) receives cur.
 *   res_w, rms_w, onw   [H] bf16 bits (onw NULL = no output norm).
 *   out_f64 [T, H]      the output before rounding (may be NULL).
 *   out_bf16 [T, H]     bits of RNE_bf16(output).
 *   logits, probs  [T, nb+1] each (may be NULL): per-source logit and weight.
 *
 * Returns 0, or -1 for arguments the definition does not cover.
 */
int oracle_attnres_fwd(int64_t T, int64_t H, uint16_t *prefix, const uint16_t *delta,
                       uint16_t *blocks, int64_t token_stride, int64_t slot_stride,
                       int cap, int nb, const uint16_t *res_w, const uint16_t *rms_w,
                       double rms_eps, const uint16_t *onw, double out_eps, int widx,
                       double *out_f64, uint16_t *out_bf16, double *logits, double *probs)
{
    if (T < 0 || H <= 0 || nb < 0 || nb > cap || widx < -1 || widx >= cap)
        return -1;
    if (nb > 0 && blocks == NULL)
        return -1;
    if (widx >= 0 && blocks == NULL)
        return -1;

    const int nsrc = nb + 1;
    double *src = (double *)malloc(sizeof(double) * (size_t)nsrc * (size_t)H);
    double *cur = (double *)malloc(sizeof(double) * (size_t)H);
    double *xhat = (double *)malloc(sizeof(double) * (size_t)H);
    double *y = (double *)malloc(sizeof(double) * (size_t)H);
    double *l = (double *)malloc(sizeof(double) * (size_t)nsrc);
    double *p = (double *)malloc(sizeof(double) * (size_t)nsrc);
    if (!src || !cur || !xhat || !y || !l || !p) {
        free(src); free(cur); free(xhat); free(y); free(l); free(p);
        return -2;
    }

    for (int64_t t = 0; t < T; ++t) {
        /* Current-layer residual (R2): prefix, plus delta rounded once. */
        for (int64_t h = 0; h < H; ++h) {
            double pv = bf16_bits_to_double(prefix[t * H + h]);
            cur[h] = delta ? round_to_bf16(pv + bf16_bits_to_double(delta[t * H + h])) : pv;
        }

        /* Gather sources in order (R6), all read before any write (R5). */
        for (int j = 0; j < nb; ++j) {
            const uint16_t *row = blocks + t * token_stride + (int64_t)j * slot_stride;
            for (int64_t h = 0; h < H; ++h)
                src[(int64_t)j * H + h] = bf16_bits_to_double(row[h]);
        }
        memcpy(src + (int64_t)nb * H, cur, sizeof(double) * (size_t)H);

        /* Score each source: logit = proj_w . (RMSNorm(x) with norm_w)  (R7, R8).
         * rms_w is the norm's weight, res_w the scoring projection. */
        for (int j = 0; j < nsrc; ++j) {
            rms_normalise(src + (int64_t)j * H, H, rms_eps, xhat);
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double normed = xhat[h] * bf16_bits_to_double(rms_w[h]);
                acc += bf16_bits_to_double(res_w[h]) * normed;
            }
            l[j] = acc;
        }

        /* Softmax over the nb+1 valid sources (max-shifted).  A single
         * source has weight exactly 1 (R12), also when its logit is not a
         * number (eps = 0 and an all-zero row make it 0/0). */
        if (nsrc == 1) {
            p[0] = 1.0;
        } else {
            double m = l[0];
            for (int j = 1; j < nsrc; ++j)
                if (l[j] > m)
                    m = l[j];
            double z = 0.0;
            for (int j = 0; j < nsrc; ++j) {
                p[j] = exp(l[j] - m);
                z += p[j];
            }
            for (int j = 0; j < nsrc; ++j)
                p[j] /= z;
        }

        /* Weighted sum of the RAW source rows (R1). */
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int j = 0; j < nsrc; ++j)
                acc += p[j] * src[(int64_t)j * H + h];
            y[h] = acc;
        }

        /* Optional output RMSNorm on the unrounded mixture (R7, R10). */
        if (onw) {
            rms_normalise(y, H, out_eps, xhat);
            for (int64_t h = 0; h < H; ++h)
                y[h] = xhat[h] * bf16_bits_to_double(onw[h]);
        }

        for (int64_t h = 0; h < H; ++h) {
            if (out_f64)
                out_f64[t * H + h] = y[h];
            out_bf16[t * H + h] = bf16_value_to_bits(round_to_bf16(y[h]));
        }
        if (logits)
            for (int j = 0; j < nsrc; ++j)
                logits[t * nsrc + j] = l[j];
        if (probs)
            for (int j = 0; j < nsrc; ++j)
                probs[t * nsrc + j] = p[j];

        /* In-place writes, after every read of this token (R3, R4, R5). */
        if (delta)
            for (int64_t h = 0; h < H; ++h)
                prefix[t * H + h] = bf16_value_to_bits(cur[h]);
        if (widx >= 0) {
            uint16_t *row = blocks + t * token_stride + (int64_t)widx * slot_stride;
            for (int64_t h = 0; h < H; ++h)
                row[h] = bf16_value_to_bits(cur[h]);
        }
    }

    free(src); free(cur); free(xhat); free(y); free(l); free(p);
    return 0;
}

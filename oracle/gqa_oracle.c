/*
 * gqa_oracle.c -- plain, slow fp64 CPU reference for grouped-query
 * scaled-dot-product attention and for the group-affine 4-bit KV encoding.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg are the only callers.  Nothing here is shared with the HIP
 * library: no headers, no helpers, no constants.
 *
 * What is computed (one output row per (b, h, i)):
 *
 *   O[b,h,i,:] = sum_{j in J} softmax_j( scale * <Q[b,h,i,:], K[b,g,j,:]> ) V[b,g,j,:]
 *
 *   g = floor(h / G), G = Hq / Hkv   (query heads come in contiguous groups
 *                                     that share one KV head)
 *   J = { j : j < n_b  and  (not causal  or  j <= i + (n_b - Tq)) }
 *
 * with n_b the number of valid key rows of request b.  Sources:
 *  - "2x faster Qwen2 decode on Metal in Candle", section "Why It Matters: 7x
 *    KV Expansion": the fused kernel reads the few KV heads directly through a
 *    GQA stride instead of materialising one copy per query head.
 *  - "Fused attention makes a 4,096-token Qwen2 prefill on Metal 4.5x faster",
 *    section "Cause and workaround", points 1 and 2: K/V are given before
 *    repeat_kv (query heads a multiple of KV heads) and, with the causal flag,
 *    the queries are aligned to the end of the keys, so query i of a chunk
 *    that starts at key offset Tk - Tq attends to every key up to i + Tk - Tq.
 *  - same page, section "Cause and workaround", its opening paragraph on the
 *    cause: the unfused path is repeat_kv, a matmul, scale, mask, softmax and
 *    a second matmul -- the plain definition written out below.
 *
 * A row whose visible set J is empty (possible only for a zero-length request)
 * gets an all-zero output.
 *
 * Two options (gqa_oracle_attend_ex), from the pages' remarks on what the
 * fused kernels leave out -- the Fornace prefill page, "What this does not
 * prove" (no sliding window is applied; Qwen2.5's window never masks, other
 * models can differ) and the VeloxQuant-MLX "attention" posts, "Part 4" (the
 * SDPA signature the fused decode path intercepts carries `sinks`):
 *  - window W >= 1: only the W most recent keys up to the row's own position
 *    are visible, J = { j in J : j > i + (n_b - Tq) - W } (for decode, the
 *    last W keys);
 *  - sinks: one logit sink_h per query head (in the units of the scaled
 *    scores) that joins the softmax's normaliser and carries no value:
 *      O = sum_j e^{s_j} V_j / (e^{sink_h} + sum_j e^{s_j}).
 *
 * Arithmetic: every stored element is widened exactly to double by the
 * caller; dot products, exp (libm) and sums run in double in ascending index
 * order; the result is returned unrounded.
 *
 * Pins: every function here is checked by tests/test_oracle_*.py against a
 * brute force with explicitly repeated KV heads, a library attention routine,
 * closed forms and invariants (see the test files' headers).
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

int gqa_oracle_version(void) { return 1; }

int gqa_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * q     [B, Hq,  Tq,    D]
 * k, v  [B, Hkv, s_cap, D]   (only rows j < n_b are read)
 * out   [B, Hq,  Tq,    D]
 * kv_lens[b] = n_b, 0 <= n_b <= s_cap
 * probs (optional, may be NULL) [B, Hq, Tq, s_cap]: the softmax weights,
 *       zero where a key is not visible.
 * nthreads <= 0 means the OpenMP default.
 */
int gqa_oracle_attend_ex(const double *q, const double *k, const double *v, double *out,
                         int B, int Hq, int Hkv, int Tq, int D, int s_cap,
                         const int32_t *kv_lens, int causal, double scale, int window,
                         const double *sinks, double *probs, int nthreads);

int gqa_oracle_attend(const double *q, const double *k, const double *v, double *out,
                      int B, int Hq, int Hkv, int Tq, int D, int s_cap,
                      const int32_t *kv_lens, int causal, double scale,
                      double *probs, int nthreads)
{
    return gqa_oracle_attend_ex(q, k, v, out, B, Hq, Hkv, Tq, D, s_cap, kv_lens, causal, scale, 0, NULL,
                                probs, nthreads);
}

/* window <= 0: no window; sinks: NULL or [Hq] logits. */
int gqa_oracle_attend_ex(const double *q, const double *k, const double *v, double *out,
                         int B, int Hq, int Hkv, int Tq, int D, int s_cap,
                         const int32_t *kv_lens, int causal, double scale, int window,
                         const double *sinks, double *probs, int nthreads)
{
    if (!q || !k || !v || !out || !kv_lens)
        return ORACLE_ERR_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || D < 1 || s_cap < 1)
        return ORACLE_ERR_ARG;
    if (Hq % Hkv != 0)
        return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (kv_lens[b] < 0 || kv_lens[b] > s_cap)
            return ORACLE_ERR_ARG;

    const int G = Hq / Hkv;
    const long n_rows = (long)B * Hq * Tq;
    int failed = 0;

#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)s_cap);
        if (!s) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long r = 0; r < n_rows; ++r) {
            if (!s)
                continue;
            const int i = (int)(r % Tq);
            const int h = (int)((r / Tq) % Hq);
            const int b = (int)(r / ((long)Tq * Hq));
            const int g = h / G;
            const int n = kv_lens[b];

            /* visible keys: first <= j < limit; j < n, and j <= i + (n - Tq)
               when causal; with a window, j > (last visible key) - window */
            long limit = n;
            if (causal) {
                long last = (long)i + ((long)n - Tq);
                if (last + 1 < limit)
                    limit = last + 1;
                if (limit < 0)
                    limit = 0;
            }
            long first = 0;
            if (window > 0 && limit - window > 0)
                first = limit - window;

            const double *qi = q + (size_t)r * D;
            const double *kb = k + ((size_t)b * Hkv + g) * (size_t)s_cap * D;
            const double *vb = v + ((size_t)b * Hkv + g) * (size_t)s_cap * D;
            double *oi = out + (size_t)r * D;
            double *pi = probs ? probs + (size_t)r * s_cap : NULL;

            if (pi)
                for (int j = 0; j < s_cap; ++j)
                    pi[j] = 0.0;

            if (limit == 0) {
                for (int d = 0; d < D; ++d)
                    oi[d] = 0.0;
                continue;
            }

            /* scores */
            double m = -INFINITY;
            for (long j = first; j < limit; ++j) {
                const double *kj = kb + (size_t)j * D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += qi[d] * kj[d];
                s[j] = scale * dot;
                if (s[j] > m)
                    m = s[j];
            }

            /* softmax weights (shifted by the row maximum, the sink
               included) and their sum; the sink adds to the sum only */
            const double sink = sinks ? sinks[h] : -INFINITY;
            if (sink > m)
                m = sink;
            double l = 0.0;
            for (long j = first; j < limit; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            if (sinks)
                l += exp(sink - m);

            /* weighted sum of value rows */
            for (int d = 0; d < D; ++d)
                oi[d] = 0.0;
            for (long j = first; j < limit; ++j) {
                const double *vj = vb + (size_t)j * D;
                for (int d = 0; d < D; ++d)
                    oi[d] += s[j] * vj[d];
            }
            for (int d = 0; d < D; ++d)
                oi[d] /= l;

            if (pi)
                for (long j = first; j < limit; ++j)
                    pi[j] = s[j] / l;
        }
        free(s);
    }
    return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Group-affine 4-bit KV encoding (VeloxQuant-MLX "attention" posts: the
 * fused group-affine decode+attention kernel behind the KIVI-style cache, and
 * its call that passes codes, scales and biases with the group size).
 *
 * Layout of one cache row of D elements: D/2 bytes, element 2j in the low
 * nibble of byte j and element 2j+1 in the high nibble; one f16 scale s and
 * one f16 bias b per group of `group` consecutive elements.  The value of
 * element e with code c in group e/group is  s*c + b,  rounded once to
 * float32 (s*c is exact in float32: an 11-bit significand times a 4-bit
 * integer, so this equals a fused multiply-add).
 * ------------------------------------------------------------------------- */

/* IEEE 754 binary16 -> binary32, from the format's definition (exact). */
static float half_bits_to_float(uint16_t hbits)
{
    const int sign = (hbits >> 15) & 1;
    const int expo = (hbits >> 10) & 0x1F;
    const int frac = hbits & 0x3FF;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);                 /* subnormal or zero */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25);  /* (1 + frac/1024) * 2^(expo-15) */
    return (float)(sign ? -mag : mag);
}

/*
 * IEEE 754 binary32 -> binary16 bits, rounded to nearest, ties to even, from
 * the format's definition: a finite magnitude below 2^-14 is a multiple of
 * 2^-24 (subnormal; 1024 * 2^-24 is the smallest normal, whose encoding
 * 0x0400 the same integer gives); otherwise 1.f * 2^e with 10 fraction bits
 * and e + 15 in 1..30; magnitudes that round past 65504 become infinity.
 * Every step is exact in double except the one rint (ties to even).
 */
static uint16_t float_to_half_bits(float f)
{
    const uint16_t sign = signbit(f) ? 0x8000 : 0;
    const double a = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00);
    if (isinf(f))
        return (uint16_t)(sign | 0x7C00);
    if (a < ldexp(1.0, -14)) {
        const double n = rint(a * ldexp(1.0, 24));   /* 0 .. 1024 */
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e;
    const double m = frexp(a, &e);                   /* a = m * 2^e, m in [0.5, 1) */
    double n = rint(m * 2048.0);                     /* 1024 .. 2048: 11 significant bits */
    e -= 1;                                          /* a = (n / 1024) * 2^e */
    if (n == 2048.0) {
        n = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7C00);            /* rounds past 65504 */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

int gqa_oracle_f32_to_f16(const float *in, uint16_t *out, long n)
{
    if (!in || !out || n < 0)
        return ORACLE_ERR_ARG;
    for (long i = 0; i < n; ++i)
        out[i] = float_to_half_bits(in[i]);
    return ORACLE_OK;
}

int gqa_oracle_f16_to_f32(const uint16_t *in, float *out, long n)
{
    if (!in || !out || n < 0)
        return ORACLE_ERR_ARG;
    for (long i = 0; i < n; ++i)
        out[i] = half_bits_to_float(in[i]);
    return ORACLE_OK;
}

/* codes [n_rows, D] (one byte per element, 0..15) from packed [n_rows, D/2] */
int gqa_oracle_q4_unpack(const uint8_t *packed, long n_rows, int D, uint8_t *codes)
{
    if (!packed || !codes || n_rows < 0 || D < 2 || D % 2)
        return ORACLE_ERR_ARG;
    for (long r = 0; r < n_rows; ++r) {
        const uint8_t *row = packed + (size_t)r * (D / 2);
        for (int e = 0; e < D; ++e) {
            const uint8_t byte = row[e / 2];
            codes[(size_t)r * D + e] = (e % 2 == 0) ? (uint8_t)(byte & 0x0F) : (uint8_t)(byte >> 4);
        }
    }
    return ORACLE_OK;
}

/* out [n_rows, D] float32 = s*c + b per element (single rounding) */
int gqa_oracle_q4_dequant(const uint8_t *packed, const uint16_t *scales, const uint16_t *biases,
                          long n_rows, int D, int group, float *out)
{
    if (!packed || !scales || !biases || !out || n_rows < 0 || D < 2 || D % 2 ||
        group < 1 || D % group)
        return ORACLE_ERR_ARG;
    const int n_groups = D / group;
    uint8_t *codes = (uint8_t *)malloc((size_t)D);
    if (!codes)
        return ORACLE_ERR_NOMEM;
    for (long r = 0; r < n_rows; ++r) {
        gqa_oracle_q4_unpack(packed + (size_t)r * (D / 2), 1, D, codes);
        for (int e = 0; e < D; ++e) {
            const int grp = e / group;
            const float s = half_bits_to_float(scales[(size_t)r * n_groups + grp]);
            const float b = half_bits_to_float(biases[(size_t)r * n_groups + grp]);
            out[(size_t)r * D + e] = fmaf(s, (float)codes[e], b);
        }
    }
    free(codes);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Min-max group-affine 4-bit quantizer: what the incremental cache append
 * computes for each new row (VeloxQuant-MLX "attention" posts, "Part 4":
 * re-quantizing the whole K/V history every decode step cost ~25 ms/step,
 * fixed by quantizing only the newly aged rows; the encoding is the one the
 * fused decode reads: codes, and an f16 scale and bias per group).
 *
 * The pages do not print the quantizer; the reading taken is the plain
 * min-max affine map onto the 16 codes, in float32 on the input values
 * (f16, bf16 and f32 inputs all widen exactly), for each group of `group`
 * consecutive elements of a row:
 *   lo = min x, hi = max x                        (exact)
 *   s16 = f16(fl32(fl32(hi - lo) / 15)),  b16 = f16(lo)     (ties to even;
 *         a zero minimum or step is taken as +0, so that a group holding
 *         both -0 and +0 has one encoding)
 *   s = f32(s16), b = f32(b16)
 *   c  = 0                                        if s == 0
 *        clamp(rint(fl32(fl32(x - b) / s)), 0, 15) otherwise (rint: ties to even)
 * Inputs must be finite, with lo and (hi - lo) / 15 inside the f16 range.
 * ------------------------------------------------------------------------- */

/* x [n_rows, D] float32 -> packed codes [n_rows, D/2], scale and bias bits
   [n_rows, D/group] (IEEE binary16) */
int gqa_oracle_q4_quantize(const float *x, long n_rows, int D, int group, uint8_t *packed,
                           uint16_t *scales, uint16_t *biases)
{
    if (!x || !packed || !scales || !biases || n_rows < 0 || D < 2 || D % 2 || group < 1 || D % group)
        return ORACLE_ERR_ARG;
    const int n_groups = D / group;
    for (long r = 0; r < n_rows; ++r) {
        const float *xr = x + (size_t)r * D;
        uint8_t *pr = packed + (size_t)r * (D / 2);
        memset(pr, 0, (size_t)(D / 2));
        for (int g = 0; g < n_groups; ++g) {
            const float *xg = xr + (size_t)g * group;
            float lo = xg[0], hi = xg[0];
            for (int e = 1; e < group; ++e) {
                if (xg[e] < lo)
                    lo = xg[e];
                if (xg[e] > hi)
                    hi = xg[e];
            }
            if (lo == 0.0f)
                lo = 0.0f;                               /* +0 */
            const float range = hi - lo;
            float step = range / 15.0f;
            if (step == 0.0f)
                step = 0.0f;                             /* +0 */
            const uint16_t sh = float_to_half_bits(step);
            const uint16_t bh = float_to_half_bits(lo);
            scales[(size_t)r * n_groups + g] = sh;
            biases[(size_t)r * n_groups + g] = bh;
            const float sv = half_bits_to_float(sh);
            const float bv = half_bits_to_float(bh);
            for (int e = 0; e < group; ++e) {
                int c = 0;
                if (sv != 0.0f) {
                    const float t = xg[e] - bv;
                    const float u = t / sv;
                    const float k = rintf(u);
                    c = k < 0.0f ? 0 : (k > 15.0f ? 15 : (int)k);
                }
                const int idx = g * group + e;
                pr[idx / 2] |= (uint8_t)((idx % 2 == 0) ? c : (c << 4));
            }
        }
    }
    return ORACLE_OK;
}

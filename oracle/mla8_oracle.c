/*
 * mla8 oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of what the fp8 latent-KV
 * MLA decode path computes, in double precision wherever the pages leave the
 * precision open.  Only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load this file's library.  It shares no code, header,
 * table or constant generator with the HIP library under fp8_mla_latent_amd/.
 *
 * Sources (cited by page title and passage, see the citation key in the repo
 * design notes):
 *   [KV8-base]  colibri PR #300 "KV8 long-context CUDA: fp8 device shadow,
 *               split-T kernels, DSA-aware gather", first commit message
 *               ("KV8 base"), the c/kv_fp8.h and attention_rows bullets.
 *   [KV8-long]  same page, second commit message ("KV8 long-context CUDA"),
 *               the kv_dev_sync8 / split-T / DSA-gather bullets, and the PR
 *               description that restates them.
 *   [B1-FMHA]   "B1 Mixed FP8/BF16 FMHA first pass": the mixed cache format,
 *               noPE part as e4m3 bytes with a per-row f32 scale and the RoPE
 *               part kept in bf16 (the 512 / 448 / 64 shape).
 *   [B2-indexer] "B1 Mixed FP8/BF16 FMHA first pass" site, commit message of
 *               the B2 fp8 indexer score + top-k kernel: the query (64 indexer
 *               heads x 128) quantized to fp8, the keys read as e4m3, then
 *               dequantization by q_scale * k_scale, ReLU, a weighted sum over
 *               the heads and a top-k over the rows.
 *
 * Readings of points the pages leave open are listed in the design notes; the
 * ones this file depends on are repeated next to the code that takes them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------- */
/* e4m3 decode.  [KV8-base] names a 256-entry decode table for the e4m3 byte
 * format whose finite range is +/-448; that range identifies the OCP "E4M3FN"
 * variant: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, and S.1111.111 reserved for NaN.  The value is computed here from
 * that definition, byte by byte, rather than typed in. */
EXPORT double mla8o_dec(uint8_t c)
{
    int s = c >> 7;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN; /* the format's only NaN encodings, 0x7F and 0xFF */
    if (e == 0)
        v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------- */
/* e4m3 encode.  [KV8-base] c/kv_fp8.h bullet: round-to-nearest-even encoder,
 * saturating at +/-448, signed zero preserved, NaN stored as an inert zero.
 * Readings: one rounding from the f32 input to the nearest e4m3 value with ties
 * to the even mantissa; anything at or beyond 448 in magnitude (infinity
 * included) becomes +/-448; NaN of either sign becomes the byte 0x00.
 * Written from the definition of rounding to a 3-bit mantissa: scale |x| so the
 * kept bits become the integer part, round that integer half-to-even with rint()
 * (the C default rounding mode), then rebuild the byte. */
EXPORT uint8_t mla8o_enc(float x)
{
    if (isnan(x))
        return 0x00;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal e4m3 range: multiples of 2^-9; 8 * 2^-9 is the smallest
         * normal 2^-6, whose byte 0x08 is exactly the integer 8 */
        double q = rint(a * 512.0); /* exact product, 0..8 */
        return sign | (uint8_t)q;
    }
    int ex;
    (void)frexp(a, &ex);  /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;       /* a in [2^e, 2^(e+1)), e in [-6, 8] */
    double q = rint(ldexp(a, 3 - e)); /* 3 kept bits after the leading one: 8..16 */
    if (q == 16.0) {      /* rounding carried into the next binade */
        q = 8.0;
        e += 1;
    }
    return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

EXPORT void mla8o_encode_array(const float* x, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = mla8o_enc(x[i]);
}

EXPORT void mla8o_decode_array(const uint8_t* c, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = mla8o_dec(c[i]);
}

/* ------------------------------------------------------------------------- */
/* Per-row quantizer.  [KV8-base]: rows of Lc kv_lora then Rc qk_rope values
 * are stored as e4m3 bytes with one f32 scale per row equal to amax/448; the
 * quantizer guards against a subnormal amax, for which 448/amax would overflow
 * to +inf.  Readings: amax is taken over the finite entries only; the stored
 * scale is the f32 quotient amax/448; entries are encoded from the f32 product
 * x * f32(448/amax); when that inverse is not finite the guard sets it to 0,
 * so the row's codes are signed zeros (NaN inputs give 0x00).  All of this is
 * f32 arithmetic because the page fixes the scale as an f32. */
EXPORT void mla8o_quantize_row(const float* x, int32_t d, uint8_t* codes, float* scale)
{
    float amax = 0.0f;
    for (int32_t i = 0; i < d; ++i) {
        float v = x[i];
        if (isfinite(v) && fabsf(v) > amax)
            amax = fabsf(v);
    }
    volatile float num = 448.0f; /* keep both quotients as run-time f32 divisions */
    float sc = amax / num;
    float inv = num / amax;
    if (!isfinite(inv))
        inv = 0.0f;
    for (int32_t i = 0; i < d; ++i) {
        volatile float y = x[i] * inv;
        codes[i] = mla8o_enc(y);
    }
    *scale = sc;
}

EXPORT void mla8o_quantize_rows(const float* x, int64_t n, int32_t d, uint8_t* codes,
                                float* scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        mla8o_quantize_row(x + r * (int64_t)d, d, codes + r * (int64_t)d, scales + r);
}

/* ------------------------------------------------------------------------- */
/* Absorbed attention of one query vector over a list of cached rows.
 * [KV8-base]: in the absorbed form the latent row is both key and value.
 * Readings: the key is the whole dequantized row (Lc then Rc, D = Lc + Rc
 * values), the value is its first Lc entries; the query is q_lat || q_rope;
 * the score is sm * q . k; softmax uses the natural exponential; the output is
 * the softmax-weighted sum of values and lse = ln sum_t e^{s_t}.
 * Row list entries outside [0, t_rows) are skipped.  If no row is left the
 * output is all zeros and lse = -inf.
 * Everything is computed in double: dec(c) * scale is exact in double. */
static void attend_rows(const uint8_t* codes, const float* scales, int64_t t_rows, int32_t lc,
                        int32_t rc, const int64_t* rows, int64_t nrows, const double* q,
                        double sm, double* out, double* lse)
{
    int32_t d = lc + rc;
    double* s = (double*)malloc(sizeof(double) * (nrows > 0 ? nrows : 1));
    double smax = -INFINITY;
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t t = rows[j];
        if (t < 0 || t >= t_rows) {
            s[j] = -INFINITY;
            continue;
        }
        double acc = 0.0;
        for (int32_t i = 0; i < d; ++i)
            acc += q[i] * (mla8o_dec(codes[t * d + i]) * (double)scales[t]);
        s[j] = sm * acc;
        if (s[j] > smax)
            smax = s[j];
    }
    for (int32_t i = 0; i < lc; ++i)
        out[i] = 0.0;
    if (smax == -INFINITY) {
        *lse = -INFINITY;
        free(s);
        return;
    }
    double z = 0.0;
    for (int64_t j = 0; j < nrows; ++j) {
        if (s[j] == -INFINITY)
            continue;
        int64_t t = rows[j];
        double p = exp(s[j] - smax);
        z += p;
        for (int32_t i = 0; i < lc; ++i)
            out[i] += p * (mla8o_dec(codes[t * d + i]) * (double)scales[t]);
    }
    for (int32_t i = 0; i < lc; ++i)
        out[i] /= z;
    *lse = smax + log(z);
    free(s);
}

static void make_query(const float* q_lat, const float* q_rope, int32_t lc, int32_t rc,
                       double* q)
{
    for (int32_t i = 0; i < lc; ++i)
        q[i] = (double)q_lat[i];
    for (int32_t i = 0; i < rc; ++i)
        q[lc + i] = (double)q_rope[i];
}

/* Dense decode: every head attends rows [0, t_rows).  [KV8-long] split-T
 * bullet: decode attends the whole device-resident shadow. */
EXPORT void mla8o_decode(const uint8_t* codes, const float* scales, int64_t t_rows, int32_t lc,
                         int32_t rc, const float* q_lat, const float* q_rope, int32_t n_heads,
                         float sm_scale, double* out, double* lse)
{
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (t_rows > 0 ? t_rows : 1));
    for (int64_t t = 0; t < t_rows; ++t)
        rows[t] = t;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t h = 0; h < n_heads; ++h) {
        double q[4096];
        make_query(q_lat + (int64_t)h * lc, q_rope + (int64_t)h * rc, lc, rc, q);
        attend_rows(codes, scales, t_rows, lc, rc, rows, t_rows, q, (double)sm_scale,
                    out + (int64_t)h * lc, lse + h);
    }
    free(rows);
}

/* Selected-row decode.  [KV8-long] DSA bullet: attend only the selected rows,
 * given as absolute row indices into the shadow.  Readings: the selection is a
 * multiset (a repeated index counts as often as it appears); entries outside
 * [0, t_rows) are skipped. */
EXPORT void mla8o_decode_sel(const uint8_t* codes, const float* scales, int64_t t_rows,
                             int32_t lc, int32_t rc, const int32_t* sel, int64_t ns,
                             const float* q_lat, const float* q_rope, int32_t n_heads,
                             float sm_scale, double* out, double* lse)
{
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (ns > 0 ? ns : 1));
    for (int64_t j = 0; j < ns; ++j)
        rows[j] = sel[j];
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t h = 0; h < n_heads; ++h) {
        double q[4096];
        make_query(q_lat + (int64_t)h * lc, q_rope + (int64_t)h * rc, lc, rc, q);
        attend_rows(codes, scales, t_rows, lc, rc, rows, ns, q, (double)sm_scale,
                    out + (int64_t)h * lc, lse + h);
    }
    free(rows);
}

/* Batched causal attention.  [KV8-long]: the batch/prefill path runs one
 * (query, head) pair per block over the cached rows.  Reading: query s sits at
 * absolute position pos0 + s and attends rows 0 .. pos0 + s inclusive (its own
 * freshly appended row included). */
EXPORT void mla8o_batch(const uint8_t* codes, const float* scales, int64_t t_rows, int32_t lc,
                        int32_t rc, const float* q_lat, const float* q_rope, int32_t n_q,
                        int64_t pos0, int32_t n_heads, float sm_scale, double* out,
                        double* lse)
{
    int64_t n = pos0 + n_q;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
    for (int64_t t = 0; t < n; ++t)
        rows[t] = t;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sh = 0; sh < (int64_t)n_q * n_heads; ++sh) {
        int64_t s = sh / n_heads;
        double q[4096];
        make_query(q_lat + sh * lc, q_rope + sh * rc, lc, rc, q);
        attend_rows(codes, scales, t_rows, lc, rc, rows, pos0 + s + 1, q, (double)sm_scale,
                    out + sh * lc, lse + sh);
    }
    free(rows);
}

/* ------------------------------------------------------------------------- */
/* Split-T form of the dense decode.  [KV8-long] split-T bullet: the rows are
 * cut into P chunks; each chunk yields an online-softmax partial (context
 * cl[K], running max m, normaliser z) and a log-sum-exp merge combines them:
 *   M = max_p m_p,  w_p = e^{m_p - M},
 *   out = sum_p w_p cl_p / sum_p w_p z_p,  lse = M + ln sum_p w_p z_p.
 * Inside a chunk the partial is written in its streaming form: a running max
 * that, when it grows, rescales z and cl by e^{m_old - m_new}.
 * An empty chunk has m = -inf, z = 0, cl = 0 and weight 0. */
EXPORT void mla8o_decode_chunked(const uint8_t* codes, const float* scales, int64_t t_rows,
                                 int32_t lc, int32_t rc, const float* q_lat,
                                 const float* q_rope, int32_t n_heads, float sm_scale,
                                 int64_t n_chunks, double* out, double* lse)
{
    int32_t d = lc + rc;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t h = 0; h < n_heads; ++h) {
        double q[4096];
        make_query(q_lat + (int64_t)h * lc, q_rope + (int64_t)h * rc, lc, rc, q);
        double* pm = (double*)malloc(sizeof(double) * n_chunks);
        double* pz = (double*)malloc(sizeof(double) * n_chunks);
        double* pcl = (double*)calloc((size_t)n_chunks * lc, sizeof(double));
        for (int64_t p = 0; p < n_chunks; ++p) {
            int64_t t0 = t_rows * p / n_chunks, t1 = t_rows * (p + 1) / n_chunks;
            double m = -INFINITY, z = 0.0;
            double* cl = pcl + p * lc;
            for (int64_t t = t0; t < t1; ++t) {
                double acc = 0.0;
                for (int32_t i = 0; i < d; ++i)
                    acc += q[i] * (mla8o_dec(codes[t * d + i]) * (double)scales[t]);
                double st = (double)sm_scale * acc;
                if (st > m) {
                    double r = exp(m - st); /* 0 when m = -inf */
                    z *= r;
                    for (int32_t i = 0; i < lc; ++i)
                        cl[i] *= r;
                    m = st;
                }
                double e = exp(st - m);
                z += e;
                for (int32_t i = 0; i < lc; ++i)
                    cl[i] += e * (mla8o_dec(codes[t * d + i]) * (double)scales[t]);
            }
            pm[p] = m;
            pz[p] = z;
        }
        double mmax = -INFINITY;
        for (int64_t p = 0; p < n_chunks; ++p)
            if (pm[p] > mmax)
                mmax = pm[p];
        double* o = out + (int64_t)h * lc;
        for (int32_t i = 0; i < lc; ++i)
            o[i] = 0.0;
        if (mmax == -INFINITY) {
            lse[h] = -INFINITY;
        } else {
            double zz = 0.0;
            for (int64_t p = 0; p < n_chunks; ++p) {
                double w = (pm[p] == -INFINITY) ? 0.0 : exp(pm[p] - mmax);
                zz += w * pz[p];
                for (int32_t i = 0; i < lc; ++i)
                    o[i] += w * pcl[p * lc + i];
            }
            for (int32_t i = 0; i < lc; ++i)
                o[i] /= zz;
            lse[h] = mmax + log(zz);
        }
        free(pm);
        free(pz);
        free(pcl);
    }
}

/* Threads for the following calls (timing the oracle on one core or all);
 * n < 1 restores the runtime's default.  No effect without OpenMP. */
EXPORT void mla8o_set_threads(int n)
{
#ifdef _OPENMP
    static int dflt = 0;
    if (dflt == 0)
        dflt = omp_get_max_threads();
    omp_set_num_threads(n >= 1 ? n : dflt);
#else
    (void)n;
#endif
}

/* Number of threads the OpenMP runtime will use (for reporting). */
EXPORT int mla8o_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}

/* ------------------------------------------------------------------------- */
/* Indexer scores.  [B2-indexer]: for one query token, indexer head j has a
 * query vector q_j of ihd values, quantized to e4m3 with a scale q_scale_j;
 * the keys are e4m3 rows with a scale k_scale_t; a head's score for row t is
 * the dot product of the two byte vectors dequantized by q_scale_j * k_scale_t,
 * passed through ReLU, and the row's index score is the sum over heads of
 * w_j times that.  Readings: q_j is quantized with the per-row quantizer
 * above (its scale is the head's amax/448); the keys are rows of the same
 * shadow format with Lc = ihd and Rc = 0; w is f32 of either sign.
 *     I_t = sum_j w_j * max(0, q_scale_j * k_scale_t * sum_d dec(q8_jd) dec(k8_td))
 * The dot product of decoded bytes is exact in double (each product has at
 * most 8 significant bits and their exponents span less than 53 bits for
 * ihd <= 256), so I_t carries only the rounding of its last few operations. */
EXPORT void mla8o_index_scores(const uint8_t* k_codes, const float* k_scales, int64_t t_rows,
                               int32_t ihd, const float* q, const float* w, int32_t n_ih,
                               double* scores)
{
    uint8_t* qc = (uint8_t*)malloc((size_t)n_ih * (size_t)ihd);
    float* qs = (float*)malloc(sizeof(float) * (size_t)(n_ih > 0 ? n_ih : 1));
    for (int32_t j = 0; j < n_ih; ++j)
        mla8o_quantize_row(q + (int64_t)j * ihd, ihd, qc + (int64_t)j * ihd, qs + j);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < t_rows; ++t) {
        double acc = 0.0;
        for (int32_t j = 0; j < n_ih; ++j) {
            double dot = 0.0;
            for (int32_t i = 0; i < ihd; ++i)
                dot += mla8o_dec(qc[(int64_t)j * ihd + i]) * mla8o_dec(k_codes[t * ihd + i]);
            double sj = (double)qs[j] * (double)k_scales[t] * dot;
            acc += (double)w[j] * (sj > 0.0 ? sj : 0.0);
        }
        scores[t] = acc;
    }
    free(qc);
    free(qs);
}

/* ------------------------------------------------------------------------- */
/* bf16.  [B1-FMHA]: the RoPE part of a mixed row stays in bf16.  Readings: one
 * round-to-nearest-even rounding of the f32 value onto bfloat16 (8 significant
 * bits, the f32 exponent range, subnormals included); a value that rounds to
 * 2^128 or beyond becomes +/-inf; +/-inf stay; NaN becomes the quiet NaN 0x7FC0
 * with its sign.  Written from the definition: scale |x| so that the kept bits
 * are the integer part, round with rint, and take the bf16 bit pattern of the
 * (exactly representable) result, which is the top half of its f32 pattern. */
EXPORT uint16_t mla8o_bf16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    if (isnan(x))
        return sign | 0x7FC0;
    if (isinf(x))
        return sign | 0x7F80;
    double a = fabs((double)x);
    if (a == 0.0)
        return sign;
    int ex;
    (void)frexp(a, &ex);
    int e = ex - 1;        /* a in [2^e, 2^(e+1)) */
    if (e < -126)
        e = -126;          /* subnormal range: quantum 2^-133 */
    double v = ldexp(rint(ldexp(a, 7 - e)), e - 7);
    if (v >= ldexp(1.0, 128))
        return sign | 0x7F80;
    float fv = (float)v;   /* exact */
    uint32_t b;
    memcpy(&b, &fv, 4);
    return sign | (uint16_t)(b >> 16);
}

EXPORT void mla8o_bf16_array(const float* x, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = mla8o_bf16(x[i]);
}

/* Value of a bf16 bit pattern, from the format's definition: 1 sign bit, 8
 * exponent bits with bias 127, 7 mantissa bits. */
EXPORT double mla8o_bf16_value(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 0xFF, m = b & 0x7F;
    double v;
    if (e == 0xFF)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -133);
    else
        v = ldexp(1.0 + m / 128.0, e - 127);
    return s ? -v : v;
}

/* Mixed rows.  [B1-FMHA] storage format.  Readings: a row is lc noPE values
 * then rc RoPE values (the page's 448 + 64); the noPE part goes through the
 * per-row quantizer above (its scale is the noPE part's amax/448); the RoPE part
 * is stored as bf16; a stored row is lc code bytes then rc little-endian bf16
 * values, lc + 2 rc bytes. */
EXPORT void mla8o_quantize_rows_mx(const float* x, int64_t n, int32_t lc, int32_t rc,
                                   uint8_t* rows, float* scales)
{
    int64_t d = lc + rc, rb = lc + 2 * (int64_t)rc;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        mla8o_quantize_row(x + r * d, lc, rows + r * rb, scales + r);
        for (int32_t i = 0; i < rc; ++i) {
            uint16_t b = mla8o_bf16(x[r * d + lc + i]);
            rows[r * rb + lc + 2 * i] = (uint8_t)(b & 0xFF);
            rows[r * rb + lc + 2 * i + 1] = (uint8_t)(b >> 8);
        }
    }
}

/* Attention over mixed rows, for one head, over a list of row indices (a
 * multiset; entries outside [0, t_rows) are skipped, as for attend_rows).
 * Readings: the key of row t is the noPE part dequantized (dec(code) *
 * scale_t) followed by the RoPE part's bf16 values, unscaled; the value is the
 * dequantized noPE part (output width lc); the rest is the attention of
 * attend_rows above. */
static void attend_rows_mx(const uint8_t* rows, const float* scales, int64_t t_rows, int32_t lc,
                           int32_t rc, const int64_t* list, int64_t nlist, const double* q,
                           double sm, double* o, double* lse)
{
    int64_t rb = lc + 2 * (int64_t)rc;
    double* s = (double*)malloc(sizeof(double) * (nlist > 0 ? nlist : 1));
    double smax = -INFINITY;
    for (int64_t j = 0; j < nlist; ++j) {
        int64_t t = list[j];
        if (t < 0 || t >= t_rows) {
            s[j] = -INFINITY;
            continue;
        }
        const uint8_t* row = rows + t * rb;
        double acc = 0.0;
        for (int32_t i = 0; i < lc; ++i)
            acc += q[i] * (mla8o_dec(row[i]) * (double)scales[t]);
        for (int32_t i = 0; i < rc; ++i) {
            uint16_t b = (uint16_t)(row[lc + 2 * i] | (row[lc + 2 * i + 1] << 8));
            acc += q[lc + i] * mla8o_bf16_value(b);
        }
        s[j] = sm * acc;
        if (s[j] > smax)
            smax = s[j];
    }
    for (int32_t i = 0; i < lc; ++i)
        o[i] = 0.0;
    if (smax == -INFINITY) {
        *lse = -INFINITY;
        free(s);
        return;
    }
    double z = 0.0;
    for (int64_t j = 0; j < nlist; ++j) {
        if (s[j] == -INFINITY)
            continue;
        int64_t t = list[j];
        double p = exp(s[j] - smax);
        z += p;
        for (int32_t i = 0; i < lc; ++i)
            o[i] += p * (mla8o_dec(rows[t * rb + i]) * (double)scales[t]);
    }
    for (int32_t i = 0; i < lc; ++i)
        o[i] /= z;
    *lse = smax + log(z);
    free(s);
}

/* Selected-row decode over mixed rows ([KV8-long] DSA bullet with the mixed
 * row of [B1-FMHA]). */
EXPORT void mla8o_decode_sel_mx(const uint8_t* rows, const float* scales, int64_t t_rows,
                                int32_t lc, int32_t rc, const int32_t* sel, int64_t ns,
                                const float* q_lat, const float* q_rope, int32_t n_heads,
                                float sm_scale, double* out, double* lse)
{
    int64_t* list = (int64_t*)malloc(sizeof(int64_t) * (ns > 0 ? ns : 1));
    for (int64_t j = 0; j < ns; ++j)
        list[j] = sel[j];
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t h = 0; h < n_heads; ++h) {
        double q[4096];
        make_query(q_lat + (int64_t)h * lc, q_rope + (int64_t)h * rc, lc, rc, q);
        attend_rows_mx(rows, scales, t_rows, lc, rc, list, ns, q, (double)sm_scale,
                       out + (int64_t)h * lc, lse + h);
    }
    free(list);
}

/* Dense decode over mixed rows. */
EXPORT void mla8o_decode_mx(const uint8_t* rows, const float* scales, int64_t t_rows, int32_t lc,
                            int32_t rc, const float* q_lat, const float* q_rope, int32_t n_heads,
                            float sm_scale, double* out, double* lse)
{
    int64_t rb = lc + 2 * (int64_t)rc;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t h = 0; h < n_heads; ++h) {
        double q[4096];
        make_query(q_lat + (int64_t)h * lc, q_rope + (int64_t)h * rc, lc, rc, q);
        double* o = out + (int64_t)h * lc;
        double* s = (double*)malloc(sizeof(double) * (t_rows > 0 ? t_rows : 1));
        double smax = -INFINITY;
        for (int64_t t = 0; t < t_rows; ++t) {
            const uint8_t* row = rows + t * rb;
            double acc = 0.0;
            for (int32_t i = 0; i < lc; ++i)
                acc += q[i] * (mla8o_dec(row[i]) * (double)scales[t]);
            for (int32_t i = 0; i < rc; ++i) {
                uint16_t b = (uint16_t)(row[lc + 2 * i] | (row[lc + 2 * i + 1] << 8));
                acc += q[lc + i] * mla8o_bf16_value(b);
            }
            s[t] = (double)sm_scale * acc;
            if (s[t] > smax)
                smax = s[t];
        }
        for (int32_t i = 0; i < lc; ++i)
            o[i] = 0.0;
        if (smax == -INFINITY) {
            lse[h] = -INFINITY;
            free(s);
            continue;
        }
        double z = 0.0;
        for (int64_t t = 0; t < t_rows; ++t) {
            double p = exp(s[t] - smax);
            z += p;
            for (int32_t i = 0; i < lc; ++i)
                o[i] += p * (mla8o_dec(rows[t * rb + i]) * (double)scales[t]);
        }
        for (int32_t i = 0; i < lc; ++i)
            o[i] /= z;
        lse[h] = smax + log(z);
        free(s);
    }
}

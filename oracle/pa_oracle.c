/*
 * pa_oracle.c -- plain fp64 CPU oracle for batched grouped-query decode
 * attention over a token-granular paged KV pool, for the chunked-prefill
 * variant over the same pool, and for the log-sum-exp merge of split
 * partitions.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; it shares no header, helper or constant with the GPU
 * path.  Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.
 *
 * What is computed, and where it comes from:
 *   - The KV pool is token-granular (one slot per token, page size 1) and is
 *     shared by every request in the batch; each request owns a list of slot
 *     ids.  Agent-Infer page ("Agent-Infer: 纯 Rust 编写的高性能 LLM 推理引擎"),
 *     section "分页 KV 缓存" (TokenToKVPool with page size 1, batched decode
 *     across all requests).  The list is stored as CSR: kv_indptr[b]..
 *     kv_indptr[b+1] delimit request b's entries in kv_indices.
 *   - Grouped-query attention: Hq query heads share Hkv KV heads, Hq/Hkv query
 *     heads per KV head (32 query heads over 8 KV heads, head_dim 128 for
 *     Qwen3; head_dim 256 for the Qwen3.5 full-attention layers).  Pegainfer
 *     page ("Pegainfer: 纯Rust+CUDA构建的LLM推理引擎"), section "关键技术实现",
 *     items 1 (注意力机制优化) and 2 (Qwen3.5的混合架构支持).
 *     Reading: query head h reads KV head h / (Hq/Hkv) (contiguous groups).
 *   - Attention itself is the textbook softmax attention; the pages name it
 *     (FlashInfer paged decode, FlashAttention-2 in the kernel layer: Agent-Infer
 *     page, sections "3. CUDA 内核层" and the table in "优化历程") without
 *     writing it out.  Reading: for query row q and visible slots S_0..S_{n-1}
 *         s_j  = scale * <q, K[S_j]>
 *         out  = sum_j exp(s_j - m) V[S_j] / sum_j exp(s_j - m),  m = max_j s_j
 *         lse  = m + ln(sum_j exp(s_j - m))          (natural log)
 *     with an empty list giving out = 0 and lse = -inf.
 *   - Chunked prefill: a long prompt is cut into chunks (512 tokens, 64 while
 *     decodes are running) that attend to the cached prefix plus the chunk.
 *     Agent-Infer page, section "连续批处理".  Reading: the chunk's C tokens are
 *     the last C entries of the request's slot list; chunk row i sees list
 *     positions 0 .. P+i inclusive, P = L - C (causal inside the chunk).
 *   - Merge of split partitions: the pages do not describe one.  Reading: a
 *     range cut into parts with per-part results (o_i, lse_i) recombines as
 *         M = max_i lse_i,  w_i = exp(lse_i - M),
 *         o = sum_i w_i o_i / sum_i w_i,  lse = M + ln(sum_i w_i).
 *
 *   - Rotary position embedding of the rows appended to the pool (the step
 *     before attention: new tokens' K/V rows are written to their slots, K
 *     stored already rotated).  Pegainfer page, section "核心组件概览" (RoPE is
 *     one of the GPU operators of ops.rs); the appended slots are the
 *     TokenToKVPool slots of the Agent-Infer page, section "分页 KV 缓存".  The
 *     pages do not write RoPE out.  Reading (the rotate-half form used by the
 *     Qwen3 family): for head dimension D, pair i < D/2 couples elements i and
 *     i + D/2 and turns them by the angle pos * theta^(-2i/D):
 *         y[i]       = x[i] cos(a_i) - x[i + D/2] sin(a_i)
 *         y[i + D/2] = x[i + D/2] cos(a_i) + x[i] sin(a_i)
 *
 *   - 8-bit floating-point KV pool (quantisation, FP8 among the formats, is
 *     on the Agent-Infer page's roadmap, section "模型支持与发展路线图"; the
 *     pages give no format).  Reading: K and V rows stored as OCP FP8 E4M3
 *     codes (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; no
 *     infinities; exponent and mantissa all ones is NaN), with one scale per
 *     pool: the row values are k_scale * value(code) and v_scale * value(code),
 *     formed in double precision, and the attention above runs on those
 *     values unchanged:
 *         s_j = scale * <q, k_scale * value(Kcode[S_j])>
 *         out = sum_j exp(s_j - m) * v_scale * value(Vcode[S_j]) / sum_j exp(s_j - m)
 *     Writing such a pool (the append step for 8-bit pools): a K row is
 *     rotated as above in double precision, then each element y is stored as
 *     the E4M3 code nearest to y / k_scale; a V element x (bf16, widened) as
 *     the code nearest to x / v_scale.  Reading of "nearest": round to
 *     nearest, ties to even, among the finite codes, so that magnitudes past
 *     the largest finite value 448 saturate to +-448 (a KV cache keeps a
 *     finite value rather than NaN); NaN inputs give the NaN code 0x7F.
 *     Chunked prefill over such pools: the prefill rows above on these
 *     values.
 *
 * All arithmetic is in double precision.  bf16 inputs are widened exactly
 * (a bf16 bit pattern is the upper half of an IEEE binary32).  The softmax
 * scale is given as a float and widened, so both sides use the same value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* status codes */
#define ORACLE_OK 0
#define ORACLE_BAD_SHAPE 1
#define ORACLE_BAD_INDPTR 2
#define ORACLE_BAD_SLOT 3
#define ORACLE_CHUNK_TOO_LONG 4
#define ORACLE_NO_MEMORY 5

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Softmax attention of one query row over an explicit list of n slots.
 * q_row points at D bf16 values; the KV row of slot s for KV head kh starts
 * at element s * slot_stride + kh * D of each pool.  `s` is scratch of n
 * doubles.
 */
static void attend_one_row(int D, const uint16_t *q_row,
                           const uint16_t *k_pool, const uint16_t *v_pool,
                           int64_t slot_stride, int kh,
                           const int32_t *slots, int64_t n, double scale,
                           double *s, double *out, double *lse)
{
    int64_t j;
    int d;

    if (n == 0) {
        for (d = 0; d < D; d++)
            out[d] = 0.0;
        *lse = -INFINITY;
        return;
    }

    /* scores */
    for (j = 0; j < n; j++) {
        const uint16_t *k_row = k_pool + (int64_t)slots[j] * slot_stride + (int64_t)kh * D;
        double dot = 0.0;
        for (d = 0; d < D; d++)
            dot += widen_bf16(q_row[d]) * widen_bf16(k_row[d]);
        s[j] = scale * dot;
    }

    /* softmax weights, shifted by the maximum */
    double m = s[0];
    for (j = 1; j < n; j++)
        if (s[j] > m)
            m = s[j];
    double z = 0.0;
    for (j = 0; j < n; j++) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }

    /* weighted sum of value rows */
    for (d = 0; d < D; d++)
        out[d] = 0.0;
    for (j = 0; j < n; j++) {
        const uint16_t *v_row = v_pool + (int64_t)slots[j] * slot_stride + (int64_t)kh * D;
        for (d = 0; d < D; d++)
            out[d] += s[j] * widen_bf16(v_row[d]);
    }
    for (d = 0; d < D; d++)
        out[d] /= z;
    *lse = m + log(z);
}

static int check_common(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D,
                        int64_t num_slots, int64_t slot_stride,
                        const int32_t *kv_indptr, const int32_t *kv_indices)
{
    int32_t b;
    int64_t j;

    if (batch < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0)
        return ORACLE_BAD_SHAPE;
    if (slot_stride < (int64_t)Hkv * D || num_slots < 0)
        return ORACLE_BAD_SHAPE;
    if (kv_indptr[0] != 0)
        return ORACLE_BAD_INDPTR;
    for (b = 0; b < batch; b++)
        if (kv_indptr[b + 1] < kv_indptr[b])
            return ORACLE_BAD_INDPTR;
    for (j = 0; j < kv_indptr[batch]; j++)
        if (kv_indices[j] < 0 || kv_indices[j] >= num_slots)
            return ORACLE_BAD_SLOT;
    return ORACLE_OK;
}

static int64_t longest_list(int32_t batch, const int32_t *kv_indptr)
{
    int64_t longest = 1;
    for (int32_t b = 0; b < batch; b++)
        if (kv_indptr[b + 1] - kv_indptr[b] > longest)
            longest = kv_indptr[b + 1] - kv_indptr[b];
    return longest;
}

/*
 * Decode: one query token per request.
 *   q       [batch, Hq, D] bf16 bits
 *   k_pool, v_pool: bf16 bits; slot s, head kh row at s*slot_stride + kh*D
 *   out     [batch, Hq, D] doubles, lse [batch, Hq] doubles
 *   sel     optional list of flat rows (b*Hq + h) to compute; NULL = all.
 *           Rows not selected are left untouched.
 */
int pa_oracle_decode(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D,
                     const uint16_t *q,
                     const uint16_t *k_pool, const uint16_t *v_pool,
                     int64_t num_slots, int64_t slot_stride,
                     const int32_t *kv_indptr, const int32_t *kv_indices,
                     float sm_scale, double *out, double *lse,
                     const int32_t *sel, int64_t n_sel)
{
    int rc = check_common(batch, Hq, Hkv, D, num_slots, slot_stride, kv_indptr, kv_indices);
    if (rc != ORACLE_OK)
        return rc;

    const int32_t group = Hq / Hkv;
    const int64_t n_rows = sel ? n_sel : (int64_t)batch * Hq;
    const int64_t longest = longest_list(batch, kv_indptr);
    int failed = 0;

    for (int64_t r = 0; r < n_rows; r++) {
        int64_t row = sel ? sel[r] : r;
        if (row < 0 || row >= (int64_t)batch * Hq)
            return ORACLE_BAD_SHAPE;
    }

#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * (size_t)longest);
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; r++) {
            if (!scratch)
                continue;
            int64_t row = sel ? sel[r] : r;
            int32_t b = (int32_t)(row / Hq);
            int32_t h = (int32_t)(row % Hq);
            int32_t kh = h / group;
            attend_one_row(D, q + row * D, k_pool, v_pool, slot_stride, kh,
                           kv_indices + kv_indptr[b],
                           (int64_t)kv_indptr[b + 1] - kv_indptr[b],
                           (double)sm_scale, scratch, out + row * D, lse + row);
        }
        free(scratch);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Chunked prefill appended to a paged context.
 *   q         [T, Hq, D] bf16 bits, T = qo_indptr[batch]
 *   qo_indptr [batch+1]: request b's chunk rows are qo_indptr[b]..qo_indptr[b+1]-1
 *   the chunk is the last C entries of the request's slot list (L >= C required);
 *   chunk row i sees list positions 0 .. (L - C) + i.
 *   out [T, Hq, D], lse [T, Hq]; sel lists flat rows t*Hq + h (NULL = all).
 */
int pa_oracle_prefill(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D,
                      const uint16_t *q,
                      const uint16_t *k_pool, const uint16_t *v_pool,
                      int64_t num_slots, int64_t slot_stride,
                      const int32_t *qo_indptr,
                      const int32_t *kv_indptr, const int32_t *kv_indices,
                      float sm_scale, double *out, double *lse,
                      const int32_t *sel, int64_t n_sel)
{
    int rc = check_common(batch, Hq, Hkv, D, num_slots, slot_stride, kv_indptr, kv_indices);
    if (rc != ORACLE_OK)
        return rc;
    if (qo_indptr[0] != 0)
        return ORACLE_BAD_INDPTR;
    for (int32_t b = 0; b < batch; b++) {
        if (qo_indptr[b + 1] < qo_indptr[b])
            return ORACLE_BAD_INDPTR;
        if (qo_indptr[b + 1] - qo_indptr[b] > kv_indptr[b + 1] - kv_indptr[b])
            return ORACLE_CHUNK_TOO_LONG;
    }

    const int32_t group = Hq / Hkv;
    const int64_t total_rows = (int64_t)qo_indptr[batch] * Hq;
    const int64_t n_rows = sel ? n_sel : total_rows;
    const int64_t longest = longest_list(batch, kv_indptr);
    int failed = 0;

    for (int64_t r = 0; r < n_rows; r++) {
        int64_t row = sel ? sel[r] : r;
        if (row < 0 || row >= total_rows)
            return ORACLE_BAD_SHAPE;
    }

#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * (size_t)longest);
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; r++) {
            if (!scratch)
                continue;
            int64_t row = sel ? sel[r] : r;
            int64_t t = row / Hq;
            int32_t h = (int32_t)(row % Hq);
            int32_t kh = h / group;
            int32_t b = 0;
            while (qo_indptr[b + 1] <= t)
                b++;
            int64_t chunk = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
            int64_t i = t - qo_indptr[b];
            int64_t L = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
            int64_t prefix = L - chunk;
            attend_one_row(D, q + row * D, k_pool, v_pool, slot_stride, kh,
                           kv_indices + kv_indptr[b], prefix + i + 1,
                           (double)sm_scale, scratch, out + row * D, lse + row);
        }
        free(scratch);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Log-sum-exp merge of n partial results of one query row.
 *   o_parts [n, D], lse_parts [n]  ->  out [D], *lse
 * Parts with lse = -inf (empty ranges) carry no weight; if every part is
 * empty the result is out = 0, lse = -inf.
 */
int pa_oracle_merge(int32_t n, int32_t D, const double *o_parts,
                    const double *lse_parts, double *out, double *lse)
{
    if (n < 0 || D <= 0)
        return ORACLE_BAD_SHAPE;
    double M = -INFINITY;
    for (int32_t i = 0; i < n; i++)
        if (lse_parts[i] > M)
            M = lse_parts[i];
    for (int32_t d = 0; d < D; d++)
        out[d] = 0.0;
    if (M == -INFINITY) {
        *lse = -INFINITY;
        return ORACLE_OK;
    }
    double wsum = 0.0;
    for (int32_t i = 0; i < n; i++) {
        double w = exp(lse_parts[i] - M);
        wsum += w;
        for (int32_t d = 0; d < D; d++)
            out[d] += w * o_parts[(int64_t)i * D + d];
    }
    for (int32_t d = 0; d < D; d++)
        out[d] /= wsum;
    *lse = M + log(wsum);
    return ORACLE_OK;
}

/*
 * Rotary position embedding of n rows of D bf16 values (rows of `heads`
 * consecutive heads per token): row r belongs to token r / heads, whose
 * position is positions[r / heads].  Output: n * D doubles (not rounded).
 */
int pa_oracle_rope(int64_t tokens, int32_t heads, int32_t D, const uint16_t *x_bits,
                   const int32_t *positions, double theta, double *y)
{
    if (tokens < 0 || heads <= 0 || D <= 0 || D % 2 != 0 || !(theta > 0.0))
        return ORACLE_BAD_SHAPE;
    const int half = D / 2;
    for (int64_t t = 0; t < tokens; t++) {
        for (int32_t h = 0; h < heads; h++) {
            const uint16_t *x = x_bits + (t * heads + h) * (int64_t)D;
            double *out = y + (t * heads + h) * (int64_t)D;
            for (int i = 0; i < half; i++) {
                const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
                const double a = (double)positions[t] * inv_freq;
                const double c = cos(a), sn = sin(a);
                const double x1 = widen_bf16(x[i]), x2 = widen_bf16(x[i + half]);
                out[i] = x1 * c - x2 * sn;
                out[i + half] = x2 * c + x1 * sn;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Value of an OCP FP8 E4M3 code: (-1)^s * 2^(e - 7) * (1 + m/8) for e > 0,
 * (-1)^s * 2^-6 * (m/8) for e = 0 (subnormals), NaN for e = 15, m = 7.
 */
static double e4m3_value(uint8_t code)
{
    const int sign = code >> 7, e = (code >> 3) & 0xF, m = code & 0x7;
    if (e == 0xF && m == 0x7)
        return NAN;
    const double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/*
 * E4M3 codes -> the bf16 bit patterns of the same values (exact: 3 mantissa
 * bits and exponents 2^-9 .. 2^8 all fit bf16).  NaN codes give a bf16 NaN.
 */
int pa_oracle_e4m3_to_bf16(int64_t n, const uint8_t *codes, uint16_t *bits)
{
    if (n < 0)
        return ORACLE_BAD_SHAPE;
    for (int64_t i = 0; i < n; i++) {
        const float f = (float)e4m3_value(codes[i]);
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        bits[i] = (uint16_t)(u >> 16);   /* exact: the low 16 bits are zero */
    }
    return ORACLE_OK;
}

/* Values of n E4M3 codes (for the pins). */
int pa_oracle_e4m3_values(int64_t n, const uint8_t *codes, double *values)
{
    if (n < 0)
        return ORACLE_BAD_SHAPE;
    for (int64_t i = 0; i < n; i++)
        values[i] = e4m3_value(codes[i]);
    return ORACLE_OK;
}

/*
 * The E4M3 code of one double: the finite code whose value is nearest, a tie
 * going to the code whose last mantissa bit is 0 (round to nearest even).
 * Being nearest among the finite codes only, magnitudes at or beyond 448
 * (infinities included) give +-448; NaN gives 0x7F; the sign of a zero result
 * is the sign of the input.  Plain search over the 127 finite magnitudes.
 */
static uint8_t e4m3_encode(double x)
{
    if (isnan(x))
        return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const double a = fabs(x);
    if (a >= 448.0)
        return sign | 0x7E;
    int best = 0;
    double best_err = a;              /* distance to code 0 (value 0) */
    for (int c = 1; c <= 0x7E; c++) {
        const double err = fabs(e4m3_value((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

/*
 * Codes of n doubles divided by a scale: codes[i] = E4M3 code of x[i] / scale
 * (the quotient formed in double precision; the scale is given as a float and
 * widened).  The write side of the 8-bit pool: a value stored under pool
 * scale s is the code of value / s, so that s * value(code) approximates it.
 */
int pa_oracle_e4m3_encode(int64_t n, const double *x, float scale, uint8_t *codes)
{
    if (n < 0 || !(scale > 0.0f) || isinf(scale))
        return ORACLE_BAD_SHAPE;
    for (int64_t i = 0; i < n; i++)
        codes[i] = e4m3_encode(x[i] / (double)scale);
    return ORACLE_OK;
}

/*
 * Softmax attention of one query row over n slots of E4M3 pools: the same
 * formula as attend_one_row, on the values k_scale * value(code) and
 * v_scale * value(code), all in double precision.
 */
static void attend_one_row_e4m3(int D, const uint16_t *q_row,
                                const uint8_t *k_codes, const uint8_t *v_codes,
                                int64_t slot_stride, int kh,
                                const int32_t *slots, int64_t n, double scale,
                                double k_scale, double v_scale,
                                double *w, double *out, double *lse)
{
    if (n == 0) {
        for (int d = 0; d < D; d++)
            out[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    for (int64_t j = 0; j < n; j++) {
        const uint8_t *kc = k_codes + (int64_t)slots[j] * slot_stride + (int64_t)kh * D;
        double acc = 0.0;
        for (int d = 0; d < D; d++)
            acc += widen_bf16(q_row[d]) * (k_scale * e4m3_value(kc[d]));
        w[j] = scale * acc;
    }
    double top = w[0];
    for (int64_t j = 1; j < n; j++)
        top = w[j] > top ? w[j] : top;
    double total = 0.0;
    for (int64_t j = 0; j < n; j++) {
        w[j] = exp(w[j] - top);
        total += w[j];
    }
    for (int d = 0; d < D; d++)
        out[d] = 0.0;
    for (int64_t j = 0; j < n; j++) {
        const uint8_t *vc = v_codes + (int64_t)slots[j] * slot_stride + (int64_t)kh * D;
        for (int d = 0; d < D; d++)
            out[d] += w[j] * (v_scale * e4m3_value(vc[d]));
    }
    for (int d = 0; d < D; d++)
        out[d] = out[d] / total;
    *lse = top + log(total);
}

/*
 * Decode over E4M3 pools with per-pool scales (codes: 1 byte per element,
 * slot s, head kh row at s*slot_stride + kh*D).  Arguments otherwise as
 * pa_oracle_decode; the scales are given as floats and widened.
 */
int pa_oracle_decode_e4m3(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D,
                          const uint16_t *q,
                          const uint8_t *k_codes, const uint8_t *v_codes,
                          int64_t num_slots, int64_t slot_stride,
                          const int32_t *kv_indptr, const int32_t *kv_indices,
                          float sm_scale, float k_scale, float v_scale,
                          double *out, double *lse,
                          const int32_t *sel, int64_t n_sel)
{
    int rc = check_common(batch, Hq, Hkv, D, num_slots, slot_stride, kv_indptr, kv_indices);
    if (rc != ORACLE_OK)
        return rc;
    const int32_t per_kv_head = Hq / Hkv;
    const int64_t n_rows = sel ? n_sel : (int64_t)batch * Hq;
    const int64_t longest = longest_list(batch, kv_indptr);
    int failed = 0;
    for (int64_t r = 0; r < n_rows; r++) {
        int64_t row = sel ? sel[r] : r;
        if (row < 0 || row >= (int64_t)batch * Hq)
            return ORACLE_BAD_SHAPE;
    }
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)longest);
        if (!w) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; r++) {
            if (!w)
                continue;
            const int64_t row = sel ? sel[r] : r;
            const int32_t b = (int32_t)(row / Hq);
            const int32_t head = (int32_t)(row % Hq);
            attend_one_row_e4m3(D, q + row * D, k_codes, v_codes, slot_stride,
                                head / per_kv_head, kv_indices + kv_indptr[b],
                                (int64_t)kv_indptr[b + 1] - kv_indptr[b],
                                (double)sm_scale, (double)k_scale, (double)v_scale,
                                w, out + row * D, lse + row);
        }
        free(w);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Chunked prefill over E4M3 pools with per-pool scales: the rows of
 * pa_oracle_prefill (chunk row i of request b sees list positions
 * 0 .. L - C + i, the chunk being the last C entries of the list) on the
 * row values of pa_oracle_decode_e4m3 (k_scale * value(code),
 * v_scale * value(code), in double precision).
 */
int pa_oracle_prefill_e4m3(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D,
                           const uint16_t *q,
                           const uint8_t *k_codes, const uint8_t *v_codes,
                           int64_t num_slots, int64_t slot_stride,
                           const int32_t *qo_indptr,
                           const int32_t *kv_indptr, const int32_t *kv_indices,
                           float sm_scale, float k_scale, float v_scale,
                           double *out, double *lse,
                           const int32_t *sel, int64_t n_sel)
{
    int rc = check_common(batch, Hq, Hkv, D, num_slots, slot_stride, kv_indptr, kv_indices);
    if (rc != ORACLE_OK)
        return rc;
    if (qo_indptr[0] != 0)
        return ORACLE_BAD_INDPTR;
    for (int32_t b = 0; b < batch; b++) {
        if (qo_indptr[b + 1] < qo_indptr[b])
            return ORACLE_BAD_INDPTR;
        if (qo_indptr[b + 1] - qo_indptr[b] > kv_indptr[b + 1] - kv_indptr[b])
            return ORACLE_CHUNK_TOO_LONG;
    }
    const int64_t all_rows = (int64_t)qo_indptr[batch] * Hq;
    const int64_t n_rows = sel ? n_sel : all_rows;
    for (int64_t r = 0; r < n_rows; r++) {
        const int64_t row = sel ? sel[r] : r;
        if (row < 0 || row >= all_rows)
            return ORACLE_BAD_SHAPE;
    }
    const int64_t longest = longest_list(batch, kv_indptr);
    int failed = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)longest);
        if (!w) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; r++) {
            if (!w)
                continue;
            const int64_t row = sel ? sel[r] : r;
            const int64_t tok = row / Hq;          /* chunk token (flat over requests) */
            const int32_t head = (int32_t)(row % Hq);
            int32_t b = 0;
            while (qo_indptr[b + 1] <= tok)
                b++;
            const int64_t c_len = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
            const int64_t pos_in_chunk = tok - qo_indptr[b];
            const int64_t visible = ((int64_t)kv_indptr[b + 1] - kv_indptr[b]) - c_len + pos_in_chunk + 1;
            attend_one_row_e4m3(D, q + row * D, k_codes, v_codes, slot_stride,
                                head / (Hq / Hkv),
                                kv_indices + kv_indptr[b], visible, (double)sm_scale,
                                (double)k_scale, (double)v_scale, w, out + row * D, lse + row);
        }
        free(w);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Threads an OpenMP region of this library uses (1 without OpenMP). */
int pa_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

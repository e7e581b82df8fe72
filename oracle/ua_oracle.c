/*
 * ua_oracle.c -- plain fp64 CPU oracle for unified paged attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no source
 * with the HIP path and is deliberately slow: one query row at a time, every
 * key of the sequence, no tiling, no online softmax, no reordering.
 *
 * What it computes follows "Unified paged attention on gfx950, from the math
 * up" (section 1, the specification, and section 0, the paged/varlen layout),
 * with the empty-row convention of "The winning kernel, from the math up"
 * (section 6, the epilogue: 1/l is taken as 0 when l = 0).  For one sequence
 * s, local query row i (0 <= i < q_len), query head h:
 *
 *   kv head     hk   = h / (H_q / H_k)            (consecutive query heads share)
 *   ctx              = S_k - q_len,  q_abs = ctx + i
 *   gather      K_k  = K[block_table[s][k / b]][k mod b][hk][:]   (V likewise)
 *   1. scale    x_k  = tau * <Q_i, K_k>
 *   2. softcap  x_k  = c * tanh(x_k / c)                           (if enabled)
 *   3. ALiBi    x_k += slope_h * (k - ctx)                         (if enabled)
 *   4. QQ-bias  x_k += bias[i][k - ctx]  for k >= ctx (the query    (if enabled)
 *               section); one matrix shared by all heads and sequences
 *   5. causal   k > q_abs              -> masked                   (if enabled)
 *   6. window   k <= q_abs - W         -> masked (W keys remain)   (if enabled)
 *   7. sinks    one extra softmax column with logit sink_h and no value row
 *   then O_i = sum_{k visible} e^{x_k - m} V_k / Z,
 *      Z   = sum_{k visible} e^{x_k - m} + [sinks] e^{sink_h - m},
 *      m   = max over the visible x_k and the sink logit;  O_i = 0 if nothing
 *      is visible.
 *
 * Stored 16-bit and 8-bit values are decoded exactly from their bit patterns
 * (bfloat16, IEEE binary16, OCP e4m3fn); fp8 K/V are multiplied by their
 * per-tensor scale in fp64 after decoding.  The sink logit is taken in natural
 * log units and is not scaled, capped or biased.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define UAO_DT_BF16 0
#define UAO_DT_F16 1
#define UAO_DT_FP8_E4M3 2

/* Sliding-window reading: the window keeps exactly W keys, q_abs-W < k <= q_abs
 * (the dense prefill page keeps keys [q-W+1, q]).  Set to 1 to keep W+1 keys
 * instead (the one-line paraphrase on the unified page, k >= q_abs - W). */
#define UAO_WINDOW_EXTRA_KEY 0

typedef struct uao_problem {
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t q_dtype;          /* UAO_DT_BF16 or UAO_DT_F16 */
    int32_t kv_dtype;         /* UAO_DT_BF16, UAO_DT_F16 or UAO_DT_FP8_E4M3 */
    int32_t causal;
    int32_t use_softcap;
    int32_t use_alibi;
    int32_t use_window;
    int32_t use_sinks;
    int32_t window;
    int32_t block_table_stride; /* entries per block-table row */
    int64_t q_stride_tok;       /* elements between consecutive tokens of Q */
    double scale;
    double softcap;
    double k_scale;
    double v_scale;
    int32_t use_qq_bias;
    int32_t qq_bias_stride;     /* elements between rows of qq_bias */
    const float* qq_bias;       /* [q_local][k_local] over the query section */
} uao_problem;

/* ---- exact decoders ----------------------------------------------------- */

static double uao_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double uao_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double uao_e4m3fn(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int m = c & 0x7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;                                 /* e4m3fn has no infinities */
    else if (e == 0)
        v = ldexp((double)m, -9);                /* subnormal: (m/8) * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10);      /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

static double uao_load16(const void* base, int64_t idx, int dtype) {
    uint16_t h = ((const uint16_t*)base)[idx];
    return dtype == UAO_DT_BF16 ? uao_bf16(h) : uao_f16(h);
}

static double uao_load_kv(const void* base, int64_t idx, int dtype, double fp8_scale) {
    if (dtype == UAO_DT_FP8_E4M3)
        return uao_e4m3fn(((const uint8_t*)base)[idx]) * fp8_scale;
    return uao_load16(base, idx, dtype);
}

/* Exported decoders, so tests can compare them with a library's conversion. */
double uao_decode(int dtype, uint32_t bits) {
    if (dtype == UAO_DT_FP8_E4M3) return uao_e4m3fn((uint8_t)bits);
    return dtype == UAO_DT_BF16 ? uao_bf16((uint16_t)bits) : uao_f16((uint16_t)bits);
}

/* ---- one output row ----------------------------------------------------- */

/* Computes O[token, head, :] into out[0..d) and, when lse != NULL, the natural
 * log of Z plus m (the log-sum-exp over the visible keys and the sink; -inf
 * when the row sees nothing).  Returns 0, or -1 on an inconsistent input. */
static int uao_row(const uao_problem* p, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q,
                   const float* slopes, const float* sinks, int32_t seq, int32_t token,
                   int32_t head, double* out, double* lse, double* xbuf, unsigned char* vis) {
    const int d = p->head_dim;
    const int g = p->num_q_heads / p->num_kv_heads;
    const int hk = head / g;
    const int64_t sk = seq_lens[seq];
    const int64_t q_len = (int64_t)cu_q[seq + 1] - cu_q[seq];
    const int64_t i = (int64_t)token - cu_q[seq];
    if (i < 0 || i >= q_len || q_len > sk) return -1;
    const int64_t ctx = sk - q_len;
    const int64_t q_abs = ctx + i;
    const int64_t q_off = (int64_t)token * p->q_stride_tok + (int64_t)head * d;
    const int64_t row_elems = (int64_t)p->num_kv_heads * d;

    double m = -INFINITY;
    int64_t n_vis = 0;
    for (int64_t k = 0; k < sk; ++k) {
        int64_t phys = block_table[(int64_t)seq * p->block_table_stride + k / p->block_size];
        int64_t slot = k % p->block_size;
        int64_t k_off = (phys * p->block_size + slot) * row_elems + (int64_t)hk * d;
        /* 1. scale */
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += uao_load16(q, q_off + e, p->q_dtype) *
                   uao_load_kv(k_cache, k_off + e, p->kv_dtype, p->k_scale);
        double x = p->scale * dot;
        /* 2. softcap */
        if (p->use_softcap) x = p->softcap * tanh(x / p->softcap);
        /* 3. ALiBi */
        if (p->use_alibi) x += (double)slopes[head] * (double)(k - ctx);
        /* 4. QQ-bias, for keys inside the query section (k >= ctx) */
        if (p->use_qq_bias && k >= ctx)
            x += (double)p->qq_bias[i * p->qq_bias_stride + (k - ctx)];
        /* 5. causal, 6. window */
        int visible = 1;
        if (p->causal && k > q_abs) visible = 0;
        if (p->use_window && k < q_abs - p->window + 1 - UAO_WINDOW_EXTRA_KEY) visible = 0;
        xbuf[k] = x;
        vis[k] = (unsigned char)visible;
        if (visible) {
            ++n_vis;
            if (x > m) m = x;
        }
    }
    /* 7. sinks take part in the max and the denominator only */
    double sink = p->use_sinks ? (double)sinks[head] : 0.0;
    if (p->use_sinks && sink > m) m = sink;

    for (int e = 0; e < d; ++e) out[e] = 0.0;
    if (n_vis == 0) {
        if (lse) *lse = p->use_sinks ? sink : -INFINITY;
        return 0;
    }
    /* the softmax-weighted sum of V */
    double z = p->use_sinks ? exp(sink - m) : 0.0;
    for (int64_t k = 0; k < sk; ++k) {
        if (!vis[k]) continue;
        double w = exp(xbuf[k] - m);
        z += w;
        int64_t phys = block_table[(int64_t)seq * p->block_table_stride + k / p->block_size];
        int64_t slot = k % p->block_size;
        int64_t v_off = (phys * p->block_size + slot) * row_elems + (int64_t)hk * d;
        for (int e = 0; e < d; ++e)
            out[e] += w * uao_load_kv(v_cache, v_off + e, p->kv_dtype, p->v_scale);
    }
    for (int e = 0; e < d; ++e) out[e] /= z;
    if (lse) *lse = m + log(z);
    return 0;
}

static int32_t uao_seq_of(const int32_t* cu_q, int32_t num_seqs, int64_t token) {
    /* last s with cu_q[s] <= token (sequences with q_len 0 own no token) */
    int32_t s = 0;
    while (s + 1 < num_seqs && cu_q[s + 1] <= token) ++s;
    return s;
}

static int uao_check(const uao_problem* p) {
    if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads) return -1;
    if (p->head_dim <= 0 || p->block_size <= 0 || p->num_seqs < 0) return -1;
    return 0;
}

/* Selected rows: rows[r] = token * H_q + head.  out is [n_rows, d], lse is
 * [n_rows] or NULL.  Rows are independent; nthreads > 1 uses OpenMP. */
int uao_rows(const uao_problem* p, const void* q, const void* k_cache, const void* v_cache,
             const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q,
             const float* slopes, const float* sinks, const int64_t* rows, int64_t n_rows,
             double* out, double* lse, int nthreads) {
    if (uao_check(p)) return -1;
    int64_t max_sk = 0;
    for (int32_t s = 0; s < p->num_seqs; ++s)
        if (seq_lens[s] > max_sk) max_sk = seq_lens[s];
    int err = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double* xbuf = (double*)malloc(sizeof(double) * (size_t)(max_sk + 1));
        unsigned char* vis = (unsigned char*)malloc((size_t)(max_sk + 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t token = rows[r] / p->num_q_heads;
            int32_t head = (int32_t)(rows[r] % p->num_q_heads);
            int32_t seq = uao_seq_of(cu_q, p->num_seqs, token);
            int rc = (xbuf && vis)
                         ? uao_row(p, q, k_cache, v_cache, block_table, seq_lens, cu_q, slopes,
                                   sinks, seq, (int32_t)token, head, out + r * p->head_dim,
                                   lse ? lse + r : NULL, xbuf, vis)
                         : -1;
            if (rc) {
#pragma omp atomic write
                err = rc;
            }
        }
        free(xbuf);
        free(vis);
    }
    return err;
}

/* Every row: out is [total_q, H_q, d] (fp64), lse is [total_q, H_q] or NULL. */
int uao_attention(const uao_problem* p, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q,
                  const float* slopes, const float* sinks, double* out, double* lse,
                  int nthreads) {
    if (uao_check(p)) return -1;
    int64_t total = (int64_t)cu_q[p->num_seqs] * p->num_q_heads;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(total > 0 ? total : 1));
    if (!rows) return -1;
    for (int64_t r = 0; r < total; ++r) rows[r] = r;
    int rc = uao_rows(p, q, k_cache, v_cache, block_table, seq_lens, cu_q, slopes, sinks, rows,
                      total, out, lse, nthreads);
    free(rows);
    return rc;
}

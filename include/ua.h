/*
 * ua.h -- unified paged attention forward pass for MI355X (gfx950).
 *
 * One kernel family computes, for every packed query row of a varlen batch,
 *
 *     O_i = sum_j softmax_j( bias/mask( tau * Q_i K_j^T ) ) V_j
 *
 * over a block-table-paged KV cache with grouped-query heads, serving decode
 * (S_q = 1), chunked prefill (1 < S_q < S_k) and prefill (S_q = S_k) alike.
 * The operation and its bias/mask order (scale, softcap, ALiBi, causal,
 * sliding window, sinks) are the specification of "Unified paged attention on
 * gfx950, from the math up", section 1; the layouts are its section 0; the
 * two kernel strategies (a 2D query-tile kernel and a 3D split-KV kernel with a
 * log-sum-exp reduce) and the shape rule between them are its sections 4-6.
 *
 * Conventions for every entry point:
 *  - Plain C ABI; no C++ exceptions cross it.  Every call returns a status
 *    code; on failure ua_last_error() returns a thread-local message.
 *  - "device" pointers are HIP device memory owned by the caller; the library
 *    never allocates, frees or synchronises on the run path.
 *  - Streams are passed as `void*` holding a hipStream_t (NULL = the default
 *    stream).
 */
#ifndef UA_H
#define UA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ua_status {
    UA_OK = 0,
    UA_ERR_INVALID_ARG = 1,  /* a descriptor field or run argument is out of range */
    UA_ERR_UNSUPPORTED = 2,  /* valid, but no kernel is built for it (e.g. head_dim 96) */
    UA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than ua_workspace_size() */
    UA_ERR_HIP = 4           /* a HIP launch reported an error */
} ua_status_t;

/* Storage types.  Q and O share q_dtype; K and V share kv_dtype, which is
 * q_dtype or UA_DTYPE_FP8_E4M3 (OCP e4m3fn codes times a per-tensor scale;
 * "Unified paged attention on gfx950", section 7.3). */
typedef enum ua_dtype {
    UA_DTYPE_BF16 = 0,
    UA_DTYPE_F16 = 1,
    UA_DTYPE_FP8_E4M3 = 2
} ua_dtype_t;

/* Problem flags (section 1 of the unified page, one flag per bias/mask). */
enum {
    UA_FLAG_CAUSAL = 1u << 0,   /* mask keys k > q_abs (q_abs = ctx + local row) */
    UA_FLAG_SOFTCAP = 1u << 1,  /* s <- c tanh(s / c) after the scale */
    UA_FLAG_ALIBI = 1u << 2,    /* s += slope_h (k - ctx) */
    UA_FLAG_WINDOW = 1u << 3,   /* keep the last `window` keys: q_abs - W < k <= q_abs */
    UA_FLAG_SINKS = 1u << 4,    /* per-head logit joins the softmax with no value row */
    UA_FLAG_QQ_BIAS = 1u << 5,  /* bias[q_local][k - ctx] on keys of the query section */
    UA_FLAG_DENSE_KV = 1u << 6, /* K/V packed per sequence: rows cu_seqlens_k[s] + k */
    UA_FLAG_BF16_PARTIALS = 1u << 7, /* split-KV partial o kept in bf16 in the workspace
                                    (m and l stay f32): about half the partial bytes
                                    and a smaller ua_workspace_size; each partial is
                                    rounded to bf16 (2^-9 relative) before the merge */
    UA_FLAG_FORCE_2D = 1u << 8, /* testing/benchmarking: bypass the shape rule */
    UA_FLAG_FORCE_3D = 1u << 9,
    UA_FLAG_PERSISTENT = 1u << 10 /* a lone 2D launch of four-wave q-blocks on the LDS
                                    ring runs on the persistent schedule of section
                                    8.2 of the unified page: one workgroup per resident
                                    slot drawing q-blocks, heaviest first, from eight
                                    work queues (one per XCD, so a kv head's work
                                    runs on one XCD); results are bitwise those of the
                                    default grid.  Needs 256 bytes of workspace
                                    (included in ua_workspace_size); other launches
                                    keep the default grid. */
};

/* Element type of caller-held partial states (ua_run_args_t.partial_o and
 * ua_merge_args_t). */
enum {
    UA_PARTIAL_F32 = 0,
    UA_PARTIAL_BF16 = 1
};

/* Problem description: everything that fixes the kernel and the plan bounds.
 * All fields are host values; creating a problem touches no device. */
typedef struct ua_problem_desc {
    int32_t num_q_heads;         /* H_q > 0 */
    int32_t num_kv_heads;        /* H_k > 0, H_q % H_k == 0, g = H_q / H_k <= 128 */
    int32_t head_dim;            /* d in {64, 128, 256} */
    int32_t block_size;          /* b: power of two <= 1024 (KV positions per physical
                                    block); 1 with UA_FLAG_DENSE_KV */
    int32_t q_dtype;             /* UA_DTYPE_BF16 or UA_DTYPE_F16 */
    int32_t kv_dtype;            /* q_dtype or UA_DTYPE_FP8_E4M3 */
    uint32_t flags;              /* UA_FLAG_* */
    float scale;                 /* tau > 0 (usually 1/sqrt(d)) */
    float softcap;               /* c > 0 when UA_FLAG_SOFTCAP */
    int32_t window;              /* W > 0 when UA_FLAG_WINDOW */
    float k_scale;               /* fp8 only: real K = decode(code) * k_scale (> 0) */
    float v_scale;               /* fp8 only: real V = decode(code) * v_scale (> 0) */
    int64_t num_blocks;          /* physical blocks in each of the K and V pools */
    int32_t max_num_seqs;        /* upper bound for ua_run_args.num_seqs */
    int32_t max_blocks_per_seq;  /* upper bound for ua_run_args.block_table_stride use */
    int64_t max_total_q;         /* upper bound for ua_run_args.total_q */
    int32_t max_seqlen_k;        /* upper bound for any S_k (sizes the split workspace) */
    int32_t split_segment_tiles; /* 0 = automatic; else KV tiles per split-KV segment
                                    (>= 1; a tuning override of the plan) */
    int32_t num_cus;             /* compute units the shape rule sizes for (its thresholds
                                    are workgroups per CU, section 6).  0 = automatic:
                                    ua_run queries the current device once per device;
                                    ua_query_plan, which touches no device, assumes the
                                    MI355X's 256.  >= 0. */
} ua_problem_desc_t;

typedef struct ua_problem* ua_problem_t;

/* Arguments of one forward pass.
 *  q            device, [total_q, H_q, d] in q_dtype; token stride q_stride_tok
 *               elements, heads and d contiguous.
 *  k_cache,
 *  v_cache      device, [num_blocks, b, H_k, d] in kv_dtype, contiguous.
 *  o            device, [total_q, H_q, d] in q_dtype; token stride o_stride_tok.
 *               Must not alias q or the caches.
 *  block_table  device int32 [num_seqs, block_table_stride]; entry [s][j] is the
 *               physical block of sequence s's logical block j.  Entries past
 *               ceil(S_k / b) are never read.
 *  seq_lens     device int32 [num_seqs]: S_k per sequence (cached + new tokens).
 *  cu_seqlens_q device int32 [num_seqs + 1]: prefix sums of the query lengths;
 *               sequence s owns tokens [cu[s], cu[s+1]) which are its last
 *               q_len key positions (ctx = S_k - q_len).
 *  alibi_slopes device f32 [H_q] when UA_FLAG_ALIBI, else NULL.
 *  sinks        device f32 [H_q] (natural-log logits) when UA_FLAG_SINKS, else NULL.
 *  cu_seqlens_k device int32 [num_seqs + 1] when UA_FLAG_DENSE_KV, else NULL:
 *               the packed varlen layout of the dense sibling (section 8 of the
 *               unified page; the varlen variant of the dense-prefill page)
 *               stores key k of sequence s, kv-head h at row cu_seqlens_k[s] + k
 *               of k_cache / v_cache [rows, H_k, d], and S_k = cu_seqlens_k[s+1]
 *               - cu_seqlens_k[s].  The problem's block_size must be 1 and
 *               num_blocks counts rows.  block_table, block_table_stride and
 *               seq_lens are not read (may be NULL / 0).  Queries keep their
 *               own cu_seqlens_q: q_len < S_k is a chunk at the sequence's end.
 *  qq_bias      device f32 matrix when UA_FLAG_QQ_BIAS, else NULL: step 4 of
 *               section 1 of the unified page adds qq_bias[i * qq_bias_stride +
 *               (k - ctx)] (natural-log units, after ALiBi, before the masks)
 *               to the score of local query row i and key k when k >= ctx,
 *               i.e. for keys inside the sequence's query section.  One matrix
 *               serves all heads and sequences; it must cover max_seqlen_q rows
 *               and columns (qq_bias_stride >= max_seqlen_q), 4-byte aligned.
 *  workspace    device, >= ua_workspace_size() bytes, 256-byte aligned; used
 *               only by the split-KV path (may be NULL if that size is 0).
 *  num_seqs, total_q, max_seqlen_q, max_seqlen_k are host copies of the
 *  batch's shape (no device reads on the host side).
 *  timing_events  optional hipEvent_t handles (NULL to skip each): [0] is
 *               recorded on the stream before the attention kernel, [1] after
 *               it (before the split-KV reduce, if any), [2] after the last
 *               kernel, so a caller can time the kernels one by one.  On a
 *               class-split run (ua_plan_info.class_split) [0] precedes both
 *               launches and [1], [2] follow both, reduces included.
 *  lse          optional device f32 [total_q, H_q] (token-major, NULL to skip):
 *               the natural-log log-sum-exp of each row's softmax denominator,
 *               ln(sum over visible keys of e^{s_k} (+ e^{sink_h})), with s_k
 *               the scores after scale, softcap and ALiBi; -inf for a row
 *               with no visible key.  This is the per-row statistic that
 *               merges independent attention results over disjoint key sets
 *               (section 5 of the unified page's re-base, in natural log).
 *               The denominator sums the same 16-bit-rounded p as O, so it
 *               agrees with the exact value to about 2^-9 relative (LSE to
 *               about 2e-3 absolute).  4-byte aligned.
 *  partial_o    optional device [total_q, H_q, d] (16-byte aligned; NULL = a
 *               normal run).  When set the run leaves its result unnormalised
 *               across calls ("skip the final merge"): instead of O (which
 *               may then be NULL) and `lse` it writes, per row, the
 *               merge-ready state of the (o, m, l) recurrence over this call's
 *               keys: o / l (times v_scale for fp8 V) here, in partial_dtype,
 *               and ln l + m ln 2, the row's natural-log LSE, to partial_lse
 *               (0 and -inf for a row that saw no key).  Sinks are left out,
 *               so that ua_merge can join them exactly once.  Section 5 of the
 *               unified page merges such states associatively; callers use
 *               this for shared-prefix (cascade) batches and for keys split
 *               over devices or calls.
 *  partial_lse  device f32 [total_q, H_q], 4-byte aligned; required with partial_o.
 *  partial_dtype  UA_PARTIAL_F32 or UA_PARTIAL_BF16 (bf16 rounds o / l to 8
 *               significant bits; the LSE stays f32).
 * Device metadata is trusted: 0 <= q_len <= S_k <= max_seqlen_k, and used
 * block-table entries lie in [0, num_blocks). */
typedef struct ua_run_args {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    void* o;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* cu_seqlens_q;
    const float* alibi_slopes;
    const float* sinks;
    void* workspace;
    size_t workspace_bytes;
    int32_t num_seqs;
    int32_t max_seqlen_q;
    int64_t total_q;
    int32_t max_seqlen_k;
    int32_t block_table_stride;
    int64_t q_stride_tok;
    int64_t o_stride_tok;
    void* timing_events[3];
    float* lse;
    const float* qq_bias;
    int32_t qq_bias_stride;
    const int32_t* cu_seqlens_k;
    void* partial_o;
    float* partial_lse;
    int32_t partial_dtype;
} ua_run_args_t;

/* Most partial states one ua_merge call combines. */
#define UA_MAX_MERGE_SETS 8

/* Arguments of ua_merge: num_sets partial states of the same rows, each as
 * ua_run writes them with partial_o set (row r = token * H_q + head).
 *  partial_o[i]    device [total_q, H_q, head_dim] in partial_dtype, 16-byte aligned
 *  partial_lse[i]  device f32 [total_q, H_q] natural-log LSE (-inf: empty set)
 *  sinks           optional device f32 [H_q] natural-log sink logits (NULL: none),
 *                  joined once into every row's denominator
 *  o               device [total_q, H_q, head_dim] in o_dtype (bf16 / f16), token
 *                  stride o_stride_tok elements (>= H_q * head_dim, multiple of 8)
 *  lse             optional device f32 [total_q, H_q]: the merged natural-log LSE */
typedef struct ua_merge_args {
    int32_t num_sets;
    int32_t partial_dtype;
    const void* partial_o[UA_MAX_MERGE_SETS];
    const float* partial_lse[UA_MAX_MERGE_SETS];
    int64_t total_q;
    int32_t num_q_heads;
    int32_t head_dim;
    int32_t o_dtype;
    int64_t o_stride_tok;
    void* o;
    float* lse;
    const float* sinks;
} ua_merge_args_t;

/* Which kernel strategy a run takes (section 6 of the unified page). */
typedef struct ua_plan_info {
    int32_t path;            /* 2 = 2D query-tile kernel, 3 = 3D split-KV + reduce */
    int32_t block_m;         /* query rows (position, head) per workgroup */
    int32_t block_q;         /* query positions per workgroup */
    int32_t tile_n;          /* keys per KV tile */
    int32_t waves;           /* wave64s per workgroup */
    int32_t num_segments;    /* split-KV segments per q-block (1 on the 2D path) */
    int32_t tiles_per_segment; /* a q-block with n live tiles is cut into
                                min(num_segments, ceil(n / tiles_per_segment))
                                near-equal runs (segmented split path) */
    int32_t grid[3];         /* launch grid of the attention kernel */
    int32_t use_i64_kv;      /* 1 when the KV pool exceeds 2^31 bytes */
    int32_t stream_k;        /* 1 when single-wave (decode-shaped) rows take the split
                                path with KV tiles balanced over resident workers
                                (never for head_dim 256 with 16-bit K/V, the QQ bias
                                and q-blocks of more than 16 rows: that kernel is
                                not built, and such batches take the segmented split
                                or the 2D path) */
    int32_t class_split;     /* 1 when a wide batch's decode-shaped sequences run in a
                                stream-K launch and the rest in the launch described above */
} ua_plan_info_t;

/* Validate a description and build a problem handle (host only; no device
 * access).  The description carries section 1's per-flag fields of the
 * unified page (one problem object whose flags select the bias and mask
 * steps) and the section 0 layout parameters.  `out` receives a handle the
 * caller releases with ua_destroy_problem; on failure it is set to NULL and
 * UA_ERR_INVALID_ARG (a field out of range) or UA_ERR_UNSUPPORTED (valid but
 * not built, e.g. head_dim 96) is returned with a message. */
ua_status_t ua_create_problem(const ua_problem_desc_t* desc, ua_problem_t* out);

/* Bytes of device workspace ua_run needs at the description's maxima: the
 * split-KV partials of section 5 of the unified page (un-normalised o, the
 * running max m and the denominator l per query row, head and segment, plus
 * the stream-K slots).  The caller allocates and owns it; ua_run only
 * borrows it for the duration of the enqueued work.  0 for a NULL handle. */
size_t ua_workspace_size(ua_problem_t problem);

/* The plan ua_run would launch for these host-side shape values: section 6 of
 * the unified page's choice between the 2D query-tile kernel and the 3D
 * split-KV kernel, with its geometry (host only; planned for
 * desc.num_cus, or 256 compute units when that is 0).  Returns
 * UA_ERR_INVALID_ARG when a shape exceeds the problem's maxima. */
ua_status_t ua_query_plan(ua_problem_t problem, int32_t num_seqs, int64_t total_q,
                          int32_t max_seqlen_q, int32_t max_seqlen_k, ua_plan_info_t* info);

/* Enqueue one forward pass on `stream`: section 1's operation of the unified
 * page for every row of the batch, by the strategy of sections 4-6
 * (asynchronous; nothing is read back to the host).  Arguments are described
 * at ua_run_args_t; the caller keeps every buffer alive until the stream has
 * run the work.  Validation errors (UA_ERR_INVALID_ARG, UA_ERR_WORKSPACE)
 * return before anything is enqueued; UA_ERR_HIP reports a failed launch.  A
 * class-split run forks its stream-K launch onto a stream the handle owns
 * (created, at default priority, on the first such run; the handle then stays
 * on that device) and joins it back into `stream` before returning, so work
 * enqueued on `stream` afterwards sees the whole output.  A handle serves one
 * host thread at a time. */
ua_status_t ua_run(ua_problem_t problem, const ua_run_args_t* args, void* stream);

/* Combine partial states over disjoint key sets of the same rows into O (and
 * optionally the LSE): section 5 of the unified page's log-sum-exp re-base,
 * LSE = ln(sum_i e^{lse_i} + e^{sink}) and O = sum_i o_i e^{lse_i - LSE}, with
 * the sink (one more softmax column without a value row, section 1) joined
 * exactly once.  A row whose sets are all empty and that has no sink gets
 * O = 0 and LSE = -inf.  Asynchronous on `stream`; the sets may be any of
 * this or other calls' outputs (they are only read).  UA_ERR_INVALID_ARG for
 * a count outside [1, UA_MAX_MERGE_SETS], a NULL or misaligned pointer, or a
 * shape or type out of range; UA_ERR_HIP for a failed launch. */
ua_status_t ua_merge(const ua_merge_args_t* args, void* stream);

/* ua_run for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * plan and kernels as ua_run, but the split-KV partials live in a scratch
 * array the library holds on each GPU it runs on (128 MiB, kept until the
 * process ends), so `workspace` must be NULL and `workspace_bytes` 0
 * (UA_ERR_INVALID_ARG otherwise).  Nothing is allocated or freed: a batch
 * whose partials do not fit returns UA_ERR_WORKSPACE before anything is
 * enqueued (the stream-K workers are capped to the slots the scratch holds;
 * a segmented split must fit whole), except a decode-shaped batch whose
 * stream-K slots do not fit, which runs on the 2D path (no partials).  A
 * class-split batch runs its two launches one after the other on `stream`
 * instead of forking a side stream.
 * No part of the scratch needs to start at zero: every partial the reduce
 * reads is written earlier by the same call.  Calls on one GPU share its
 * scratch, so calls whose work overlaps on that GPU (other streams, other
 * threads) race: serialise them.  The first call on a device looks up the
 * scratch's device address (HIP may load the library's code object then). */
ua_status_t ua_run_no_alloc(ua_problem_t problem, const ua_run_args_t* args, void* stream);

/* Release a handle made by ua_create_problem (NULL is ignored).  Work already
 * enqueued with it must have completed (it may own a side stream). */
void ua_destroy_problem(ua_problem_t problem);

/* Thread-local text of the last failure in this thread ("" if none): the
 * reason a validation step rejected its input, in the manner of the dense
 * prefill page's argument checks.  The string stays valid until the thread's
 * next call into the library. */
const char* ua_last_error(void);

/* Library version, "major.minor.patch" (a static string). */
const char* ua_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UA_H */

// ua_internal.h -- parameters shared by the host plan and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Everything a kernel of the family reads, passed by value at launch.
struct UaKernelParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* cu_q;
    const float* slopes;      // ALiBi slopes (natural units) or null
    const float* sinks;       // sink logits (natural units) or null
    float* lse;               // optional [total_q, H_q] natural-log row LSE (NULL: skip)
    const float* qq_bias;     // [q_local][k_local] query-section bias (QQ_BIAS flag)
    const int32_t* cu_k;      // dense K/V: first row of each sequence (else NULL)
    int qq_stride;
    void* ws_o;               // split partials: un-normalised o  [rows, NS, D] (f32, or
                              // bf16 when ws_bf16)
    float* ws_m;              //                 running max (log2 units) [rows, NS]
    float* ws_l;              //                 denominator           [rows, NS]
    int64_t q_stride_tok;     // elements
    int64_t o_stride_tok;     // elements
    int64_t kv_slot_stride;   // elements between consecutive slots = H_k * D
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;            // g = H_q / H_k
    int32_t block_size_log2;
    int32_t bt_stride;
    int32_t block_q;          // query positions per q-block
    int32_t rows_used;        // block_q * g  (<= rows per workgroup)
    int32_t tile_n;           // keys per KV tile of the attention kernel
    int32_t tiles_per_seg;    // split path: KV tiles per segment
    int32_t num_segments;     // split path: segments per q-block (workspace stride)
    uint32_t flags;           // UA_FLAG_* bits
    int32_t window;
    float qk_scale_log2;      // tau * k_scale * log2(e)
    float softcap_in;         // tau * k_scale / c
    float softcap_in2;        // 2 log2(e) tau * k_scale / c (argument of 2^x for e^{2y})
    float softcap_out;        // c * log2(e)
    float out_scale;          // v_scale for fp8 V, else 1
    int32_t sk_workers;       // stream-K split: number of workers W
    int32_t class_mode;       // 0: every sequence; 1: only sequences with q_len <=
                              // small_block_q; 2: only the others
    int32_t small_block_q;    // query positions of a single-wave q-block (32 / g)
    int32_t reduce_by_seq;    // stream-K reduce rows enumerated as (seq, head, i)
    int32_t sk_heads;         // stream-K: kv heads one worker serves together (a wave each)
    int32_t ws_bf16;          // split partials' o stored as bf16 (UA_FLAG_BF16_PARTIALS)
    // partial-output mode (NULL: normal run): each row's normalised o over
    // this call's keys, [total_q, H_q, D] f32 or bf16, and its natural-log
    // LSE [total_q, H_q], both without sinks, instead of O
    void* part_o;
    float* part_lse;
    int32_t part_bf16;
    int32_t* queue;           // persistent schedule: kPersistQueues work-queue counters
    int32_t persist_slots;    // persistent schedule: q-block slots per kv head
};

// Work queues of the persistent 2D schedule (one per XCD of an MI355X).
constexpr int kPersistQueues = 8;

// Upper bound on stream-K workers (sizes the workspace before the device is known).
constexpr int kMaxStreamKWorkers = 8192;
// Waves of the widest stream-K worker (one per kv head of its group).
constexpr int kSkMaxWorkerWaves = 8;
// KV tile of the single-wave (decode) geometry, the only one the stream-K split uses.
constexpr int kSkTile = 32;

struct UaLaunch {
    int path;        // 2 or 3
    int waves;       // 1 or 4
    int tile_n;
    int head_dim;
    int q_dtype;     // UA_DTYPE_BF16 / UA_DTYPE_F16
    int kv_fp8;      // 1 when K/V are e4m3fn
    unsigned grid[3];
    int stream_k;    // split path: 1 = stream-K workers (single-wave geometry)
    int rows16;      // stream-K with 16-row q-blocks (16x16x32 MFMA engine)
    int64_t reduce_rows;  // split path: total_q * H_q
    hipEvent_t events[3]; // optional: before attention, between kernels, at the end
    int sk_waves_cap;     // stream-K: at most this many workers * waves per worker (the
                          // workspace holds that many slots beyond one per (seq, kv head))
    int persistent;       // 2D LDS-ring launch on the persistent schedule
};

// Caller-held partial states merged by ua_merge (one wave per row).
constexpr int kMaxMergeSets = 8;
struct UaMergeParams {
    const void* o[kMaxMergeSets];    // per set: [rows, D] o / l (f32 or bf16)
    const float* lse[kMaxMergeSets]; // per set: [rows] natural-log LSE
    int num_sets;
    int part_bf16;
    int64_t rows;                    // total_q * H_q
    int num_q_heads;
    int head_dim;
    int out_dtype;                   // UA_DTYPE_BF16 / UA_DTYPE_F16
    void* out;                       // [total_q, H_q, D], token stride out_stride_tok
    int64_t out_stride_tok;
    float* out_lse;                  // optional [rows]
    const float* sinks;              // optional [H_q] natural-log logits
};

hipError_t ua_launch_merge(const UaMergeParams& p, hipStream_t s);
hipError_t ua_launch_d64(const UaKernelParams& p, const UaLaunch& l, hipStream_t s);
hipError_t ua_launch_d128(const UaKernelParams& p, const UaLaunch& l, hipStream_t s);
hipError_t ua_launch_d256(const UaKernelParams& p, const UaLaunch& l, hipStream_t s);

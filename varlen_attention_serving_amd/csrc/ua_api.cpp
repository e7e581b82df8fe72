// ua_api.cpp -- the C boundary: validation, the shape plan and the launches.
//
// The plan follows "Unified paged attention on gfx950, from the math up",
// section 6: the 2D query-tile kernel when the q-block x kv-head grid already
// fills the device (at least 4 workgroups per compute unit), when the
// context is short (S_k <= 512) or under a sliding window; otherwise the 3D
// split-KV kernel plus its log-sum-exp reduce.  Everything is decided from
// host values (no device reads, no synchronisation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <string>

#include "ua.h"
#include "ua_internal.h"

namespace {

constexpr int kNumCUs = 256;            // MI355X compute units
constexpr int kMinTilesPerSegment = 4;  // keep each split segment worth its partials
constexpr int kSplitTargetWorkgroups = 8 * kNumCUs;
constexpr size_t kWorkspaceCap = size_t(2) << 30;
constexpr float kLog2e = 1.4426950408889634f;

thread_local std::string g_error;

ua_status_t fail(ua_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) { int l = 0; while ((int64_t(1) << l) < x) ++l; return l; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct ua_problem {
    ua_problem_desc_t d;
    int group;
    int log2_block;
    bool fp8;
    size_t ws_bytes;
};

namespace {

int row_bytes(const ua_problem& P) { return (P.d.head_dim + 2) * 4; }

struct Plan {
    int path, waves, tile_n, block_m, block_q, num_segments, tiles_per_seg, stream_k;
    int64_t slots;
    unsigned grid[3];
};

// stream-K partial slots: one per (sequence, kv-head) pair plus one per worker
size_t stream_k_bytes(const ua_problem& P, int64_t num_seqs, int rows_per_slot) {
    return (size_t)(num_seqs * P.d.num_kv_heads + kMaxStreamKWorkers) * rows_per_slot *
           (size_t)row_bytes(P);
}

ua_status_t make_plan(const ua_problem& P, int32_t num_seqs, int64_t total_q, int32_t max_q,
                      int32_t max_k, Plan* out) {
    const ua_problem_desc_t& d = P.d;
    Plan pl{};
    // geometry: one wave of 32 rows when the rows of any q-block fit in it
    // (decode-like batches), else four waves (128 rows) sharing each KV tile;
    // 32-key tiles keep every variant at three or more waves per SIMD
    const bool small = (int64_t)std::max(max_q, 1) * P.group <= 32;
#if defined(UA_EXPERIMENT_WIDE)
    pl.waves = small ? 1 : UA_WIDE_WAVES;
    pl.tile_n = small ? 32 : (d.head_dim >= 256 ? 32 : UA_WIDE_TILE_N);
#else
    pl.waves = small ? 1 : 4;
    pl.tile_n = 32;
#endif
    {
        // a tile must hold whole passes of the workgroup's 16-byte row chunks
        const int chunks_per_row = d.head_dim * (P.fp8 ? 1 : 2) / 16;
        const int rows_per_pass = pl.waves * 64 / chunks_per_row;
        pl.tile_n = std::max(pl.tile_n, rows_per_pass);
    }
    pl.block_m = 32 * pl.waves;
    pl.block_q = pl.block_m / P.group;
    pl.slots = total_q / pl.block_q + num_seqs;
    if (pl.slots > INT32_MAX / 2) return fail(UA_ERR_UNSUPPORTED, "too many query blocks");

    const bool window = d.flags & UA_FLAG_WINDOW;
    bool two_d = (int64_t)d.num_kv_heads * pl.slots >= 4 * kNumCUs || max_k <= 512 || window;
    if (d.flags & UA_FLAG_FORCE_2D) two_d = true;
    if (d.flags & UA_FLAG_FORCE_3D) two_d = false;

    if (two_d) {
        pl.path = 2;
        pl.num_segments = 1;
        pl.tiles_per_seg = 0;
        pl.grid[0] = d.num_kv_heads;
        pl.grid[1] = (unsigned)pl.slots;
        pl.grid[2] = 1;
    } else if (small && d.split_segment_tiles == 0 &&
               (int64_t)num_seqs * d.num_kv_heads * (cdiv(std::max(max_k, 1), kSkTile) + 1) <
                   INT32_MAX) {
        // every sequence's rows fit one q-block: balance KV tiles over workers
        pl.path = 3;
        pl.stream_k = 1;
        pl.num_segments = 0;
        pl.tiles_per_seg = 0;
        pl.grid[0] = 0;  // resident worker count, fixed at launch
        pl.grid[1] = 1;
        pl.grid[2] = 1;
        if (stream_k_bytes(P, num_seqs, pl.block_q * P.group) > P.ws_bytes)
            return fail(UA_ERR_WORKSPACE, "workspace too small for the split path");
    } else {
        pl.path = 3;
        const int64_t max_tiles = std::max<int64_t>(1, cdiv(std::max(max_k, 1), pl.tile_n));
        // expected live tiles (ragged lengths: about half of the maximum) over
        // the workgroups we want resident
        const int64_t live_blocks = std::min<int64_t>(pl.slots, num_seqs + total_q / pl.block_q);
        const int64_t work = std::max<int64_t>(1, d.num_kv_heads * live_blocks * max_tiles / 2);
        int64_t tps = std::max<int64_t>(kMinTilesPerSegment, cdiv(work, kSplitTargetWorkgroups));
        if (d.split_segment_tiles > 0) tps = d.split_segment_tiles;
        tps = std::min(tps, max_tiles);
        int64_t ns = cdiv(max_tiles, tps);
        const int64_t rows = std::max<int64_t>(1, total_q * d.num_q_heads);
        const int64_t cap = (int64_t)(P.ws_bytes / ((size_t)rows * row_bytes(P)));
        if (cap < 1) return fail(UA_ERR_WORKSPACE, "workspace too small for the split path");
        if (ns > cap) {
            tps = cdiv(max_tiles, cap);
            ns = cdiv(max_tiles, tps);
        }
        pl.num_segments = (int)ns;
        pl.tiles_per_seg = (int)tps;
        pl.grid[0] = (unsigned)pl.slots;
        pl.grid[1] = d.num_kv_heads;
        pl.grid[2] = (unsigned)ns;
    }
    *out = pl;
    return UA_OK;
}

}  // namespace

extern "C" {

const char* ua_version(void) { return "0.1.0"; }

const char* ua_last_error(void) { return g_error.c_str(); }

ua_status_t ua_create_problem(const ua_problem_desc_t* desc, ua_problem_t* out) {
    g_error.clear();
    if (!desc || !out) return fail(UA_ERR_INVALID_ARG, "null descriptor or output handle");
    *out = nullptr;
    const ua_problem_desc_t& d = *desc;
    if (d.num_q_heads <= 0 || d.num_kv_heads <= 0)
        return fail(UA_ERR_INVALID_ARG, "head counts must be positive (H_q=%d, H_k=%d)",
                    d.num_q_heads, d.num_kv_heads);
    if (d.num_q_heads % d.num_kv_heads)
        return fail(UA_ERR_INVALID_ARG, "H_q (%d) must be a multiple of H_k (%d)", d.num_q_heads,
                    d.num_kv_heads);
    const int g = d.num_q_heads / d.num_kv_heads;
    if (g > 128) return fail(UA_ERR_UNSUPPORTED, "GQA group %d exceeds 128", g);
    if (d.head_dim <= 0) return fail(UA_ERR_INVALID_ARG, "head_dim must be positive");
    if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
        return fail(UA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128, 256)", d.head_dim);
    if (!is_pow2(d.block_size) || d.block_size > 1024)
        return fail(UA_ERR_INVALID_ARG, "block_size %d must be a power of two <= 1024",
                    d.block_size);
    if (d.q_dtype != UA_DTYPE_BF16 && d.q_dtype != UA_DTYPE_F16)
        return fail(UA_ERR_UNSUPPORTED, "q_dtype %d unsupported (bf16, f16)", d.q_dtype);
    if (d.kv_dtype != d.q_dtype && d.kv_dtype != UA_DTYPE_FP8_E4M3)
        return fail(UA_ERR_UNSUPPORTED, "kv_dtype %d must equal q_dtype or be fp8 e4m3",
                    d.kv_dtype);
    const uint32_t known = UA_FLAG_CAUSAL | UA_FLAG_SOFTCAP | UA_FLAG_ALIBI | UA_FLAG_WINDOW |
                           UA_FLAG_SINKS | UA_FLAG_FORCE_2D | UA_FLAG_FORCE_3D;
    if (d.flags & ~known) return fail(UA_ERR_INVALID_ARG, "unknown flag bits 0x%x", d.flags & ~known);
    if ((d.flags & UA_FLAG_FORCE_2D) && (d.flags & UA_FLAG_FORCE_3D))
        return fail(UA_ERR_INVALID_ARG, "FORCE_2D and FORCE_3D are exclusive");
    if (!(d.scale > 0.0f) || !std::isfinite(d.scale))
        return fail(UA_ERR_INVALID_ARG, "scale must be positive and finite");
    if ((d.flags & UA_FLAG_SOFTCAP) && (!(d.softcap > 0.0f) || !std::isfinite(d.softcap)))
        return fail(UA_ERR_INVALID_ARG, "softcap must be positive and finite when flagged");
    if ((d.flags & UA_FLAG_WINDOW) && d.window <= 0)
        return fail(UA_ERR_INVALID_ARG, "window must be positive when flagged");
    if (d.kv_dtype == UA_DTYPE_FP8_E4M3 &&
        (!(d.k_scale > 0.0f) || !(d.v_scale > 0.0f) || !std::isfinite(d.k_scale) ||
         !std::isfinite(d.v_scale)))
        return fail(UA_ERR_INVALID_ARG, "fp8 K/V need positive finite k_scale and v_scale");
    if (d.num_blocks <= 0) return fail(UA_ERR_INVALID_ARG, "num_blocks must be positive");
    if (d.max_num_seqs < 0 || d.max_total_q < 0 || d.max_seqlen_k < 0 || d.max_blocks_per_seq < 0)
        return fail(UA_ERR_INVALID_ARG, "negative maxima");
    if (d.max_total_q > INT32_MAX) return fail(UA_ERR_UNSUPPORTED, "max_total_q exceeds 2^31");
    if (d.split_segment_tiles < 0)
        return fail(UA_ERR_INVALID_ARG, "split_segment_tiles must be >= 0");
    if ((int64_t)d.max_blocks_per_seq * d.block_size < d.max_seqlen_k)
        return fail(UA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size < max_seqlen_k");

    ua_problem* P = new (std::nothrow) ua_problem;
    if (!P) return fail(UA_ERR_INVALID_ARG, "out of host memory");
    P->d = d;
    P->group = g;
    P->log2_block = ilog2(d.block_size);
    P->fp8 = d.kv_dtype == UA_DTYPE_FP8_E4M3;
    // split workspace: enough segments for the smallest tile (32 keys) and the
    // minimum segment length at the maxima, capped at 2 GiB (a larger batch
    // then gets fewer, longer segments)
    const size_t rows = (size_t)std::max<int64_t>(1, d.max_total_q) * d.num_q_heads;
    const size_t per_seg = rows * (size_t)row_bytes(*P);
    const int64_t min_tps = d.split_segment_tiles > 0
                                ? std::min<int64_t>(d.split_segment_tiles, kMinTilesPerSegment)
                                : kMinTilesPerSegment;
    const int64_t ns_max =
        std::max<int64_t>(1, cdiv(cdiv(std::max(d.max_seqlen_k, 1), 32), min_tps));
    const int64_t ns_cap = std::max<int64_t>(1, (int64_t)(kWorkspaceCap / per_seg));
    P->ws_bytes = per_seg * (size_t)std::min(ns_max, ns_cap);
    // the stream-K split (single-wave geometry, 32 rows per q-block)
    P->ws_bytes = std::max(P->ws_bytes, stream_k_bytes(*P, std::max(d.max_num_seqs, 1), 32));
    *out = P;
    return UA_OK;
}

size_t ua_workspace_size(ua_problem_t p) { return p ? p->ws_bytes : 0; }

void ua_destroy_problem(ua_problem_t p) { delete p; }

ua_status_t ua_query_plan(ua_problem_t p, int32_t num_seqs, int64_t total_q, int32_t max_seqlen_q,
                          int32_t max_seqlen_k, ua_plan_info_t* info) {
    g_error.clear();
    if (!p || !info) return fail(UA_ERR_INVALID_ARG, "null handle or output");
    if (num_seqs < 0 || num_seqs > p->d.max_num_seqs || total_q < 0 ||
        total_q > p->d.max_total_q || max_seqlen_k < 0 || max_seqlen_k > p->d.max_seqlen_k ||
        max_seqlen_q < 0 || max_seqlen_q > max_seqlen_k)
        return fail(UA_ERR_INVALID_ARG, "shape outside the problem's maxima");
    Plan pl;
    ua_status_t st = make_plan(*p, num_seqs, total_q, max_seqlen_q, max_seqlen_k, &pl);
    if (st != UA_OK) return st;
    info->path = pl.path;
    info->block_m = pl.block_m;
    info->block_q = pl.block_q;
    info->tile_n = pl.tile_n;
    info->waves = pl.waves;
    info->num_segments = pl.num_segments;
    info->tiles_per_segment = pl.tiles_per_seg;
    for (int i = 0; i < 3; ++i) info->grid[i] = (int32_t)pl.grid[i];
    const int esz = p->fp8 ? 1 : 2;
    info->stream_k = pl.stream_k;
    info->use_i64_kv =
        (double)p->d.num_blocks * p->d.block_size * p->d.num_kv_heads * p->d.head_dim * esz >
        2147483648.0;
    return UA_OK;
}

ua_status_t ua_run(ua_problem_t p, const ua_run_args_t* a, void* stream) {
    g_error.clear();
    if (!p || !a) return fail(UA_ERR_INVALID_ARG, "null handle or arguments");
    const ua_problem_desc_t& d = p->d;
    if (a->num_seqs < 0 || a->num_seqs > d.max_num_seqs)
        return fail(UA_ERR_INVALID_ARG, "num_seqs %d outside [0, %d]", a->num_seqs, d.max_num_seqs);
    if (a->total_q < 0 || a->total_q > d.max_total_q)
        return fail(UA_ERR_INVALID_ARG, "total_q %lld outside [0, %lld]", (long long)a->total_q,
                    (long long)d.max_total_q);
    if (a->max_seqlen_k < 0 || a->max_seqlen_k > d.max_seqlen_k)
        return fail(UA_ERR_INVALID_ARG, "max_seqlen_k %d outside [0, %d]", a->max_seqlen_k,
                    d.max_seqlen_k);
    if (a->max_seqlen_q < 0 || a->max_seqlen_q > a->max_seqlen_k ||
        (int64_t)a->max_seqlen_q > a->total_q)
        return fail(UA_ERR_INVALID_ARG, "max_seqlen_q %d inconsistent", a->max_seqlen_q);
    if (a->num_seqs == 0 || a->total_q == 0) return UA_OK;

    const int64_t row_elems = (int64_t)d.num_q_heads * d.head_dim;
    if (a->q_stride_tok < row_elems || a->o_stride_tok < row_elems)
        return fail(UA_ERR_INVALID_ARG, "token strides must be >= H_q * head_dim");
    if (a->q_stride_tok % 8 || a->o_stride_tok % 8)
        return fail(UA_ERR_INVALID_ARG, "token strides must be multiples of 8 elements");
    if (a->block_table_stride < cdiv(a->max_seqlen_k, d.block_size) ||
        a->block_table_stride > std::max(d.max_blocks_per_seq, 1))
        return fail(UA_ERR_INVALID_ARG, "block_table_stride %d outside [ceil(max_seqlen_k/b), %d]",
                    a->block_table_stride, d.max_blocks_per_seq);
    if (!a->q || !a->k_cache || !a->v_cache || !a->o || !a->block_table || !a->seq_lens ||
        !a->cu_seqlens_q)
        return fail(UA_ERR_INVALID_ARG, "null required device pointer");
    if ((d.flags & UA_FLAG_ALIBI) && !a->alibi_slopes)
        return fail(UA_ERR_INVALID_ARG, "ALiBi flagged but alibi_slopes is null");
    if ((d.flags & UA_FLAG_SINKS) && !a->sinks)
        return fail(UA_ERR_INVALID_ARG, "sinks flagged but sinks is null");
    if (((uintptr_t)a->q | (uintptr_t)a->o | (uintptr_t)a->k_cache | (uintptr_t)a->v_cache) & 15)
        return fail(UA_ERR_INVALID_ARG, "q, o, k_cache and v_cache must be 16-byte aligned");

    Plan pl;
    ua_status_t st = make_plan(*p, a->num_seqs, a->total_q, a->max_seqlen_q, a->max_seqlen_k, &pl);
    if (st != UA_OK) return st;

    UaKernelParams kp{};
    kp.q = a->q;
    kp.k = a->k_cache;
    kp.v = a->v_cache;
    kp.o = a->o;
    kp.block_table = a->block_table;
    kp.seq_lens = a->seq_lens;
    kp.cu_q = a->cu_seqlens_q;
    kp.slopes = (d.flags & UA_FLAG_ALIBI) ? a->alibi_slopes : nullptr;
    kp.sinks = (d.flags & UA_FLAG_SINKS) ? a->sinks : nullptr;
    kp.q_stride_tok = a->q_stride_tok;
    kp.o_stride_tok = a->o_stride_tok;
    kp.kv_slot_stride = (int64_t)d.num_kv_heads * d.head_dim;
    kp.num_seqs = a->num_seqs;
    kp.num_q_heads = d.num_q_heads;
    kp.num_kv_heads = d.num_kv_heads;
    kp.group = p->group;
    kp.block_size_log2 = p->log2_block;
    kp.bt_stride = a->block_table_stride;
    kp.block_q = pl.block_q;
    kp.rows_used = pl.block_q * p->group;
    kp.tile_n = pl.tile_n;
    kp.tiles_per_seg = pl.tiles_per_seg;
    kp.num_segments = pl.num_segments;
    kp.flags = d.flags;
    kp.window = (d.flags & UA_FLAG_WINDOW) ? d.window : 0;
    const float kscale = p->fp8 ? d.k_scale : 1.0f;
    kp.qk_scale_log2 = d.scale * kscale * kLog2e;
    kp.softcap_in = (d.flags & UA_FLAG_SOFTCAP) ? d.scale * kscale / d.softcap : 0.0f;
    kp.softcap_out = (d.flags & UA_FLAG_SOFTCAP) ? d.softcap * kLog2e : 0.0f;
    kp.out_scale = p->fp8 ? d.v_scale : 1.0f;

    if (pl.path == 3 && pl.stream_k) {
        const int rows_per_slot = pl.block_q * p->group;
        const size_t slots = (size_t)a->num_seqs * d.num_kv_heads + kMaxStreamKWorkers;
        const size_t need = stream_k_bytes(*p, a->num_seqs, rows_per_slot);
        if (!a->workspace || a->workspace_bytes < need)
            return fail(UA_ERR_WORKSPACE, "split path needs %zu workspace bytes, got %zu", need,
                        a->workspace ? a->workspace_bytes : (size_t)0);
        if ((uintptr_t)a->workspace & 255)
            return fail(UA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        float* ws = static_cast<float*>(a->workspace);
        const size_t rows = slots * rows_per_slot;
        kp.ws_o = ws;
        kp.ws_m = ws + rows * d.head_dim;
        kp.ws_l = kp.ws_m + rows;
    } else if (pl.path == 3) {
        const size_t rows = (size_t)a->total_q * d.num_q_heads;
        const size_t need = rows * (size_t)pl.num_segments * row_bytes(*p);
        if (!a->workspace || a->workspace_bytes < need)
            return fail(UA_ERR_WORKSPACE, "split path needs %zu workspace bytes, got %zu", need,
                        a->workspace ? a->workspace_bytes : (size_t)0);
        if ((uintptr_t)a->workspace & 255)
            return fail(UA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        float* ws = static_cast<float*>(a->workspace);
        kp.ws_o = ws;
        kp.ws_m = ws + rows * pl.num_segments * d.head_dim;
        kp.ws_l = kp.ws_m + rows * pl.num_segments;
    }

    UaLaunch l{};
    l.path = pl.path;
    l.waves = pl.waves;
    l.tile_n = pl.tile_n;
    l.head_dim = d.head_dim;
    l.q_dtype = d.q_dtype;
    l.kv_fp8 = p->fp8;
    for (int i = 0; i < 3; ++i) l.grid[i] = pl.grid[i];
    l.stream_k = pl.stream_k;
    l.reduce_rows = a->total_q * d.num_q_heads;
    for (int i = 0; i < 3; ++i) l.events[i] = static_cast<hipEvent_t>(a->timing_events[i]);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (d.head_dim) {
        case 64: e = ua_launch_d64(kp, l, s); break;
        case 128: e = ua_launch_d128(kp, l, s); break;
        default: e = ua_launch_d256(kp, l, s); break;
    }
    if (e != hipSuccess) return fail(UA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return UA_OK;
}

}  // extern "C"

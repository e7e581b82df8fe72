// ua_api.cpp -- the C boundary: validation, the shape plan and the launches.
//
// The plan follows "Unified paged attention on gfx950, from the math up",
// section 6: the 2D query-tile kernel when the q-block x kv-head grid already
// fills the device (at least 4 workgroups per compute unit) or when a q-block
// visits few keys (a short context or a short sliding window); otherwise the
// 3D split-KV kernel plus its log-sum-exp reduce.  In a batch of wide
// q-blocks the decode-shaped sequences go to a stream-K launch that runs
// beside the wide one.  Everything is decided from host values (no device
// reads, no synchronisation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "ua.h"
#include "ua_internal.h"

namespace {

constexpr int kDefaultCUs = 256;        // MI355X compute units (plans made without a device)
constexpr int kMinTilesPerSegment = 4;  // keep each split segment worth its partials
constexpr int kSplitWorkgroupsPerCU = 8;
constexpr int kWideResidentPerCU = 3;   // four-wave workgroups resident per CU
constexpr int kMaxWideSegments = 2;
constexpr size_t kWorkspaceCap = size_t(2) << 30;
constexpr size_t kQueueBytes = 256;     // persistent schedule: queue counters
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
    bool ws_bf16;  // split partial o stored as bf16
    size_t ws_bytes;
    // a split batch runs its stream-K launch on a second stream, forked from
    // and joined back into the caller's (created on the first split run)
    int side_device = -1;
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    ~ua_problem() {
        if (side) (void)hipStreamDestroy(side);
        if (fork) (void)hipEventDestroy(fork);
        if (join) (void)hipEventDestroy(join);
    }
};

namespace {

// workspace bytes of one partial row: o (f32, or bf16) then m and l (f32)
int row_bytes(const ua_problem& P) { return P.d.head_dim * (P.ws_bf16 ? 2 : 4) + 8; }
int o_elem_bytes(const ua_problem& P) { return P.ws_bf16 ? 2 : 4; }

// One kernel launch of the plan (plus its reduce on the split path).
struct Sub {
    int path;          // 2 = query-tile kernel, 3 = split-KV kernel + reduce
    int stream_k;      // split path: balanced workers (single-wave geometry)
    int waves, tile_n, block_m, block_q, num_segments, tiles_per_seg;
    int class_mode;    // 0 all sequences, 1 single-wave ones only, 2 the others
    int rows16;        // stream-K with 16-row q-blocks
    int64_t slots;
    unsigned grid[3];
};

struct Plan {
    int n;             // 1, or 2 when decode rows of a wide batch go to stream-K
    Sub sub[2];        // sub[n - 1] holds the rows of the widest geometry
    int small_block_q; // positions of a stream-K q-block (16 / g on the 16-row
                       // engine, else 32 / g; 0 if g > 32)
};

// stream-K partial slots: one per (sequence, kv-head) pair plus one per
// worker wave (at most `extra` of them)
size_t stream_k_bytes(const ua_problem& P, int64_t num_seqs, int rows_per_slot,
                      int64_t extra = kMaxStreamKWorkers) {
    const size_t b = (size_t)(num_seqs * P.d.num_kv_heads + extra) * rows_per_slot *
                     (size_t)row_bytes(P);
    return (b + 255) & ~size_t(255);
}

void geometry(const ua_problem& P, int waves, Sub* g) {
    const ua_problem_desc_t& d = P.d;
    g->waves = waves;
    g->tile_n = 32;
    // a tile must hold whole passes of the workgroup's 16-byte row chunks
    const int chunks_per_row = d.head_dim * (P.fp8 ? 1 : 2) / 16;
    g->tile_n = std::max(g->tile_n, waves * 64 / chunks_per_row);
    g->block_m = 32 * waves;
    g->block_q = g->block_m / P.group;
}

// Stream-K q-blocks of 16 rows (the 16x16x32 decode engine; g <= 16), taken
// at d = 256, where the 32-row engine's accumulators hold it to one wave per
// SIMD (measured: at d <= 128 the 32-row engine streams faster).
bool use_rows16(const ua_problem& P) { return P.d.head_dim == 256 && P.group <= 16; }

// The 32-row stream-K engine is not built for d = 256 with 16-bit K/V and the
// QQ bias: in that instantiation the compiler (hipcc, ROCm 7.2) spills part of
// a Q fragment and then feeds the MFMA a stale register in its place (a copy
// it makes is never read), so its scores are wrong.  Such batches take the
// segmented split or the 2D path instead.
bool sk32_built(const ua_problem& P) {
    return !(P.d.head_dim == 256 && !P.fp8 && (P.d.flags & UA_FLAG_QQ_BIAS));
}

void rows16(const ua_problem& P, Sub* g) {
    g->rows16 = 1;
    g->tile_n = kSkTile;
    g->block_m = 16;
    g->block_q = 16 / P.group;
}

// The segmented split: grid z holds the segments; each q-block cuts its own
// live tile range into up to that many near-equal runs of about
// tiles_per_seg tiles (the kernel and the reduce agree on the cut).
ua_status_t segmented(const ua_problem& P, int cus, int64_t total_q, int64_t live_blocks,
                      int64_t span, size_t ws_cap, Sub* g) {
    const ua_problem_desc_t& d = P.d;
    g->path = 3;
    const int64_t max_tiles = std::max<int64_t>(1, cdiv(std::max<int64_t>(span, 1), g->tile_n) + 1);
    // expected live tiles (ragged lengths: about half of the maximum) over
    // the workgroups we want resident
    const int64_t work = std::max<int64_t>(1, d.num_kv_heads * live_blocks * max_tiles / 2);
    int64_t tps = std::max<int64_t>(kMinTilesPerSegment, cdiv(work, (int64_t)kSplitWorkgroupsPerCU * cus));
    int64_t ns = 0;
    if (g->waves > 1 && d.split_segment_tiles == 0) {
        // about two resident rounds of wide workgroups: each q-block cuts its
        // own tile range into up to ns runs of at least kMinTilesPerSegment
        const int64_t grid = std::max<int64_t>(1, d.num_kv_heads * (total_q / g->block_q + 1));
        ns = std::min<int64_t>(kMaxWideSegments, cdiv((int64_t)2 * kWideResidentPerCU * cus, grid));
        tps = kMinTilesPerSegment;
        ns = std::max<int64_t>(1, std::min(ns, cdiv(max_tiles, tps)));
    } else {
        if (d.split_segment_tiles > 0) tps = d.split_segment_tiles;
        tps = std::min(tps, max_tiles);
        ns = cdiv(max_tiles, tps);
    }
    const int64_t rows = std::max<int64_t>(1, total_q * d.num_q_heads);
    const int64_t cap = (int64_t)(ws_cap / ((size_t)rows * row_bytes(P)));
    if (cap < 1) return fail(UA_ERR_WORKSPACE, "workspace too small for the split path");
    if (ns > cap) {
        tps = cdiv(max_tiles, cap);
        ns = cdiv(max_tiles, tps);
    }
    g->num_segments = (int)ns;
    g->tiles_per_seg = (int)tps;
    g->grid[0] = (unsigned)g->slots;
    g->grid[1] = d.num_kv_heads;
    g->grid[2] = (unsigned)ns;
    return UA_OK;
}

// sk_cap: bytes the stream-K partials may take (the caller's workspace, or
// the no-alloc scratch)
ua_status_t make_plan(const ua_problem& P, int cus, int32_t num_seqs, int64_t total_q,
                      int32_t max_q, int32_t max_k, size_t sk_cap, Plan* out) {
    const ua_problem_desc_t& d = P.d;
    Plan pl{};
    pl.small_block_q = use_rows16(P) ? 16 / P.group : P.group <= 32 ? 32 / P.group : 0;
    const bool force2 = d.flags & UA_FLAG_FORCE_2D;
    const bool force3 = d.flags & UA_FLAG_FORCE_3D;
    // Keys one q-block can visit.  The shape rule of section 6 of the unified
    // page keeps short contexts and sliding windows on the query-tile path
    // because they leave a q-block only a few KV tiles; the span states that
    // directly (a window of thousands of keys is not short).
    const int64_t span = (d.flags & UA_FLAG_WINDOW)
                             ? std::min<int64_t>(max_k, (int64_t)d.window + std::max(max_q, 1))
                             : max_k;
    // geometry: one wave of 32 rows when every q-block fits in it (decode-like
    // batches), else four waves (128 rows) sharing each KV tile
    const bool small = (int64_t)std::max(max_q, 1) * P.group <= 32;
    const int64_t sk_tiles = (int64_t)num_seqs * d.num_kv_heads * (cdiv(std::max<int64_t>(span, 1), kSkTile) + 2);
    const bool sk_fits = sk_tiles < INT32_MAX;
    // the stream-K engine a decode-shaped batch would take is built
    const bool sk16 = use_rows16(P) && (int64_t)std::max(max_q, 1) * P.group <= 16;
    const bool sk_ok = sk_fits && (sk16 || sk32_built(P));

    Sub& w = pl.sub[0];
    geometry(P, small ? 1 : 4, &w);
    w.slots = total_q / w.block_q + num_seqs;
    if (w.slots > INT32_MAX / 2) return fail(UA_ERR_UNSUPPORTED, "too many query blocks");
    // q-blocks that carry rows (at most one partial block per sequence)
    const int64_t live_blocks = std::min<int64_t>(w.slots, num_seqs + total_q / w.block_q);
    // Decode-shaped batches stream on the stream-K workers whatever their
    // size once a q-block's keys are not short: section 6's grid threshold
    // would send a batch of 128 or more decode rows (at H_k = 8) to the 2D
    // path, where each single-wave q-block walks its own sequence and the
    // ragged lengths leave a tail (measured at d = 128: 128 rows 0.522 ->
    // 0.347 ms, 256 rows 0.890 -> 0.677 ms, 512 rows of 256-4096 keys 0.860 ->
    // 0.730 ms; d = 64: 0.300 -> 0.191 ms).  A batch whose stream-K slots do
    // not fit sk_cap keeps the 2D path, which needs no workspace.
    // Decode-shaped batches without a built stream-K engine follow the wide
    // rule: 2D once the grid fills the device, else the segmented split.
    const bool sk_room = stream_k_bytes(P, num_seqs, 32, kSkMaxWorkerWaves) <= sk_cap;
    const bool grid_full = (int64_t)d.num_kv_heads * w.slots >= (int64_t)4 * cus;
    bool two_d = span <= 512 || (small && sk_ok ? !sk_room : grid_full);
    if (!small && !two_d) {
        // Wide q-blocks carry 128 fp32 rows of partials per segment, so split
        // them only when the query-tile grid is short of one resident round
        // (three four-wave workgroups per CU), and only as far as needed.
        const int64_t wide_grid = (int64_t)d.num_kv_heads * (total_q / w.block_q + 1);
        two_d = wide_grid >= (int64_t)kWideResidentPerCU * cus;
    }
    // Wide q-blocks of 16-bit K/V run on the LDS ring (at d = 256 not with
    // the QQ bias; blocks must hold one copy's 512 / d key rows), which
    // streams a decode-shaped q-block's keys at HBM speed inside the same
    // launch: keep the whole batch in one 2D launch once its full grid
    // (every sequence's slots) fills a resident round.
    const bool ring = !P.fp8 && (d.head_dim <= 128 || !(d.flags & UA_FLAG_QQ_BIAS)) &&
                      (int64_t(1) << P.log2_block) * d.head_dim >= 512 &&
                      (int64_t)d.num_kv_heads * d.head_dim * 2 * (512 / d.head_dim) < (int64_t(1) << 31);
    const bool ring_fills =
        !small && ring && (int64_t)d.num_kv_heads * w.slots >= (int64_t)kWideResidentPerCU * cus;
    if (ring_fills) two_d = true;
    if (force2) two_d = true;
    if (force3) two_d = false;

    // Otherwise the decode-shaped sequences of a wide batch go to the
    // stream-K kernel, beside the wide launch that keeps the rest: for
    // register-staged wide launches (fp8 K/V, d = 256 with the QQ bias,
    // blocks below one copy's rows) and for d = 256 ring batches too small
    // to fill a round (measured with 64 decode rows and 4 chunks of 512:
    // H_k = 8 fills it, one launch 0.70 ms against 0.75 split; H_k = 2 does
    // not, split 0.353 ms against 0.385 in one launch).  A d <= 128 ring batch
    // keeps one launch (the split measured slower there).
    // No split when no sequence can be decode-shaped: the shortest holds at
    // least total_q - (num_seqs - 1) * max_q queries (a loose bound from the
    // caller only costs the split, since the wide launch alone serves every
    // sequence), and a stream-K launch with nothing to do still costs a
    // launch and the wide q-blocks their segments (measured: two fp8 d = 256
    // sequences of 1024 queries, 0.090 -> 0.080 ms a step).
    const bool maybe_decode =
        total_q - (int64_t)(num_seqs - 1) * std::max(max_q, 1) <= (int64_t)pl.small_block_q;
    const bool split = !small && !ring_fills && (!ring || d.head_dim > 128) && !force2 &&
                       !force3 && pl.small_block_q > 0 && maybe_decode && sk_fits &&
                       d.split_segment_tiles == 0 && (use_rows16(P) || sk32_built(P));
    w.class_mode = split ? 2 : 0;
    // Beside a concurrent stream-K launch the wide q-blocks need no segments
    // to fill the device (measured: variant_mix 0.148 -> 0.125 ms unsplit).
    if (split) two_d = true;
    size_t ws_seg = P.ws_bytes;
    if (split) {
        Sub& k = pl.sub[0];
        Sub wide = w;
        geometry(P, 1, &k);
        if (use_rows16(P)) rows16(P, &k);
        k.slots = num_seqs;
        k.path = 3;
        k.stream_k = 1;
        k.class_mode = 1;
        k.grid[0] = 0;
        k.grid[1] = k.grid[2] = 1;
        const size_t skb = stream_k_bytes(P, num_seqs, k.block_q * P.group);
        if (skb > P.ws_bytes) return fail(UA_ERR_WORKSPACE, "workspace too small for the split path");
        ws_seg = P.ws_bytes - skb;
        pl.sub[1] = wide;
        pl.n = 2;
    } else {
        pl.n = 1;
    }
    Sub& g = pl.sub[pl.n - 1];
    if (two_d) {
        g.path = 2;
        g.num_segments = 1;
        g.tiles_per_seg = 0;
        g.grid[0] = d.num_kv_heads;
        g.grid[1] = (unsigned)g.slots;
        g.grid[2] = 1;
    } else if (small && d.split_segment_tiles == 0 && sk_ok) {
        // every sequence's rows fit one q-block: balance KV tiles over workers
        if (sk16) rows16(P, &g);
        g.path = 3;
        g.stream_k = 1;
        g.grid[0] = 0;  // resident worker count, fixed at launch
        g.grid[1] = g.grid[2] = 1;
        if (stream_k_bytes(P, num_seqs, g.block_q * P.group) > P.ws_bytes)
            return fail(UA_ERR_WORKSPACE, "workspace too small for the split path");
    } else {
        ua_status_t st = segmented(P, cus, total_q, live_blocks, span, ws_seg, &g);
        if (st != UA_OK) return st;
    }
    *out = pl;
    return UA_OK;
}

// Compute units of the current device, queried once per device (the plan's
// thresholds are in workgroups per compute unit).  0 when no device answers.
int device_cus() {
    static std::mutex mu;
    static std::vector<std::pair<int, int>> cache;  // (device, CUs)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : cache)
        if (e.first == dev) return e.second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        return 0;
    cache.push_back({dev, cus});
    return cus;
}

// The compute units a plan is sized for: the descriptor's count, else (on the
// run path) the device's, else the MI355X's 256.
int plan_cus(const ua_problem& P, bool on_device) {
    if (P.d.num_cus > 0) return P.d.num_cus;
    const int c = on_device ? device_cus() : 0;
    return c > 0 ? c : kDefaultCUs;
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
                           UA_FLAG_SINKS | UA_FLAG_QQ_BIAS | UA_FLAG_DENSE_KV |
                           UA_FLAG_BF16_PARTIALS | UA_FLAG_PERSISTENT | UA_FLAG_FORCE_2D |
                           UA_FLAG_FORCE_3D;
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
    if (d.num_cus < 0) return fail(UA_ERR_INVALID_ARG, "num_cus must be >= 0");
    const bool dense = (d.flags & UA_FLAG_DENSE_KV) != 0;
    if (dense && d.block_size != 1)
        return fail(UA_ERR_INVALID_ARG, "the dense K/V layout needs block_size 1 (got %d)",
                    d.block_size);
    if (!dense && (int64_t)d.max_blocks_per_seq * d.block_size < d.max_seqlen_k)
        return fail(UA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size < max_seqlen_k");
    if (dense && d.max_seqlen_k > (1 << 30))
        return fail(UA_ERR_UNSUPPORTED, "dense max_seqlen_k above 2^30");

    ua_problem* P = new (std::nothrow) ua_problem;
    if (!P) return fail(UA_ERR_INVALID_ARG, "out of host memory");
    P->d = d;
    P->group = g;
    // the kernels see a dense sequence as one block of 2^30 rows
    P->log2_block = dense ? 30 : ilog2(d.block_size);
    P->fp8 = d.kv_dtype == UA_DTYPE_FP8_E4M3;
    P->ws_bf16 = (d.flags & UA_FLAG_BF16_PARTIALS) != 0;
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
    // the segmented split region, then the stream-K region (single-wave
    // geometry, at most 32 rows per q-block)
    P->ws_bytes = ((per_seg * (size_t)std::min(ns_max, ns_cap) + 255) & ~size_t(255)) +
                  stream_k_bytes(*P, std::max(d.max_num_seqs, 1), 32);
    // the persistent schedule's queue counters (a 2D launch, which uses no
    // other workspace)
    if (d.flags & UA_FLAG_PERSISTENT) P->ws_bytes = std::max<size_t>(P->ws_bytes, kQueueBytes);
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
    ua_status_t st = make_plan(*p, plan_cus(*p, false), num_seqs, total_q, max_seqlen_q,
                               max_seqlen_k, p->ws_bytes, &pl);
    if (st != UA_OK) return st;
    const Sub& g = pl.sub[pl.n - 1];  // the launch holding the widest rows
    info->path = g.path;
    info->block_m = g.block_m;
    info->block_q = g.block_q;
    info->tile_n = g.tile_n;
    info->waves = g.waves;
    info->num_segments = g.num_segments;
    info->tiles_per_segment = g.tiles_per_seg;
    for (int i = 0; i < 3; ++i) info->grid[i] = (int32_t)g.grid[i];
    const int esz = p->fp8 ? 1 : 2;
    info->stream_k = pl.sub[0].stream_k;
    info->class_split = pl.n == 2;
    info->use_i64_kv =
        (double)p->d.num_blocks * p->d.block_size * p->d.num_kv_heads * p->d.head_dim * esz >
        2147483648.0;
    return UA_OK;
}

}  // extern "C"

namespace {

// Scratch for callers that cannot allocate (ua_run_no_alloc): the split-KV
// partials of a run live here instead of in a caller workspace.  Every GPU
// the library runs on holds its own copy until the process ends; calls on
// one GPU share it.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of this device's scratch, looked up once per device
// (with that device current) and kept: in host code `scratch` names a host
// stand-in, not device memory.
ua_status_t scratch_address(void** out) {
    static std::mutex mu;
    static std::vector<std::pair<int, void*>> table;  // (device, address)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(UA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& t : table)
        if (t.first == dev) {
            *out = t.second;
            return UA_OK;
        }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        return fail(UA_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    table.push_back({dev, ptr});
    *out = ptr;
    return UA_OK;
}

// One forward pass.  With `no_alloc` the split partials go to this device's
// scratch (the caller's workspace fields must be empty), the stream-K workers
// are capped to the slots the scratch holds, and a class split runs its two
// launches one after the other on `stream` (no side stream is created).
ua_status_t run_impl(ua_problem_t p, const ua_run_args_t* a, void* stream, bool no_alloc) {
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
    const bool dense = (d.flags & UA_FLAG_DENSE_KV) != 0;
    if (!dense && (a->block_table_stride < cdiv(a->max_seqlen_k, d.block_size) ||
                   a->block_table_stride > std::max(d.max_blocks_per_seq, 1)))
        return fail(UA_ERR_INVALID_ARG, "block_table_stride %d outside [ceil(max_seqlen_k/b), %d]",
                    a->block_table_stride, d.max_blocks_per_seq);
    const bool partial = a->partial_o != nullptr;
    if (!a->q || !a->k_cache || !a->v_cache || (!a->o && !partial) || !a->cu_seqlens_q ||
        (!dense && (!a->block_table || !a->seq_lens)))
        return fail(UA_ERR_INVALID_ARG, "null required device pointer");
    if (partial) {
        if (!a->partial_lse || ((uintptr_t)a->partial_lse & 3))
            return fail(UA_ERR_INVALID_ARG, "partial_o needs a 4-byte aligned partial_lse");
        if ((uintptr_t)a->partial_o & 15)
            return fail(UA_ERR_INVALID_ARG, "partial_o must be 16-byte aligned");
        if (a->partial_dtype != UA_PARTIAL_F32 && a->partial_dtype != UA_PARTIAL_BF16)
            return fail(UA_ERR_INVALID_ARG, "partial_dtype %d unknown", a->partial_dtype);
    }
    if (dense && (!a->cu_seqlens_k || ((uintptr_t)a->cu_seqlens_k & 3)))
        return fail(UA_ERR_INVALID_ARG, "dense K/V need a 4-byte aligned cu_seqlens_k");
    if ((d.flags & UA_FLAG_ALIBI) && !a->alibi_slopes)
        return fail(UA_ERR_INVALID_ARG, "ALiBi flagged but alibi_slopes is null");
    if ((d.flags & UA_FLAG_SINKS) && !a->sinks)
        return fail(UA_ERR_INVALID_ARG, "sinks flagged but sinks is null");
    if (((uintptr_t)a->q | (uintptr_t)a->o | (uintptr_t)a->k_cache | (uintptr_t)a->v_cache) & 15)
        return fail(UA_ERR_INVALID_ARG, "q, o, k_cache and v_cache must be 16-byte aligned");
    if ((uintptr_t)a->lse & 3) return fail(UA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (d.flags & UA_FLAG_QQ_BIAS) {
        if (!a->qq_bias) return fail(UA_ERR_INVALID_ARG, "QQ-bias flagged but qq_bias is null");
        if ((uintptr_t)a->qq_bias & 3)
            return fail(UA_ERR_INVALID_ARG, "qq_bias must be 4-byte aligned");
        if (a->qq_bias_stride < a->max_seqlen_q)
            return fail(UA_ERR_INVALID_ARG, "qq_bias_stride %d below max_seqlen_q %d",
                        a->qq_bias_stride, a->max_seqlen_q);
    }

    Plan pl;
    ua_status_t st = make_plan(*p, plan_cus(*p, true), a->num_seqs, a->total_q, a->max_seqlen_q,
                               a->max_seqlen_k, no_alloc ? kScratchBytes : p->ws_bytes, &pl);
    if (st != UA_OK) return st;

    UaKernelParams base{};
    base.q = a->q;
    base.k = a->k_cache;
    base.v = a->v_cache;
    base.o = a->o;
    base.block_table = dense ? nullptr : a->block_table;
    base.seq_lens = dense ? nullptr : a->seq_lens;
    base.cu_k = dense ? a->cu_seqlens_k : nullptr;
    base.cu_q = a->cu_seqlens_q;
    base.slopes = (d.flags & UA_FLAG_ALIBI) ? a->alibi_slopes : nullptr;
    base.sinks = (d.flags & UA_FLAG_SINKS) ? a->sinks : nullptr;
    base.lse = a->lse;
    base.qq_bias = (d.flags & UA_FLAG_QQ_BIAS) ? a->qq_bias : nullptr;
    base.qq_stride = a->qq_bias_stride;
    base.q_stride_tok = a->q_stride_tok;
    base.o_stride_tok = a->o_stride_tok;
    base.kv_slot_stride = (int64_t)d.num_kv_heads * d.head_dim;
    base.num_seqs = a->num_seqs;
    base.num_q_heads = d.num_q_heads;
    base.num_kv_heads = d.num_kv_heads;
    base.group = p->group;
    base.block_size_log2 = p->log2_block;
    base.bt_stride = dense ? 1 : a->block_table_stride;
    base.flags = d.flags;
    base.window = (d.flags & UA_FLAG_WINDOW) ? d.window : 0;
    const float kscale = p->fp8 ? d.k_scale : 1.0f;
    base.qk_scale_log2 = d.scale * kscale * kLog2e;
    base.softcap_in = (d.flags & UA_FLAG_SOFTCAP) ? d.scale * kscale / d.softcap : 0.0f;
    base.softcap_in2 = 2.0f * kLog2e * base.softcap_in;
    base.softcap_out = (d.flags & UA_FLAG_SOFTCAP) ? d.softcap * kLog2e : 0.0f;
    base.out_scale = p->fp8 ? d.v_scale : 1.0f;
    base.small_block_q = pl.small_block_q;
    base.sk_heads = 1;
    base.ws_bf16 = p->ws_bf16;
    if (partial) {
        // merge-ready states without the sinks, which ua_merge joins once
        base.part_o = a->partial_o;
        base.part_lse = a->partial_lse;
        base.part_bf16 = a->partial_dtype == UA_PARTIAL_BF16;
        base.flags &= ~(uint32_t)UA_FLAG_SINKS;
        base.sinks = nullptr;
        base.lse = nullptr;
    }

    // workspace: [segmented partials][stream-K partials], both 256-byte aligned
    if (no_alloc && (a->workspace || a->workspace_bytes))
        return fail(UA_ERR_INVALID_ARG,
                    "ua_run_no_alloc uses its own scratch: workspace must be NULL and 0 bytes");
    if (a->workspace && ((uintptr_t)a->workspace & 255))
        return fail(UA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    size_t need = 0;
    size_t seg_bytes = 0, sk_bytes = 0;
    int64_t sk_extra = kMaxStreamKWorkers;  // stream-K slots beyond one per (seq, kv head)
    int sk_rows = 0;
    for (int i = 0; i < pl.n; ++i) {
        const Sub& g = pl.sub[i];
        if (g.path == 3 && g.stream_k)
            sk_rows = g.block_q * p->group;
        else if (g.path == 3)
            seg_bytes = ((size_t)a->total_q * d.num_q_heads * g.num_segments * row_bytes(*p) + 255) &
                        ~size_t(255);
    }
    if (no_alloc && sk_rows) {
        // as many worker slots as the scratch holds beside the segmented
        // region, at least one eight-wave worker, at most the usual bound
        const size_t per_slot = (size_t)sk_rows * row_bytes(*p);
        const int64_t fit = seg_bytes < kScratchBytes
                                ? (int64_t)((kScratchBytes - seg_bytes - 255) / per_slot) -
                                      (int64_t)a->num_seqs * d.num_kv_heads
                                : 0;
        sk_extra = std::min<int64_t>(kMaxStreamKWorkers, fit);
        if (sk_extra < kSkMaxWorkerWaves)
            return fail(UA_ERR_WORKSPACE,
                        "batch too large for ua_run_no_alloc: its split partials need more than "
                        "the %zu-byte scratch (use ua_run with a workspace)",
                        kScratchBytes);
    }
    if (sk_rows) sk_bytes = stream_k_bytes(*p, a->num_seqs, sk_rows, sk_extra);
    need = seg_bytes + sk_bytes;
    // the persistent schedule applies to a lone 2D launch of four-wave
    // q-blocks (the LDS-ring kernel takes it; others keep the default grid)
    const Sub& g0 = pl.sub[pl.n - 1];
    const bool persistent = (d.flags & UA_FLAG_PERSISTENT) && pl.n == 1 && g0.path == 2 &&
                            g0.waves == 4 && (int64_t)g0.grid[0] * g0.grid[1] < (int64_t(1) << 30);
    if (persistent) need = std::max(need, kQueueBytes);
    void* ws_base = a->workspace;
    if (no_alloc) {
        if (need > kScratchBytes)
            return fail(UA_ERR_WORKSPACE,
                        "batch too large for ua_run_no_alloc: its split partials need %zu bytes, "
                        "the scratch holds %zu (use ua_run with a workspace)",
                        need, kScratchBytes);
        if (need) {
            ua_status_t sst = scratch_address(&ws_base);
            if (sst != UA_OK) return sst;
        }
    } else if (need && (!a->workspace || a->workspace_bytes < need)) {
        return fail(UA_ERR_WORKSPACE, "split path needs %zu workspace bytes, got %zu", need,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    }
    // a no-alloc class split runs both launches on the caller's stream
    const bool use_side = pl.n == 2 && !no_alloc;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t* tev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(a->timing_events));
    if (use_side) {
        // The two launches share no data until the output: fork the stream-K
        // (HBM-bound) launch onto the side stream so it fills the compute
        // units the wide (MFMA-bound) launch leaves free.
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(UA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        if (!p->side) {
            hipStream_t side = nullptr;
            hipEvent_t fork = nullptr, join = nullptr;
            if ((e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking)) == hipSuccess &&
                (e = hipEventCreateWithFlags(&fork, hipEventDisableTiming)) == hipSuccess)
                e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
            if (e != hipSuccess) {
                if (side) (void)hipStreamDestroy(side);
                if (fork) (void)hipEventDestroy(fork);
                return fail(UA_ERR_HIP, "side stream set-up: %s", hipGetErrorString(e));
            }
            p->side = side;
            p->fork = fork;
            p->join = join;
            p->side_device = dev;
        } else if (p->side_device != dev) {
            return fail(UA_ERR_UNSUPPORTED,
                        "split batches of one problem run on one device (%d, now %d)",
                        p->side_device, dev);
        }
        if ((tev[0] && (e = hipEventRecord(tev[0], s)) != hipSuccess) ||
            (e = hipEventRecord(p->fork, s)) != hipSuccess ||
            (e = hipStreamWaitEvent(p->side, p->fork, 0)) != hipSuccess)
            return fail(UA_ERR_HIP, "fork: %s", hipGetErrorString(e));
    }
    // the wide launch first (it holds the longest workgroups), then stream-K
    for (int i = pl.n - 1; i >= 0; --i) {
        const Sub& g = pl.sub[i];
        UaKernelParams kp = base;
        kp.block_q = g.block_q;
        kp.rows_used = g.block_q * p->group;
        kp.tile_n = g.tile_n;
        kp.tiles_per_seg = g.tiles_per_seg;
        kp.num_segments = g.num_segments;
        kp.class_mode = g.class_mode;
        UaLaunch l{};
        l.path = g.path;
        l.waves = g.waves;
        l.tile_n = g.tile_n;
        l.head_dim = d.head_dim;
        l.q_dtype = d.q_dtype;
        l.kv_fp8 = p->fp8;
        l.stream_k = g.stream_k;
        l.rows16 = g.rows16;
        for (int j = 0; j < 3; ++j) l.grid[j] = g.grid[j];
        l.reduce_rows = a->total_q * d.num_q_heads;
        l.sk_waves_cap = (int)sk_extra;
        if (persistent) {
            l.persistent = 1;
            kp.queue = static_cast<int32_t*>(ws_base);
        }
        if (g.path == 3 && g.stream_k) {
            char* ws = static_cast<char*>(ws_base) + seg_bytes;
            const size_t rows = ((size_t)a->num_seqs * d.num_kv_heads + sk_extra) * kp.rows_used;
            kp.ws_o = ws;
            kp.ws_m = reinterpret_cast<float*>(ws + rows * d.head_dim * o_elem_bytes(*p));
            kp.ws_l = kp.ws_m + rows;
            // enumerate reduce rows by (sequence, head, position) when most
            // tokens belong to the other launch
            const int64_t by_seq = (int64_t)a->num_seqs * d.num_q_heads * kp.small_block_q;
            kp.reduce_by_seq = g.class_mode == 1 && by_seq < l.reduce_rows;
            if (kp.reduce_by_seq) l.reduce_rows = by_seq;
        } else if (g.path == 3) {
            const size_t rows = (size_t)a->total_q * d.num_q_heads * g.num_segments;
            char* ws = static_cast<char*>(ws_base);
            kp.ws_o = ws;
            kp.ws_m = reinterpret_cast<float*>(ws + rows * d.head_dim * o_elem_bytes(*p));
            kp.ws_l = kp.ws_m + rows;
        }
        // timing events of a single launch: [0] before the kernel, [1] after
        // it, [2] after its reduce; a split batch records its own around both
        if (pl.n == 1)
            for (int j = 0; j < 3; ++j) l.events[j] = tev[j];
        else if (!use_side && i == pl.n - 1)
            l.events[0] = tev[0];
        hipStream_t st = i == 0 && use_side ? p->side : s;
        hipError_t e;
        switch (d.head_dim) {
            case 64: e = ua_launch_d64(kp, l, st); break;
            case 128: e = ua_launch_d128(kp, l, st); break;
            default: e = ua_launch_d256(kp, l, st); break;
        }
        if (e != hipSuccess) return fail(UA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    }
    if (pl.n == 2 && !use_side) {
        hipError_t e;
        if ((tev[1] && (e = hipEventRecord(tev[1], s)) != hipSuccess) ||
            (tev[2] && (e = hipEventRecord(tev[2], s)) != hipSuccess))
            return fail(UA_ERR_HIP, "timing events: %s", hipGetErrorString(e));
    } else if (pl.n == 2) {
        hipError_t e;
        if ((e = hipEventRecord(p->join, p->side)) != hipSuccess ||
            (e = hipStreamWaitEvent(s, p->join, 0)) != hipSuccess ||
            (tev[1] && (e = hipEventRecord(tev[1], s)) != hipSuccess) ||
            (tev[2] && (e = hipEventRecord(tev[2], s)) != hipSuccess))
            return fail(UA_ERR_HIP, "join: %s", hipGetErrorString(e));
    }
    return UA_OK;
}

}  // namespace

extern "C" {

ua_status_t ua_run(ua_problem_t p, const ua_run_args_t* a, void* stream) {
    g_error.clear();
    return run_impl(p, a, stream, false);
}

ua_status_t ua_run_no_alloc(ua_problem_t p, const ua_run_args_t* a, void* stream) {
    g_error.clear();
    return run_impl(p, a, stream, true);
}

ua_status_t ua_merge(const ua_merge_args_t* a, void* stream) {
    g_error.clear();
    if (!a) return fail(UA_ERR_INVALID_ARG, "null merge arguments");
    if (a->num_sets < 1 || a->num_sets > UA_MAX_MERGE_SETS)
        return fail(UA_ERR_INVALID_ARG, "num_sets %d outside [1, %d]", a->num_sets,
                    UA_MAX_MERGE_SETS);
    if (a->partial_dtype != UA_PARTIAL_F32 && a->partial_dtype != UA_PARTIAL_BF16)
        return fail(UA_ERR_INVALID_ARG, "partial_dtype %d unknown", a->partial_dtype);
    if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
        return fail(UA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128, 256)", a->head_dim);
    if (a->num_q_heads <= 0 || a->total_q < 0)
        return fail(UA_ERR_INVALID_ARG, "merge shape out of range");
    if (a->o_dtype != UA_DTYPE_BF16 && a->o_dtype != UA_DTYPE_F16)
        return fail(UA_ERR_INVALID_ARG, "o_dtype %d must be bf16 or f16", a->o_dtype);
    if (a->o_stride_tok < (int64_t)a->num_q_heads * a->head_dim || a->o_stride_tok % 8)
        return fail(UA_ERR_INVALID_ARG, "o_stride_tok must be >= H_q * head_dim and a multiple of 8");
    if (a->total_q == 0) return UA_OK;
    if (!a->o || ((uintptr_t)a->o & 15)) return fail(UA_ERR_INVALID_ARG, "o must be 16-byte aligned");
    if ((uintptr_t)a->lse & 3 || (uintptr_t)a->sinks & 3)
        return fail(UA_ERR_INVALID_ARG, "lse and sinks must be 4-byte aligned");
    UaMergeParams mp{};
    for (int i = 0; i < a->num_sets; ++i) {
        if (!a->partial_o[i] || !a->partial_lse[i] || ((uintptr_t)a->partial_o[i] & 15) ||
            ((uintptr_t)a->partial_lse[i] & 3))
            return fail(UA_ERR_INVALID_ARG, "partial set %d: null or misaligned pointer", i);
        mp.o[i] = a->partial_o[i];
        mp.lse[i] = a->partial_lse[i];
    }
    mp.num_sets = a->num_sets;
    mp.part_bf16 = a->partial_dtype == UA_PARTIAL_BF16;
    mp.rows = a->total_q * a->num_q_heads;
    mp.num_q_heads = a->num_q_heads;
    mp.head_dim = a->head_dim;
    mp.out_dtype = a->o_dtype;
    mp.out = a->o;
    mp.out_stride_tok = a->o_stride_tok;
    mp.out_lse = a->lse;
    mp.sinks = a->sinks;
    const hipError_t e = ua_launch_merge(mp, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(UA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
    return UA_OK;
}

}  // extern "C"

// ua_attn_impl.h -- the unified paged attention kernel family for gfx950.
//
// One template serves both strategies of "Unified paged attention on gfx950,
// from the math up":
//   * the 2D path (section 4): one workgroup per (q-block, kv-head) walks the
//     whole key range of its q-block and writes normalised O;
//   * the 3D split-KV path (section 5): one workgroup per (q-block, kv-head,
//     segment) walks a fixed number of KV tiles and writes fp32 (o, m, l)
//     partials, merged by ua_reduce (the associative re-base of section 5).
// Both run the streaming softmax of section 2 in base 2 (tau * log2 e folded
// into one multiplier).
//
// Work layout.  A q-block holds block_q consecutive query positions of one
// sequence times the g query heads of one KV head, packed as rows
// r = pos_local * g + head_local (section 4: the MFMA rows carry
// (position, head) pairs so one K/V tile serves the whole GQA group).  Each
// wave64 owns 32 rows.  Scores are formed transposed, S^T = K Q^T, on the
// 32x32x16 MFMA: lane l then owns query row (l mod 32) and 16 keys of every
// 32-key sub-tile, so the row max/sum are an in-lane reduction plus one
// exchange with lane l^32 (the dense prefill page, section 8: keys on the
// per-lane accumulator registers).  The exponentiated scores of an S^T
// accumulator are, register for register, the B operand of the PV MFMA
// computing O^T = V^T P^T, provided the 16 keys of each PV step are taken in
// the order the accumulator holds them; V^T is read in exactly that order
// from the V tile in LDS with the transposing read ds_read_b64_tr_b16 (the
// FlashInfer transposing-LDS-read change, whose lane map
// out(16g+4a+b)[j] = in(16g+4j+a)[b] this code relies on).
//
// Paged gather.  Key position k of sequence s lives in physical block
// block_table[s][k >> log2 b], slot k & (b - 1); its row for KV head h_k is
// D contiguous elements at ((phys * b + slot) * H_k + h_k) * D, computed in
// 64-bit so pools above 2^31 bytes address correctly (section 7.2).  Each KV
// tile is copied global -> registers -> LDS (rows padded by 8 elements for K
// and 32 for V, which spreads the K fragment reads and the transposing V
// reads over all 64 banks).  Keys at or past S_k are written as zeros and
// masked, so poisoned tail slots and unused blocks never reach O.  The next
// tile's global loads are issued before the current tile is computed.
//
// fp8 e4m3 K/V (section 7.3) are converted to the Q type on the way into LDS
// (exact); k_scale is folded into the score multiplier and v_scale into the
// output scale, so the MFMA path is unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ua.h"
#include "ua_internal.h"

namespace ua {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKPad = 8;   // K LDS row padding (elements)
constexpr int kVPad = 32;  // V LDS row padding (elements)

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T> struct QType;
template <> struct QType<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // two e4m3 codes from the low (hi=false) or high half of `w`
    static __device__ __forceinline__ u32x2 cvt_fp8x4(unsigned w) {
        bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
        bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
        return u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
    }
};
template <> struct QType<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ u32x2 cvt_fp8x4(unsigned w) {
        f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false);
        f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true);
        return u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// tanh(y) = sign(y) (1 - e^{-2|y|}) / (1 + e^{-2|y|}), with e^z via 2^(z log2 e)
__device__ __forceinline__ float tanh_f32(float y) {
    float e = fast_exp2(-2.0f * kLog2e * fabsf(y));
    float t = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    return copysignf(t, y);
}

// Number of indices j in [1, n) with pred(j); every lane of the wave gets it.
template <typename Pred>
__device__ __forceinline__ int wave_count(int n, Pred pred) {
    const int lane = threadIdx.x & 63;
    int cnt = 0;
    for (int base = 1; base < n; base += 64) {
        int j = base + lane;
        bool v = j < n && pred(j);
        cnt += __popcll(__ballot(v));
    }
    return cnt;
}

// Sequence owning q-block slot `slot`: slots of sequence s start at
// cu_q[s] / block_q + s, a strictly increasing sequence.
__device__ __forceinline__ int qblock_seq(const int32_t* cu_q, int n, int block_q, int slot) {
    return wave_count(n, [&](int j) { return cu_q[j] / block_q + j <= slot; });
}

// Sequence owning packed query token `tok`.
__device__ __forceinline__ int token_seq(const int32_t* cu_q, int n, int tok) {
    return wave_count(n + 1, [&](int j) { return cu_q[j] <= tok; });
}

// Key range a q-block needs, and the key interval in which every row of the
// block is unmasked.  Positions p0..p_last are local rows of the sequence.
struct KeyRange {
    int lo, hi;           // keys [lo, hi) are visible to at least one row
    int full_lo, full_hi; // keys in [full_lo, full_hi] are visible to every row
};

__device__ __forceinline__ KeyRange key_range(uint32_t flags, int window, int s_k, int ctx,
                                              int p0, int p_last) {
    KeyRange r;
    const bool causal = flags & UA_FLAG_CAUSAL;
    const bool win = flags & UA_FLAG_WINDOW;
    r.hi = causal ? min(s_k, ctx + p_last + 1) : s_k;
    r.lo = win ? max(0, ctx + p0 - window + 1) : 0;
    r.full_hi = causal ? min(s_k - 1, ctx + p0) : s_k - 1;
    r.full_lo = win ? max(0, ctx + p_last - window + 1) : 0;
    return r;
}

template <int D, int NW, int BN, typename QT, bool FP8, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void ua_attn_kernel(UaKernelParams p) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    constexpr int NT = NW * 64;
    constexpr int KSTR = D + kKPad;
    constexpr int VSTR = D + kVPad;
    constexpr int ESZ = FP8 ? 1 : 2;       // bytes per cached element
    constexpr int EPC = 16 / ESZ;          // cached elements per 16-byte chunk
    constexpr int CPR = D / EPC;           // chunks per key row
    static_assert(NT % CPR == 0, "a thread's chunks must share one column");
    constexpr int RSTEP = NT / CPR;        // key rows covered per pass of the workgroup
    static_assert(BN % RSTEP == 0, "tile rows must divide evenly");
    constexpr int NCH = BN / RSTEP;        // chunks per thread per tile (K, and again V)
    constexpr int NKT = BN / 32;           // 32-key sub-tiles (S^T accumulators)
    constexpr int NDT = D / 32;            // 32-wide d tiles (O^T accumulators)
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shapes");

    __shared__ __attribute__((aligned(16))) unsigned short k_lds[BN * KSTR];
    __shared__ __attribute__((aligned(16))) unsigned short v_lds[BN * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;

    int hk, slot, seg;
    if (SPLIT) {
        slot = blockIdx.x; hk = blockIdx.y; seg = blockIdx.z;
    } else {
        hk = blockIdx.x; slot = blockIdx.y; seg = 0;
    }

    // ---- which sequence and positions this workgroup owns ----
    const int s = qblock_seq(p.cu_q, p.num_seqs, p.block_q, slot);
    const int q_start = p.cu_q[s];
    const int q_len = p.cu_q[s + 1] - q_start;
    const int p0 = (slot - (q_start / p.block_q + s)) * p.block_q;
    if (p0 >= q_len) return;
    // S_k beyond the block table's width would read past the table (a violated
    // precondition); clamp so the gather stays inside it.
    const int s_k = min(p.seq_lens[s], p.bt_stride << p.block_size_log2);
    const int ctx = s_k - q_len;
    const int p_last = min(p0 + p.block_q, q_len) - 1;
    const KeyRange kr = key_range(p.flags, p.window, s_k, ctx, p0, p_last);
    int t_lo = kr.lo / BN;
    int t_hi = (kr.hi + BN - 1) / BN;
    if (SPLIT) {
        const int a = t_lo + seg * p.tiles_per_seg;
        if (a >= t_hi) return;
        t_lo = a;
        t_hi = min(t_hi, a + p.tiles_per_seg);
    }

    // ---- this lane's query row ----
    const int r = wave * 32 + (lane & 31);
    const int pr = r / p.group;
    const int hr = r - pr * p.group;
    const bool row_ok = r < p.rows_used && p0 + pr < q_len;
    const int tok = q_start + p0 + pr;
    const int head = hk * p.group + hr;
    const int q_abs = ctx + p0 + pr;
    const bool causal = p.flags & UA_FLAG_CAUSAL;
    const int kmax_row = causal ? min(q_abs, s_k - 1) : s_k - 1;
    const int kmin_row = (p.flags & UA_FLAG_WINDOW) ? q_abs - p.window + 1 : 0;
    const int r0 = wave * 32;
    const bool wave_active = r0 < p.rows_used && p0 + r0 / p.group < q_len;

    // Q fragments: B operand of S^T = K Q^T, lane holds Q[row][16 kc + 8 half + 0..7]
    v8 qf[D / 16];
    {
        const QT* qp = reinterpret_cast<const QT*>(p.q) + (int64_t)tok * p.q_stride_tok +
                       (int64_t)head * D + 8 * half;
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row_ok) w = *reinterpret_cast<const u32x4*>(qp + 16 * kc);
            qf[kc] = __builtin_bit_cast(v8, w);
        }
    }
    const float slope2 = (p.flags & UA_FLAG_ALIBI) ? p.slopes[head] * kLog2e : 0.0f;

    // ---- running softmax state (log2 units) ----
    float m_run = -INFINITY;
    float l_run = 0.0f;
    if (!SPLIT && (p.flags & UA_FLAG_SINKS)) {
        // the sink is one more softmax column: start from (m, l) = (sink, 1)
        m_run = p.sinks[head] * kLog2e;
        l_run = half == 0 ? 1.0f : 0.0f;
    }
    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};

    // ---- tile loader: chunk column and rows of this thread ----
    const int cc = tid % CPR;
    const int row0 = tid / CPR;
    const int lb = p.block_size_log2;
    const int bmask = (1 << lb) - 1;
    const int32_t* bt = p.block_table + (int64_t)s * p.bt_stride;
    const unsigned char* kbase =
        reinterpret_cast<const unsigned char*>(p.k) + ((int64_t)hk * D + cc * EPC) * ESZ;
    const unsigned char* vbase =
        reinterpret_cast<const unsigned char*>(p.v) + ((int64_t)hk * D + cc * EPC) * ESZ;
    const int64_t slot_bytes = p.kv_slot_stride * ESZ;

    u32x4 kreg[NCH], vreg[NCH];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int key = t * BN + row0 + i * RSTEP;
            u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
            if (key < s_k) {
                const int64_t phys = bt[key >> lb];
                const int64_t off = ((phys << lb) + (key & bmask)) * slot_bytes;
                kw = *reinterpret_cast<const u32x4*>(kbase + off);
                vw = *reinterpret_cast<const u32x4*>(vbase + off);
            }
            kreg[i] = kw;
            vreg[i] = vw;
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int row = row0 + i * RSTEP;
            if (FP8) {
                // 16 codes -> 16 elements of the Q type (two 16-byte LDS writes)
                u32x4 k0, k1, v0, v1;
                u32x2 t;
                t = Q::cvt_fp8x4(kreg[i][0]); k0[0] = t[0]; k0[1] = t[1];
                t = Q::cvt_fp8x4(kreg[i][1]); k0[2] = t[0]; k0[3] = t[1];
                t = Q::cvt_fp8x4(kreg[i][2]); k1[0] = t[0]; k1[1] = t[1];
                t = Q::cvt_fp8x4(kreg[i][3]); k1[2] = t[0]; k1[3] = t[1];
                t = Q::cvt_fp8x4(vreg[i][0]); v0[0] = t[0]; v0[1] = t[1];
                t = Q::cvt_fp8x4(vreg[i][1]); v0[2] = t[0]; v0[3] = t[1];
                t = Q::cvt_fp8x4(vreg[i][2]); v1[0] = t[0]; v1[1] = t[1];
                t = Q::cvt_fp8x4(vreg[i][3]); v1[2] = t[0]; v1[3] = t[1];
                *reinterpret_cast<u32x4*>(&k_lds[row * KSTR + cc * 16]) = k0;
                *reinterpret_cast<u32x4*>(&k_lds[row * KSTR + cc * 16 + 8]) = k1;
                *reinterpret_cast<u32x4*>(&v_lds[row * VSTR + cc * 16]) = v0;
                *reinterpret_cast<u32x4*>(&v_lds[row * VSTR + cc * 16 + 8]) = v1;
            } else {
                *reinterpret_cast<u32x4*>(&k_lds[row * KSTR + cc * 8]) = kreg[i];
                *reinterpret_cast<u32x4*>(&v_lds[row * VSTR + cc * 8]) = vreg[i];
            }
        }
    };

    // per-lane LDS offsets of the K fragment read and the transposing V read
    const int k_frag = (lane & 31) * KSTR + 8 * half;
    const int g16 = lane >> 4;
    const int v_frag = (4 * (g16 >> 1) + ((lane & 15) >> 2)) * VSTR + 16 * (g16 & 1) + 4 * (lane & 3);

    load_tile(t_lo);
    for (int t = t_lo; t < t_hi; ++t) {
        __syncthreads();  // every wave is done with the previous tile
        store_tile();
        __syncthreads();
        if (t + 1 < t_hi) load_tile(t + 1);  // in flight while this tile computes
        if (!wave_active) continue;

        // S^T = K Q^T for BN keys
        f32x16 sacc[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            sacc[kt] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < D / 16; ++kc) {
                v8 a = *reinterpret_cast<const v8*>(&k_lds[k_frag + kt * 32 * KSTR + 16 * kc]);
                sacc[kt] = Q::mma(a, qf[kc], sacc[kt]);
            }
        }

        // scale -> softcap -> ALiBi -> masks (log2 units)
        const int key0 = t * BN;
        const bool need_mask = !(key0 >= kr.full_lo && key0 + BN - 1 <= kr.full_hi);
        float mt = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
                float x = sacc[kt][i];
                float sv = (p.flags & UA_FLAG_SOFTCAP) ? p.softcap_out * tanh_f32(x * p.softcap_in)
                                                       : x * p.qk_scale_log2;
                if (p.flags & UA_FLAG_ALIBI) sv += slope2 * (float)(key - ctx);
                if (need_mask) sv = (key >= kmin_row && key <= kmax_row) ? sv : -INFINITY;
                sacc[kt][i] = sv;
                mt = fmaxf(mt, sv);
            }
        }
        mt = fmaxf(mt, xor32(mt));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;

        // O^T += V^T P^T, 16 keys per step in accumulator order
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc) {
            const int kt = kc >> 1, q8 = (kc & 1) * 8;
            v8 pf;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                QT e = (QT)fast_exp2(sacc[kt][q8 + j] - m_use);
                l_run += (float)e;
                pf[j] = e;
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int off = v_frag + kc * 16 * VSTR + dt * 32;
                i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&v_lds[off]);
                i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&v_lds[off + 8 * VSTR]);
                u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                u32x4 w = {lo2[0], lo2[1], hi2[0], hi2[1]};
                oacc[dt] = Q::mma(__builtin_bit_cast(v8, w), pf, oacc[dt]);
            }
        }
    }

    if (!wave_active) return;
    const float l_tot = l_run + xor32(l_run);
    if (!row_ok) return;
    if (SPLIT) {
        const int64_t rid = ((int64_t)tok * p.num_q_heads + head) * p.num_segments + seg;
        float* wo = p.ws_o + rid * D + 4 * half;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                f32x4 v = {oacc[dt][4 * ig], oacc[dt][4 * ig + 1], oacc[dt][4 * ig + 2],
                           oacc[dt][4 * ig + 3]};
                *reinterpret_cast<f32x4*>(wo + 32 * dt + 8 * ig) = v;
            }
        if (half == 0) {
            p.ws_m[rid] = m_run;
            p.ws_l[rid] = l_tot;
        }
    } else {
        const float inv = l_tot > 0.0f ? p.out_scale / l_tot : 0.0f;
        QT* op = reinterpret_cast<QT*>(p.o) + (int64_t)tok * p.o_stride_tok + (int64_t)head * D +
                 4 * half;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                typename Q::v4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = (QT)(oacc[dt][4 * ig + j] * inv);
                *reinterpret_cast<typename Q::v4*>(op + 32 * dt + 8 * ig) = v;
            }
    }
}

// Log-sum-exp merge of the split partials (section 5: re-base each segment to
// the global max and sum), sinks folded in once, then /L and the cast.  One
// wave per (token, query head); four per workgroup.
template <int D, typename QT>
__global__ __launch_bounds__(256) void ua_reduce_kernel(UaKernelParams p, int64_t n_rows) {
    constexpr int EPL = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int tok = (int)(row / p.num_q_heads);
    const int head = (int)(row - (int64_t)tok * p.num_q_heads);
    const int s = token_seq(p.cu_q, p.num_seqs, tok);
    const int q_start = p.cu_q[s];
    const int q_len = p.cu_q[s + 1] - q_start;
    const int s_k = min(p.seq_lens[s], p.bt_stride << p.block_size_log2);
    const int ctx = s_k - q_len;
    const int p0 = ((tok - q_start) / p.block_q) * p.block_q;
    const int p_last = min(p0 + p.block_q, q_len) - 1;
    const KeyRange kr = key_range(p.flags, p.window, s_k, ctx, p0, p_last);
    const int t_lo = kr.lo / p.tile_n;
    const int t_hi = (kr.hi + p.tile_n - 1) / p.tile_n;
    const int n_live = t_hi > t_lo ? min(p.num_segments,
                                         (t_hi - t_lo + p.tiles_per_seg - 1) / p.tiles_per_seg)
                                   : 0;

    const int64_t base = row * p.num_segments;
    const bool sinks = p.flags & UA_FLAG_SINKS;
    const float sink2 = sinks ? p.sinks[head] * kLog2e : -INFINITY;
    float mx = sink2;
    for (int g = 0; g < n_live; ++g) mx = fmaxf(mx, p.ws_m[base + g]);
    float L = sinks ? fast_exp2(sink2 - mx) : 0.0f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    for (int g = 0; g < n_live; ++g) {
        const float mg = p.ws_m[base + g];
        if (mg == -INFINITY) continue;
        const float w = fast_exp2(mg - mx);
        L += p.ws_l[base + g] * w;
        const float* src = p.ws_o + (base + g) * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += w * src[e];
    }
    const float inv = L > 0.0f ? p.out_scale / L : 0.0f;
    QT* dst = reinterpret_cast<QT*>(p.o) + (int64_t)tok * p.o_stride_tok + (int64_t)head * D +
              lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = (QT)(acc[e] * inv);
}

template <int D, int NW, int BN, typename QT, bool FP8>
hipError_t launch_attn(const UaKernelParams& p, const UaLaunch& l, hipStream_t st) {
    dim3 grid(l.grid[0], l.grid[1], l.grid[2]);
    hipError_t e = hipSuccess;
    if (l.events[0] && (e = hipEventRecord(l.events[0], st)) != hipSuccess) return e;
    if (l.path == 3) {
        hipLaunchKernelGGL((ua_attn_kernel<D, NW, BN, QT, FP8, true>), grid, dim3(NW * 64), 0, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (l.events[1] && (e = hipEventRecord(l.events[1], st)) != hipSuccess) return e;
        const unsigned nb = (unsigned)((l.reduce_rows + 3) / 4);
        hipLaunchKernelGGL((ua_reduce_kernel<D, QT>), dim3(nb), dim3(256), 0, st, p, l.reduce_rows);
    } else {
        hipLaunchKernelGGL((ua_attn_kernel<D, NW, BN, QT, FP8, false>), grid, dim3(NW * 64), 0, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (l.events[1] && (e = hipEventRecord(l.events[1], st)) != hipSuccess) return e;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (l.events[2] && (e = hipEventRecord(l.events[2], st)) != hipSuccess) return e;
    return hipSuccess;
}

template <int D, typename QT, bool FP8>
hipError_t launch_geometry(const UaKernelParams& p, const UaLaunch& l, hipStream_t st) {
    constexpr int BN4 = D >= 256 ? 32 : 64;
    if (l.waves == 1 && l.tile_n == 32) return launch_attn<D, 1, 32, QT, FP8>(p, l, st);
    if (l.waves == 4 && l.tile_n == BN4) return launch_attn<D, 4, BN4, QT, FP8>(p, l, st);
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_head_dim(const UaKernelParams& p, const UaLaunch& l, hipStream_t st) {
    if (l.q_dtype == UA_DTYPE_BF16)
        return l.kv_fp8 ? launch_geometry<D, __bf16, true>(p, l, st)
                        : launch_geometry<D, __bf16, false>(p, l, st);
    return l.kv_fp8 ? launch_geometry<D, _Float16, true>(p, l, st)
                    : launch_geometry<D, _Float16, false>(p, l, st);
}

}  // namespace ua

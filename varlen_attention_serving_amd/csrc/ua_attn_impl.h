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
// 64-bit so pools above 2^31 bytes address correctly (section 7.2).  The dense
// layout of section 8 is the same with one block of 2^30 rows per sequence,
// based at its cu_seqlens_k row.  Tiles of 16-bit K/V in four-wave workgroups
// (d <= 128) are copied global -> LDS directly into a three-stage ring with
// 16-byte chunks permuted against bank conflicts; every other tile goes global
// -> registers -> LDS rows padded by 8 (K) and 32 (V) elements, which spread the
// K fragment reads and the transposing V reads over all 64 banks.  Keys at or
// past S_k read slot S_k - 1 (finite data) and are masked, so poisoned tail
// slots and unused blocks never reach O.
//
// Decode-shaped batches run as stream-K workers over the flattened (sequence,
// kv-head group, tile) space with a log-sum-exp reduce; at d = 256 their
// q-blocks are 16 rows on the 16x16x32 MFMA.
//
// fp8 e4m3 K/V (section 7.3) are converted to the Q type on the way into LDS
// (exact); k_scale is folded into the score multiplier and v_scale into the
// output scale, so the MFMA path is unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

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
constexpr float kLn2 = 0.6931471805599453f;

// natural-log LSE of a row from its reference max m (log2 units) and the
// denominator l relative to it; -inf when nothing was visible
__device__ __forceinline__ float row_lse(float m, float l) {
    return l > 0.0f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}
constexpr int kKPad = 8;   // K LDS row padding (elements)
constexpr int kVPad = 32;  // V LDS row padding (elements)
// Register budget: at least two resident waves per SIMD, so one wave's MFMAs
// overlap another's softmax arithmetic and memory waits.
#ifndef UA_MIN_WAVES_PER_SIMD
#define UA_MIN_WAVES_PER_SIMD 2
#endif
constexpr int kMinWavesPerSimd = UA_MIN_WAVES_PER_SIMD;
// four-wave workgroups with d <= 128: three resident per CU (168 VGPRs per lane)
constexpr int kMinWavesPerSimdWide = 3;
// d = 256 holds a 32-row O accumulator of 128 registers: one wave per SIMD for
// the single-wave geometry, two for the four-wave one
constexpr int min_waves_per_simd(int d, int waves) {
    return d > 128 ? (waves >= 4 ? 2 : 1) : (waves >= 4 ? kMinWavesPerSimdWide : kMinWavesPerSimd);
}
// 16-bit K/V tiles of four-wave workgroups are copied straight into an LDS
// ring (0 keeps every tile on the register-staged path)
#ifndef UA_LDS_RING
#define UA_LDS_RING 1
#endif
// largest head dim built with the ring
#ifndef UA_LDS_RING_MAX_D
#define UA_LDS_RING_MAX_D 256
#endif
// kv heads a stream-K worker workgroup serves together (a power of two; the
// launch takes the largest that divides H_k)
#ifndef UA_SK_HEADS
#define UA_SK_HEADS 8
#endif
constexpr int kSkMaxHeads = UA_SK_HEADS;
static_assert(kSkMaxHeads <= kSkMaxWorkerWaves, "the workspace bound counts at most 8 waves a worker");

// Score transforms a kernel is compiled for: none (the scale folds into the
// exponent), softcap and/or ALiBi (tested per tile from the flags), those plus
// the QQ-bias, whose per-element loads cost registers the others need not pay
// for, or softcap alone (its last step folds into the exponent).
constexpr int kXfNone = 0;
constexpr int kXfScore = 1;
constexpr int kXfQQ = 2;
constexpr int kXfCap = 3;
// log2-unit slack before the running reference max is moved (p <= 2^8)
constexpr float kLazyRescale = 8.0f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T> struct QType;
template <> struct QType<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // c + a + b in fp32 (one dot2 against (1, 1))
    static __device__ __forceinline__ float sum2(__bf16 a, __bf16 b, float c) {
        const bf16x2 x = {a, b}, one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(x, one, c, false);
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
    static __device__ __forceinline__ f32x4 mma16(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float sum2(_Float16 a, _Float16 b, float c) {
        const f16x2 x = {a, b}, one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(x, one, c, false);
    }
    static __device__ __forceinline__ u32x2 cvt_fp8x4(unsigned w) {
        f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false);
        f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true);
        return u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// the value of lane l ^ 32 (one v_permlane32_swap, no LDS round trip)
__device__ __forceinline__ float xor32(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// max(x of lane l, x of lane l ^ 32) in every lane.  One swap of x with itself
// leaves x's low half in both halves of one result and its high half in both
// halves of the other; the max is taken in assembly so no canonicalisation of
// the swapped values is added (scores are finite or -inf, never NaN).
__device__ __forceinline__ float max_halves(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(r[0]), "v"(r[1]));
    return m;
}

// min(x of lane l, x of lane l ^ 32) in every lane, as max_halves (values
// are finite or +inf, never NaN).
__device__ __forceinline__ float min_halves(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    float m;
    asm("v_min_f32 %0, %1, %2" : "=v"(m) : "v"(r[0]), "v"(r[1]));
    return m;
}

// The running max a row starts from when no sink logit sets it: a finite
// stand-in for -inf, so exponents 2^(x c - m) need no guard.  Every finite
// score exceeds it by more than the lazy-rescale slack, so the first tile with
// a visible key moves the max (and re-bases O and l, both still 0); a row that
// never sees a key keeps l = 0 and gets O = 0 and LSE = -inf.
constexpr float kMaxStart = -1.0e30f;

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

// Split-KV pieces of a q-block with n live tiles: min(segments, ceil(n /
// tiles)) runs of near-equal length, so runs hold at most `tiles` tiles while
// the grid has segments to spare and ceil(n / segments) when it has not.
// Piece i covers tiles [i n / pieces, (i + 1) n / pieces) of the range.
__device__ __forceinline__ int seg_pieces(int n, int segments, int tiles) {
    return n > 0 ? min(segments, (n + tiles - 1) / tiles) : 0;
}


// ---------------------------------------------------------------------------
// K/V tile gather: global -> registers -> padded LDS
// ---------------------------------------------------------------------------

template <int D, int NW, int BN, bool FP8>
struct TileGeom {
    static constexpr int NT = NW * 64;
    static constexpr int KSTR = D + kKPad;
    static constexpr int VSTR = D + kVPad;
    static constexpr int ESZ = FP8 ? 1 : 2;   // bytes per cached element
    static constexpr int EPC = 16 / ESZ;      // cached elements per 16-byte chunk
    static constexpr int CPR = D / EPC;       // chunks per key row
    static_assert(NT % CPR == 0, "a thread's chunks must share one column");
    static constexpr int RSTEP = NT / CPR;    // key rows covered per pass of the workgroup
    static_assert(BN % RSTEP == 0, "tile rows must divide evenly");
    static constexpr int NCH = BN / RSTEP;    // chunks per thread per tile (K, and again V)
    static constexpr int NKT = BN / 32;       // 32-key sub-tiles (S^T accumulators)
    static constexpr int NDT = D / 32;        // 32-wide d tiles (O^T accumulators)
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shapes");
};

// Each thread owns one 16-byte column chunk of NCH key rows of a tile.  Block
// ids are fetched one tile ahead of the K/V loads that use them, so a tile's
// gather never waits on a block-table read.  Loads are branch-free: a key past
// S_k reads the sequence's last valid slot (finite data; its score is masked,
// so its p is exactly 0).  The loaded words go to their registers untouched:
// any use at load time (a select, say) would make each load wait for its data
// and serialise the tile's gather.
// One K/V load of type T: plain, or with the non-temporal hint (NT) for
// gathers that read each byte once (the decode engines): a load-only probe of
// the decode batch's paged reads moves 6.8 TB/s with the hint against 6.0
// without it.
template <bool NT, typename T>
__device__ __forceinline__ T load_kv(const unsigned char* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
    return *reinterpret_cast<const T*>(p);
}

template <int D, int NW, int BN, typename QT, bool FP8, bool NT = false>
struct KvLoader {
    typedef TileGeom<D, NW, BN, FP8> G;
    u32x4 kreg[G::NCH], vreg[G::NCH];
    int phys[G::NCH];
    int cc, row0;

    __device__ __forceinline__ void init(int tid) {
        cc = tid % G::CPR;
        row0 = tid / G::CPR;
    }
    __device__ __forceinline__ void ids(const int32_t* bt_row, int t, int s_k, int lb) {
#pragma unroll
        for (int i = 0; i < G::NCH; ++i) {
            const int key = min(t * BN + row0 + i * G::RSTEP, s_k - 1);
            phys[i] = bt_row[key >> lb];
        }
    }
    // base_k / base_v point at element (slot 0, head, 0) of the caches (bytes)
    __device__ __forceinline__ void load(const unsigned char* base_k, const unsigned char* base_v,
                                         int t, int s_k, int lb, int64_t slot_bytes) {
        const int bmask = (1 << lb) - 1;
        const int col = cc * G::EPC * G::ESZ;
#pragma unroll
        for (int i = 0; i < G::NCH; ++i) {
            const int key = t * BN + row0 + i * G::RSTEP;
            const int kc = min(key, s_k - 1);
            const int64_t off = (((int64_t)phys[i] << lb) + (kc & bmask)) * slot_bytes + col;
            kreg[i] = load_kv<NT, u32x4>(base_k + off);
            vreg[i] = load_kv<NT, u32x4>(base_v + off);
        }
    }
    __device__ __forceinline__ void store(unsigned short* k_lds, unsigned short* v_lds) const {
        typedef QType<QT> Q;
#pragma unroll
        for (int i = 0; i < G::NCH; ++i) {
            const int row = row0 + i * G::RSTEP;
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
                *reinterpret_cast<u32x4*>(&k_lds[row * G::KSTR + cc * 16]) = k0;
                *reinterpret_cast<u32x4*>(&k_lds[row * G::KSTR + cc * 16 + 8]) = k1;
                *reinterpret_cast<u32x4*>(&v_lds[row * G::VSTR + cc * 16]) = v0;
                *reinterpret_cast<u32x4*>(&v_lds[row * G::VSTR + cc * 16 + 8]) = v1;
            } else {
                *reinterpret_cast<u32x4*>(&k_lds[row * G::KSTR + cc * 8]) = kreg[i];
                *reinterpret_cast<u32x4*>(&v_lds[row * G::VSTR + cc * 8]) = vreg[i];
            }
        }
    }
};

// ---------------------------------------------------------------------------
// K/V tiles copied global -> LDS directly (16-bit K/V, four-wave workgroups)
// ---------------------------------------------------------------------------
//
// gfx950's global_load_lds_dwordx4 writes each lane's 16 bytes to LDS at
// M0 + 16 lane without passing through registers, so tiles can be in flight
// while earlier ones are computed: a ring of STAGES tile buffers, with tile
// t + STAGES - 1 issued while tile t is computed.  One copy fills 1 KB of
// LDS, so the tile image is unpadded (rows of 2D bytes) and bank conflicts
// are avoided by permuting the 16-byte chunks of a row instead: chunk c of
// key row r sits in slot c ^ swz(r), and the lane that fills a slot fetches
// the chunk that belongs there.  The copies are issued from inline assembly
// so that the compiler, which would wait for every outstanding copy before
// any LDS read, leaves the waiting to the explicit counter waits: before
// computing a tile the loop waits until that tile's copies have landed
// (later tiles' copies may stay in flight), then meets the barrier.

// Per-lane LDS offsets (elements) of the K fragment read and of the
// transposing V read; kx / vx are the lane's chunk swizzles (swizzled tiles).
struct Frag {
    int k, v, kx, vx;
};

template <int D>
struct LdsGeom {
    static constexpr int BN = 32;                   // keys per tile
    static constexpr int RB = 2 * D;                // bytes per key row
    static constexpr int CPR = RB / 16;             // 16-byte chunks per row
    static constexpr int ROWS_PER_OP = 1024 / RB;   // key rows one wave-wide copy fills
    static constexpr int OPS = 2 * BN * RB / 1024;  // copies per tile (K image, then V)
    static constexpr int GROUPS = OPS / 8;          // row groups per wave (a K and a V copy each)
    static constexpr int OPS_W = 2 * GROUPS;        // copies per wave per tile
    // three stages (two tiles in flight) where three fit beside two other
    // workgroups' rings; at d = 256 a stage is 32 KB and two keep two
    // workgroups resident per CU
    static constexpr int STAGES = D > 128 ? 2 : 3;
    static constexpr int TILE_ELEMS = BN * D;       // one K or V image (16-bit elements)
    static constexpr uint32_t STAGE_BYTES = 4 * TILE_ELEMS;
    static_assert(OPS % 8 == 0, "four waves copy whole row groups");
};

// Chunk permutations: the K fragment read of one chunk from 16 consecutive
// rows, and the transposing V read of 64 contiguous bytes from 4 consecutive
// rows, each touch distinct banks.
template <int D>
__host__ __device__ constexpr int swz_k(int r) {
    return D == 64 ? (r >> 1) & 7 : r & 15;
}
template <int D>
__host__ __device__ constexpr int swz_v(int r) {
    return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
}

// The padded-tile lane offsets of padded_frag, moved to the swizzled image:
// k / v are the row bases plus the swizzle-independent part of the column.
template <int D>
__host__ __device__ inline Frag swizzled_frag(int lane) {
    const int g16 = lane >> 4;
    const int m = lane & 31;
    const int half = lane >> 5;
    const int fk = swz_k<D>(m);
    const int rv = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    Frag f;
    f.k = m * D + 8 * ((half ^ fk) & 1);
    f.kx = fk & ~1;
    f.v = rv * D + 8 * (2 * (g16 & 1) + ((lane & 3) >> 1)) + 4 * (lane & 1);
    f.vx = swz_v<D>(rv) >> 2;
    return f;
}

// Where a lane's copies of one tile come from: in row group g of wave w the
// K copy fills image bytes [1024 (w + 4 g), +1024) and the V copy the same
// range of the V image, i.e. key rows (w + 4 g) ROWS_PER_OP + lane / CPR.
template <int D>
struct LdsCopy {
    typedef LdsGeom<D> L;
    // Groups g and g + KD have the same chunk permutation (their rows differ
    // by a multiple of the permutations' periods), so a lane keeps KD K
    // offsets and one V offset.
    static constexpr int KD = D > 128 ? 2 : 1;
    int wave, lane;
    // byte offsets from the group's first key row (that row's slot in the
    // caches is the copy's scalar base when every key of the tile is valid)
    uint32_t krel_[KD], vrel_;

    // key row of group g and the byte offsets of its fetched K / V chunks
    __host__ __device__ int row(int g) const { return (wave + 4 * g) * L::ROWS_PER_OP + lane / L::CPR; }
    __host__ __device__ int koff(int g) const { return 16 * ((lane % L::CPR) ^ swz_k<D>(row(g))); }
    __host__ __device__ int voff(int g) const { return 16 * ((lane % L::CPR) ^ swz_v<D>(row(g))); }
    __host__ __device__ uint32_t krel(int g) const { return krel_[g % KD]; }
    __host__ __device__ uint32_t vrel(int) const { return vrel_; }

    __host__ __device__ void init(int wave_, int lane_, uint32_t slot_bytes) {
        wave = wave_;
        lane = lane_;
        for (int g = 0; g < KD; ++g)
            krel_[g] = (uint32_t)(lane / L::CPR) * slot_bytes + (uint32_t)koff(g);
        vrel_ = (uint32_t)(lane / L::CPR) * slot_bytes + (uint32_t)voff(0);
    }
};
static_assert(swz_k<256>(0) == swz_k<256>(4 * 2 * LdsGeom<256>::ROWS_PER_OP) &&
                  swz_k<128>(0) == swz_k<128>(4 * LdsGeom<128>::ROWS_PER_OP) &&
                  swz_k<64>(0) == swz_k<64>(4 * LdsGeom<64>::ROWS_PER_OP),
              "the K permutation repeats every KD groups");

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// one wave-wide 16-byte-per-lane copy global -> LDS at m0 + 16 lane
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
                 : "memory", "m0");
}
// the same copy from a scalar base plus a 32-bit lane offset
__device__ __forceinline__ void lds_copy16_s(uint32_t lane_off, const void* base, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base),
                 "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// wait until at most N of this wave's copies are outstanding and its LDS
// reads are done, then meet the other waves
template <int N>
__device__ __forceinline__ void lds_tile_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt = 0 only
constexpr int kWaitVmcntZero = 0x0F70;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

// Block ids of a tile's row groups for wave w: rows of one group lie in one
// block (block size >= ROWS_PER_OP), so each is one scalar load.  Keys past
// S_k are fetched from slot S_k - 1, which lies in the same group's block.
template <int D>
__device__ __forceinline__ void lds_tile_ids(const_i32_ptr bt_row, int t, int s_k, int lb, int wave,
                                             int (&id)[LdsGeom<D>::GROUPS]) {
    typedef LdsGeom<D> L;
#pragma unroll
    for (int g = 0; g < L::GROUPS; ++g) {
        const int key = min(t * L::BN + (wave + 4 * g) * L::ROWS_PER_OP, s_k - 1);
        id[g] = bt_row[__builtin_amdgcn_readfirstlane(key >> lb)];
    }
}

// Issue tile t's copies into the stage at LDS byte address m0_stage.  A tile
// whose keys are all below S_k addresses each copy as the scalar slot of its
// group's first row plus the lane's fixed offset; the last, partial tile
// clamps every lane's key to S_k - 1 in 64-bit lane addresses.
template <int D>
__device__ __forceinline__ void lds_tile_issue(const LdsCopy<D>& cp, const unsigned char* base_k,
                                               const unsigned char* base_v, int t, int s_k, int lb,
                                               uint64_t slot_bytes,
                                               const int (&id)[LdsGeom<D>::GROUPS],
                                               uint32_t m0_stage, int wave) {
    typedef LdsGeom<D> L;
    const int bmask = (1 << lb) - 1;
    if ((t + 1) * L::BN <= s_k) {
#pragma unroll
        for (int g = 0; g < L::GROUPS; ++g) {
            const int first = t * L::BN + (wave + 4 * g) * L::ROWS_PER_OP;
            const uint64_t slot = ((uint64_t)(uint32_t)id[g] << lb) + (uint32_t)(first & bmask);
            const uint64_t off = slot * slot_bytes;
            const uint32_t m0 = m0_stage + (uint32_t)(wave + 4 * g) * 1024u;
            lds_copy16_s(cp.krel(g), base_k + off, m0);
            lds_copy16_s(cp.vrel(g), base_v + off, m0 + (uint32_t)(2 * L::TILE_ELEMS));
        }
        return;
    }
#pragma unroll
    for (int g = 0; g < L::GROUPS; ++g) {
        const int key = min(t * L::BN + cp.row(g), s_k - 1);
        const uint64_t slot = ((uint64_t)(uint32_t)id[g] << lb) + (uint32_t)(key & bmask);
        const uint64_t off = slot * slot_bytes;
        const uint32_t m0 = m0_stage + (uint32_t)(wave + 4 * g) * 1024u;
        lds_copy16(base_k + off + cp.koff(g), m0);
        lds_copy16(base_v + off + cp.voff(g), m0 + (uint32_t)(2 * L::TILE_ELEMS));
    }
}

// ---------------------------------------------------------------------------
// One wave's 32 query rows against one KV tile in LDS
// ---------------------------------------------------------------------------

// Per-lane facts of the lane's query row.
struct RowCtx {
    int ctx;     // S_k - q_len of the row's sequence
    int kmin;    // first visible key
    int kmax;    // last visible key
    float slope2;  // ALiBi slope in log2 units (0 when off)
    int qloc;    // the row's local query index (clamped into the section)
    int qlast;   // q_len - 1 of the row's sequence
};

// QQ-bias of (row, key) in log2 units for a key of the query section; the
// column is clamped so keys past S_k (masked) read inside the matrix
__device__ __forceinline__ float qq_bias2(const UaKernelParams& p, const RowCtx& rc, int key) {
    const int kl = min(max(key - rc.ctx, 0), rc.qlast);
    const float b = p.qq_bias[(int64_t)rc.qloc * p.qq_stride + kl] * kLog2e;
    return key >= rc.ctx ? b : 0.0f;
}

// Scale -> softcap -> ALiBi -> QQ-bias on one lane's scores s[v][i] (key
// key_of(v, i)), to log2 units.  Each step is one pass under one uniform
// test of the problem's flags, so a tile pays only for the steps the problem
// asks for and the passes stay branch-free inside.
template <int NV, int W, typename V, typename KeyOf>
__device__ __forceinline__ void transform_scores(const UaKernelParams& p, V (&s)[NV], KeyOf key_of,
                                                 const RowCtx& rc, bool qq) {
    if (p.flags & UA_FLAG_SOFTCAP) {
        // c tanh(y) = c - 2c / (1 + e^{2y}), with e^{2y} = 2^{x * softcap_in2}:
        // saturates to +-c for large |y| (1 / inf = 0) without a clamp
        const float c2 = 2.0f * p.softcap_out;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int i = 0; i < W; ++i)
                s[v][i] = p.softcap_out -
                          c2 * __builtin_amdgcn_rcpf(1.0f + fast_exp2(s[v][i] * p.softcap_in2));
    } else {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int i = 0; i < W; ++i) s[v][i] *= p.qk_scale_log2;
    }
    if (p.flags & UA_FLAG_ALIBI) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int i = 0; i < W; ++i)
                s[v][i] = __builtin_fmaf(rc.slope2, (float)(key_of(v, i) - rc.ctx), s[v][i]);
    }
    if (qq) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int i = 0; i < W; ++i) s[v][i] += qq_bias2(p, rc, key_of(v, i));
    }
}

// Rows of one q-block: pos_local = r / g, head_local = r % g.
struct RowInfo {
    bool ok;
    int tok, head;
    RowCtx rc;
};

__device__ __forceinline__ RowInfo row_info(const UaKernelParams& p, int r, int hk, int q_start,
                                            int q_len, int s_k, int p0) {
    RowInfo ri;
    const int pr = r / p.group;
    const int hr = r - pr * p.group;
    ri.ok = r < p.rows_used && p0 + pr < q_len;
    ri.tok = q_start + p0 + pr;
    ri.head = hk * p.group + hr;
    const int q_abs = s_k - q_len + p0 + pr;
    ri.rc.ctx = s_k - q_len;
    ri.rc.kmax = (p.flags & UA_FLAG_CAUSAL) ? min(q_abs, s_k - 1) : s_k - 1;
    ri.rc.kmin = (p.flags & UA_FLAG_WINDOW) ? q_abs - p.window + 1 : 0;
    ri.rc.slope2 = (p.flags & UA_FLAG_ALIBI) ? p.slopes[ri.head] * kLog2e : 0.0f;
    ri.rc.qloc = min(p0 + pr, q_len - 1);
    ri.rc.qlast = q_len - 1;
    return ri;
}

// Q fragments: B operand of S^T = K Q^T; lane holds Q[row][16 kc + 8 half + 0..7].
template <int D, typename QT>
__device__ __forceinline__ void load_q(const UaKernelParams& p, const RowInfo& ri, int half,
                                       typename QType<QT>::v8 (&qf)[D / 16]) {
    typedef typename QType<QT>::v8 v8;
    const QT* qp = reinterpret_cast<const QT*>(p.q) + (int64_t)ri.tok * p.q_stride_tok +
                   (int64_t)ri.head * D + 8 * half;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ri.ok) w = *reinterpret_cast<const u32x4*>(qp + 16 * kc);
        qf[kc] = __builtin_bit_cast(v8, w);
    }
}

// S^T = K Q^T for one tile: sacc[kt] holds keys 32 kt .. 32 kt + 31 of the
// tile against the lane's query row (raw scores).
template <int D, int BN, typename QT, bool SWZ>
__device__ __forceinline__ void qk_tile(const unsigned short* __restrict__ k_lds,
                                        const typename QType<QT>::v8 (&qf)[D / 16], const Frag& fr,
                                        f32x16 (&sacc)[BN / 32]) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    constexpr int KSTR = D + kKPad;
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt) {
        v8 a[D / 16];
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
            // kx < 16, so chunks 16 and up keep their high bit: eight lane
            // bases serve every kc, the rest is an immediate offset
            const int off = SWZ ? fr.k + kt * 32 * D + 128 * (kc >> 3) + 8 * ((2 * (kc & 7)) ^ fr.kx)
                                : fr.k + kt * 32 * KSTR + 16 * kc;
            a[kc] = *reinterpret_cast<const v8*>(&k_lds[off]);
        }
        sacc[kt] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) sacc[kt] = Q::mma(a[kc], qf[kc], sacc[kt]);
        if constexpr (SWZ) {
            // On the ring, keep AH fragment reads ahead of the MFMA chain
            // (then one read per MFMA): the default schedule kept fewer, and
            // each MFMA waited on its read.  AH = 4 at d <= 128 (about
            // +0.6-3% on prefill); at d = 256, where the O and Q registers
            // leave less room, AH = 2 (d = 256 prefill 0.731 -> 0.708 ms;
            // AH = 4 spilled 12 registers).
            constexpr int AH = D <= 128 ? 4 : 2;
            __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);  // DS reads
#pragma unroll
            for (int i = 0; i < D / 16 - AH; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
        }
    }
}

// Scores of one tile to log2 units with masks applied, and the running max
// (O and l are re-based here when the reference max moves).
template <int D, int BN, int XF>
__device__ __forceinline__ void softmax_max(const UaKernelParams& p, f32x16 (&sacc)[BN / 32],
                                            f32x16 (&oacc)[D / 32], float& m_run, float& l_run,
                                            int key0, bool need_mask, const RowCtx& rc, int half) {
    constexpr int NKT = BN / 32;
    constexpr int NDT = D / 32;
    // Scores to log2 units.  Without softcap/ALiBi the multiplier c > 0 keeps
    // the order, so the max is taken on raw scores and the scale is folded
    // into the exponent as one FMA: 2^(x c - m).
    const float c = XF != 0 ? 1.0f : p.qk_scale_log2;
    float mt = -INFINITY;
    if constexpr (XF == kXfCap) {
        // Softcap alone: the score in log2 units is C tanh(y) = C - 2C r with
        // r = 1 / (1 + e^{2y}) and C = c log2(e), a decreasing function of r.
        // Keep r in place of the score (masked keys: r = +inf), take the tile
        // max as C - 2C min(r) (-inf when every key is masked), and let
        // softmax_exp form the exponent (C - m) - 2C r in one FMA.
        float rt = INFINITY;
        // the masked and the plain tile in separate loops under one uniform
        // test, so plain tiles carry no per-key compares
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool keep = (key >= rc.kmin) & (key <= rc.kmax);
                    const float r =
                        __builtin_amdgcn_rcpf(1.0f + fast_exp2(sacc[kt][i] * p.softcap_in2));
                    sacc[kt][i] = keep ? r : INFINITY;
                    rt = fminf(rt, sacc[kt][i]);
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sacc[kt][i] = __builtin_amdgcn_rcpf(1.0f + fast_exp2(sacc[kt][i] * p.softcap_in2));
                    rt = fminf(rt, sacc[kt][i]);
                }
        }
        mt = __builtin_fmaf(-2.0f * p.softcap_out, min_halves(rt), p.softcap_out);
    } else {
        if (XF != 0) {
            // QQ-bias only on tiles that reach the query section (ctx is the same
            // for every row of a q-block, so the test is uniform)
            const bool qq = XF == kXfQQ && key0 + BN > rc.ctx;
            transform_scores<NKT, 16>(
                p, sacc,
                [&](int kt, int i) { return key0 + 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3); }, rc,
                qq);
        }
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool keep = (key >= rc.kmin) & (key <= rc.kmax);
                    const float sv = keep ? sacc[kt][i] : -INFINITY;
                    sacc[kt][i] = sv;
                    mt = fmaxf(mt, sv);
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kt][i]);
        }
        mt = max_halves(mt) * c;
    }
    // Lazy reference max: exponents are taken against m_run, which moves only
    // when some row's tile max exceeds it by more than kLazyRescale (log2
    // units).  Softmax is shift-invariant, so o and l stay exact relative to
    // m_run; between moves p <= 2^kLazyRescale.  A move re-bases O and l by
    // 2^(m_old - m_new).
    if (__ballot(mt > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mt);
        const float m_base = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_base);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
    }
}

// p = 2^(x c - m) in the Q type, and the running denominator.
template <int BN, typename QT, int XF>
__device__ __forceinline__ void softmax_exp(const UaKernelParams& p, const f32x16 (&sacc)[BN / 32],
                                            float m_run, float& l_run,
                                            typename QType<QT>::v8 (&pf)[BN / 16]) {
    typedef QType<QT> Q;
    // softcap alone: sacc holds r, the exponent is (C - m) - 2C r (softmax_max)
    const float c = XF == kXfCap ? -2.0f * p.softcap_out : XF != 0 ? 1.0f : p.qk_scale_log2;
    const float b = XF == kXfCap ? p.softcap_out - m_run : -m_run;
#pragma unroll
    for (int kc = 0; kc < BN / 16; ++kc) {
        const int kt = kc >> 1, q8 = (kc & 1) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            pf[kc][j] = (QT)fast_exp2(__builtin_fmaf(sacc[kt][q8 + j], c, b));
        // the denominator sums the same rounded p the PV product uses
#pragma unroll
        for (int j = 0; j < 8; j += 2) l_run = Q::sum2(pf[kc][j], pf[kc][j + 1], l_run);
    }
}

// O^T += V^T P^T for one tile, V^T read transposed from LDS.
template <int D, int BN, typename QT, bool SWZ>
__device__ __forceinline__ void pv_tile(const unsigned short* __restrict__ v_lds,
                                        const typename QType<QT>::v8 (&pf)[BN / 16],
                                        f32x16 (&oacc)[D / 32], const Frag& fr) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    constexpr int VSTR = D + kVPad;
#pragma unroll
    for (int kc = 0; kc < BN / 16; ++kc) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            // vx < 4: four lane bases, the rest immediate (as for K)
            const int off = SWZ ? fr.v + kc * 16 * D + 128 * (dt >> 2) + 32 * ((dt & 3) ^ fr.vx)
                                : fr.v + kc * 16 * VSTR + dt * 32;
            constexpr int HI = 8 * (SWZ ? D : VSTR);
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&v_lds[off]);
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&v_lds[off + HI]);
            u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            u32x4 w = {lo2[0], lo2[1], hi2[0], hi2[1]};
            oacc[dt] = Q::mma(__builtin_bit_cast(v8, w), pf[kc], oacc[dt]);
        }
    }
}

// One tile: scores, scale -> softcap -> ALiBi -> QQ-bias -> masks (log2 units), the
// online-softmax update, then O^T += V^T P^T.  key0 is the tile's first key
// position.  XF = kXfNone compiles the plain scale for problems without
// softcap and ALiBi.
template <int D, int BN, typename QT, int XF, bool SWZ = false>
__device__ __forceinline__ void attend_tile(const UaKernelParams& p,
                                            const unsigned short* __restrict__ k_lds,
                                            const unsigned short* __restrict__ v_lds,
                                            const typename QType<QT>::v8 (&qf)[D / 16],
                                            f32x16 (&oacc)[D / 32], float& m_run, float& l_run,
                                            int key0, bool need_mask, const RowCtx& rc,
                                            const Frag& fr, int half) {
    f32x16 sacc[BN / 32];
    typename QType<QT>::v8 pf[BN / 16];
    // On the ring, a wave runs its scores, their transforms and the tile max
    // at raised priority, so the SIMD's arbiter favours the wave whose next
    // work is the QK MFMA chain and its dependent vector work over waves in
    // their exponentials and PV product (measured: the softcap batch
    // chunked_prefill_mix 0.297 -> 0.275 ms, plain prefill unchanged; ending
    // the raise after the QK chain or after the exponentials was neutral or
    // 2.5% slower, and the register-staged kernel gained nothing from it).
    if (SWZ) __builtin_amdgcn_s_setprio(1);
    qk_tile<D, BN, QT, SWZ>(k_lds, qf, fr, sacc);
    softmax_max<D, BN, XF>(p, sacc, oacc, m_run, l_run, key0, need_mask, rc, half);
    if (SWZ) __builtin_amdgcn_s_setprio(0);
    softmax_exp<BN, QT, XF>(p, sacc, m_run, l_run, pf);
    pv_tile<D, BN, QT, SWZ>(v_lds, pf, oacc, fr);
}

// Lane offsets into padded tiles: the K fragment read takes row lane % 32,
// elements 8 (lane / 32) + 16 kc; the transposing V read takes, per 16-lane
// group g, key row 4 (g / 2) + (lane % 16) / 4 and elements
// 16 (g % 2) + 4 (lane % 4) of each 32-wide d tile.
template <int D>
__device__ __forceinline__ Frag padded_frag(int lane) {
    const int g16 = lane >> 4;
    Frag f;
    f.k = (lane & 31) * (D + kKPad) + 8 * (lane >> 5);
    f.v = (4 * (g16 >> 1) + ((lane & 15) >> 2)) * (D + kVPad) + 16 * (g16 & 1) + 4 * (lane & 3);
    f.kx = f.vx = 0;
    return f;
}

// Four consecutive fp32 values of a partial row, stored as fp32 or (bf16)
// rounded to nearest even; `base` is the row's first element.
__device__ __forceinline__ void store4(void* base, int64_t elem, f32x4 v, bool bf16) {
    if (bf16) {
        const bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(base) + elem) = b;
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(base) + elem) = v;
    }
}

// Un-normalised partial of the lane's row: o (fp32, or bf16 with ws_bf16),
// the running max m (log2 units) and the denominator l, at workspace row `rid`.
template <int D>
__device__ __forceinline__ void write_partial(const UaKernelParams& p, int64_t rid, int half,
                                              const f32x16 (&oacc)[D / 32], float m, float l) {
    const int64_t e0 = rid * D + 4 * half;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
            f32x4 v = {oacc[dt][4 * ig], oacc[dt][4 * ig + 1], oacc[dt][4 * ig + 2],
                       oacc[dt][4 * ig + 3]};
            store4(p.ws_o, e0 + 32 * dt + 8 * ig, v, p.ws_bf16);
        }
    if (half == 0) {
        p.ws_m[rid] = m;
        p.ws_l[rid] = l;
    }
}

// ---------------------------------------------------------------------------
// 2D query-tile kernel and the segmented 3D split-KV kernel
// ---------------------------------------------------------------------------

// The one block id of the dense K/V layout: a whole sequence is one block
// (block_size_log2 = 30) whose rows start at the sequence's row offset.
// (global memory, like the block table, so the table read stays a global load)
static __device__ int32_t kDenseBlockId[1] = {0};

// S_k of sequence s.  Paged: clamped to the block table's width, since a
// longer length would read past the table (a violated precondition).  Dense:
// the difference of cu_seqlens_k.
__device__ __forceinline__ int seq_keys(const UaKernelParams& p, int s) {
    if (p.cu_k) return p.cu_k[s + 1] - p.cu_k[s];
    return min(p.seq_lens[s], p.bt_stride << p.block_size_log2);
}
// Byte offset of sequence s's first K/V row (dense layout; 0 when paged).
__device__ __forceinline__ int64_t seq_kv_bytes(const UaKernelParams& p, int s, int64_t slot_bytes) {
    return p.cu_k ? (int64_t)p.cu_k[s] * slot_bytes : 0;
}
// Block-table row of sequence s (the single zero id when dense).
__device__ __forceinline__ const int32_t* table_row(const UaKernelParams& p, int s) {
    return p.block_table ? p.block_table + (int64_t)s * p.bt_stride : kDenseBlockId;
}

// The q-block (and, split, the run of its KV tiles) a workgroup owns; false
// when it owns nothing.
struct QBlockWork {
    int s, q_start, q_len, p0, s_k, t_lo, t_hi;
    KeyRange kr;
    bool whole;  // the workgroup covers the q-block's whole key range (writes O)
};

template <int BN, bool SPLIT>
__device__ __forceinline__ bool qblock_work(const UaKernelParams& p, int slot, int seg,
                                            QBlockWork& w) {
    w.s = qblock_seq(p.cu_q, p.num_seqs, p.block_q, slot);
    w.q_start = p.cu_q[w.s];
    w.q_len = p.cu_q[w.s + 1] - w.q_start;
    // A sequence's q-blocks are dispatched last block first: under a causal
    // mask the late blocks carry the most keys, so the long workgroups start
    // early and the short ones fill the tail.
    const int local = slot - (w.q_start / p.block_q + w.s);
    const int blocks = (w.q_len + p.block_q - 1) / p.block_q;
    if (local >= blocks) return false;
    w.p0 = (blocks - 1 - local) * p.block_q;
    if (p.class_mode == 2 && w.q_len <= p.small_block_q) return false;  // the decode kernel's rows
    w.s_k = seq_keys(p, w.s);
    const int p_last = min(w.p0 + p.block_q, w.q_len) - 1;
    w.kr = key_range(p.flags, p.window, w.s_k, w.s_k - w.q_len, w.p0, p_last);
    w.t_lo = w.kr.lo / BN;
    w.t_hi = (w.kr.hi + BN - 1) / BN;
    w.whole = true;
    if (SPLIT) {
        // this segment's run of the q-block's tiles; the reduce derives the
        // same piece count (and leaves a one-piece q-block's rows, written
        // here as O, alone)
        const int n = w.t_hi - w.t_lo;
        const int pieces = seg_pieces(n, p.num_segments, p.tiles_per_seg);
        if (seg >= pieces) return false;
        w.whole = pieces == 1;
        w.t_hi = w.t_lo + (int)((int64_t)(seg + 1) * n / pieces);
        w.t_lo = w.t_lo + (int)((int64_t)seg * n / pieces);
    }
    return true;
}

// A wave's rows after the last tile: normalised O, or the split partial.
// A split workgroup that covers its q-block's whole key range (`whole`)
// finishes like the 2D path; its sink, which a split run leaves to the
// reduce, joins here as one more softmax term: (m, l) <- (max(m, sink),
// l 2^(m - m') + 2^(sink - m')), O scaled by 2^(m - m').
template <int D, typename QT, bool SPLIT>
__device__ __forceinline__ void finish_rows(const UaKernelParams& p, const RowInfo& ri, int half,
                                            int seg, bool whole, const f32x16 (&oacc)[D / 32],
                                            float m_run, float l_run) {
    typedef QType<QT> Q;
    float l_tot = l_run + xor32(l_run);
    if (!ri.ok) return;
    if (SPLIT && !whole) {
        const int64_t rid = ((int64_t)ri.tok * p.num_q_heads + ri.head) * p.num_segments + seg;
        write_partial<D>(p, rid, half, oacc, m_run, l_tot);
        return;
    }
    float alpha = 1.0f;
    if (SPLIT && (p.flags & UA_FLAG_SINKS)) {
        const float s2 = p.sinks[ri.head] * kLog2e;
        const float m2 = fmaxf(m_run, s2);
        alpha = fast_exp2(m_run - m2);
        l_tot = l_tot * alpha + fast_exp2(s2 - m2);
        m_run = m2;
    }
    if (p.part_o) {
        // the row's merge-ready state over this call's keys: o / l and its LSE
        const int64_t row = (int64_t)ri.tok * p.num_q_heads + ri.head;
        if (half == 0) p.part_lse[row] = row_lse(m_run, l_tot);
        const float inv = l_tot > 0.0f ? p.out_scale * alpha / l_tot : 0.0f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                f32x4 v = {oacc[dt][4 * ig] * inv, oacc[dt][4 * ig + 1] * inv,
                           oacc[dt][4 * ig + 2] * inv, oacc[dt][4 * ig + 3] * inv};
                store4(p.part_o, row * D + 4 * half + 32 * dt + 8 * ig, v, p.part_bf16);
            }
    } else {
        if (p.lse && half == 0) p.lse[(int64_t)ri.tok * p.num_q_heads + ri.head] = row_lse(m_run, l_tot);
        const float inv = l_tot > 0.0f ? p.out_scale * alpha / l_tot : 0.0f;
        QT* op = reinterpret_cast<QT*>(p.o) + (int64_t)ri.tok * p.o_stride_tok +
                 (int64_t)ri.head * D + 4 * half;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                typename Q::v4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = (QT)(oacc[dt][4 * ig + j] * inv);
                *reinterpret_cast<typename Q::v4*>(op + 32 * dt + 8 * ig) = v;
            }
    }
}

template <int D, int NW, int BN, typename QT, bool FP8, bool SPLIT, int XF>
__global__ __launch_bounds__(NW * 64, min_waves_per_simd(D, NW)) void ua_attn_kernel(UaKernelParams p) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    typedef TileGeom<D, NW, BN, FP8> G;

    __shared__ __attribute__((aligned(16))) unsigned short k_lds[BN * G::KSTR];
    __shared__ __attribute__((aligned(16))) unsigned short v_lds[BN * G::VSTR];

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

    QBlockWork qb;
    if (!qblock_work<BN, SPLIT>(p, slot, seg, qb)) return;
    const int s = qb.s, s_k = qb.s_k;
    const KeyRange kr = qb.kr;
    const int t_lo = qb.t_lo, t_hi = qb.t_hi;

    const RowInfo ri = row_info(p, wave * 32 + (lane & 31), hk, qb.q_start, qb.q_len, s_k, qb.p0);
    const int r0 = wave * 32;
    const bool wave_active = r0 < p.rows_used && qb.p0 + r0 / p.group < qb.q_len;
    v8 qf[D / 16];
    load_q<D, QT>(p, ri, half, qf);

    // ---- running softmax state (log2 units) ----
    float m_run = kMaxStart;
    float l_run = 0.0f;
    if (!SPLIT && (p.flags & UA_FLAG_SINKS)) {
        // the sink is one more softmax column: start from (m, l) = (sink, 1)
        m_run = p.sinks[ri.head] * kLog2e;
        l_run = half == 0 ? 1.0f : 0.0f;
    }
    f32x16 oacc[G::NDT];
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) oacc[dt] = f32x16{};

    const int lb = p.block_size_log2;
    const int32_t* bt = table_row(p, s);
    const int64_t slot_bytes = p.kv_slot_stride * G::ESZ;
    const int64_t kv0 = seq_kv_bytes(p, s, slot_bytes) + (int64_t)hk * D * G::ESZ;
    const unsigned char* base_k = reinterpret_cast<const unsigned char*>(p.k) + kv0;
    const unsigned char* base_v = reinterpret_cast<const unsigned char*>(p.v) + kv0;
    KvLoader<D, NW, BN, QT, FP8> ld;
    ld.init(tid);
    const Frag fr = padded_frag<D>(lane);

    // The next tile's loads are issued before this tile's compute, except for
    // four-wave workgroups at d = 256: there the O and Q registers leave no
    // room to hold a tile in flight, and the spills it forced (each reload
    // waiting for every load in flight) cost more than the overlap gave
    // (measured: d = 256 prefill 482 -> 618 TFLOP/s without it).  Those
    // workgroups load each tile after the barrier and rely on the other
    // workgroup on the CU to cover the latency.
    constexpr bool PF = !(D == 256 && NW == 4);
    ld.ids(bt, t_lo, s_k, lb);
    if (PF) {
        ld.load(base_k, base_v, t_lo, s_k, lb, slot_bytes);
        if (t_lo + 1 < t_hi) ld.ids(bt, t_lo + 1, s_k, lb);
    }
    for (int t = t_lo; t < t_hi; ++t) {
        if (!PF) {
            ld.load(base_k, base_v, t, s_k, lb, slot_bytes);
            if (t + 1 < t_hi) ld.ids(bt, t + 1, s_k, lb);
        }
        __syncthreads();  // every wave is done with the previous tile
        ld.store(k_lds, v_lds);
        __syncthreads();
        if (PF && t + 1 < t_hi) {
            ld.load(base_k, base_v, t + 1, s_k, lb, slot_bytes);  // in flight during compute
            if (t + 2 < t_hi) ld.ids(bt, t + 2, s_k, lb);
        }
        if (!wave_active) continue;
        const int key0 = t * BN;
        const bool need_mask = !(key0 >= kr.full_lo && key0 + BN - 1 <= kr.full_hi);
        attend_tile<D, BN, QT, XF>(p, k_lds, v_lds, qf, oacc, m_run, l_run, key0, need_mask, ri.rc,
                               fr, half);
    }

    if (!wave_active) return;
    finish_rows<D, QT, SPLIT>(p, ri, half, seg, qb.whole, oacc, m_run, l_run);
}

// The same q-block work for 16-bit K/V with four waves and block sizes of at
// least ROWS_PER_OP keys: tiles arrive through the LDS ring instead of
// registers (STAGES - 1 tiles in flight, one barrier per tile).
template <int D, typename QT, bool SPLIT, int XF>
__device__ __forceinline__ void lds_qblock(const UaKernelParams& p, unsigned short* tiles, int hk,
                                           int slot, int seg) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    typedef LdsGeom<D> L;
    constexpr int BN = L::BN;
    constexpr int S = L::STAGES;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;

    QBlockWork qb;
    if (!qblock_work<BN, SPLIT>(p, slot, seg, qb)) return;
    const int s_k = qb.s_k;
    const KeyRange kr = qb.kr;
    const int t_lo = qb.t_lo, t_hi = qb.t_hi;

    const RowInfo ri = row_info(p, wave * 32 + (lane & 31), hk, qb.q_start, qb.q_len, s_k, qb.p0);
    const bool wave_active = wave * 32 < p.rows_used && qb.p0 + wave * 32 / p.group < qb.q_len;
    v8 qf[D / 16];
    load_q<D, QT>(p, ri, half, qf);

    float m_run = kMaxStart;
    float l_run = 0.0f;
    if (!SPLIT && (p.flags & UA_FLAG_SINKS)) {
        m_run = p.sinks[ri.head] * kLog2e;
        l_run = half == 0 ? 1.0f : 0.0f;
    }
    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};

    const int lb = p.block_size_log2;
    const const_i32_ptr bt = (const_i32_ptr)table_row(p, qb.s);
    const uint64_t slot_bytes = (uint64_t)p.kv_slot_stride * 2;
    const int64_t kv0 = seq_kv_bytes(p, qb.s, (int64_t)slot_bytes) + (int64_t)hk * D * 2;
    const unsigned char* base_k = reinterpret_cast<const unsigned char*>(p.k) + kv0;
    const unsigned char* base_v = reinterpret_cast<const unsigned char*>(p.v) + kv0;
    LdsCopy<D> cp;
    cp.init(wave, lane, (uint32_t)slot_bytes);
    const Frag fr = swizzled_frag<D>(lane);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(tiles));

    // The compiler cannot see the copies, so let it retire its own loads (Q,
    // row facts) here: a wait it placed inside the loop would also wait for
    // the copies in flight.
    __builtin_amdgcn_s_waitcnt(kWaitVmcntZero);
    // prologue: tiles t_lo, t_lo + 1 into stages 0, 1
    int id[L::GROUPS];
#pragma unroll
    for (int i = 0; i < S - 1; ++i) {
        if (t_lo + i < t_hi) {
            lds_tile_ids<D>(bt, t_lo + i, s_k, lb, wave, id);
            lds_tile_issue<D>(cp, base_k, base_v, t_lo + i, s_k, lb, slot_bytes, id,
                              lds0 + (uint32_t)i * L::STAGE_BYTES, wave);
        }
    }
    // ids of the next tile to issue, fetched one iteration ahead of use
    if (t_lo + S - 1 < t_hi) lds_tile_ids<D>(bt, t_lo + S - 1, s_k, lb, wave, id);

    // Tile t sits in stage (t - t_lo) % 3.  The loop is unrolled by the ring
    // size so every stage address is a constant of the instructions.
    auto step = [&](auto stage_c, int t) {
        constexpr int ST = decltype(stage_c)::value;
        // tile t has landed (with three stages tile t + 1 may still be in
        // flight) and every wave is done with tile t - 1, whose stage is
        // refilled next
        if (t + 1 < t_hi)
            lds_tile_barrier<(S - 2) * L::OPS_W>();
        else
            lds_tile_barrier<0>();
        const int t_next = t + S - 1;
        if (t_next < t_hi) {
            lds_tile_issue<D>(cp, base_k, base_v, t_next, s_k, lb, slot_bytes, id,
                              lds0 + (uint32_t)((ST + S - 1) % S) * L::STAGE_BYTES, wave);
            if (t_next + 1 < t_hi) lds_tile_ids<D>(bt, t_next + 1, s_k, lb, wave, id);
        }
        if (wave_active) {
            const unsigned short* k_lds = tiles + ST * 2 * L::TILE_ELEMS;
            const int key0 = t * BN;
            const bool need_mask = !(key0 >= kr.full_lo && key0 + BN - 1 <= kr.full_hi);
            attend_tile<D, BN, QT, XF, true>(p, k_lds, k_lds + L::TILE_ELEMS, qf, oacc, m_run,
                                                l_run, key0, need_mask, ri.rc, fr, half);
        }
    };
    if constexpr (S == 3) {
        for (int t = t_lo; t < t_hi; t += 3) {
            step(std::integral_constant<int, 0>{}, t);
            if (t + 1 < t_hi) step(std::integral_constant<int, 1>{}, t + 1);
            if (t + 2 < t_hi) step(std::integral_constant<int, 2>{}, t + 2);
        }
    } else {
        static_assert(S == 2, "the loop is unrolled for two or three stages");
        for (int t = t_lo; t < t_hi; t += 2) {
            step(std::integral_constant<int, 0>{}, t);
            if (t + 1 < t_hi) step(std::integral_constant<int, 1>{}, t + 1);
        }
    }

    if (!wave_active) return;
    finish_rows<D, QT, SPLIT>(p, ri, half, seg, qb.whole, oacc, m_run, l_run);
}

template <int D, typename QT, bool SPLIT, int XF>
__global__ __launch_bounds__(256, min_waves_per_simd(D, 4)) void ua_attn_lds_kernel(UaKernelParams p) {
    typedef LdsGeom<D> L;
    __shared__ __attribute__((aligned(1024))) unsigned short tiles[L::STAGES * 2 * L::TILE_ELEMS];
    if (SPLIT)
        lds_qblock<D, QT, SPLIT, XF>(p, tiles, blockIdx.y, blockIdx.x, blockIdx.z);
    else
        lds_qblock<D, QT, SPLIT, XF>(p, tiles, blockIdx.x, blockIdx.y, 0);
}

// Persistent schedule of the same 2D work (UA_FLAG_PERSISTENT): one
// workgroup per resident slot, each taking q-blocks until none are left.
// The work items keep the default grid's order, item = slot * H_k + h_k (a
// sequence's heaviest q-block first), and are dealt from kPersistQueues
// queues by item mod kPersistQueues.  Workgroup j draws from queue
// j mod kPersistQueues: the dispatcher deals a launch's workgroups to the
// XCDs round robin, so with H_k = 8 each XCD serves one kv head, whose K/V
// is then read through that XCD's L2, as in the default grid, while the queue
// balances the ragged q-blocks dynamically (the item order is fixed, so
// every q-block is computed exactly as in the default grid).
template <int D, typename QT, int XF>
__global__ __launch_bounds__(256, min_waves_per_simd(D, 4)) void ua_attn_persist_kernel(UaKernelParams p) {
    typedef LdsGeom<D> L;
    __shared__ __attribute__((aligned(1024))) unsigned short tiles[L::STAGES * 2 * L::TILE_ELEMS];
    __shared__ int next_item;
    const int q = blockIdx.x % kPersistQueues;
    const int64_t n_items = (int64_t)p.num_kv_heads * p.persist_slots;
    for (;;) {
        if (threadIdx.x == 0) next_item = q + kPersistQueues * atomicAdd(&p.queue[q], 1);
        __syncthreads();
        const int64_t item = __builtin_amdgcn_readfirstlane(next_item);  // uniform: scalar copies
        // every wave has the item (and is done with the previous one's LDS)
        // before the next draw overwrites it
        __syncthreads();
        if (item >= n_items) break;
        lds_qblock<D, QT, false, XF>(p, tiles, (int)(item % p.num_kv_heads),
                                     (int)(item / p.num_kv_heads), 0);
    }
}

// Clears the persistent schedule's queue counters (a kernel rather than a
// memset, so a caller may capture the run in a graph).
template <int N>
__global__ __launch_bounds__(64) void ua_queue_reset_kernel(int32_t* queue) {
    if (threadIdx.x < N) queue[threadIdx.x] = 0;
}

// ---------------------------------------------------------------------------
// Stream-K split for decode-shaped batches
// ---------------------------------------------------------------------------
//
// When every sequence's query rows fit one q-block (decode and short chunks),
// the units of KV work are the (sequence, kv-head) pairs, taken in the order
// p = s * H_k + h.  Flatten their KV tiles into one index space of T tiles and
// give worker j of W the contiguous range [floor(jT/W), floor((j+1)T/W)).  All
// workers then carry equal work whatever the length mix, and each pays the
// metadata prelude once.  A worker writes one partial per pair it touches, at
// slot p + j: along a worker's range p and j never decrease together, so p + j
// is unique per (pair, worker).  The reduce finds a pair's workers from its
// first and last flattened tile.

// Per-sequence facts of that geometry, one sequence per lane.
struct SeqLane {
    int q_start, q_len, s_k, t_lo, n;  // n = KV tiles of the sequence's q-block
};

template <int BN>
__device__ __forceinline__ SeqLane seq_lane(const UaKernelParams& p, int s) {
    SeqLane r = {0, 0, 0, 0, 0};
    if (s >= p.num_seqs) return r;
    r.q_start = p.cu_q[s];
    r.q_len = p.cu_q[s + 1] - r.q_start;
    r.s_k = seq_keys(p, s);
    if (r.q_len <= 0) return r;
    if (p.class_mode == 1 && r.q_len > p.small_block_q) return r;  // another kernel's rows
    const KeyRange kr = key_range(p.flags, p.window, r.s_k, r.s_k - r.q_len, 0, r.q_len - 1);
    r.t_lo = kr.lo / BN;
    r.n = max(0, (kr.hi + BN - 1) / BN - r.t_lo);
    return r;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// The stream-K order flattens (sequence, kv-head group, tile).  A worker is a
// workgroup of sk_heads waves, one per kv head of a group, that walk the same
// tiles together, so the heads of one cached key row are fetched at the same
// time (one contiguous run of H_k * d elements per key instead of H_k
// separate d-element pieces at different times).
__device__ __forceinline__ int sk_groups(const UaKernelParams& p) {
    return p.num_kv_heads / p.sk_heads;
}

// Total tiles T and, for flattened tile x, the sequence holding it and that
// sequence's first flattened tile.  Every lane of the wave gets the results.
// The scans below take sequences 256 at a time: the facts of four 64-lane
// chunks are loaded together (one round of loads instead of four), then
// scanned chunk by chunk.
constexpr int kSkScanChunks = 4;

// tile counts of sequences base + 64 c + lane, c < kSkScanChunks
template <int BN>
__device__ __forceinline__ void sk_counts(const UaKernelParams& p, int base,
                                          int (&n)[kSkScanChunks]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < kSkScanChunks; ++c) n[c] = seq_lane<BN>(p, base + 64 * c + lane).n;
}

template <int BN>
__device__ __forceinline__ int sk_total(const UaKernelParams& p) {
    int total = 0;
    for (int base = 0; base < p.num_seqs; base += 64 * kSkScanChunks) {
        int n[kSkScanChunks];
        sk_counts<BN>(p, base, n);
#pragma unroll
        for (int c = 0; c < kSkScanChunks; ++c)
            total += readlane(wave_incl_scan(n[c] * sk_groups(p)), 63);
    }
    return total;
}

template <int BN>
__device__ __forceinline__ int sk_locate(const UaKernelParams& p, int64_t x, int* seq_first) {
    int carry = 0;
    for (int base = 0; base < p.num_seqs; base += 64 * kSkScanChunks) {
        int n[kSkScanChunks];
        sk_counts<BN>(p, base, n);
#pragma unroll
        for (int c = 0; c < kSkScanChunks; ++c) {
            const int v = n[c] * sk_groups(p);
            const int incl = wave_incl_scan(v);
            const uint64_t hit = __ballot((int64_t)carry + incl > x);
            if (hit) {
                const int l = __builtin_ctzll(hit);
                *seq_first = carry + readlane(incl - v, l);
                return base + 64 * c + l;
            }
            carry += readlane(incl, 63);
        }
    }
    *seq_first = carry;
    return p.num_seqs;
}

// worker j of W owns flattened tiles [floor(jT/W), floor((j+1)T/W)); the
// worker holding tile x is ceil((x+1) W / T) - 1
__host__ __device__ inline int sk_worker_of(int64_t x, int64_t T, int64_t W) {
    return (int)(((x + 1) * W + T - 1) / T - 1);
}

// A position in the flattened tile space with the facts of its pair.
struct SkPos {
    int s, h, t, t_lo, t_end, q_start, q_len, s_k;
    int kv_row;  // the sequence's first K/V row (dense layout; 0 when paged)
};

template <int BN>
__device__ __forceinline__ SkPos sk_pos(const UaKernelParams& p, int s, int h, int t) {
    const SeqLane q = seq_lane<BN>(p, s);  // uniform s: every lane reads the same facts
    SkPos r;
    r.s = s; r.h = h; r.t = t;
    r.t_lo = q.t_lo; r.t_end = q.t_lo + q.n;
    r.q_start = q.q_start; r.q_len = q.q_len; r.s_k = q.s_k;
    r.kv_row = p.cu_k ? p.cu_k[s] : 0;
    return r;
}

// the next tile of the flattened order (callers never step past their range)
template <int BN>
__device__ __forceinline__ SkPos sk_next(const UaKernelParams& p, const SkPos& c) {
    SkPos r = c;
    if (c.t + 1 < c.t_end) {
        r.t = c.t + 1;
        return r;
    }
    if (c.h + 1 < sk_groups(p)) {
        r.h = c.h + 1;
        r.t = c.t_lo;
        return r;
    }
    int s = c.s + 1;
    SeqLane q = seq_lane<BN>(p, s);
    while (q.n == 0 && s + 1 < p.num_seqs) q = seq_lane<BN>(p, ++s);
    r.s = s; r.h = 0; r.t = q.t_lo; r.t_lo = q.t_lo; r.t_end = q.t_lo + q.n;
    r.q_start = q.q_start; r.q_len = q.q_len; r.s_k = q.s_k;
    r.kv_row = p.cu_k ? p.cu_k[s] : 0;
    return r;
}

// first flattened tile of sequence s, its tile count and the total T
template <int BN>
__device__ __forceinline__ int sk_seq_prefix(const UaKernelParams& p, int s, int* n_s, int* total) {
    int carry = 0, first = 0, n = 0;
    for (int base = 0; base < p.num_seqs; base += 64 * kSkScanChunks) {
        int nc[kSkScanChunks];
        sk_counts<BN>(p, base, nc);
#pragma unroll
        for (int c = 0; c < kSkScanChunks; ++c) {
            const int b = base + 64 * c;
            const int v = nc[c] * sk_groups(p);
            const int incl = wave_incl_scan(v);
            if (s >= b && s < b + 64) {
                first = carry + readlane(incl - v, s - b);
                n = readlane(nc[c], s - b);
            }
            carry += readlane(incl, 63);
        }
    }
    *n_s = n;
    *total = carry;
    return first;
}

// LDS of one stream-K wave (its own padded K and V tiles), in 16-bit elements
template <int D, int BN, bool FP8>
constexpr int sk_wave_lds_elems() {
    return BN * (TileGeom<D, 1, BN, FP8>::KSTR + TileGeom<D, 1, BN, FP8>::VSTR);
}

// heads (waves) of one stream-K worker: as many as fit on a CU at the
// kernel's waves per SIMD, so a worker never lowers the register budget
template <int D>
constexpr int sk_max_heads() {
    return kSkMaxHeads < 4 * min_waves_per_simd(D, 1) ? kSkMaxHeads : 4 * min_waves_per_simd(D, 1);
}

template <int D, int BN, typename QT, bool FP8, int XF>
__global__ __launch_bounds__(64 * sk_max_heads<D>(), min_waves_per_simd(D, 1)) void ua_decode_sk_kernel(
    UaKernelParams p) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    typedef TileGeom<D, 1, BN, FP8> G;
    static_assert(BN == kSkTile, "the reduce locates stream-K partials with this tile size");

    // A decode launch of its own raises its waves' issue priority (measured
    // on one box, interleaved: decode_batch 0.1863 -> 0.1846 ms, decode_large
    // 0.7136 -> 0.7068 ms).  Beside a concurrent wide launch (a class split)
    // it does not: the wide workgroups, starved, hold their compute units
    // longer, and the decode workers queued behind them start later (the
    // 128-row fp8 mix without its window 0.285 -> 0.337 ms, against 0.1192
    // -> 0.1179 ms with it).
    if (p.class_mode != 1) __builtin_amdgcn_s_setprio(2);
    // sk_heads waves, each with its own tiles (dynamic LDS sized at launch)
    extern __shared__ __attribute__((aligned(16))) unsigned short sk_lds[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned short* k_lds = sk_lds + wave * sk_wave_lds_elems<D, BN, FP8>();
    unsigned short* v_lds = k_lds + BN * G::KSTR;

    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int64_t W = gridDim.x;
    const int64_t j = blockIdx.x;
    const int T = sk_total<BN>(p);
    const int64_t A = j * T / W;
    const int64_t B = (j + 1) * T / W;
    if (A >= B) return;

    int seq_first;
    const int s0 = sk_locate<BN>(p, A, &seq_first);
    SkPos pc = sk_pos<BN>(p, s0, 0, 0);
    {
        const int n = pc.t_end - pc.t_lo;
        const int off = (int)(A - seq_first);
        pc.h = off / n;
        pc.t = pc.t_lo + (off - pc.h * n);
    }
    SkPos p1 = pc, p2 = pc;
    if (A + 1 < B) p1 = sk_next<BN>(p, pc);
    if (A + 2 < B) p2 = sk_next<BN>(p, p1);

    const int lb = p.block_size_log2;
    const int64_t slot_bytes = p.kv_slot_stride * G::ESZ;
    const unsigned char* kc = reinterpret_cast<const unsigned char*>(p.k);
    const unsigned char* vc = reinterpret_cast<const unsigned char*>(p.v);
    auto bt_row = [&](const SkPos& q) { return table_row(p, q.s); };
    // this wave's kv head within the position's head group
    auto head = [&](const SkPos& q) { return q.h * p.sk_heads + wave; };
    auto hoff = [&](const SkPos& q) {
        return q.kv_row * slot_bytes + (int64_t)head(q) * D * G::ESZ;
    };

    KvLoader<D, 1, BN, QT, FP8, true> ld;  // each key row is read once: non-temporal
    ld.init(lane);
    const Frag fr = padded_frag<D>(lane);
    ld.ids(bt_row(pc), pc.t, pc.s_k, lb);
    ld.load(kc + hoff(pc), vc + hoff(pc), pc.t, pc.s_k, lb, slot_bytes);
    if (A + 1 < B) ld.ids(bt_row(p1), p1.t, p1.s_k, lb);

    // state of the pair being accumulated
    RowInfo ri;
    KeyRange kr;
    v8 qf[D / 16];
    f32x16 oacc[G::NDT];
    float m_run, l_run;
    auto begin_pair = [&](const SkPos& q) {
        ri = row_info(p, lane & 31, head(q), q.q_start, q.q_len, q.s_k, 0);
        kr = key_range(p.flags, p.window, q.s_k, q.s_k - q.q_len, 0, q.q_len - 1);
        load_q<D, QT>(p, ri, half, qf);
        m_run = kMaxStart;
        l_run = 0.0f;
#pragma unroll
        for (int dt = 0; dt < G::NDT; ++dt) oacc[dt] = f32x16{};
    };
    begin_pair(pc);

    // Each wave owns its tiles and its LDS operations run in order, so the
    // waves need no barrier for correctness.  With 16-bit K/V they still meet
    // once per tile: in step, the worker's waves (its kv heads) read each key
    // row's heads together, contiguous in the cache (measured: decode_batch
    // 0.216 -> 0.223 ms without a barrier).  With fp8 K/V, where each wave
    // also converts its tile, they run free (fp8 decode at d = 128: 0.144 ->
    // 0.129 ms).
    constexpr bool WG_SYNC = !FP8;
    for (int64_t x = A; x < B; ++x) {
        if (WG_SYNC) __syncthreads(); else asm volatile("" ::: "memory");
        ld.store(k_lds, v_lds);
        asm volatile("" ::: "memory");
        if (x + 1 < B) {
            ld.load(kc + hoff(p1), vc + hoff(p1), p1.t, p1.s_k, lb, slot_bytes);
            if (x + 2 < B) ld.ids(bt_row(p2), p2.t, p2.s_k, lb);
        }
        const int key0 = pc.t * BN;
        const bool need_mask = !(key0 >= kr.full_lo && key0 + BN - 1 <= kr.full_hi);
        attend_tile<D, BN, QT, XF>(p, k_lds, v_lds, qf, oacc, m_run, l_run, key0, need_mask, ri.rc,
                               fr, half);
        if (x + 1 == B || pc.t + 1 == pc.t_end) {
            const float l_tot = l_run + xor32(l_run);
            if (ri.ok) {
                // unit (sequence, head group) u and worker j give the slot
                // (u + j) * sk_heads + wave: unique, since u and j never
                // decrease together along the flattened order
                const int64_t unit = (int64_t)pc.s * sk_groups(p) + pc.h;
                const int64_t slot = (unit + j) * p.sk_heads + wave;
                write_partial<D>(p, slot * p.rows_used + (lane & 31), half, oacc, m_run, l_tot);
            }
            if (x + 1 < B) begin_pair(p1);
        }
        pc = p1;
        p1 = p2;
        if (x + 3 < B) p2 = sk_next<BN>(p, p2);
    }
}

// ---------------------------------------------------------------------------
// Stream-K decode with 16-row q-blocks (16x16x32 MFMA)
// ---------------------------------------------------------------------------
//
// Decode rows of one (sequence, kv-head) pair are g (times the few positions
// of a short chunk), so a 32-row tile wastes most of its accumulators.  This
// engine packs 16 rows per wave on v_mfma_f32_16x16x32:
//   * S^T = K Q^T per 16-key block kb: lane l holds keys 16 kb + 4 (l / 16) + i
//     (i < 4) of query row l % 16;
//   * K is loaded from the cache straight into the A operand (lane l: key
//     16 kb + l % 16, elements 32 kc + 8 (l / 16) .. + 7), so K needs no LDS;
//   * P feeds O^T += V^T P^T with the 32 keys of a tile taken in the order
//     pi(8 g + j) = 4 g + j (j < 4), 16 + 4 g + j - 4 (j >= 4): exactly the
//     eight scores lane l holds, so P needs no data movement;
//   * V^T is read in that key order from a padded V tile in LDS by two
//     transposing reads per 16 d: lane 16 G + 4 J + A reads row 4 G + J (and
//     16 + 4 G + J), elements 16 dblk + 4 A .. + 3;
//   * a row's max and sum combine the four lanes l % 16 + 16 {0..3}.
// O takes 4 registers per 16 d (half the 32-row engine's), which leaves room
// for more resident waves, i.e. more K/V bytes in flight.

constexpr int kVPad16 = 16;  // V row padding (elements) of the 16-row engine

template <int D, bool FP8>
struct Geom16 {
    static constexpr int BN = 32;
    static constexpr int ESZ = FP8 ? 1 : 2;
    static constexpr int VSTR = D + kVPad16;
    static constexpr int NKC = D / 32;               // 32-element d chunks (QK steps)
    static constexpr int NDB = D / 16;               // 16-wide d blocks (PV steps)
    static constexpr int EPC = 16 / ESZ;             // cached elements per 16-byte chunk
    static constexpr int CPR = D / EPC;              // chunks per key row
    static constexpr int RSTEP = 64 / CPR;           // V rows per wave pass
    static constexpr int NCH = BN / RSTEP;           // V chunks per lane per tile
    static constexpr int KB = FP8 ? 8 : 16;          // bytes of one K operand load
    static_assert(64 % CPR == 0 && BN % RSTEP == 0, "V tile rows must divide evenly");
};

// BIG: blocks of at least 16 keys, so each 16-key half of a tile lies in one
// block and the V rows take their half's block id (no per-row table reads).
template <int D, typename QT, bool FP8, bool BIG, bool NT = false>
struct Loader16 {
    typedef Geom16<D, FP8> G;
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    // K operands: [buffer][kb][kc], 16 bytes (8 for fp8) per lane.  fp8 K
    // with blocks of 16 keys or more takes two buffers, so the next tile's K
    // is in flight while this one's is in use (32 registers); 16-bit K, and
    // smaller blocks with their per-row V block ids, have room for one.
    typedef typename std::conditional<FP8, u32x2, u32x4>::type kword;
    static constexpr int KBUF = FP8 && BIG ? 2 : 1;
    kword kreg[KBUF][2][G::NKC];
    u32x4 vreg[G::NCH];
    int kphys[2], vphys[BIG ? 1 : G::NCH];
    int vcc, vrow0;

    __device__ __forceinline__ void init(int lane) {
        vcc = lane % G::CPR;
        vrow0 = lane / G::CPR;
    }
    __device__ __forceinline__ void ids(const int32_t* bt_row, int t, int s_k, int lb, int lane) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = min(t * G::BN + 16 * kb + (lane & 15), s_k - 1);
            kphys[kb] = bt_row[key >> lb];
        }
        if constexpr (!BIG) {
#pragma unroll
            for (int i = 0; i < G::NCH; ++i) {
                const int key = min(t * G::BN + vrow0 + i * G::RSTEP, s_k - 1);
                vphys[i] = bt_row[key >> lb];
            }
        }
    }
    // K straight into operand registers, V rows as 16-byte chunks; keys past
    // S_k read slot S_k - 1 and are masked (p = 0)
    __device__ __forceinline__ void load(const unsigned char* base_k, const unsigned char* base_v,
                                         int t, int s_k, int lb, int64_t slot_bytes, int lane) {
        load_k<0>(base_k, t, s_k, lb, slot_bytes, lane);
        load_v(base_v, t, s_k, lb, slot_bytes);
    }
    template <int BUF>
    __device__ __forceinline__ void load_k(const unsigned char* base_k, int t, int s_k, int lb,
                                           int64_t slot_bytes, int lane) {
        const int bmask = (1 << lb) - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = min(t * G::BN + 16 * kb + (lane & 15), s_k - 1);
            const unsigned char* row =
                base_k + (((int64_t)kphys[kb] << lb) + (key & bmask)) * slot_bytes +
                (lane >> 4) * 8 * G::ESZ;
#pragma unroll
            for (int kc = 0; kc < G::NKC; ++kc) {
                // K: plain loads.  With the non-temporal hint the K operand
                // loads (16 key rows x 4 chunks a wave) measured slower: 64-row
                // bf16 decode at d = 256 0.362 -> 0.395 ms, fp8 variant_mix's
                // decode rows 0.055 -> 0.073 ms; V's 16-byte row chunks gain
                kreg[BUF][kb][kc] = load_kv<false, kword>(row + 32 * G::ESZ * kc);
            }
        }
    }
    __device__ __forceinline__ void load_v(const unsigned char* base_v, int t, int s_k, int lb,
                                           int64_t slot_bytes) {
        const int bmask = (1 << lb) - 1;
        const int col = vcc * 16;
#pragma unroll
        for (int i = 0; i < G::NCH; ++i) {
            const int key = t * G::BN + vrow0 + i * G::RSTEP;
            const int kc2 = min(key, s_k - 1);
            const int ph = BIG ? ((vrow0 + i * G::RSTEP) >= 16 ? kphys[1] : kphys[0])
                               : vphys[BIG ? 0 : i];
            const int64_t off = (((int64_t)ph << lb) + (kc2 & bmask)) * slot_bytes + col;
            vreg[i] = load_kv<NT, u32x4>(base_v + off);  // untouched until stored
        }
    }
    // the K operand of (kb, kc) in the Q type
    template <int BUF>
    __device__ __forceinline__ v8 kop(int kb, int kc) const {
        if constexpr (FP8) {
            const u32x2 lo = Q::cvt_fp8x4(kreg[BUF][kb][kc][0]);
            const u32x2 hi = Q::cvt_fp8x4(kreg[BUF][kb][kc][1]);
            return __builtin_bit_cast(v8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        } else {
            return __builtin_bit_cast(v8, kreg[BUF][kb][kc]);
        }
    }
    __device__ __forceinline__ void store_v(unsigned short* v_lds) const {
#pragma unroll
        for (int i = 0; i < G::NCH; ++i) {
            const int row = vrow0 + i * G::RSTEP;
            if (FP8) {
                u32x4 v0, v1;
                u32x2 t2;
                t2 = Q::cvt_fp8x4(vreg[i][0]); v0[0] = t2[0]; v0[1] = t2[1];
                t2 = Q::cvt_fp8x4(vreg[i][1]); v0[2] = t2[0]; v0[3] = t2[1];
                t2 = Q::cvt_fp8x4(vreg[i][2]); v1[0] = t2[0]; v1[1] = t2[1];
                t2 = Q::cvt_fp8x4(vreg[i][3]); v1[2] = t2[0]; v1[3] = t2[1];
                *reinterpret_cast<u32x4*>(&v_lds[row * G::VSTR + vcc * 16]) = v0;
                *reinterpret_cast<u32x4*>(&v_lds[row * G::VSTR + vcc * 16 + 8]) = v1;
            } else {
                *reinterpret_cast<u32x4*>(&v_lds[row * G::VSTR + vcc * 8]) = vreg[i];
            }
        }
    }
};

// the value of lane l ^ 16
__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16, 64); }

// per-lane offset (elements) of the first transposing V read of d block 0
template <int D>
__host__ __device__ inline int v16_frag_offset(int lane) {
    const int G = lane >> 4, J = (lane & 15) >> 2, A = lane & 3;
    return (4 * G + J) * (D + kVPad16) + 4 * A;
}

// S^T of one tile from the K operands in registers (buffer BUF)
template <int BUF, int D, typename QT, bool FP8, bool BIG, bool NT>
__device__ __forceinline__ void qk_tile16(const Loader16<D, QT, FP8, BIG, NT>& ld,
                                          const typename QType<QT>::v8 (&qf)[D / 32],
                                          f32x4 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x4{};
#pragma unroll
        for (int kc = 0; kc < D / 32; ++kc)
            sacc[kb] = QType<QT>::mma16(ld.template kop<BUF>(kb, kc), qf[kc], sacc[kb]);
    }
}

// transform, masks, online softmax and O^T += V^T P^T for one tile
template <int D, typename QT, bool FP8, int XF>
__device__ __forceinline__ void softmax_pv16(const UaKernelParams& p, f32x4 (&sacc)[2],
                                             const unsigned short* __restrict__ v_lds,
                                             f32x4 (&oacc)[D / 16], float& m_run, float& l_run,
                                             int key0, bool need_mask, const RowCtx& rc, int grp,
                                             int v_frag) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    typedef Geom16<D, FP8> G;
    const float c = XF != 0 ? 1.0f : p.qk_scale_log2;
    if (XF != 0) {
        const bool qq = XF == kXfQQ && key0 + G::BN > rc.ctx;
        transform_scores<2, 4>(
            p, sacc, [&](int kb, int i) { return key0 + 16 * kb + 4 * grp + i; }, rc, qq);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = key0 + 16 * kb + 4 * grp + i;
            float sv = sacc[kb][i];
            if (need_mask) sv = ((key >= rc.kmin) & (key <= rc.kmax)) ? sv : -INFINITY;
            sacc[kb][i] = sv;
            mt = fmaxf(mt, sv);
        }
    mt = fmaxf(mt, xor16(mt));
    mt = max_halves(mt) * c;
    // lazy reference max, as in the 32-row engine
    if (__ballot(mt > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mt);
        const float m_base = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_base);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) oacc[db] *= alpha;
        m_run = m_new;
    }
    v8 pf;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        pf[j] = (QT)fast_exp2(__builtin_fmaf(sacc[j >> 2][j & 3], c, -m_run));
#pragma unroll
    for (int j = 0; j < 8; j += 2) l_run = Q::sum2(pf[j], pf[j + 1], l_run);
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        const int off = v_frag + 16 * db;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&v_lds[off]);
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&v_lds[off + 16 * G::VSTR]);
        u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        u32x4 w = {lo2[0], lo2[1], hi2[0], hi2[1]};
        oacc[db] = Q::mma16(__builtin_bit_cast(v8, w), pf, oacc[db]);
    }
}

// resident waves per SIMD the 16-row engine's registers allow
constexpr int min_waves16(int d, bool fp8) {
    return d <= 64 ? 4 : d <= 128 ? (fp8 ? 3 : 2) : (fp8 ? 2 : 1);
}
// heads (waves) of one 16-row stream-K worker, as for the 32-row engine
constexpr int sk16_max_heads(int d, bool fp8) {
    return kSkMaxHeads < 4 * min_waves16(d, fp8) ? kSkMaxHeads : 4 * min_waves16(d, fp8);
}

template <int D, typename QT, bool FP8, int XF, bool BIG>
__global__ __launch_bounds__(64 * sk16_max_heads(D, FP8), min_waves16(D, FP8)) void ua_decode16_kernel(
    UaKernelParams p) {
    typedef QType<QT> Q;
    typedef typename Q::v8 v8;
    typedef Geom16<D, FP8> G;
    constexpr int BN = G::BN;
    static_assert(BN == kSkTile, "the reduce locates stream-K partials with this tile size");

    // issue priority when not beside a wide launch, as in ua_decode_sk_kernel
    if (p.class_mode != 1) __builtin_amdgcn_s_setprio(2);
    // one V tile per wave (dynamic LDS sized at launch); the waves of a worker
    // share nothing else
    extern __shared__ __attribute__((aligned(16))) unsigned short sk16_lds[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned short* v_lds = sk16_lds + wave * (BN * G::VSTR);

    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4;
    const int64_t W = gridDim.x;
    const int64_t j = blockIdx.x;
    const int T = sk_total<BN>(p);
    const int64_t A = j * T / W;
    const int64_t B = (j + 1) * T / W;
    if (A >= B) return;

    int seq_first;
    const int s0 = sk_locate<BN>(p, A, &seq_first);
    SkPos pc = sk_pos<BN>(p, s0, 0, 0);
    {
        const int n = pc.t_end - pc.t_lo;
        const int off = (int)(A - seq_first);
        pc.h = off / n;
        pc.t = pc.t_lo + (off - pc.h * n);
    }
    SkPos p1 = pc, p2 = pc;
    if (A + 1 < B) p1 = sk_next<BN>(p, pc);
    if (A + 2 < B) p2 = sk_next<BN>(p, p1);

    const int lb = p.block_size_log2;
    const int64_t slot_bytes = p.kv_slot_stride * G::ESZ;
    const unsigned char* kc = reinterpret_cast<const unsigned char*>(p.k);
    const unsigned char* vc = reinterpret_cast<const unsigned char*>(p.v);
    auto bt_row = [&](const SkPos& q) { return table_row(p, q.s); };
    auto head = [&](const SkPos& q) { return q.h * p.sk_heads + wave; };
    auto hoff = [&](const SkPos& q) {
        return q.kv_row * slot_bytes + (int64_t)head(q) * D * G::ESZ;
    };

    Loader16<D, QT, FP8, BIG, true> ld;  // each key row is read once: non-temporal
    ld.init(lane);
    const int v_frag = v16_frag_offset<D>(lane);
    ld.ids(bt_row(pc), pc.t, pc.s_k, lb, lane);
    ld.load(kc + hoff(pc), vc + hoff(pc), pc.t, pc.s_k, lb, slot_bytes, lane);
    if (A + 1 < B) ld.ids(bt_row(p1), p1.t, p1.s_k, lb, lane);

    RowInfo ri;
    KeyRange kr;
    v8 qf[G::NKC];
    f32x4 oacc[G::NDB];
    float m_run, l_run;
    auto begin_pair = [&](const SkPos& q) {
        ri = row_info(p, lane & 15, head(q), q.q_start, q.q_len, q.s_k, 0);
        kr = key_range(p.flags, p.window, q.s_k, q.s_k - q.q_len, 0, q.q_len - 1);
        const QT* qp = reinterpret_cast<const QT*>(p.q) + (int64_t)ri.tok * p.q_stride_tok +
                       (int64_t)ri.head * D + 8 * grp;
#pragma unroll
        for (int k2 = 0; k2 < G::NKC; ++k2) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (ri.ok) w = *reinterpret_cast<const u32x4*>(qp + 32 * k2);
            qf[k2] = __builtin_bit_cast(v8, w);
        }
        m_run = kMaxStart;
        l_run = 0.0f;
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) oacc[db] = f32x4{};
    };
    begin_pair(pc);

    // The worker's waves meet once per tile with 16-bit K/V, as in the 32-row
    // engine (measured: bf16 decode at d = 256, 0.229 -> 0.217 ms with four kv
    // heads per worker, 0.419 -> 0.404 with eight); each wave's own LDS order
    // needs no barrier, and fp8 workers run free (a barrier there cost 1%,
    // and 4% on variant_mix).
    constexpr bool WG_SYNC = !FP8;
    constexpr int KBUF = Loader16<D, QT, FP8, BIG, true>::KBUF;
    // One tile; its K operands sit in buffer BUF.  The next tile's V is
    // loaded as soon as this tile's has left the registers, and its K into
    // the other buffer before this tile's QK (two K buffers), else once QK
    // has consumed this tile's operands.
    auto step = [&](auto buf_c, int64_t x) {
        constexpr int BUF = decltype(buf_c)::value;
        constexpr int NXT = (BUF + 1) % KBUF;
        // this tile's V into LDS (the previous tile's reads are done: one
        // wave, LDS operations in order)
        if (WG_SYNC) __syncthreads();
        ld.store_v(v_lds);
        if (x + 1 < B) {
            ld.load_v(vc + hoff(p1), p1.t, p1.s_k, lb, slot_bytes);
            if (KBUF == 2) {
                ld.template load_k<NXT>(kc + hoff(p1), p1.t, p1.s_k, lb, slot_bytes, lane);
                if (x + 2 < B) ld.ids(bt_row(p2), p2.t, p2.s_k, lb, lane);
            }
        }
        const int key0 = pc.t * BN;
        const bool need_mask = !(key0 >= kr.full_lo && key0 + BN - 1 <= kr.full_hi);
        f32x4 sacc[2];
        qk_tile16<BUF>(ld, qf, sacc);
        if (KBUF == 1 && x + 1 < B) {
            ld.template load_k<NXT>(kc + hoff(p1), p1.t, p1.s_k, lb, slot_bytes, lane);
            if (x + 2 < B) ld.ids(bt_row(p2), p2.t, p2.s_k, lb, lane);
        }
        softmax_pv16<D, QT, FP8, XF>(p, sacc, v_lds, oacc, m_run, l_run, key0, need_mask, ri.rc,
                                        grp, v_frag);
        if (x + 1 == B || pc.t + 1 == pc.t_end) {
            float l_tot = l_run + xor16(l_run);
            l_tot += xor32(l_tot);
            if (ri.ok) {
                const int64_t unit = (int64_t)pc.s * sk_groups(p) + pc.h;
                const int64_t slot = (unit + j) * p.sk_heads + wave;
                const int64_t rid = slot * p.rows_used + (lane & 15);
#pragma unroll
                for (int db = 0; db < G::NDB; ++db)
                    store4(p.ws_o, rid * D + 4 * grp + 16 * db, oacc[db], p.ws_bf16);
                if (grp == 0) {
                    p.ws_m[rid] = m_run;
                    p.ws_l[rid] = l_tot;
                }
            }
            if (x + 1 < B) begin_pair(p1);
        }
        pc = p1;
        p1 = p2;
        if (x + 3 < B) p2 = sk_next<BN>(p, p2);
    };
    if constexpr (KBUF == 2) {
        for (int64_t x = A; x < B; x += 2) {
            step(std::integral_constant<int, 0>{}, x);
            if (x + 1 < B) step(std::integral_constant<int, 1>{}, x + 1);
        }
    } else {
        for (int64_t x = A; x < B; ++x) step(std::integral_constant<int, 0>{}, x);
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split partials
// ---------------------------------------------------------------------------
//
// The re-base of section 5 of the unified page: M = max over partials (and the
// sink), L = sum l_i 2^(m_i - M) (+ 2^(sink - M)), O = sum o_i 2^(m_i - M) / L,
// then the cast.  Partials with m = -inf saw no visible key and are skipped.
// One wave per (token, query head); four per workgroup.  Partials are merged
// in a fixed order, four at a time with all their loads issued together, so
// the result is the same on every run.
// N consecutive partial values (f32, or bf16 when `bf16`) from element
// `elem` of `base` as one vector load of 4 N or 2 N bytes (elem is a
// multiple of N and the buffer 16-byte aligned).
template <int N>
__device__ __forceinline__ void load_row_part(const void* base, int64_t elem, bool bf16,
                                              float (&out)[N]) {
    if (bf16) {
        typedef __bf16 vb __attribute__((ext_vector_type(N)));
        const vb x = *reinterpret_cast<const vb*>(static_cast<const __bf16*>(base) + elem);
#pragma unroll
        for (int e = 0; e < N; ++e) out[e] = (float)x[e];
    } else {
        typedef float vf __attribute__((ext_vector_type(N)));
        const vf x = *reinterpret_cast<const vf*>(static_cast<const float*>(base) + elem);
#pragma unroll
        for (int e = 0; e < N; ++e) out[e] = x[e];
    }
}

template <int D, typename QT>
__device__ __forceinline__ void merge_partials(const UaKernelParams& p, int64_t first, int64_t stride,
                                               int count, int64_t j0, int64_t T, int64_t W, bool sk,
                                               int tok, int head) {
    constexpr int EPL = D / 64;  // elements per lane
    constexpr int U = 4;
    const int lane = threadIdx.x & 63;
    const bool sinks = p.flags & UA_FLAG_SINKS;
    float mx = sinks ? p.sinks[head] * kLog2e : -INFINITY;
    float L = sinks ? 1.0f : 0.0f;  // the sink term, at its own max
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    for (int g0 = 0; g0 < count; g0 += U) {
        float mg[U], lg[U], og[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u;
            const int64_t j = j0 + g;
            const bool live = g < count && (!sk || j * T / W < (j + 1) * T / W);
            const int64_t rid = first + (int64_t)(live ? g : 0) * stride;
            mg[u] = live ? p.ws_m[rid] : -INFINITY;
            lg[u] = live ? p.ws_l[rid] : 0.0f;
            load_row_part<EPL>(p.ws_o, rid * D + lane * EPL, p.ws_bf16, og[u]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) og[u][e] = live ? og[u][e] : 0.0f;
        }
        float bm = mx;
#pragma unroll
        for (int u = 0; u < U; ++u) bm = fmaxf(bm, mg[u]);
        if (bm == -INFINITY) continue;
        const float a = fast_exp2(mx - bm);  // 0 when nothing was merged yet
        L *= a;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] *= a;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = fast_exp2(mg[u] - bm);  // 0 for dead partials
            L += lg[u] * w;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] += w * og[u][e];
        }
        mx = bm;
    }
    const float inv = L > 0.0f ? p.out_scale / L : 0.0f;
    if (p.part_o) {
        // partial-output mode: the merged row's o / L and its LSE
        const int64_t row = (int64_t)tok * p.num_q_heads + head;
        if (lane == 0) p.part_lse[row] = row_lse(mx, L);
        if (p.part_bf16) {
            __bf16* dst = static_cast<__bf16*>(p.part_o) + row * D + lane * EPL;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dst[e] = (__bf16)(acc[e] * inv);
        } else {
            float* dst = static_cast<float*>(p.part_o) + row * D + lane * EPL;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dst[e] = acc[e] * inv;
        }
        return;
    }
    if (p.lse && lane == 0) p.lse[(int64_t)tok * p.num_q_heads + head] = row_lse(mx, L);
    QT* dst = reinterpret_cast<QT*>(p.o) + (int64_t)tok * p.o_stride_tok + (int64_t)head * D +
              lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = (QT)(acc[e] * inv);
}

template <int D, typename QT, bool SK>
__global__ __launch_bounds__(256) void ua_reduce_kernel(UaKernelParams p, int64_t n_rows) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int tok = (int)(row / p.num_q_heads);
    const int head = (int)(row - (int64_t)tok * p.num_q_heads);

    if (SK && p.reduce_by_seq) {
        // rows enumerated as (sequence, query head, local position)
        const int per_seq = p.num_q_heads * p.small_block_q;
        const int s = (int)(row / per_seq);
        const int rem = (int)(row - (int64_t)s * per_seq);
        const int head2 = rem / p.small_block_q;
        const int i = rem - head2 * p.small_block_q;
        const int q_start = p.cu_q[s];
        const int q_len = p.cu_q[s + 1] - q_start;
        if (i >= q_len || q_len > p.small_block_q) return;
        int n, total;
        const int xs = sk_seq_prefix<kSkTile>(p, s, &n, &total);
        const int64_t T = total;
        const int64_t W = p.sk_workers;
        const int hk = head2 / p.group;
        const int hg = hk / p.sk_heads, wv = hk - hg * p.sk_heads;
        const int64_t x0 = xs + (int64_t)hg * n;
        const int j0 = T > 0 ? sk_worker_of(x0, T, W) : 0;
        const int j1 = T > 0 ? sk_worker_of(x0 + n - 1, T, W) : 0;
        const int r = i * p.group + (head2 - hk * p.group);
        const int count = (n > 0 && T > 0) ? j1 - j0 + 1 : 0;
        const int64_t slot0 = ((int64_t)s * sk_groups(p) + hg + j0) * p.sk_heads + wv;
        merge_partials<D, QT>(p, slot0 * p.rows_used + r, (int64_t)p.sk_heads * p.rows_used, count,
                              j0, T, W, true, q_start + i, head2);
    } else if (SK) {
        // one pass over the sequences: the token's sequence s, the first
        // flattened tile of s, its tile count and the total T
        int carry = 0, s = -1, xs = 0, n = 0, q_start = 0, q_len = 0;
        for (int base = 0; base < p.num_seqs; base += 64 * kSkScanChunks) {
            SeqLane qc[kSkScanChunks];
#pragma unroll
            for (int c = 0; c < kSkScanChunks; ++c) qc[c] = seq_lane<kSkTile>(p, base + 64 * c + lane);
#pragma unroll
            for (int c = 0; c < kSkScanChunks; ++c) {
                const SeqLane& q = qc[c];
                const int b = base + 64 * c;
                const int v = q.n * sk_groups(p);
                const int incl = wave_incl_scan(v);
                const bool past = b + lane < p.num_seqs && q.q_start + q.q_len <= tok;
                const uint64_t before = __ballot(!past && b + lane < p.num_seqs);
                if (s < 0 && before) {
                    const int l = __builtin_ctzll(before);
                    s = b + l;
                    xs = carry + readlane(incl - v, l);
                    n = readlane(q.n, l);
                    q_start = readlane(q.q_start, l);
                    q_len = readlane(q.q_len, l);
                }
                carry += readlane(incl, 63);
            }
        }
        // rows of the wide launch's sequences are that launch's to write
        if (p.class_mode == 1 && q_len > p.small_block_q) return;
        const int64_t T = carry;
        const int64_t W = p.sk_workers;
        const int hk = head / p.group;
        const int hg = hk / p.sk_heads, wv = hk - hg * p.sk_heads;
        const int64_t x0 = xs + (int64_t)hg * n;
        const int j0 = T > 0 ? sk_worker_of(x0, T, W) : 0;
        const int j1 = T > 0 ? sk_worker_of(x0 + n - 1, T, W) : 0;
        const int r = (tok - q_start) * p.group + (head - hk * p.group);
        const int count = (s >= 0 && n > 0 && T > 0) ? j1 - j0 + 1 : 0;
        const int64_t slot0 = ((int64_t)s * sk_groups(p) + hg + j0) * p.sk_heads + wv;
        merge_partials<D, QT>(p, slot0 * p.rows_used + r, (int64_t)p.sk_heads * p.rows_used, count,
                              j0, T, W, true, tok, head);
    } else {
        const int s = token_seq(p.cu_q, p.num_seqs, tok);
        const int q_start = p.cu_q[s];
        const int q_len = p.cu_q[s + 1] - q_start;
        if (p.class_mode == 2 && q_len <= p.small_block_q) return;  // the decode kernel's rows
        const int s_k = seq_keys(p, s);
        const int ctx = s_k - q_len;
        const int p0 = ((tok - q_start) / p.block_q) * p.block_q;
        const int p_last = min(p0 + p.block_q, q_len) - 1;
        const KeyRange kr = key_range(p.flags, p.window, s_k, ctx, p0, p_last);
        const int t_lo = kr.lo / p.tile_n;
        const int t_hi = (kr.hi + p.tile_n - 1) / p.tile_n;
        const int count = seg_pieces(t_hi - t_lo, p.num_segments, p.tiles_per_seg);
        if (count == 1) return;  // one piece: the attention kernel wrote the row
        merge_partials<D, QT>(p, row * p.num_segments, 1, count, 0, 1, 1, false, tok, head);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Workers of the stream-K split: as many workgroups of `waves` waves (and
// `lds` bytes of dynamic LDS) as the device holds at once.  Queried once per
// (device, kernel, shape): every kernel of the family has the same function
// type, so the kernel's address is part of the key.
struct ResidentKey {
    int dev;
    const void* kernel;
    int waves;
    size_t lds;
};

inline int resident_workgroups_of(const void* kernel, int waves, size_t lds) {
    static std::mutex mu;
    static std::vector<std::pair<ResidentKey, int>> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : cache)
        if (e.first.dev == dev && e.first.kernel == kernel && e.first.waves == waves &&
            e.first.lds == lds)
            return e.second;
    int per_cu = 0, cus = 0;
    if (lds > 0)
        (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * waves, lds) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    cache.push_back({ResidentKey{dev, kernel, waves, lds}, per_cu * cus});
    return per_cu * cus;
}

template <typename K>
int resident_workgroups(K kernel, int waves = 1, size_t lds = 0) {
    return resident_workgroups_of(reinterpret_cast<const void*>(kernel), waves, lds);
}

template <int D, int NW, int BN, typename QT, bool FP8, int XF>
hipError_t launch_attn(const UaKernelParams& p0, const UaLaunch& l, hipStream_t st) {
    UaKernelParams p = p0;
    dim3 grid(l.grid[0], l.grid[1], l.grid[2]);
    hipError_t e = hipSuccess;
    if (l.events[0] && (e = hipEventRecord(l.events[0], st)) != hipSuccess) return e;
    const unsigned nb = (unsigned)((l.reduce_rows + 3) / 4);
    if (l.path == 3 && l.stream_k) {
        if constexpr (NW == 1 && BN == kSkTile) {
            int workers = 0;
            if (l.rows16) {
                // built for d = 256 only (the plan asks for it there)
                if constexpr (D == 256) {
                    int gh = sk16_max_heads(D, FP8);
                    while (gh > 1 && p.num_kv_heads % gh) gh >>= 1;
                    p.sk_heads = gh;
                    const size_t lds = (size_t)gh * Geom16<D, FP8>::BN * Geom16<D, FP8>::VSTR * 2;
                    auto kern = p.block_size_log2 >= 4 ? ua_decode16_kernel<D, QT, FP8, XF, true>
                                                       : ua_decode16_kernel<D, QT, FP8, XF, false>;
                    workers = std::min(resident_workgroups(kern, gh, lds), l.sk_waves_cap / gh);
                    p.sk_workers = workers;
                    hipLaunchKernelGGL(kern, dim3(workers), dim3(64 * gh), lds, st, p);
                } else {
                    return hipErrorInvalidValue;
                }
            } else if constexpr (D == 256 && !FP8 && XF == kXfQQ) {
                // not built: the compiler miscompiles this instantiation (it
                // drops a register copy of a spilled Q fragment); the plan
                // never asks for it
                return hipErrorInvalidValue;
            } else {
                // workers of sk_heads waves, one kv head each
                int gh = sk_max_heads<D>();
                while (gh > 1 && p.num_kv_heads % gh) gh >>= 1;
                p.sk_heads = gh;
                const size_t lds = (size_t)gh * sk_wave_lds_elems<D, BN, FP8>() * 2;
                auto kern = ua_decode_sk_kernel<D, BN, QT, FP8, XF>;
                workers = std::min(resident_workgroups(kern, gh, lds), l.sk_waves_cap / gh);
                p.sk_workers = workers;
                hipLaunchKernelGGL(kern, dim3(workers), dim3(64 * gh), lds, st, p);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (l.events[1] && (e = hipEventRecord(l.events[1], st)) != hipSuccess) return e;
            hipLaunchKernelGGL((ua_reduce_kernel<D, QT, true>), dim3(nb), dim3(256), 0, st, p,
                               l.reduce_rows);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        // 16-bit K/V in four-wave workgroups take the LDS ring when one
        // wave-wide copy's key rows always share a block.  At d = 256 not
        // with the QQ bias, whose per-element loads the ring's registers
        // cannot hold; with softcap or ALiBi the d = 256 ring spills, but only
        // in its masked and partial-tile branches, and still beats the
        // register path, which loads each tile after the barrier.
        constexpr bool ring_built = UA_LDS_RING && NW == 4 && BN == LdsGeom<D>::BN && !FP8 &&
                                    D <= UA_LDS_RING_MAX_D && (D <= 128 || XF != kXfQQ);
        const bool ring = ring_built && (1 << p.block_size_log2) >= LdsGeom<D>::ROWS_PER_OP &&
                          p.kv_slot_stride * 2 * LdsGeom<D>::ROWS_PER_OP < (int64_t(1) << 31);
        const bool split = l.path == 3;
        if constexpr (ring_built) {
            if (ring && split)
                hipLaunchKernelGGL((ua_attn_lds_kernel<D, QT, true, XF>), grid, dim3(256), 0, st, p);
            if (ring && !split && l.persistent) {
                // as many workgroups as are resident at once, at most one per item
                auto kern = ua_attn_persist_kernel<D, QT, XF>;
                const int64_t items = (int64_t)grid.x * grid.y;
                p.persist_slots = (int32_t)grid.y;
                // every queue that holds items gets at least one workgroup
                int64_t wgs = std::min<int64_t>(items, resident_workgroups(kern, 4));
                if (items >= kPersistQueues)
                    wgs = std::max<int64_t>(kPersistQueues, wgs / kPersistQueues * kPersistQueues);
                hipLaunchKernelGGL(ua_queue_reset_kernel<kPersistQueues>, dim3(1), dim3(64), 0, st, p.queue);
                hipLaunchKernelGGL(kern, dim3((unsigned)std::max<int64_t>(wgs, 1)), dim3(256), 0, st, p);
            } else if (ring && !split) {
                hipLaunchKernelGGL((ua_attn_lds_kernel<D, QT, false, XF>), grid, dim3(256), 0, st, p);
            }
        }
        if (!ring && split)
            hipLaunchKernelGGL((ua_attn_kernel<D, NW, BN, QT, FP8, true, XF>), grid, dim3(NW * 64),
                               0, st, p);
        if (!ring && !split)
            hipLaunchKernelGGL((ua_attn_kernel<D, NW, BN, QT, FP8, false, XF>), grid, dim3(NW * 64),
                               0, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (l.events[1] && (e = hipEventRecord(l.events[1], st)) != hipSuccess) return e;
        if (split)
            hipLaunchKernelGGL((ua_reduce_kernel<D, QT, false>), dim3(nb), dim3(256), 0, st, p,
                               l.reduce_rows);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (l.events[2] && (e = hipEventRecord(l.events[2], st)) != hipSuccess) return e;
    return hipSuccess;
}

// a geometry is built only where every thread's tile rows divide evenly
template <int D, int NW, int BN, bool FP8>
constexpr bool geometry_ok() {
    constexpr int cpr = D / (FP8 ? 16 : 8);
    return (NW * 64) % cpr == 0 && BN % ((NW * 64) / cpr) == 0;
}

template <int D, int NW, int BN, typename QT, bool FP8, int XF>
hipError_t launch_if_built(const UaKernelParams& p, const UaLaunch& l, hipStream_t st) {
    if constexpr (geometry_ok<D, NW, BN, FP8>()) return launch_attn<D, NW, BN, QT, FP8, XF>(p, l, st);
    return hipErrorInvalidValue;
}

template <int D, typename QT, bool FP8, int XF>
hipError_t launch_geometry(const UaKernelParams& p, const UaLaunch& l, hipStream_t st) {
    if (l.waves == 1 && l.tile_n == 32) return launch_if_built<D, 1, 32, QT, FP8, XF>(p, l, st);
    if (l.waves == 4 && l.tile_n == 32) return launch_if_built<D, 4, 32, QT, FP8, XF>(p, l, st);
    if constexpr (D == 64) {
        // 64-key tiles: four-wave fp8 tiles at d = 64 (a tile holds whole
        // passes of 256 threads' 16-byte chunks)
        if (l.waves == 4 && l.tile_n == 64) return launch_if_built<D, 4, 64, QT, FP8, XF>(p, l, st);
    }
    return hipErrorInvalidValue;
}

template <int D, typename QT, bool FP8>
hipError_t launch_xform(const UaKernelParams& p, const UaLaunch& l, hipStream_t st) {
    if (p.flags & UA_FLAG_QQ_BIAS) return launch_geometry<D, QT, FP8, kXfQQ>(p, l, st);
    // softcap alone folds into the exponent where the registers allow (at
    // d = 256 the register path would spill)
    if constexpr (D <= 128)
        if ((p.flags & UA_FLAG_SOFTCAP) && !(p.flags & UA_FLAG_ALIBI))
            return launch_geometry<D, QT, FP8, kXfCap>(p, l, st);
    if (p.flags & (UA_FLAG_SOFTCAP | UA_FLAG_ALIBI))
        return launch_geometry<D, QT, FP8, kXfScore>(p, l, st);
    return launch_geometry<D, QT, FP8, kXfNone>(p, l, st);
}

template <int D>
hipError_t launch_head_dim(const UaKernelParams& p, const UaLaunch& l, hipStream_t st) {
    if (l.q_dtype == UA_DTYPE_BF16)
        return l.kv_fp8 ? launch_xform<D, __bf16, true>(p, l, st)
                        : launch_xform<D, __bf16, false>(p, l, st);
    return l.kv_fp8 ? launch_xform<D, _Float16, true>(p, l, st)
                    : launch_xform<D, _Float16, false>(p, l, st);
}

}  // namespace ua

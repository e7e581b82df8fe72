// Test-only probe of the K/V tile gathers and of two hardware facts the
// kernels rely on.  Each gather workgroup runs the kernels' own gather
// routines (the LDS ring's copies, the register-staged KvLoader, or the
// 16-row engine's Loader16) for one (sequence, kv-head, tile), then copies the
// gathered tile out to a dense [tile][32 keys][d] buffer of 16-bit elements,
// undoing the ring's chunk permutation, the register path's padding or the
// operand-register layout.  The test compares those bytes with a host gather
// of the same keys, bit for bit.  Two more probes return what the transposing
// LDS read delivers to each of the 64 lanes, and what the kernels' fp8
// conversion makes of every e4m3 code.  Nothing else in the build calls this
// library.
#include "ua_attn_impl.h"

using namespace ua;

namespace {

struct ProbeArgs {
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* tiles;  // [n][3] = (sequence, kv-head, tile index)
    unsigned short* out_k;  // [n][32][d]
    unsigned short* out_v;
    int64_t kv_slot_stride;  // H_k * d elements
    int bt_stride, block_size_log2;
};

template <int D>
__global__ __launch_bounds__(256) void probe_ring(ProbeArgs a) {
    typedef LdsGeom<D> L;
    __shared__ __attribute__((aligned(1024))) unsigned short stage[2 * L::TILE_ELEMS];
    const int i = blockIdx.x;
    const int s = a.tiles[3 * i], hk = a.tiles[3 * i + 1], t = a.tiles[3 * i + 2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lb = a.block_size_log2;
    const int s_k = min(a.seq_lens[s], a.bt_stride << lb);
    const uint64_t slot_bytes = (uint64_t)a.kv_slot_stride * 2;
    const unsigned char* base_k = reinterpret_cast<const unsigned char*>(a.k) + (int64_t)hk * D * 2;
    const unsigned char* base_v = reinterpret_cast<const unsigned char*>(a.v) + (int64_t)hk * D * 2;
    const const_i32_ptr bt = (const_i32_ptr)(a.block_table + (int64_t)s * a.bt_stride);
    LdsCopy<D> cp;
    cp.init(wave, lane, (uint32_t)slot_bytes);
    int id[L::GROUPS];
    __builtin_amdgcn_s_waitcnt(kWaitVmcntZero);
    lds_tile_ids<D>(bt, t, s_k, lb, wave, id);
    lds_tile_issue<D>(cp, base_k, base_v, t, s_k, lb, slot_bytes, id,
                      __builtin_amdgcn_readfirstlane(lds_address(stage)), wave);
    lds_tile_barrier<0>();
    for (int x = tid; x < L::BN * L::CPR; x += 256) {
        const int r = x / L::CPR, c = x % L::CPR;
        const u32x4 kw = *reinterpret_cast<const u32x4*>(&stage[r * D + 8 * (c ^ swz_k<D>(r))]);
        const u32x4 vw =
            *reinterpret_cast<const u32x4*>(&stage[L::TILE_ELEMS + r * D + 8 * (c ^ swz_v<D>(r))]);
        *reinterpret_cast<u32x4*>(&a.out_k[((int64_t)i * L::BN + r) * D + 8 * c]) = kw;
        *reinterpret_cast<u32x4*>(&a.out_v[((int64_t)i * L::BN + r) * D + 8 * c]) = vw;
    }
}

template <int D, int NW, typename QT, bool FP8>
__global__ __launch_bounds__(NW * 64) void probe_registers(ProbeArgs a) {
    constexpr int BN = 32;
    typedef TileGeom<D, NW, BN, FP8> G;
    __shared__ __attribute__((aligned(16))) unsigned short k_lds[BN * G::KSTR];
    __shared__ __attribute__((aligned(16))) unsigned short v_lds[BN * G::VSTR];
    const int i = blockIdx.x;
    const int s = a.tiles[3 * i], hk = a.tiles[3 * i + 1], t = a.tiles[3 * i + 2];
    const int lb = a.block_size_log2;
    const int s_k = min(a.seq_lens[s], a.bt_stride << lb);
    const int64_t slot_bytes = a.kv_slot_stride * G::ESZ;
    const unsigned char* base_k = reinterpret_cast<const unsigned char*>(a.k) + (int64_t)hk * D * G::ESZ;
    const unsigned char* base_v = reinterpret_cast<const unsigned char*>(a.v) + (int64_t)hk * D * G::ESZ;
    KvLoader<D, NW, BN, QT, FP8> ld;
    ld.init(threadIdx.x);
    ld.ids(a.block_table + (int64_t)s * a.bt_stride, t, s_k, lb);
    ld.load(base_k, base_v, t, s_k, lb, slot_bytes);
    ld.store(k_lds, v_lds);
    __syncthreads();
    for (int x = threadIdx.x; x < BN * D; x += NW * 64) {
        const int r = x / D, e = x % D;
        a.out_k[((int64_t)i * BN + r) * D + e] = k_lds[r * G::KSTR + e];
        a.out_v[((int64_t)i * BN + r) * D + e] = v_lds[r * G::VSTR + e];
    }
}

// The 16-row decode engine's gather (Loader16), one wave per tile: the K
// operands it loads straight into MFMA A-operand registers (lane l holds key
// 16 kb + l % 16, elements 32 kc + 8 (l / 16) .. + 7, converted to the Q type)
// and the V tile it writes to padded LDS, both copied out densely.
template <int D, typename QT, bool FP8, bool BIG>
__global__ __launch_bounds__(64) void probe_loader16(ProbeArgs a) {
    typedef Geom16<D, FP8> G;
    typedef typename QType<QT>::v8 v8;
    __shared__ __attribute__((aligned(16))) unsigned short v_lds[G::BN * G::VSTR];
    const int i = blockIdx.x;
    const int s = a.tiles[3 * i], hk = a.tiles[3 * i + 1], t = a.tiles[3 * i + 2];
    const int lane = threadIdx.x;
    const int lb = a.block_size_log2;
    const int s_k = min(a.seq_lens[s], a.bt_stride << lb);
    const int64_t slot_bytes = a.kv_slot_stride * G::ESZ;
    const unsigned char* base_k = reinterpret_cast<const unsigned char*>(a.k) + (int64_t)hk * D * G::ESZ;
    const unsigned char* base_v = reinterpret_cast<const unsigned char*>(a.v) + (int64_t)hk * D * G::ESZ;
    Loader16<D, QT, FP8, BIG, true> ld;  // as the 16-row engine instantiates it
    ld.init(lane);
    ld.ids(a.block_table + (int64_t)s * a.bt_stride, t, s_k, lb, lane);
    ld.load(base_k, base_v, t, s_k, lb, slot_bytes, lane);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kc = 0; kc < G::NKC; ++kc) {
            const v8 x = ld.template kop<0>(kb, kc);
            const int64_t row = (int64_t)i * G::BN + 16 * kb + (lane & 15);
            *reinterpret_cast<u32x4*>(&a.out_k[row * D + 32 * kc + 8 * (lane >> 4)]) =
                __builtin_bit_cast(u32x4, x);
        }
    ld.store_v(v_lds);
    __syncthreads();
    for (int x = lane; x < G::BN * D; x += 64) {
        const int r = x / D, e = x % D;
        a.out_v[((int64_t)i * G::BN + r) * D + e] = v_lds[r * G::VSTR + e];
    }
}

// One wave's transposing LDS read: LDS element x holds the value x; lane l
// reads the four 16-bit elements at element offset addr[l] (a multiple of 4)
// with ds_read_b64_tr_b16 and stores what it receives at out[4 l .. 4 l + 3].
constexpr int kTrLdsElems = 4096;
__global__ __launch_bounds__(64) void probe_read_tr(const int32_t* addr, unsigned short* out) {
    __shared__ __attribute__((aligned(16))) unsigned short lds[kTrLdsElems];
    const int lane = threadIdx.x;
    for (int x = lane; x < kTrLdsElems; x += 64) lds[x] = (unsigned short)x;
    __syncthreads();
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&lds[addr[lane]]);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * lane + j] = (unsigned short)v[j];
}

// Every e4m3 code through the kernels' own conversion (QType::cvt_fp8x4, the
// v_cvt_scalef32_pk_{bf16,f16}_fp8 pair): lane l converts the word holding
// codes 4 l .. 4 l + 3 and stores the 16-bit results in code order.
__global__ __launch_bounds__(64) void probe_fp8_codes(unsigned short* out_bf16, unsigned short* out_f16) {
    const int lane = threadIdx.x;
    const unsigned w = (unsigned)(4 * lane) | (unsigned)(4 * lane + 1) << 8 |
                       (unsigned)(4 * lane + 2) << 16 | (unsigned)(4 * lane + 3) << 24;
    const u32x2 b = QType<__bf16>::cvt_fp8x4(w);
    const u32x2 h = QType<_Float16>::cvt_fp8x4(w);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        out_bf16[4 * lane + 2 * j] = (unsigned short)(b[j] & 0xFFFF);
        out_bf16[4 * lane + 2 * j + 1] = (unsigned short)(b[j] >> 16);
        out_f16[4 * lane + 2 * j] = (unsigned short)(h[j] & 0xFFFF);
        out_f16[4 * lane + 2 * j + 1] = (unsigned short)(h[j] >> 16);
    }
}

template <int D>
hipError_t launch(int path, int waves, int fp8_to, const ProbeArgs& a, int n, hipStream_t st) {
    if (path == 0) {
        hipLaunchKernelGGL(probe_ring<D>, dim3(n), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    // fp8_to: 0 = 16-bit cache, 1 = e4m3 -> bf16, 2 = e4m3 -> f16
    if (waves == 1 && fp8_to == 0) hipLaunchKernelGGL((probe_registers<D, 1, __bf16, false>), dim3(n), dim3(64), 0, st, a);
    else if (waves == 4 && fp8_to == 0) hipLaunchKernelGGL((probe_registers<D, 4, __bf16, false>), dim3(n), dim3(256), 0, st, a);
    else if (waves == 1 && fp8_to == 1) hipLaunchKernelGGL((probe_registers<D, 1, __bf16, true>), dim3(n), dim3(64), 0, st, a);
    else if (waves == 1 && fp8_to == 2) hipLaunchKernelGGL((probe_registers<D, 1, _Float16, true>), dim3(n), dim3(64), 0, st, a);
    else if constexpr (D >= 128) {
        // four-wave fp8 tiles of 32 keys need d >= 128 (whole row passes)
        if (waves == 4 && fp8_to == 1) hipLaunchKernelGGL((probe_registers<D, 4, __bf16, true>), dim3(n), dim3(256), 0, st, a);
        else if (waves == 4 && fp8_to == 2) hipLaunchKernelGGL((probe_registers<D, 4, _Float16, true>), dim3(n), dim3(256), 0, st, a);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

template <typename QT, bool FP8>
hipError_t launch16(const ProbeArgs& a, int n, hipStream_t st) {
    // the engine serves d = 256; BIG when blocks hold at least 16 keys
    if (a.block_size_log2 >= 4)
        hipLaunchKernelGGL((probe_loader16<256, QT, FP8, true>), dim3(n), dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((probe_loader16<256, QT, FP8, false>), dim3(n), dim3(64), 0, st, a);
    return hipGetLastError();
}

// path 0 = LDS ring (16-bit, block size >= 1024 / (2 d)); path 1 =
// register-staged gather with `waves` waves; path 2 = the 16-row engine's
// loader (d = 256, one wave).  Returns 0 on success.
extern "C" int uap_gather(int path, int waves, int fp8_to, int head_dim, const void* k, const void* v,
                          const int32_t* block_table, const int32_t* seq_lens, int bt_stride,
                          int block_size_log2, int64_t kv_slot_stride, const int32_t* tiles,
                          int n_tiles, void* out_k, void* out_v, void* stream) {
    if (n_tiles <= 0) return 0;
    ProbeArgs a{k, v, block_table, seq_lens, tiles, static_cast<unsigned short*>(out_k),
                static_cast<unsigned short*>(out_v), kv_slot_stride, bt_stride, block_size_log2};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (path == 2) {
        // the 16-row engine's loader (d = 256 only)
        if (head_dim != 256) return -1;
        if (fp8_to == 0) e = launch16<__bf16, false>(a, n_tiles, st);
        else if (fp8_to == 1) e = launch16<__bf16, true>(a, n_tiles, st);
        else e = launch16<_Float16, true>(a, n_tiles, st);
        return e == hipSuccess ? 0 : (int)e;
    }
    switch (head_dim) {
        case 64: e = launch<64>(path, waves, fp8_to, a, n_tiles, st); break;
        case 128: e = launch<128>(path, waves, fp8_to, a, n_tiles, st); break;
        case 256: e = launch<256>(path, waves, fp8_to, a, n_tiles, st); break;
        default: return -1;
    }
    return e == hipSuccess ? 0 : (int)e;
}

// 64 element offsets (multiples of 4 below 4093) -> out[64][4].  Returns 0 on success.
extern "C" int uap_read_tr(const int32_t* addr, void* out, void* stream) {
    hipLaunchKernelGGL(probe_read_tr, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), addr,
                       static_cast<unsigned short*>(out));
    return (int)hipGetLastError();
}

// the 256 e4m3 codes -> out_bf16[256], out_f16[256].  Returns 0 on success.
extern "C" int uap_fp8_codes(void* out_bf16, void* out_f16, void* stream) {
    hipLaunchKernelGGL(probe_fp8_codes, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<unsigned short*>(out_bf16), static_cast<unsigned short*>(out_f16));
    return (int)hipGetLastError();
}

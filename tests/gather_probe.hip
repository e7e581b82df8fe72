// Test-only probe of the K/V tile gathers.  Each workgroup runs the kernels'
// own gather routines (the LDS ring's copies, or the register-staged
// KvLoader) for one (sequence, kv-head, tile), then copies the LDS tile out
// to a dense [tile][32 keys][d] buffer of 16-bit elements, undoing the ring's
// chunk permutation or the register path's padding.  The test compares those
// bytes with a host gather of the same keys, bit for bit.  Nothing else in
// the build calls this library.
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

// path 0 = LDS ring (16-bit, block size >= 1024 / (2 d)); path 1 =
// register-staged gather with `waves` waves.  Returns 0 on success.
extern "C" int uap_gather(int path, int waves, int fp8_to, int head_dim, const void* k, const void* v,
                          const int32_t* block_table, const int32_t* seq_lens, int bt_stride,
                          int block_size_log2, int64_t kv_slot_stride, const int32_t* tiles,
                          int n_tiles, void* out_k, void* out_v, void* stream) {
    if (n_tiles <= 0) return 0;
    ProbeArgs a{k, v, block_table, seq_lens, tiles, static_cast<unsigned short*>(out_k),
                static_cast<unsigned short*>(out_v), kv_slot_stride, bt_stride, block_size_log2};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (head_dim) {
        case 64: e = launch<64>(path, waves, fp8_to, a, n_tiles, st); break;
        case 128: e = launch<128>(path, waves, fp8_to, a, n_tiles, st); break;
        case 256: e = launch<256>(path, waves, fp8_to, a, n_tiles, st); break;
        default: return -1;
    }
    return e == hipSuccess ? 0 : (int)e;
}

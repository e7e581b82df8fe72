// Test-only probes of what the hardware delivers to kernels shaped like the
// library's, without the library's math: the ceilings its roofline fractions
// are read against.
//
//  * uac_stream_read: a read-only stream over one buffer: each wave reads
//    eight consecutive 1 KB runs per pass (16-byte loads, eight in flight
//    per lane), passes striding over the buffer.
//  * uac_paged_read: the decode kernel's memory traffic alone.  A workgroup
//    of eight waves (one per kv head) walks a contiguous run of the batch's
//    flattened (sequence, 32-key tile) list, as the stream-K workers do; per
//    tile a wave loads the tile's K and V rows of its head through the block
//    table (one load instruction covers four 256-byte rows, 16 loads in
//    flight per lane) and folds them into a checksum: no LDS, no math.
//  * uac_issue_rate: cycles per wave64 instruction of v_fma_f32, v_exp_f32
//    and the two interleaved, from the shader clock of one wave per workgroup
//    (sixteen independent chains, so latency does not limit the issue, and
//    128 of them per loop pass, so the loop's own instructions do not).
//
// Nothing else in the build calls this library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// one 16-byte load, plain or non-temporal (the nt hint: streamed once, do not keep)
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, int64_t n_vec,
                                                   uint32_t* __restrict__ out) {
    // each wave reads 8 consecutive 1 KB runs per pass (8 loads in flight per
    // lane), passes striding over the buffer
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    uint32_t acc = 0;
    int64_t base = wave * U * 64;
    for (; base + U * 64 <= n_vec; base += n_waves * U * 64) {
        u32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = load16<NT>(src + base + j * 64 + lane);
#pragma unroll
        for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (int64_t i = base + lane; i < n_vec && i < base + U * 64; i += 64) {
        const u32x4 a = load16<NT>(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

struct PagedArgs {
    const unsigned char* k;
    const unsigned char* v;
    const int32_t* block_table;  // [num_seqs][bt_stride]
    const int32_t* seq_lens;     // [num_seqs]
    const int32_t* tile_seq;     // flattened tiles: sequence of tile x
    const int32_t* tile_idx;     //                  tile index within it
    int64_t n_tiles;
    int bt_stride;
    int block_size_log2;
    int num_kv_heads;            // = waves per workgroup
    uint32_t* out;               // one word per lane
};

// d = 128, 16-bit K/V: a key row of one head is 256 bytes (16 chunks of 16)
template <bool NT>
__global__ __launch_bounds__(512) void paged_read(PagedArgs a) {
    const int lane = threadIdx.x & 63;
    const int head = threadIdx.x >> 6;
    const int64_t w = blockIdx.x, nw = gridDim.x;
    const int64_t x0 = w * a.n_tiles / nw, x1 = (w + 1) * a.n_tiles / nw;
    const int64_t slot_bytes = (int64_t)a.num_kv_heads * 128 * 2;
    const int chunk = lane & 15, row0 = lane >> 4;
    uint32_t acc = 0;
    for (int64_t x = x0; x < x1; ++x) {
        const int s = a.tile_seq[x];
        const int t = a.tile_idx[x];
        const int s_k = a.seq_lens[s];
        const int32_t* bt = a.block_table + (int64_t)s * a.bt_stride;
        u32x4 kv[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = min(t * 32 + row0 + 4 * i, s_k - 1);  // past S_k: reread the last key
            const int64_t slot = ((int64_t)bt[key >> a.block_size_log2] << a.block_size_log2) +
                                 (key & ((1 << a.block_size_log2) - 1));
            const int64_t off = slot * slot_bytes + (int64_t)head * 256 + chunk * 16;
            kv[i] = load16<NT>(reinterpret_cast<const u32x4*>(a.k + off));
            kv[8 + i] = load16<NT>(reinterpret_cast<const u32x4*>(a.v + off));
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc ^= kv[i].x ^ kv[i].y ^ kv[i].z ^ kv[i].w;
    }
    a.out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// 16 independent chains of KIND (0: v_fma_f32, 1: v_exp_f32, 2: both in
// turn), eight rounds per loop pass, `iters` passes; out: [wave] shader-clock
// cycles, [wave] 100 MHz real-time ticks, and a value that keeps the chains
// live
template <int KIND>
__device__ __forceinline__ void round16(float (&x)[16], float m, float c) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (KIND == 0 || (KIND == 2 && (j & 1) == 0))
            asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[j]) : "v"(m), "v"(c));
        else
            asm volatile("v_exp_f32 %0, %0" : "+v"(x[j]));
    }
}

template <int KIND>
__global__ __launch_bounds__(64) void issue_rate(int iters, uint64_t* cycles, uint64_t* ticks,
                                                 float* sink) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 0.25f + 0.01f * (threadIdx.x + j);
    const float m = 0.999f, c = 1.0e-3f;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r) round16<KIND>(x, m, c);
    }
    const uint64_t c1 = __builtin_readcyclecounter();
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
    sink[(int64_t)blockIdx.x * 64 + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        cycles[blockIdx.x] = c1 - c0;
        ticks[blockIdx.x] = t1 - t0;
    }
}

}  // namespace

// Read n_bytes (a multiple of 16) of src with `blocks` workgroups of 256
// threads (nt: non-temporal loads); out holds blocks * 256 words.  Returns 0
// or the HIP error.
extern "C" int uac_stream_read(const void* src, int64_t n_bytes, int blocks, int nt, void* out,
                               void* stream) {
    if (n_bytes % 16 || blocks < 1) return -1;
    hipLaunchKernelGGL(nt ? stream_read<true> : stream_read<false>, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n_bytes / 16,
                       static_cast<uint32_t*>(out));
    return (int)hipGetLastError();
}

// The decode-shaped paged read: `workers` workgroups of num_kv_heads waves
// (nt: non-temporal loads); out holds workers * 64 * num_kv_heads words.
// d = 128, 16-bit K/V.
extern "C" int uac_paged_read(const void* k, const void* v, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* tile_seq,
                              const int32_t* tile_idx, int64_t n_tiles, int bt_stride,
                              int block_size_log2, int num_kv_heads, int workers, int nt,
                              void* out, void* stream) {
    if (num_kv_heads < 1 || num_kv_heads > 8 || workers < 1 || n_tiles < 0) return -1;
    PagedArgs a{static_cast<const unsigned char*>(k), static_cast<const unsigned char*>(v),
                block_table, seq_lens, tile_seq, tile_idx, n_tiles, bt_stride, block_size_log2,
                num_kv_heads, static_cast<uint32_t*>(out)};
    hipLaunchKernelGGL(nt ? paged_read<true> : paged_read<false>, dim3(workers), dim3(64 * num_kv_heads), 0,
                       static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

// `waves` one-wave workgroups; cycles and ticks hold `waves` entries, sink
// waves * 64 floats.
extern "C" int uac_issue_rate(int kind, int iters, int waves, void* cycles, void* ticks, void* sink,
                              void* stream) {
    if (kind < 0 || kind > 2 || iters < 1 || waves < 1) return -1;
    auto kern = kind == 0 ? issue_rate<0> : kind == 1 ? issue_rate<1> : issue_rate<2>;
    hipLaunchKernelGGL(kern, dim3(waves), dim3(64), 0, static_cast<hipStream_t>(stream), iters,
                       static_cast<uint64_t*>(cycles), static_cast<uint64_t*>(ticks),
                       static_cast<float*>(sink));
    return (int)hipGetLastError();
}

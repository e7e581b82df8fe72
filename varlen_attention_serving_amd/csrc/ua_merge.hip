// ua_merge.hip -- combine caller-held partial attention states into O.
//
// Attention over the union of disjoint key sets, from each set's result over
// its own keys: the associative log-sum-exp re-base of section 5 of "Unified
// paged attention on gfx950, from the math up", here on merge-ready states.
// Set i gives, per row, v_i = (sum of p v) / (sum of p) over its keys and
// lse_i = ln(sum of e^s) over them (-inf when it saw none).  With the optional
// per-head sink logit (one more softmax column with no value row, joined
// exactly once here):
//     LSE = ln( sum_i e^{lse_i} + e^{sink} ),   O = sum_i v_i e^{lse_i - LSE},
// computed in base 2 against the largest term.  A row whose sets are all
// empty and that has no sink gets O = 0 and LSE = -inf.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ua.h"
#include "ua_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// N consecutive values of a partial row as one vector load (elem is a
// multiple of N; the sets are 16-byte aligned).
template <int N, bool BF16>
__device__ __forceinline__ void load_part(const void* base, int64_t elem, float (&out)[N]) {
    typedef typename std::conditional<BF16, __bf16, float>::type T;
    typedef T v __attribute__((ext_vector_type(N)));
    const v x = *reinterpret_cast<const v*>(static_cast<const T*>(base) + elem);
#pragma unroll
    for (int e = 0; e < N; ++e) out[e] = (float)x[e];
}

// One wave per (token, head) row, four rows per workgroup; lane l owns
// elements [l D / 64, (l + 1) D / 64) of the row.
template <int D, typename OT, bool BF16>
__global__ __launch_bounds__(256) void ua_merge_kernel(UaMergeParams p) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.rows) return;
    const int64_t tok = row / p.num_q_heads;
    const int head = (int)(row - tok * p.num_q_heads);

    float s[kMaxMergeSets];
    float mx = p.sinks ? p.sinks[head] * kLog2e : -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxMergeSets; ++i) {
        s[i] = i < p.num_sets ? p.lse[i][row] * kLog2e : -INFINITY;
        mx = fmaxf(mx, s[i]);
    }
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    float L = 0.0f;
    if (mx != -INFINITY) {
        if (p.sinks) L = __builtin_amdgcn_exp2f(p.sinks[head] * kLog2e - mx);
#pragma unroll
        for (int i = 0; i < kMaxMergeSets; ++i) {
            if (i >= p.num_sets || s[i] == -INFINITY) continue;  // an empty set adds nothing
            const float w = __builtin_amdgcn_exp2f(s[i] - mx);
            L += w;
            float v[EPL];
            load_part<EPL, BF16>(p.o[i], row * D + lane * EPL, v);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] += w * v[e];
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    OT* dst = static_cast<OT*>(p.out) + tok * p.out_stride_tok + (int64_t)head * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = (OT)(acc[e] * inv);
    if (p.out_lse && lane == 0)
        p.out_lse[row] = L > 0.0f ? (mx + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

template <int D, typename OT>
hipError_t launch_merge_t(const UaMergeParams& p, hipStream_t st) {
    const unsigned nb = (unsigned)((p.rows + 3) / 4);
    if (p.part_bf16)
        hipLaunchKernelGGL((ua_merge_kernel<D, OT, true>), dim3(nb), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((ua_merge_kernel<D, OT, false>), dim3(nb), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_merge_d(const UaMergeParams& p, hipStream_t st) {
    return p.out_dtype == UA_DTYPE_BF16 ? launch_merge_t<D, __bf16>(p, st)
                                        : launch_merge_t<D, _Float16>(p, st);
}

}  // namespace

hipError_t ua_launch_merge(const UaMergeParams& p, hipStream_t st) {
    if (p.rows <= 0) return hipSuccess;
    switch (p.head_dim) {
        case 64: return launch_merge_d<64>(p, st);
        case 128: return launch_merge_d<128>(p, st);
        case 256: return launch_merge_d<256>(p, st);
        default: return hipErrorInvalidValue;
    }
}

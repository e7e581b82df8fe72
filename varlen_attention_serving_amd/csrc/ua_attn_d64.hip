// Kernel instantiations for head_dim 64 (bf16/f16 Q; 16-bit or e4m3 K/V; 2D and 3D paths).
#include "ua_attn_impl.h"

hipError_t ua_launch_d64(const UaKernelParams& p, const UaLaunch& l, hipStream_t s) {
    return ua::launch_head_dim<64>(p, l, s);
}

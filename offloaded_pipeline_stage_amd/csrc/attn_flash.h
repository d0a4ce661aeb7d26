// MFMA flash-attention kernels (bf16, head_dim 128).
#pragma once

#include "ops.h"

namespace rp {

// whether the flash kernels cover this shape
bool flash_supported(const AttnDesc& a);
rp_status flash_fwd(const AttnDesc& a, const void* qkv, void* o, float* lse, hipStream_t s);
// rope_inv: a RoPE table ((cos, sin) of position p and pair i at
// [64 p + i]) that dQ and dK are taken back through before they are stored,
// or null
rp_status flash_bwd(const AttnDesc& a, const void* qkv, const void* o, const void* dout,
                    const float* lse, float* Dbuf, void* dqkv, hipStream_t s, const float2* rope_inv = nullptr);
}  // namespace rp

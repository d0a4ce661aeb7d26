// MFMA flash attention for bf16, head_dim 128 (forward and backward).
#include "attn_flash.h"

namespace rp {

namespace {
bool g_flash_on = true;
}

void flash_enable(bool on) { g_flash_on = on; }

bool flash_supported(const AttnDesc& a) {
  (void)a;
  return false;  // the reference-grade kernels in attn.hip cover every shape until these land
}

rp_status flash_fwd(const AttnDesc&, const void*, void*, float*, hipStream_t) {
  set_error("flash attention forward not available");
  return RP_ERR_UNSUPPORTED;
}

rp_status flash_bwd(const AttnDesc&, const void*, const void*, const void*, const float*, float*, void*,
                    hipStream_t) {
  set_error("flash attention backward not available");
  return RP_ERR_UNSUPPORTED;
}

}  // namespace rp

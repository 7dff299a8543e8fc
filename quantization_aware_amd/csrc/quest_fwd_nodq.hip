// Forward quantisation with no dequantised output, for bf16 and fp32 inputs.
#include "quest_kernels.h"

namespace quest {

hipError_t launch_fwd_nodq(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a) {
  if (x_is_bf16) return fwd_dispatch_block<uint16_t, void>(static_cast<const uint16_t*>(x), log_block, bits, a);
  return fwd_dispatch_block<float, void>(static_cast<const float*>(x), log_block, bits, a);
}

}  // namespace quest

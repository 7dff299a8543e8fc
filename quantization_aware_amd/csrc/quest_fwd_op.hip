// Forward quantisation writing the matrix-core operand (FP6 E2M3, tiled) in
// place of a dequantised output, for bf16 and fp32 inputs.
#include "quest_kernels.h"

namespace quest {

hipError_t launch_fwd_op(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a) {
  if (x_is_bf16) return fwd_dispatch_block<uint16_t, OperandOut>(static_cast<const uint16_t*>(x), log_block, bits, a);
  return fwd_dispatch_block<float, OperandOut>(static_cast<const float*>(x), log_block, bits, a);
}

}  // namespace quest

// Launch entry points behind the C ABI: the forward router (one translation
// unit per dequantised-output type), the trust backward and dequantisation.
#include "quest_kernels.h"

namespace quest {

hipError_t launch_quantize_fwd(const void* x, int x_is_bf16, int log_block, int bits, int dq_kind,
                               const FwdLaunch& a) {
  switch (dq_kind) {
    case 1: return launch_fwd_dq_bf16(x, x_is_bf16, log_block, bits, a);
    case 2: return launch_fwd_dq_f32(x, x_is_bf16, log_block, bits, a);
    case 3: return launch_fwd_op(x, x_is_bf16, log_block, bits, a);
    default: return launch_fwd_nodq(x, x_is_bf16, log_block, bits, a);
  }
}

hipError_t launch_dequantize(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int bits,
                             void* out, int out_is_bf16, hipStream_t stream) {
  if (out_is_bf16) return dequant_dispatch(codes, scale, rows, cols, bits, static_cast<uint16_t*>(out), stream);
  return dequant_dispatch(codes, scale, rows, cols, bits, static_cast<float*>(out), stream);
}

hipError_t launch_codes_to_operand(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint8_t* operand,
                                   hipStream_t stream) {
  switch (bits) {
    case 1: return codes_to_operand_launch<1>(codes, rows, cols, operand, stream);
    case 2: return codes_to_operand_launch<2>(codes, rows, cols, operand, stream);
    case 3: return codes_to_operand_launch<3>(codes, rows, cols, operand, stream);
    default: return codes_to_operand_launch<4>(codes, rows, cols, operand, stream);
  }
}

hipError_t launch_trust_bwd(const void* grad, int g_is_bf16, const uint8_t* mask, int64_t rows, int64_t cols,
                            int log_block, void* grad_out, bool allow_mfma, hipStream_t stream) {
  if (g_is_bf16)
    return bwd_dispatch(static_cast<const uint16_t*>(grad), mask, rows, cols, log_block,
                        static_cast<uint16_t*>(grad_out), allow_mfma, stream);
  return bwd_dispatch(static_cast<const float*>(grad), mask, rows, cols, log_block, static_cast<float*>(grad_out),
                      false, stream);
}

}  // namespace quest

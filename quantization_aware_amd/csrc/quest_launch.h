// Internal launch entry points of libquest (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quest {

// x_is_bf16: 1 = bf16 input, 0 = fp32.  allow_mfma: bf16 rows of 16 m runs
// use the matrix-core transform.  codes may be null (not written).  dq_kind:
// 0 = no dequantised output, 1 = bf16, 2 = fp32 into dq.  All sizes already
// validated.
hipError_t launch_quantize_fwd(const void* x, int x_is_bf16, int64_t rows, int64_t cols, int log_block, int bits,
                               double alpha, bool allow_mfma, uint8_t* codes, float* scale, uint8_t* mask, void* dq,
                               int dq_kind, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int bits,
                             void* out, int out_is_bf16, hipStream_t stream);

hipError_t launch_trust_bwd(const void* grad, int g_is_bf16, const uint8_t* mask, int64_t rows, int64_t cols,
                            int log_block, void* grad_out, hipStream_t stream);

}  // namespace quest

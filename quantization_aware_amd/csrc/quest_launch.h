// Internal launch entry points of libquest (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quest {

// Arguments of one forward launch, already validated.
struct FwdLaunch {
  int64_t rows, cols;
  double alpha;     // clip scale alpha_b
  double trust;     // outer trust factor: trusted iff |y| <= s + trust * Delta / 2
  bool allow_mfma;  // bf16 rows of 16 m runs (b <= 4) use the matrix-core transform
  uint8_t* codes;   // may be null: codes are not written
  float* scale;
  uint8_t* mask;
  void* dq;  // dequantised output (type given by dq_kind), or null
  hipStream_t stream;
};

// x_is_bf16: 1 = bf16 input, 0 = fp32.  dq_kind: 0 = no dequantised output,
// 1 = bf16, 2 = fp32 into a.dq, 3 = the matrix-core operand into a.dq
// (bits <= 4, cols a multiple of 128).  All sizes already validated.
hipError_t launch_quantize_fwd(const void* x, int x_is_bf16, int log_block, int bits, int dq_kind,
                               const FwdLaunch& a);

// The forward for one dequantised-output type (separate translation units).
hipError_t launch_fwd_nodq(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a);
hipError_t launch_fwd_dq_bf16(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a);
hipError_t launch_fwd_dq_f32(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a);
hipError_t launch_fwd_op(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a);

// One tensor of a grouped forward (quest_quantize_fwd_group).
struct FwdGroupItem {
  const void* x;  // bf16
  int64_t rows;
  int64_t cols;
  uint8_t* codes;
  float* scale;
  uint8_t* mask;
};

// Whether a bf16 tensor of `cols` entries per row (bits <= 4) takes the
// grouped launch: as a tile tensor (512, 1024, 2048) or as a wide one (a
// multiple of 512 from 2560 to 8192).
inline bool fwd_group_tile_cols(int64_t cols) { return cols == 512 || cols == 1024 || cols == 2048; }
inline bool fwd_group_wide_cols(int64_t cols) { return cols > 2048 && cols <= 8192 && cols % 512 == 0; }

// The forward (trust 1) of bf16 tensors, bits <= 4: `count` tile tensors
// whose rows all have `cols` entries (512, 1024 or 2048) and `wide_count`
// wide tensors, in launches of at most eight tile and four wide tensors;
// rows >= 1 for every item.  All arguments already validated.
hipError_t launch_fwd_group(const FwdGroupItem* items, int count, int64_t cols, const FwdGroupItem* wide,
                            int wide_count, int log_block, int bits, double alpha, hipStream_t stream);

// One tensor of a grouped operand forward (quest_quantize_fwd_op_group).
struct FwdOpGroupItem {
  const void* x;  // bf16
  int64_t rows;   // >= 1
  uint8_t* codes;  // may be null
  float* scale;
  uint8_t* mask;  // may be null
  uint8_t* operand;
};

// Operand forwards of bf16 tensors (bits <= 4) whose rows all have `cols`
// entries, 512, 1024 or 2048, in launches of at most four tensors.  All
// arguments already validated.
hipError_t launch_fwd_op_group(const FwdOpGroupItem* items, int count, int64_t cols, int log_block, int bits,
                               double alpha, double trust, hipStream_t stream);

// Packed codes (bits <= 4, cols a multiple of 128) to the tiled FP6 operand.
hipError_t launch_codes_to_operand(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint8_t* operand,
                                   hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int bits,
                             void* out, int out_is_bf16, hipStream_t stream);

// allow_mfma: bf16 gradients use the matrix-core transform (fp32 ones always
// the vector-ALU one).
hipError_t launch_trust_bwd(const void* grad, int g_is_bf16, const uint8_t* mask, int64_t rows, int64_t cols,
                            int log_block, void* grad_out, bool allow_mfma, hipStream_t stream);

// Arguments of one product of two matrix-core operands, already validated:
// out (m x n, row-major) = Delta_a Delta_b * (A B^T) with Delta = scale * k*.
struct GemmLaunch {
  const uint8_t* a;  // tiled E2M3 operand, m rows
  const float* sa;   // clip scale per row of a
  int m;
  const uint8_t* b;  // tiled E2M3 operand, n rows
  const float* sb;
  int n;
  int k;     // a multiple of 128
  float ka;  // 2 / (L_a - 1)
  float kb;  // 2 / (L_b - 1)
  void* out;
  hipStream_t stream;
};

hipError_t launch_gemm_e2m3(const GemmLaunch& g, bool out_bf16);

// Arguments of one forward onto the FP4 grid (sparse24 = 0) or the 2:4-sparse
// b-bit grid (sparse24 = 1), already validated.
struct GridLaunch {
  int64_t rows, cols;
  double alpha, trust;
  int bits, sparse24;
  bool allow_mfma;  // bf16 rows of 512, 1024 or 2048 columns: the matrix-core kernels
  uint8_t* codes;  // may be null
  uint8_t* index;  // 2:4 positions, may be null
  float* scale;
  uint8_t* mask;
  void* dq;  // dequantised output or null
  hipStream_t stream;
};

hipError_t launch_fwd_grid(const void* x, int x_is_bf16, int log_block, int dq_kind, const GridLaunch& a);
hipError_t launch_dequantize_fp4(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, void* out,
                                 int out_is_bf16, hipStream_t stream);
hipError_t launch_dequantize_sparse24(const uint8_t* codes, const uint8_t* index, const float* scale, int64_t rows,
                                      int64_t cols, int bits, void* out, int out_is_bf16, hipStream_t stream);

}  // namespace quest

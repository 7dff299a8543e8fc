// Forward quantisation writing the matrix-core operand (FP6 E2M3, tiled) in
// place of a dequantised output, for bf16 and fp32 inputs, and the grouped
// operand forward of several bf16 tensors.
#include "quest_kernels.h"

namespace quest {

hipError_t launch_fwd_op(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a) {
  if (x_is_bf16) return fwd_dispatch_block<uint16_t, OperandOut>(static_cast<const uint16_t*>(x), log_block, bits, a);
  return fwd_dispatch_block<float, OperandOut>(static_cast<const float*>(x), log_block, bits, a);
}

namespace {

template <int LOGN>
hipError_t op_group_bits(const FwdOpGroup& g, int64_t cols, int bits, double alpha, double trust, bool quant,
                         hipStream_t stream) {
  switch (bits) {
    case 1: return fwd_op_group_dispatch<LOGN, 1>(g, cols, alpha, trust, quant, stream);
    case 2: return fwd_op_group_dispatch<LOGN, 2>(g, cols, alpha, trust, quant, stream);
    case 3: return fwd_op_group_dispatch<LOGN, 3>(g, cols, alpha, trust, quant, stream);
    default: return fwd_op_group_dispatch<LOGN, 4>(g, cols, alpha, trust, quant, stream);
  }
}

}  // namespace

hipError_t launch_fwd_op_group(const FwdOpGroupItem* items, int count, int64_t cols, int log_block, int bits,
                               double alpha, double trust, hipStream_t stream) {
  const int64_t runs_per_row = cols / RUN;
  for (int first = 0; first < count;) {
    FwdOpGroup g = {};
    g.count = count - first < kFwdOpGroupMax ? count - first : kFwdOpGroupMax;
    int64_t wgs = 0;
    bool quant = false;
    for (int i = 0; i < g.count; ++i) {
      const FwdOpGroupItem& it = items[first + i];
      g.first_wg[i] = wgs;
      g.total_runs[i] = it.rows * runs_per_row;
      g.x[i] = static_cast<const uint16_t*>(it.x);
      g.codes[i] = it.codes;
      g.scale[i] = it.scale;
      g.mask[i] = reinterpret_cast<uint32_t*>(it.mask);
      g.operand[i] = it.operand;
      quant = quant || it.codes || it.mask;
      wgs += ((g.total_runs[i] + 63) / 64 + 3) / 4;  // four 64-run tiles per workgroup
    }
    g.first_wg[g.count] = wgs;
    first += g.count;
    hipError_t e;
    switch (log_block) {
      case 6: e = op_group_bits<6>(g, cols, bits, alpha, trust, quant, stream); break;
      case 7: e = op_group_bits<7>(g, cols, bits, alpha, trust, quant, stream); break;
      default: e = op_group_bits<8>(g, cols, bits, alpha, trust, quant, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace quest

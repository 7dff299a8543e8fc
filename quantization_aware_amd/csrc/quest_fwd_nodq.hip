// Forward quantisation with no dequantised output, for bf16 and fp32 inputs,
// and the grouped forward of several bf16 tensors.
#include "quest_kernels.h"

namespace quest {

hipError_t launch_fwd_nodq(const void* x, int x_is_bf16, int log_block, int bits, const FwdLaunch& a) {
  if (x_is_bf16) return fwd_dispatch_block<uint16_t, void>(static_cast<const uint16_t*>(x), log_block, bits, a);
  return fwd_dispatch_block<float, void>(static_cast<const float*>(x), log_block, bits, a);
}

namespace {

template <int LOGN>
hipError_t group_bits(const FwdGroup& g, int64_t cols, int bits, double alpha, hipStream_t stream) {
  switch (bits) {
    case 1: return fwd_group_dispatch<LOGN, 1>(g, cols, alpha, stream);
    case 2: return fwd_group_dispatch<LOGN, 2>(g, cols, alpha, stream);
    case 3: return fwd_group_dispatch<LOGN, 3>(g, cols, alpha, stream);
    default: return fwd_group_dispatch<LOGN, 4>(g, cols, alpha, stream);
  }
}

}  // namespace

hipError_t launch_fwd_group(const FwdGroupItem* items, int count, int64_t cols, const FwdGroupItem* wide,
                            int wide_count, int log_block, int bits, double alpha, hipStream_t stream) {
  const int64_t runs_per_row = cols / RUN;
  int first = 0, wfirst = 0;
  while (first < count || wfirst < wide_count) {
    FwdGroup g = {};
    g.count = count - first < kFwdGroupMax ? count - first : kFwdGroupMax;
    int64_t tiles = 0;
    for (int i = 0; i < g.count; ++i) {
      const FwdGroupItem& it = items[first + i];
      g.first_tile[i] = tiles;
      g.total_runs[i] = it.rows * runs_per_row;
      g.x[i] = static_cast<const uint16_t*>(it.x);
      g.codes[i] = it.codes;
      g.scale[i] = it.scale;
      g.mask[i] = reinterpret_cast<uint32_t*>(it.mask);
      tiles += (g.total_runs[i] + 63) / 64;
    }
    g.first_tile[g.count] = tiles;
    g.wide_count = wide_count - wfirst < kFwdGroupWideMax ? wide_count - wfirst : kFwdGroupWideMax;
    int64_t wrows = 0;
    for (int i = 0; i < g.wide_count; ++i) {
      const FwdGroupItem& it = wide[wfirst + i];
      g.wide_first_row[i] = wrows;
      g.wide_runs[i] = static_cast<int>(it.cols / RUN);
      g.wide_inv_cols[i] = static_cast<float>(1.0 / double(it.cols));
      g.wide_x[i] = static_cast<const uint16_t*>(it.x);
      g.wide_codes[i] = it.codes;
      g.wide_scale[i] = it.scale;
      g.wide_mask[i] = reinterpret_cast<uint32_t*>(it.mask);
      wrows += it.rows;
    }
    g.wide_first_row[g.wide_count] = wrows;
    first += g.count;
    wfirst += g.wide_count;
    hipError_t e;
    switch (log_block) {
      case 6: e = group_bits<6>(g, cols, bits, alpha, stream); break;
      case 7: e = group_bits<7>(g, cols, bits, alpha, stream); break;
      default: e = group_bits<8>(g, cols, bits, alpha, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace quest

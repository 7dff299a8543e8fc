// C ABI of libquest: argument checks, the clip-scale table and dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <cstdint>
#include <limits>
#include <mutex>
#include <vector>

#include "../../include/quest.h"
#include "quest_launch.h"

namespace {

// ----------------------------------------------------------------------------
// alpha_b: the clip scale of the b-bit grid that minimises the expected
// squared error for a standard Gaussian (pith.science review of QuEST, "What
// carries the argument" and "Assumptions & free parameters").
//
// With levels c_k alpha, c_k = (2k - L + 1)/(L - 1), and cells bounded by the
// midpoints of neighbouring levels, let
//   F(alpha) = sum_k c_k E[X; cell k] / sum_k c_k^2 P(cell k),
// E[X; [a, c)] = phi(a) - phi(c),  P([a, c)) = Phi(c) - Phi(a): the
// least-squares alpha for the cells that alpha itself defines.  The error's
// derivative is dMSE/d alpha = -2 (sum_k c_k^2 P_k) (F(alpha) - alpha), so
// F(alpha) - alpha is positive below the optimum and negative above it.
// Bisection on that sign over [0.01, 32] pins alpha_b to the last bit.
// ----------------------------------------------------------------------------
double gauss_pdf(double t) {
  if (std::isinf(t)) return 0.0;
  return std::exp(-0.5 * t * t) * 0.39894228040143267793994605993438;
}

double gauss_cdf(double t) {
  if (t == std::numeric_limits<double>::infinity()) return 1.0;
  if (t == -std::numeric_limits<double>::infinity()) return 0.0;
  return 0.5 * std::erfc(-t * 0.70710678118654752440084436210485);
}

double alpha_update(double alpha, int b) {
  const int levels = 1 << b;
  double num = 0.0, den = 0.0;
  for (int k = 0; k < levels; ++k) {
    const double ck = double(2 * k - levels + 1) / double(levels - 1);
    const double lo = (k == 0) ? -std::numeric_limits<double>::infinity()
                               : double(2 * k - levels) * alpha / double(levels - 1);
    const double hi = (k == levels - 1) ? std::numeric_limits<double>::infinity()
                                        : double(2 * k + 2 - levels) * alpha / double(levels - 1);
    num += ck * (gauss_pdf(lo) - gauss_pdf(hi));
    den += ck * ck * (gauss_cdf(hi) - gauss_cdf(lo));
  }
  return num / den;
}

double solve_alpha(int b) {
  double lo = 0.01, hi = 32.0;
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (alpha_update(mid, b) > mid)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

// The same least-squares fixed point for an arbitrary symmetric level set
// (levels c_k alpha with the largest c_k = 1): used for the FP4 grid, whose
// E2M1 magnitudes over 6 are 0, 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1.
constexpr double kFp4Unit[15] = {-1.0,      -4.0 / 6.0, -3.0 / 6.0, -2.0 / 6.0, -1.5 / 6.0, -1.0 / 6.0,
                                 -0.5 / 6.0, 0.0,       0.5 / 6.0,  1.0 / 6.0,  1.5 / 6.0,  2.0 / 6.0,
                                 3.0 / 6.0,  4.0 / 6.0, 1.0};

double alpha_update_levels(double alpha, const double* unit, int n) {
  double num = 0.0, den = 0.0;
  for (int k = 0; k < n; ++k) {
    const double lo = k == 0 ? -std::numeric_limits<double>::infinity() : 0.5 * (unit[k - 1] + unit[k]) * alpha;
    const double hi = k == n - 1 ? std::numeric_limits<double>::infinity() : 0.5 * (unit[k] + unit[k + 1]) * alpha;
    num += unit[k] * (gauss_pdf(lo) - gauss_pdf(hi));
    den += unit[k] * unit[k] * (gauss_cdf(hi) - gauss_cdf(lo));
  }
  return num / den;
}

double solve_alpha_fp4() {
  double lo = 0.01, hi = 32.0;
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (alpha_update_levels(mid, kFp4Unit, 15) > mid)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

constexpr int kMaxBits = 8;
double g_alpha[kMaxBits + 1];
double g_alpha_fp4 = 0.0;
std::once_flag g_alpha_once;

void fill_alpha_table() {
  for (int b = 1; b <= kMaxBits; ++b) g_alpha[b] = solve_alpha(b);
  g_alpha_fp4 = solve_alpha_fp4();
}

// Kernel selection, read once per process: QUEST_FWD_KERNEL=valu keeps bf16
// forwards of 512 or more columns, QUEST_BWD_KERNEL=valu bf16 backwards, on
// the vector-ALU transform instead of the matrix cores (same results up to
// fp32 rounding order; for A/B timing).
std::once_flag g_env_once;
bool g_allow_mfma = true;
bool g_allow_mfma_bwd = true;

bool env_is(const char* name, const char* value) {
  const char* v = std::getenv(name);
  return v && std::strcmp(v, value) == 0;
}

void read_env() {
  g_allow_mfma = !env_is("QUEST_FWD_KERNEL", "valu");
  g_allow_mfma_bwd = !env_is("QUEST_BWD_KERNEL", "valu");
}

// ----------------------------------------------------------------------------
// Argument checks.
// ----------------------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

int log2_block(int block) {
  switch (block) {
    case 64: return 6;
    case 128: return 7;
    case 256: return 8;
    default: return -1;
  }
}

size_t dtype_size(quest_dtype d) { return d == QUEST_BF16 ? 2 : 4; }

bool dtype_ok(quest_dtype d) { return d == QUEST_F32 || d == QUEST_BF16; }

// rows * cols must stay below 2^36 so that the number of 32-element runs fits
// in 31 bits.
constexpr int64_t kMaxElements = int64_t(1) << 36;

quest_status check_shape(int64_t rows, int64_t cols, int multiple_of) {
  if (rows < 0 || cols <= 0 || cols % multiple_of != 0) return QUEST_EINVAL;
  if (cols > QUEST_MAX_COLS) return QUEST_EUNSUPPORTED;
  if (rows > kMaxElements / cols) return QUEST_EUNSUPPORTED;
  return QUEST_OK;
}

quest_status from_hip(hipError_t e) { return e == hipSuccess ? QUEST_OK : QUEST_EHIP; }

// The argument checks of quantize_fwd_common, without the launch.
quest_status check_fwd(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b, double trust,
                       uint8_t* codes, bool codes_required, float* scale, uint8_t* mask, bool mask_required, void* dq,
                       quest_dtype dq_dtype, bool dq_required, uint8_t* operand);
// Forward with codes (null allowed unless codes_required), an optional
// dequantised output (null allowed unless dq_required; dq_dtype is checked
// only when dq is given) and the outer trust factor.  Checks every argument
// before launching.
quest_status quantize_fwd_common(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                 double trust, uint8_t* codes, bool codes_required, float* scale, uint8_t* mask,
                                 bool mask_required, void* dq, quest_dtype dq_dtype, bool dq_required,
                                 uint8_t* operand, void* stream);

// Forward onto the FP4 grid (b == 0) or the 2:4-sparse b-bit grid.  Codes,
// index and dq may be NULL; scale and mask are required.
quest_status quantize_grid_common(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                  double trust, uint8_t* codes, uint8_t* index, float* scale, uint8_t* mask, void* dq,
                                  quest_dtype dq_dtype, void* stream);

// Largest contraction length of quest_gemm: sums of k products of
// half-integers up to 7.5 stay below 2^22 in magnitude, so fp32 accumulates
// them exactly.
constexpr int64_t kGemmMaxK = 65536;
constexpr int64_t kGemmMaxN = int64_t(1) << 20;
constexpr int64_t kGemmMaxM = int64_t(1) << 30;
constexpr int64_t kGemmMaxTiles = (int64_t(1) << 23) - 1;  // 256 x 256 output tiles

}  // namespace

extern "C" {

double quest_fit_alpha(int b) {
  if (b < 1 || b > kMaxBits) return std::numeric_limits<double>::quiet_NaN();
  std::call_once(g_alpha_once, fill_alpha_table);
  return g_alpha[b];
}

size_t quest_codes_bytes(int64_t rows, int64_t cols, int b) {
  if (rows < 0 || cols <= 0 || b < 1 || b > kMaxBits || (cols * b) % 8 != 0) return 0;
  if (rows > kMaxElements / cols) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(cols * b / 8);
}

size_t quest_mask_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return 0;
  if (rows > kMaxElements / cols) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(cols / 8);
}

const char* quest_status_string(quest_status s) {
  switch (s) {
    case QUEST_OK: return "ok";
    case QUEST_EINVAL: return "invalid argument";
    case QUEST_EUNSUPPORTED: return "unsupported block, bit width or size";
    case QUEST_EALIGN: return "buffer not 16-byte aligned";
    case QUEST_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

quest_status quest_quantize_fwd(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                uint8_t* codes, float* scale, uint8_t* mask, void* stream) {
  return quantize_fwd_common(x, x_dtype, rows, cols, block, b, 1.0, codes, true, scale, mask, true, nullptr,
                             QUEST_BF16, false, nullptr, stream);
}

quest_status quest_quantize_fwd_group(const quest_fwd_tensor* tensors, int count, quest_dtype x_dtype, int block,
                                      int b, void* stream) {
  if (count < 0 || (count > 0 && !tensors)) return QUEST_EINVAL;
  // Every tensor as quest_quantize_fwd would check it ...
  for (int i = 0; i < count; ++i) {
    const quest_fwd_tensor& t = tensors[i];
    const quest_status st = check_fwd(t.x, x_dtype, t.rows, t.cols, block, b, 1.0, t.codes, true, t.scale, t.mask,
                                      true, nullptr, QUEST_BF16, false, nullptr);
    if (st != QUEST_OK) return st;
  }
  // ... and no output of one tensor on an input or output of another.
  auto spans = [&](const quest_fwd_tensor& t, size_t (&n)[4]) {
    n[0] = static_cast<size_t>(t.rows * t.cols) * dtype_size(x_dtype);
    n[1] = quest_codes_bytes(t.rows, t.cols, b);
    n[2] = static_cast<size_t>(t.rows) * sizeof(float);
    n[3] = quest_mask_bytes(t.rows, t.cols);
  };
  for (int i = 0; i < count; ++i) {
    if (tensors[i].rows == 0) continue;
    size_t ni[4];
    spans(tensors[i], ni);
    const void* bi[4] = {tensors[i].x, tensors[i].codes, tensors[i].scale, tensors[i].mask};
    for (int j = i + 1; j < count; ++j) {
      if (tensors[j].rows == 0) continue;
      size_t nj[4];
      spans(tensors[j], nj);
      const void* bj[4] = {tensors[j].x, tensors[j].codes, tensors[j].scale, tensors[j].mask};
      for (int p = 0; p < 4; ++p)
        for (int q = 0; q < 4; ++q)
          if ((p > 0 || q > 0) && overlaps(bi[p], ni[p], bj[q], nj[q])) return QUEST_EINVAL;
    }
  }
  std::call_once(g_env_once, read_env);
  const int lb = log2_block(block);
  const double alpha = quest_fit_alpha(b);
  // bf16 tensors with b <= 4 go in grouped launches: rows of 512, 1024 or
  // 2048 entries one launch per width, rows of 2560 to 8192 entries (a
  // multiple of 512) with the first of them (or on their own); everything
  // else as quest_quantize_fwd.
  std::vector<quest::FwdGroupItem> group[3], wide;
  const bool grouped = x_dtype == QUEST_BF16 && b <= 4 && g_allow_mfma;
  for (int i = 0; i < count; ++i) {
    const quest_fwd_tensor& t = tensors[i];
    if (t.rows == 0) continue;
    const quest::FwdGroupItem item = {t.x, t.rows, t.cols, t.codes, t.scale, t.mask};
    if (grouped && quest::fwd_group_tile_cols(t.cols)) {
      group[t.cols == 512 ? 0 : t.cols == 1024 ? 1 : 2].push_back(item);
    } else if (grouped && quest::fwd_group_wide_cols(t.cols)) {
      wide.push_back(item);
    } else {
      const quest_status st = quantize_fwd_common(t.x, x_dtype, t.rows, t.cols, block, b, 1.0, t.codes, true, t.scale,
                                                  t.mask, true, nullptr, QUEST_BF16, false, nullptr, stream);
      if (st != QUEST_OK) return st;
    }
  }
  for (int w = 0; w < 3; ++w) {
    if (group[w].empty()) continue;
    const hipError_t e = quest::launch_fwd_group(group[w].data(), static_cast<int>(group[w].size()), 512 << w,
                                                 wide.data(), static_cast<int>(wide.size()), lb, b, alpha,
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return QUEST_EHIP;
    wide.clear();
  }
  if (!wide.empty()) {
    const hipError_t e = quest::launch_fwd_group(nullptr, 0, 2048, wide.data(), static_cast<int>(wide.size()), lb, b,
                                                 alpha, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return QUEST_EHIP;
  }
  return QUEST_OK;
}

quest_status quest_quantize_fwd_dq(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                   uint8_t* codes, float* scale, uint8_t* mask, void* dq, quest_dtype dq_dtype,
                                   void* stream) {
  return quantize_fwd_common(x, x_dtype, rows, cols, block, b, 1.0, codes, false, scale, mask, true, dq, dq_dtype,
                             true, nullptr, stream);
}

quest_status quest_quantize_fwd_ex(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                   double trust, uint8_t* codes, float* scale, uint8_t* mask, void* dq,
                                   quest_dtype dq_dtype, void* stream) {
  return quantize_fwd_common(x, x_dtype, rows, cols, block, b, trust, codes, false, scale, mask, true, dq, dq_dtype,
                             false, nullptr, stream);
}

size_t quest_operand_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || cols % 128 != 0) return 0;
  return static_cast<size_t>((rows + 31) / 32) * 32 * static_cast<size_t>(cols / 4 * 3);
}

quest_status quest_quantize_fwd_op(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                   double trust, uint8_t* codes, float* scale, uint8_t* mask, uint8_t* operand,
                                   void* stream) {
  if (rows > 0 && !operand) return QUEST_EINVAL;
  return quantize_fwd_common(x, x_dtype, rows, cols, block, b, trust, codes, false, scale, mask, false, nullptr,
                             QUEST_BF16, false, rows > 0 ? operand : nullptr, stream);
}

quest_status quest_quantize_fwd_op_group(const quest_fwd_op_tensor* tensors, int count, quest_dtype x_dtype,
                                         int block, int b, double trust, void* stream) {
  if (count < 0 || (count > 0 && !tensors)) return QUEST_EINVAL;
  // Every tensor as quest_quantize_fwd_op would check it ...
  for (int i = 0; i < count; ++i) {
    const quest_fwd_op_tensor& t = tensors[i];
    if (t.rows > 0 && !t.operand) return QUEST_EINVAL;
    const quest_status st = check_fwd(t.x, x_dtype, t.rows, t.cols, block, b, trust, t.codes, false, t.scale, t.mask,
                                      false, nullptr, QUEST_BF16, false, t.rows > 0 ? t.operand : nullptr);
    if (st != QUEST_OK) return st;
  }
  // ... and no output of one tensor on an input or output of another.
  auto spans = [&](const quest_fwd_op_tensor& t, const void* (&p)[5], size_t (&n)[5]) {
    p[0] = t.x;
    p[1] = t.codes;
    p[2] = t.scale;
    p[3] = t.mask;
    p[4] = t.operand;
    n[0] = static_cast<size_t>(t.rows * t.cols) * dtype_size(x_dtype);
    n[1] = t.codes ? quest_codes_bytes(t.rows, t.cols, b) : 0;
    n[2] = static_cast<size_t>(t.rows) * sizeof(float);
    n[3] = t.mask ? quest_mask_bytes(t.rows, t.cols) : 0;
    n[4] = quest_operand_bytes(t.rows, t.cols);
  };
  for (int i = 0; i < count; ++i) {
    if (tensors[i].rows == 0) continue;
    const void* bi[5];
    size_t ni[5];
    spans(tensors[i], bi, ni);
    for (int j = i + 1; j < count; ++j) {
      if (tensors[j].rows == 0) continue;
      const void* bj[5];
      size_t nj[5];
      spans(tensors[j], bj, nj);
      for (int p = 0; p < 5; ++p)
        for (int q = 0; q < 5; ++q)
          if ((p > 0 || q > 0) && overlaps(bi[p], ni[p], bj[q], nj[q])) return QUEST_EINVAL;
    }
  }
  std::call_once(g_env_once, read_env);
  const int lb = log2_block(block);
  const double alpha = quest_fit_alpha(b);
  // bf16 tensors of 512, 1024 or 2048 columns go in grouped launches, one
  // per width; the others as quest_quantize_fwd_op.
  std::vector<quest::FwdOpGroupItem> group[3];
  const bool grouped = x_dtype == QUEST_BF16 && g_allow_mfma;
  for (int i = 0; i < count; ++i) {
    const quest_fwd_op_tensor& t = tensors[i];
    if (t.rows == 0) continue;
    if (grouped && quest::fwd_group_tile_cols(t.cols)) {
      group[t.cols == 512 ? 0 : t.cols == 1024 ? 1 : 2].push_back({t.x, t.rows, t.codes, t.scale, t.mask, t.operand});
    } else {
      const quest_status st = quantize_fwd_common(t.x, x_dtype, t.rows, t.cols, block, b, trust, t.codes, false,
                                                  t.scale, t.mask, false, nullptr, QUEST_BF16, false, t.operand,
                                                  stream);
      if (st != QUEST_OK) return st;
    }
  }
  for (int w = 0; w < 3; ++w) {
    if (group[w].empty()) continue;
    const hipError_t e = quest::launch_fwd_op_group(group[w].data(), static_cast<int>(group[w].size()), 512 << w, lb,
                                                    b, alpha, trust, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return QUEST_EHIP;
  }
  return QUEST_OK;
}

quest_status quest_gemm(const uint8_t* a, const float* a_scale, int64_t m, int a_bits, const uint8_t* b,
                        const float* b_scale, int64_t n, int b_bits, int64_t k, void* out, quest_dtype out_dtype,
                        void* stream) {
  if (a_bits < 1 || a_bits > 4 || b_bits < 1 || b_bits > 4) return QUEST_EUNSUPPORTED;
  if (!dtype_ok(out_dtype) || m < 0 || n < 0 || k <= 0) return QUEST_EINVAL;
  if (k % 128 != 0 || k > kGemmMaxK || n > kGemmMaxN || m > kGemmMaxM) return QUEST_EUNSUPPORTED;
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  // 512 work-items per tile: the launch's work-item count must fit 32 bits.
  if (tiles > kGemmMaxTiles) return QUEST_EUNSUPPORTED;
  if (m == 0 || n == 0) return QUEST_OK;
  if (!a || !a_scale || !b || !b_scale || !out) return QUEST_EINVAL;
  if (!aligned16(a) || !aligned16(a_scale) || !aligned16(b) || !aligned16(b_scale) || !aligned16(out))
    return QUEST_EALIGN;
  const size_t no = static_cast<size_t>(m) * static_cast<size_t>(n) * dtype_size(out_dtype);
  if (overlaps(out, no, a, quest_operand_bytes(m, k)) || overlaps(out, no, b, quest_operand_bytes(n, k)) ||
      overlaps(out, no, a_scale, static_cast<size_t>(m) * 4) || overlaps(out, no, b_scale, static_cast<size_t>(n) * 4))
    return QUEST_EINVAL;
  quest::GemmLaunch g;
  g.a = a;
  g.sa = a_scale;
  g.m = static_cast<int>(m);
  g.b = b;
  g.sb = b_scale;
  g.n = static_cast<int>(n);
  g.k = static_cast<int>(k);
  g.ka = static_cast<float>(2.0 / double((1 << a_bits) - 1));
  g.kb = static_cast<float>(2.0 / double((1 << b_bits) - 1));
  g.out = out;
  g.stream = static_cast<hipStream_t>(stream);
  return from_hip(quest::launch_gemm_e2m3(g, out_dtype == QUEST_BF16));
}

double quest_fit_alpha_fp4(void) {
  std::call_once(g_alpha_once, fill_alpha_table);
  return g_alpha_fp4;
}

size_t quest_sparse24_codes_bytes(int64_t rows, int64_t cols, int b) {
  if (rows < 0 || cols <= 0 || cols % 64 != 0 || b < 1 || b > 4) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(cols / 2 * b / 8);
}

size_t quest_sparse24_index_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || cols % 64 != 0) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(cols / 8);
}

quest_status quest_quantize_fwd_fp4(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                    double trust, uint8_t* codes, float* scale, uint8_t* mask, void* dq,
                                    quest_dtype dq_dtype, void* stream) {
  return quantize_grid_common(x, x_dtype, rows, cols, block, 0, trust, codes, nullptr, scale, mask, dq, dq_dtype,
                              stream);
}

quest_status quest_quantize_fwd_sparse24(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                         int b, double trust, uint8_t* codes, uint8_t* index, float* scale,
                                         uint8_t* mask, void* dq, quest_dtype dq_dtype, void* stream) {
  if (b < 1 || b > 4) return QUEST_EUNSUPPORTED;
  return quantize_grid_common(x, x_dtype, rows, cols, block, b, trust, codes, index, scale, mask, dq, dq_dtype,
                              stream);
}

quest_status quest_dequantize_fp4(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, void* out,
                                  quest_dtype out_dtype, void* stream) {
  if (!dtype_ok(out_dtype)) return QUEST_EINVAL;
  const quest_status sh = check_shape(rows, cols, 64);
  if (sh != QUEST_OK) return sh;
  if (rows == 0) return QUEST_OK;
  if (!codes || !scale || !out) return QUEST_EINVAL;
  if (!aligned16(codes) || !aligned16(scale) || !aligned16(out)) return QUEST_EALIGN;
  const size_t nc = quest_codes_bytes(rows, cols, 4);
  const size_t ns = static_cast<size_t>(rows) * sizeof(float);
  const size_t no = static_cast<size_t>(rows * cols) * dtype_size(out_dtype);
  if (overlaps(out, no, codes, nc) || overlaps(out, no, scale, ns)) return QUEST_EINVAL;
  return from_hip(quest::launch_dequantize_fp4(codes, scale, rows, cols, out, out_dtype == QUEST_BF16,
                                               static_cast<hipStream_t>(stream)));
}

quest_status quest_dequantize_sparse24(const uint8_t* codes, const uint8_t* index, const float* scale, int64_t rows,
                                       int64_t cols, int b, void* out, quest_dtype out_dtype, void* stream) {
  if (b < 1 || b > 4) return QUEST_EUNSUPPORTED;
  if (!dtype_ok(out_dtype)) return QUEST_EINVAL;
  const quest_status sh = check_shape(rows, cols, 64);
  if (sh != QUEST_OK) return sh;
  if (rows == 0) return QUEST_OK;
  if (!codes || !index || !scale || !out) return QUEST_EINVAL;
  if (!aligned16(codes) || !aligned16(index) || !aligned16(scale) || !aligned16(out)) return QUEST_EALIGN;
  const size_t nc = quest_sparse24_codes_bytes(rows, cols, b);
  const size_t ni = quest_sparse24_index_bytes(rows, cols);
  const size_t ns = static_cast<size_t>(rows) * sizeof(float);
  const size_t no = static_cast<size_t>(rows * cols) * dtype_size(out_dtype);
  if (overlaps(out, no, codes, nc) || overlaps(out, no, index, ni) || overlaps(out, no, scale, ns)) return QUEST_EINVAL;
  return from_hip(quest::launch_dequantize_sparse24(codes, index, scale, rows, cols, b, out, out_dtype == QUEST_BF16,
                                                    static_cast<hipStream_t>(stream)));
}

quest_status quest_dequantize(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int b, void* out,
                              quest_dtype out_dtype, void* stream) {
  if (b < 1 || b > kMaxBits) return QUEST_EUNSUPPORTED;
  if (!dtype_ok(out_dtype)) return QUEST_EINVAL;
  const quest_status sh = check_shape(rows, cols, 64);
  if (sh != QUEST_OK) return sh;
  if (rows == 0) return QUEST_OK;
  if (!codes || !scale || !out) return QUEST_EINVAL;
  if (!aligned16(codes) || !aligned16(scale) || !aligned16(out)) return QUEST_EALIGN;
  const size_t nc = quest_codes_bytes(rows, cols, b);
  const size_t ns = static_cast<size_t>(rows) * sizeof(float);
  const size_t no = static_cast<size_t>(rows * cols) * dtype_size(out_dtype);
  if (overlaps(out, no, codes, nc) || overlaps(out, no, scale, ns)) return QUEST_EINVAL;
  return from_hip(quest::launch_dequantize(codes, scale, rows, cols, b, out, out_dtype == QUEST_BF16,
                                           static_cast<hipStream_t>(stream)));
}

quest_status quest_codes_to_operand(const uint8_t* codes, int64_t rows, int64_t cols, int b, uint8_t* operand,
                                    void* stream) {
  if (b < 1 || b > 4) return QUEST_EUNSUPPORTED;
  const quest_status sh = check_shape(rows, cols, 128);
  if (sh != QUEST_OK) return sh;
  if (rows == 0) return QUEST_OK;
  if (!codes || !operand) return QUEST_EINVAL;
  if (!aligned16(codes) || !aligned16(operand)) return QUEST_EALIGN;
  if (overlaps(operand, quest_operand_bytes(rows, cols), codes, quest_codes_bytes(rows, cols, b))) return QUEST_EINVAL;
  return from_hip(quest::launch_codes_to_operand(codes, rows, cols, b, operand, static_cast<hipStream_t>(stream)));
}

quest_status quest_trust_bwd(const void* grad, quest_dtype g_dtype, const uint8_t* mask, int64_t rows, int64_t cols,
                             int block, void* grad_out, void* stream) {
  const int lb = log2_block(block);
  if (lb < 0) return QUEST_EUNSUPPORTED;
  if (!dtype_ok(g_dtype)) return QUEST_EINVAL;
  const quest_status sh = check_shape(rows, cols, block);
  if (sh != QUEST_OK) return sh;
  if (rows == 0) return QUEST_OK;
  if (!grad || !mask || !grad_out) return QUEST_EINVAL;
  if (!aligned16(grad) || !aligned16(mask) || !aligned16(grad_out)) return QUEST_EALIGN;
  const size_t ng = static_cast<size_t>(rows * cols) * dtype_size(g_dtype);
  const size_t nm = quest_mask_bytes(rows, cols);
  if (grad_out != grad && overlaps(grad, ng, grad_out, ng)) return QUEST_EINVAL;
  if (overlaps(grad_out, ng, mask, nm) || overlaps(grad, ng, mask, nm)) return QUEST_EINVAL;
  std::call_once(g_env_once, read_env);
  return from_hip(quest::launch_trust_bwd(grad, g_dtype == QUEST_BF16, mask, rows, cols, lb, grad_out,
                                          g_allow_mfma_bwd, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The argument checks of the forward entry points (QUEST_OK also for rows == 0,
// which launches nothing).
quest_status check_fwd(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b, double trust,
                       uint8_t* codes, bool codes_required, float* scale, uint8_t* mask, bool mask_required, void* dq,
                       quest_dtype dq_dtype, bool dq_required, uint8_t* operand) {
  const int lb = log2_block(block);
  if (lb < 0 || b < 1 || b > kMaxBits) return QUEST_EUNSUPPORTED;
  if (operand && (b > 4 || cols % 128 != 0)) return QUEST_EUNSUPPORTED;
  if (!dtype_ok(x_dtype)) return QUEST_EINVAL;
  if ((dq || dq_required) && !dtype_ok(dq_dtype)) return QUEST_EINVAL;
  if (!(trust >= 0.0) || !std::isfinite(trust)) return QUEST_EINVAL;
  const quest_status sh = check_shape(rows, cols, block);
  if (sh != QUEST_OK) return sh;
  if (rows == 0) return QUEST_OK;
  if (!x || !scale || (mask_required && !mask) || (codes_required && !codes) || (dq_required && !dq)) return QUEST_EINVAL;
  if (!aligned16(x) || (codes && !aligned16(codes)) || !aligned16(scale) || (mask && !aligned16(mask)) ||
      (dq && !aligned16(dq)) || (operand && !aligned16(operand)))
    return QUEST_EALIGN;
  const size_t nx = static_cast<size_t>(rows * cols) * dtype_size(x_dtype);
  const size_t nc = codes ? quest_codes_bytes(rows, cols, b) : 0;
  const size_t ns = static_cast<size_t>(rows) * sizeof(float);
  const size_t nm = mask ? quest_mask_bytes(rows, cols) : 0;
  const size_t nd = dq ? static_cast<size_t>(rows * cols) * dtype_size(dq_dtype) : 0;
  const size_t no = operand ? quest_operand_bytes(rows, cols) : 0;
  if (overlaps(x, nx, codes, nc) || overlaps(x, nx, scale, ns) || overlaps(x, nx, mask, nm) ||
      overlaps(codes, nc, scale, ns) || overlaps(codes, nc, mask, nm) || overlaps(scale, ns, mask, nm) ||
      overlaps(dq, nd, x, nx) || overlaps(dq, nd, codes, nc) || overlaps(dq, nd, scale, ns) ||
      overlaps(dq, nd, mask, nm) || overlaps(operand, no, x, nx) || overlaps(operand, no, codes, nc) ||
      overlaps(operand, no, scale, ns) || overlaps(operand, no, mask, nm))
    return QUEST_EINVAL;
  return QUEST_OK;
}

quest_status quantize_fwd_common(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                 double trust, uint8_t* codes, bool codes_required, float* scale, uint8_t* mask,
                                 bool mask_required, void* dq, quest_dtype dq_dtype, bool dq_required,
                                 uint8_t* operand, void* stream) {
  const quest_status st = check_fwd(x, x_dtype, rows, cols, block, b, trust, codes, codes_required, scale, mask,
                                    mask_required, dq, dq_dtype, dq_required, operand);
  if (st != QUEST_OK || rows == 0) return st;
  const int lb = log2_block(block);
  std::call_once(g_env_once, read_env);
  quest::FwdLaunch a;
  a.rows = rows;
  a.cols = cols;
  a.alpha = quest_fit_alpha(b);
  a.trust = trust;
  a.allow_mfma = g_allow_mfma;
  a.codes = codes;
  a.scale = scale;
  a.mask = mask;
  a.dq = operand ? static_cast<void*>(operand) : dq;
  a.stream = static_cast<hipStream_t>(stream);
  const int dq_kind = operand ? 3 : dq ? (dq_dtype == QUEST_BF16 ? 1 : 2) : 0;
  return from_hip(quest::launch_quantize_fwd(x, x_dtype == QUEST_BF16, lb, b, dq_kind, a));
}

}  // namespace

namespace {

quest_status quantize_grid_common(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block, int b,
                                  double trust, uint8_t* codes, uint8_t* index, float* scale, uint8_t* mask, void* dq,
                                  quest_dtype dq_dtype, void* stream) {
  const int lb = log2_block(block);
  if (lb < 0) return QUEST_EUNSUPPORTED;
  if (!dtype_ok(x_dtype) || (dq && !dtype_ok(dq_dtype))) return QUEST_EINVAL;
  if (!(trust >= 0.0) || !std::isfinite(trust)) return QUEST_EINVAL;
  const quest_status sh = check_shape(rows, cols, block);
  if (sh != QUEST_OK) return sh;
  if (rows == 0) return QUEST_OK;
  if (!x || !scale || !mask) return QUEST_EINVAL;
  if (!aligned16(x) || (codes && !aligned16(codes)) || (index && !aligned16(index)) || !aligned16(scale) ||
      !aligned16(mask) || (dq && !aligned16(dq)))
    return QUEST_EALIGN;
  const size_t nx = static_cast<size_t>(rows * cols) * dtype_size(x_dtype);
  const size_t nc = codes ? (b == 0 ? quest_codes_bytes(rows, cols, 4) : quest_sparse24_codes_bytes(rows, cols, b)) : 0;
  const size_t ni = index ? quest_sparse24_index_bytes(rows, cols) : 0;
  const size_t ns = static_cast<size_t>(rows) * sizeof(float);
  const size_t nm = quest_mask_bytes(rows, cols);
  const size_t nd = dq ? static_cast<size_t>(rows * cols) * dtype_size(dq_dtype) : 0;
  const void* bufs[6] = {x, codes, index, scale, mask, dq};
  const size_t lens[6] = {nx, nc, ni, ns, nm, nd};
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(bufs[i], lens[i], bufs[j], lens[j])) return QUEST_EINVAL;
  std::call_once(g_alpha_once, fill_alpha_table);
  quest::GridLaunch a;
  a.rows = rows;
  a.cols = cols;
  a.alpha = b == 0 ? g_alpha_fp4 : g_alpha[b];
  a.trust = trust;
  a.bits = b == 0 ? 4 : b;
  a.sparse24 = b == 0 ? 0 : 1;
  std::call_once(g_env_once, read_env);
  a.allow_mfma = g_allow_mfma;
  a.codes = codes;
  a.index = index;
  a.scale = scale;
  a.mask = mask;
  a.dq = dq;
  a.stream = static_cast<hipStream_t>(stream);
  const int dq_kind = dq ? (dq_dtype == QUEST_BF16 ? 1 : 2) : 0;
  return from_hip(quest::launch_fwd_grid(x, x_dtype == QUEST_BF16, lb, dq_kind, a));
}

}  // namespace

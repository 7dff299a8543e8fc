// The three kernels of libquest and their launchers (gfx950).
//
// Forward (QuEST quantiser; atlas.scime.ai summary of QuEST, "Approach";
// pith.science review of QuEST, "What carries the argument"):
//   per row: blockwise Hadamard -> sum of squares -> clip scale
//   s = alpha_b * RMS -> codes, trust mask -> packed stores.
// Backward (trust estimator; pith.science review, "What carries the
// argument" and Figure 2 caption): mask * gradient -> Hadamard -> store.
// Dequantise: codes -> grid values (2u - L + 1) s / (L - 1).
//
// All three stream through HBM once.  The forward transform is computed
// unnormalised (entries scaled by sqrt(n)); codes and mask only depend on
// y / Delta, so the factor is folded into the per-row constants instead of
// costing a multiply per element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "quest_device.h"
#include "quest_launch.h"

namespace quest {

template <int LOGN>
struct BlockConst {
  // 1/sqrt(n) and sqrt(n) for n = 2^LOGN, exact to fp32 rounding.
  static constexpr double kRsqrt2 = 0.70710678118654752440084436210485;
  static constexpr float rsqrt_n =
      static_cast<float>((LOGN & 1) ? kRsqrt2 / double(1 << (LOGN / 2)) : 1.0 / double(1 << (LOGN / 2)));
  static constexpr float sqrt_n =
      static_cast<float>((LOGN & 1) ? double(1 << (LOGN / 2)) / kRsqrt2 : double(1 << (LOGN / 2)));
};

// ----------------------------------------------------------------------------
// Forward quantisation.
//
// Workgroup = rows_per_wg rows; a row is runs_per_row = cols/32 consecutive
// lanes.  WAVE_LOCAL: runs_per_row is a power of two <= 64, so a row lives
// inside one wavefront and its sum of squares is a butterfly over lanes.
// Otherwise a row spans several wavefronts: lanes reduce in aligned groups of
// `group` lanes (a power of two dividing runs_per_row), group sums go through
// LDS and every lane adds up the groups of its row in the same order.
// Lanes past the last row load row 0 and compute like the others (DPP needs
// every lane of a quad), but store nothing.
// ----------------------------------------------------------------------------
// Quantise 32 transformed values v (= tau * sqrt(n) * y) into b-bit codes.
// kk = tau * (L - 1) / (2 s sqrt(n)), so v * kk = y / Delta.
template <int B>
__device__ __forceinline__ CodeWords<B> quantise_run(const float (&v)[RUN], float kk) {
  constexpr float L = static_cast<float>(1 << B);
  CodeWords<B> cw;
  if constexpr (B == 1) {
    // u = [y >= 0]
    float p[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) p[j] = v[j] * kk;
    uint32_t w = 0u;
    push16_nonneg(w, p + 16);
    push16_nonneg(w, p);
    cw.w[0] = w;
  } else if constexpr (B == 2 || B == 4) {
    // u = clamp(floor(y / Delta + L/2), 0, L-1) = RNE(min(y / Delta + (L-1)/2, L-1)), saturated
    // at 0 by v_cvt_pk_u8_f32; the two differ only when y / Delta is exactly an integer
    // (y exactly on a decision threshold), where round-to-even may pick the upper code.
    // Byte k of accumulator j collects code (per-word index) k * (8/B) + j; the accumulators
    // are then interleaved into B-bit fields.
    constexpr int PER_BYTE = 8 / B;
    constexpr int PER_WORD = 32 / B;
    const float off = 0.5f * (L - 1.f);
#pragma unroll
    for (int w = 0; w < B; ++w) {
      uint32_t acc[PER_BYTE];
#pragma unroll
      for (int j = 0; j < PER_BYTE; ++j) acc[j] = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < PER_BYTE; ++j) {
          const float t = __builtin_fminf(__builtin_fmaf(v[w * PER_WORD + k * PER_BYTE + j], kk, off), L - 1.f);
          acc[j] = __builtin_amdgcn_cvt_pk_u8_f32(t, k, acc[j]);
        }
      }
      uint32_t word = acc[0];
#pragma unroll
      for (int j = 1; j < PER_BYTE; ++j) word |= acc[j] << (B * j);
      cw.w[w] = word;
    }
  } else {
    // b = 3: codes straddle dword boundaries; clamp(floor(t), 0, L-1) = trunc(clamp(t, 0, L-1)).
#pragma unroll
    for (int i = 0; i < B; ++i) cw.w[i] = 0u;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(v[j], kk, 0.5f * L), 0.f, L - 1.f);
      put_code<B>(cw, j, static_cast<uint32_t>(t));
    }
  }
  return cw;
}

template <typename In, int LOGN, int B, bool WAVE_LOCAL>
__global__ void __launch_bounds__(WAVE_LOCAL ? 256 : 1024)
    quest_fwd_kernel(const In* __restrict__ x, int64_t rows, int runs_per_row, int rows_per_wg, int group,
                     float alpha, float inv_cols, uint8_t* __restrict__ codes, float* __restrict__ scale,
                     uint32_t* __restrict__ mask) {
  constexpr int U = sizeof(In) * 2;  // 16-byte pieces per run
  constexpr int WAVES = (WAVE_LOCAL ? 256 : 1024) / 64;
  __shared__ u32x4 stage_all[WAVES][64 * U];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lrow = tid / runs_per_row;
  const int run_in_row = tid - lrow * runs_per_row;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * rows_per_wg + lrow;
  const bool valid = (lrow < rows_per_wg) && (row < rows);
  // Lane t of the workgroup holds run (first run of the workgroup) + t; runs of
  // lanes past the workgroup's rows belong to the next workgroup or lie past
  // the tensor, and are loaded (or stood in for) but never stored.
  const int64_t wg_first_run = static_cast<int64_t>(blockIdx.x) * rows_per_wg * runs_per_row;
  const int64_t run = wg_first_run + tid;
  const int64_t total_pieces = rows * runs_per_row * U;

  uint32_t raw[4 * U];
  wave_load_runs<U>(reinterpret_cast<const u32x4*>(x), (wg_first_run + (tid & ~63)) * U, total_pieces, lane,
                    stage_all[tid >> 6], raw);

  // The row's RMS is taken from the inputs: the orthonormal transform keeps the
  // sum of squares (Parseval), so it equals the RMS of the transformed row.
  float v[RUN];
  float ss;
  if constexpr (sizeof(In) == 2) {
    ss = sum_squares_bf16(raw);
    first_stages_bf16(raw, v);
    fwht_in_lane<4>(v);
  } else {
    widen_run(raw, v);
    ss = sum_squares(v);
    fwht_in_lane<1>(v);
  }
  const float tau = fwht_cross_lanes<LOGN>(v, tid);

  if constexpr (WAVE_LOCAL) {
    for (int off = 1; off < runs_per_row; off <<= 1) ss += __shfl_xor(ss, off);
  } else {
    __shared__ float part[1024];
    for (int off = 1; off < group; off <<= 1) ss += __shfl_xor(ss, off);
    if ((tid & (group - 1)) == 0) part[tid / group] = ss;
    __syncthreads();
    const int per_row = runs_per_row / group;
    ss = 0.f;
    if (lrow < rows_per_wg) {
      const float* pr = part + lrow * per_row;
      for (int i = 0; i < per_row; ++i) ss += pr[i];
    }
  }

  // s = alpha * RMS, RMS^2 = sum(x^2) / cols.
  const float s = alpha * sqrtf(ss * inv_cols);
  if (valid && run_in_row == 0) scale[row] = s;

  constexpr float L = static_cast<float>(1 << B);
  // With v = tau * sqrt(n) * y:  y / Delta = v * kk,  and
  // trusted <=> |y| <= s L / (L - 1) <=> |v| <= thr.
  float kk = 0.f, thr = 0.f;
  if (s > 0.f) {
    kk = tau * ((L - 1.f) / (2.f * s)) * BlockConst<LOGN>::rsqrt_n;
    thr = s * (L / (L - 1.f)) * BlockConst<LOGN>::sqrt_n;
  }

  const CodeWords<B> cw = quantise_run<B>(v, kk);
  uint32_t mw = 0u;
  push16_abs_le(mw, v + 16, thr);
  push16_abs_le(mw, v, thr);
  if (valid) {
    store_codes<B>(codes, run, cw);
    mask[run] = mw;
  }
}

// ----------------------------------------------------------------------------
// Trust-masked backward: one lane per run, no cross-row work.
// grad and grad_out may be the same buffer: every run is read and written by
// the same lane only, and its loads come before its stores.
// ----------------------------------------------------------------------------
template <typename G, int LOGN>
__global__ void __launch_bounds__(256)
    quest_bwd_kernel(const G* grad, const uint32_t* mask, int64_t total_runs, G* grad_out) {
  constexpr int U = sizeof(G) * 2;
  __shared__ u32x4 stage_all[4][64 * U];
  const int lane = threadIdx.x & 63;
  u32x4* stage = stage_all[threadIdx.x >> 6];
  const int64_t run0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t first_piece = (run0 - lane) * U;
  const uint32_t m = __builtin_nontemporal_load(mask + (run0 < total_runs ? run0 : 0));
  uint32_t raw[4 * U];
  wave_load_runs<U>(reinterpret_cast<const u32x4*>(grad), first_piece, total_runs * U, lane, stage, raw);
  float v[RUN];
  widen_run_masked(raw, m, v);
  const float tau = fwht_block<LOGN>(v, threadIdx.x);
  const float k = tau * BlockConst<LOGN>::rsqrt_n;
#pragma unroll
  for (int j = 0; j < RUN; ++j) v[j] *= k;
  narrow_run(v, raw);
  wave_store_runs<U>(reinterpret_cast<u32x4*>(grad_out), first_piece, total_runs * U, lane, stage, raw);
}

// ----------------------------------------------------------------------------
// Dequantise: one lane per run.
// ----------------------------------------------------------------------------
template <typename Out, int B>
__global__ void __launch_bounds__(256)
    quest_dequant_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scale, uint32_t total_runs,
                         uint32_t runs_per_row, Out* __restrict__ out) {
  constexpr int U = sizeof(Out) * 2;
  __shared__ u32x4 stage_all[4][64 * U];
  const int lane = threadIdx.x & 63;
  const uint32_t run0 = blockIdx.x * 256u + threadIdx.x;
  const uint32_t run = run0 < total_runs ? run0 : 0u;
  const uint32_t row = run / runs_per_row;
  const float c = scale[row] / static_cast<float>((1 << B) - 1);
  const CodeWords<B> cw = load_codes<B>(codes, run);
  float v[RUN];
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    const int u = static_cast<int>(get_code<B>(cw, j));
    v[j] = static_cast<float>(2 * u - (1 << B) + 1) * c;
  }
  uint32_t raw[4 * U];
  narrow_run(v, raw);
  wave_store_runs<U>(reinterpret_cast<u32x4*>(out), (static_cast<int64_t>(run0) - lane) * U,
                     static_cast<int64_t>(total_runs) * U, lane, stage_all[threadIdx.x >> 6], raw);
}

// ----------------------------------------------------------------------------
// Launchers.
// ----------------------------------------------------------------------------
namespace {

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

template <typename In, int LOGN, int B>
hipError_t fwd_dispatch_wave(const In* x, int64_t rows, int64_t cols, float alpha, uint8_t* codes, float* scale,
                             uint8_t* mask, hipStream_t stream) {
  const int runs_per_row = static_cast<int>(cols / RUN);
  const float inv_cols = static_cast<float>(1.0 / double(cols));
  uint32_t* mask32 = reinterpret_cast<uint32_t*>(mask);
  if (runs_per_row <= 64 && (runs_per_row & (runs_per_row - 1)) == 0) {
    const int rows_per_wg = 256 / runs_per_row;
    const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((quest_fwd_kernel<In, LOGN, B, true>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                       x, rows, runs_per_row, rows_per_wg, 0, alpha, inv_cols, codes, scale, mask32);
  } else {
    int group = runs_per_row & -runs_per_row;
    if (group > 64) group = 64;
    int rows_per_wg = 64 / gcd_int(runs_per_row, 64);
    if (rows_per_wg * runs_per_row > 1024) rows_per_wg = 1024 / runs_per_row;
    if (rows_per_wg < 1) rows_per_wg = 1;
    const int threads = ((rows_per_wg * runs_per_row + 63) / 64) * 64;
    const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((quest_fwd_kernel<In, LOGN, B, false>), dim3(static_cast<uint32_t>(grid)), dim3(threads), 0,
                       stream, x, rows, runs_per_row, rows_per_wg, group, alpha, inv_cols, codes, scale, mask32);
  }
  return hipGetLastError();
}

template <typename In, int LOGN>
hipError_t fwd_dispatch_bits(const In* x, int64_t rows, int64_t cols, int bits, float alpha, uint8_t* codes,
                             float* scale, uint8_t* mask, hipStream_t stream) {
  switch (bits) {
    case 1: return fwd_dispatch_wave<In, LOGN, 1>(x, rows, cols, alpha, codes, scale, mask, stream);
    case 2: return fwd_dispatch_wave<In, LOGN, 2>(x, rows, cols, alpha, codes, scale, mask, stream);
    case 3: return fwd_dispatch_wave<In, LOGN, 3>(x, rows, cols, alpha, codes, scale, mask, stream);
    default: return fwd_dispatch_wave<In, LOGN, 4>(x, rows, cols, alpha, codes, scale, mask, stream);
  }
}

template <typename In>
hipError_t fwd_dispatch_block(const In* x, int64_t rows, int64_t cols, int log_block, int bits, float alpha,
                              uint8_t* codes, float* scale, uint8_t* mask, hipStream_t stream) {
  switch (log_block) {
    case 6: return fwd_dispatch_bits<In, 6>(x, rows, cols, bits, alpha, codes, scale, mask, stream);
    case 7: return fwd_dispatch_bits<In, 7>(x, rows, cols, bits, alpha, codes, scale, mask, stream);
    default: return fwd_dispatch_bits<In, 8>(x, rows, cols, bits, alpha, codes, scale, mask, stream);
  }
}

template <typename G>
hipError_t bwd_dispatch(const G* grad, const uint8_t* mask, int64_t rows, int64_t cols, int log_block, G* out,
                        hipStream_t stream) {
  const int64_t total_runs = rows * (cols / RUN);
  const int64_t grid = (total_runs + 255) / 256;
  const uint32_t* mask32 = reinterpret_cast<const uint32_t*>(mask);
  switch (log_block) {
    case 6:
      hipLaunchKernelGGL((quest_bwd_kernel<G, 6>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, grad,
                         mask32, total_runs, out);
      break;
    case 7:
      hipLaunchKernelGGL((quest_bwd_kernel<G, 7>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, grad,
                         mask32, total_runs, out);
      break;
    default:
      hipLaunchKernelGGL((quest_bwd_kernel<G, 8>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, grad,
                         mask32, total_runs, out);
      break;
  }
  return hipGetLastError();
}

template <typename Out>
hipError_t dequant_dispatch(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int bits, Out* out,
                            hipStream_t stream) {
  const uint32_t runs_per_row = static_cast<uint32_t>(cols / RUN);
  const uint32_t total_runs = static_cast<uint32_t>(rows) * runs_per_row;
  const uint32_t grid = (total_runs + 255u) / 256u;
  switch (bits) {
    case 1:
      hipLaunchKernelGGL((quest_dequant_kernel<Out, 1>), dim3(grid), dim3(256), 0, stream, codes, scale, total_runs,
                         runs_per_row, out);
      break;
    case 2:
      hipLaunchKernelGGL((quest_dequant_kernel<Out, 2>), dim3(grid), dim3(256), 0, stream, codes, scale, total_runs,
                         runs_per_row, out);
      break;
    case 3:
      hipLaunchKernelGGL((quest_dequant_kernel<Out, 3>), dim3(grid), dim3(256), 0, stream, codes, scale, total_runs,
                         runs_per_row, out);
      break;
    default:
      hipLaunchKernelGGL((quest_dequant_kernel<Out, 4>), dim3(grid), dim3(256), 0, stream, codes, scale, total_runs,
                         runs_per_row, out);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fwd(const void* x, int x_is_bf16, int64_t rows, int64_t cols, int log_block, int bits,
                               float alpha, uint8_t* codes, float* scale, uint8_t* mask, hipStream_t stream) {
  if (x_is_bf16)
    return fwd_dispatch_block(static_cast<const uint16_t*>(x), rows, cols, log_block, bits, alpha, codes, scale, mask,
                              stream);
  return fwd_dispatch_block(static_cast<const float*>(x), rows, cols, log_block, bits, alpha, codes, scale, mask,
                            stream);
}

hipError_t launch_dequantize(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int bits,
                             void* out, int out_is_bf16, hipStream_t stream) {
  if (out_is_bf16) return dequant_dispatch(codes, scale, rows, cols, bits, static_cast<uint16_t*>(out), stream);
  return dequant_dispatch(codes, scale, rows, cols, bits, static_cast<float*>(out), stream);
}

hipError_t launch_trust_bwd(const void* grad, int g_is_bf16, const uint8_t* mask, int64_t rows, int64_t cols,
                            int log_block, void* grad_out, hipStream_t stream) {
  if (g_is_bf16)
    return bwd_dispatch(static_cast<const uint16_t*>(grad), mask, rows, cols, log_block,
                        static_cast<uint16_t*>(grad_out), stream);
  return bwd_dispatch(static_cast<const float*>(grad), mask, rows, cols, log_block, static_cast<float*>(grad_out),
                      stream);
}

}  // namespace quest

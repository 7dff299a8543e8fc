// The kernels of libquest (gfx950) and the templates that launch them.  The
// translation units quest_fwd_*.hip instantiate the forward for one output
// type each, quest_launch.hip the rest, so the build compiles them in
// parallel.
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
// y / Delta, so the factor is folded into per-row constants instead of
// costing a multiply per element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "quest_device.h"
#include "quest_launch.h"

namespace quest {

template <int LOGN>
struct BlockConst {
  // 1/sqrt(n) for n = 2^LOGN, rounded once to fp32.
  static constexpr double kRsqrt2 = 0.70710678118654752440084436210485;
  static constexpr float rsqrt_n =
      static_cast<float>((LOGN & 1) ? kRsqrt2 / double(1 << (LOGN / 2)) : 1.0 / double(1 << (LOGN / 2)));
};

// Byte offset that lies past every window: a buffer store there is dropped.
constexpr int kNowhere = 0x7FFFFFF0;

// ----------------------------------------------------------------------------
// Forward quantisation
// ----------------------------------------------------------------------------

// Per-bit-width constants computed on the host in float64 and rounded once:
//   alpha = alpha_b,  kk = (L - 1) / (2 alpha_b sqrt(n)),  thr = alpha_b L sqrt(n) / (L - 1).
// With m = mean of x^2 over the row (RMS^2) and v = tau * sqrt(n) * y:
//   s = alpha * sqrt(m),  y / Delta = v * tau * kk / sqrt(m),  trusted <=> |v| <= thr * sqrt(m).
struct FwdConsts {
  float alpha;
  float kk;
  float thr;
  float inv_cols;
  int chunks;  // cols / 128: 3072-byte blocks per row block of the matrix-core operand
};

// Quantise 32 transformed values v (= tau * sqrt(n) * y) into b-bit codes,
// given kk = y / (Delta v).
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
  } else if constexpr (B == 2 || B == 4 || B == 8) {
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
    // b = 3, 5, 6, 7: codes straddle dword boundaries; clamp(floor(t), 0, L-1) = trunc(clamp(t, 0, L-1)).
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

// b = 2 or 4: the codes of 8 transformed values as bytes, 8 / b entries
// interleaved over the dwords: entry (8 / b) k + j is byte k of acc[j]
// (v_cvt_pk_u8_f32 rounds to nearest even and saturates, as grid_code).
template <int B>
__device__ __forceinline__ void quantise8_bytes(const float* v, float kk, uint32_t (&acc)[8 / B]) {
  static_assert(B == 2 || B == 4, "byte codes of 2 or 4 bits");
  constexpr int PER_BYTE = 8 / B;
  constexpr float L = static_cast<float>(1 << B);
  const float off = 0.5f * (L - 1.f);
#pragma unroll
  for (int j = 0; j < PER_BYTE; ++j) acc[j] = 0u;
#pragma unroll
  for (int k = 0; k < 8 / PER_BYTE; ++k) {
#pragma unroll
    for (int j = 0; j < PER_BYTE; ++j) {
      const float t = __builtin_fminf(__builtin_fmaf(v[k * PER_BYTE + j], kk, off), L - 1.f);
      acc[j] = __builtin_amdgcn_cvt_pk_u8_f32(t, k, acc[j]);
    }
  }
}

// The byte codes of quantise8_bytes packed LSB-first (entry i in bits
// [b i, b i + b)).
template <int B>
__device__ __forceinline__ uint32_t pack8_bytes(const uint32_t (&acc)[8 / B]) {
  uint32_t w = acc[0];
#pragma unroll
  for (int j = 1; j < 8 / B; ++j) w |= acc[j] << (B * j);
  return w;
}

// The levels h = u - (L - 1)/2 of the byte codes of quantise8_bytes, entry
// order (each byte converted by one v_cvt_f32_ubyte).
template <int B>
__device__ __forceinline__ void levels8_from_bytes(const uint32_t (&acc)[8 / B], float* h) {
  constexpr int PER_BYTE = 8 / B;
  constexpr float kHalf = 0.5f * static_cast<float>((1 << B) - 1);
#pragma unroll
  for (int k = 0; k < 8 / PER_BYTE; ++k)
#pragma unroll
    for (int j = 0; j < PER_BYTE; ++j)
      h[k * PER_BYTE + j] = static_cast<float>((acc[j] >> (8 * k)) & 0xFFu) - kHalf;
}

// Quantise 8 transformed values (a quarter run) into b-bit codes packed
// LSB-first into the low 8 b bits of the result: the same arithmetic as
// quantise_run, on 8 entries.
template <int B>
__device__ __forceinline__ uint32_t quantise8(const float* v, float kk) {
  static_assert(B >= 1 && B <= 4, "8 codes of at most 4 bits fit one dword");
  constexpr float L = static_cast<float>(1 << B);
  if constexpr (B == 1) {
    // Code 1 where v kk >= 0: v kk + 0 is +0 for a zero product of either
    // sign, so the code is the complement of the sign bit, pushed in with one
    // funnel shift per entry (entry j ends in bit j).
    uint32_t s = 0u;
#pragma unroll
    for (int j = 7; j >= 0; --j) s = __builtin_amdgcn_alignbit(s, __float_as_uint(__builtin_fmaf(v[j], kk, 0.f)), 31);
    return ~s & 0xFFu;
  } else if constexpr (B == 2 || B == 4) {
    uint32_t acc[8 / B];
    quantise8_bytes<B>(v, kk, acc);
    return pack8_bytes<B>(acc);
  } else {
    uint32_t w = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(v[j], kk, 0.5f * L), 0.f, L - 1.f);
      w |= static_cast<uint32_t>(t) << (3 * j);
    }
    return w;
  }
}

// Transform one run per lane: returns tau and the lane's share of the row's
// sum of squares.  The row's RMS is taken from the inputs: the orthonormal
// transform keeps the sum of squares (Parseval), so it equals the RMS of the
// transformed row.
template <typename In, int LOGN>
__device__ __forceinline__ float fwd_transform(const uint32_t (&raw)[8 * sizeof(In)], float (&v)[RUN], float& ss,
                                               int lane_bits) {
  if constexpr (sizeof(In) == 2) {
    ss = sum_squares_bf16(raw);
    first_stages_bf16(raw, v);
    fwht_in_lane<4>(v);
  } else {
    widen_run(raw, v);
    ss = sum_squares(v);
    fwht_in_lane<1>(v);
  }
  return fwht_cross_lanes<LOGN>(v, lane_bits);
}

// Per-row constants from a row's sum of squares: the scale s = alpha RMS, the
// code factor kk (times this lane's sign tau) and the trust threshold on v.
struct RowConsts {
  float scale, kk, thr;
};

__device__ __forceinline__ RowConsts row_consts(float ss, float tau, const FwdConsts& k) {
  const float ms = ss * k.inv_cols;
  const float rms = __builtin_amdgcn_sqrtf(ms);
  RowConsts c;
  c.scale = k.alpha * rms;
  // A zero row (ms = 0) keeps kk = 0: every code is the middle one, every entry trusted.
  c.kk = ms > 0.f ? tau * k.kk * __builtin_amdgcn_rsqf(ms) : 0.f;
  c.thr = k.thr * rms;
  return c;
}

// Optional dequantised output of the forward pass: Dq = void (none),
// uint16_t (bf16) or float.  U is the number of 16-byte pieces per run.
template <typename Dq>
struct DqOut {
  static constexpr bool kOn = true;
  static constexpr int U = static_cast<int>(sizeof(Dq)) * 2;
};
template <>
struct DqOut<void> {
  static constexpr bool kOn = false;
  static constexpr int U = 1;
};

// Code u of one entry as a float, computed from v with factor kk by the
// arithmetic of quantise_run / quantise8, so it equals the stored code.
template <int B>
__device__ __forceinline__ float grid_code(float v, float kk) {
  constexpr float L = static_cast<float>(1 << B);
  if constexpr (B == 1) {
    return v * kk >= 0.f ? 1.f : 0.f;
  } else if constexpr (B == 2 || B == 4 || B == 8) {
    const float t = __builtin_fminf(__builtin_fmaf(v, kk, 0.5f * (L - 1.f)), L - 1.f);
    return __builtin_fmaxf(__builtin_rintf(t), 0.f);
  } else {
    return __builtin_truncf(__builtin_amdgcn_fmed3f(__builtin_fmaf(v, kk, 0.5f * L), 0.f, L - 1.f));
  }
}

// Grid values (2u - L + 1) s / (L - 1) of N entries (codes from grid_code).
// c = s / (L - 1), rounded as by quest_dequantize, and the product is
// rounded once, so the values equal quest_dequantize's on the same codes and
// scale.
template <int B, int N>
__device__ __forceinline__ void grid_values(const float* v, float kk, float c, float* q) {
  constexpr float L = static_cast<float>(1 << B);
#pragma unroll
  for (int i = 0; i < N; ++i) q[i] = __builtin_fmaf(grid_code<B>(v[i], kk), 2.f, 1.f - L) * c;
}

// c = s / (L - 1) for the grid values (a correctly rounded fp32 division, as
// in quest_dequantize).
template <int B>
__device__ __forceinline__ float grid_step_half(float s) {
  return s / static_cast<float>((1 << B) - 1);
}

// Matrix-core operand output (quest_quantize_fwd_op): for every run (32
// consecutive entries of a row) the half-integers u - (L - 1)/2, b <= 4, as
// FP6 E2M3 fields in the run's 24-byte lane slot of the tiled layout that
// quest_gemm reads.  Rows form blocks of 32, a row block holds `chunks`
// 3072-byte blocks of 128 columns, and run j of row r sits at
//   (r / 32) * chunks * 3072 + (j / 4) * 3072 + (j / 2 % 2) * 1536 + (32 (j % 2) + r % 32) * 24.
struct OperandOut {};
template <>
struct DqOut<OperandOut> {
  static constexpr bool kOn = true;
  static constexpr int U = 1;
};
template <typename Dq>
constexpr bool kIsOperand = std::is_same<Dq, OperandOut>::value;

// Workgroup index of the forward kernels.  Workgroups are dealt to the 8 XCDs
// round-robin; an operand's 128-byte lines each hold parts of several
// neighbouring rows, so for the operand workgroup b takes the logical index
// (b % 8) * (G / 8) + b / 8: each XCD then works through one contiguous range
// of rows and every line is completed inside one L2 (the last G % 8
// workgroups keep their index).  Other outputs keep the launch order.
template <typename Dq>
__device__ __forceinline__ int64_t fwd_wg_index() {
  const int64_t b = blockIdx.x;
  if constexpr (!kIsOperand<Dq>) {
    return b;
  } else {
    const int64_t full = static_cast<int64_t>(gridDim.x) & ~int64_t(7);
    return b < full ? (b & 7) * (full >> 3) + (b >> 3) : b;
  }
}

constexpr int kOpBlockBytes = 3072;  // 32 rows x 128 columns at 6 bits
constexpr int kOpStorePolicy = 0;    // cache policy of the staged operand stores

// Offset of run j of a row inside its row block.
__device__ __forceinline__ int operand_slot(int row_in_block, int j) {
  return (j >> 2) * kOpBlockBytes + ((j >> 1) & 1) * 1536 + (32 * (j & 1) + row_in_block) * 24;
}

// 32 values in field order (value i -> bits [6 i, 6 i + 6)) to six dwords.
// The conversion takes the even-indexed values first and the odd-indexed
// second and interleaves them; every input is a half-integer of magnitude at
// most 7.5, so it is exact.
__device__ __forceinline__ void e2m3_pack32(const float (&h)[RUN], uint32_t (&w)[6]) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  f32x16 ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = h[2 * i];
    od[i] = h[2 * i + 1];
  }
  const auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
  w[0] = r[0];
  w[1] = r[1];
  w[2] = r[2];
  w[3] = r[3];
  w[4] = r[4];
  w[5] = r[5];
}

// One run per lane: the lane's 32 values v (factor kk) into the operand
// window `op_r` at byte offset `off` (kNowhere drops the run).
template <int B>
__device__ __forceinline__ void store_operand_run(const float (&v)[RUN], float kk, rsrc_t op_r, int off) {
  constexpr float kHalf = 0.5f * static_cast<float>((1 << B) - 1);
  float h[RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) h[i] = grid_code<B>(v[i], kk) - kHalf;
  uint32_t w[6];
  e2m3_pack32(h, w);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, op_r, off, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[2], w[3]}, op_r, off == kNowhere ? kNowhere : off + 8, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[4], w[5]}, op_r, off == kNowhere ? kNowhere : off + 16, 0, 0);
}

// Matrix-core kernels: v[8 j .. 8 j + 7] of lane (g, n) are entries
// 8 g .. 8 g + 7 of run 16 j + n (factor kk[j]).  Each slot's eight fields
// (48 bits) are split into a low dword and a high half-word, and a
// transpose between lane quarters and slots hands lane l the four quarters
// of run l: its six dwords, in field order.
// The operand words of levels h already computed (in the layout of v).
__device__ __forceinline__ void mfma_operand_words_of_levels(const float (&h)[RUN], uint32_t (&w)[6]) {
  uint32_t d[6];
  e2m3_pack32(h, d);
  uint32_t lo[4] = {d[0], (d[1] >> 16) | (d[2] << 16), d[3], (d[4] >> 16) | (d[5] << 16)};
  uint32_t hi[4] = {d[1] & 0xFFFFu, d[2] >> 16, d[4] & 0xFFFFu, d[5] >> 16};
  transpose_quarters(lo);
  transpose_quarters(hi);
  w[0] = lo[0];
  w[1] = hi[0] | (lo[1] << 16);
  w[2] = (lo[1] >> 16) | (hi[1] << 16);
  w[3] = lo[2];
  w[4] = hi[2] | (lo[3] << 16);
  w[5] = (lo[3] >> 16) | (hi[3] << 16);
}

template <int B>
__device__ __forceinline__ void mfma_operand_words(const float (&v)[RUN], const float (&kk)[4], uint32_t (&w)[6]) {
  constexpr float kHalf = 0.5f * static_cast<float>((1 << B) - 1);
  float h[RUN];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) h[8 * j + i] = grid_code<B>(v[8 * j + i], kk[j]) - kHalf;
  mfma_operand_words_of_levels(h, w);
}

// Six operand dwords (one run) to byte offset `off` of `op_r` (kNowhere drops them).
__device__ __forceinline__ void store_operand_words(const uint32_t (&w)[6], rsrc_t op_r, int off) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, op_r, off, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[2], w[3]}, op_r, off == kNowhere ? kNowhere : off + 8, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[4], w[5]}, op_r, off == kNowhere ? kNowhere : off + 16, 0, 0);
}

// Operand staging in LDS for a workgroup that holds R consecutive rows of one
// 32-row block (R divides 32, the first row a multiple of R): in the tiled
// layout the R rows' slots of one run j are adjacent, 24 R contiguous bytes.
// Run j of row r goes to LDS byte j (24 R + 16) + 24 r (the 16-byte pad
// spreads the runs over the banks and keeps pieces 16-byte aligned); the
// pieces are then written out by the whole workgroup as 16-byte stores (8-byte
// ones when R is odd) that cover whole pieces, not 24-byte slots.
constexpr int kOpStagePad = 16;

__device__ __forceinline__ void stage_operand_words(uint8_t* st, int j, int r, int R, const uint32_t (&w)[6]) {
  u32x2* d = reinterpret_cast<u32x2*>(st + j * (24 * R + kOpStagePad) + 24 * r);
  d[0] = u32x2{w[0], w[1]};
  d[1] = u32x2{w[2], w[3]};
  d[2] = u32x2{w[4], w[5]};
}

// Write the staged pieces of runs 0 .. runs - 1 (R rows from row r0 of its
// block) through `op_r`, the window of that row block.  Thread t of n takes
// the words t, t + n, ...
__device__ __forceinline__ void flush_operand(const uint8_t* st, int R, int runs, int r0_in_block, rsrc_t op_r, int t,
                                              int n) {
  const int stride = 24 * R + kOpStagePad;
  if ((R & 1) == 0) {
    const int per = 3 * R / 2;  // 16-byte words per piece
    const int words = runs * per;
    for (int q = t; q < words; q += n) {
      const int j = q / per, within = q - j * per;
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + j * stride + 16 * within);
      __builtin_amdgcn_raw_buffer_store_b128(v, op_r, operand_slot(r0_in_block, j) + 16 * within, 0, kOpStorePolicy);
    }
  } else {
    const int per = 3 * R;  // 8-byte words per piece
    const int words = runs * per;
    for (int q = t; q < words; q += n) {
      const int j = q / per, within = q - j * per;
      const u32x2 v = *reinterpret_cast<const u32x2*>(st + j * stride + 8 * within);
      __builtin_amdgcn_raw_buffer_store_b64(v, op_r, operand_slot(r0_in_block, j) + 8 * within, 0, kOpStorePolicy);
    }
  }
}

// Codes, mask and scale of one run per lane, once its row's sum of squares is
// known.  The lane's codes go to offset 4 B lane of `codes_r`, its mask word to
// 4 lane of `mask_r`, and the row scale to `scale_off` of `scale_r` (kNowhere
// for all lanes but one per row).
template <int B>
__device__ __forceinline__ RowConsts fwd_quantise_store(const float (&v)[RUN], float tau, float ss,
                                                        const FwdConsts& k, int lane, rsrc_t codes_r, rsrc_t mask_r,
                                                        rsrc_t scale_r, int scale_off) {
  const RowConsts c = row_consts(ss, tau, k);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c.scale), scale_r, scale_off, 0, 0);
  const CodeWords<B> cw = quantise_run<B>(v, c.kk);
  uint32_t mw = 0u;
  push16_abs_le(mw, v + 16, c.thr);
  push16_abs_le(mw, v, c.thr);
  store_codes<B>(codes_r, lane, cw);
  __builtin_amdgcn_raw_buffer_store_b32(mw, mask_r, lane * 4, 0, kNonTemporal);
  return c;
}

// Dequantised values of the lane's run, stored through the wave's LDS stage
// as run first_run + lane of `dq` (runs at or past end_run dropped).
template <int B, typename Dq>
__device__ __forceinline__ void fwd_store_dq(const float (&v)[RUN], const RowConsts& c, Dq* dq, int64_t first_run,
                                             int64_t end_run, int lane, u32x4* stage) {
  if constexpr (DqOut<Dq>::kOn) {
    constexpr int UD = DqOut<Dq>::U;
    float q[RUN];
    grid_values<B, RUN>(v, c.kk, grid_step_half<B>(c.scale), q);
    uint32_t raw[4 * UD];
    narrow_run(q, raw);
    wave_store_runs<UD>(dq, first_run * UD, end_run * UD, lane, stage, raw);
  }
}

// Rows of at most 64 runs (cols <= 2048) with a power-of-two run count: a
// wave's 64 lanes hold 64 consecutive runs ("a tile", 64 / runs_per_row
// whole rows), so the row reduction stays inside the wave.  Each wave walks
// tiles tile0, tile0 + stride, ... with its loads running two tiles ahead of
// the arithmetic.
template <typename In, int LOGN, int B, typename Dq>
__global__ void __launch_bounds__(256)
    quest_fwd_tiles_kernel(const In* __restrict__ x, int64_t total_runs, int log_runs_per_row, FwdConsts k,
                           uint8_t* __restrict__ codes, float* __restrict__ scale, uint32_t* __restrict__ mask,
                           Dq* __restrict__ dq) {
  constexpr int U = sizeof(In) * 2;  // 16-byte pieces per run
  constexpr int US = U > DqOut<Dq>::U ? U : DqOut<Dq>::U;
  __shared__ u32x4 stage_all[4][64 * US];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  u32x4* stage = stage_all[wave];
  const int64_t total_pieces = total_runs * U;
  const int64_t rows = total_runs >> log_runs_per_row;
  const int64_t tiles = (total_runs + 63) >> 6;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  int64_t tile = fwd_wg_index<Dq>() * 4 + wave;
  if (tile >= tiles) return;
  const int rows_per_tile = 64 >> log_runs_per_row;
  const int scale_off = (lane & ((1 << log_runs_per_row) - 1)) == 0 ? (lane >> log_runs_per_row) * 4 : kNowhere;
  const int64_t codes_total = codes ? total_runs * 4 * B : 0;  // no codes: every code store is dropped

  auto process = [&](int64_t t, const u32x4 (&pieces)[U]) {
    uint32_t raw[4 * U];
    wave_stage<U>(pieces, lane, stage, raw);
    float v[RUN];
    float ss;
    const float tau = fwd_transform<In, LOGN>(raw, v, ss, lane);
    ss = group_sum(ss, log_runs_per_row);
    const int64_t run0 = t * 64;
    const rsrc_t codes_r = window_at(codes, run0 * 4 * B, codes_total, 64 * 4 * B);
    const rsrc_t mask_r = window_at(mask, run0 * 4, mask ? total_runs * 4 : 0, 64 * 4);
    const rsrc_t scale_r = window_at(scale, t * rows_per_tile * 4, rows * 4, rows_per_tile * 4);
    const RowConsts c = fwd_quantise_store<B>(v, tau, ss, k, lane, codes_r, mask_r, scale_r, scale_off);
    if constexpr (kIsOperand<Dq>) {
      // The tile's rows lie in one 32-row block (rows_per_tile divides 32).
      const int64_t row0 = t * rows_per_tile;
      const int64_t rb_bytes = static_cast<int64_t>(k.chunks) * kOpBlockBytes;
      const rsrc_t op_r = window_at(dq, (row0 >> 5) * rb_bytes, ((rows + 31) >> 5) * rb_bytes,
                                    static_cast<uint32_t>(rb_bytes));
      const int slot = operand_slot(static_cast<int>(row0 & 31) + (lane >> log_runs_per_row),
                                    lane & ((1 << log_runs_per_row) - 1));
      store_operand_run<B>(v, c.kk, op_r, run0 + lane < total_runs ? slot : kNowhere);
    } else {
      fwd_store_dq<B>(v, c, dq, run0, total_runs, lane, stage);
    }
  };

  // Three tile buffers, fetched two tiles ahead.  Every fetch is issued (past
  // the last tile it reads zeros), so each wait only has to cover loads
  // issued two tiles earlier: the stores of the previous tile and the newer
  // fetches stay in flight (loads and stores share one counter).
  u32x4 a[U], b[U], c[U];
  wave_fetch<U>(x, tile * 64 * U, total_pieces, lane, a);
  wave_fetch<U>(x, (tile + stride) * 64 * U, total_pieces, lane, b);
  for (;;) {
    wave_fetch<U>(x, (tile + 2 * stride) * 64 * U, total_pieces, lane, c);
    process(tile, a);
    tile += stride;
    if (tile >= tiles) break;
    wave_fetch<U>(x, (tile + 2 * stride) * 64 * U, total_pieces, lane, a);
    process(tile, b);
    tile += stride;
    if (tile >= tiles) break;
    wave_fetch<U>(x, (tile + 2 * stride) * 64 * U, total_pieces, lane, b);
    process(tile, c);
    tile += stride;
    if (tile >= tiles) break;
  }
}

// FP4 codes of 8 entries (factor kz), one dword, entry i in bits [4 i, 4 i + 4).
// The conversion keeps the sign of zero; the zero level gets the +0 code.
__device__ __forceinline__ uint32_t fp4_codes8(const float* v, float kz) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * kz, v[1] * kz, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * kz, v[3] * kz, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * kz, v[5] * kz, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * kz, v[7] * kz, 1.0f, 3);
  const uint32_t t = ~w;
  const uint32_t neg_zero = (w >> 3) & (t >> 2) & (t >> 1) & t & 0x11111111u;  // nibbles equal to 8
  return w ^ (neg_zero << 3);
}

// E2M1 magnitude of a 3-bit code.
__device__ __forceinline__ float e2m1_mag(uint32_t c) {
  const uint32_t e = c >> 1, m = c & 1u;
  return e == 0 ? 0.5f * static_cast<float>(m) : (1.f + 0.5f * static_cast<float>(m)) * static_cast<float>(1u << (e - 1));
}

// Codes and mask of a wave's four 16-run groups after the matrix-core
// transform: v[8 j .. 8 j + 7] of lane (g, n) are outputs 8 g .. 8 g + 7 of
// run 16 j + n, quantised with kk[j] and tested against thr[j].  Codes and
// mask bits are packed per slot (8 entries); a transpose between lane
// quarters and slots then hands lane l all four quarters of run l, stored at
// run l of the windows `codes_r` (4 B bytes per run) and `mask_r` (a dword
// per run).
// kFp4: FP4 codes (E2M1 patterns of the nearest level, B = 4) instead of the
// midrise grid's.
// kLevels (b = 2 or 4, midrise grid): also returns in h the levels
// h = u - (L - 1)/2 of the codes, in the layout of v, converted from the code
// bytes (for the matrix-core operand, which holds those levels).
template <int B, bool kFp4 = false, bool kLevels = false>
__device__ __forceinline__ void mfma_quantise_store(const float (&v)[RUN], const float (&kk)[4],
                                                    const float (&thr)[4], int lane, rsrc_t codes_r, rsrc_t mask_r,
                                                    float* h = nullptr) {
  static_assert(!kFp4 || B == 4, "FP4 codes are 4 bits");
  static_assert(!kLevels || (!kFp4 && (B == 2 || B == 4)), "levels from byte codes: midrise grid, b = 2 or 4");
  uint32_t cp[4], mp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kLevels) {
      uint32_t acc[8 / B];
      quantise8_bytes<B>(v + 8 * j, kk[j], acc);
      cp[j] = pack8_bytes<B>(acc);
      levels8_from_bytes<B>(acc, h + 8 * j);
    } else {
      cp[j] = kFp4 ? fp4_codes8(v + 8 * j, kk[j]) : quantise8<B>(v + 8 * j, kk[j]);
    }
    mp[j] = 0u;
    push8_abs_le(mp[j], v + 8 * j, thr[j]);
  }
  transpose_quarters(cp);
  transpose_quarters(mp);
  CodeWords<B> cw;
  if constexpr (B == 1) {
    cw.w[0] = cp[0] | (cp[1] << 8) | (cp[2] << 16) | (cp[3] << 24);
  } else if constexpr (B == 2) {
    cw.w[0] = cp[0] | (cp[1] << 16);
    cw.w[1] = cp[2] | (cp[3] << 16);
  } else if constexpr (B == 3) {
    cw.w[0] = cp[0] | (cp[1] << 24);
    cw.w[1] = (cp[1] >> 8) | (cp[2] << 16);
    cw.w[2] = (cp[2] >> 16) | (cp[3] << 8);
  } else {
    cw.w[0] = cp[0];
    cw.w[1] = cp[1];
    cw.w[2] = cp[2];
    cw.w[3] = cp[3];
  }
  const uint32_t mw = mp[0] | (mp[1] << 8) | (mp[2] << 16) | (mp[3] << 24);
  // Default cache policy: measured 0.4 us faster than non-temporal stores at
  // 16384 x 2048 (the loads stay non-temporal).
  store_codes<B, 0>(codes_r, lane, cw);
  __builtin_amdgcn_raw_buffer_store_b32(mw, mask_r, lane * 4, 0, 0);
}

// Dequantised values of the wave's four 16-run groups (layout of
// mfma_quantise_store's inputs) into the window `dq_r` of the wave's 64 runs:
// lane (g, n) holds entries 8 g .. 8 g + 7 of run 16 j + n in slot j, which
// it stores as 16 (bf16) or 32 (fp32) contiguous bytes; each store
// instruction covers one contiguous stretch, as the loads do.
// kFp4: FP4 levels, c = s / 6, as quest_dequantize_fp4 computes them.
template <int B, typename Dq, bool kFp4 = false>
__device__ __forceinline__ void mfma_store_dq(const float (&v)[RUN], const float (&kk)[4], const float (&c)[4],
                                              int lane, rsrc_t dq_r) {
  if constexpr (DqOut<Dq>::kOn) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float q[8];
      if constexpr (kFp4) {
        const uint32_t w = fp4_codes8(v + 8 * j, kk[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t code = (w >> (4 * i)) & 15u;
          const float mag = e2m1_mag(code & 7u) * c[j];
          q[i] = (code & 8u) ? -mag : mag;
        }
      } else {
        grid_values<B, 8>(v + 8 * j, kk[j], c[j], q);
      }
      if constexpr (sizeof(Dq) == 2) {
        const u32x4 w = {pack_bf16x2(q[0], q[1]), pack_bf16x2(q[2], q[3]), pack_bf16x2(q[4], q[5]),
                         pack_bf16x2(q[6], q[7])};
        __builtin_amdgcn_raw_buffer_store_b128(w, dq_r, 64 * (16 * j + n) + 16 * g, 0, kNonTemporal);
      } else {
        const u32x4 w0 = {__float_as_uint(q[0]), __float_as_uint(q[1]), __float_as_uint(q[2]), __float_as_uint(q[3])};
        const u32x4 w1 = {__float_as_uint(q[4]), __float_as_uint(q[5]), __float_as_uint(q[6]), __float_as_uint(q[7])};
        __builtin_amdgcn_raw_buffer_store_b128(w0, dq_r, 128 * (16 * j + n) + 32 * g, 0, kNonTemporal);
        __builtin_amdgcn_raw_buffer_store_b128(w1, dq_r, 128 * (16 * j + n) + 32 * g + 16, 0, kNonTemporal);
      }
    }
  }
}

// bf16 rows of 16, 32 or 64 runs (512, 1024 or 2048 columns) on the matrix
// cores.  A wave's tile is 64 runs (64 / 2^LOGR whole rows) held as four
// 16-run groups: slot j of lane (g, n) holds outputs 8 g .. 8 g + 7 of run
// 16 j + n (H_32 applied by the MFMA), then the cross-lane stages finish the
// block (runs of one block are neighbouring n).  Codes and mask bits are
// packed per slot (8 entries) and a transpose between lane quarters and
// slots hands lane l all four quarters of run l, which it stores as in the
// run-per-lane kernels.  Each wave takes one tile and the launch covers every
// tile: short-lived waves of few registers (50 at b = 4), eight per SIMD,
// which the hardware refills as they finish, kept more loads in flight than
// a grid-stride loop with its loads one to three tiles ahead.
// kQuant = false (operand calls without codes and mask) leaves the codes and
// mask work out of the build.
template <int LOGN, int B, int LOGR, typename Dq, bool kQuant, bool kFp4 = false>
__device__ __forceinline__ void fwd_mfma_tile(const uint16_t* __restrict__ x, int64_t total_runs, const FwdConsts& k,
                                              uint8_t* __restrict__ codes, float* __restrict__ scale,
                                              uint32_t* __restrict__ mask, Dq* __restrict__ dq, int64_t tile, int lane,
                                              int wave, uint8_t* opstage) {
  static_assert(LOGR >= 4 && LOGR <= 6, "16, 32 or 64 runs per row");
  constexpr int ROWS = 64 >> LOGR;  // rows per tile
  const int64_t rows = total_runs >> LOGR;
  const bf16x8_t h0 = hadamard_fragment(lane, 0);
  const bf16x8_t h1 = hadamard_fragment(lane, 1);
  const int in_off = 64 * (lane & 15) + 16 * (lane >> 4);
  const int scale_off = lane < ROWS ? lane * 4 : kNowhere;
  const int64_t codes_total = codes ? total_runs * 4 * B : 0;  // no codes: every code store is dropped

  auto fetch = [&](int64_t t, u32x4 (&f)[4]) {
    const rsrc_t r = window_at(x, t * 4096, total_runs * 64, 4096);
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __builtin_amdgcn_raw_buffer_load_b128(r, in_off + 1024 * j, 0, kNonTemporal);
  };

  auto process = [&](int64_t t, const u32x4 (&f)[4]) {
    float v[RUN];
    float part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mfma_run_outputs(h0, h1, f[j], v + 8 * j);
      part[j] = sum_squares_fragment(f[j]);
    }
    // Row sums of squares: slot j belongs to row j / (4 / ROWS) of the tile.
    float ss[ROWS];
    if constexpr (ROWS == 1) {
      ss[0] = group_sum((part[0] + part[1]) + (part[2] + part[3]), 6);
    } else if constexpr (ROWS == 2) {
      ss[0] = group_sum(part[0] + part[1], 6);
      ss[1] = group_sum(part[2] + part[3], 6);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) ss[j] = group_sum(part[j], 6);
    }
    const float tau = fwht_cross_lanes<LOGN, true>(v, lane);
    float kk[4], thr[4], ch[4], sc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const RowConsts c = row_consts(ss[r], tau, k);
      sc[r] = c.scale;
#pragma unroll
      for (int j = r * (4 / ROWS); j < (r + 1) * (4 / ROWS); ++j) {
        kk[j] = c.kk;
        thr[j] = c.thr;
        ch[j] = kFp4 ? c.scale / 6.f : grid_step_half<B>(c.scale);
      }
    }
    const int64_t run0 = t * 64;
    // With codes and an operand, the operand's levels come from the code
    // bytes (b = 2, 4) instead of a second rounding of v.
    constexpr bool kLevels = kIsOperand<Dq> && kQuant && !kFp4 && (B == 2 || B == 4);
    float h[kLevels ? RUN : 1];
    if (kQuant)
      mfma_quantise_store<B, kFp4, kLevels>(v, kk, thr, lane,
                                            window_at(codes, run0 * 4 * B, codes_total, 64 * 4 * B),
                                            window_at(mask, run0 * 4, mask ? total_runs * 4 : 0, 64 * 4), h);
    if constexpr (kIsOperand<Dq>) {
      // After the transpose lane l holds run l of the tile.  The workgroup's
      // four tiles are 4 ROWS consecutive rows of one 32-row block.
      uint32_t w[6];
      if constexpr (kLevels)
        mfma_operand_words_of_levels(h, w);
      else
        mfma_operand_words<B>(v, kk, w);
      stage_operand_words(opstage, lane & ((1 << LOGR) - 1), wave * ROWS + (lane >> LOGR), 4 * ROWS, w);
      __syncthreads();
      const int64_t row0 = (t - wave) * ROWS;
      const int64_t rb_bytes = static_cast<int64_t>(k.chunks) * kOpBlockBytes;
      const rsrc_t op_r = window_at(dq, (row0 >> 5) * rb_bytes, ((rows + 31) >> 5) * rb_bytes,
                                    static_cast<uint32_t>(rb_bytes));
      flush_operand(opstage, 4 * ROWS, 1 << LOGR, static_cast<int>(row0 & 31), op_r, static_cast<int>(threadIdx.x),
                    256);
      __syncthreads();
    } else if constexpr (DqOut<Dq>::kOn) {
      constexpr int64_t RB = 32 * sizeof(Dq);  // bytes per run
      mfma_store_dq<B, Dq, kFp4>(v, kk, ch, lane, window_at(dq, run0 * RB, total_runs * RB, 64 * RB));
    }
    float my_scale = sc[0];
#pragma unroll
    for (int r = 1; r < ROWS; ++r) my_scale = lane == r ? sc[r] : my_scale;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(my_scale),
                                          window_at(scale, t * ROWS * 4, rows * 4, ROWS * 4), scale_off, 0, 0);
  };

  u32x4 f[4];
  fetch(tile, f);
  process(tile, f);
}

template <int LOGN, int B, int LOGR, typename Dq, bool kQuant = true, bool kFp4 = false>
__global__ void __launch_bounds__(256)
    quest_fwd_mfma_kernel(const uint16_t* __restrict__ x, int64_t total_runs, FwdConsts k,
                          uint8_t* __restrict__ codes, float* __restrict__ scale, uint32_t* __restrict__ mask,
                          Dq* __restrict__ dq) {
  constexpr int ROWS = 64 >> LOGR;  // rows per tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t tiles = (total_runs + 63) >> 6;
  const int64_t tile = fwd_wg_index<Dq>() * 4 + wave;
  // The operand is staged per workgroup (a barrier), so all four waves of
  // the last workgroup run: a wave past the last tile computes on zeros and
  // every store it makes is dropped or lands in padding.
  if (!kIsOperand<Dq> && tile >= tiles) return;
  __shared__ __attribute__((aligned(16))) uint8_t opstage[kIsOperand<Dq> ? 64 * (24 * 4 * ROWS + kOpStagePad) : 16];
  fwd_mfma_tile<LOGN, B, LOGR, Dq, kQuant, kFp4>(x, total_runs, k, codes, scale, mask, dq, tile, lane, wave,
                                                 opstage);
}

// Several tensors in one launch (quest_quantize_fwd_group): tensors of one
// width of at most 2048 columns, each tensor's tiles following the previous
// tensor's (a wave finds its tensor by comparing its tile with the running
// tile counts: a scan over compile-time indices, so the table stays in
// scalar registers; per tensor the work is quest_fwd_mfma_kernel's, and a
// workgroup may span two tensors, with no barrier in this path), then the
// rows of wider tensors (2560 to 8192 columns), one row per workgroup as in
// the matrix-core row kernel.  The launch takes the wide rows' workgroups
// first, then the tile workgroups.
constexpr int kFwdGroupMax = 8;
constexpr int kFwdGroupWideMax = 4;

struct FwdGroup {
  int count;                               // tensors in this launch, 0 .. kFwdGroupMax
  int64_t first_tile[kFwdGroupMax + 1];    // running tile counts; first_tile[count] = all tiles
  int64_t total_runs[kFwdGroupMax];
  const uint16_t* x[kFwdGroupMax];
  uint8_t* codes[kFwdGroupMax];
  float* scale[kFwdGroupMax];
  uint32_t* mask[kFwdGroupMax];
  // Wide tensors (rows of 16 m runs, 4 < m <= 16): one row per workgroup,
  // before the tile workgroups.
  int wide_count;                               // 0 .. kFwdGroupWideMax
  int64_t wide_first_row[kFwdGroupWideMax + 1];  // running row counts
  int wide_runs[kFwdGroupWideMax];               // runs per row
  float wide_inv_cols[kFwdGroupWideMax];
  const uint16_t* wide_x[kFwdGroupWideMax];
  uint8_t* wide_codes[kFwdGroupWideMax];
  float* wide_scale[kFwdGroupWideMax];
  uint32_t* wide_mask[kFwdGroupWideMax];
};

// Dynamic LDS of the row-per-workgroup kernels (sized at launch).
extern __shared__ u32x4 rows_lds[];

// bf16 rows of 16 m runs (m > 4: more than 2048 columns, a multiple of 512)
// on the matrix cores.  A workgroup holds rows_per_wg whole rows; wave w
// takes runs 64 w .. 64 w + 63 of the workgroup as four 16-run groups, each
// inside one row, transformed and quantised as in quest_fwd_mfma_kernel.
// Each group's sum of squares goes to LDS; after a barrier every wave adds
// up the groups of its rows in a fixed order.  Groups past the workgroup's
// rows (when rows_per_wg * runs_per_row is not a multiple of 64) read zeros
// and their stores fall outside the workgroup's windows.  One workgroup per
// block of rows (no grid-stride loop): with a barrier per block, letting the
// hardware refill compute units as workgroups finish hides latency better
// than a resident loop.
template <int LOGN, int B, typename Dq, bool kQuant, bool kMayIdle = false>
__device__ __forceinline__ void fwd_mfma_rows(const uint16_t* __restrict__ x, int64_t rows, int runs_per_row,
                                              int rows_per_wg, const FwdConsts& k, uint8_t* __restrict__ codes,
                                              float* __restrict__ scale, uint32_t* __restrict__ mask,
                                              Dq* __restrict__ dq, int64_t wg) {
  __shared__ float group_ss[64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t total_runs = rows * runs_per_row;
  const uint32_t wg_runs = static_cast<uint32_t>(rows_per_wg * runs_per_row);
  const int64_t wg_first_run = wg * wg_runs;
  const int groups_per_row = runs_per_row >> 4;
  const bf16x8_t h0 = hadamard_fragment(lane, 0);
  const bf16x8_t h1 = hadamard_fragment(lane, 1);

  // kMayIdle: the grouped launch, whose 256-lane workgroups each take one
  // row of at most 256 runs.  A wave holding no run of that row skips the
  // loads and the transform and leaves after the barrier (the other launches
  // start only the waves their rows need).
  const bool idle = kMayIdle && 64 * wave >= static_cast<int>(wg_runs);
  float v[RUN];
  float tau = 1.f;
  if (!idle) {
    const rsrc_t in_r = window_at(x, wg_first_run * 64, total_runs * 64, wg_runs * 64);
    const int in_off = wave * 4096 + 64 * (lane & 15) + 16 * (lane >> 4);
    u32x4 f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __builtin_amdgcn_raw_buffer_load_b128(in_r, in_off + 1024 * j, 0, kNonTemporal);
    float part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mfma_run_outputs(h0, h1, f[j], v + 8 * j);
      part[j] = group_sum(sum_squares_fragment(f[j]), 6);
    }
    if (lane < 4) group_ss[4 * wave + lane] = lane == 0 ? part[0] : lane == 1 ? part[1] : lane == 2 ? part[2] : part[3];
    tau = fwht_cross_lanes<LOGN, true>(v, lane);
  }
  __syncthreads();
  if constexpr (kMayIdle && !kIsOperand<Dq>) {
    if (idle) return;
  }

  // Row of each slot (wave-uniform); a wave's 64 runs touch at most two rows.
  const int row_a = (4 * wave) / groups_per_row;
  const int row_b = (4 * wave + 3) / groups_per_row;
  float ss_a = 0.f, ss_b = 0.f;
  if (row_a < rows_per_wg) {
    const float* g = group_ss + row_a * groups_per_row;
    for (int i = 0; i < groups_per_row; ++i) ss_a += g[i];
  }
  if (row_b != row_a && row_b < rows_per_wg) {
    const float* g = group_ss + row_b * groups_per_row;
    for (int i = 0; i < groups_per_row; ++i) ss_b += g[i];
  } else {
    ss_b = ss_a;
  }
  const RowConsts ca = row_consts(ss_a, tau, k);
  const RowConsts cb = row_consts(ss_b, tau, k);
  float kk[4], thr[4], ch[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool in_a = (4 * wave + j) / groups_per_row == row_a;
    kk[j] = in_a ? ca.kk : cb.kk;
    thr[j] = in_a ? ca.thr : cb.thr;
    ch[j] = grid_step_half<B>(in_a ? ca.scale : cb.scale);
  }
  // The wave's windows end where the workgroup's rows end: runs past them
  // belong to the next workgroup.
  const int64_t run0 = wg_first_run + 64 * wave;
  const int64_t run_end = wg_first_run + wg_runs < total_runs ? wg_first_run + wg_runs : total_runs;
  // With codes and an operand, the operand's levels come from the code bytes
  // (b = 2, 4) instead of a second rounding of v.
  constexpr bool kLevels = kIsOperand<Dq> && kQuant && (B == 2 || B == 4);
  float h[kLevels ? RUN : 1];
  if (kQuant)
    mfma_quantise_store<B, false, kLevels>(v, kk, thr, lane,
                                           window_at(codes, run0 * 4 * B, codes ? run_end * 4 * B : 0, 64 * 4 * B),
                                           window_at(mask, run0 * 4, mask ? run_end * 4 : 0, 64 * 4), h);
  if constexpr (kIsOperand<Dq>) {
    // After the transpose lane l holds run 64 w + l of the workgroup.  The
    // workgroup's rows lie in one 32-row block (rows_per_wg divides 32 and
    // the first row is a multiple of it), where run j of its rows is one
    // piece of 24 rows_per_wg bytes: the runs are staged in LDS and written
    // as whole pieces.  In the last block rows past `rows` land in the
    // padding rows.
    const int64_t row0 = wg * rows_per_wg;
    const int64_t rb_bytes = static_cast<int64_t>(k.chunks) * kOpBlockBytes;
    const rsrc_t op_r = window_at(dq, (row0 >> 5) * rb_bytes, ((rows + 31) >> 5) * rb_bytes,
                                  static_cast<uint32_t>(rb_bytes));
    const int wr = 64 * wave + lane;
    const int lrow = wr / runs_per_row;
    uint32_t w[6];
    if constexpr (kLevels)
      mfma_operand_words_of_levels(h, w);
    else
      mfma_operand_words<B>(v, kk, w);
    uint8_t* st = reinterpret_cast<uint8_t*>(rows_lds);
    if (lrow < rows_per_wg) stage_operand_words(st, wr - lrow * runs_per_row, lrow, rows_per_wg, w);
    __syncthreads();
    flush_operand(st, rows_per_wg, runs_per_row, static_cast<int>(row0 & 31), op_r, static_cast<int>(threadIdx.x),
                  static_cast<int>(blockDim.x));
  } else if constexpr (DqOut<Dq>::kOn) {
    constexpr int64_t RB = 32 * sizeof(Dq);  // bytes per run
    mfma_store_dq<B, Dq>(v, kk, ch, lane, window_at(dq, run0 * RB, run_end * RB, 64 * RB));
  }
  // Slot j stores its row's scale when it holds the row's first group.
  const int my_group = 4 * wave + (lane & 3);
  const int my_row = my_group / groups_per_row;
  const bool first = lane < 4 && my_group % groups_per_row == 0 && my_row < rows_per_wg;
  const float my_scale = my_row == row_a ? ca.scale : cb.scale;
  const rsrc_t scale_r =
      window_at(scale, wg * rows_per_wg * 4, rows * 4, rows_per_wg * 4);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(my_scale), scale_r, first ? my_row * 4 : kNowhere, 0, 0);
}

template <int LOGN, int B, typename Dq, bool kQuant = true>
__global__ void __launch_bounds__(1024)
    quest_fwd_mfma_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int runs_per_row, int rows_per_wg,
                               FwdConsts k, uint8_t* __restrict__ codes, float* __restrict__ scale,
                               uint32_t* __restrict__ mask, Dq* __restrict__ dq) {
  fwd_mfma_rows<LOGN, B, Dq, kQuant>(x, rows, runs_per_row, rows_per_wg, k, codes, scale, mask, dq,
                                     fwd_wg_index<Dq>());
}

// The operand output of bf16 rows of 16 m runs, 4 < m <= 4 NC, one row per
// wave and four rows per workgroup.  The wave loads its whole row at once (m 16-run groups as
// in quest_fwd_mfma_kernel; groups past the row read zeros), adds the
// groups' sums of squares in group order (the row kernel's order, so the
// scale is the same) and then transforms and quantises the row 64 runs at a
// time: no barrier before the quantisation.  The operand output stages the
// four rows' pieces in LDS (one barrier) and writes them as 96-byte pieces,
// as the row kernel does.
constexpr int kRowWaveRows = 4;  // rows (waves) per workgroup of quest_fwd_mfma_rowwave_kernel

template <int LOGN, int B, typename Dq, bool kQuant, int NC>
__global__ void __launch_bounds__(64 * kRowWaveRows)
    quest_fwd_mfma_rowwave_kernel(const uint16_t* __restrict__ x, int64_t rows, int runs_per_row, FwdConsts k,
                                  uint8_t* __restrict__ codes, float* __restrict__ scale,
                                  uint32_t* __restrict__ mask, Dq* __restrict__ dq) {
  constexpr int R = kRowWaveRows;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t row0 = fwd_wg_index<Dq>() * R;
  const int64_t row = row0 + wave;
  const int groups = runs_per_row >> 4;
  const int64_t total_runs = rows * runs_per_row;
  const int64_t run_first = row * runs_per_row;  // past the tensor for rows past `rows`
  const int64_t run_end = run_first + runs_per_row < total_runs ? run_first + runs_per_row : total_runs;
  const bf16x8_t h0 = hadamard_fragment(lane, 0);
  const bf16x8_t h1 = hadamard_fragment(lane, 1);
  const rsrc_t in_r = window_at(x, run_first * 64, total_runs * 64, static_cast<uint32_t>(runs_per_row) * 64);
  const int in_off = 64 * (lane & 15) + 16 * (lane >> 4);
  u32x4 f[4 * NC];
#pragma unroll
  for (int j = 0; j < 4 * NC; ++j) f[j] = __builtin_amdgcn_raw_buffer_load_b128(in_r, in_off + 1024 * j, 0, kNonTemporal);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4 * NC; ++j)
    if (j < groups) ss += group_sum(sum_squares_fragment(f[j]), 6);
  static_assert(kIsOperand<Dq>, "the operand output");
  uint8_t* st = reinterpret_cast<uint8_t*>(rows_lds);
  float row_scale = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float v[RUN];
#pragma unroll
    for (int j = 0; j < 4; ++j) mfma_run_outputs(h0, h1, f[4 * c + j], v + 8 * j);
    const float tau = fwht_cross_lanes<LOGN, true>(v, lane);
    const RowConsts rc = row_consts(ss, tau, k);
    row_scale = rc.scale;
    const float kk[4] = {rc.kk, rc.kk, rc.kk, rc.kk};
    const float thr[4] = {rc.thr, rc.thr, rc.thr, rc.thr};
    const int64_t run0 = run_first + 64 * c;
    constexpr bool kLevels = kQuant && (B == 2 || B == 4);
    float h[kLevels ? RUN : 1];
    if (kQuant)
      mfma_quantise_store<B, false, kLevels>(v, kk, thr, lane,
                                             window_at(codes, run0 * 4 * B, codes ? run_end * 4 * B : 0, 64 * 4 * B),
                                             window_at(mask, run0 * 4, mask ? run_end * 4 : 0, 64 * 4), h);
    // After the transpose lane l holds run 64 c + l of the row.
    uint32_t w[6];
    if constexpr (kLevels)
      mfma_operand_words_of_levels(h, w);
    else
      mfma_operand_words<B>(v, kk, w);
    if (64 * c + lane < runs_per_row) stage_operand_words(st, 64 * c + lane, wave, R, w);
  }
  const rsrc_t scale_r = window_at(scale, row0 * 4, rows * 4, R * 4);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(row_scale), scale_r, lane == 0 ? wave * 4 : kNowhere, 0, 0);
  // The four rows lie in one 32-row block (row0 is a multiple of 4); rows
  // past `rows` land in the last block's padding rows.
  const int64_t rb_bytes = static_cast<int64_t>(k.chunks) * kOpBlockBytes;
  const rsrc_t op_r = window_at(dq, (row0 >> 5) * rb_bytes, ((rows + 31) >> 5) * rb_bytes,
                                static_cast<uint32_t>(rb_bytes));
  __syncthreads();
  flush_operand(st, R, runs_per_row, static_cast<int>(row0 & 31), op_r, static_cast<int>(threadIdx.x), 64 * R);
}

template <int LOGN, int B, int LOGR>
__global__ void __launch_bounds__(256) quest_fwd_mfma_group_kernel(FwdGroup g, FwdConsts k) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t wide_wgs = g.wide_first_row[g.wide_count];
  if (static_cast<int64_t>(blockIdx.x) < wide_wgs) {
    // A row of a wide tensor: the row kernel's work with one row per
    // workgroup of four waves (runs past the row read zeros and store
    // nothing; a wave wholly past it only joins the barrier).  These
    // workgroups, each a longer chain (row load, barrier, quantise), are
    // dispatched first so that the short tile workgroups fill in behind them
    // instead of leaving them as the launch's tail.
    const int64_t row = static_cast<int64_t>(blockIdx.x);
    int i = 0;
#pragma unroll
    for (int j = 1; j < kFwdGroupWideMax; ++j)
      if (j < g.wide_count && row >= g.wide_first_row[j]) i = j;
    FwdConsts kw = k;
    kw.inv_cols = g.wide_inv_cols[i];
    fwd_mfma_rows<LOGN, B, void, true, true>(g.wide_x[i], g.wide_first_row[i + 1] - g.wide_first_row[i],
                                             g.wide_runs[i], 1, kw, g.wide_codes[i], g.wide_scale[i], g.wide_mask[i],
                                             nullptr, row - g.wide_first_row[i]);
    return;
  }
  const int64_t tile = (static_cast<int64_t>(blockIdx.x) - wide_wgs) * 4 + wave;
  const uint16_t* x = g.x[0];
  uint8_t* codes = g.codes[0];
  float* scale = g.scale[0];
  uint32_t* mask = g.mask[0];
  int64_t runs = g.total_runs[0], first = 0, end = g.first_tile[1];
#pragma unroll
  for (int i = 1; i < kFwdGroupMax; ++i) {
    if (i < g.count && tile >= g.first_tile[i]) {
      x = g.x[i];
      codes = g.codes[i];
      scale = g.scale[i];
      mask = g.mask[i];
      runs = g.total_runs[i];
      first = g.first_tile[i];
      end = g.first_tile[i + 1];
    }
  }
  if (tile >= end) return;
  fwd_mfma_tile<LOGN, B, LOGR, void, true>(x, runs, k, codes, scale, mask, nullptr, tile - first, lane, wave,
                                           nullptr);
}

// Several operand forwards in one launch (quest_quantize_fwd_op_group): bf16
// tensors whose rows all have 512, 1024 or 2048 entries.  Each tensor starts
// at a workgroup of its own, so a workgroup's four tiles are consecutive
// tiles of one tensor and stage its operand pieces together as in
// quest_fwd_mfma_kernel (a wave past its tensor's last tile computes on
// zeros, and its stores are dropped or land in the operand's padding rows);
// the XCD mapping of fwd_wg_index runs over the whole launch.  Per tensor the
// work is quest_fwd_mfma_kernel's, tile for tile, so the outputs are those
// of one call per tensor.
constexpr int kFwdOpGroupMax = 4;

struct FwdOpGroup {
  int count;                               // tensors in this launch, 1 .. kFwdOpGroupMax
  int64_t first_wg[kFwdOpGroupMax + 1];    // running workgroup counts; first_wg[count] = the grid
  int64_t total_runs[kFwdOpGroupMax];
  const uint16_t* x[kFwdOpGroupMax];
  uint8_t* codes[kFwdOpGroupMax];          // may be null (not written)
  float* scale[kFwdOpGroupMax];
  uint32_t* mask[kFwdOpGroupMax];          // may be null (not written)
  uint8_t* operand[kFwdOpGroupMax];
};

template <int LOGN, int B, int LOGR, bool kQuant>
__global__ void __launch_bounds__(256) quest_fwd_mfma_op_group_kernel(FwdOpGroup g, FwdConsts k) {
  constexpr int ROWS = 64 >> LOGR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t wg = fwd_wg_index<OperandOut>();
  const uint16_t* x = g.x[0];
  uint8_t* codes = g.codes[0];
  float* scale = g.scale[0];
  uint32_t* mask = g.mask[0];
  uint8_t* operand = g.operand[0];
  int64_t runs = g.total_runs[0], first = 0;
#pragma unroll
  for (int i = 1; i < kFwdOpGroupMax; ++i) {
    if (i < g.count && wg >= g.first_wg[i]) {
      x = g.x[i];
      codes = g.codes[i];
      scale = g.scale[i];
      mask = g.mask[i];
      operand = g.operand[i];
      runs = g.total_runs[i];
      first = g.first_wg[i];
    }
  }
  __shared__ __attribute__((aligned(16))) uint8_t opstage[64 * (24 * 4 * ROWS + kOpStagePad)];
  fwd_mfma_tile<LOGN, B, LOGR, OperandOut, kQuant>(x, runs, k, codes, scale, mask,
                                                   reinterpret_cast<OperandOut*>(operand), (wg - first) * 4 + wave,
                                                   lane, wave, opstage);
}


// LDS of the row-per-workgroup kernels, sized at launch by their wave count:
// per wave a staging area of 64 * US 16-byte slots, then one float per lane
// for the partial row sums.

inline size_t rows_lds_bytes(int threads, int us) {
  return static_cast<size_t>(threads / 64) * 64 * static_cast<size_t>(us) * 16 + static_cast<size_t>(threads) * 4;
}

template <int US>
__device__ __forceinline__ float* rows_part() {
  return reinterpret_cast<float*>(rows_lds + (blockDim.x >> 6) * 64 * US);
}

// Rows that span several wavefronts (or whose run count is not a power of
// two): a workgroup holds rows_per_wg whole rows, lane t holding run
// (first run of the workgroup) + t.  Lanes reduce in aligned groups of
// 2^log_group lanes (a power of two dividing runs_per_row), group sums go
// through LDS and every lane adds up the groups of its row in the same order.
// Lanes past the workgroup's rows compute on whatever they loaded (DPP needs
// whole quads) and their stores fall outside the workgroup's windows.
template <typename In, int LOGN, int B, typename Dq>
__global__ void __launch_bounds__(1024)
    quest_fwd_rows_kernel(const In* __restrict__ x, int64_t rows, int runs_per_row, int rows_per_wg, int log_group,
                          FwdConsts k, uint8_t* __restrict__ codes, float* __restrict__ scale,
                          uint32_t* __restrict__ mask, Dq* __restrict__ dq) {
  constexpr int U = sizeof(In) * 2;
  constexpr int US = U > DqOut<Dq>::U ? U : DqOut<Dq>::U;
  u32x4* const stage_all = rows_lds;
  float* const part = rows_part<US>();
  const int64_t wg = fwd_wg_index<Dq>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lrow = tid / runs_per_row;
  const int run_in_row = tid - lrow * runs_per_row;
  const int64_t total_runs = rows * runs_per_row;
  const int64_t wg_first_run = wg * rows_per_wg * runs_per_row;
  const int wave_tid0 = __builtin_amdgcn_readfirstlane(tid) & ~63;

  uint32_t raw[4 * U];
  u32x4* const stage = stage_all + (wave_tid0 >> 6) * 64 * US;
  wave_load_runs<U>(x, (wg_first_run + wave_tid0) * U, total_runs * U, lane, stage, raw);
  float v[RUN];
  float ss;
  const float tau = fwd_transform<In, LOGN>(raw, v, ss, tid);

  ss = group_sum(ss, log_group);
  if ((tid & ((1 << log_group) - 1)) == 0) part[tid >> log_group] = ss;
  __syncthreads();
  const int per_row = runs_per_row >> log_group;
  ss = 0.f;
  if (lrow < rows_per_wg) {
    const float* pr = part + lrow * per_row;
    for (int i = 0; i < per_row; ++i) ss += pr[i];
  }
  const uint32_t wg_runs = static_cast<uint32_t>(rows_per_wg * runs_per_row);
  const rsrc_t codes_r = window_at(codes, wg_first_run * 4 * B, codes ? total_runs * 4 * B : 0, wg_runs * 4 * B);
  const rsrc_t mask_r = window_at(mask, wg_first_run * 4, mask ? total_runs * 4 : 0, wg_runs * 4);
  const rsrc_t scale_r =
      window_at(scale, wg * rows_per_wg * 4, rows * 4, rows_per_wg * 4);
  const int scale_off = (run_in_row == 0 && lrow < rows_per_wg) ? lrow * 4 : kNowhere;
  const RowConsts c = fwd_quantise_store<B>(v, tau, ss, k, tid, codes_r, mask_r, scale_r, scale_off);
  // Lanes past the workgroup's rows must not write the next workgroup's runs.
  const int64_t wg_end = wg_first_run + wg_runs < total_runs ? wg_first_run + wg_runs : total_runs;
  if constexpr (kIsOperand<Dq>) {
    const int64_t row0 = wg * rows_per_wg;
    const int64_t last = (row0 + rows_per_wg < rows ? row0 + rows_per_wg : rows) - 1;
    const int64_t rb_bytes = static_cast<int64_t>(k.chunks) * kOpBlockBytes;
    const int64_t rb0 = row0 >> 5;
    const rsrc_t op_r = window_at(dq, rb0 * rb_bytes, ((rows + 31) >> 5) * rb_bytes,
                                  static_cast<uint32_t>(((last >> 5) - rb0 + 1) * rb_bytes));
    const int64_t row = row0 + lrow;
    const bool live = lrow < rows_per_wg && row < rows;
    const int off = live ? static_cast<int>(((row >> 5) - rb0) * rb_bytes) +
                               operand_slot(static_cast<int>(row & 31), run_in_row)
                         : kNowhere;
    store_operand_run<B>(v, c.kk, op_r, off);
  } else {
    fwd_store_dq<B>(v, c, dq, wg_first_run + wave_tid0, wg_end, lane, stage);
  }
}

// ----------------------------------------------------------------------------
// Trust-masked backward: one lane per run, no cross-row work.
// grad and grad_out may be the same buffer: every chunk is read and written
// by the same wave only, and its loads come before its stores.
// ----------------------------------------------------------------------------
template <typename G, int LOGN>
__global__ void __launch_bounds__(256)
    quest_bwd_kernel(const G* grad, const uint32_t* mask, int64_t total_runs, G* grad_out) {
  constexpr int U = sizeof(G) * 2;
  __shared__ u32x4 stage_all[4][64 * U];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  u32x4* stage = stage_all[wave];
  const int64_t run0 = static_cast<int64_t>(blockIdx.x) * 256 + wave * 64;  // first run of the wave
  const rsrc_t mask_r = window_at(mask, run0 * 4, total_runs * 4, 64 * 4);
  const uint32_t m = __builtin_amdgcn_raw_buffer_load_b32(mask_r, lane * 4, 0, kNonTemporal);
  uint32_t raw[4 * U];
  wave_load_runs<U>(grad, run0 * U, total_runs * U, lane, stage, raw);
  float v[RUN];
  widen_run_masked(raw, m, v);
  const float tau = fwht_block<LOGN>(v, lane);
  const float k = tau * BlockConst<LOGN>::rsqrt_n;
#pragma unroll
  for (int j = 0; j < RUN; ++j) v[j] *= k;
  narrow_run(v, raw);
  wave_store_runs<U>(grad_out, run0 * U, total_runs * U, lane, stage, raw);
}

// The same for bf16 gradients on the matrix cores, in the layout of
// quest_fwd_mfma_kernel: a wave's tile is 64 runs held as four 16-run groups,
// lane (g, n) loading the 16 bytes at 64 n + 16 g of each group (elements
// 8 g .. 8 g + 7 of run 16 j + n in slot j; one contiguous kilobyte per load
// instruction).  Each lane loads the mask dword of run l, and the transpose
// between lane quarters and slots hands slot j the mask of run 16 j + n.  The
// untrusted entries are zeroed in the bf16 fragment (each bit sign-extended
// over its half of a dword), H_32 is applied by two matrix instructions per
// group and the cross-run stages by DPP; the outputs, scaled by tau/sqrt(n)
// and narrowed to bf16, are stored in the pattern of the loads.  No LDS and
// no in-lane butterflies.  Tiles may straddle rows (the transform is per
// block, a block never straddles a 16-run group); a tile past the end of the
// tensor reads zeros and its stores are dropped.  In place is allowed: each
// tile is read and written by one wave, its loads before its stores.
template <int LOGN>
__global__ void __launch_bounds__(256)
    quest_bwd_mfma_kernel(const uint16_t* grad, const uint32_t* mask, int64_t total_runs, uint16_t* grad_out) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (tile * 64 >= total_runs) return;
  const int in_off = 64 * (lane & 15) + 16 * (lane >> 4);
  const rsrc_t g_r = window_at(grad, tile * 4096, total_runs * 64, 4096);
  u32x4 f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = __builtin_amdgcn_raw_buffer_load_b128(g_r, in_off + 1024 * j, 0, kNonTemporal);
  const uint32_t m = __builtin_amdgcn_raw_buffer_load_b32(window_at(mask, tile * 256, total_runs * 4, 256), lane * 4,
                                                          0, kNonTemporal);
  const bf16x8_t h0 = hadamard_fragment(lane, 0);
  const bf16x8_t h1 = hadamard_fragment(lane, 1);
  uint32_t mq[4] = {m, m, m, m};
  transpose_quarters(mq);  // slot j: the mask of run 16 j + n
  const int shift = 8 * (lane >> 4);
  float v[RUN];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bits = static_cast<int>(mq[j] >> shift);  // bit e: element 8 g + e of the run
    const uint32_t d[4] = {f[j].x, f[j].y, f[j].z, f[j].w};
    uint32_t md[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t keep_lo = static_cast<uint32_t>(__builtin_amdgcn_sbfe(bits, 2 * i, 1));
      const uint32_t keep_hi = static_cast<uint32_t>(__builtin_amdgcn_sbfe(bits, 2 * i + 1, 1));
      md[i] = d[i] & ((keep_lo & 0xFFFFu) | (keep_hi & 0xFFFF0000u));
    }
    mfma_run_outputs(h0, h1, u32x4{md[0], md[1], md[2], md[3]}, v + 8 * j);
  }
  const float tau = fwht_cross_lanes<LOGN, true>(v, lane);
  const float k = tau * BlockConst<LOGN>::rsqrt_n;
  const rsrc_t o_r = window_at(grad_out, tile * 4096, total_runs * 64, 4096);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float* w = v + 8 * j;
    const u32x4 o = {pack_bf16x2(w[0] * k, w[1] * k), pack_bf16x2(w[2] * k, w[3] * k),
                     pack_bf16x2(w[4] * k, w[5] * k), pack_bf16x2(w[6] * k, w[7] * k)};
    __builtin_amdgcn_raw_buffer_store_b128(o, o_r, in_off + 1024 * j, 0, kNonTemporal);
  }
}

// ----------------------------------------------------------------------------
// Dequantise: one lane per run.
// ----------------------------------------------------------------------------
template <typename Out, int B>
__global__ void __launch_bounds__(256)
    quest_dequant_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scale, int64_t total_runs,
                         uint32_t runs_per_row, Out* __restrict__ out) {
  constexpr int U = sizeof(Out) * 2;
  __shared__ u32x4 stage_all[4][64 * U];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t run0 = static_cast<int64_t>(blockIdx.x) * 256 + wave * 64;
  // rows * 4 bytes stay below 2^32 (rows * cols < 2^36, cols >= 64).
  const uint32_t row = static_cast<uint32_t>((run0 + lane) / runs_per_row);
  const int64_t rows = total_runs / runs_per_row;
  const rsrc_t scale_r = window_at(scale, 0, rows * 4, 0xFFFFFFF0u);
  const float c = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(scale_r, static_cast<int>(row * 4), 0, 0)) /
                  static_cast<float>((1 << B) - 1);
  const CodeWords<B> cw = load_codes<B>(window_at(codes, run0 * 4 * B, total_runs * 4 * B, 64 * 4 * B), lane);
  float v[RUN];
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    const int u = static_cast<int>(get_code<B>(cw, j));
    v[j] = static_cast<float>(2 * u - (1 << B) + 1) * c;
  }
  uint32_t raw[4 * U];
  narrow_run(v, raw);
  // Default cache policy: a rebuilt operand is read by the product that
  // follows (the QAT layer's gradient products), which then finds it in the
  // last-level cache (a training step of the layer 12 us faster than with
  // non-temporal stores).
  wave_store_runs<U, 0>(out, run0 * U, total_runs * U, lane, stage_all[wave], raw);
}

// ----------------------------------------------------------------------------
// Packed b-bit codes (b <= 4) to the matrix-core operand: the levels
// h = u - (L - 1)/2 that quest_quantize_fwd_op writes for the same codes.  A
// workgroup takes one 32-row block and eight runs (two 128-column chunks):
// thread t converts run 8 G + t / 32 of row 32 R + t % 32, so a wave's 64 runs
// are 64 consecutive slots of the tiled layout (1536 contiguous bytes) and
// the workgroup's loads cover 128 contiguous code bytes of each of its 32
// rows.  Runs past the row and rows past the tensor are skipped (the
// operand's padding rows are not written).
// ----------------------------------------------------------------------------
template <int B>
__global__ void __launch_bounds__(256)
    quest_codes_to_operand_kernel(const uint8_t* __restrict__ codes, int64_t rows, int runs_per_row, int run_groups,
                                  uint8_t* __restrict__ operand) {
  constexpr float kHalf = 0.5f * static_cast<float>((1 << B) - 1);
  const int t = threadIdx.x;
  const int64_t rb = blockIdx.x / run_groups;  // 32-row block
  const int grp = static_cast<int>(blockIdx.x - rb * run_groups);
  const int r = t & 31, j = 8 * grp + (t >> 5);
  const bool live = rb * 32 + r < rows && j < runs_per_row;
  const int64_t row_bytes = static_cast<int64_t>(runs_per_row) * 4 * B;
  const rsrc_t codes_r = window_at(codes, rb * 32 * row_bytes, rows * row_bytes, static_cast<uint32_t>(32 * row_bytes));
  const CodeWords<B> cw = load_codes_at<B>(codes_r, live ? static_cast<int>(r * row_bytes) + 4 * B * j : kNowhere);
  float h[RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) h[i] = static_cast<float>(get_code<B>(cw, i)) - kHalf;
  uint32_t w[6];
  e2m3_pack32(h, w);
  const int64_t rb_bytes = static_cast<int64_t>(runs_per_row / 4) * kOpBlockBytes;
  const rsrc_t op_r = window_at(operand, rb * rb_bytes, ((rows + 31) >> 5) * rb_bytes, static_cast<uint32_t>(rb_bytes));
  store_operand_words(w, op_r, live ? operand_slot(r, j) : kNowhere);
}

// ----------------------------------------------------------------------------
// Launchers.
// ----------------------------------------------------------------------------
inline int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

inline int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// Workgroups (of four waves) launched for the tiled forward kernels: two per
// compute unit on the 256-CU MI355X, so each wave walks several tiles and its
// loads run ahead of the arithmetic.
constexpr int64_t kFwdTileWorkgroups = 512;

// Rows per workgroup of the matrix-core row kernel when it writes the operand.
constexpr int kOpRowsPerWorkgroup = 4;



// Per-launch constants of the forward kernels for rows of `cols` entries.
template <int LOGN, int B>
FwdConsts fwd_consts(double alpha, double trust, int64_t cols) {
  const double L = double(1 << B), sqrt_n = std::sqrt(double(1 << LOGN));
  FwdConsts k;
  k.alpha = static_cast<float>(alpha);
  k.kk = static_cast<float>((L - 1.0) / (2.0 * alpha * sqrt_n));
  // Trusted: |y| <= s + trust * Delta / 2, i.e. |v| <= alpha sqrt(n) (1 + trust / (L - 1)) RMS.
  k.thr = static_cast<float>(alpha * sqrt_n * (1.0 + trust / (L - 1.0)));
  k.inv_cols = static_cast<float>(1.0 / double(cols));
  k.chunks = static_cast<int>(cols / 128);
  return k;
}

// One grouped launch: every tile tensor of `g` has rows of `cols` entries,
// cols 512, 1024 or 2048 (16, 32 or 64 runs; any of them when g has no tile
// tensor), and its wide tensors rows of 2560 to 8192 entries; bf16, b <= 4.
template <int LOGN, int B>
hipError_t fwd_group_dispatch(const FwdGroup& g, int64_t cols, double alpha, hipStream_t stream) {
  const FwdConsts k = fwd_consts<LOGN, B>(alpha, 1.0, cols);
  const dim3 grid(static_cast<uint32_t>((g.first_tile[g.count] + 3) / 4 + g.wide_first_row[g.wide_count]));
  switch (cols / RUN) {
    case 16:
      hipLaunchKernelGGL((quest_fwd_mfma_group_kernel<LOGN, B, 4>), grid, dim3(256), 0, stream, g, k);
      break;
    case 32:
      hipLaunchKernelGGL((quest_fwd_mfma_group_kernel<LOGN, B, 5>), grid, dim3(256), 0, stream, g, k);
      break;
    default:
      hipLaunchKernelGGL((quest_fwd_mfma_group_kernel<LOGN, B, 6>), grid, dim3(256), 0, stream, g, k);
      break;
  }
  return hipGetLastError();
}

// One grouped operand launch: every tensor of `g` is bf16 with rows of
// `cols` entries (512, 1024 or 2048), b <= 4.  quant: some tensor asks for
// codes or mask (those of the others are null, so their stores are dropped).
template <int LOGN, int B>
hipError_t fwd_op_group_dispatch(const FwdOpGroup& g, int64_t cols, double alpha, double trust, bool quant,
                                 hipStream_t stream) {
  const FwdConsts k = fwd_consts<LOGN, B>(alpha, trust, cols);
  const dim3 grid(static_cast<uint32_t>(g.first_wg[g.count]));
  auto run = [&](auto logr, auto q) {
    hipLaunchKernelGGL((quest_fwd_mfma_op_group_kernel<LOGN, B, decltype(logr)::value, decltype(q)::value>), grid,
                       dim3(256), 0, stream, g, k);
  };
  auto run_logr = [&](auto logr) {
    if (quant)
      run(logr, std::true_type{});
    else
      run(logr, std::false_type{});
  };
  switch (cols / RUN) {
    case 16: run_logr(std::integral_constant<int, 4>{}); break;
    case 32: run_logr(std::integral_constant<int, 5>{}); break;
    default: run_logr(std::integral_constant<int, 6>{}); break;
  }
  return hipGetLastError();
}

template <typename In, int LOGN, int B, typename Dq>
hipError_t fwd_dispatch(const In* x, const FwdLaunch& a) {
  const int64_t rows = a.rows;
  const int runs_per_row = static_cast<int>(a.cols / RUN);
  const FwdConsts k = fwd_consts<LOGN, B>(a.alpha, a.trust, a.cols);
  uint32_t* mask32 = reinterpret_cast<uint32_t*>(a.mask);
  Dq* dq = static_cast<Dq*>(a.dq);
  hipStream_t stream = a.stream;
  if constexpr (sizeof(In) == 2 && B <= 4) {
    if constexpr (kIsOperand<Dq>) {
      if (a.allow_mfma && runs_per_row > 64 && runs_per_row <= 256 && runs_per_row % 16 == 0) {
        // The operand of rows up to 8192 columns: one row per wave
        // (quest_fwd_mfma_rowwave_kernel).  At 16384 x 5632 46.2-47.2 us
        // against 62.4-62.5 for the row kernel below, and 64.8-67.5 against
        // 80.7-83.0 with codes and mask.  The other outputs keep the row
        // kernel, which was faster for them (codes and mask alone: 46.2-47.4
        // against 58.1-58.2 us with one row per wave).
        const int nc = (runs_per_row / 16 + 3) / 4;  // 64-run chunks per row: 2, 3 or 4
        const int64_t grid = (rows + kRowWaveRows - 1) / kRowWaveRows;
        const size_t lds = static_cast<size_t>(runs_per_row) * (24 * kRowWaveRows + kOpStagePad);
        auto run = [&](auto chunks, auto quant) {
          hipLaunchKernelGGL(
              (quest_fwd_mfma_rowwave_kernel<LOGN, B, Dq, decltype(quant)::value, decltype(chunks)::value>),
              dim3(static_cast<uint32_t>(grid)), dim3(64 * kRowWaveRows), lds, stream, x, rows, runs_per_row, k,
              a.codes, a.scale, mask32, dq);
        };
        auto run_nc = [&](auto quant) {
          if (nc == 2)
            run(std::integral_constant<int, 2>{}, quant);
          else if (nc == 3)
            run(std::integral_constant<int, 3>{}, quant);
          else
            run(std::integral_constant<int, 4>{}, quant);
        };
        if (a.codes || a.mask)
          run_nc(std::true_type{});
        else
          run_nc(std::false_type{});
        return hipGetLastError();
      }
    }
    if (a.allow_mfma && runs_per_row > 64 && runs_per_row % 16 == 0) {
      // One row per workgroup when its last wave leaves at most an eighth of
      // the lanes idle (5632 columns: 176 runs in 3 waves): small workgroups
      // fill more of each compute unit's wave slots than one of whole waves
      // (4 rows, 11 waves: two per unit, 22 of 32 slots), 44.2 against
      // 47.0 us at 16384 x 5632.  Otherwise the fewest rows that fill whole
      // waves.
      const int padded = ((runs_per_row + 63) / 64) * 64;
      int rows_per_wg = 1;
      size_t lds = 0;
      if constexpr (kIsOperand<Dq>) {
        // The operand: several rows of one 32-row block per workgroup (a
        // power of two, at most kOpRowsPerWorkgroup and 1024 threads), so
        // that its pieces are 24 rows_per_wg contiguous bytes.
        rows_per_wg = kOpRowsPerWorkgroup;
        while (rows_per_wg > 1 && rows_per_wg * runs_per_row > 1024) rows_per_wg >>= 1;
        lds = static_cast<size_t>(runs_per_row) * (24 * rows_per_wg + kOpStagePad);
      } else if (8 * (padded - runs_per_row) > padded) {
        rows_per_wg = 64 / gcd_int(runs_per_row, 64);
        if (rows_per_wg * runs_per_row > 1024) rows_per_wg = 1024 / runs_per_row;
        if (rows_per_wg < 1) rows_per_wg = 1;
      }
      const int threads = ((rows_per_wg * runs_per_row + 63) / 64) * 64;
      const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
      // An operand call that asks for neither codes nor mask runs the build without them.
      auto run = [&](auto quant) {
        hipLaunchKernelGGL((quest_fwd_mfma_rows_kernel<LOGN, B, Dq, decltype(quant)::value>),
                           dim3(static_cast<uint32_t>(grid)), dim3(threads), lds, stream, x, rows, runs_per_row,
                           rows_per_wg, k, a.codes, a.scale, mask32, dq);
      };
      bool quant = true;
      if constexpr (kIsOperand<Dq>) quant = a.codes || a.mask;
      if (quant)
        run(std::true_type{});
      else if constexpr (kIsOperand<Dq>)
        run(std::false_type{});
      return hipGetLastError();
    }
    if (a.allow_mfma && (runs_per_row == 16 || runs_per_row == 32 || runs_per_row == 64)) {
      const int64_t total_runs = rows * runs_per_row;
      const int64_t tiles = (total_runs + 63) / 64;
      const dim3 grid(static_cast<uint32_t>((tiles + 3) / 4));  // one tile per wave
      // An operand call that asks for neither codes nor mask runs the build without them.
      auto run = [&](auto logr, auto quant) {
        hipLaunchKernelGGL((quest_fwd_mfma_kernel<LOGN, B, decltype(logr)::value, Dq, decltype(quant)::value>), grid,
                           dim3(256), 0, stream, x, total_runs, k, a.codes, a.scale, mask32, dq);
      };
      auto run_logr = [&](auto logr) {
        if constexpr (kIsOperand<Dq>) {
          if (!a.codes && !a.mask) return run(logr, std::false_type{});
        }
        run(logr, std::true_type{});
      };
      if (runs_per_row == 16)
        run_logr(std::integral_constant<int, 4>{});
      else if (runs_per_row == 32)
        run_logr(std::integral_constant<int, 5>{});
      else
        run_logr(std::integral_constant<int, 6>{});
      return hipGetLastError();
    }
  }
  if (runs_per_row <= 64 && (runs_per_row & (runs_per_row - 1)) == 0) {
    const int64_t total_runs = rows * runs_per_row;
    const int64_t tiles = (total_runs + 63) / 64;
    int64_t wgs = (tiles + 3) / 4;
    if (wgs > kFwdTileWorkgroups) wgs = kFwdTileWorkgroups;
    hipLaunchKernelGGL((quest_fwd_tiles_kernel<In, LOGN, B, Dq>), dim3(static_cast<uint32_t>(wgs)), dim3(256), 0,
                       stream, x, total_runs, log2_exact(runs_per_row), k, a.codes, a.scale, mask32, dq);
  } else {
    int group = runs_per_row & -runs_per_row;
    if (group > 64) group = 64;
    int rows_per_wg = 64 / gcd_int(runs_per_row, 64);
    if (rows_per_wg * runs_per_row > 1024) rows_per_wg = 1024 / runs_per_row;
    if (rows_per_wg < 1) rows_per_wg = 1;
    const int threads = ((rows_per_wg * runs_per_row + 63) / 64) * 64;
    const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
    constexpr int US = 2 * sizeof(In) > DqOut<Dq>::U ? 2 * sizeof(In) : DqOut<Dq>::U;
    hipLaunchKernelGGL((quest_fwd_rows_kernel<In, LOGN, B, Dq>), dim3(static_cast<uint32_t>(grid)), dim3(threads),
                       rows_lds_bytes(threads, US), stream, x, rows, runs_per_row, rows_per_wg, log2_exact(group), k, a.codes, a.scale, mask32,
                       dq);
  }
  return hipGetLastError();
}

template <typename In, int LOGN, typename Dq>
hipError_t fwd_dispatch_bits(const In* x, int bits, const FwdLaunch& a) {
  if constexpr (kIsOperand<Dq>) {  // the operand holds grids of at most 4 bits
    switch (bits) {
      case 1: return fwd_dispatch<In, LOGN, 1, Dq>(x, a);
      case 2: return fwd_dispatch<In, LOGN, 2, Dq>(x, a);
      case 3: return fwd_dispatch<In, LOGN, 3, Dq>(x, a);
      default: return fwd_dispatch<In, LOGN, 4, Dq>(x, a);
    }
  } else {
    switch (bits) {
      case 1: return fwd_dispatch<In, LOGN, 1, Dq>(x, a);
      case 2: return fwd_dispatch<In, LOGN, 2, Dq>(x, a);
      case 3: return fwd_dispatch<In, LOGN, 3, Dq>(x, a);
      case 4: return fwd_dispatch<In, LOGN, 4, Dq>(x, a);
      case 5: return fwd_dispatch<In, LOGN, 5, Dq>(x, a);
      case 6: return fwd_dispatch<In, LOGN, 6, Dq>(x, a);
      case 7: return fwd_dispatch<In, LOGN, 7, Dq>(x, a);
      default: return fwd_dispatch<In, LOGN, 8, Dq>(x, a);
    }
  }
}

template <typename In, typename Dq>
hipError_t fwd_dispatch_block(const In* x, int log_block, int bits, const FwdLaunch& a) {
  switch (log_block) {
    case 6: return fwd_dispatch_bits<In, 6, Dq>(x, bits, a);
    case 7: return fwd_dispatch_bits<In, 7, Dq>(x, bits, a);
    default: return fwd_dispatch_bits<In, 8, Dq>(x, bits, a);
  }
}


template <typename G>
hipError_t bwd_dispatch(const G* grad, const uint8_t* mask, int64_t rows, int64_t cols, int log_block, G* out,
                        bool allow_mfma, hipStream_t stream) {
  const int64_t total_runs = rows * (cols / RUN);
  const int64_t grid = (total_runs + 255) / 256;
  const uint32_t* mask32 = reinterpret_cast<const uint32_t*>(mask);
  if constexpr (sizeof(G) == 2) {
    if (allow_mfma) {  // bf16: one 64-run tile per wave, four waves per workgroup
      switch (log_block) {
        case 6:
          hipLaunchKernelGGL((quest_bwd_mfma_kernel<6>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                             grad, mask32, total_runs, out);
          break;
        case 7:
          hipLaunchKernelGGL((quest_bwd_mfma_kernel<7>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                             grad, mask32, total_runs, out);
          break;
        default:
          hipLaunchKernelGGL((quest_bwd_mfma_kernel<8>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                             grad, mask32, total_runs, out);
          break;
      }
      return hipGetLastError();
    }
  }
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

// Codes to operand: one workgroup per 32-row block and eight runs.
template <int B>
hipError_t codes_to_operand_launch(const uint8_t* codes, int64_t rows, int64_t cols, uint8_t* operand,
                                   hipStream_t stream) {
  const int runs_per_row = static_cast<int>(cols / RUN);
  const int run_groups = (runs_per_row + 7) / 8;
  const int64_t grid = ((rows + 31) / 32) * run_groups;
  hipLaunchKernelGGL((quest_codes_to_operand_kernel<B>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                     codes, rows, runs_per_row, run_groups, operand);
  return hipGetLastError();
}

template <typename Out, int B>
hipError_t dequant_launch(const uint8_t* codes, const float* scale, int64_t total_runs, uint32_t runs_per_row, Out* out,
                          hipStream_t stream) {
  const uint32_t grid = static_cast<uint32_t>((total_runs + 255) / 256);
  hipLaunchKernelGGL((quest_dequant_kernel<Out, B>), dim3(grid), dim3(256), 0, stream, codes, scale, total_runs,
                     runs_per_row, out);
  return hipGetLastError();
}

template <typename Out>
hipError_t dequant_dispatch(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int bits, Out* out,
                            hipStream_t stream) {
  const uint32_t runs_per_row = static_cast<uint32_t>(cols / RUN);
  const int64_t total_runs = rows * runs_per_row;
  switch (bits) {
    case 1: return dequant_launch<Out, 1>(codes, scale, total_runs, runs_per_row, out, stream);
    case 2: return dequant_launch<Out, 2>(codes, scale, total_runs, runs_per_row, out, stream);
    case 3: return dequant_launch<Out, 3>(codes, scale, total_runs, runs_per_row, out, stream);
    case 4: return dequant_launch<Out, 4>(codes, scale, total_runs, runs_per_row, out, stream);
    case 5: return dequant_launch<Out, 5>(codes, scale, total_runs, runs_per_row, out, stream);
    case 6: return dequant_launch<Out, 6>(codes, scale, total_runs, runs_per_row, out, stream);
    case 7: return dequant_launch<Out, 7>(codes, scale, total_runs, runs_per_row, out, stream);
    default: return dequant_launch<Out, 8>(codes, scale, total_runs, runs_per_row, out, stream);
  }
}

}  // namespace quest

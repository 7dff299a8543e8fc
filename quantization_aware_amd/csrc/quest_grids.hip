// Forward quantisation onto the other grids of the pages and their
// dequantisation: FP4 levels and 2:4-sparse b-bit codes.
//
// The pages extend QuEST to an FP4 format and to 2:4-sparse INT4
// (pith.science review of QuEST, the list of contributions and the captions
// of Figures 3 and 4; atlas.scime.ai summary, "Key results"; the ablation
// table: 2:4 sparsity added to INT4).
//
// FP4: the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (OCP MX v1.0) times
// s / 6, s = alpha_fp4 * RMS, alpha_fp4 minimising the Gaussian MSE of that
// grid.  Code = the E2M1 pattern of the level nearest to 6 y / s (ties to the
// even code, saturating at 6; the zero level is +0), stored 4 bits per
// element LSB-first.  Trusted iff |y| <= s (1 + t / 6): beyond the grid, t
// times half the outermost interval; inside it nearest rounding never errs by
// more than half the local interval.
//
// 2:4: in every group of 4 consecutive Hadamard-domain entries the 2 largest
// |y| are kept (on equal magnitudes the lower index), the b-bit grid is
// scaled by the kept entries' RMS, kept entries take the dense quantiser's
// code, pruned ones reconstruct as 0.  Stored per row: the kept codes (C / 2
// codes of b bits, LSB-first, in index order), their positions in their group
// (C / 2 2-bit fields) and the mask, whose pruned entries are trusted iff
// |y| <= Delta / 2 (the literal trust rule with reconstruction 0).
//
// Kernel layout as quest_fwd_rows_kernel: a workgroup holds whole rows, a
// lane holds one 32-entry run (8 groups of 4), the row's sum of squares goes
// through aligned lane groups and LDS in a fixed order.  FP4 of bf16 rows of
// 512, 1024 or 2048 columns instead runs the dense matrix-core forward
// (quest_fwd_mfma_kernel with FP4 codes).
#include "quest_kernels.h"

namespace quest {

enum class Grid { kFp4, kSparse24 };

namespace {

struct GridConsts {
  float alpha;     // alpha of the grid
  float kz;        // FP4: 6 / (alpha sqrt(n)); 2:4: (L - 1) / (2 alpha sqrt(n))
  float thr;       // trusted (kept entries): |v| <= thr * RMS
  float prune_ratio;  // 2:4: thr / (the pruned entries' threshold Delta / 2) = L - 1 + t
  float inv_count; // 1 / (entries the RMS runs over): 1 / C (FP4), 2 / C (2:4)
};

// Per-lane conditions of the 2:4 selection are kept as wave lane masks
// (one bit per lane), so that their logic runs on the scalar unit: a compare
// writes the mask, scalar ops combine masks, and a select or an
// add-with-carry reads one directly.
using lanes_t = unsigned long long;

__device__ __forceinline__ lanes_t lanes(bool c) { return __builtin_amdgcn_ballot_w64(c); }
__device__ __forceinline__ bool lane_in(lanes_t m) { return __builtin_amdgcn_inverse_ballot_w64(m); }

// w = 2 w + (this lane's bit of m): one add with carry-in.  gfx950 needs two
// wait states between a vector write of an SGPR and a vector read of it,
// which the compiler cannot see inside asm: m and the masks of select_lanes
// must come from scalar ops (the callers pass combinations of compare
// masks), never straight from a compare.
__device__ __forceinline__ void push_lane_bit(uint32_t& w, lanes_t m) {
  asm volatile("v_addc_co_u32_e64 %0, %1, %0, %0, %1" : "+v"(w), "+s"(m));
}

// (this lane's bit of m) ? if_set : if_clear, one select on the mask.
__device__ __forceinline__ float select_lanes(lanes_t m, float if_set, float if_clear) {
  float r;
  asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(m));
  return r;
}

// The kept pair of one group of 4 entries: entry i is kept iff fewer than
// two entries beat it (a larger magnitude, or an equal one at a lower
// index).  The six pairwise comparisons rank the four entries; "fewer than
// two of three" is the negated majority of entry i's three beat flags.
struct Keep4 {
  lanes_t k0, k1, k2, k3;  // lanes that keep entry i
};

__device__ __forceinline__ lanes_t majority3(lanes_t x, lanes_t y, lanes_t z) { return (x & y) | (z & (x | y)); }

__device__ __forceinline__ Keep4 keep4(const float* v) {
  const float a0 = __builtin_fabsf(v[0]), a1 = __builtin_fabsf(v[1]);
  const float a2 = __builtin_fabsf(v[2]), a3 = __builtin_fabsf(v[3]);
  // bji: entry j beats entry i, for j > i (a strictly larger magnitude)
  const lanes_t b10 = lanes(a1 > a0), b20 = lanes(a2 > a0), b30 = lanes(a3 > a0);
  const lanes_t b21 = lanes(a2 > a1), b31 = lanes(a3 > a1), b32 = lanes(a3 > a2);
  return {~majority3(b10, b20, b30), ~majority3(~b10, b21, b31), ~majority3(~b20, ~b21, b32),
          ~majority3(~b30, ~b31, ~b32)};
}

template <typename In, int LOGN, Grid G, int B, typename Dq>
__global__ void __launch_bounds__(1024)
    quest_fwd_grid_kernel(const In* __restrict__ x, int64_t rows, int runs_per_row, int rows_per_wg, int log_group,
                          GridConsts k, uint8_t* __restrict__ codes, uint32_t* __restrict__ index,
                          float* __restrict__ scale, uint32_t* __restrict__ mask, Dq* __restrict__ dq) {
  constexpr int U = sizeof(In) * 2;
  constexpr int US = U > DqOut<Dq>::U ? U : DqOut<Dq>::U;
  constexpr float L = static_cast<float>(1 << B);
  float* const part = rows_part<US>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lrow = tid / runs_per_row;
  const int run_in_row = tid - lrow * runs_per_row;
  const int64_t total_runs = rows * runs_per_row;
  const int64_t wg = blockIdx.x;
  const int64_t wg_first_run = wg * rows_per_wg * runs_per_row;
  const int wave_tid0 = __builtin_amdgcn_readfirstlane(tid) & ~63;

  u32x4* const stage = rows_lds + (wave_tid0 >> 6) * 64 * US;
  uint32_t raw[4 * U];
  wave_load_runs<U>(x, (wg_first_run + wave_tid0) * U, total_runs * U, lane, stage, raw);
  float v[RUN];
  float ss;
  const float tau = fwd_transform<In, LOGN>(raw, v, ss, tid);

  // 2:4: the kept pair of group g (slots 2 g, 2 g + 1), its values and
  // positions, and each entry's trust magnitude e: |v| for a kept entry,
  // |v| (L - 1 + t) for a pruned one, so that both are trusted iff e <= thr
  // (the pruned entries' bound Delta / 2 is thr / (L - 1 + t)).
  // v = tau sqrt(n) y: the kept pattern of |v| is that of |y|, and the kept
  // entries' sum of squares is sum v^2 / n.
  constexpr int NS = G == Grid::kSparse24 ? 8 : 1;
  float first[NS], second[NS], e[G == Grid::kSparse24 ? RUN : 1];
  uint32_t pos = 0u;
  if constexpr (G == Grid::kSparse24) {
    float sk = 0.f;
#pragma unroll
    for (int g = 7; g >= 0; --g) {
      const float* w = v + 4 * g;
      const Keep4 kp = keep4(w);
      // the first kept entry is entry 0, 1 or 2 of the group, the second entry 1, 2 or 3
      first[g] = select_lanes(kp.k0, w[0], select_lanes(kp.k1, w[1], w[2]));
      second[g] = select_lanes(kp.k3, w[3], select_lanes(kp.k2, w[2], w[1]));
      // positions i0 | i1 << 2 at bits 4 g .. 4 g + 3, pushed from the top (group 7 first)
      push_lane_bit(pos, kp.k3 | kp.k2);    // bit 1 of i1 (i1 = 3, 2 or 1)
      push_lane_bit(pos, kp.k3 | ~kp.k2);   // bit 0 of i1
      push_lane_bit(pos, ~kp.k0 & ~kp.k1);  // bit 1 of i0 (i0 = 0, 1 or 2)
      push_lane_bit(pos, ~kp.k0 & kp.k1);   // bit 0 of i0
      const lanes_t kept[4] = {kp.k0, kp.k1, kp.k2, kp.k3};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = __builtin_fabsf(w[j]);
        e[4 * g + j] = select_lanes(kept[j], a, a * k.prune_ratio);
      }
      sk = __builtin_fmaf(first[g], first[g], sk);
      sk = __builtin_fmaf(second[g], second[g], sk);
    }
    ss = sk * (1.f / static_cast<float>(1 << LOGN));
  }
  ss = group_sum(ss, log_group);
  if ((tid & ((1 << log_group) - 1)) == 0) part[tid >> log_group] = ss;
  __syncthreads();
  const int per_row = runs_per_row >> log_group;
  ss = 0.f;
  if (lrow < rows_per_wg) {
    const float* pr = part + lrow * per_row;
    for (int i = 0; i < per_row; ++i) ss += pr[i];
  }
  const float ms = ss * k.inv_count;
  const float rms = __builtin_amdgcn_sqrtf(ms);
  const float s = k.alpha * rms;
  const float kz = ms > 0.f ? tau * k.kz * __builtin_amdgcn_rsqf(ms) : 0.f;  // zero row: every code the middle one
  const float thr = k.thr * rms;

  const uint32_t wg_runs = static_cast<uint32_t>(rows_per_wg * runs_per_row);
  const int64_t wg_end = wg_first_run + wg_runs < total_runs ? wg_first_run + wg_runs : total_runs;
  const bool live = wg_first_run + tid < wg_end;
  const int64_t run = wg_first_run + tid;
  const rsrc_t mask_r = window_at(mask, wg_first_run * 4, mask ? total_runs * 4 : 0, wg_runs * 4);
  const rsrc_t scale_r = window_at(scale, wg * rows_per_wg * 4, rows * 4, rows_per_wg * 4);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), scale_r,
                                        (run_in_row == 0 && lrow < rows_per_wg) ? lrow * 4 : kNowhere, 0, 0);
  uint32_t mw = 0u;
  float q[RUN];
  // level unit s / 6 or s / (L - 1), a correctly rounded division as in the dequantisers
  const float c = G == Grid::kFp4 ? s / 6.f : s / (L - 1.f);
  if constexpr (G == Grid::kFp4) {
    uint32_t cw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cw[j] = fp4_codes8(v + 8 * j, kz);
    push16_abs_le(mw, v + 16, thr);
    push16_abs_le(mw, v, thr);
    const rsrc_t codes_r = window_at(codes, wg_first_run * 16, codes ? total_runs * 16 : 0, wg_runs * 16);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{cw[0], cw[1], cw[2], cw[3]}, codes_r, live ? tid * 16 : kNowhere, 0,
                                           kNonTemporal);
    if constexpr (DqOut<Dq>::kOn) {
#pragma unroll
      for (int i = 0; i < RUN; ++i) {
        const uint32_t code = (cw[i >> 3] >> (4 * (i & 7))) & 15u;
        const float mag = e2m1_mag(code & 7u) * c;
        q[i] = (code & 8u) ? -mag : mag;
      }
    }
  } else {
    // 16 kept codes of B bits (2 B bytes per run), slot 2 g + j at bits B (2 g + j).
    uint64_t packed = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float u0 = grid_code<B>(first[g], kz), u1 = grid_code<B>(second[g], kz);
      packed |= static_cast<uint64_t>(static_cast<uint32_t>(u0) | (static_cast<uint32_t>(u1) << B)) << (2 * B * g);
      if constexpr (DqOut<Dq>::kOn) {
        const float l0 = __builtin_fmaf(u0, 2.f, 1.f - L) * c, l1 = __builtin_fmaf(u1, 2.f, 1.f - L) * c;
        const uint32_t i0 = (pos >> (4 * g)) & 3u, i1 = (pos >> (4 * g + 2)) & 3u;
#pragma unroll
        for (int j = 0; j < 4; ++j) q[4 * g + j] = i0 == static_cast<uint32_t>(j) ? l0 : i1 == static_cast<uint32_t>(j) ? l1 : 0.f;
      }
    }
    // e >= 0, so |e| <= thr is e <= thr
    push16_abs_le(mw, e + 16, thr);
    push16_abs_le(mw, e, thr);
    const rsrc_t codes_r = window_at(codes, wg_first_run * 2 * B, codes ? total_runs * 2 * B : 0, wg_runs * 2 * B);
    const int coff = live ? tid * 2 * B : kNowhere;
    const uint32_t lo = static_cast<uint32_t>(packed), hi = static_cast<uint32_t>(packed >> 32);
    if constexpr (B == 1) {
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(lo), codes_r, coff, 0, 0);
    } else if constexpr (B == 2) {
      __builtin_amdgcn_raw_buffer_store_b32(lo, codes_r, coff, 0, 0);
    } else if constexpr (B == 3) {
      __builtin_amdgcn_raw_buffer_store_b32(lo, codes_r, coff, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(hi), codes_r, coff == kNowhere ? kNowhere : coff + 4,
                                            0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, codes_r, coff, 0, 0);
    }
    const rsrc_t index_r = window_at(index, wg_first_run * 4, index ? total_runs * 4 : 0, wg_runs * 4);
    __builtin_amdgcn_raw_buffer_store_b32(pos, index_r, live ? tid * 4 : kNowhere, 0, 0);
  }
  __builtin_amdgcn_raw_buffer_store_b32(mw, mask_r, live ? tid * 4 : kNowhere, 0, kNonTemporal);
  if constexpr (DqOut<Dq>::kOn) {
    uint32_t rawq[4 * DqOut<Dq>::U];
    narrow_run(q, rawq);
    wave_store_runs<DqOut<Dq>::U>(dq, (wg_first_run + wave_tid0) * DqOut<Dq>::U, wg_end * DqOut<Dq>::U, lane, stage,
                                  rawq);
  }
  (void)run;
}

// Dequantisers: one lane per run.
template <typename Out>
__global__ void __launch_bounds__(256)
    quest_dequant_fp4_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scale, int64_t total_runs,
                             uint32_t runs_per_row, Out* __restrict__ out) {
  __shared__ u32x4 stage_all[4][64 * DqOut<Out>::U];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t run0 = static_cast<int64_t>(blockIdx.x) * 256 + wave * 64;
  const int64_t run = run0 + lane;
  const rsrc_t cr = window_at(codes, run0 * 16, total_runs * 16, 64 * 16);
  const u32x4 cw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, lane * 16, 0, kNonTemporal));
  const int64_t row = run < total_runs ? run / runs_per_row : 0;
  const float c = scale[row] / 6.f;
  const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
  float q[RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const uint32_t code = (w[i >> 3] >> (4 * (i & 7))) & 15u;
    const float mag = e2m1_mag(code & 7u) * c;
    q[i] = (code & 8u) ? -mag : mag;
  }
  uint32_t raw[4 * DqOut<Out>::U];
  narrow_run(q, raw);
  wave_store_runs<DqOut<Out>::U>(out, run0 * DqOut<Out>::U, total_runs * DqOut<Out>::U, lane, stage_all[wave], raw);
}

template <typename Out, int B>
__global__ void __launch_bounds__(256)
    quest_dequant_sparse24_kernel(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ index,
                                  const float* __restrict__ scale, int64_t total_runs, uint32_t runs_per_row,
                                  Out* __restrict__ out) {
  constexpr float L = static_cast<float>(1 << B);
  __shared__ u32x4 stage_all[4][64 * DqOut<Out>::U];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int64_t run0 = static_cast<int64_t>(blockIdx.x) * 256 + wave * 64;
  const int64_t run = run0 + lane;
  const rsrc_t cr = window_at(codes, run0 * 2 * B, total_runs * 2 * B, 64 * 2 * B);
  const rsrc_t ir = window_at(index, run0 * 4, total_runs * 4, 64 * 4);
  uint64_t packed;
  if constexpr (B == 1) {
    packed = __builtin_amdgcn_raw_buffer_load_b16(cr, lane * 2, 0, 0);
  } else if constexpr (B == 2) {
    packed = __builtin_amdgcn_raw_buffer_load_b32(cr, lane * 4, 0, 0);
  } else if constexpr (B == 3) {
    packed = static_cast<uint64_t>(__builtin_amdgcn_raw_buffer_load_b32(cr, lane * 6, 0, 0)) |
             (static_cast<uint64_t>(__builtin_amdgcn_raw_buffer_load_b16(cr, lane * 6 + 4, 0, 0)) << 32);
  } else {
    const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(cr, lane * 8, 0, 0));
    packed = static_cast<uint64_t>(t.x) | (static_cast<uint64_t>(t.y) << 32);
  }
  const uint32_t pos = __builtin_amdgcn_raw_buffer_load_b32(ir, lane * 4, 0, 0);
  const int64_t row = run < total_runs ? run / runs_per_row : 0;
  const float c = scale[row] / (L - 1.f);
  float q[RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) q[i] = 0.f;
#pragma unroll
  for (int slot = 0; slot < 16; ++slot) {
    const uint32_t u = static_cast<uint32_t>(packed >> (B * slot)) & ((1u << B) - 1u);
    const int at = 4 * (slot >> 1) + static_cast<int>((pos >> (2 * slot)) & 3u);
    const float val = __builtin_fmaf(static_cast<float>(u), 2.f, 1.f - L) * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[4 * (slot >> 1) + i] = at == 4 * (slot >> 1) + i ? val : q[4 * (slot >> 1) + i];
  }
  uint32_t raw[4 * DqOut<Out>::U];
  narrow_run(q, raw);
  wave_store_runs<DqOut<Out>::U>(out, run0 * DqOut<Out>::U, total_runs * DqOut<Out>::U, lane, stage_all[wave], raw);
}

template <typename In, int LOGN, Grid G, int B, typename Dq>
hipError_t grid_launch(const In* x, const GridLaunch& a) {
  const int runs_per_row = static_cast<int>(a.cols / RUN);
  int group = runs_per_row & -runs_per_row;
  if (group > 64) group = 64;
  int rows_per_wg = 64 / gcd_int(runs_per_row, 64);
  if (rows_per_wg * runs_per_row > 1024) rows_per_wg = 1024 / runs_per_row;
  if (rows_per_wg < 1) rows_per_wg = 1;
  const int threads = ((rows_per_wg * runs_per_row + 63) / 64) * 64;
  const int64_t grid = (a.rows + rows_per_wg - 1) / rows_per_wg;
  const double sqrt_n = std::sqrt(double(1 << LOGN));
  GridConsts k;
  k.alpha = static_cast<float>(a.alpha);
  if constexpr (G == Grid::kFp4) {
    k.kz = static_cast<float>(6.0 / (a.alpha * sqrt_n));
    k.thr = static_cast<float>(a.alpha * sqrt_n * (1.0 + a.trust / 6.0));
    k.prune_ratio = 1.f;
    k.inv_count = static_cast<float>(1.0 / double(a.cols));
  } else {
    const double lm1 = double((1 << B) - 1);
    k.kz = static_cast<float>(lm1 / (2.0 * a.alpha * sqrt_n));
    k.thr = static_cast<float>(a.alpha * sqrt_n * (1.0 + a.trust / lm1));
    k.prune_ratio = static_cast<float>(lm1 + a.trust);
    k.inv_count = static_cast<float>(2.0 / double(a.cols));
  }
  if constexpr (G == Grid::kFp4 && sizeof(In) == 2) {
    if (a.allow_mfma && (runs_per_row == 16 || runs_per_row == 32 || runs_per_row == 64)) {
      // bf16 rows of 512, 1024 or 2048 columns: the dense matrix-core forward
      // with FP4 codes (same transform, RMS from the inputs, nibble per entry).
      FwdConsts kf;
      kf.alpha = k.alpha;
      kf.kk = k.kz;
      kf.thr = k.thr;
      kf.inv_cols = k.inv_count;
      kf.chunks = static_cast<int>(a.cols / 128);
      const int64_t total_runs = a.rows * runs_per_row;
      const dim3 grid4(static_cast<uint32_t>((total_runs + 255) / 256));
      auto run = [&](auto logr) {
        hipLaunchKernelGGL((quest_fwd_mfma_kernel<LOGN, 4, decltype(logr)::value, Dq, true, true>), grid4, dim3(256),
                           0, a.stream, x, total_runs, kf, a.codes, a.scale, reinterpret_cast<uint32_t*>(a.mask),
                           static_cast<Dq*>(a.dq));
      };
      if (runs_per_row == 16)
        run(std::integral_constant<int, 4>{});
      else if (runs_per_row == 32)
        run(std::integral_constant<int, 5>{});
      else
        run(std::integral_constant<int, 6>{});
      return hipGetLastError();
    }
  }
  constexpr int US = 2 * sizeof(In) > DqOut<Dq>::U ? 2 * sizeof(In) : DqOut<Dq>::U;
  hipLaunchKernelGGL((quest_fwd_grid_kernel<In, LOGN, G, B, Dq>), dim3(static_cast<uint32_t>(grid)), dim3(threads),
                     rows_lds_bytes(threads, US), a.stream, x, a.rows, runs_per_row, rows_per_wg, log2_exact(group), k, a.codes,
                     reinterpret_cast<uint32_t*>(a.index), a.scale, reinterpret_cast<uint32_t*>(a.mask),
                     static_cast<Dq*>(a.dq));
  return hipGetLastError();
}

template <typename In, Grid G, int B, typename Dq>
hipError_t grid_block(const In* x, int log_block, const GridLaunch& a) {
  switch (log_block) {
    case 6: return grid_launch<In, 6, G, B, Dq>(x, a);
    case 7: return grid_launch<In, 7, G, B, Dq>(x, a);
    default: return grid_launch<In, 8, G, B, Dq>(x, a);
  }
}

template <typename In, typename Dq>
hipError_t grid_dispatch(const In* x, int log_block, const GridLaunch& a) {
  if (a.sparse24 == 0) return grid_block<In, Grid::kFp4, 4, Dq>(x, log_block, a);
  switch (a.bits) {
    case 1: return grid_block<In, Grid::kSparse24, 1, Dq>(x, log_block, a);
    case 2: return grid_block<In, Grid::kSparse24, 2, Dq>(x, log_block, a);
    case 3: return grid_block<In, Grid::kSparse24, 3, Dq>(x, log_block, a);
    default: return grid_block<In, Grid::kSparse24, 4, Dq>(x, log_block, a);
  }
}

template <typename In>
hipError_t grid_dq(const In* x, int log_block, int dq_kind, const GridLaunch& a) {
  switch (dq_kind) {
    case 1: return grid_dispatch<In, uint16_t>(x, log_block, a);
    case 2: return grid_dispatch<In, float>(x, log_block, a);
    default: return grid_dispatch<In, void>(x, log_block, a);
  }
}

template <typename Out>
hipError_t deq_fp4(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, Out* out,
                   hipStream_t stream) {
  const uint32_t runs_per_row = static_cast<uint32_t>(cols / RUN);
  const int64_t total_runs = rows * runs_per_row;
  hipLaunchKernelGGL((quest_dequant_fp4_kernel<Out>), dim3(static_cast<uint32_t>((total_runs + 255) / 256)),
                     dim3(256), 0, stream, codes, scale, total_runs, runs_per_row, out);
  return hipGetLastError();
}

template <typename Out, int B>
hipError_t deq_s24_b(const uint8_t* codes, const uint8_t* index, const float* scale, int64_t rows, int64_t cols,
                     Out* out, hipStream_t stream) {
  const uint32_t runs_per_row = static_cast<uint32_t>(cols / RUN);
  const int64_t total_runs = rows * runs_per_row;
  hipLaunchKernelGGL((quest_dequant_sparse24_kernel<Out, B>), dim3(static_cast<uint32_t>((total_runs + 255) / 256)),
                     dim3(256), 0, stream, codes, reinterpret_cast<const uint32_t*>(index), scale, total_runs,
                     runs_per_row, out);
  return hipGetLastError();
}

template <typename Out>
hipError_t deq_s24(const uint8_t* codes, const uint8_t* index, const float* scale, int64_t rows, int64_t cols,
                   int bits, Out* out, hipStream_t stream) {
  switch (bits) {
    case 1: return deq_s24_b<Out, 1>(codes, index, scale, rows, cols, out, stream);
    case 2: return deq_s24_b<Out, 2>(codes, index, scale, rows, cols, out, stream);
    case 3: return deq_s24_b<Out, 3>(codes, index, scale, rows, cols, out, stream);
    default: return deq_s24_b<Out, 4>(codes, index, scale, rows, cols, out, stream);
  }
}

}  // namespace

hipError_t launch_fwd_grid(const void* x, int x_is_bf16, int log_block, int dq_kind, const GridLaunch& a) {
  if (x_is_bf16) return grid_dq(static_cast<const uint16_t*>(x), log_block, dq_kind, a);
  return grid_dq(static_cast<const float*>(x), log_block, dq_kind, a);
}

hipError_t launch_dequantize_fp4(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, void* out,
                                 int out_is_bf16, hipStream_t stream) {
  if (out_is_bf16) return deq_fp4(codes, scale, rows, cols, static_cast<uint16_t*>(out), stream);
  return deq_fp4(codes, scale, rows, cols, static_cast<float*>(out), stream);
}

hipError_t launch_dequantize_sparse24(const uint8_t* codes, const uint8_t* index, const float* scale, int64_t rows,
                                      int64_t cols, int bits, void* out, int out_is_bf16, hipStream_t stream) {
  if (out_is_bf16) return deq_s24(codes, index, scale, rows, cols, bits, static_cast<uint16_t*>(out), stream);
  return deq_s24(codes, index, scale, rows, cols, bits, static_cast<float*>(out), stream);
}

}  // namespace quest

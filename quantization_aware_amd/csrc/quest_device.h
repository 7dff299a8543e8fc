// Device-side building blocks of libquest (gfx950 / CDNA4).
//
// Data layout in registers: every lane owns a "run" of RUN = 32 consecutive
// elements of one row.  A Hadamard block of n = 2^LOGN entries therefore
// spans n/32 neighbouring lanes (2, 4 or 8).  The 5 butterfly stages that
// pair elements 1..16 apart are done inside the lane; the remaining
// LOGN - 5 stages pair lanes and use DPP (lane xor 1 and xor 2) or a
// ds_swizzle (lane xor 4).  Runs are consecutive in memory, so run g of a
// tensor starts at element 32 g, its codes at byte 4 b g and its mask bits at
// dword g: loads are 64 B (bf16) or 128 B (fp32) per lane and every store of
// codes and mask is one contiguous dword..dwordx4 per lane, so a wave writes
// one contiguous stretch of memory.
//
// Sign bookkeeping of the cross-lane butterflies.  A butterfly on lanes
// (a, b) must leave a + b in lane a and a - b in lane b, i.e. a different
// operation per lane.  Each lane instead computes self + sigma * partner with
// sigma = +1 in lane a and -1 in lane b, which is one v_fmac_f32 with a DPP
// operand.  Lane b then holds b - a = -(a - b): the lane's values carry a
// known sign tau = (-1)^popcount(lane bits used).  The sign is folded into
// the per-lane quantisation constant (forward) or output scale (backward),
// so it costs nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quest {

constexpr int RUN = 32;

// ----------------------------------------------------------------------------
// Global memory goes through buffer instructions.  A buffer resource covers a
// window of at most 4 GB; accesses at or past its end read zero and write
// nothing.  Kernels build a resource per chunk of work (a few scalar
// instructions) and pass 32-bit per-lane offsets, so there is no per-lane
// bounds test and no divergent branch around a store: the code between waits
// is straight-line and the wait counts stay exact (loads and stores share one
// counter on gfx950, and a guarded store makes every later wait conservative).
// ----------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kNonTemporal = 2;             // cache policy bit "nt"
constexpr int kRawBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format

// Bytes of the window [start, start + window) that lie inside [0, size).
__device__ __forceinline__ uint32_t window_bytes(int64_t start, int64_t size, uint32_t window) {
  const int64_t rem = size - start;
  return rem <= 0 ? 0u : (rem >= static_cast<int64_t>(window) ? window : static_cast<uint32_t>(rem));
}

// Resource for the window starting `start` bytes into an array of `size` bytes at p.
__device__ __forceinline__ rsrc_t window_at(const void* p, int64_t start, int64_t size, uint32_t window) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(start);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(a), static_cast<short>(0),
                                           static_cast<int>(window_bytes(start, size, window)), kRawBufferWord3);
}

// ----------------------------------------------------------------------------
// Coalesced traffic through a wave-private LDS stage.
//
// Lanes compute on runs of 32 consecutive elements, but a wave reading its 64
// runs run-by-run (64 or 128 B per lane, lanes 64 or 128 B apart) only
// reaches about half of HBM bandwidth.  Instead the wave moves its chunk of
// 64 runs with fully coalesced 16-byte-per-lane non-temporal accesses
// (instruction k touches the k-th kilobyte of the chunk) and transposes
// through LDS.  A run is U 16-byte pieces (U = 4 for bf16, 8 for fp32);
// piece c of run r lives in LDS slot 64 c + (r ^ h[c]).  The XOR offsets h
// keep both the coalesced side and the run side free of bank conflicts
// whether the LDS serves 8 lanes per pass over 32 banks or 16 lanes over 64.
// LDS instructions of one wave complete in order, so no barrier is needed
// between a wave's writes and its reads of its own stage.
// ----------------------------------------------------------------------------

// h[c] for U = 4 is {0, 10, 4, 14} and for U = 8 {0, 2, 4, 6, 9, 11, 13, 15};
// both are linear in the bits of c, which keeps them arithmetic (no table).
template <int U>
__device__ __forceinline__ constexpr int stage_xor(int c) {
  if constexpr (U == 4) {
    return ((c & 1) * 10) ^ ((c & 2) * 2);
  } else {
    return ((c & 3) * 2) ^ ((c >> 2) * 9);
  }
}

// Issue the coalesced loads of a wave's chunk: piece first_piece + 64 k + lane
// into t[k].  Pieces at or past total_pieces read as zero.
template <int U>
__device__ __forceinline__ void wave_fetch(const void* base, int64_t first_piece, int64_t total_pieces, int lane,
                                           u32x4 (&t)[U]) {
  const rsrc_t r = window_at(base, first_piece * 16, total_pieces * 16, 64 * U * 16);
#pragma unroll
  for (int k = 0; k < U; ++k) t[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64 * k) * 16, 0, kNonTemporal);
}

// Transpose fetched pieces through the wave's LDS stage: lane l receives the
// 4U dwords of run l of the chunk.
// (Runs are handed out as plain dword arrays: element access on
// ext_vector_type values inside unrolled loops has been seen to miscompile.)
template <int U>
__device__ __forceinline__ void wave_stage(const u32x4 (&t)[U], int lane, u32x4* stage, uint32_t (&out)[4 * U]) {
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int q = 64 * k + lane;
    const int r = q / U, c = q % U;
    stage[64 * c + (r ^ stage_xor<U>(c))] = t[k];
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int c = 0; c < U; ++c) {
    const u32x4 w = stage[64 * c + (lane ^ stage_xor<U>(c))];
    out[4 * c + 0] = w.x;
    out[4 * c + 1] = w.y;
    out[4 * c + 2] = w.z;
    out[4 * c + 3] = w.w;
  }
}

// Load the 64 runs of a wave: lane l receives the 4U dwords of run
// first_piece / U + l (zeros past the tensor).
template <int U>
__device__ __forceinline__ void wave_load_runs(const void* base, int64_t first_piece, int64_t total_pieces, int lane,
                                               u32x4* stage, uint32_t (&out)[4 * U]) {
  u32x4 t[U];
  wave_fetch<U>(base, first_piece, total_pieces, lane, t);
  wave_stage<U>(t, lane, stage, out);
}

// Store the 64 runs of a wave (lane l holds the 4U dwords of run
// first_piece / U + l); pieces at or past total_pieces are dropped.  P is
// the stores' cache policy.
template <int U, int P = kNonTemporal>
__device__ __forceinline__ void wave_store_runs(void* base, int64_t first_piece, int64_t total_pieces, int lane,
                                                u32x4* stage, const uint32_t (&in)[4 * U]) {
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int c = 0; c < U; ++c) {
    u32x4 w;
    w.x = in[4 * c + 0];
    w.y = in[4 * c + 1];
    w.z = in[4 * c + 2];
    w.w = in[4 * c + 3];
    stage[64 * c + (lane ^ stage_xor<U>(c))] = w;
  }
  __builtin_amdgcn_wave_barrier();
  const rsrc_t r = window_at(base, first_piece * 16, total_pieces * 16, 64 * U * 16);
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int q = 64 * k + lane;
    const int rr = q / U, c = q % U;
    const u32x4 t = stage[64 * c + (rr ^ stage_xor<U>(c))];
    __builtin_amdgcn_raw_buffer_store_b128(t, r, q * 16, 0, P);
  }
}

// Widen a run held as raw dwords to fp32 (bf16: upper half of an fp32).
__device__ __forceinline__ void widen_run(const uint32_t (&d)[16], float (&v)[RUN]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = __uint_as_float(d[i] << 16);
    v[2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void widen_run(const uint32_t (&d)[32], float (&v)[RUN]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(d[i]);
}

// The same with element j replaced by +0 unless bit j of m is set: the bit is
// sign-extended to an all-ones or all-zeros dword and ANDed onto the bits.
__device__ __forceinline__ void widen_run_masked(const uint32_t (&d)[16], uint32_t m, float (&v)[RUN]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t keep_lo = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(m), 2 * i, 1));
    const uint32_t keep_hi = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(m), 2 * i + 1, 1));
    v[2 * i] = __uint_as_float((d[i] << 16) & keep_lo);
    v[2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u & keep_hi);
  }
}

__device__ __forceinline__ void widen_run_masked(const uint32_t (&d)[32], uint32_t m, float (&v)[RUN]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t keep = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(m), i, 1));
    v[i] = __uint_as_float(d[i] & keep);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi);

// Narrow a run of fp32 results to raw dwords of the output type.
__device__ __forceinline__ void narrow_run(const float (&v)[RUN], uint32_t (&d)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) d[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
}

__device__ __forceinline__ void narrow_run(const float (&v)[RUN], uint32_t (&d)[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) d[i] = __float_as_uint(v[i]);
}

// ----------------------------------------------------------------------------
// Sum over aligned groups of 2^log_g lanes (log_g <= 6, wave-uniform); every
// lane of a group ends with the group's sum, added in the same order.  After
// the two quad steps all lanes of a quad agree, so the half-row mirror (lane
// i with 7 - i) and the row mirror (i with 15 - i) pair whole quads and whole
// half-rows; lanes 16 apart meet through ds_swizzle, the two halves of the
// wave through v_readlane.
// ----------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_read(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float group_sum(float x, int log_g) {
  if (log_g > 0) x += dpp_read<0xB1>(x);   // quad_perm [1,0,3,2]
  if (log_g > 1) x += dpp_read<0x4E>(x);   // quad_perm [2,3,0,1]
  if (log_g > 2) x += dpp_read<0x141>(x);  // row_half_mirror
  if (log_g > 3) x += dpp_read<0x140>(x);  // row_mirror
  if (log_g > 4) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // lane ^ 16
  if (log_g > 5) {
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    x = lo + hi;
  }
  return x;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// r = x.lo * c.lo + x.hi * c.hi (+ acc) for bf16 pairs, fp32 result.  The
// VOP3P form keeps the accumulator a separate operand, so one partial sum can
// feed two outputs without a copy.
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t c) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(c));
  return r;
}

__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t c, float acc) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(c), "v"(acc));
  return r;
}

// The first two butterfly stages (pairs 1 and 2 apart) fused with the
// widening to fp32.  For packed pairs d0 = (x0, x1), d1 = (x2, x3):
//   a = x0 + x1,  b = x0 - x1             (dot2 against (1,1) and (1,-1))
//   y0 = a + (x2 + x3),  y2 = a - (x2 + x3)
//   y1 = b + (x2 - x3),  y3 = b - (x2 - x3)  (dot2 with a or b as accumulator)
// Products of bf16 values by +-1 are exact, so each output is rounded at most
// twice, as with fp32 adds of the widened values: six dot2 per four outputs.
__device__ __forceinline__ void first_stages_bf16(const uint32_t (&d)[16], float (&v)[RUN]) {
  const uint32_t pp = 0x3F803F80u;  // (+1, +1)
  const uint32_t pm = 0xBF803F80u;  // (+1, -1)
  const uint32_t mm = 0xBF80BF80u;  // (-1, -1)
  const uint32_t mp = 0x3F80BF80u;  // (-1, +1)
#pragma unroll
  for (int i = 0; i < RUN / 4; ++i) {
    const uint32_t d0 = d[2 * i], d1 = d[2 * i + 1];
    const float a = dot2_bf16(d0, pp);
    const float b = dot2_bf16(d0, pm);
    v[4 * i + 0] = dot2_bf16(d1, pp, a);
    v[4 * i + 2] = dot2_bf16(d1, mm, a);
    v[4 * i + 1] = dot2_bf16(d1, pm, b);
    v[4 * i + 3] = dot2_bf16(d1, mp, b);
  }
}

// Sum of squares of the 32 inputs, lo^2 + hi^2 per packed pair (products of
// bf16 values are exact in fp32), four accumulation chains.
__device__ __forceinline__ float sum_squares_bf16(const uint32_t (&d)[16]) {
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RUN / 2; ++i) {
    const bf16x2_t x = __builtin_bit_cast(bf16x2_t, d[i]);
    a[i & 3] = __builtin_amdgcn_fdot2_f32_bf16(x, x, a[i & 3], false);
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

__device__ __forceinline__ float sum_squares(const float (&v)[RUN]) {
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RUN; ++i) a[i & 3] = __builtin_fmaf(v[i], v[i], a[i & 3]);
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// ----------------------------------------------------------------------------
// fp32 to bf16, two at a time.
// ----------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // Round to nearest even: the gfx950 conversion instruction does this.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {lo, hi};
  const bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// ----------------------------------------------------------------------------
// Unnormalised Walsh-Hadamard butterflies (Sylvester order).
// ----------------------------------------------------------------------------

// In-lane stages: pairs FIRST, 2 FIRST, ..., 16 apart (FIRST = 1 does all five).
template <int FIRST = 1>
__device__ __forceinline__ void fwht_in_lane(float (&v)[RUN]) {
#pragma unroll
  for (int s = FIRST; s < RUN; s <<= 1) {
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
      if ((i & s) == 0) {
        const float a = v[i];
        const float b = v[i + s];
        v[i] = a + b;
        v[i + s] = a - b;
      }
    }
  }
}

// v[i] += sigma * v[i] of the partner lane, the partner chosen by a DPP
// quad permutation.  The leading s_nop 1 gives the two wait states gfx9
// requires between a VALU write of a VGPR and a DPP read of it; inside the
// block every DPP source is a different register, untouched by the block.
#define QUEST_FMAC_DPP8(PERM) QUEST_FMAC_DPP8_AFTER(PERM, "s_nop 1\n\t")

// The same block preceded by a given wait.  The compiler counts wait states
// only for instructions it can see, not for reads inside inline asm, so a
// block whose inputs come straight from a matrix-core instruction supplies
// the VALU-read-after-MFMA-write wait itself: 8 wait states for
// v_mfma_f32_16x16x32_bf16 on gfx950 (the count the compiler inserts before
// its own reads), given here as 10.
#define QUEST_FMAC_DPP8_AFTER(PERM, WAIT)                                                                  \
  asm volatile(                                                                                            \
      WAIT                                                                                                 \
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf"                          \
      : "+v"(v[k + 0]), "+v"(v[k + 1]), "+v"(v[k + 2]), "+v"(v[k + 3]), "+v"(v[k + 4]), "+v"(v[k + 5]),     \
        "+v"(v[k + 6]), "+v"(v[k + 7])                                                                     \
      : "v"(sigma))

// Butterfly between lanes l and l ^ 1.
__device__ __forceinline__ void fwht_lane_xor1(float (&v)[RUN], float sigma) {
#pragma unroll
  for (int k = 0; k < RUN; k += 8) QUEST_FMAC_DPP8("[1,0,3,2]");
}

// The same on values just written by v_mfma_f32_16x16x32_bf16.
__device__ __forceinline__ void fwht_lane_xor1_after_mfma(float (&v)[RUN], float sigma) {
#pragma unroll
  for (int k = 0; k < RUN; k += 8) QUEST_FMAC_DPP8_AFTER("[1,0,3,2]", "s_nop 7\n\ts_nop 1\n\t");
}

// Butterfly between lanes l and l ^ 2.
__device__ __forceinline__ void fwht_lane_xor2(float (&v)[RUN], float sigma) {
#pragma unroll
  for (int k = 0; k < RUN; k += 8) QUEST_FMAC_DPP8("[2,3,0,1]");
}

// Butterfly between lanes l and l ^ 4 (ds_swizzle in bit-mask mode:
// and_mask = 0x1f, or_mask = 0, xor_mask = 4).
__device__ __forceinline__ void fwht_lane_xor4(float (&v)[RUN], float sigma) {
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const float p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[i]), 0x101F));
    v[i] = __builtin_fmaf(sigma, p, v[i]);
  }
}

// Full unnormalised transform of a block of 2^LOGN entries spread over
// 2^(LOGN-5) lanes.  Returns tau, the sign every value of this lane carries.
// Cross-lane stages only (the in-lane ones done by the caller).
template <int LOGN, bool AFTER_MFMA = false>
__device__ __forceinline__ float fwht_cross_lanes(float (&v)[RUN], int lane) {
  static_assert(LOGN >= 6 && LOGN <= 8, "block sizes 64, 128 and 256");
  const float s1 = (lane & 1) ? -1.0f : 1.0f;
  if constexpr (AFTER_MFMA) {
    fwht_lane_xor1_after_mfma(v, s1);
  } else {
    fwht_lane_xor1(v, s1);
  }
  float tau = s1;
  if constexpr (LOGN >= 7) {
    const float s2 = (lane & 2) ? -1.0f : 1.0f;
    fwht_lane_xor2(v, s2);
    tau *= s2;
  }
  if constexpr (LOGN >= 8) {
    const float s4 = (lane & 4) ? -1.0f : 1.0f;
    fwht_lane_xor4(v, s4);
    tau *= s4;
  }
  return tau;
}

template <int LOGN>
__device__ __forceinline__ float fwht_block(float (&v)[RUN], int lane) {
  fwht_in_lane<1>(v);
  return fwht_cross_lanes<LOGN>(v, lane);
}

// ----------------------------------------------------------------------------
// One bit per element, gathered LSB-first into a dword: a comparison writes a
// lane mask and v_addc doubles the word and adds the carry, two VALU
// operations per element.  Elements are pushed from the last to the first, so
// element j ends in bit j once all 32 have been pushed.
//
// gfx950 needs two wait states between a VALU write of an SGPR and a VALU read
// of it.  Each block of 16 pushes therefore rotates three SGPR pairs: every
// v_addc reads a carry written at least two instructions earlier, with no
// s_nop in between.
// ----------------------------------------------------------------------------

// w = (w << 16) | bits, bit j = [ |v[j]| <= thr ], j = 0..15.
__device__ __forceinline__ void push16_abs_le(uint32_t& w, const float* v, float thr) {
  uint64_t p0, p1, p2;
  asm(
      "v_cmp_ge_f32_e64 %1, %20, |%19|\n\t"
      "v_cmp_ge_f32_e64 %2, %20, |%18|\n\t"
      "v_cmp_ge_f32_e64 %3, %20, |%17|\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_ge_f32_e64 %1, %20, |%16|\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_ge_f32_e64 %2, %20, |%15|\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_ge_f32_e64 %3, %20, |%14|\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_ge_f32_e64 %1, %20, |%13|\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_ge_f32_e64 %2, %20, |%12|\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_ge_f32_e64 %3, %20, |%11|\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_ge_f32_e64 %1, %20, |%10|\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_ge_f32_e64 %2, %20, |%9|\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_ge_f32_e64 %3, %20, |%8|\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_ge_f32_e64 %1, %20, |%7|\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_ge_f32_e64 %2, %20, |%6|\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_ge_f32_e64 %3, %20, |%5|\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_ge_f32_e64 %1, %20, |%4|\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      : "+v"(w), "=&s"(p0), "=&s"(p1), "=&s"(p2)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]), "v"(thr));
}

// w = (w << 16) | bits, bit j = [ v[j] >= 0 ] (true for -0), j = 0..15.
__device__ __forceinline__ void push16_nonneg(uint32_t& w, const float* v) {
  uint64_t p0, p1, p2;
  asm(
      "v_cmp_le_f32_e64 %1, 0, %19\n\t"
      "v_cmp_le_f32_e64 %2, 0, %18\n\t"
      "v_cmp_le_f32_e64 %3, 0, %17\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_le_f32_e64 %1, 0, %16\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_le_f32_e64 %2, 0, %15\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_le_f32_e64 %3, 0, %14\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_le_f32_e64 %1, 0, %13\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_le_f32_e64 %2, 0, %12\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_le_f32_e64 %3, 0, %11\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_le_f32_e64 %1, 0, %10\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_le_f32_e64 %2, 0, %9\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_le_f32_e64 %3, 0, %8\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_le_f32_e64 %1, 0, %7\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_le_f32_e64 %2, 0, %6\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_le_f32_e64 %3, 0, %5\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_le_f32_e64 %1, 0, %4\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      : "+v"(w), "=&s"(p0), "=&s"(p1), "=&s"(p2)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
}

// w = (w << 8) | bits, bit j = [ |v[j]| <= thr ], j = 0..7 (same scheme, 8 elements).
__device__ __forceinline__ void push8_abs_le(uint32_t& w, const float* v, float thr) {
  uint64_t p0, p1, p2;
  asm(
      "v_cmp_ge_f32_e64 %1, %12, |%11|\n\t"
      "v_cmp_ge_f32_e64 %2, %12, |%10|\n\t"
      "v_cmp_ge_f32_e64 %3, %12, |%9|\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_ge_f32_e64 %1, %12, |%8|\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_ge_f32_e64 %2, %12, |%7|\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_ge_f32_e64 %3, %12, |%6|\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_ge_f32_e64 %1, %12, |%5|\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_ge_f32_e64 %2, %12, |%4|\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      : "+v"(w), "=&s"(p0), "=&s"(p1), "=&s"(p2)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(thr));
}

// w = (w << 8) | bits, bit j = [ v[j] >= 0 ] (true for -0), j = 0..7.
__device__ __forceinline__ void push8_nonneg(uint32_t& w, const float* v) {
  uint64_t p0, p1, p2;
  asm(
      "v_cmp_le_f32_e64 %1, 0, %11\n\t"
      "v_cmp_le_f32_e64 %2, 0, %10\n\t"
      "v_cmp_le_f32_e64 %3, 0, %9\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_le_f32_e64 %1, 0, %8\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_le_f32_e64 %2, 0, %7\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_cmp_le_f32_e64 %3, 0, %6\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_cmp_le_f32_e64 %1, 0, %5\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_cmp_le_f32_e64 %2, 0, %4\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %3\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      : "+v"(w), "=&s"(p0), "=&s"(p1), "=&s"(p2)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
}

// ----------------------------------------------------------------------------
// Matrix-core transform of 32-element runs (bf16 input).
//
// v_mfma_f32_16x16x32_bf16 computes D = A B for a 16 x 32 A, a 32 x 16 B and
// a 16 x 16 fp32 D.  Lane l = 16 g + n holds B[8 g + e][n] (e = 0..7, eight
// consecutive bf16 of one 16-byte load), A[n][8 g + e] and D[4 g + i][n]
// (i = 0..3).  Taking column n of B to be run n of a group of 16 runs and A
// to be 16 rows of the +-1 Sylvester matrix H_32, one instruction applies
// half of H_32 to 16 runs; two (row sets m = 0, 1) give all 32 outputs.  The
// rows are permuted so that lane (g, n) ends with outputs 8 g .. 8 g + 7 of
// run n, in order: row 4 g + i of row set m is Hadamard row 8 g + 4 m + i.
// Loads of the group (lane (g, n) reads 16 bytes at 64 n + 16 g) cover one
// contiguous kilobyte per instruction.  Products of bf16 values by +-1 are
// exact; the sums are accumulated in fp32.
// ----------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The A operand of row set m for this lane: entries (-1)^popcount(r & k) of
// Hadamard row r = 8 (n / 4) + 4 m + n % 4, columns k = 8 g .. 8 g + 7.
__device__ __forceinline__ bf16x8_t hadamard_fragment(int lane, int m) {
  const int n = lane & 15, g = lane >> 4;
  const int r = 8 * (n >> 2) + 4 * m + (n & 3);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const uint32_t lo = 0x3F80u | ((static_cast<uint32_t>(__builtin_popcount(r & (8 * g + e))) & 1u) << 15);
    const uint32_t hi = 0x3F80u | ((static_cast<uint32_t>(__builtin_popcount(r & (8 * g + e + 1))) & 1u) << 15);
    w[e / 2] = lo | (hi << 16);
  }
  return __builtin_bit_cast(bf16x8_t, u32x4{w[0], w[1], w[2], w[3]});
}

// Outputs 8 g .. 8 g + 7 of the lane's run of a 16-run group held in `f`
// (the lane's 16-byte B fragment), written to v[0..7].
__device__ __forceinline__ void mfma_run_outputs(const bf16x8_t& h0, const bf16x8_t& h1, const u32x4& f, float* v) {
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, f);
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  const f32x4_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h0, b, zero, 0, 0, 0);
  const f32x4_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h1, b, zero, 0, 0, 0);
  v[0] = d0.x;
  v[1] = d0.y;
  v[2] = d0.z;
  v[3] = d0.w;
  v[4] = d1.x;
  v[5] = d1.y;
  v[6] = d1.z;
  v[7] = d1.w;
}

// Sum of squares of the eight bf16 values of a fragment.  The dwords are
// copied out before the bit casts: __builtin_bit_cast applied directly to an
// element of an ext_vector_type value has been seen to read element 0 for
// every element.
__device__ __forceinline__ float sum_squares_fragment(const u32x4& f) {
  const uint32_t fx = f.x, fy = f.y, fz = f.z, fw = f.w;
  const bf16x2_t a = __builtin_bit_cast(bf16x2_t, fx), b = __builtin_bit_cast(bf16x2_t, fy);
  const bf16x2_t c = __builtin_bit_cast(bf16x2_t, fz), d = __builtin_bit_cast(bf16x2_t, fw);
  const float s0 = __builtin_amdgcn_fdot2_f32_bf16(b, b, __builtin_amdgcn_fdot2_f32_bf16(a, a, 0.f, false), false);
  const float s1 = __builtin_amdgcn_fdot2_f32_bf16(d, d, __builtin_amdgcn_fdot2_f32_bf16(c, c, 0.f, false), false);
  return s0 + s1;
}

// 4 x 4 transpose between lane quarters (g = lane / 16) and slots: afterwards
// slot j of quarter g holds what slot g of quarter j held (same lane within
// the quarter).  v_permlane32_swap exchanges the upper half-wave of its first
// operand with the lower half-wave of its second; v_permlane16_swap the odd
// 16-lane rows of its first operand with the even rows of its second.
__device__ __forceinline__ void transpose_quarters(uint32_t (&x)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  x[0] = c[0];
  x[1] = c[1];
  x[2] = d[0];
  x[3] = d[1];
}

// ----------------------------------------------------------------------------
// Packing of 32 b-bit codes into 4 b bytes (LSB-first stream).
// ----------------------------------------------------------------------------

template <int B>
struct CodeWords {
  uint32_t w[B];
};

template <int B>
__device__ __forceinline__ void put_code(CodeWords<B>& cw, int j, uint32_t code) {
  const int bit = j * B;
  const int wi = bit >> 5;
  const int off = bit & 31;
  cw.w[wi] |= code << off;
  if (off + B > 32) cw.w[wi + 1] |= code >> (32 - off);
}

// Store the codes of run `lane` of a window (4 B bytes per run): one access
// of 4..16 bytes for b <= 4, a 16-byte access plus one of 4..16 bytes above.
// P: the stores' cache policy (non-temporal by default).
template <int B, int P = kNonTemporal>
__device__ __forceinline__ void store_codes(rsrc_t r, int lane, const CodeWords<B>& cw) {
  const int off = lane * 4 * B;
  if constexpr (B == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(cw.w[0], r, off, 0, P);
  } else if constexpr (B == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{cw.w[0], cw.w[1]}, r, off, 0, P);
  } else if constexpr (B == 3) {
    __builtin_amdgcn_raw_buffer_store_b96(u32x3{cw.w[0], cw.w[1], cw.w[2]}, r, off, 0, P);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{cw.w[0], cw.w[1], cw.w[2], cw.w[3]}, r, off, 0, P);
    if constexpr (B == 5) {
      __builtin_amdgcn_raw_buffer_store_b32(cw.w[4], r, off + 16, 0, P);
    } else if constexpr (B == 6) {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{cw.w[4], cw.w[5]}, r, off + 16, 0, P);
    } else if constexpr (B == 7) {
      __builtin_amdgcn_raw_buffer_store_b96(u32x3{cw.w[4], cw.w[5], cw.w[6]}, r, off + 16, 0, P);
    } else if constexpr (B == 8) {
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{cw.w[4], cw.w[5], cw.w[6], cw.w[7]}, r, off + 16, 0,
                                             P);
    }
  }
}

template <int B>
__device__ __forceinline__ uint32_t get_code(const CodeWords<B>& cw, int j) {
  const int bit = j * B;
  const int wi = bit >> 5;
  const int off = bit & 31;
  uint32_t c = cw.w[wi] >> off;
  if (off + B > 32) c |= cw.w[wi + 1] << (32 - off);
  return c & ((1u << B) - 1u);
}

// Load the codes of the run at byte offset `off` of a window (zeros past its end).
template <int B>
__device__ __forceinline__ CodeWords<B> load_codes_at(rsrc_t r, int off) {
  CodeWords<B> cw;
  if constexpr (B == 1) {
    cw.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (B == 2) {
    const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    cw.w[0] = t.x;
    cw.w[1] = t.y;
  } else if constexpr (B == 3) {
    const u32x3 t = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    cw.w[0] = t.x;
    cw.w[1] = t.y;
    cw.w[2] = t.z;
  } else {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    cw.w[0] = t.x;
    cw.w[1] = t.y;
    cw.w[2] = t.z;
    cw.w[3] = t.w;
    if constexpr (B == 5) {
      cw.w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 16, 0, 0);
    } else if constexpr (B == 6) {
      const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(r, off + 16, 0, 0);
      cw.w[4] = h.x;
      cw.w[5] = h.y;
    } else if constexpr (B == 7) {
      const u32x3 h = __builtin_amdgcn_raw_buffer_load_b96(r, off + 16, 0, 0);
      cw.w[4] = h.x;
      cw.w[5] = h.y;
      cw.w[6] = h.z;
    } else if constexpr (B == 8) {
      const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
      cw.w[4] = h.x;
      cw.w[5] = h.y;
      cw.w[6] = h.z;
      cw.w[7] = h.w;
    }
  }
  return cw;
}

// Load the codes of run `lane` of a window (zeros past its end).
template <int B>
__device__ __forceinline__ CodeWords<B> load_codes(rsrc_t r, int lane) {
  return load_codes_at<B>(r, lane * 4 * B);
}

}  // namespace quest

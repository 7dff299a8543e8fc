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
// Loads: one run of 32 elements, widened exactly to fp32.
// ----------------------------------------------------------------------------

__device__ __forceinline__ void load_run(const uint16_t* __restrict__ p, float (&v)[RUN]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = q[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // bf16 is the upper half of an fp32: widening is a shift or a mask.
      v[8 * i + 2 * j] = __uint_as_float(d[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ void load_run(const float* __restrict__ p, float (&v)[RUN]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 t = q[i];
    v[4 * i] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
}

// Masked loads for the backward pass: element j is kept when bit j of `m`
// is set, otherwise it becomes +0.  The bit is sign-extended to an all-ones
// or all-zeros dword and ANDed onto the fp32 bit pattern.
__device__ __forceinline__ void load_run_masked(const uint16_t* __restrict__ p, uint32_t m, float (&v)[RUN]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = q[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 8 * i + 2 * j;
      const uint32_t keep_lo = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(m), e, 1));
      const uint32_t keep_hi = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(m), e + 1, 1));
      v[e] = __uint_as_float((d[j] << 16) & keep_lo);
      v[e + 1] = __uint_as_float(d[j] & 0xFFFF0000u & keep_hi);
    }
  }
}

__device__ __forceinline__ void load_run_masked(const float* __restrict__ p, uint32_t m, float (&v)[RUN]) {
  load_run(p, v);
#pragma unroll
  for (int e = 0; e < RUN; ++e) {
    const uint32_t keep = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(m), e, 1));
    v[e] = __uint_as_float(__float_as_uint(v[e]) & keep);
  }
}

// ----------------------------------------------------------------------------
// Stores of a run of fp32 results, rounded to the output type.
// ----------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // Round to nearest even: the gfx950 conversion instruction does this.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {lo, hi};
  const bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void store_run(uint16_t* __restrict__ p, const float (&v)[RUN]) {
  uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 t;
    t.x = pack_bf16x2(v[8 * i + 0], v[8 * i + 1]);
    t.y = pack_bf16x2(v[8 * i + 2], v[8 * i + 3]);
    t.z = pack_bf16x2(v[8 * i + 4], v[8 * i + 5]);
    t.w = pack_bf16x2(v[8 * i + 6], v[8 * i + 7]);
    q[i] = t;
  }
}

__device__ __forceinline__ void store_run(float* __restrict__ p, const float (&v)[RUN]) {
  float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// ----------------------------------------------------------------------------
// Unnormalised Walsh-Hadamard butterflies (Sylvester order).
// ----------------------------------------------------------------------------

// In-lane stages: pairs 1, 2, 4, 8, 16 apart.
__device__ __forceinline__ void fwht_in_lane(float (&v)[RUN]) {
#pragma unroll
  for (int s = 1; s < RUN; s <<= 1) {
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
#define QUEST_FMAC_DPP8(PERM)                                                                              \
  asm volatile(                                                                                            \
      "s_nop 1\n\t"                                                                                        \
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
template <int LOGN>
__device__ __forceinline__ float fwht_block(float (&v)[RUN], int lane) {
  static_assert(LOGN >= 6 && LOGN <= 8, "block sizes 64, 128 and 256");
  fwht_in_lane(v);
  const float s1 = (lane & 1) ? -1.0f : 1.0f;
  fwht_lane_xor1(v, s1);
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

template <int B>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ codes, int64_t run, const CodeWords<B>& cw) {
  uint32_t* p = reinterpret_cast<uint32_t*>(codes) + run * B;
  if constexpr (B == 1) {
    p[0] = cw.w[0];
  } else if constexpr (B == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(cw.w[0], cw.w[1]);
  } else if constexpr (B == 3) {
    p[0] = cw.w[0];
    p[1] = cw.w[1];
    p[2] = cw.w[2];
  } else {
    *reinterpret_cast<uint4*>(p) = make_uint4(cw.w[0], cw.w[1], cw.w[2], cw.w[3]);
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

template <int B>
__device__ __forceinline__ CodeWords<B> load_codes(const uint8_t* __restrict__ codes, int64_t run) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(codes) + run * B;
  CodeWords<B> cw;
  if constexpr (B == 1) {
    cw.w[0] = p[0];
  } else if constexpr (B == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    cw.w[0] = t.x;
    cw.w[1] = t.y;
  } else if constexpr (B == 3) {
    cw.w[0] = p[0];
    cw.w[1] = p[1];
    cw.w[2] = p[2];
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    cw.w[0] = t.x;
    cw.w[1] = t.y;
    cw.w[2] = t.z;
    cw.w[3] = t.w;
  }
  return cw;
}

}  // namespace quest

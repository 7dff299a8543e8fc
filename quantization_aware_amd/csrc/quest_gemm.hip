// Product of two QuEST-quantised operands on the gfx950 matrix cores.
//
// QuEST's 4-bit layers multiply two quantised operands, whose levels are
// half-integer multiples of each row's step (pith.science review of QuEST,
// Figure 5 caption: per-layer speedups of the 4-bit product over BF16,
// quantisation, dequantisation and Hadamard costs included; atlas.scime.ai
// summary, "Key results").  For b <= 4 each level over its row's step,
// u - (L - 1)/2, is a half-integer of magnitude at most 7.5, which the FP6
// E2M3 element type holds exactly (OCP Microscaling Formats v1.0).  So
//   y[i][j] = Delta_a[i] Delta_b[j] * sum_k va[i][k] vb[j][k]
// is one FP6 x FP6 matrix product (v_mfma_scale_f32_32x32x64_f8f6f4 with
// unit block scales) followed by a per-row and per-column scaling.  Products
// of half-integers are quarter-integers and their sums stay below 2^22 in
// magnitude for k <= 65536, so the fp32 accumulation is exact; the only
// roundings are those of Delta, Delta_a Delta_b and the final product.
//
// Operand layout (written by the forward pass, see include/quest.h): rows in
// blocks of 32, k in chunks of 128; block (rb, c) is 3072 contiguous bytes at
// (rb * k / 128 + c) * 3072, holding two 1536-byte fragments (k-halves of 64),
// each 64 lane slots of 24 bytes: slot l carries row 32 rb + l % 32, the 32
// values starting at k = 128 c + 64 ks + 32 (l / 32), as 6-bit fields
// LSB-first -- exactly the register operand of one lane of the 32x32x64
// instruction.
//
// Kernel: a workgroup of 8 waves (two per SIMD) computes a 256 x 256 output
// tile, each wave 128 rows x 64 columns (8 accumulator tiles of 32 x 32).
// Operand blocks stream from HBM/L2 straight into LDS (buffer loads with the
// LDS-destination bit, 1 KB per wave instruction), three stages deep.  Per
// stage (k = 128) a wave runs 16 MFMAs in two halves, reading the next half's
// fragments from LDS meanwhile; one barrier per stage publishes the next
// stage.  With two waves per SIMD one wave's fragment reads and waits overlap
// the other's MFMAs.  The clip scales reach LDS the same way.  The epilogue
// scales by Delta_a Delta_b and writes whole row segments through LDS.  When
// the tiles are more than one round, one workgroup per compute unit walks
// several tiles, requesting the next tile's first stages before it stores the
// finished one.
#include <atomic>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "quest_launch.h"

namespace quest {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileM = 256, kTileN = 256;  // workgroup output tile
constexpr int kFrag = 64 * 24;             // one 32-row x 64-k fragment
constexpr int kBlock = 2 * kFrag;          // one 32-row x 128-k block
constexpr int kOpStage = 8 * kBlock;       // one operand's 256 rows of a stage
constexpr int kStage = 2 * kOpStage;       // both operands
constexpr int kNowhereOff = 0x7FFFFFF0;    // past every window: stores there are dropped

// Raw buffer resource: base, byte count, 32-bit raw format; out-of-range
// loads return zero and out-of-range stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// The same resource as four dwords, for the asm loads below.
__device__ __forceinline__ i32x4 raw_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4{static_cast<int32_t>(static_cast<uint32_t>(a)), static_cast<int32_t>((a >> 32) & 0xFFFFu),
               static_cast<int32_t>(bytes), 0x00020000};
}

// Two floats to bf16 with round to nearest even (the gfx950 conversion instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// 16 bytes from global memory into LDS at lds_base + 16 * lane.  Written as
// asm so that the compiler's wait counting leaves these loads alone: each
// stage is read only after an explicit vmcnt wait and a barrier.  The load
// has no register results.
__device__ __forceinline__ void dma16(uint32_t lds_base, int32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory");
}

// 4 bytes from global memory into LDS at lds_base + 4 * lane (as dma16).
__device__ __forceinline__ void dma4(uint32_t lds_base, int32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory");
}

// s_waitcnt with only the vector-memory counter limited (lgkm and exp left
// open); the count's low four bits go to bits 3..0, the high two to 15..14.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x3F70 | (N & 15) | ((N >> 4) << 14));
}

// A workgroup barrier that waits for this wave's LDS accesses only (a
// __syncthreads would also wait for every load and store in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Output tiles of one workgroup: rounds r = 0, 1, ... of tile_of(r, tm, col0)
// until it returns false.  Each tile covers rows 256 tm .. + 255 and columns
// col0 .. col0 + 128 WNB - 1 (WNB B blocks of 32 per wave: 2 for a full
// 256-column tile, 1 for a half tile), 8 waves as 2 x 4, each 128 rows x
// 32 WNB columns.  Between two tiles the next tile's first two stages are
// requested before the finished tile's output is stored, so that the stores
// drain while the next tile's operands arrive; this takes a bf16 output
// (the output slab then fits the third stage buffer) with 16-byte stores
// (16 per wave, which the first waits of the next tile let pass).
template <typename Out, bool kVec, int WNB, typename TileOf>
__device__ __forceinline__ void gemm_tiles(const uint8_t* __restrict__ a, const float* __restrict__ sa, int m,
                                           const uint8_t* __restrict__ b, const float* __restrict__ sb, int n, int k,
                                           float ka, float kb, Out* __restrict__ out, uint8_t* lds, TileOf tile_of) {
  constexpr int kTileW = 128 * WNB;  // columns of the tile
  constexpr int kOut = static_cast<int>(sizeof(Out));
  constexpr int kPer = 16 / kOut;              // outputs per 16-byte chunk
  constexpr int kLanesPerRow = 32 * WNB / kPer;
  constexpr int kPitch = 32 * WNB * kOut + 16;  // slab row pitch in bytes
  // Memory operations a wave issues after the next tile's first two stages,
  // when those go first: the load of the next tile's scales into LDS and the
  // epilogue's 16-byte stores.
  constexpr int kAfterStages = 1 + 4 * (32 * kLanesPerRow / 64);
  constexpr bool kOverlap = kVec && kOut == 2 && WNB == 2;
  static_assert(!kOverlap || 8 * 32 * kPitch <= kStage, "bf16 slabs fit the third stage buffer");
  static_assert(8 * 32 * kPitch <= 2 * kStage, "slabs fit in the second and third stage buffers");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  auto stage_mem = [&](auto bi) -> uint8_t* { return lds + decltype(bi)::value * kStage; };
  // Clip scales of a tile: [0, 256) rows, [256, 512) columns, two buffers
  // (tile r uses buffer r % 2, so that the next tile's can land while this
  // tile's epilogue reads its own).
  auto scales_mem = [&](int r) -> float* { return reinterpret_cast<float*>(lds + 3 * kStage) + (r & 1) * 512; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid) >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  // The lane's addresses are derived from `lane` afresh in each phase of a
  // tile (main loop, epilogue): `renew` hides its value from the compiler,
  // so that it does not compute one phase's addresses ahead and keep them in
  // registers through the other.
  int lane = tid & 63;
  auto renew = [&]() { asm volatile("" : "+v"(lane)); };
  const int chunks = k >> 7;
  const int stages = chunks;
  const uint32_t rb_bytes = static_cast<uint32_t>(chunks) * kBlock;  // one 32-row block, all of k
  const int rb_a = (m + 31) >> 5, rb_b = (n + 31) >> 5;

  struct Tile {
    int tm, col0;
    i32x4 ra, rb;
  };
  auto make_tile = [&](int tm, int col0) -> Tile {
    Tile t;
    t.tm = tm;
    t.col0 = col0;
    t.ra = raw_rsrc(a + static_cast<size_t>(tm) * 8 * rb_bytes, min(rb_a - tm * 8, 8) * rb_bytes);
    // (a half tile can lie wholly past n: then its windows are empty and every
    // load reads zeros)
    const int cb0 = col0 >> 5;
    const int b_blocks = __builtin_amdgcn_readfirstlane(max(min(rb_b - cb0, 4 * WNB), 0));
    t.rb = raw_rsrc(b + static_cast<size_t>(cb0) * rb_bytes, b_blocks * rb_bytes);
    return t;
  };
  // The tile's row and column clip scales into scales_mem(r): wave w < 4
  // loads rows 64 w .. 64 w + 63, wave 4 + c columns 64 c .. 64 c + 63, one
  // load into LDS each (entries past m or n read zero).
  auto fetch_scales = [&](const Tile& t, int r) {
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(scales_mem(r))) + 256 * wave;
    if (wave < 4) {
      const int first = t.tm * kTileM + 64 * wave;
      const int count = __builtin_amdgcn_readfirstlane(max(min(m - first, 64), 0));
      dma4(base, lane * 4, raw_rsrc(sa + first, count * 4));
    } else {
      const int first = t.col0 + 64 * (wave - 4);
      const int count = __builtin_amdgcn_readfirstlane(max(min(n - first, 64), 0));
      dma4(base, lane * 4, raw_rsrc(sb + first, count * 4));
    }
  };

  // Stage st of tile t into LDS: A's 8 blocks are 24 KB = 24 wave
  // instructions, wave w issuing t = w + 8 u, u < 3.  B's 4 WNB blocks are
  // 12 WNB instructions: for a full tile spread the same way; for a half tile
  // (12) wave w issues t = (w + 8 u) % 12, u < 2, so waves 4..7 repeat four of
  // them (the same bytes to the same place) and every wave issues the same
  // number of loads.
  constexpr int kLoads = WNB == 2 ? 6 : 5;  // loads one wave issues per stage
  auto fetch = [&](const Tile& tl, int st, auto bi) {
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage_mem(bi)));
    const i32x4 qa = tl.ra, qb = tl.rb;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int t = wave + 8 * u, blk = t / 3, part = t % 3;
      const int goff = blk * static_cast<int>(rb_bytes) + st * kBlock + part * 1024 + lane * 16;
      const uint32_t la = base + blk * kBlock + part * 1024;
      dma16(__builtin_amdgcn_readfirstlane(la), goff, qa);
      if constexpr (WNB == 2) {
        dma16(__builtin_amdgcn_readfirstlane(la + kOpStage), goff, qb);
      } else if (u < 2) {
        const int tb = t % 12, bblk = tb / 3, bpart = tb % 3;
        const int bgoff = bblk * static_cast<int>(rb_bytes) + st * kBlock + bpart * 1024 + lane * 16;
        dma16(__builtin_amdgcn_readfirstlane(base + kOpStage + bblk * kBlock + bpart * 1024), bgoff, qb);
      }
    }
  };

  // Fragment (block rbk, k-half ks) of operand op: this lane's 24 bytes.
  auto frag = [&](auto bi, int op, int rbk, int ks) -> v8i {
    const u32x2* s = reinterpret_cast<const u32x2*>(stage_mem(bi) + op * kOpStage + rbk * kBlock + ks * kFrag + lane * 24);
    const u32x2 x0 = s[0], x1 = s[1], x2 = s[2];
    return v8i{static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x1[0]),
               static_cast<int>(x1[1]), static_cast<int>(x2[0]), static_cast<int>(x2[1]), 0, 0};
  };

  int tm0, col00;
  if (!tile_of(0, tm0, col00)) return;
  Tile cur = make_tile(tm0, col00);
  fetch_scales(cur, 0);
  fetch(cur, 0, I0{});
  fetch(cur, stages > 1 ? 1 : 0, I1{});
  bool stores_pending = false;  // the previous tile's output stores follow this tile's first two stages

  for (int r = 0;; ++r) {
    // acc[j][i]: 32 x 32 tile of the product B A^T for B block j and A block
    // i, so lane l holds output row 32 i + l % 32 and four consecutive
    // columns per register quad.
    v16f acc[WNB][4];
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = v16f{};

    renew();
    // Stage 0 has landed (stage 1 and the previous tile's stores may be in flight).
    if (kOverlap && stores_pending)
      wait_vmcnt<kLoads + kAfterStages>();
    else
      wait_vmcnt<kLoads>();
    lds_barrier();
    v8i f0a[4], f0b[WNB], f1a[4], f1b[WNB];
#pragma unroll
    for (int i = 0; i < 4; ++i) f0a[i] = frag(I0{}, 0, wm * 4 + i, 0);
#pragma unroll
    for (int j = 0; j < WNB; ++j) f0b[j] = frag(I0{}, 1, wn * WNB + j, 0);
    // One stage: bi holds stage s, bn stage s + 1, b2 receives stage s + 2.
    // b2 last held stage s - 1, whose reads every wave finished before the
    // previous barrier.  Stages past the last are fetched again (the last
    // one), so that every stage's wait counts the same loads.
    auto step = [&](int s, auto bi, auto bn, auto b2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) f1a[i] = frag(bi, 0, wm * 4 + i, 1);
#pragma unroll
      for (int j = 0; j < WNB; ++j) f1b[j] = frag(bi, 1, wn * WNB + j, 1);
#pragma unroll
      for (int j = 0; j < WNB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f0b[j], f0a[i], acc[j][i], 2, 2, 0, 127, 0, 127);
      fetch(cur, s + 2 < stages ? s + 2 : stages - 1, b2);
      // stage s + 1 has landed (on the first stage the previous tile's
      // scale load and stores, issued before this stage's loads, may still
      // be in flight)
      if (kOverlap && stores_pending && s == 0)
        wait_vmcnt<kLoads + kAfterStages>();
      else
        wait_vmcnt<kLoads>();
      lds_barrier();  // and every wave's LDS reads of stage s are done
#pragma unroll
      for (int i = 0; i < 4; ++i) f0a[i] = frag(bn, 0, wm * 4 + i, 0);
#pragma unroll
      for (int j = 0; j < WNB; ++j) f0b[j] = frag(bn, 1, wn * WNB + j, 0);
#pragma unroll
      for (int j = 0; j < WNB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f1b[j], f1a[i], acc[j][i], 2, 2, 0, 127, 0, 127);
    };
    int s = 0;
    for (; s + 3 <= stages; s += 3) {
      step(s, I0{}, I1{}, I2{});
      step(s + 1, I1{}, I2{}, I0{});
      step(s + 2, I2{}, I0{}, I1{});
    }
    if (s < stages) step(s++, I0{}, I1{}, I2{});
    if (s < stages) step(s++, I1{}, I2{}, I0{});
    wait_vmcnt<0>();  // no load into LDS in flight before it is reused
    lds_barrier();

    renew();
    // The next tile: its first two stages go out before this tile's stores
    // (only with kOverlap; otherwise after them), its scale once this
    // tile's has been used.
    int tm_n = 0, col0_n = 0;
    const bool has_next = tile_of(r + 1, tm_n, col0_n);
    const Tile next = has_next ? make_tile(tm_n, col0_n) : cur;
    if (kOverlap && has_next) {
      fetch(next, 0, I0{});
      fetch(next, stages > 1 ? 1 : 0, I1{});
    }

    // Epilogue.  The row and column factors are Delta = s * 2 / (L - 1).
    if (kOverlap && has_next) fetch_scales(next, r + 1);
    const float* fac = scales_mem(r);
    // Each wave stages a 32 x 32 WNB slab of its part in its own LDS region
    // (the third stage buffer when the next tile's stages fill the first two)
    // and writes it as whole row segments.
    uint8_t* slab = lds + (kOverlap ? 2 : 1) * kStage + wave * 32 * kPitch;
    const int rows_left = m - cur.tm * kTileM;
    const auto rout = make_rsrc(out + static_cast<size_t>(cur.tm) * kTileM * n,
                                static_cast<uint32_t>(min(rows_left, kTileM)) * static_cast<uint32_t>(n) * kOut);
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float fa = fac[wm * 128 + 32 * i + r32] * ka;
#pragma unroll
      for (int j = 0; j < WNB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cl = 32 * j + 8 * q + 4 * h;  // column within the wave's 32 WNB
          // column factors of the lane's columns cl .. cl + 3
          const float4 sbv = *reinterpret_cast<const float4*>(&fac[kTileM + wn * 32 * WNB + cl]);
          const float4 fb = make_float4(sbv.x * kb, sbv.y * kb, sbv.z * kb, sbv.w * kb);
          const float y0 = acc[j][i][4 * q + 0] * (fa * fb.x), y1 = acc[j][i][4 * q + 1] * (fa * fb.y);
          const float y2 = acc[j][i][4 * q + 2] * (fa * fb.z), y3 = acc[j][i][4 * q + 3] * (fa * fb.w);
          uint8_t* d = slab + r32 * kPitch + cl * kOut;
          if constexpr (kOut == 4) {
            *reinterpret_cast<u32x4*>(d) =
                u32x4{__float_as_uint(y0), __float_as_uint(y1), __float_as_uint(y2), __float_as_uint(y3)};
          } else {
            *reinterpret_cast<u32x2*>(d) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
          }
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < 32 * kLanesPerRow / 64; ++t) {
        const int sr = t * (64 / kLanesPerRow) + lane / kLanesPerRow, sc = (lane % kLanesPerRow) * kPer;
        const int row = wm * 128 + 32 * i + sr;  // within the tile
        const int col = cur.col0 + wn * 32 * WNB + sc;
        const uint8_t* src = slab + sr * kPitch + sc * kOut;
        if constexpr (kVec) {
          // n is a multiple of kPer: a chunk is wholly inside or wholly past the row
          const u32x4 v = *reinterpret_cast<const u32x4*>(src);
          const int off = col < n ? (row * n + col) * kOut : kNowhereOff;
          __builtin_amdgcn_raw_buffer_store_b128(v, rout, off, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < kPer; ++e) {
            const int off = col + e < n ? (row * n + col + e) * kOut : kNowhereOff;
            if constexpr (kOut == 4) {
              __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(src + 4 * e), rout, off, 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b16(*reinterpret_cast<const uint16_t*>(src + 2 * e), rout, off, 0, 0);
            }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (!has_next) return;
    if (!kOverlap) {
      // every wave's slab reads are done before the next stages land there
      lds_barrier();
      fetch_scales(next, r + 1);
      fetch(next, 0, I0{});
      fetch(next, stages > 1 ? 1 : 0, I1{});
    }
    cur = next;
    stores_pending = kOverlap;
  }
}

// Tile index -> (tm, tn): groups of 8 tile rows, walked column by column.
__device__ __forceinline__ void tile_at(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = 8 * tiles_n;
  const int first_m = (pid / group) * 8;
  const int gm = min(tiles_m - first_m, 8);
  tm = first_m + (pid % group) % gm;
  tn = (pid % group) / gm;
}

// Full tiles (WNB = 2), tiles 0 .. tile_count - 1 of the tile order above.
// Workgroups are dealt to the 8 XCDs round-robin; each XCD takes a
// contiguous range of tiles, so that the tiles sharing operand blocks share
// an L2.  Without kWalk every workgroup computes one tile (the last
// tile_count % 8 keep their own index); with it the grid is a multiple of 8
// workgroups that each walk their XCD's range, gridDim.x / 8 tiles per XCD
// at a time.  Half tiles (WNB = 1): workgroup w computes half w % 2 of
// tile first_tile + w / 2, for the tiles of a last round that would hold at
// most half the compute units.
template <typename Out, bool kVec, int WNB, bool kWalk = false>
__global__ void __launch_bounds__(512, 1)
    quest_gemm_e2m3_kernel(const uint8_t* __restrict__ a, const float* __restrict__ sa, int m,
                           const uint8_t* __restrict__ b, const float* __restrict__ sb, int n, int k, float ka,
                           float kb, Out* __restrict__ out, int tile_count, int first_tile) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[3 * kStage + 2 * 2 * kTileM * 4];
  const int tiles_m = (m + kTileM - 1) / kTileM, tiles_n = (n + kTileN - 1) / kTileN;
  if constexpr (WNB == 2) {
    const int bid = blockIdx.x;
    if constexpr (!kWalk) {
      gemm_tiles<Out, kVec, 2>(a, sa, m, b, sb, n, k, ka, kb, out, lds, [&](int r, int& tm, int& col0) {
        if (r > 0) return false;
        int pid = bid, tn;
        const int full = tile_count & ~7;
        if (pid < full) pid = (pid & 7) * (full >> 3) + (pid >> 3);
        tile_at(pid, tiles_m, tiles_n, tm, tn);
        col0 = tn * kTileN;
        return true;
      });
    } else {
      const int per_xcd = tile_count >> 3, per_round = static_cast<int>(gridDim.x) >> 3;
      const int xcd = bid & 7, slot = bid >> 3;
      gemm_tiles<Out, kVec, 2>(a, sa, m, b, sb, n, k, ka, kb, out, lds, [&](int r, int& tm, int& col0) {
        const int q = r * per_round + slot;
        if (q >= per_xcd) return false;
        int tn;
        tile_at(xcd * per_xcd + q, tiles_m, tiles_n, tm, tn);
        col0 = tn * kTileN;
        return true;
      });
    }
  } else {
    const int h = blockIdx.x;
    gemm_tiles<Out, kVec, 1>(a, sa, m, b, sb, n, k, ka, kb, out, lds, [&](int r, int& tm, int& col0) {
      if (r > 0) return false;
      int tn;
      tile_at(first_tile + (h >> 1), tiles_m, tiles_n, tm, tn);
      col0 = tn * kTileN + (h & 1) * (kTileN / 2);
      return true;
    });
  }
}

// Compute units of the current device (cached per device; concurrent first
// calls on one device may both query it and store the same value).
int device_cus() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

template <typename Out, bool kVec>
hipError_t launch(const GemmLaunch& g) {
  const int tiles = ((g.m + kTileM - 1) / kTileM) * ((g.n + kTileN - 1) / kTileN);
  // One workgroup per compute unit at a time (LDS): if the last round would
  // hold at most half the compute units, its tiles are split in halves.
  const int cus = device_cus();
  const int last = tiles % cus;
  const int full_tiles = tiles > cus && last > 0 && 2 * last <= cus ? tiles - last : tiles;
  // Several tiles per workgroup (the next tile's first stages requested
  // before the last one's stores) for a bf16 output of whole 16-byte chunks
  // and at least three stages, when the full tiles are more than one round
  // and split evenly over the XCDs.
  const bool walk = sizeof(Out) == 2 && kVec && g.k >= 3 * 128 && full_tiles > cus && full_tiles % 8 == 0 &&
                    cus % 8 == 0;
  bool launched = false;
  if constexpr (sizeof(Out) == 2 && kVec) {
    if (walk) {
      hipLaunchKernelGGL((quest_gemm_e2m3_kernel<Out, kVec, 2, true>), dim3(cus), dim3(512), 0,
                         static_cast<hipStream_t>(g.stream), g.a, g.sa, g.m, g.b, g.sb, g.n, g.k, g.ka, g.kb,
                         static_cast<Out*>(g.out), full_tiles, 0);
      launched = true;
    }
  }
  if (!launched)
    hipLaunchKernelGGL((quest_gemm_e2m3_kernel<Out, kVec, 2>), dim3(full_tiles), dim3(512), 0,
                       static_cast<hipStream_t>(g.stream), g.a, g.sa, g.m, g.b, g.sb, g.n, g.k, g.ka, g.kb,
                       static_cast<Out*>(g.out), full_tiles, 0);
  if (full_tiles < tiles) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((quest_gemm_e2m3_kernel<Out, kVec, 1>), dim3(2 * (tiles - full_tiles)), dim3(512), 0,
                       static_cast<hipStream_t>(g.stream), g.a, g.sa, g.m, g.b, g.sb, g.n, g.k, g.ka, g.kb,
                       static_cast<Out*>(g.out), tiles - full_tiles, full_tiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_e2m3(const GemmLaunch& g, bool out_bf16) {
  if (out_bf16) return g.n % 8 == 0 ? launch<uint16_t, true>(g) : launch<uint16_t, false>(g);
  return g.n % 4 == 0 ? launch<float, true>(g) : launch<float, false>(g);
}

}  // namespace quest

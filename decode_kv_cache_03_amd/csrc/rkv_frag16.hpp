// 16x16x32 bf16 MFMA fragments and lane-quarter reductions (gfx950), shared
// by the kernels that hold keys in registers in this layout
// (k2_resident.hip, k2_long.hip).
//
// Fragments. A 16-row operand of v_mfma_f32_16x16x32_bf16 gives lane l row
// l % 16 and the 8 k-values of its quarter q = l / 16. Over a 128-element
// row, k-step ks takes the 16-byte chunk q + 4*ks, so the four quarters of a
// row cover 64 contiguous bytes per k-step, and A and B fragments of the same
// rows are the same registers. The accumulator of a 16x16 tile gives lane l
// rows 4q + v (v = 0..3) of column l % 16.
//
// Importance: softmax attention of the window queries over the unit's keys
// (query r sees keys j <= N-w+r; every key without the causal window), mean
// over a head's w queries, max (or, as the pooling ablation, mean) over the
// G heads of the GQA group ("R-KV: Redundancy-aware KV Cache Compression for
// Reasoning Models", atlas.scime.ai summary, "Approach" and "Measured
// effects reported in the paper").
#pragma once

#include "rkv_device.hpp"

namespace rkv {
namespace frag16 {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The value of lane l and of lane l ^ 16 (or l ^ 32), the lower lane's first,
// from one VALU lane swap (gfx950): a butterfly step is op(lo, hi), the same
// operands in the same order in both lanes.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float sum_quarters(float x) {   // over lanes l, l^16, l^32, l^48
  const LanePair a = pair16(x);
  const LanePair b = pair32(a.lo + a.hi);
  return b.lo + b.hi;
}

// max(a, b) that propagates NaN (IEEE 754-2019 maximum; -0 < +0). Unlike
// fmaxf it needs no quieting of its inputs, so a running max over products
// compiles to one v_maximum3_f32 per one or two new values, and a max of
// values that came through a lane swap or from LDS is one instruction, not
// three. The scores here hold no NaN, where the two agree up to the sign of
// a zero.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float max_quarters(float x) {
  const LanePair a = pair16(x);
  const LanePair b = pair32(vmax(a.lo, a.hi));
  return vmax(b.lo, b.hi);
}

// Scheduling hint for one pipeline stage of 8 MFMA and 12 VALU instructions
// (products of one row half-block, maxima of the previous one): two MFMA,
// then six times two VALU and one MFMA, so the VALU work sits between the
// matrix instructions instead of after all of them.
__device__ __forceinline__ void interleave_8mfma_12valu() {
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// acc += A * B over 32 k-values (16x16 tile): lane l gives row / column
// l % 16 and k-values 8*(l/16).. of its operand; lane l receives
// C[4*(l/16) + v][l % 16] in acc[v].
__device__ __forceinline__ void mma16(f32x4_t& acc, u32x4_t a, u32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                               __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// Fragment of 16 rows of a swizzled 128-row tile (or of the query block):
// lane l takes row r0 + l % 16, chunk (l / 16) + 4*ks for k-step ks.
__device__ __forceinline__ void load_frag(const char* base, int r0, int lane, u32x4_t (&f)[4]) {
  const int row = r0 + (lane & 15), q = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) f[ks] = ld16(base + frag_offset<bf16_bits>(row, q + 4 * ks));
}

// Query fragments of the window: MFMA row m = 16*qs + l%16 is query row r of
// head g with m = g * 2^rpg_shift + r; padding rows are zero (kZeroPad), or
// a copy of row 0 where the caller discards them anyway (the softmax
// statistics: padding columns are marked unseen when they are merged).
template <bool kZeroPad = true>
__device__ __forceinline__ void load_queries(const char* qlds, int lane, int W, int G, int rpg_shift,
                                             u32x4_t (&qf)[2][4]) {
  const int rpg_mask = (1 << rpg_shift) - 1;
  const int q = lane >> 4;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int m = qs * 16 + (lane & 15);
    const int g = m >> rpg_shift, r = m & rpg_mask;
    const bool ok = g < G && r < W;
    const int n = ok ? g * W + r : 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4_t x = ld16(qlds + frag_offset<bf16_bits>(n, q + 4 * ks));
      qf[qs][ks] = (!kZeroPad || ok) ? x : zero16();
    }
  }
}

// Importance of 16 keys key0 + l%16 from their fragments (lane l's key is
// l % 16 in every quarter): weights of the window queries as MFMA rows
// (queries 16*qs + 4*(l/16) + v in acc[qs][v]), summed over a head's rows
// and pooled over heads by in-lane steps and two lane exchanges, then
// scaled by inv_pool (1/w; 1/(w*G) under mean pooling).
__device__ __forceinline__ float key_importance16(const u32x4_t (&kf)[4], const u32x4_t (&qf)[2][4],
                                                  const float (&smax)[2][4],
                                                  const float (&sinv)[2][4], int key0, int N,
                                                  int W, int rpg_shift, bool causal, bool mean,
                                                  float inv_pool, int lane) {
  asm volatile("" : "+v"(lane));   // per call: keeps lane-derived masks out of loop preheaders
  const int rpg_mask = (1 << rpg_shift) - 1;
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) mma16(acc[qs], qf[qs][ks], kf[ks]);   // C[query][key]
  const int key = key0 + (lane & 15);
  const int q = lane >> 4;
  // bit b of the query index m = 16 qs + 4 q + v: summed within a head
  // (b < rpg_shift) or under mean pooling, else max over heads
  auto comb = [&](float a, float b, int bit) {
    return (mean || bit < rpg_shift) ? a + b : vmax(a, b);
  };
  // probabilities; keys before the window are seen by every window query
  // (a block-uniform test), so only later keys take the causal mask
  float w[2][4];
  const bool all_seen = !causal || key0 + 15 <= N - W;
  if (all_seen) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        w[qs][v] = fast_exp2(acc[qs][v] * kLogitScaleLog2 - smax[qs][v]) * sinv[qs][v];
  } else {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = qs * 16 + 4 * q + v;
        const float pr = fast_exp2(acc[qs][v] * kLogitScaleLog2 - smax[qs][v]) * sinv[qs][v];
        w[qs][v] = key <= N - W + (m & rpg_mask) ? pr : 0.f;
      }
  }
  if (!mean && rpg_shift == 3) {
    // 8 rows per head (windows of 5..8 queries), max over heads: bits 0..2
    // of the query index are summed, bits 3 and 4 maxed
    float x[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      x[qs] = (w[qs][0] + w[qs][1]) + (w[qs][2] + w[qs][3]);
      const LanePair a = pair16(x[qs]);
      x[qs] = a.lo + a.hi;
      const LanePair b = pair32(x[qs]);
      x[qs] = vmax(b.lo, b.hi);
    }
    return vmax(x[0], x[1]) * inv_pool;
  }
  float x[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    x[qs] = comb(comb(w[qs][0], w[qs][1], 0), comb(w[qs][2], w[qs][3], 0), 1);
    const LanePair a = pair16(x[qs]);
    const LanePair b = pair32(comb(a.lo, a.hi, 2));
    x[qs] = comb(b.lo, b.hi, 3);
  }
  return comb(x[0], x[1], 4) * inv_pool;
}

}  // namespace frag16
}  // namespace rkv

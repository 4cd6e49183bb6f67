// Pieces shared by the kernels that stream 128-row bf16 key tiles through an
// LDS ring with direct global->LDS loads (k2_wide.hip, k2_long.hip): waits on
// the vector-memory counter that complete one tile without draining the
// ring, and the importance of a lane's key from MFMA fragments.
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
namespace stream {

constexpr int kNch = 8;              // 16-byte chunks per half row (bf16)
constexpr int kLoadsPerTile = 4;     // per wave: 4 x 1 KiB of a 32 KiB tile

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int vm_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Wait until every tile issued up to the one a step needs has landed:
// `tiles_after` tiles were issued after it, each as kPer loads per wave.
// Other memory operations issued meanwhile only make the wait longer.
template <int kPer = kLoadsPerTile>
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  static_assert(3 * kPer <= 63, "vmcnt holds 6 bits");
  if (tiles_after <= 0)
    __builtin_amdgcn_s_waitcnt(vm_imm(0));
  else if (tiles_after == 1)
    __builtin_amdgcn_s_waitcnt(vm_imm(kPer));
  else if (tiles_after == 2)
    __builtin_amdgcn_s_waitcnt(vm_imm(2 * kPer));
  else
    __builtin_amdgcn_s_waitcnt(vm_imm(3 * kPer));
}

// Importance of one key per lane from the lane's key fragments (both halves
// of the wave hold the same key). Query rows are padded per head to
// 2^rpg_shift rows; padding rows have zero queries and zero 1/sum.
template <int NQB>
__device__ __forceinline__ float key_importance(const char* qlds, const u32x2_t* slds,
                                                const u32x4_t (&kf)[kNch], int key, int n_u,
                                                int W, int G, int rpg_shift, bool causal,
                                                bool mean, int lane) {
  const int rpg_mask = (1 << rpg_shift) - 1;
  const int octets_per_group = (1 << rpg_shift) >> 3;
  const float inv_w = 1.0f / (float)W;
  asm volatile("" : "+v"(lane));   // per call: keeps lane-derived values out of the callers' loops
  const int half = lane >> 5;
  float best = 0.f, run = 0.f;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    u32x4_t qf[kNch];
    {
      const int m = qb * 32 + (lane & 31);
      const int g = m >> rpg_shift, r = m & rpg_mask;
      const bool qok = g < G && r < W;
      const int n = qok ? g * W + r : 0;
#pragma unroll
      for (int c = 0; c < kNch; ++c)
        qf[c] = qok ? ld16(qlds + frag_offset<bf16_bits>(n, half * kNch + c)) : zero16();
    }
    f32x16_t acc = {};
#pragma unroll
    for (int c = 0; c < kNch; ++c) mma_chunk<bf16_bits>(acc, qf[c], kf[c]);   // C[query][key]
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float os = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = 4 * t + j;
        const int m = qb * 32 + acc_row(v, lane);
        const u32x2_t st = slds[m];   // (max, 1/sum) as bits
        const float pr =
            fast_exp2(acc[v] * kLogitScaleLog2 - __uint_as_float(st.x)) * __uint_as_float(st.y);
        const float vis = (!causal || key <= n_u - W + (m & rpg_mask)) ? 1.f : 0.f;
        os = fmaf(pr, vis, os);
      }
      os += __shfl_xor(os, 32, 64);
      run += os;
      const int o = qb * 4 + t;
      if (((o + 1) & (octets_per_group - 1)) == 0) {
        if (o / octets_per_group < G) best = mean ? best + run * inv_w : fmaxf(best, run * inv_w);
        run = 0.f;
      }
    }
  }
  return mean ? best / (float)G : best;
}

}  // namespace stream
}  // namespace rkv

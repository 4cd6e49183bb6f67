// Importance I: softmax attention of the window queries over the candidates,
// mean over the w queries of each query head, max over the G heads of the
// GQA group.
//
// Pages: importance is derived from attention weights (sourcepulse summary
// of R-KV, "How It Works"; "R-KV: Redundancy-aware KV Cache Compression for
// Reasoning Models", atlas.scime.ai summary, "Approach"), and GQA attention
// is pooled by max, mean pooling being the weaker ablation (same summary,
// "Measured effects reported in the paper", last row). Window query r sees
// candidates j <= N-w+r; logits are q.k/sqrt(128). Variants: without the
// causal window every query sees all N candidates; mean instead of max over
// the GQA heads (the pooling ablation of the same section).
//
// This file holds the first two launches; the weights themselves are formed
// in the redundancy kernel (k2_redundancy.hip), which already holds every key
// row in registers as MFMA fragments:
//   k1_stats     per (unit, 256-key chunk): logits on MFMA with the keys as
//                the A operand, so each lane owns one query column and its
//                running max / sum of exp stay in registers; also writes
//                1/||k|| for every key, and for paged bf16 units copies the
//                keys to contiguous rows for the long-unit kernel. bf16 key
//                rows reach LDS by direct loads of whole rows per
//                instruction; fragments and the copy read them from there
//                (loads of one row per lane touch 64 cache lines per
//                instruction, 16 bytes of each).
//   k1_combine   per unit: merges the chunks' (max, sum) per query row into
//                (max, 1/sum).
// A query row's normaliser needs every key before any weight can be formed,
// hence the separate statistics pass over the keys.
//
// Query rows are laid out in groups of `rpg` rows (8, 16 or 32 >= w) per
// query head: MFMA row m is query head m / rpg, window query m % rpg; rows
// with m % rpg >= w or m / rpg >= G are padding and never contribute.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"

namespace rkv {

// 16 bytes from global memory into LDS with the streaming (non-temporal)
// cache policy: the statistics pass reads each key row once.
__device__ __forceinline__ void load16_to_lds_stream(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_dst), 16, 0,
                                   kCachePolicyStream);
}

// Load the lane's half (64 elements) of a 128-element row, or zeros.
template <typename T>
__device__ __forceinline__ void load_half_row(u32x4_t (&f)[Elem<T>::kHalfChunks], const T* row,
                                              int half, bool valid) {
  constexpr int NCH = Elem<T>::kHalfChunks;
  const char* p = reinterpret_cast<const char*>(row) + half * (NCH * 16);
#pragma unroll
  for (int c = 0; c < NCH; ++c) f[c] = valid ? ld16(p + 16 * c) : zero16();
}

template <typename T, int NQB, class P>
__device__ __forceinline__ void load_queries(u32x4_t (&qf)[NQB][Elem<T>::kHalfChunks], const P& p,
                                             int u, int lane, int rpg_shift) {
  const int half = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int m = qb * 32 + (lane & 31);
    const int g = m >> rpg_shift;
    const int r = m & ((1 << rpg_shift) - 1);
    const bool valid = g < p.G && r < p.W;
    const T* row = p.q(u) + (valid ? (int64_t)(g * p.W + r) * kD : 0);
    load_half_row<T>(qf[qb], row, half, valid);
  }
}

template <typename T, int NQB, class P>
__global__ __launch_bounds__(256) void k1_stats_kernel(P p, float* __restrict__ part,
                                                       float* __restrict__ rinv, int rpg_shift) {
  constexpr int NCH = Elem<T>::kHalfChunks;
  int u, chunk;
  if (!p.k1_item(blockIdx.x, u, chunk)) return;
  const int N = p.n(u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int rpg_mask = (1 << rpg_shift) - 1;

  u32x4_t qf[NQB][NCH];
  load_queries<T, NQB>(qf, p, u, lane, rpg_shift);

  float mloc[NQB], sloc[NQB];
  float lg[2][NQB][16];
  // bf16: the wave's 64 key rows come into LDS by direct loads, 16 lanes per
  // row (whole rows per instruction), position q of row r holding chunk
  // q ^ (r & 15); fragments and the paged key copy read them from there
  __shared__ __attribute__((aligned(16))) char kst[sizeof(T) == 2 ? 4 * 64 * 256 : 16];
  char* const ws = kst + (sizeof(T) == 2 ? wave * 64 * 256 : 0);
  const int rbase = chunk * kK1Keys + wave * 64;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = 4 * i + (lane >> 4);
      const int key = min(rbase + rr, N - 1);   // rows past N repeat row N-1
      load16_to_lds_stream(reinterpret_cast<const char*>(p.krow(u, key)) + (((lane & 15) ^ (rr & 15)) << 4),
                    ws + i * 1024);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's rows are in
    // paged units scored by the long-unit kernel: their keys to contiguous
    // rows, a whole row per 16 lanes, as streaming stores (the copy is far
    // larger than the caches; the long-unit kernel reads it back later)
    if (p.copy_dst(u, 0) != nullptr) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = 4 * i + (lane >> 4);
        const int key = rbase + rr;
        if (key < N)
          __builtin_nontemporal_store(
              ld16(ws + i * 1024 + lane * 16),
              reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(p.copy_dst(u, key)) +
                                         (((lane & 15) ^ (rr & 15)) << 4)));
      }
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kbase = rbase + kb * 32;
    const int key = kbase + (lane & 31);
    const bool kvalid = key < N;
    u32x4_t kf[NCH];
    if constexpr (sizeof(T) == 2) {
      const int rr = kb * 32 + (lane & 31);
#pragma unroll
      for (int c = 0; c < NCH; ++c) kf[c] = kvalid ? ld16(ws + frag_offset<T>(rr, half * NCH + c)) : zero16();
    } else {
      load_half_row<T>(kf, kvalid ? p.krow(u, key) : p.krow(u, 0), half, kvalid);
      // paged units scored by the long-unit kernel: their keys to contiguous rows
      if (kvalid) {
        T* dst = p.copy_dst(u, key);
        if (dst != nullptr) {
#pragma unroll
          for (int c = 0; c < NCH; ++c) st16(reinterpret_cast<char*>(dst) + half * (NCH * 16) + 16 * c, kf[c]);
        }
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) ss += sumsq_chunk<T>(kf[c]);
    ss += __shfl_xor(ss, 32, 64);
    if (half == 0 && kvalid) rinv[p.score_off(u) + key] = ss > 0.f ? __frsqrt_rn(ss) : 0.f;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x16_t acc = {};
#pragma unroll
      for (int c = 0; c < NCH; ++c) mma_chunk<T>(acc, kf[c], qf[qb][c]);   // C[key][query]
      const int m = qb * 32 + (lane & 31);
      const int r = m & rpg_mask;
      const bool qvalid = (m >> rpg_shift) < p.G && r < p.W;
      // last key visible to window query r (all keys without the causal window)
      const int last = p.causal() ? N - p.W + r : N - 1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = kbase + acc_row(v, lane);
        lg[kb][qb][v] = (qvalid && kk <= last) ? acc[v] * kLogitScaleLog2 : -INFINITY;
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) m = fmaxf(m, lg[kb][qb][v]);
    float s = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += fast_exp2(lg[kb][qb][v] - m);
    }
    // merge with the other half (same query column, other keys)
    const float m2 = __shfl_xor(m, 32, 64);
    const float s2 = __shfl_xor(s, 32, 64);
    const float mm = fmaxf(m, m2);
    float st = 0.f;
    if (mm != -INFINITY) st = (m != -INFINITY ? s * fast_exp2(m - mm) : 0.f) +
                              (m2 != -INFINITY ? s2 * fast_exp2(m2 - mm) : 0.f);
    mloc[qb] = mm;
    sloc[qb] = st;
  }
  __shared__ float2 sm[4][NQB * 32];
  if (half == 0) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) sm[wave][qb * 32 + lane] = make_float2(mloc[qb], sloc[qb]);
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < NQB * 32) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sm[w][t].x);
    float st = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float2 e = sm[w][t];
        if (e.x != -INFINITY) st += e.y * fast_exp2(e.x - mm);
      }
    }
    reinterpret_cast<float2*>(part)[p.k1_slot(u, chunk) * (NQB * 32) + t] = make_float2(mm, st);
  }
}

// Per unit and query row: M = max over chunks, S = sum of the chunk sums
// rescaled to M. Writes (M, 1/S), or (0, 0) for a row that sees no key.
// Also clears the redundancy kernel's counters, if any: [8] item claims
// (by workgroup 0), then one arrival counter per scored unit.
template <int NQB, class P>
__global__ __launch_bounds__(128) void k1_combine_kernel(P p, const float* __restrict__ part,
                                                         float* __restrict__ fin, int num_units,
                                                         int32_t* __restrict__ counters) {
  const int u = blockIdx.x;
  const int t = threadIdx.x;
  if (counters != nullptr && u == 0 && t < 8) counters[t] = 0;
  if (u >= num_units || p.n(u) <= p.budget(u)) return;   // unscored unit
  if (counters != nullptr && t == 0) counters[8 + u] = 0;
  if (t >= NQB * 32) return;
  const int nc = p.k1_nchunks(u);
  const float2* pp = reinterpret_cast<const float2*>(part) + p.k1_slot(u, 0) * (NQB * 32) + t;
  float mm = -INFINITY;
  for (int c = 0; c < nc; ++c) mm = fmaxf(mm, pp[(int64_t)c * NQB * 32].x);
  float st = 0.f;
  if (mm != -INFINITY) {
    for (int c = 0; c < nc; ++c) {
      const float2 e = pp[(int64_t)c * NQB * 32];
      if (e.x != -INFINITY) st += e.y * fast_exp2(e.x - mm);
    }
  }
  const float2 out = (mm != -INFINITY && st > 0.f) ? make_float2(mm, 1.0f / st) : make_float2(0.f, 0.f);
  reinterpret_cast<float2*>(fin)[(int64_t)u * NQB * 32 + t] = out;
}

// ---------------------------------------------------------------------------
template <typename T, int NQB, class P>
static hipError_t run_k1_t(const P& p, int k1_items, int num_units, float* part, float* fin,
                           float* rinv, int32_t* counters, int rpg_shift, hipStream_t st) {
  hipError_t e = launch("rkv_k1_stats", k1_stats_kernel<T, NQB, P>, dim3(k1_items), dim3(256), 0, st,
                        p, part, rinv, rpg_shift);
  if (e != hipSuccess) return e;
  return launch("rkv_k1_combine", k1_combine_kernel<NQB, P>, dim3(num_units), dim3(128), 0, st, p,
                (const float*)part, fin, num_units, counters);
}

template <typename T, class P>
hipError_t run_k1(const P& p, int nqb, int k1_items, int num_units, float* part, float* fin,
                  float* rinv, int32_t* counters, int rpg_shift, hipStream_t st) {
  // fp32 inputs are limited to two query blocks on the host (register budget)
  if constexpr (sizeof(T) == 4) {
    if (nqb == 1) return run_k1_t<T, 1>(p, k1_items, num_units, part, fin, rinv, counters, rpg_shift, st);
    return run_k1_t<T, 2>(p, k1_items, num_units, part, fin, rinv, counters, rpg_shift, st);
  } else {
    switch (nqb) {
      case 1: return run_k1_t<T, 1>(p, k1_items, num_units, part, fin, rinv, counters, rpg_shift, st);
      case 2: return run_k1_t<T, 2>(p, k1_items, num_units, part, fin, rinv, counters, rpg_shift, st);
      case 3: return run_k1_t<T, 3>(p, k1_items, num_units, part, fin, rinv, counters, rpg_shift, st);
      default: return run_k1_t<T, 4>(p, k1_items, num_units, part, fin, rinv, counters, rpg_shift, st);
    }
  }
}

template hipError_t run_k1<bf16_bits, DenseProblem<bf16_bits>>(const DenseProblem<bf16_bits>&, int, int, int, float*, float*, float*, int32_t*, int, hipStream_t);
template hipError_t run_k1<float, DenseProblem<float>>(const DenseProblem<float>&, int, int, int, float*, float*, float*, int32_t*, int, hipStream_t);
template hipError_t run_k1<bf16_bits, PagedProblem<bf16_bits>>(const PagedProblem<bf16_bits>&, int, int, int, float*, float*, float*, int32_t*, int, hipStream_t);
template hipError_t run_k1<float, PagedProblem<float>>(const PagedProblem<float>&, int, int, int, float*, float*, float*, int32_t*, int, hipStream_t);

}  // namespace rkv

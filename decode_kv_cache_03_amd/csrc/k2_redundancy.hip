// Redundancy R, importance I and joint score Z, one pass over the keys.
//
// Pages: redundancy is measured by the cosine similarity of key vectors and
// serves to find and prune near-duplicates (sourcepulse summary of R-KV,
// "How It Works"; "R-KV: Redundancy-aware KV Cache Compression for Reasoning
// Models", atlas.scime.ai summary, "Approach"); what is removed is the
// duplicate of something already in the cache ("R-KV: decoding-time KV cache
// compression for reasoning models", hysenlabs page, "How this differs from
// attention-sink and heavy-hitter eviction"). Reading used here:
// R_i = max over earlier candidates j < i of cos(k_i, k_j), R_0 = 0.
// Importance is the window queries' softmax attention, mean over a head's
// queries, max over the GQA group (atlas.scime.ai summary, "Approach" and
// "Measured effects reported in the paper"). The joint score is
// Z = lambda*I - (1-lambda)*R (same summary, "Approach").
//
// The cosine matrix is the one dense contraction of the step (N x N x 128
// per unit), so it runs on bf16 MFMA with fp32 accumulation on the raw keys
// (bf16 products are exact in fp32); the norms 1/||k|| are applied in the
// fp32 epilogue, which keeps the cosine within fp32 rounding of exact.
// Nothing N x N is ever stored: each lane keeps running row maxima in
// registers.
//
// Work item = (unit, block of 128 rows). Column tiles of 128 keys are staged
// in LDS (double-buffered, XOR-swizzled 16-byte chunks so fragment reads hit
// distinct banks). The 4 waves form a 2x2 grid over each 128x128 step: wave
// (r, c) holds rows 64r..64r+63 of the block as MFMA A fragments in registers
// and multiplies them by columns 64c..64c+63 of the tile, as 2x2 tiles of
// 32x32x16 per k-step. The block's own (diagonal) tile comes first: it
// supplies the A fragments and is the only step that needs the j < i mask.
// Tiles 0..blk-1 lie wholly left of the diagonal and run unmasked.
//
// The grid is persistent: about two workgroups per CU walk the work items,
// workgroup w taking items w, w+G, w+2G, ... (G = grid size, a multiple of
// 8, so every item a workgroup takes maps to its own XCD, where all blocks of
// a unit are scheduled together and share the unit's keys in that XCD's L2).
// The tile stream never stops between items: during an item's last step the
// next item's diagonal tile and query rows are already being loaded, so the
// per-item start-up latency is hidden.
//
// Per item, after the A fragments are read, the block's keys are scored for
// importance: with the key rows as the B operand of Q x K^T each lane holds
// one key and 16 query rows, so the mean over a head's window queries and the
// max over heads reduce inside the lane (plus one exchange between the
// 32-lane halves), against the softmax normalisers merged beforehand.
// At the end of the item the row maxima are reduced across lanes by a
// butterfly that halves the values per lane at each exchange, so no large
// LDS buffer competes with the tile buffers.
//
// The MFMA issue rate is the budget, so per-lane addresses are computed once:
// tiles arrive by direct global->LDS loads from a uniform base plus a fixed
// per-lane offset, and fragment reads use fixed per-lane LDS offsets.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"

namespace rkv {

template <typename T>
struct K2Cfg {
  static constexpr int NCH = Elem<T>::kHalfChunks;
  static constexpr int RC = Elem<T>::kRowChunks;
  static constexpr int RB = Elem<T>::kRowBytes;
  static constexpr int TILE_BYTES = kK2Cols * RB;
  static constexpr int LOADS = kK2Cols * RB / 1024 / 4;   // KiB of tile per wave
  static constexpr int ROWS_PER_KB = 1024 / RB;
};

// Byte offset, inside a tile, of the slot holding chunk `chunk` of tile row n:
// the slot at position pos holds global chunk pos ^ (n & 15) of the row.
template <typename T>
__device__ __forceinline__ int frag_offset(int n, int chunk) {
  return n * Elem<T>::kRowBytes + ((chunk ^ (n & 15)) << 4);
}

// One butterfly exchange of the row-max reduction: lanes whose bit W is set
// keep values W..2W-1 of the current range, the others keep 0..W-1; each
// receives the half it keeps from the partner lane l ^ W.
template <int W>
__device__ __forceinline__ void max_butterfly_step(float (&val)[32], int lane) {
  const bool upper = (lane & W) != 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const float keep = upper ? val[i + W] : val[i];
    const float send = upper ? val[i] : val[i + W];
    val[i] = fmaxf(keep, __shfl_xor(send, W, 64));
  }
}

template <typename T, int NQB, class P>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k2_redundancy_kernel(
    P p, int total_items, const float* __restrict__ rinv, const float* __restrict__ fin,
    float* __restrict__ Z, float* __restrict__ Rdbg, float* __restrict__ Idbg, float lam,
    int rpg_shift) {
  using C = K2Cfg<T>;
  constexpr int NCH = C::NCH;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int gw = p.G * p.W;
  const K2Lds plan = k2_lds_plan(C::RB, gw, NQB);
  char* const tiles = lds + plan.tiles;
  char* const qlds = lds + plan.q;
  float2* const slds = reinterpret_cast<float2*>(lds + plan.stats);
  float* const imp_l = reinterpret_cast<float*>(lds + plan.imp);
  float* const comb = reinterpret_cast<float*>(lds + plan.comb);

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;      // row group, column group of this wave
  const int stride = gridDim.x;
  const int rpg_mask = (1 << rpg_shift) - 1;
  const int octets_per_group = (1 << rpg_shift) >> 3;
  const float inv_w = 1.0f / (float)p.W;

  // next valid work item at or after k (in steps of the grid size)
  auto next_item = [&](int k, int& u, int& blk) -> int {
    for (; k < total_items; k += stride)
      if (p.k2_item(k, u, blk)) {
        u = __builtin_amdgcn_readfirstlane(u);
        blk = __builtin_amdgcn_readfirstlane(blk);
        return k;
      }
    return total_items;
  };

  // Per-lane tile-load offsets. Wave w fills KiB w*LOADS + i of a tile; lane
  // l of load i writes row ROWS_PER_KB*i + l/RC of the wave's rows at slot
  // l % RC, fetching chunk slot ^ (row & 15). Row & 15 repeats every
  // 16/ROWS_PER_KB loads, so a few offsets cover them all.
  constexpr int PER = 16 / C::ROWS_PER_KB;
  int lofs[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int r16 = (q * C::ROWS_PER_KB + lane / C::RC) & 15;   // (tile row) & 15 for load i = q mod PER
    lofs[q] = (lane / C::RC) * C::RB + (((lane % C::RC) ^ r16) << 4);
  }
  // Rows first_row.. of unit u into tile buffer buf; rows past the unit
  // (only in a diagonal tile) repeat its last row.
  auto tile_load = [&](int u, int n_u, int first_row, int buf, bool clamp) {
    char* dst = tiles + buf * C::TILE_BYTES + wave * C::LOADS * 1024;
    const int wrow = first_row + wave * C::LOADS * C::ROWS_PER_KB;   // first row this wave loads
    if constexpr (P::kRowsContiguous) {
      if (!clamp) {
        const char* src = reinterpret_cast<const char*>(p.krow(u, wrow));
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
          load16_to_lds(src + i * 1024 + lofs[i % PER], dst + i * 1024);
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int r = min(wrow + i * C::ROWS_PER_KB + lane / C::RC, n_u - 1);
      const int chunk_ofs = lofs[i % PER] - (lane / C::RC) * C::RB;
      load16_to_lds(reinterpret_cast<const char*>(p.krow(u, r)) + chunk_ofs, dst + i * 1024);
    }
  };
  // The unit's window queries (G*w rows, swizzled) and softmax normalisers.
  auto q_load = [&](int u) {
    const char* q = reinterpret_cast<const char*>(p.q(u));
    const int qkb = (gw * C::RB + 1023) / 1024;
    for (int kb = wave; kb < qkb; kb += 4) {
      const int n = kb * C::ROWS_PER_KB + lane / C::RC;
      const int c = (lane % C::RC) ^ (n & 15);
      const int nn = min(n, gw - 1);
      load16_to_lds(q + nn * C::RB + c * 16, qlds + kb * 1024);
    }
    if (wave == 0 && lane < NQB * 16)
      load16_to_lds(reinterpret_cast<const char*>(fin) + ((int64_t)u * NQB * 32 + 2 * lane) * 8,
                    reinterpret_cast<char*>(slds));
  };

  // Fragment read offsets: rows (A) wr*64 + rb*32 + l32, columns (B)
  // wc*64 + cb*32 + l32, chunk half*NCH + c. Adding 32 to a row leaves
  // (row & 15) unchanged, so the second 32 rows/columns sit 32*RB further.
  int boff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) boff[c] = frag_offset<T>(wc * 64 + l32, half * NCH + c);
  // rows and columns differ by a multiple of 64 rows, which keeps row & 15
  const int a_minus_b = (wr - wc) * 64 * C::RB;

  auto tile_mma = [&](const char* tb, const u32x4_t (&af)[2][NCH], f32x16_t (&acc)[2][2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x16_t{};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4_t b0 = ld16(tb + boff[c]);
      const u32x4_t b1 = ld16(tb + boff[c] + 32 * C::RB);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        mma_chunk<T>(acc[rb][0], af[rb][c], b0);
        mma_chunk<T>(acc[rb][1], af[rb][c], b1);
      }
    }
  };

  // Importance of one 32-key half of the wave's rows (key = row of kf).
  // Padding query rows (r >= w or g >= G) have zero queries and zero 1/sum,
  // so they add nothing; only keys among the last w need the causal test.
  auto importance_of = [&](const u32x4_t (&kf)[NCH], int key, int n_u, bool causal) -> float {
    float best = 0.f, run = 0.f;
    int lane_v = lane;   // re-materialised per item: keeps per-lane masks out of the loop preheader
    asm volatile("" : "+v"(lane_v));
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      u32x4_t qf[NCH];
      {
        const int m = qb * 32 + (lane_v & 31);
        const int g = m >> rpg_shift, r = m & rpg_mask;
        const bool qok = g < p.G && r < p.W;
        const int n = qok ? g * p.W + r : 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          qf[c] = qok ? ld16(qlds + frag_offset<T>(n, half * NCH + c)) : zero16();
      }
      f32x16_t acc = {};
#pragma unroll
      for (int c = 0; c < NCH; ++c) mma_chunk<T>(acc, qf[c], kf[c]);   // C[query][key]
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float os = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * t + j;
          const int m = qb * 32 + acc_row(v, lane_v);
          const float2 st = slds[m];
          const float pr = fast_exp2(acc[v] * kLogitScaleLog2 - st.x) * st.y;
          const float vis = (!causal || key <= n_u - p.W + (m & rpg_mask)) ? 1.f : 0.f;
          os = fmaf(pr, vis, os);   // arithmetic, not a branch around the exp
        }
        os += __shfl_xor(os, 32, 64);
        run += os;
        const int o = qb * 4 + t;
        if (((o + 1) & (octets_per_group - 1)) == 0) {
          if (o / octets_per_group < p.G) best = fmaxf(best, run * inv_w);
          run = 0.f;
        }
      }
    }
    return best;
  };

  int u, blk;
  int k = next_item(blockIdx.x, u, blk);
  if (k >= total_items) return;
  int N = p.n(u);
  tile_load(u, N, blk * kK2Rows, 0, true);
  q_load(u);
  int cur = 0;   // buffer holding the current tile

  while (true) {
    const int base = blk * kK2Rows;
    const int row0 = base + wr * 64;
    const bool wave_live = row0 < N;
    const int64_t so = p.score_off(u);
    int un = 0, bn = 0;
    const int kn = next_item(k + stride, un, bn);
    const bool has_next = kn < total_items;
    const int Nn = has_next ? p.n(un) : 0;

    // 1. the diagonal tile (and this unit's queries) have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    u32x4_t af[2][NCH];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        af[rb][c] = ld16(tiles + cur * C::TILE_BYTES + boff[c] + a_minus_b + rb * 32 * C::RB);

    // 2. importance of the block's keys; wave (r, c) takes keys r*64 + c*32 + l32
    if (wave_live) {
      const int key = row0 + wc * 32 + l32;
      const bool causal = base + kK2Rows > N - p.W;   // block reaches the window's keys
      const float best = (wc == 0) ? importance_of(af[0], key, N, causal)
                                   : importance_of(af[1], key, N, causal);
      if (half == 0) imp_l[wr * 64 + wc * 32 + l32] = best;
    }
    __syncthreads();   // queries are no longer read: the prefetch below may replace them

    // 3. prefetch: tile 0 of this block, or the next item's diagonal tile
    if (blk > 0) {
      tile_load(u, N, 0, cur ^ 1, false);
    } else if (has_next) {
      tile_load(un, Nn, bn * kK2Rows, cur ^ 1, true);
      q_load(un);
    }

    float mx[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx[rb][v] = -INFINITY;

    // 4. diagonal step: wave (0,1) lies above the diagonal, (1,0) below it;
    // (0,0) and (1,1) straddle it and mask per element (j < i)
    if (wave_live && wc <= wr) {
      f32x16_t acc[2][2];
      tile_mma(tiles + cur * C::TILE_BYTES, af, acc);
      float rc[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int col = base + wc * 64 + cb * 32 + l32;
        rc[cb] = col < N ? rinv[so + col] : 0.f;
      }
      if (wc < wr) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * rc[0], acc[rb][1][v] * rc[1]));
      } else {
        // rows and columns are the same 64 keys: row rb*32 + a follows column
        // cb*32 + b iff rb > cb, or rb == cb and a > b
        int lane_v = lane;   // re-materialised per item (see importance_of)
        asm volatile("" : "+v"(lane_v));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb <= rb; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const bool ok = (rb > cb) || (acc_row(v, lane_v) > (lane_v & 31));
              if (ok) mx[rb][v] = fmaxf(mx[rb][v], acc[rb][cb][v] * rc[cb]);
            }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    cur ^= 1;

    // 5. tiles 0..blk-1, wholly left of the diagonal; tile J is in buffer cur
    const float* rcol = rinv + so + wc * 64 + l32;
    for (int J = 0; J < blk; ++J) {
      if (J + 1 < blk) {
        tile_load(u, N, (J + 1) * kK2Cols, cur ^ 1, false);
      } else if (has_next) {
        tile_load(un, Nn, bn * kK2Rows, cur ^ 1, true);
        q_load(un);
      }
      if (wave_live) {
        f32x16_t acc[2][2];
        tile_mma(tiles + cur * C::TILE_BYTES, af, acc);
        const float r0 = rcol[J * kK2Cols], r1 = rcol[J * kK2Cols + 32];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * r0, acc[rb][1][v] * r1));
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      cur ^= 1;
    }

    // 6. row maxima. Value j = rb*16 + v of a lane belongs to row
    // rb*32 + acc_row(v, lane); the 32 lanes of a half share rows. A butterfly
    // over lane bits 4..0 keeps half of the remaining values at each exchange,
    // so lane l ends with the max over its half for value j = l & 31.
    float val[32];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) val[rb * 16 + v] = mx[rb][v];
    max_butterfly_step<16>(val, lane);
    max_butterfly_step<8>(val, lane);
    max_butterfly_step<4>(val, lane);
    max_butterfly_step<2>(val, lane);
    max_butterfly_step<1>(val, lane);
    if (wave_live) {
      const int rl = wr * 64 + (l32 >> 4) * 32 + acc_row(l32 & 15, lane);   // row within the block
      comb[wc * kK2Rows + rl] = val[0];
    }
    __syncthreads();

    // 7. R, I and Z for the block's rows
    if (tid < kK2Rows) {
      const int row = base + tid;
      if (row < N) {
        const float m = fmaxf(comb[tid], comb[kK2Rows + tid]);
        const float R = (row == 0) ? 0.f : m * rinv[so + row];
        const float I = imp_l[tid];
        const float z = lam * I - (1.0f - lam) * R;
        Z[so + row] = z + 0.0f;   // folds -0 onto +0
        if (Rdbg != nullptr) Rdbg[so + row] = R;
        if (Idbg != nullptr) Idbg[so + row] = I;
      }
    }

    if (!has_next) break;
    k = kn;
    u = un;
    blk = bn;
    N = Nn;
  }
}

template <typename T, int NQB, class P>
static hipError_t run_k2_t(const P& p, int k2_items, const float* rinv, const float* fin, float* Z,
                           float* dbg_R, float* dbg_I, float lam, int rpg_shift, hipStream_t st) {
  const K2Lds plan = k2_lds_plan(Elem<T>::kRowBytes, p.G * p.W, NQB);
  auto kern = k2_redundancy_kernel<T, NQB, P>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, plan.total);
  int dev = 0, cus = 0, per_cu = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, plan.total);
  if (e != hipSuccess) return e;
  int grid = 8 * ((max(1, per_cu) * cus + 7) / 8);
  grid = min(grid, 8 * ((k2_items + 7) / 8));
  return launch("rkv_k2_redundancy", kern, dim3(grid), dim3(256), plan.total, st, p, k2_items, rinv,
                fin, Z, dbg_R, dbg_I, lam, rpg_shift);
}

template <typename T, class P>
hipError_t run_k2(const P& p, int nqb, int k2_items, const float* rinv, const float* fin, float* Z,
                  float* dbg_R, float* dbg_I, float lam, int rpg_shift, hipStream_t st) {
  if constexpr (sizeof(T) == 4) {
    if (nqb == 1) return run_k2_t<T, 1>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, st);
    return run_k2_t<T, 2>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, st);
  } else {
    switch (nqb) {
      case 1: return run_k2_t<T, 1>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, st);
      case 2: return run_k2_t<T, 2>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, st);
      case 3: return run_k2_t<T, 3>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, st);
      default: return run_k2_t<T, 4>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, st);
    }
  }
}

template hipError_t run_k2<bf16_bits, DenseProblem<bf16_bits>>(const DenseProblem<bf16_bits>&, int, int, const float*, const float*, float*, float*, float*, float, int, hipStream_t);
template hipError_t run_k2<float, DenseProblem<float>>(const DenseProblem<float>&, int, int, const float*, const float*, float*, float*, float*, float, int, hipStream_t);
template hipError_t run_k2<bf16_bits, PagedProblem<bf16_bits>>(const PagedProblem<bf16_bits>&, int, int, const float*, const float*, float*, float*, float*, float, int, hipStream_t);
template hipError_t run_k2<float, PagedProblem<float>>(const PagedProblem<float>&, int, int, const float*, const float*, float*, float*, float*, float, int, hipStream_t);

}  // namespace rkv

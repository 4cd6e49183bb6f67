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
// The joint score is Z = lambda*I - (1-lambda)*R (atlas.scime.ai summary,
// "Approach").
//
// The cosine matrix is the one dense contraction of the step (N x N x 128
// per unit), so it runs on bf16 MFMA with fp32 accumulation on the raw keys
// (bf16 products are exact in fp32); the norms 1/||k|| are applied in the
// fp32 epilogue, which keeps the cosine within fp32 rounding of exact.
// Nothing N x N is ever stored: each lane keeps running row maxima in
// registers.
//
// Work item = (unit, block of 128 rows); column tiles of 128 keys are staged
// in LDS (double-buffered, XOR-swizzled 16-byte chunks so fragment reads hit
// distinct banks). The 4 waves form a 2x2 grid over each 128x128 step: wave
// (r, c) holds rows 64r..64r+63 of the block as MFMA A fragments in registers
// for the whole item and multiplies them by columns 64c..64c+63 of the tile,
// as 2x2 tiles of 32x32x16 per k-step.
//
// The block's own tile (the diagonal one) is loaded first: it supplies the A
// fragments (read from LDS, so the rows are fetched once) and is the only
// step that needs the j < i mask; the wave above the diagonal idles on it.
// The remaining tiles 0..blk-1 lie wholly left of the diagonal and run
// unmasked. ~95% of wave-steps do useful work at N = 1152.
//
// After the tile loop the block's key rows, still in registers, are reused
// for the importance weights (Q x K^T against the softmax normalisers the
// statistics pass produced), so Z leaves the kernel without a second read of
// the keys.
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
  static constexpr int RED_STRIDE = 68;                   // floats per row of partial maxima
  static constexpr int RED_BYTES = kK2Rows * RED_STRIDE * 4 + kK2Rows * 4;   // + importance
  static constexpr int LDS_BYTES = (2 * TILE_BYTES > RED_BYTES) ? 2 * TILE_BYTES : RED_BYTES;
};

// Byte offset, inside a tile, of LDS chunk slot `pos` of tile row n: the slot
// holds global chunk pos ^ (n & 15) of that row.
template <typename T>
__device__ __forceinline__ int frag_offset(int n, int chunk) {
  return n * Elem<T>::kRowBytes + ((chunk ^ (n & 15)) << 4);
}

template <typename T, int NQB, class P>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k2_redundancy_kernel(
    P p, const float* __restrict__ rinv, const float* __restrict__ fin, float* __restrict__ Z,
    float* __restrict__ Rdbg, float* __restrict__ Idbg, float lam, int rpg_shift) {
  using C = K2Cfg<T>;
  constexpr int NCH = C::NCH;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];

  int u, blk;
  if (!p.k2_item(blockIdx.x, u, blk)) return;
  u = __builtin_amdgcn_readfirstlane(u);
  blk = __builtin_amdgcn_readfirstlane(blk);
  const int N = p.n(u);
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;      // row group, column group of this wave
  const int base = blk * kK2Rows;               // first row (and first column of the diagonal tile)
  const int row0 = base + wr * 64;
  const bool wave_live = row0 < N;
  const int64_t so = p.score_off(u);

  // Per-lane tile-load offsets (bytes from the tile's first row) and LDS
  // destinations: wave w fills KiB w*LOADS .. w*LOADS+LOADS-1 of the tile.
  int trow[C::LOADS], tcol[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int kb = wave * C::LOADS + i;
    trow[i] = kb * C::ROWS_PER_KB + lane / C::RC;
    tcol[i] = ((lane % C::RC) ^ (trow[i] & 15)) << 4;
  }
  auto tile_load = [&](int first_row, int buf, bool clamp) {
    char* dst = lds + buf * C::TILE_BYTES + wave * C::LOADS * 1024;
    if constexpr (P::kRowsContiguous) {
      if (!clamp) {
        const char* src = reinterpret_cast<const char*>(p.krow(u, first_row));
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
          load16_to_lds(src + trow[i] * C::RB + tcol[i], dst + i * 1024);
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int r = min(first_row + trow[i], N - 1);
      load16_to_lds(reinterpret_cast<const char*>(p.krow(u, r)) + tcol[i], dst + i * 1024);
    }
  };

  // Fragment read offsets: rows (A) wr*64 + rb*32 + l32, columns (B)
  // wc*64 + cb*32 + l32, chunk half*NCH + c. Adding 32 to a row leaves
  // (row & 15) unchanged, so the second 32 rows/columns sit 32*RB further.
  int aoff[NCH], boff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    aoff[c] = frag_offset<T>(wr * 64 + l32, half * NCH + c);
    boff[c] = frag_offset<T>(wc * 64 + l32, half * NCH + c);
  }

  // 1. the block's own tile -> LDS buffer 0, A fragments from it
  tile_load(base, 0, true);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  u32x4_t af[2][NCH];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c) af[rb][c] = ld16(lds + aoff[c] + rb * 32 * C::RB);
  if (blk > 0) tile_load(0, 1, false);          // prefetch tile 0

  float mx[2][16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx[rb][v] = -INFINITY;

  auto tile_mma = [&](const char* tb, f32x16_t (&acc)[2][2]) {
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

  // 2. diagonal step (masked): columns base + wc*64 + cb*32 + l32
  if (wave_live && wc <= wr) {
    f32x16_t acc[2][2];
    tile_mma(lds, acc);
    float rc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int col = base + wc * 64 + cb * 32 + l32;
      rc[cb] = col < N ? rinv[so + col] : 0.f;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int j = base + wc * 64 + cb * 32 + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = row0 + rb * 32 + acc_row(v, lane);
          if (j < i) mx[rb][v] = fmaxf(mx[rb][v], acc[rb][cb][v] * rc[cb]);
        }
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 3. tiles 0..blk-1, wholly left of the diagonal; tile J sits in buffer (J+1)&1
  const float* rcol = rinv + so + wc * 64 + l32;
  for (int J = 0; J < blk; ++J) {
    if (J + 1 < blk) tile_load((J + 1) * kK2Cols, J & 1, false);
    if (wave_live) {
      f32x16_t acc[2][2];
      tile_mma(lds + ((J + 1) & 1) * C::TILE_BYTES, acc);
      const float r0 = rcol[J * kK2Cols], r1 = rcol[J * kK2Cols + 32];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * r0, acc[rb][1][v] * r1));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // 4. row maxima: the 32 lanes of a half and the two column-group waves hold
  // 64 partial maxima per row; they meet in LDS (row-major, padded rows).
  float* red = reinterpret_cast<float*>(lds);
  float* imp_l = red + kK2Rows * C::RED_STRIDE;   // importance of the block's keys
  if (wave_live) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        red[(wr * 64 + rb * 32 + acc_row(v, lane)) * C::RED_STRIDE + wc * 32 + l32] = mx[rb][v];
  }

  // 5. importance of the block's keys. The key rows are already in registers
  // as A fragments; used as the B operand of Q x K^T they give one key per
  // lane and 16 query rows per register set, so the mean over each head's
  // window queries and the max over the G heads reduce inside the lane plus
  // one exchange between the 32-lane halves. Query rows come in groups of
  // 2^rpg_shift (>= w) per head; the normalisers (max, 1/sum) were merged
  // over all keys beforehand. The two waves of a row group split its two
  // 32-key halves.
  if (wave_live) {
    const int rpg_mask = (1 << rpg_shift) - 1;
    const int octets_per_group = (1 << rpg_shift) >> 3;
    const float inv_w = 1.0f / (float)p.W;
    const int key = row0 + wc * 32 + l32;
    const T* qrow0 = p.q(u);
    const float2* fp = reinterpret_cast<const float2*>(fin) + (int64_t)u * NQB * 32;
    // the key fragments are taken by compile-time index (a runtime index
    // would move the register array to scratch memory)
    auto importance_of = [&](const u32x4_t (&kf)[NCH]) -> float {
      float best = 0.f, run = 0.f;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        u32x4_t qf[NCH];
        {
          const int m = qb * 32 + l32;
          const bool qok = (m >> rpg_shift) < p.G && (m & rpg_mask) < p.W;
          const char* q = reinterpret_cast<const char*>(
                              qrow0 + (qok ? (int64_t)((m >> rpg_shift) * p.W + (m & rpg_mask)) * kD : 0)) +
                          half * (NCH * 16);
#pragma unroll
          for (int c = 0; c < NCH; ++c) qf[c] = qok ? ld16(q + 16 * c) : zero16();
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
            const int m = qb * 32 + acc_row(v, lane);
            const float2 st = fp[m];
            const bool vis = (m >> rpg_shift) < p.G && (m & rpg_mask) < p.W &&
                             key <= N - p.W + (m & rpg_mask);
            const float pr = fast_exp2(acc[v] * kLogitScaleLog2 - st.x) * st.y;
            os += vis ? pr : 0.f;
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
    const float best = (wc == 0) ? importance_of(af[0]) : importance_of(af[1]);
    if (half == 0) imp_l[wr * 64 + wc * 32 + l32] = best;
  }
  __syncthreads();

  // 6. R, I and Z per row: two threads per row, 32 partial maxima each
  const int rl = tid >> 1;
  const float4* pr = reinterpret_cast<const float4*>(red + rl * C::RED_STRIDE + (tid & 1) * 32);
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 q = pr[k];
    m = fmaxf(m, fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w)));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  const int row = base + rl;
  if ((tid & 1) == 0 && row < N) {
    const float R = (row == 0) ? 0.f : m * rinv[so + row];
    const float I = imp_l[rl];
    const float z = lam * I - (1.0f - lam) * R;
    Z[so + row] = z + 0.0f;   // folds -0 onto +0
    if (Rdbg != nullptr) Rdbg[so + row] = R;
    if (Idbg != nullptr) Idbg[so + row] = I;
  }
}

template <typename T, int NQB, class P>
static hipError_t run_k2_t(const P& p, int k2_items, const float* rinv, const float* fin, float* Z,
                           float* dbg_R, float* dbg_I, float lam, int rpg_shift, hipStream_t st) {
  return launch("rkv_k2_redundancy", k2_redundancy_kernel<T, NQB, P>, dim3(k2_items), dim3(256), 0,
                st, p, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift);
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

// Redundancy R and joint score Z.
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
// Work item = (unit, block of 256 rows). The block's 4 waves own 64 rows
// each, held as MFMA A fragments in registers for the whole item. Column
// tiles of 64 keys are staged in LDS (double-buffered, XOR-swizzled 16-byte
// chunks so fragment reads hit distinct banks) and every wave multiplies its
// 64 rows by the tile: 2x2 tiles of 32x32x16 per k-step. Only tiles left of
// the diagonal are visited; tiles crossing it are masked per element.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"

namespace rkv {

template <typename T>
struct K2Cfg {
  static constexpr int NCH = Elem<T>::kHalfChunks;
  static constexpr int RC = Elem<T>::kRowChunks;
  static constexpr int RB = Elem<T>::kRowBytes;
  static constexpr int TILE_BYTES = kK2Cols * RB;
  static constexpr int LOADS = kK2Cols * RC / 256;
  static constexpr int RED_STRIDE = kK2Rows + 1;   // floats; odd stride avoids bank conflicts
  static constexpr int RED_BYTES = 32 * RED_STRIDE * 4;
  static constexpr int LDS_BYTES = (2 * TILE_BYTES > RED_BYTES) ? 2 * TILE_BYTES : RED_BYTES;
};

template <typename T, class P>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k2_redundancy_kernel(P p, const float* __restrict__ rinv,
                                                               const float* __restrict__ imp,
                                                               float* __restrict__ Z,
                                                               float* __restrict__ Rdbg, float lam) {
  using C = K2Cfg<T>;
  constexpr int NCH = C::NCH;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];

  int u, blk;
  if (!p.k2_item(blockIdx.x, u, blk)) return;
  const int N = p.n(u);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int row0 = blk * kK2Rows + wave * 64;
  const int blk_last = min(N, (blk + 1) * kK2Rows) - 1;
  const int ntile = (blk_last + kK2Cols - 1) / kK2Cols;
  const bool wave_live = row0 < N;
  const int wave_last = min(row0 + 63, N - 1);
  const int64_t so = p.score_off(u);

  u32x4_t af[2][NCH];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = row0 + rb * 32 + (lane & 31);
    const bool ok = row < N;
    const char* src = reinterpret_cast<const char*>(p.krow(u, ok ? row : 0)) + half * (NCH * 16);
#pragma unroll
    for (int c = 0; c < NCH; ++c) af[rb][c] = ok ? ld16(src + 16 * c) : zero16();
  }

  float mx[2][16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx[rb][v] = -INFINITY;

  u32x4_t stage[C::LOADS];
  auto gload = [&](int J) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int q = i * 256 + tid;
      const int n = q / C::RC, c = q % C::RC;
      const int col = J * kK2Cols + n;
      stage[i] = col < N ? ld16(reinterpret_cast<const char*>(p.krow(u, col)) + 16 * c) : zero16();
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int q = i * 256 + tid;
      const int n = q / C::RC, c = q % C::RC;
      st16(lds + buf * C::TILE_BYTES + n * C::RB + ((c ^ (n & 15)) << 4), stage[i]);
    }
  };

  if (ntile > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int J = 0; J < ntile; ++J) {
    if (J + 1 < ntile) gload(J + 1);
    const int col0 = J * kK2Cols;
    if (wave_live && wave_last > col0) {
      const char* tb = lds + (J & 1) * C::TILE_BYTES;
      float rc[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int col = col0 + cb * 32 + (lane & 31);
        rc[cb] = col < N ? rinv[so + col] : 0.f;
      }
      f32x16_t acc[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x16_t{};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        u32x4_t bfr[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int n = cb * 32 + (lane & 31);
          const int cc = half * NCH + c;
          bfr[cb] = ld16(tb + n * C::RB + ((cc ^ (n & 15)) << 4));
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) mma_chunk<T>(acc[rb][cb], af[rb][c], bfr[cb]);
      }
      if (col0 + kK2Cols - 1 < row0) {
        // every column precedes every row of this wave
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * rc[0], acc[rb][1][v] * rc[1]));
      } else {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const int j = col0 + cb * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int i = row0 + rb * 32 + acc_row(v, lane);
              if (j < i) mx[rb][v] = fmaxf(mx[rb][v], acc[rb][cb][v] * rc[cb]);
            }
          }
      }
    }
    if (J + 1 < ntile) sstore((J + 1) & 1);
    __syncthreads();
  }

  // Row maxima: lanes of a half hold the same rows for different columns.
  float* red = reinterpret_cast<float*>(lds);
  if (wave_live) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        red[(lane & 31) * C::RED_STRIDE + wave * 64 + rb * 32 + acc_row(v, lane)] = mx[rb][v];
  }
  __syncthreads();
  const int row = blk * kK2Rows + tid;
  if (row < N) {
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < 32; ++c) m = fmaxf(m, red[c * C::RED_STRIDE + tid]);
    const float R = (row == 0) ? 0.f : m * rinv[so + row];
    const float z = lam * imp[so + row] - (1.0f - lam) * R;
    Z[so + row] = z + 0.0f;   // folds -0 onto +0
    if (Rdbg != nullptr) Rdbg[so + row] = R;
  }
}

template <typename T, class P>
hipError_t run_k2(const P& p, int k2_items, const float* rinv, const float* imp, float* Z,
                  float* dbg_R, float lam, hipStream_t st) {
  return launch("rkv_k2_redundancy", k2_redundancy_kernel<T, P>, dim3(k2_items), dim3(256), 0, st,
                p, rinv, imp, Z, dbg_R, lam);
}

template hipError_t run_k2<bf16_bits, DenseProblem<bf16_bits>>(const DenseProblem<bf16_bits>&, int, const float*, const float*, float*, float*, float, hipStream_t);
template hipError_t run_k2<float, DenseProblem<float>>(const DenseProblem<float>&, int, const float*, const float*, float*, float*, float, hipStream_t);
template hipError_t run_k2<bf16_bits, PagedProblem<bf16_bits>>(const PagedProblem<bf16_bits>&, int, const float*, const float*, float*, float*, float, hipStream_t);
template hipError_t run_k2<float, PagedProblem<float>>(const PagedProblem<float>&, int, const float*, const float*, float*, float*, float, hipStream_t);

}  // namespace rkv

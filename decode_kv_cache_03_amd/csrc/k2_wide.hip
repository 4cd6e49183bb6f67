// Dense bf16 caches: the whole compression step of a unit in one 8-wave
// workgroup (statistics, redundancy, importance, joint score, selection and
// gather), persistent over units, one workgroup per CU.
//
// Same arithmetic as k1_importance.hip and k2_redundancy.hip (pages and
// readings cited there): softmax of the window queries over the unit's keys
// (query r sees keys j <= N-w+r), mean over a head's w queries, max over the
// GQA group; R_i = max_{j<i} cos(k_i, k_j) on bf16 MFMA with fp32
// accumulation and the norms applied in the epilogue; Z = lambda*I -
// (1-lambda)*R; the window plus the top B-w by (Z desc, index asc), ascending;
// the kept K/V rows gathered.
//
// Shape, chosen so that tiles stream without stalls:
//  * the unit's key tiles (128 rows each) stream through a ring of S = 4
//    (or 3, 2) LDS slots filled by direct global->LDS loads; S - 1 tiles are
//    in flight while one is consumed, and a step waits only for its own tile
//    (s_waitcnt vmcnt counts the loads issued after it). The stream runs
//    across phases and units without draining: the next unit's first tiles
//    and its window queries are loaded while the current unit finishes;
//  * phase S streams the unit's tiles once: four waves form the logits of
//    their 32 keys against the window queries (keys as the MFMA A operand,
//    so each lane owns one query column and keeps a running max and sum of
//    exponentials), four waves form the 1/||k|| of their 32 rows; both land
//    in LDS for the whole unit;
//  * phase R streams blocks of 256 rows (two tiles; the first block is a
//    single tile when the tile count is odd). The 8 waves hold the block's
//    rows as MFMA A fragments in a 4x2 grid (rows 64r.., columns 64c.. of
//    each 128-column tile): the block's own tile(s) first, masked j < i where
//    a wave's rows meet its columns, then tiles 0..t0-1 unmasked. The block's
//    keys are scored for importance from the same fragments;
//  * Z stays in LDS; the selection runs on it, and the gather reads the kept
//    indices from LDS.
// Variants: for the symmetric R (a separate instantiation) every block also
// sweeps the tiles right of it and masks only j == i on its diagonal and
// columns past N in the last tile; without the causal window the statistics
// and weights mask only padding keys; mean pooling sums the heads' window
// means and divides by G. Under head-shared selection the kernel stops after
// writing Z (a later launch selects for each group of units and gathers).
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"
#include "rkv_stream.hpp"

namespace rkv {
namespace fused {

using stream::key_importance;
using stream::kLoadsPerTile;
using stream::kNch;
using stream::wait_tiles;

constexpr int kThreads = 512;
constexpr int kRowBytes = 256;                  // bf16 row of 128
constexpr int kTileBytes = 128 * kRowBytes;

// Row block i (0..ni-1) of a unit with nb = ceil(N/128) tiles: first tile t0,
// nt tiles. Blocks are laid from the end, so only block 0 can be a single
// tile. A block streams its own tile(s) first, then the `ext` other tiles:
// 0..t0-1, and for the symmetric R also t0+nt..nb-1.
struct Block {
  int t0, nt, ext;
  __device__ int len() const { return nt + ext; }
  __device__ int tile(int k) const {
    return k < nt ? t0 + k : (k - nt < t0 ? k - nt : k);
  }
};
__device__ __forceinline__ Block block_of(int i, bool odd, int nb, bool sym) {
  Block b;
  if (odd) {
    b.t0 = i == 0 ? 0 : 2 * i - 1;
    b.nt = i == 0 ? 1 : 2;
  } else {
    b.t0 = 2 * i;
    b.nt = 2;
  }
  b.ext = sym ? nb - b.nt : b.t0;
  return b;
}

// Position in a unit's tile stream: phase 0 = statistics (tile k), phase 1
// = block `blk`, position k.
struct StreamPos {
  int u, par, phase, blk, k;
};

template <int NQB, bool kSym>
__global__ __launch_bounds__(kThreads, 1) void k2f_kernel(
    DenseProblem<bf16_bits> p, float* __restrict__ Zdbg, float* __restrict__ Rdbg,
    float* __restrict__ Idbg, float lam, int rpg_shift, int32_t* __restrict__ kept_all,
    bf16_bits* __restrict__ K_out, bf16_bits* __restrict__ V_out, int64_t out_stride,
    int score_only, FusedPlan L) {
  using T = bf16_bits;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int S = L.slots;
  const int N = p.N, W = p.W, G = p.G, gw = G * W, B = p.B;
  const int nb = (N + 127) / 128;
  const int ni = (nb + 1) / 2;
  const bool odd = (nb & 1) != 0;
  constexpr bool sym = kSym;   // symmetric R: every block sweeps every column tile
  // keys past lim_s are masked in the statistics: padding rows past N, and
  // keys that a window query cannot see
  const bool causal = p.causal();
  const int rpg_mask = (1 << rpg_shift) - 1;
  u32x2_t* const stats = reinterpret_cast<u32x2_t*>(lds + L.stats);   // (max, 1/sum) bits
  // per-wave max and sum partials, [4][NQB*32] each, as separate 32-bit
  // arrays: 64-bit LDS accesses of them make the compiler wait for every
  // direct global->LDS load in flight
  float* const sred_m = reinterpret_cast<float*>(lds + L.sred);
  float* const sred_s = sred_m + 4 * NQB * 32;
  float* const rn = reinterpret_cast<float*>(lds + L.rn);              // [N] 1/||k||
  float* const zs = reinterpret_cast<float*>(lds + L.zs);              // [N] Z
  int32_t* const ks = reinterpret_cast<int32_t*>(lds + L.ks);          // [B] kept
  float* const imp_l = reinterpret_cast<float*>(lds + L.imp);          // [256]
  float* const comb = reinterpret_cast<float*>(lds + L.comb);          // [2][256]
  SelectScratch& ssh = *reinterpret_cast<SelectScratch*>(lds + L.sel);

  // Tile load q (0..3) of wave w fills KiB 4w + q of a slot: tile row
  // 16w + 4q + lane/16 at chunk position lane % 16, fetching chunk
  // (lane % 16) ^ (row & 15) of that row.
  int lofs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r16 = (4 * q + lane / 16) & 15;
    lofs[q] = (lane / 16) * kRowBytes + (((lane % 16) ^ r16) << 4);
  }
  int boff[kNch];   // B fragments: tile rows 64*wc + l32 (+32), chunk half*8 + c
#pragma unroll
  for (int c = 0; c < kNch; ++c) boff[c] = frag_offset<T>(wc * 64 + l32, half * kNch + c);

  // ---- loader: the tile stream of this workgroup's units, into the ring ----
  StreamPos ld{(int)blockIdx.x, 0, 0, 0, 0};
  int issued = 0, issue_slot = 0;
  // The loader runs at most one unit ahead of the consumer: the window
  // queries of two units share the two query slots.
  int ld_limit = blockIdx.x + 2 * gridDim.x;
  auto issue_next = [&]() -> bool {
    if (ld.u >= p.num_units || ld.u >= ld_limit) return false;
    int lane_v = lane;   // per call: keeps lane-derived values out of the callers' loops
    asm volatile("" : "+v"(lane_v));
    int t;
    if (ld.phase == 0) {
      if (ld.k == 0) {   // the unit's window queries, ahead of its first tile
        const char* q = reinterpret_cast<const char*>(p.q(ld.u));
        const int qkb = L.qbytes / 1024;
        char* qdst = lds + L.q + ld.par * L.qbytes;
        for (int kb = wave; kb < qkb; kb += 8) {
          const int n = kb * 4 + lane_v / 16;
          const int c = (lane_v % 16) ^ (n & 15);
          load16_to_lds(q + min(n, gw - 1) * kRowBytes + c * 16, qdst + kb * 1024);
        }
      }
      t = ld.k;
    } else {
      t = block_of(ld.blk, odd, nb, sym).tile(ld.k);
    }
    char* slot = lds + issue_slot * kTileBytes;
    const int row0 = t * 128 + wave * 16;   // first tile row this wave loads
    if ((t + 1) * 128 <= N) {
      const char* src = reinterpret_cast<const char*>(p.krow(ld.u, row0));
#pragma unroll
      for (int q = 0; q < 4; ++q) load16_to_lds(src + q * 1024 + lofs[q], slot + wave * 4096 + q * 1024);
    } else {   // last tile of the unit: rows past N repeat row N-1
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = min(row0 + 4 * q + lane_v / 16, N - 1);
        const int chunk_ofs = lofs[q] - (lane_v / 16) * kRowBytes;
        load16_to_lds(reinterpret_cast<const char*>(p.krow(ld.u, r)) + chunk_ofs,
                      slot + wave * 4096 + q * 1024);
      }
    }
    ++issued;
    issue_slot = issue_slot + 1 == S ? 0 : issue_slot + 1;
    // advance
    if (ld.phase == 0) {
      if (++ld.k == nb) {
        ld.phase = 1;
        ld.blk = 0;
        ld.k = 0;
      }
    } else if (++ld.k == block_of(ld.blk, odd, nb, sym).len()) {
      ld.k = 0;
      if (++ld.blk == ni) {
        ld.u += gridDim.x;
        ld.par ^= 1;
        ld.phase = 0;
        ld.blk = 0;
      }
    }
    return true;
  };
  auto refill = [&](int c) {
    while (issued - c < S && issue_next()) {
    }
  };
  // Tiles c..c+m-1 are needed next. When the last refill could not issue all
  // of them (a short ring, or the loader held at a unit boundary), the slots
  // they go to were freed by steps that every wave has finished only after a
  // barrier: take one, then issue.
  auto ensure_issued = [&](int c, int m) {
    if (issued < c + m) {
      lds_barrier();
      refill(c);
    }
  };
  auto slot_ptr = [&](int s0, int d) -> char* {
    const int s = s0 + d >= S ? s0 + d - S : s0 + d;
    return lds + s * kTileBytes;
  };

  int c = 0, cons_slot = 0;   // tiles consumed, c % S
  refill(0);

  int par = 0;
  for (int u = blockIdx.x; u < p.num_units; u += gridDim.x, par ^= 1) {
    ld_limit = u + 2 * gridDim.x;
    const int64_t so = p.score_off(u);
    const char* qlds = lds + L.q + par * L.qbytes;

    // ---------------- phase S: softmax statistics and norms ----------------
    float mrun[NQB], srun[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      mrun[qb] = -INFINITY;
      srun[qb] = 0.f;
    }
    for (int t = 0; t < nb; ++t) {
      ensure_issued(c, 1);
      wait_tiles(issued - (c + 1));
      lds_barrier();
      refill(c);
      const char* tb = lds + cons_slot * kTileBytes;
      int lane_v = lane;   // re-materialised per tile (see key_importance)
      asm volatile("" : "+v"(lane_v));
      const int lh = lane_v >> 5, ll = lane_v & 31;
      if (wave < 4) {
        // logits of keys 32w + ll against the window queries; this lane owns
        // query column ll of each 32-row query block
        const int kl = wave * 32 + ll;
        u32x4_t kf[kNch];
#pragma unroll
        for (int k = 0; k < kNch; ++k) kf[k] = ld16(tb + frag_offset<T>(kl, lh * kNch + k));
        // tile holds padding or keys some window query cannot see
        const bool edge = (t + 1) * 128 > (causal ? N - W : N);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const int m = qb * 32 + ll;
          const int g = m >> rpg_shift, r = m & rpg_mask;
          const bool qok = g < G && r < W;
          const int qn = qok ? g * W + r : 0;
          u32x4_t qf[kNch];
#pragma unroll
          for (int k = 0; k < kNch; ++k)
            qf[k] = qok ? ld16(qlds + frag_offset<T>(qn, lh * kNch + k)) : zero16();
          f32x16_t acc = {};
#pragma unroll
          for (int k = 0; k < kNch; ++k) mma_chunk<T>(acc, kf[k], qf[k]);   // C[key][query]
          const int last = causal ? N - W + r : N - 1;   // last key visible to window query r
          float lg[16];
          float mt = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kk = t * 128 + wave * 32 + acc_row(v, lane_v);
            lg[v] = acc[v] * kLogitScaleLog2;
            if (edge || !qok) lg[v] = (qok && kk <= last) ? lg[v] : -INFINITY;
            mt = fmaxf(mt, lg[v]);
          }
          const float mn = fmaxf(mrun[qb], mt);
          if (mn != -INFINITY) {
            float s = (mrun[qb] != -INFINITY) ? srun[qb] * fast_exp2(mrun[qb] - mn) : 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) s += fast_exp2(lg[v] - mn);
            srun[qb] = s;
            mrun[qb] = mn;
          }
        }
      } else {
        // 1/||k|| of rows 32(w-4) + ll; the two halves hold the two halves of the row
        const int row = (wave - 4) * 32 + ll;
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < kNch; ++k) ss += sumsq_chunk<T>(ld16(tb + frag_offset<T>(row, lh * kNch + k)));
        ss += __shfl_xor(ss, 32, 64);
        const int key = t * 128 + row;
        if (lh == 0 && key < N) rn[key] = ss > 0.f ? __frsqrt_rn(ss) : 0.f;
      }
      ++c;
      cons_slot = cons_slot + 1 == S ? 0 : cons_slot + 1;
    }
    // merge the statistics: the two halves of a wave, then the four waves
    if (wave < 4) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float m2 = __shfl_xor(mrun[qb], 32, 64);
        const float s2 = __shfl_xor(srun[qb], 32, 64);
        const float mm = fmaxf(mrun[qb], m2);
        float st = 0.f;
        if (mm != -INFINITY)
          st = (mrun[qb] != -INFINITY ? srun[qb] * fast_exp2(mrun[qb] - mm) : 0.f) +
               (m2 != -INFINITY ? s2 * fast_exp2(m2 - mm) : 0.f);
        if (half == 0) {
          sred_m[wave * NQB * 32 + qb * 32 + l32] = mm;
          sred_s[wave * NQB * 32 + qb * 32 + l32] = st;
        }
      }
    }
    lds_barrier();
    if (tid < NQB * 32) {
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sred_m[w * NQB * 32 + tid]);
      float st = 0.f;
      if (mm != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float em = sred_m[w * NQB * 32 + tid], es = sred_s[w * NQB * 32 + tid];
          if (em != -INFINITY) st += es * fast_exp2(em - mm);
        }
      }
      const bool seen = mm != -INFINITY && st > 0.f;
      stats[tid] = u32x2_t{__float_as_uint(seen ? mm : 0.f), __float_as_uint(seen ? 1.0f / st : 0.f)};
    }
    // (the first block's barrier publishes the statistics and the norms)

    // ---------------- phase R: redundancy, importance, Z ----------------
    for (int bi = 0; bi < ni; ++bi) {
      const Block blk = block_of(bi, odd, nb, sym);
      const int base = blk.t0 * 128;
      const int r_lo = wr * 64;   // wave's first row within the block
      const bool wave_live = r_lo < blk.nt * 128 && base + r_lo < N;

      // 1. the block's own tile(s) have landed
      ensure_issued(c, blk.nt);
      wait_tiles(issued - (c + blk.nt));
      lds_barrier();
      u32x4_t af[2][kNch];
      {
        const char* dslot = slot_ptr(cons_slot, wr >> 1);
        const int arow = (wr & 1) * 64 + l32;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int k = 0; k < kNch; ++k)
            af[rb][k] = ld16(dslot + frag_offset<T>(arow + rb * 32, half * kNch + k));
      }
      // 2. importance of the block's keys: wave (r, c) takes keys 64r + 32c + l32
      if (wave_live) {
        const int key = base + r_lo + wc * 32 + l32;
        const bool cz = causal && base + blk.nt * 128 > N - W;   // block reaches the window
        const bool mean = p.pool_mean();
        const float best = wc == 0
            ? key_importance<NQB>(qlds, stats, af[0], key, N, W, G, rpg_shift, cz, mean, lane)
            : key_importance<NQB>(qlds, stats, af[1], key, N, W, G, rpg_shift, cz, mean, lane);
        if (half == 0) imp_l[r_lo + wc * 32 + l32] = best;
      }
      // 3. keep the ring full
      refill(c);

      float mx[2][16];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx[rb][v] = -INFINITY;

      // one 64x64 sub-block of the wave against tile `t` in `slot`. mode 0 =
      // every pair counts; bit 0 = diagonal (rows and columns are the same 64
      // keys: keep j < i, or j != i for the symmetric R); bit 1 = the unit's
      // last tile, whose columns past N are masked
      auto step = [&](const char* slot, int t, int mode) {
        f32x16_t acc[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x16_t{};
#pragma unroll
        for (int k = 0; k < kNch; ++k) {
          const u32x4_t b0 = ld16(slot + boff[k]);
          const u32x4_t b1 = ld16(slot + boff[k] + 32 * kRowBytes);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            mma_chunk<T>(acc[rb][0], af[rb][k], b0);
            mma_chunk<T>(acc[rb][1], af[rb][k], b1);
          }
        }
        // column norms (clamped reads: masked columns past N take any value)
        const int col = t * 128 + wc * 64 + l32;
        const float r0 = rn[min(col, N - 1)];
        const float r1 = rn[min(col + 32, N - 1)];
        if (mode == 0) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * r0, acc[rb][1][v] * r1));
        } else {
          int lane_v = lane;   // re-materialised: keeps the masks out of loop preheaders
          asm volatile("" : "+v"(lane_v));
          const int l = lane_v & 31;
          const bool diag = (mode & 1) != 0;
          const float rcb[2] = {r0, r1};
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              if (!sym && diag && cb > rb) continue;   // wholly above the diagonal
              const bool col_ok = !(mode & 2) || col + cb * 32 < N;
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                // on the diagonal, row rb*32 + a follows column cb*32 + b iff
                // rb > cb, or rb == cb and a > b; it is the same key iff
                // rb == cb and a == b
                const int a = acc_row(v, lane_v);
                const bool pair_ok = !diag || (sym ? (rb != cb || a != l) : (rb > cb || a > l));
                if (col_ok && pair_ok) mx[rb][v] = fmaxf(mx[rb][v], acc[rb][cb][v] * rcb[cb]);
              }
            }
        }
      };
      // columns past N exist only in the unit's last tile, and only rows that
      // precede them (symmetric R) must not see them
      const bool partial_last = sym && N % 128 != 0;

      // 4. the block's own tile(s): columns 128d + 64wc against rows r_lo
      // (columns right of the rows only for the symmetric R)
      for (int d = 0; d < blk.nt; ++d) {
        const int c_lo = 128 * d + 64 * wc;
        const int t = blk.t0 + d;
        const int mode = (c_lo == r_lo ? 1 : 0) | (partial_last && t == nb - 1 ? 2 : 0);
        if (wave_live && (sym || c_lo <= r_lo)) step(slot_ptr(cons_slot, d), t, mode);
      }
      c += blk.nt;
      cons_slot = cons_slot + blk.nt >= S ? cons_slot + blk.nt - S : cons_slot + blk.nt;

      // 5. tiles 0..t0-1, wholly left of the block's rows (and for the
      // symmetric R the tiles right of it)
      for (int j = 0; j < blk.ext; ++j) {
        ensure_issued(c, 1);
        wait_tiles(issued - (c + 1));
        lds_barrier();
        refill(c);
        const int t = blk.tile(blk.nt + j);
        if (wave_live) step(lds + cons_slot * kTileBytes, t, partial_last && t == nb - 1 ? 2 : 0);
        ++c;
        cons_slot = cons_slot + 1 == S ? 0 : cons_slot + 1;
      }

      // 6. row maxima over the wave's 64 columns; value j = rb*16 + v of a
      // lane belongs to row rb*32 + acc_row(v, lane); lane l ends with value l & 31
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
        const int rl = r_lo + (l32 >> 4) * 32 + acc_row(l32 & 15, lane);
        comb[wc * 256 + rl] = val[0];
      }
      lds_barrier();

      // 7. R, I, Z of the block's rows
      if (tid < 256) {
        const int row = base + tid;
        if (tid < blk.nt * 128 && row < N) {
          const float m = fmaxf(comb[tid], comb[256 + tid]);
          const float R = (row == 0 && !sym) ? 0.f : m * rn[row];
          const float I = imp_l[tid];
          const float z = lam * I - (1.0f - lam) * R + 0.0f;   // + 0 folds -0 onto +0
          zs[row] = z;
          if (Zdbg != nullptr) Zdbg[so + row] = z;
          if (Rdbg != nullptr) Rdbg[so + row] = R;
          if (Idbg != nullptr) Idbg[so + row] = I;
        }
      }
      // (the next block's barrier orders the reuse of imp_l and comb)
    }

    // ---------------- selection and gather ----------------
    // (score_only: Z went to Zdbg; a later launch selects for groups of units)
    if (!score_only) {
      __syncthreads();
      int32_t* kept = kept_all + p.kept_off(u);
      select_block<kThreads>(zs, N, B, W, kept, ssh, ks);
      __syncthreads();
      auto srck = [&](int r) { return p.krow(u, clamp_row(r, N)); };
      auto srcv = [&](int r) { return p.vrow(u, clamp_row(r, N)); };
      // the phase R registers are free here: 12 chunks of each tensor per
      // round for budgets of 2048 or more (qwen-14b: 4% faster per event),
      // 8 below (at B = 1024 the longer rounds measured 3% slower)
      if (B >= 2048)
        gather_rows_block<T, kThreads, decltype(srck), decltype(srcv), 12>(
            ks, B, srck, srcv, K_out + (int64_t)u * out_stride, V_out + (int64_t)u * out_stride);
      else
        gather_rows_block<T, kThreads, decltype(srck), decltype(srcv), 8>(
            ks, B, srck, srcv, K_out + (int64_t)u * out_stride, V_out + (int64_t)u * out_stride);
    }
    // ks is next written by the next unit's selection, after the barriers of
    // its statistics and redundancy phases
  }
}

template <int NQB, bool kSym>
static hipError_t run_t(const DenseProblem<bf16_bits>& p, float* dbg_Z, float* dbg_R, float* dbg_I,
                        float lam, int rpg_shift, int32_t* kept, bf16_bits* K_out,
                        bf16_bits* V_out, int64_t out_stride, int score_only, const FusedPlan& L,
                        hipStream_t st) {
  auto kern = k2f_kernel<NQB, kSym>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
  int dev = 0, cus = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = min(cus, p.num_units);   // one workgroup per CU, whole units each
  return launch("rkv_k2_compress", kern, dim3(grid), dim3(kThreads), L.total, st, p, dbg_Z, dbg_R,
                dbg_I, lam, rpg_shift, kept, K_out, V_out, out_stride, score_only, L);
}

}  // namespace fused

template <int NQB>
static hipError_t run_sym(const DenseProblem<bf16_bits>& p, float* dbg_Z, float* dbg_R, float* dbg_I,
                          float lam, int rpg_shift, int32_t* kept, bf16_bits* K_out,
                          bf16_bits* V_out, int64_t out_stride, int score_only,
                          const FusedPlan& L, hipStream_t st) {
  if (p.symmetric())
    return fused::run_t<NQB, true>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out,
                                   out_stride, score_only, L, st);
  return fused::run_t<NQB, false>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out,
                                  out_stride, score_only, L, st);
}

hipError_t run_k2_fused(const DenseProblem<bf16_bits>& p, int nqb, float* dbg_Z, float* dbg_R,
                        float* dbg_I, float lam, int rpg_shift, int32_t* kept, bf16_bits* K_out,
                        bf16_bits* V_out, int64_t out_stride, int score_only, hipStream_t st) {
  const FusedPlan L = fused_plan_choose(p.N, p.B, p.G * p.W, nqb);
  if (L.total == 0 || (score_only && dbg_Z == nullptr)) return hipErrorInvalidValue;
  switch (nqb) {
    case 1: return run_sym<1>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out, out_stride, score_only, L, st);
    case 2: return run_sym<2>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out, out_stride, score_only, L, st);
    case 3: return run_sym<3>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out, out_stride, score_only, L, st);
    default: return run_sym<4>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out, out_stride, score_only, L, st);
  }
}

}  // namespace rkv

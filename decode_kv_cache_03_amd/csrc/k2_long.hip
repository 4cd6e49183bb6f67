// Long units (bf16): redundancy, importance and Z of one row block per work
// item, by an 8-wave workgroup per CU that streams the unit's key tiles
// through an LDS ring. Two kernels: items of 1024 rows held in registers as
// 16x16 fragments (namespace longr, below: the causal R with one window-query
// block), and items of 512 rows as 32x32 fragments (namespace longu: the
// symmetric R and groups of more than one query block).
//
// Same arithmetic as the other scoring kernels (pages and readings cited in
// k2_redundancy.hip): R_i = max_{j<i} cos(k_i, k_j) (every j != i for the
// symmetric variant) on bf16 MFMA with fp32 accumulation, the norms applied
// in the fp32 epilogue; importance from the softmax normalisers of the
// statistics pass (k1_importance.hip); Z = lambda*I - (1-lambda)*R. Selection
// and compaction run as separate launches.
//
// Why a separate kernel: a unit of N keys needs N^2/2 cosine pairs but only
// N rows of keys, so for long units the contraction is MFMA-bound as long as
// each key tile fetched from memory feeds enough rows. The item kernels of
// k2_redundancy.hip feed 128 rows per 32 KiB tile; here an item holds 1024
// rows in the 16x16 form (longr: wave w holds row blocks of 32 with block
// index = w mod 8) or 512 rows in the 32x32 form (longu: wave w rows
// 64w..64w+63, both 64-column halves of every tile), so a tile carries 1024
// or 512 flop per byte fetched.
//
// Shape:
//  * tiles (128 rows, 32 KiB, XOR-swizzled chunks) stream through a ring of
//    up to 4 LDS slots by direct global->LDS loads; a step waits only for its
//    own tile (the wait counts the loads issued after it), and the stream
//    runs on across items; each item's window queries and softmax normalisers
//    come with its first tile, into one of two parity buffers; the 1024-row
//    form takes two tiles per workgroup barrier (4 slots: two in use, two in
//    flight);
//  * an item streams its own tiles in descending order (each wave takes its
//    rows as A fragments, its row norms and its keys' importance when its own
//    tile arrives; tiles of lower rows come later, so every wave that needs a
//    tile as columns holds its fragments already), then tiles 0..t0-1; the
//    symmetric variant adds the tiles right of the block and, at the end, the
//    own tiles above each wave's rows again;
//  * the 1/||k|| of a tile's rows (from the statistics pass) travel with the
//    tile into the ring, one 4-byte direct load per lane: in the 512-row
//    form each wave loads 16 rows of keys and norms (5 loads per tile, the
//    waits count 5); in the 1024-row form only waves 0-3 load, 32 rows each
//    (9 loads), so that waves 4-7, which lose the matrix-pipe arbitration to
//    them, never stall in the address unit;
//  * work items go to workgroups in order of decreasing cost, alternating
//    direction each round (a greedy longest-first schedule): item k of round
//    r is k = r*G + b for workgroup b on even rounds, r*G + G-1-b on odd ones.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"
#include "rkv_stream.hpp"
#include "rkv_frag16.hpp"
#include <type_traits>

namespace rkv {
namespace longu {

using stream::key_importance;
using stream::kLoadsPerTile;
using stream::kNch;
using stream::wait_tiles;

constexpr int kThreads = 512;
constexpr int kRowBytes = 256;
constexpr int kTileBytes = 128 * kRowBytes;

// Tile order of an item: own tiles t0..t0+nt-1 descending, then the `ext`
// other tiles ascending (0..t0-1; symmetric: also t0+nt..nb-1), then, for the
// symmetric variant, own tiles t0+1..t0+nt-1 again.
struct Geo {
  int t0, nt, nb, ext, again;
  __device__ int len() const { return nt + ext + again; }
  __device__ int tile(int k) const {
    if (k < nt) return t0 + nt - 1 - k;
    const int j = k - nt;
    if (j < ext) return j < t0 ? j : j + nt;
    return t0 + 1 + (j - ext);
  }
};
__device__ __forceinline__ Geo geo_of(int n, int blk, bool sym) {
  Geo g;
  g.nb = (n + 127) / 128;
  g.t0 = 4 * blk;
  g.nt = min(4, g.nb - g.t0);
  g.ext = sym ? g.nb - g.nt : g.t0;
  g.again = sym ? g.nt - 1 : 0;
  return g;
}

__device__ __forceinline__ int sched(int r, int b, int G) {
  return r * G + ((r & 1) ? G - 1 - b : b);
}

constexpr int kPer = kLoadsPerTile + 1;   // loads per wave per tile: 4 of keys, 1 of norms

template <int NQB, bool kSym, class P>
__global__ __launch_bounds__(kThreads, 1) void k2l_kernel(P p, const float* __restrict__ rinv,
                                                         const float* __restrict__ fin,
                                                         float* __restrict__ Z,
                                                         float* __restrict__ Rdbg,
                                                         float* __restrict__ Idbg, float lam,
                                                         int rpg_shift, LongPlan L) {
  using T = bf16_bits;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool sym = kSym;
  const int S = L.slots;
  const int W = p.W, G = p.G, gw = G * W;
  const bool causal = p.causal(), mean = p.pool_mean();
  const int count = p.long_count();
  const int grid = gridDim.x, bid = blockIdx.x;
  const T* rows = p.long_rows();
  constexpr int kStatsBytes = NQB * 32 * 8;

  // Tile load q (0..3) of wave w fills KiB 4w + q of a slot: tile row
  // 16w + 4q + lane/16 at chunk position lane % 16, fetching chunk
  // (lane % 16) ^ (row & 15) of that row.
  int lofs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r16 = (4 * q + lane / 16) & 15;
    lofs[q] = (lane / 16) * kRowBytes + (((lane % 16) ^ r16) << 4);
  }
  int boff[kNch];   // B fragments: rows l32 (+32) of a 64-column half, chunk half*8 + c
#pragma unroll
  for (int c = 0; c < kNch; ++c) boff[c] = frag_offset<T>(l32, half * kNch + c);

  // ---- loader: this workgroup's items, tile by tile, into the ring ----
  struct LdPos {
    int r, par, k;
    bool valid;
    LongItem it;
    Geo g;
  };
  auto fetch = [&](int r, LongItem& it, Geo& g) -> bool {
    const int k = sched(r, bid, grid);
    if (k >= count) return false;
    it = p.long_item(k);
    it.u = __builtin_amdgcn_readfirstlane(it.u);
    it.blk = __builtin_amdgcn_readfirstlane(it.blk);
    it.n = __builtin_amdgcn_readfirstlane(it.n);
    g = geo_of(it.n, it.blk, sym);
    return true;
  };
  LdPos ld;
  ld.r = 0;
  ld.par = 0;
  ld.k = 0;
  ld.valid = fetch(0, ld.it, ld.g);
  int issued = 0, issue_slot = 0;
  // The loader runs at most one item ahead of the consumer: the queries and
  // normalisers of two items share the two parity buffers.
  int ld_limit = 2;
  auto issue_next = [&]() -> bool {
    if (!ld.valid || ld.r >= ld_limit) return false;
    int lane_v = lane;   // per call: keeps lane-derived values out of the callers' loops
    asm volatile("" : "+v"(lane_v));
    const LongItem& it = ld.it;
    if (ld.k == 0) {   // the item's window queries and normalisers, ahead of its first tile
      const char* q = reinterpret_cast<const char*>(p.q(it.u));
      const int qkb = L.qbytes / 1024;
      char* qdst = lds + L.q + ld.par * L.qbytes;
      for (int kb = wave; kb < qkb; kb += 8) {
        const int n = kb * 4 + lane_v / 16;
        const int c = (lane_v % 16) ^ (n & 15);
        load16_to_lds(q + min(n, gw - 1) * kRowBytes + c * 16, qdst + kb * 1024);
      }
      if (wave == 0 && lane_v < NQB * 16)
        load16_to_lds(reinterpret_cast<const char*>(fin) + ((int64_t)it.u * NQB * 32) * 8 + lane_v * 16,
                      lds + L.stats + ld.par * kStatsBytes);
    }
    const int t = ld.g.tile(ld.k);
    char* slot = lds + issue_slot * kTileBytes;
    const T* urows = rows + it.row_base;
    // 1/||k|| of tile rows 16w.. (rows past n repeat row n-1), 16 lanes x 4 bytes
    if (lane_v < 16) {
      const int rr = min(t * 128 + wave * 16 + lane_v, it.n - 1);
      __builtin_amdgcn_global_load_lds(rinv + it.score_off + rr,
                                       (__attribute__((address_space(3))) void*)(lds + L.rn + issue_slot * 512 + wave * 64),
                                       4, 0, 0);
    }
    const int row0 = t * 128 + wave * 16;   // first tile row this wave loads
    if ((t + 1) * 128 <= it.n) {
      const char* src = reinterpret_cast<const char*>(urows + (int64_t)row0 * kD);
#pragma unroll
      for (int q = 0; q < 4; ++q) load16_to_lds(src + q * 1024 + lofs[q], slot + wave * 4096 + q * 1024);
    } else {   // the unit's last tile: rows past n repeat row n-1
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = min(row0 + 4 * q + lane_v / 16, it.n - 1);
        const int chunk_ofs = lofs[q] - (lane_v / 16) * kRowBytes;
        load16_to_lds(reinterpret_cast<const char*>(urows + (int64_t)r * kD) + chunk_ofs,
                      slot + wave * 4096 + q * 1024);
      }
    }
    ++issued;
    issue_slot = issue_slot + 1 == S ? 0 : issue_slot + 1;
    if (++ld.k == ld.g.len()) {
      ld.k = 0;
      ++ld.r;
      ld.par ^= 1;
      ld.valid = fetch(ld.r, ld.it, ld.g);
    }
    return true;
  };
  auto refill = [&](int c) {
    while (issued - c < S && issue_next()) {
    }
  };
  // Tile c is needed next. When the last refill could not issue it (the
  // loader held at an item boundary), its slot was freed by a step that every
  // wave finished only after a barrier: take one, then issue.
  auto ensure_issued = [&](int c) {
    if (issued < c + 1) {
      lds_barrier();
      refill(c);
    }
  };

  int c = 0, cons_slot = 0;   // tiles consumed, c % S
  refill(0);

  int par = 0;
  for (int r = 0;; ++r, par ^= 1) {
    LongItem it;
    Geo g;
    if (!fetch(r, it, g)) break;
    ld_limit = r + 2;
    const int n = it.n;
    const char* qlds = lds + L.q + par * L.qbytes;
    const u32x2_t* st = reinterpret_cast<const u32x2_t*>(lds + L.stats + par * kStatsBytes);
    const int base = g.t0 * 128;
    const int r_lo = wave * 64;   // wave's first row within the block
    const int own = wave >> 1;    // block tile holding the wave's rows
    const int hw = wave & 1;      // which 64-row half of it
    const bool wave_live = r_lo < g.nt * 128 && base + r_lo < n;
    // columns past n exist only in the last tile; only rows that precede them
    // (symmetric R) must not see them
    const bool partial_last = sym && n % 128 != 0;

    u32x4_t af[2][kNch];
    float mx[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx[rb][v] = -INFINITY;
    float rnr[2] = {0.f, 0.f}, imp[2] = {0.f, 0.f};   // rows rb*32 + l32 of the wave

    // the wave's 64 rows against columns 64ch.. of tile t in `slot`. mode bit
    // 0: the columns are the wave's own rows (keep j < i, or j != i for the
    // symmetric R); bit 1: mask columns past n
    auto half_step = [&](const char* slot, const float* rns, int t, int ch, int mode) {
      f32x16_t acc[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x16_t{};
      const char* bs = slot + ch * 64 * kRowBytes;
#pragma unroll
      for (int k = 0; k < kNch; ++k) {
        const u32x4_t b0 = ld16(bs + boff[k]);
        const u32x4_t b1 = ld16(bs + boff[k] + 32 * kRowBytes);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          mma_chunk<T>(acc[rb][0], af[rb][k], b0);
          mma_chunk<T>(acc[rb][1], af[rb][k], b1);
        }
      }
      // 1/||k|| of this lane's two columns
      const float r0 = rns[ch * 64 + l32];
      const float r1 = rns[ch * 64 + 32 + l32];
      if (mode == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * r0, acc[rb][1][v] * r1));
      } else {
        int lane_m = lane;   // re-materialised: keeps the masks out of loop preheaders
        asm volatile("" : "+v"(lane_m));
        const int l = lane_m & 31;
        const bool diag = (mode & 1) != 0;
        const int col = t * 128 + ch * 64 + l;
        const float rcb[2] = {r0, r1};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            if (!sym && diag && cb > rb) continue;   // wholly above the diagonal
            const bool col_ok = !(mode & 2) || col + cb * 32 < n;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              // on the diagonal, row rb*32 + a follows column cb*32 + b iff
              // rb > cb, or rb == cb and a > b; it is the same key iff
              // rb == cb and a == b
              const int a = acc_row(v, lane_m);
              const bool pair_ok = !diag || (sym ? (rb != cb || a != l) : (rb > cb || a > l));
              if (col_ok && pair_ok) mx[rb][v] = fmaxf(mx[rb][v], acc[rb][cb][v] * rcb[cb]);
            }
          }
      }
    };

    const int len = g.len();
    for (int k = 0; k < len; ++k) {
      ensure_issued(c);
      wait_tiles<kPer>(issued - (c + 1));
      lds_barrier();
      refill(c);
      const char* slot = lds + cons_slot * kTileBytes;
      const float* rns = reinterpret_cast<const float*>(lds + L.rn + cons_slot * 512);
      const int t = g.tile(k);
      const int cm = (partial_last && t == g.nb - 1) ? 2 : 0;
      // modes of the two 64-column halves for this wave (-1: not needed)
      int m0 = -1, m1 = -1;
      if (k < g.nt) {
        // own tile d, descending
        const int d = g.nt - 1 - k;
        if (wave_live && own == d) {
          const int arow = hw * 64 + l32;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int kk = 0; kk < kNch; ++kk)
              af[rb][kk] = ld16(slot + frag_offset<T>(arow + rb * 32, half * kNch + kk));
            rnr[rb] = rns[arow + rb * 32];
          }
          // only keys among the last w need the causal test
          const bool cz = causal && base + (d + 1) * 128 > n - W;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            imp[rb] = key_importance<NQB>(qlds, st, af[rb], base + r_lo + rb * 32 + l32, n, W, G,
                                          rpg_shift, cz, mean, lane);
          // half hw of this tile holds the wave's own rows; the other half
          // lies left of them (hw = 1) or right of them (hw = 0: symmetric R)
          m0 = (hw == 0 ? 1 : 0) | cm;
          m1 = hw == 1 ? (1 | cm) : (sym ? cm : -1);
        } else if (own > d) {   // the tile lies wholly left of the wave's rows
          m0 = m1 = cm;
        }
      } else if (k < g.nt + g.ext || own < t - g.t0) {
        // other tiles; last (symmetric R), own tiles right of the wave's rows
        m0 = m1 = cm;
      }
      if (wave_live && m0 >= 0) half_step(slot, rns, t, 0, m0);
      if (wave_live && m1 >= 0) half_step(slot, rns, t, 1, m1);
      ++c;
      cons_slot = cons_slot + 1 == S ? 0 : cons_slot + 1;
    }

    // row maxima over all columns; value j = rb*16 + v of a lane belongs to
    // row rb*32 + acc_row(v, lane); lane l ends with value l & 31, i.e. the
    // wave's 64 rows one per lane
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
      const int rl = (l32 >> 4) * 32 + acc_row(l32 & 15, lane);   // row within the wave
      const int src = rl & 31;                                     // lane holding its norm
      const float n0 = __shfl(rnr[0], src, 64), n1 = __shfl(rnr[1], src, 64);
      const float i0 = __shfl(imp[0], src, 64), i1 = __shfl(imp[1], src, 64);
      const int row = base + r_lo + rl;
      if (row < n) {
        const float R = (row == 0 && !sym) ? 0.f : val[0] * (rl >= 32 ? n1 : n0);
        const float I = rl >= 32 ? i1 : i0;
        const float z = lam * I - (1.0f - lam) * R + 0.0f;   // + 0 folds -0 onto +0
        const int64_t so = it.score_off;
        Z[so + row] = z;
        if (Rdbg != nullptr) Rdbg[so + row] = R;
        if (Idbg != nullptr) Idbg[so + row] = I;
      }
    }
  }
  // every load this workgroup issued was consumed: the ring is empty
}

template <int NQB, bool kSym, class P>
static hipError_t run_t(const P& p, int count, const float* rinv, const float* fin, float* Z, float* dbg_R,
                        float* dbg_I, float lam, int rpg_shift, const LongPlan& L,
                        hipStream_t st) {
  auto kern = k2l_kernel<NQB, kSym, P>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
  int dev = 0, cus = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = min(cus, count);
  return launch("rkv_k2_long", kern, dim3(grid), dim3(kThreads), L.total, st, p, rinv, fin, Z, dbg_R,
                dbg_I, lam, rpg_shift, L);
}

template <int NQB, class P>
static hipError_t run_sym(const P& p, int count, const float* rinv, const float* fin, float* Z,
                          float* dbg_R, float* dbg_I, float lam, int rpg_shift, const LongPlan& L,
                          hipStream_t st) {
  if (p.symmetric())
    return run_t<NQB, true>(p, count, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, L, st);
  return run_t<NQB, false>(p, count, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, L, st);
}

}  // namespace longu

// ---- 1024-row items held in registers (one window-query block, causal R) ----
//
// An item's rows are held the way k2_resident.hip holds a unit's keys: row
// block b (32 rows) of the item by wave b % 8, slot b / 8, as 16x16x32 MFMA
// fragments (rkv_frag16.hpp), so each 32 KiB tile fetched feeds 1024 rows
// (1024 flop per byte). Own tiles come first, descending: when own tile d
// lands its owners copy their blocks and take the rows' norms (staged with
// the tile) and importance, and every block of tiles d.. meets its columns
// (the block of tile d under the diagonal mask). Tiles 0..t0-1 follow. A lane
// keeps, for each of its accumulator rows, the max over the columns it met of
// dot * (1/||k_j||); the max over the 16 column lanes and * (1/||k_i||) give R
// at the end of the item.
namespace longr {

using namespace frag16;
using stream::kLoadsPerTile;
using stream::wait_tiles;

constexpr int kThreads = 512;
constexpr int kRowBytes = 256;
constexpr int kTileBytes = 128 * kRowBytes;
// Only waves 0-3 load tiles: 8 loads of keys and 1 of norms each per tile.
// A wave stalls while the address unit takes its loads; waves 4-7, which
// share each SIMD's matrix pipe with them and lose the issue arbitration to
// the older waves, never do.
constexpr int kLoaders = 4;
constexpr int kPer = 2 * kLoadsPerTile + 1;

// Tile order of an item of up to 8 own tiles: own tiles descending, then
// tiles 0..t0-1.
struct Geo {
  int t0, nt, nb;
  __device__ int len() const { return nt + t0; }
  __device__ int tile(int k) const { return k < nt ? t0 + nt - 1 - k : k - nt; }
};
__device__ __forceinline__ Geo geo_of(int n, int blk) {
  Geo g;
  g.nb = (n + 127) / 128;
  g.t0 = 8 * blk;
  g.nt = min(8, g.nb - g.t0);
  return g;
}

template <class P>
__global__ __launch_bounds__(kThreads, 1) void k2lr_kernel(P p, const float* __restrict__ rinv,
                                                          const float* __restrict__ fin,
                                                          float* __restrict__ Z,
                                                          float* __restrict__ Rdbg,
                                                          float* __restrict__ Idbg, float lam,
                                                          float oml, float inv_pool, int rpg_shift,
                                                          LongPlanR L) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = L.slots;
  const int W = p.W, G = p.G, gw = G * W;
  const bool causal = p.causal(), mean = p.pool_mean();
  const int count = p.long_count();
  const int grid = gridDim.x, bid = blockIdx.x;
  const bf16_bits* rows = p.long_rows();
  constexpr int kStatsBytes = 32 * 8;
  float* const rrn = reinterpret_cast<float*>(lds + L.rrn);   // [1024] 1/||k|| of the item's rows
  float* const rim = reinterpret_cast<float*>(lds + L.rim);   // [1024] importance

  // ---- loader: this workgroup's items, tile by tile, into the ring ----
  auto fetch = [&](int r, LongItem& it, Geo& g) -> bool {
    const int k = r * grid + ((r & 1) ? grid - 1 - bid : bid);   // snake over rounds
    if (k >= count) return false;
    it = p.long_item(k);
    it.u = __builtin_amdgcn_readfirstlane(it.u);
    it.blk = __builtin_amdgcn_readfirstlane(it.blk);
    it.n = __builtin_amdgcn_readfirstlane(it.n);
    g = geo_of(it.n, it.blk);
    return true;
  };
  int ld_r = 0, ld_par = 0, ld_k = 0;
  LongItem ld_it;
  Geo ld_g;
  bool ld_valid = fetch(0, ld_it, ld_g);
  int issued = 0, issue_slot = 0;
  // The loader runs at most one item ahead of the consumer: the queries and
  // normalisers of two items share the two parity buffers.
  int ld_limit = 2;
  auto issue_next = [&]() -> bool {
    if (!ld_valid || ld_r >= ld_limit) return false;
    int lane_v = lane;   // per call: keeps lane-derived values out of the callers' loops
    asm volatile("" : "+v"(lane_v));
    if (ld_k == 0) {   // the item's window queries and normalisers, ahead of its first tile
      const char* q = reinterpret_cast<const char*>(p.q(ld_it.u));
      const int qkb = L.qbytes / 1024;
      char* qdst = lds + L.q + ld_par * L.qbytes;
      for (int kb = wave; kb < qkb; kb += 8) {
        const int n = kb * 4 + lane_v / 16;
        const int c = (lane_v % 16) ^ (n & 15);
        load16_to_lds(q + min(n, gw - 1) * kRowBytes + c * 16, qdst + kb * 1024);
      }
      if (wave == 0 && lane_v < 16)
        load16_to_lds(reinterpret_cast<const char*>(fin) + ((int64_t)ld_it.u * 32) * 8 + lane_v * 16,
                      lds + L.stats + ld_par * kStatsBytes);
    }
    const int t = ld_g.tile(ld_k);
    char* slot = lds + issue_slot * kTileBytes;
    const bf16_bits* urows = rows + ld_it.row_base;
    if (wave < kLoaders) {
      // 1/||k|| of tile rows 32w.. (rows past n repeat row n-1), 32 lanes x 4 bytes
      if (lane_v < 32) {
        const int rr = min(t * 128 + wave * 32 + lane_v, ld_it.n - 1);
        __builtin_amdgcn_global_load_lds(rinv + ld_it.score_off + rr,
                                         (__attribute__((address_space(3))) void*)(lds + L.rn + issue_slot * 512 + wave * 128),
                                         4, 0, 0);
      }
      // Tile load q (0..7) of wave w fills KiB 8w + q of a slot: tile row
      // 32w + 4q + lane/16 at chunk position lane % 16, fetching chunk
      // (lane % 16) ^ (row & 15) of that row.
      const int row0 = t * 128 + wave * 32;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int rt = row0 + 4 * q + lane_v / 16;
        const int r = min(rt, ld_it.n - 1);   // rows past n repeat row n-1
        const int c = (lane_v % 16) ^ (rt & 15);
        load16_to_lds(reinterpret_cast<const char*>(urows + (int64_t)r * kD) + c * 16,
                      slot + wave * 8192 + q * 1024);
      }
    }
    ++issued;
    issue_slot = issue_slot + 1 == S ? 0 : issue_slot + 1;
    if (++ld_k == ld_g.len()) {
      ld_k = 0;
      ++ld_r;
      ld_par ^= 1;
      ld_valid = fetch(ld_r, ld_it, ld_g);
    }
    return true;
  };
  auto refill = [&](int c) {
    while (issued - c < S && issue_next()) {
    }
  };
  auto ensure_issued = [&](int c) {
    if (issued < c + 1) {
      lds_barrier();
      refill(c);
    }
  };

  int c = 0, cons_slot = 0;   // tiles consumed, c % S
  refill(0);

  int par = 0;
  for (int r = 0;; ++r, par ^= 1) {
    LongItem it;
    Geo g;
    if (!fetch(r, it, g)) break;
    ld_limit = r + 2;
    int lane_u = lane;   // per item: keeps lane-derived values from living across items
    asm volatile("" : "+v"(lane_u));
    const int n = it.n;
    const int base = g.t0 * 128;
    const char* qlds = lds + L.q + par * L.qbytes;
    const u32x2_t* st = reinterpret_cast<const u32x2_t*>(lds + L.stats + par * kStatsBytes);
    // held slots of this wave: row blocks 8s + wave < 4 nt
    const int nheld = min(4, max(0, (4 * g.nt - wave + 7) >> 3));

    u32x4_t A[4][2][4];
    f32x4_t mx[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) mx[s][rs] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};

    // rows of held slot s (16-row half rs) against the 16 columns of bf:
    // mask 0 = every column counts; 1 = the same tile, column < row counts
    auto block = [&](auto sc, const u32x4_t (&bf)[4], float rc, int col_in_tile, int mask) {
      constexpr int s = decltype(sc)::value;
      f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) mma16(acc[rs], A[s][rs][ks], bf[ks]);   // C[row][col]
      if (mask == 0) {
#pragma unroll
        for (int rs = 0; rs < 2; ++rs)
#pragma unroll
          for (int v = 0; v < 4; ++v) mx[s][rs][v] = vmax(mx[s][rs][v], acc[rs][v] * rc);
      } else {
        int lane_m = lane_u;   // re-materialised: keeps the masks out of loop preheaders
        asm volatile("" : "+v"(lane_m));
        const int row0 = ((8 * s + wave) & 3) * 32 + 4 * (lane_m >> 4);   // row within the tile
#pragma unroll
        for (int rs = 0; rs < 2; ++rs)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (col_in_tile < row0 + rs * 16 + v) mx[s][rs][v] = vmax(mx[s][rs][v], acc[rs][v] * rc);
      }
    };
    // unmasked rows of half-block u = 2s + rs of the held slots against two
    // column sub-blocks: the products (half_mma), then the running maxima,
    // each taking both products in one three-way max (half_max)
    auto half_mma = [&](auto uc, const u32x4_t (&bf)[2][4], f32x4_t (&acc)[2]) {
      constexpr int s = decltype(uc)::value >> 1, rs = decltype(uc)::value & 1;
      acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) mma16(acc[h], A[s][rs][ks], bf[h][ks]);
    };
    auto half_max = [&](auto uc, const f32x4_t (&acc)[2], float rc0, float rc1) {
      constexpr int s = decltype(uc)::value >> 1, rs = decltype(uc)::value & 1;
#pragma unroll
      for (int v = 0; v < 4; ++v) mx[s][rs][v] = vmax(mx[s][rs][v], vmax(acc[0][v] * rc0, acc[1][v] * rc1));
    };

    // Tiles are taken two per barrier: after it, each wave works through
    // both without waiting for the others (an owner copies only its own rows,
    // and what it writes to LDS is read after the item's last barrier); the
    // two slots are given back at the next barrier.
    const int len = g.len();
    for (int k0 = 0; k0 < len; k0 += 2) {
      const int two = k0 + 1 < len ? 2 : 1;
      if (issued < c + two) {   // the pair not issued yet (start of an item)
        lds_barrier();
        refill(c);
      }
      // waves 4-7 issue only an item's window queries (and their Z stores):
      // they wait for all of theirs
      wait_tiles<kPer>(wave < kLoaders ? issued - (c + two) : 0);
      lds_barrier();
      refill(c);
#pragma unroll 1
      for (int k = k0; k < k0 + two; ++k) {
      const char* slot = lds + cons_slot * kTileBytes;
      const float* rns = reinterpret_cast<const float*>(lds + L.rn + cons_slot * 512);
      const bool own = k < g.nt;
      const int d = g.nt - 1 - k;   // own tile, relative (own steps)
      if (own && (wave >> 2) == (d & 1)) {
        // this wave's block of own tile d: registers, norms, importance
        int lane_o = lane_u;
        asm volatile("" : "+v"(lane_o));
        const int rb = wave & 3;                // block within the tile
        const int rel = (4 * d + rb) * 32;      // first row within the item
        u32x4_t qf[2][4];
        load_queries(qlds, lane_o, W, G, rpg_shift, qf);
        float smax[2][4], sinv[2][4];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const u32x2_t sv = st[qs * 16 + 4 * (lane_o >> 4) + v];
            smax[qs][v] = __uint_as_float(sv.x);
            sinv[qs][v] = __uint_as_float(sv.y);
          }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s != (d >> 1)) continue;
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) {
            load_frag(slot, rb * 32 + rs * 16, lane_o, A[s][rs]);
            const float I = key_importance16(A[s][rs], qf, smax, sinv, base + rel + rs * 16, n, W,
                                             rpg_shift, causal, mean, inv_pool, lane_o);
            if (lane_o < 16) {
              rrn[rel + rs * 16 + lane_o] = rns[rb * 32 + rs * 16 + lane_o];
              rim[rel + rs * 16 + lane_o] = I;
            }
          }
        }
      }
      // which held slots meet this tile: own tile d, blocks of tiles d..
      // (slots s_lo..), the block of tile d itself under the mask; other
      // tiles, every held slot
      const int s_lo = own ? max(0, (4 * d - wave + 7) >> 3) : 0;
      const int s_diag = own && (wave >> 2) == (d & 1) ? (d >> 1) : -1;
      if (s_lo == 0 && nheld == 4 && s_diag < 0) {
        // every held slot, no mask: straight-line runs over column pairs
#pragma unroll 1
        for (int cs = 0; cs < 8; cs += 2) {
          u32x4_t bf[2][4];
          load_frag(slot, cs * 16, lane_u, bf[0]);
          load_frag(slot, cs * 16 + 16, lane_u, bf[1]);
          const float rc0 = rns[cs * 16 + (lane_u & 15)];
          const float rc1 = rns[cs * 16 + 16 + (lane_u & 15)];
          // a software pipeline over the eight half-blocks: the maxima of
          // u - 1 are taken between the products of u
          f32x4_t acc[2][2];
          auto stage = [&](auto uc) {
            constexpr int u = decltype(uc)::value;
            half_mma(uc, bf, acc[u & 1]);
            half_max(std::integral_constant<int, u - 1>{}, acc[(u - 1) & 1], rc0, rc1);
            interleave_8mfma_12valu();
          };
          half_mma(std::integral_constant<int, 0>{}, bf, acc[0]);
          stage(std::integral_constant<int, 1>{});
          stage(std::integral_constant<int, 2>{});
          stage(std::integral_constant<int, 3>{});
          stage(std::integral_constant<int, 4>{});
          stage(std::integral_constant<int, 5>{});
          stage(std::integral_constant<int, 6>{});
          stage(std::integral_constant<int, 7>{});
          half_max(std::integral_constant<int, 7>{}, acc[1], rc0, rc1);
        }
      } else {
#pragma unroll 1
        for (int cs = 0; cs < 8; ++cs) {
          u32x4_t bf[4];
          load_frag(slot, cs * 16, lane_u, bf);
          const float rc = rns[cs * 16 + (lane_u & 15)];
          const int col = cs * 16 + (lane_u & 15);   // column within the tile
          auto one = [&](auto sc) {
            constexpr int s = decltype(sc)::value;
            if (s < s_lo || s >= nheld) return;
            if (s == s_diag) {
              // block rb of tile d: columns of the block's own rows or earlier
              if (cs * 16 < ((wave & 3) + 1) * 32) block(sc, bf, rc, col, 1);
            } else {
              block(sc, bf, rc, col, 0);
            }
          };
          one(std::integral_constant<int, 0>{});
          one(std::integral_constant<int, 1>{});
          one(std::integral_constant<int, 2>{});
          one(std::integral_constant<int, 3>{});
        }
      }
      ++c;
      cons_slot = cons_slot + 1 == S ? 0 : cons_slot + 1;
      }
    }

    // row maxima over the 16 column lanes of each quarter, then R, I, Z
    lds_barrier();   // the owners' norms and importance are in
    int lane_e = lane_u;
    asm volatile("" : "+v"(lane_e));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s >= nheld) continue;
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        float x[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float m = mx[s][rs][v];
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
          x[v] = m;
        }
        const int v = lane_e & 15;   // lanes 0..3 of each quarter write one row each
        if (v < 4) {
          const float m = v == 0 ? x[0] : (v == 1 ? x[1] : (v == 2 ? x[2] : x[3]));
          const int rel = (8 * s + wave) * 32 + rs * 16 + 4 * (lane_e >> 4) + v;
          const int row = base + rel;
          if (row < n) {
            const float R = row == 0 ? 0.f : m * rrn[rel];
            const float I = rim[rel];
            const float z = lam * I - oml * R + 0.0f;   // + 0 folds -0 onto +0
            Z[it.score_off + row] = z;
            if (Rdbg != nullptr) Rdbg[it.score_off + row] = R;
            if (Idbg != nullptr) Idbg[it.score_off + row] = I;
          }
        }
      }
    }
    // (rrn and rim are next written by the next item's own tiles, after the
    // barrier of its first step)
  }
  // every load this workgroup issued was consumed: the ring is empty
}

template <class P>
static hipError_t run_r(const P& p, int count, const float* rinv, const float* fin, float* Z,
                        float* dbg_R, float* dbg_I, float lam, int rpg_shift, hipStream_t st) {
  const LongPlanR L = long_plan_r(p.G * p.W);
  if (L.total == 0) return hipErrorInvalidValue;
  auto kern = k2lr_kernel<P>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
  int dev = 0, cus = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = min(cus, count);
  // 1 - lambda and the pooling scale as arguments: uniform values that stay in
  // scalar registers
  const float oml = 1.0f - lam;
  const float inv_pool = p.pool_mean() ? 1.0f / (float)(p.W * p.G) : 1.0f / (float)p.W;
  return launch("rkv_k2_long", kern, dim3(grid), dim3(kThreads), L.total, st, p, rinv, fin, Z, dbg_R,
                dbg_I, lam, oml, inv_pool, rpg_shift, L);
}

}  // namespace longr

template <class P>
hipError_t run_k2_long(const P& p, int nqb, int count, const float* rinv, const float* fin, float* Z,
                       float* dbg_R, float* dbg_I, float lam, int rpg_shift, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  if (long_block_rows(nqb, p.symmetric()) == 1024)
    return longr::run_r(p, count, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, st);
  const LongPlan L = long_plan_choose(p.G * p.W, nqb);
  if (L.total == 0) return hipErrorInvalidValue;
  switch (nqb) {
    case 1: return longu::run_sym<1>(p, count, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, L, st);
    case 2: return longu::run_sym<2>(p, count, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, L, st);
    case 3: return longu::run_sym<3>(p, count, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, L, st);
    default: return longu::run_sym<4>(p, count, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, L, st);
  }
}

template hipError_t run_k2_long<DenseProblem<bf16_bits>>(const DenseProblem<bf16_bits>&, int, int, const float*, const float*, float*, float*, float*, float, int, hipStream_t);
template hipError_t run_k2_long<PagedProblem<bf16_bits>>(const PagedProblem<bf16_bits>&, int, int, const float*, const float*, float*, float*, float*, float, int, hipStream_t);

}  // namespace rkv

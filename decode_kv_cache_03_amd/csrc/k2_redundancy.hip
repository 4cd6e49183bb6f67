// Redundancy R, importance I and joint score Z of fp32 caches; for dense
// caches the same kernel then selects and gathers each unit.
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
// Z = lambda*I - (1-lambda)*R (same summary, "Approach"). Variants: the
// symmetric R (max over every j != i; each block then sweeps every column
// tile), no causal window, mean pooling over the GQA heads.
//
// The cosine matrix is the one dense contraction of the step (N x N x 128
// per unit), so it runs on fp32 MFMA (v_mfma_f32_32x32x2_f32) on the raw
// keys; the norms 1/||k|| are applied in the
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
// Tiles 0..blk-1 lie wholly left of the diagonal and run unmasked. After
// the A fragments are read, the block's keys are scored for importance: with
// the key rows as the B operand of Q x K^T each lane holds one key and 16
// query rows, so the mean over a head's window queries and the max over heads
// reduce inside the lane (plus one exchange between the 32-lane halves). At
// the end the row maxima are reduced across lanes by a butterfly that halves
// the values per lane at each exchange.
//
// The kernel is persistent (about two workgroups per CU) and walks a list of
// items; item k goes to workgroup k mod G with G a multiple of 8, so all
// blocks of a unit run on one XCD and the unit's keys, re-read once per
// block, stay in that XCD's L2 (one workgroup per unit would keep ~64 units
// live per XCD, far more keys than its L2 holds). The tile stream never stops
// between items: during an item's last step the next item's diagonal tile is
// already being loaded. Per-lane addresses are computed once (tiles arrive by
// direct global->LDS loads from a uniform base plus a fixed per-lane offset;
// fragment reads use fixed per-lane LDS offsets), since the MFMA issue rate
// is the budget.
//
// Dense caches: after its block's scores are written, each workgroup counts
// the block in the unit's arrival counter; the one that completes the count
// selects the unit's kept indices and gathers its kept K/V rows, so those
// memory-bound phases overlap other workgroups' MFMA work and no workgroup
// ever waits on another. Paged caches run selection and the in-place
// compaction as separate launches (k4_select.hip, k5_compact.hip).
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"

namespace rkv {

template <typename T>
struct K2Cfg {
  static constexpr int NCH = Elem<T>::kHalfChunks;
  static constexpr int RC = Elem<T>::kRowChunks;
  static constexpr int RB = Elem<T>::kRowBytes;
  static constexpr int TILE_BYTES = kK2Cols * RB;
  static constexpr int LOADS = kK2Cols * RB / 1024 / 4;   // KiB of tile per wave
  static constexpr int ROWS_PER_KB = 1024 / RB;
  static constexpr int PER = 16 / ROWS_PER_KB;            // tile loads per swizzle period
};

// Per-workgroup context: LDS regions and per-lane constants.
template <typename T>
struct K2Ctx {
  using C = K2Cfg<T>;
  char* tiles;
  char* qlds;
  float2* slds;
  float* imp_l;
  float* comb;
  int tid, lane, half, l32, wave, wr, wc;
  int rpg_shift;
  float lam;
  int lofs[C::PER];   // tile-load offsets (bytes) by load index mod PER
  int boff[C::NCH];   // B fragment offsets; A fragments sit a_minus_b further
  int a_minus_b;

  __device__ __forceinline__ void init(char* lds, const K2Lds& plan, int rpg, float lam_) {
    tiles = lds + plan.tiles;
    qlds = lds + plan.q;
    slds = reinterpret_cast<float2*>(lds + plan.stats);
    imp_l = reinterpret_cast<float*>(lds + plan.imp);
    comb = reinterpret_cast<float*>(lds + plan.comb);
    tid = threadIdx.x;
    lane = tid & 63;
    half = lane >> 5;
    l32 = lane & 31;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wr = wave >> 1;
    wc = wave & 1;
    rpg_shift = rpg;
    lam = lam_;
    // Wave w fills KiB w*LOADS + i of a tile; lane l of load i writes row
    // ROWS_PER_KB*i + l/RC of the wave's rows at slot l % RC, fetching chunk
    // slot ^ (row & 15); row & 15 repeats every PER loads.
#pragma unroll
    for (int q = 0; q < C::PER; ++q) {
      const int r16 = (q * C::ROWS_PER_KB + lane / C::RC) & 15;
      lofs[q] = (lane / C::RC) * C::RB + (((lane % C::RC) ^ r16) << 4);
    }
    // Fragment reads: rows (A) wr*64 + rb*32 + l32, columns (B) wc*64 + cb*32
    // + l32, chunk half*NCH + c; +32 rows keeps row & 15, so it is +32*RB.
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) boff[c] = frag_offset<T>(wc * 64 + l32, half * C::NCH + c);
    a_minus_b = (wr - wc) * 64 * C::RB;
  }
};

// Rows first_row..first_row+127 of unit u into tile buffer buf; rows past the
// unit repeat its last row (only the last tile of a unit has such rows).
template <typename T, class P>
__device__ __forceinline__ void tile_load(const P& p, const K2Ctx<T>& x, int u, int n_u,
                                          int first_row, int buf, bool clamp) {
  using C = K2Cfg<T>;
  char* dst = x.tiles + buf * C::TILE_BYTES + x.wave * C::LOADS * 1024;
  const int wrow = first_row + x.wave * C::LOADS * C::ROWS_PER_KB;   // first row this wave loads
  if constexpr (P::kRowsContiguous) {
    if (!clamp) {
      const char* src = reinterpret_cast<const char*>(p.krow(u, wrow));
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i)
        load16_to_lds(src + i * 1024 + x.lofs[i % C::PER], dst + i * 1024);
      return;
    }
  }
  int lane = x.lane;
  asm volatile("" : "+v"(lane));   // per call: keeps the row offsets out of callers' loops
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int r = min(wrow + i * C::ROWS_PER_KB + lane / C::RC, n_u - 1);
    const int chunk_ofs = x.lofs[i % C::PER] - (lane / C::RC) * C::RB;
    load16_to_lds(reinterpret_cast<const char*>(p.krow(u, r)) + chunk_ofs, dst + i * 1024);
  }
}

// The unit's window queries (G*w rows, swizzled like tile rows) into LDS.
template <typename T, class P>
__device__ __forceinline__ void q_load(const P& p, const K2Ctx<T>& x, int u) {
  using C = K2Cfg<T>;
  const int gw = p.G * p.W;
  const char* q = reinterpret_cast<const char*>(p.q(u));
  const int qkb = (gw * C::RB + 1023) / 1024;
  int lane = x.lane;
  asm volatile("" : "+v"(lane));   // per call: keeps the offsets out of callers' loops
  for (int kb = x.wave; kb < qkb; kb += 4) {
    const int n = kb * C::ROWS_PER_KB + lane / C::RC;
    const int c = (lane % C::RC) ^ (n & 15);
    load16_to_lds(q + min(n, gw - 1) * C::RB + c * 16, x.qlds + kb * 1024);
  }
}

// Softmax normalisers (max, 1/sum) of the unit's query rows from global memory.
template <int NQB, typename T>
__device__ __forceinline__ void stats_load(const float* fin, const K2Ctx<T>& x, int u) {
  if (x.wave == 0 && x.lane < NQB * 16)
    load16_to_lds(reinterpret_cast<const char*>(fin) + ((int64_t)u * NQB * 32 + 2 * x.lane) * 8,
                  reinterpret_cast<char*>(x.slds));
}

template <typename T>
__device__ __forceinline__ void tile_mma(const char* tb, const K2Ctx<T>& x,
                                         const u32x4_t (&af)[2][K2Cfg<T>::NCH],
                                         f32x16_t (&acc)[2][2]) {
  using C = K2Cfg<T>;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x16_t{};
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    const u32x4_t b0 = ld16(tb + x.boff[c]);
    const u32x4_t b1 = ld16(tb + x.boff[c] + 32 * C::RB);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      mma_chunk<T>(acc[rb][0], af[rb][c], b0);
      mma_chunk<T>(acc[rb][1], af[rb][c], b1);
    }
  }
}

// Importance of one key per lane (key = row of kf; both 32-lane halves hold
// the same key). Padding query rows (r >= w or g >= G) have zero queries and
// zero 1/sum, so they add nothing; only keys among the last w need the
// causal test.
template <typename T, int NQB, class P>
__device__ __forceinline__ float block_importance(const P& p, const K2Ctx<T>& x,
                                                  const u32x4_t (&kf)[K2Cfg<T>::NCH], int key,
                                                  int n_u, bool causal) {
  using C = K2Cfg<T>;
  const int rpg_mask = (1 << x.rpg_shift) - 1;
  const int octets_per_group = (1 << x.rpg_shift) >> 3;
  const float inv_w = 1.0f / (float)p.W;
  const bool mean = p.pool_mean();
  float best = 0.f, run = 0.f;
  int lane_v = x.lane;   // re-materialised per call: keeps per-lane masks out of loop preheaders
  asm volatile("" : "+v"(lane_v));
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    u32x4_t qf[C::NCH];
    {
      const int m = qb * 32 + (lane_v & 31);
      const int g = m >> x.rpg_shift, r = m & rpg_mask;
      const bool qok = g < p.G && r < p.W;
      const int n = qok ? g * p.W + r : 0;
#pragma unroll
      for (int c = 0; c < C::NCH; ++c)
        qf[c] = qok ? ld16(x.qlds + frag_offset<T>(n, x.half * C::NCH + c)) : zero16();
    }
    f32x16_t acc = {};
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) mma_chunk<T>(acc, qf[c], kf[c]);   // C[query][key]
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float os = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = 4 * t + j;
        const int m = qb * 32 + acc_row(v, lane_v);
        const float2 st = x.slds[m];
        const float pr = fast_exp2(acc[v] * kLogitScaleLog2 - st.x) * st.y;
        const float vis = (!causal || key <= n_u - p.W + (m & rpg_mask)) ? 1.f : 0.f;
        os = fmaf(pr, vis, os);   // arithmetic, not a branch around the exp
      }
      os += __shfl_xor(os, 32, 64);
      run += os;
      const int o = qb * 4 + t;
      if (((o + 1) & (octets_per_group - 1)) == 0) {
        if (o / octets_per_group < p.G) best = mean ? best + run * inv_w : fmaxf(best, run * inv_w);
        run = 0.f;
      }
    }
  }
  return mean ? best / (float)p.G : best;
}

// What a block loads during its last step: the next block's diagonal tile,
// and for a different unit its queries and normalisers (from `fin`).
struct Prefetch {
  bool valid;
  int u, n, first_row;
  bool queries;
};

// One block (unit u, rows blk*128..): on entry its diagonal tile is in flight
// into buffer `cur`; on exit `cur` holds the prefetched tile, if any.
template <typename T, int NQB, bool kAgentZ, bool kSym, class P>
__device__ __forceinline__ void k2_block(const P& p, const K2Ctx<T>& x, int& cur, int u, int N,
                                         int blk, const float* __restrict__ rinv,
                                         const Prefetch& nx, const float* __restrict__ fin,
                                         float* __restrict__ Z, float* __restrict__ Rdbg,
                                         float* __restrict__ Idbg) {
  using C = K2Cfg<T>;
  constexpr int NCH = C::NCH;
  const int base = blk * kK2Rows;
  const int row0 = base + x.wr * 64;
  const bool wave_live = row0 < N;
  const int64_t so = p.score_off(u);
  auto prefetch_next = [&]() {
    if (!nx.valid) return;
    tile_load<T>(p, x, nx.u, nx.n, nx.first_row, cur ^ 1, true);
    if (nx.queries) {
      q_load<T>(p, x, nx.u);
      stats_load<NQB>(fin, x, nx.u);
    }
  };

  // 1. the diagonal tile (and the unit's queries) have landed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  u32x4_t af[2][NCH];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      af[rb][c] = ld16(x.tiles + cur * C::TILE_BYTES + x.boff[c] + x.a_minus_b + rb * 32 * C::RB);

  // 2. importance of the block's keys; wave (r, c) takes keys r*64 + c*32 + l32
  if (wave_live) {
    const int key = row0 + x.wc * 32 + x.l32;
    const bool causal = p.causal() && base + kK2Rows > N - p.W;   // block reaches the window's keys
    const float best = (x.wc == 0) ? block_importance<T, NQB>(p, x, af[0], key, N, causal)
                                   : block_importance<T, NQB>(p, x, af[1], key, N, causal);
    if (x.half == 0) x.imp_l[x.wr * 64 + x.wc * 32 + x.l32] = best;
  }
  __syncthreads();   // queries are no longer read: a prefetch may replace them

  // column tiles other than the diagonal one: 0..blk-1, and for the
  // symmetric R also blk+1..nb-1 (the last of which may hold rows past N)
  constexpr bool sym = kSym;
  const int nb = (N + kK2Cols - 1) / kK2Cols;
  const int ncol = sym ? nb - 1 : blk;
  auto col_tile = [&](int J) { return J < blk ? J : J + 1; };

  // 3. prefetch: the first column tile, or what follows the block
  if (ncol > 0) {
    const int t = col_tile(0);
    tile_load<T>(p, x, u, N, t * kK2Cols, cur ^ 1, (t + 1) * kK2Cols > N);
  } else {
    prefetch_next();
  }

  float mx[2][16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx[rb][v] = -INFINITY;

  // Columns past N (in the unit's last tile) meet rows past N, masked pairs,
  // or, for the symmetric R, rows below N: there they are masked too.
  auto masked_update = [&](const f32x16_t (&acc)[2][2], const float (&rc)[2], int col0, bool diag) {
    int lane_v = x.lane;   // re-materialised (see block_importance)
    asm volatile("" : "+v"(lane_v));
    const int l = lane_v & 31;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const bool col_ok = col0 + cb * 32 + l < N;
        if (!sym && diag && cb > rb) continue;   // wholly above the diagonal
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // on the diagonal, row rb*32 + a and column cb*32 + b are the same
          // 64 keys: j < i iff rb > cb, or rb == cb and a > b; j != i iff not
          // (rb == cb and a == b)
          const int a = acc_row(v, lane_v);
          const bool pair_ok = !diag || (sym ? (rb != cb || a != l) : (rb > cb || a > l));
          if (col_ok && pair_ok) mx[rb][v] = fmaxf(mx[rb][v], acc[rb][cb][v] * rc[cb]);
        }
      }
  };

  // 4. diagonal step: wave (0,1) lies above the diagonal (needed only for
  // the symmetric R), (1,0) below it; (0,0) and (1,1) straddle it and mask
  // per element
  if (wave_live && (sym || x.wc <= x.wr)) {
    f32x16_t acc[2][2];
    tile_mma<T>(x.tiles + cur * C::TILE_BYTES, x, af, acc);
    float rc[2];
    const int col0 = base + x.wc * 64 + x.l32;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) rc[cb] = col0 + cb * 32 < N ? rinv[so + col0 + cb * 32] : 0.f;
    if (x.wc != x.wr && base + kK2Cols <= N) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * rc[0], acc[rb][1][v] * rc[1]));
    } else {
      masked_update(acc, rc, col0 - x.l32, x.wc == x.wr);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  cur ^= 1;

  // 5. the other column tiles: 0..blk-1 lie wholly left of the diagonal;
  // tile col_tile(J) is in buffer cur
  const float* rcol = rinv + so + x.wc * 64 + x.l32;
  for (int J = 0; J < ncol; ++J) {
    if (J + 1 < ncol) {
      const int tn = col_tile(J + 1);
      tile_load<T>(p, x, u, N, tn * kK2Cols, cur ^ 1, (tn + 1) * kK2Cols > N);
    } else {
      prefetch_next();
    }
    if (wave_live) {
      const int t = col_tile(J);
      f32x16_t acc[2][2];
      tile_mma<T>(x.tiles + cur * C::TILE_BYTES, x, af, acc);
      if ((t + 1) * kK2Cols <= N) {
        const float r0 = rcol[t * kK2Cols], r1 = rcol[t * kK2Cols + 32];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * r0, acc[rb][1][v] * r1));
      } else {   // the unit's last, partial tile (symmetric R only)
        const int col0 = t * kK2Cols + x.wc * 64;
        float rc[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          rc[cb] = col0 + cb * 32 + x.l32 < N ? rinv[so + col0 + cb * 32 + x.l32] : 0.f;
        masked_update(acc, rc, col0, false);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    cur ^= 1;
  }

  // 6. row maxima. Value j = rb*16 + v of a lane belongs to row
  // rb*32 + acc_row(v, lane); the 32 lanes of a half share rows. The
  // butterfly over lane bits 4..0 leaves lane l with value j = l & 31.
  float val[32];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) val[rb * 16 + v] = mx[rb][v];
  max_butterfly_step<16>(val, x.lane);
  max_butterfly_step<8>(val, x.lane);
  max_butterfly_step<4>(val, x.lane);
  max_butterfly_step<2>(val, x.lane);
  max_butterfly_step<1>(val, x.lane);
  if (wave_live) {
    const int rl = x.wr * 64 + (x.l32 >> 4) * 32 + acc_row(x.l32 & 15, x.lane);   // row in block
    x.comb[x.wc * kK2Rows + rl] = val[0];
  }
  __syncthreads();

  // 7. R, I and Z for the block's rows
  if (x.tid < kK2Rows) {
    const int row = base + x.tid;
    if (row < N) {
      const float m = fmaxf(x.comb[x.tid], x.comb[kK2Rows + x.tid]);
      const float R = (row == 0 && !sym) ? 0.f : m * rinv[so + row];
      const float I = x.imp_l[x.tid];
      const float z = x.lam * I - (1.0f - x.lam) * R;
      // + 0.0f folds -0 onto +0; Z read by another workgroup of this launch
      // is stored coherently at agent scope
      if constexpr (kAgentZ)
        __hip_atomic_store(Z + so + row, z + 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        Z[so + row] = z + 0.0f;
      if (Rdbg != nullptr) Rdbg[so + row] = R;
      if (Idbg != nullptr) Idbg[so + row] = I;
    }
  }
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Persistent kernel over a list of (unit, block) items.
//
// Item order: the paged kernel walks the list statically (item k, k + G,
// ... with G the grid size). The dense kernel, where a workgroup that
// finishes a unit has extra work, claims items from a per-XCD counter
// instead (item 8c + x for the c-th claim on XCD x = blockIdx & 7), so a busy
// workgroup takes fewer items; a static walk would make it the last arrival
// of every unit it touches and load it with all their finishes.
template <typename T, int NQB, class P, bool kFinish, bool kSym>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k2_items_kernel(
    P p, int total_items, const float* __restrict__ rinv, const float* __restrict__ fin,
    float* __restrict__ Z, float* __restrict__ Rdbg, float* __restrict__ Idbg, float lam,
    int rpg_shift, Finish<T> fs) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const K2Lds plan = k2_lds_plan(K2Cfg<T>::RB, p.G * p.W, NQB);
  K2Ctx<T> x;
  x.init(lds, plan, rpg_shift, lam);
  SelectScratch& ssh = *reinterpret_cast<SelectScratch*>(lds + plan.sel);
  int* const words = reinterpret_cast<int*>(lds + plan.sel + sizeof(SelectScratch));  // [3]
  const int stride = gridDim.x;
  const int xcd = blockIdx.x & 7;
  // Item of claim c (dense) or the next valid item at or after k (paged);
  // total_items when there is none.
  auto claimed_item = [&](int c) -> int {
    const int b = 8 * c + xcd;
    int u, blk;
    return (c < total_items && b < total_items && p.k2_item(b, u, blk)) ? b : total_items;
  };
  auto static_item = [&](int k) -> int {
    int u, blk;
    for (; k < total_items; k += stride)
      if (p.k2_item(k, u, blk)) return k;
    return total_items;
  };
  auto decode = [&](int k, int& u, int& blk) {
    p.k2_item(k, u, blk);
    u = __builtin_amdgcn_readfirstlane(u);
    blk = __builtin_amdgcn_readfirstlane(blk);
  };
  int k, kn;
  if constexpr (kFinish) {
    if (x.tid == 0) {
      words[0] = atomicAdd(fs.queue + xcd, 1);
      words[1] = atomicAdd(fs.queue + xcd, 1);
    }
    __syncthreads();
    k = claimed_item(words[0]);
    kn = claimed_item(words[1]);
  } else {
    k = static_item(blockIdx.x);
    kn = static_item(k + stride);
  }
  if (k >= total_items) return;
  int u, blk;
  decode(k, u, blk);
  int N = p.n(u);
  tile_load<T>(p, x, u, N, blk * kK2Rows, 0, true);
  q_load<T>(p, x, u);
  stats_load<NQB>(fin, x, u);
  int cur = 0;
  while (true) {
    Prefetch nx;
    int un = 0, bn = 0;
    nx.valid = kn < total_items;
    if (nx.valid) decode(kn, un, bn);
    nx.u = un;
    nx.n = nx.valid ? p.n(un) : 0;
    nx.first_row = bn * kK2Rows;
    nx.queries = un != u;   // the same unit keeps its queries and normalisers
    k2_block<T, NQB, kFinish, kSym>(p, x, cur, u, N, blk, rinv, nx, fin, Z, Rdbg, Idbg);
    int k_after = total_items;
    if constexpr (kFinish) {
      // Count the block once its scores are stored. The workgroup that
      // brings the count to the unit's number of blocks finishes the unit;
      // nobody waits for anybody. Scores travel through agent-scope
      // (coherent) stores and loads, whose completion s_waitcnt orders before
      // the count, so no cache-wide release or acquire is needed: those
      // would write back and invalidate the L2 that holds the keys.
      // The same round trip claims the item after next.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (x.tid == 0) {
        words[2] = atomicAdd(fs.arrive + u, 1) == p.k2_team(u) - 1;
        if (nx.valid) words[0] = atomicAdd(fs.queue + xcd, 1);
      }
      __syncthreads();
      if (nx.valid) k_after = claimed_item(words[0]);
      if (words[2] && fs.select_units) {
        // The unit's scores and kept indices are staged in the tile buffer
        // that the prefetch left free, when they fit.
        const int Bu = p.budget(u), cand = N - p.W;
        const float* zu = Z + p.score_off(u);
        int32_t* kept = fs.kept + p.kept_off(u);
        char* freebuf = x.tiles + (cur ^ 1) * K2Cfg<T>::TILE_BYTES;
        float* zs = reinterpret_cast<float*>(freebuf);
        int32_t* ks = reinterpret_cast<int32_t*>(freebuf) + cand;
        const bool staged = (int64_t)(cand + Bu) * 4 <= K2Cfg<T>::TILE_BYTES;
        if (staged) {
          stage_scores<256>(zu, cand, zs);
          __syncthreads();
          select_block<256>(zs, N, Bu, p.W, kept, ssh, ks);
        } else {
          select_block<256>(zu, N, Bu, p.W, kept, ssh, nullptr, AgentLoad{});
        }
        __syncthreads();
        const int uu = u;
        gather_rows_block<T, 256>(staged ? ks : kept, Bu, [&](int r) { return p.krow(uu, clamp_row(r, N)); },
                             [&](int r) { return p.vrow(uu, clamp_row(r, N)); }, fs.K_out + (int64_t)u * fs.out_stride,
                             fs.V_out + (int64_t)u * fs.out_stride);
        __syncthreads();   // the staging buffer is a tile buffer again
      }
    } else {
      k_after = static_item(kn + stride);
    }
    if (!nx.valid) break;
    kn = k_after;
    u = un;
    blk = bn;
    N = nx.n;
  }
}

// ---------------------------------------------------------------------------
template <typename T, int NQB, class P>
static hipError_t run_k2_t(const P& p, int k2_items, const float* rinv, const float* fin, float* Z,
                           float* dbg_R, float* dbg_I, float lam, int rpg_shift,
                           const Finish<T>& fs, hipStream_t st) {
  constexpr bool F = P::kFinishUnits;
  const K2Lds plan = k2_lds_plan(Elem<T>::kRowBytes, p.G * p.W, NQB);
  auto kern = p.symmetric() ? k2_items_kernel<T, NQB, P, F, true> : k2_items_kernel<T, NQB, P, F, false>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, plan.total);
  int dev = 0, cus = 0, per_cu = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, plan.total);
  if (e != hipSuccess) return e;
  // persistent grid: a multiple of 8 (one XCD per item, see k2_item), no
  // larger than the work
  const int grid = min(8 * ((max(1, per_cu) * cus + 7) / 8), 8 * ((k2_items + 7) / 8));
  return launch(F ? "rkv_k2_compress" : "rkv_k2_redundancy", kern, dim3(grid), dim3(256),
                plan.total, st, p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs);
}

template <typename T, class P>
hipError_t run_k2(const P& p, int nqb, int k2_items, const float* rinv, const float* fin, float* Z,
                  float* dbg_R, float* dbg_I, float lam, int rpg_shift, int32_t* counters,
                  int32_t* kept, T* K_out, T* V_out, int64_t out_stride, int select_units,
                  hipStream_t st) {
  const Finish<T> fs{counters, counters ? counters + 8 : nullptr, kept, K_out, V_out, out_stride,
                     select_units};
  if (P::kFinishUnits && counters == nullptr) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 4) {
    if (nqb == 1) return run_k2_t<T, 1>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, st);
    return run_k2_t<T, 2>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, st);
  } else {
    switch (nqb) {
      case 1: return run_k2_t<T, 1>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, st);
      case 2: return run_k2_t<T, 2>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, st);
      case 3: return run_k2_t<T, 3>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, st);
      default: return run_k2_t<T, 4>(p, k2_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, st);
    }
  }
}

#define RKV_K2_INST(T, P)                                                                        \
  template hipError_t run_k2<T, P>(const P&, int, int, const float*, const float*, float*, float*, \
                                   float*, float, int, int32_t*, int32_t*, T*, T*, int64_t, int,  \
                                   hipStream_t);
// bf16 caches are scored by k2_wide.hip (dense units that fit a CU's LDS)
// and k2_long.hip (longer dense units, paged caches)
RKV_K2_INST(float, DenseProblem<float>)
RKV_K2_INST(float, PagedProblem<float>)

}  // namespace rkv

// Dense bf16 caches: redundancy, importance, joint score, selection and
// gather in one persistent kernel of 8-wave workgroups.
//
// Same arithmetic as k2_redundancy.hip (pages and readings cited there):
// R_i = max_{j<i} cos(k_i, k_j) on bf16 MFMA with fp32 accumulation and the
// norms applied in the epilogue; I from the window queries' softmax, mean over
// a head's queries, max over the GQA group; Z = lambda*I - (1-lambda)*R; the
// workgroup that completes a unit's last block selects and gathers it.
//
// What differs is the shape, chosen so that the MFMA pipe, not load latency,
// sets the pace:
//  * a work item is a block of 256 rows (two 128-key tiles), held by 8 waves
//    as a 4x2 grid over each 256x128 step: wave (r, c) keeps rows
//    64r..64r+63 of the block as A fragments in registers and multiplies them
//    by columns 64c..64c+63 of the tile (2x2 MFMA 32x32x16 tiles per k-step).
//    Each tile loaded into LDS thus serves 256 rows, and a step is 64 MFMA per
//    SIMD between barriers;
//  * one workgroup per CU, whose LDS holds a ring of S = 4 (or 3, 2) tile
//    slots. Tiles stream through the ring across items: S - 1 tiles are in
//    flight while one is consumed, and a step waits only for its own tile
//    (s_waitcnt vmcnt with the count of loads issued after it);
//  * each slot also holds the 1/||k|| of its 128 rows, loaded with the tile,
//    so the epilogue reads column norms from LDS;
//  * the window queries and softmax normalisers of an item are loaded, into
//    one of two LDS slots, just before the item's first tile;
//  * rows are blocked from the end: with an odd number of 128-row tiles the
//    first item is a single tile (rows 0..127), then pairs, so every other
//    item has 256 live rows. An item with first tile t0 streams its diagonal
//    tile(s) first (they supply the A fragments and need the j < i mask where
//    a wave's rows meet its columns), then tiles 0..t0-1 unmasked.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"

namespace rkv {
namespace wide {

constexpr int kThreads = 512;
constexpr int kRowBytes = 256;                  // bf16 row of 128
constexpr int kNch = 8;                         // 16-byte chunks per half row
constexpr int kTileBytes = 128 * kRowBytes;
constexpr int kSlotBytes = kTileBytes + 512;    // tile + 1/||k|| of its rows
constexpr int kLoadsPerTile = 5;                // per wave: 4 x 1 KiB of tile + 64 B of norms

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int vm_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Wait until at most `tiles_after` tiles' worth of this wave's loads are
// outstanding: every tile issued up to and including the one the step needs
// has landed. Other memory operations only make the wait longer.
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  if (tiles_after <= 0)
    __builtin_amdgcn_s_waitcnt(vm_imm(0));
  else if (tiles_after == 1)
    __builtin_amdgcn_s_waitcnt(vm_imm(kLoadsPerTile));
  else if (tiles_after == 2)
    __builtin_amdgcn_s_waitcnt(vm_imm(2 * kLoadsPerTile));
  else
    __builtin_amdgcn_s_waitcnt(vm_imm(3 * kLoadsPerTile));
}

// Item geometry of a dense unit with nb128 = ceil(N/128) tiles: ni items,
// item i (0 = first claimed, the longest) starts at tile t0 and spans nt tiles.
struct ItemGeo {
  int t0, nt;
};
__device__ __forceinline__ ItemGeo item_geo(int i, int ni, bool odd) {
  const int bi = ni - 1 - i;
  ItemGeo g;
  if (odd) {
    g.t0 = bi == 0 ? 0 : 2 * bi - 1;
    g.nt = bi == 0 ? 1 : 2;
  } else {
    g.t0 = 2 * bi;
    g.nt = 2;
  }
  return g;
}

struct Item {
  int u, t0, nt;
  __device__ int len() const { return nt + t0; }
  // tile streamed at position k of the item: diagonal tile(s) first
  __device__ int tile(int k) const { return k < nt ? t0 + k : k - nt; }
};

// Importance of one key per lane: the lane's key fragments kf (both halves of
// the wave hold the same key). Query rows are padded per head to 2^rpg_shift
// rows; padding rows have zero queries and zero 1/sum.
template <int NQB>
__device__ __forceinline__ float key_importance(const char* qlds, const u32x2_t* slds,
                                                const u32x4_t (&kf)[kNch], int key, int n_u,
                                                int W, int G, int rpg_shift, bool causal,
                                                int lane) {
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
        const u32x2_t st = slds[m];   // (max, 1/sum); read as integers, see slds
        const float pr = fast_exp2(acc[v] * kLogitScaleLog2 - __uint_as_float(st.x)) * __uint_as_float(st.y);
        const float vis = (!causal || key <= n_u - W + (m & rpg_mask)) ? 1.f : 0.f;
        os = fmaf(pr, vis, os);
      }
      os += __shfl_xor(os, 32, 64);
      run += os;
      const int o = qb * 4 + t;
      if (((o + 1) & (octets_per_group - 1)) == 0) {
        if (o / octets_per_group < G) best = fmaxf(best, run * inv_w);
        run = 0.f;
      }
    }
  }
  return best;
}

template <int NQB>
__global__ __launch_bounds__(kThreads, 1) void k2w_kernel(
    DenseProblem<bf16_bits> p, int total_items, const float* __restrict__ rinv,
    const float* __restrict__ fin, float* __restrict__ Z, float* __restrict__ Rdbg,
    float* __restrict__ Idbg, float lam, int rpg_shift, Finish<bf16_bits> fs, WidePlan L) {
  using T = bf16_bits;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int S = L.slots;
  const int N = p.N, W = p.W, G = p.G, gw = G * W;
  const int nb128 = (N + 127) / 128;
  const int ni = (nb128 + 1) / 2;
  const bool odd = (nb128 & 1) != 0;
  const int xcd = blockIdx.x & 7;
  float* const imp_l = reinterpret_cast<float*>(lds + L.imp);
  float* const comb = reinterpret_cast<float*>(lds + L.comb);
  SelectScratch& ssh = *reinterpret_cast<SelectScratch*>(lds + L.sel);
  int* const words = reinterpret_cast<int*>(lds + L.sel + sizeof(SelectScratch));

  // Per-lane constants. Tile load q (0..3) of wave w fills KiB 4w + q of a
  // slot: tile row 16w + 4q + lane/16 at chunk position lane % 16, fetching
  // chunk (lane % 16) ^ (row & 15) of that row.
  int lofs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r16 = (4 * q + lane / 16) & 15;
    lofs[q] = (lane / 16) * kRowBytes + (((lane % 16) ^ r16) << 4);
  }
  int boff[kNch];   // B fragments: tile rows 64*wc + l32 (+32), chunk half*8 + c
#pragma unroll
  for (int c = 0; c < kNch; ++c) boff[c] = frag_offset<T>(wc * 64 + l32, half * kNch + c);

  // claims: item 8c + xcd for the c-th claim on this XCD
  auto decode = [&](int c, Item& it) -> bool {
    const int b = 8 * c + xcd;
    if (c >= total_items || b >= total_items) return false;
    const int k = c;   // per-XCD index
    const int hl = k / ni, i = k - hl * ni;
    it.u = hl * 8 + xcd;
    if (it.u >= p.num_units) return false;
    const ItemGeo g = item_geo(i, ni, odd);
    it.t0 = g.t0;
    it.nt = g.nt;
    it.u = __builtin_amdgcn_readfirstlane(it.u);
    it.t0 = __builtin_amdgcn_readfirstlane(it.t0);
    it.nt = __builtin_amdgcn_readfirstlane(it.nt);
    return true;
  };

  if (tid == 0) {
    words[0] = atomicAdd(fs.queue + xcd, 1);
    words[1] = atomicAdd(fs.queue + xcd, 1);
  }
  __syncthreads();
  Item cur, nxt;
  if (!decode(words[0], cur)) return;
  bool nxt_valid = decode(words[1], nxt);
  int cur_par = 0;   // LDS query / normaliser slot of the current item

  // ---- loader: tiles of cur, then of nxt, into the ring ----
  int ld_which = 0, ld_k = 0;   // position of the next tile to issue
  int issued = 0;               // tiles issued so far
  int issue_slot = 0;           // issued % S
  auto issue_next = [&]() -> bool {
    if (ld_which == 0 && ld_k == cur.len()) {
      ld_which = 1;
      ld_k = 0;
    }
    if (ld_which == 1 && (!nxt_valid || ld_k == nxt.len())) return false;
    const Item& it = ld_which == 0 ? cur : nxt;
    const int par = ld_which == 0 ? cur_par : cur_par ^ 1;
    int lane_v = lane;   // per call: keeps lane-derived values out of the callers' loops
    asm volatile("" : "+v"(lane_v));
    if (ld_k == 0) {   // the item's queries and normalisers, ahead of its first tile
      const char* q = reinterpret_cast<const char*>(p.q(it.u));
      const int qkb = L.qbytes / 1024;
      char* qdst = lds + L.q + par * L.qbytes;
      for (int kb = wave; kb < qkb; kb += 8) {
        const int n = kb * 4 + lane_v / 16;
        const int c = (lane_v % 16) ^ (n & 15);
        load16_to_lds(q + min(n, gw - 1) * kRowBytes + c * 16, qdst + kb * 1024);
      }
      if (wave == 0 && lane_v < NQB * 16)
        load16_to_lds(reinterpret_cast<const char*>(fin) + ((int64_t)it.u * NQB * 32 + 2 * lane_v) * 8,
                      lds + L.stats + par * NQB * 256);
    }
    const int t = it.tile(ld_k);
    char* slot = lds + issue_slot * kSlotBytes;
    const int row0 = t * 128 + wave * 16;                 // first tile row this wave loads
    if ((t + 1) * 128 <= N) {
      const char* src = reinterpret_cast<const char*>(p.krow(it.u, row0));
#pragma unroll
      for (int q = 0; q < 4; ++q) load16_to_lds(src + q * 1024 + lofs[q], slot + wave * 4096 + q * 1024);
    } else {   // last tile of the unit: rows past N repeat row N-1
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = min(row0 + 4 * q + lane_v / 16, N - 1);
        const int chunk_ofs = lofs[q] - (lane_v / 16) * kRowBytes;
        load16_to_lds(reinterpret_cast<const char*>(p.krow(it.u, r)) + chunk_ofs,
                      slot + wave * 4096 + q * 1024);
      }
    }
    if (lane_v < 16)
      __builtin_amdgcn_global_load_lds(rinv + p.score_off(it.u) + min(row0 + lane_v, N - 1),
                                       (__attribute__((address_space(3))) void*)(slot + kTileBytes + wave * 64),
                                       4, 0, 0);
    ++ld_k;
    ++issued;
    issue_slot = issue_slot + 1 == S ? 0 : issue_slot + 1;
    return true;
  };
  auto slot_after = [&](int s0, int d) { return s0 + d >= S ? s0 + d - S : s0 + d; };

  int c = 0;          // tiles consumed
  int cons_slot = 0;  // c % S
  while (issued - c < S && issue_next()) {
  }

  while (true) {
    const int base = cur.t0 * 128;
    const int r_lo = wr * 64;                          // wave's first row within the item
    const bool wave_live = r_lo < cur.nt * 128 && base + r_lo < N;
    const int64_t so = p.score_off(cur.u);
    const char* qlds = lds + L.q + cur_par * L.qbytes;
    // normalisers as (max, 1/sum) bit pairs: a float2 LDS read would make the
    // compiler wait for every direct global->LDS load in flight
    const u32x2_t* slds = reinterpret_cast<const u32x2_t*>(lds + L.stats + cur_par * NQB * 256);

    // 1. the item's diagonal tile(s) have landed
    wait_tiles(issued - (c + cur.nt));
    lds_barrier();
    u32x4_t af[2][kNch];
    // 1/||k|| of the item's rows, for the end of the item (their slots are
    // reused before then)
    float row_rinv = 0.f;
    if (tid < cur.nt * 128)
      row_rinv = reinterpret_cast<const float*>(lds + slot_after(cons_slot, tid >> 7) * kSlotBytes +
                                                kTileBytes)[tid & 127];
    {
      const char* dslot = lds + slot_after(cons_slot, wr >> 1) * kSlotBytes;
      const int arow = (wr & 1) * 64 + l32;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int k = 0; k < kNch; ++k)
          af[rb][k] = ld16(dslot + frag_offset<T>(arow + rb * 32, half * kNch + k));
    }
    // 2. importance of the item's keys: wave (r, c) takes keys 64r + 32c + l32
    if (wave_live) {
      const int key = base + r_lo + wc * 32 + l32;
      const bool causal = base + cur.nt * 128 > N - W;
      const float best = wc == 0
          ? key_importance<NQB>(qlds, slds, af[0], key, N, W, G, rpg_shift, causal, lane)
          : key_importance<NQB>(qlds, slds, af[1], key, N, W, G, rpg_shift, causal, lane);
      if (half == 0) imp_l[r_lo + wc * 32 + l32] = best;
    }
    // 3. keep the ring full
    while (issued - c < S && issue_next()) {
    }

    float mx[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx[rb][v] = -INFINITY;

    // one 64x64 sub-block of the wave against the tile in `slot`; mode 0 =
    // full, 1 = diagonal (rows and columns are the same 64 keys: keep j < i)
    auto step = [&](const char* slot, int mode) {
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
      const float* rn = reinterpret_cast<const float*>(slot + kTileBytes) + wc * 64 + l32;
      const float r0 = rn[0], r1 = rn[32];
      if (mode == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mx[rb][v] = fmaxf(mx[rb][v], fmaxf(acc[rb][0][v] * r0, acc[rb][1][v] * r1));
      } else {
        int lane_v = lane;   // re-materialised: keeps the masks out of loop preheaders
        asm volatile("" : "+v"(lane_v));
        const float rc[2] = {r0, r1};
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
    };

    // 4. diagonal tile(s): columns 128d + 64wc of the item against rows r_lo
    for (int d = 0; d < cur.nt; ++d) {
      const int c_lo = 128 * d + 64 * wc;
      if (wave_live && c_lo <= r_lo) step(lds + slot_after(cons_slot, d) * kSlotBytes, c_lo == r_lo ? 1 : 0);
    }
    c += cur.nt;
    cons_slot = slot_after(cons_slot, cur.nt);

    // 5. tiles 0..t0-1, wholly left of the item's rows
    for (int j = 0; j < cur.t0; ++j) {
      wait_tiles(issued - (c + 1));
      lds_barrier();
      while (issued - c < S && issue_next()) {
      }
      if (wave_live) step(lds + cons_slot * kSlotBytes, 0);
      ++c;
      cons_slot = slot_after(cons_slot, 1);
    }

    // 6. row maxima over the wave's 64 columns; value j = rb*16 + v of a lane
    // belongs to row rb*32 + acc_row(v, lane); lane l ends with value l & 31
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

    // 7. R, I, Z of the item's rows; Z is read by another workgroup of this
    // launch, so it is stored coherently at agent scope
    if (tid < 256) {
      const int row = base + tid;
      if (tid < cur.nt * 128 && row < N) {
        const float m = fmaxf(comb[tid], comb[256 + tid]);
        const float R = row == 0 ? 0.f : m * row_rinv;
        const float I = imp_l[tid];
        const float z = lam * I - (1.0f - lam) * R;
        __hip_atomic_store(Z + so + row, z + 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (Rdbg != nullptr) Rdbg[so + row] = R;
        if (Idbg != nullptr) Idbg[so + row] = I;
      }
    }

    // 8. count the item once its scores are stored (this drains the loads in
    // flight too); the same round trip claims the item after next
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      words[2] = atomicAdd(fs.arrive + cur.u, 1) == ni - 1;
      if (nxt_valid) words[0] = atomicAdd(fs.queue + xcd, 1);
    }
    __syncthreads();
    Item after;
    bool after_valid = false;
    if (nxt_valid) after_valid = decode(words[0], after);
    if (words[2]) {
      // the unit is complete: select its kept indices and gather its rows
      const int B = p.B, cand = N - W;
      const float* zu = Z + so;
      int32_t* kept = fs.kept + p.kept_off(cur.u);
      if (L.stage_bytes > 0) {
        float* zs = reinterpret_cast<float*>(lds + L.stage);
        int32_t* ks = reinterpret_cast<int32_t*>(lds + L.stage) + cand;
        stage_scores<kThreads>(zu, cand, zs);
        __syncthreads();
        select_block<kThreads>(zs, N, B, W, kept, ssh, ks);
        __syncthreads();
        const int u = cur.u;
        gather_rows_block<T, kThreads>(ks, B, [&](int r) { return p.krow(u, r); },
                                       [&](int r) { return p.vrow(u, r); },
                                       fs.K_out + (int64_t)u * fs.out_stride,
                                       fs.V_out + (int64_t)u * fs.out_stride);
      } else {
        select_block<kThreads>(zu, N, B, W, kept, ssh, nullptr, AgentLoad{});
        __syncthreads();
        const int u = cur.u;
        gather_rows_block<T, kThreads>(kept, B, [&](int r) { return p.krow(u, r); },
                                       [&](int r) { return p.vrow(u, r); },
                                       fs.K_out + (int64_t)u * fs.out_stride,
                                       fs.V_out + (int64_t)u * fs.out_stride);
      }
      __syncthreads();   // staging and selection scratch are free again
    }

    if (!nxt_valid) break;
    // advance: the loader's position in nxt becomes its position in cur
    if (ld_which == 1) {
      ld_which = 0;
    } else {
      ld_k = 0;
    }
    cur = nxt;
    cur_par ^= 1;
    nxt = after;
    nxt_valid = after_valid;
    while (issued - c < S && issue_next()) {
    }
  }
}

template <int NQB>
static hipError_t run_t(const DenseProblem<bf16_bits>& p, int total_items, const float* rinv,
                        const float* fin, float* Z, float* dbg_R, float* dbg_I, float lam,
                        int rpg_shift, const Finish<bf16_bits>& fs, const WidePlan& L,
                        hipStream_t st) {
  auto kern = k2w_kernel<NQB>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
  int dev = 0, cus = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // one workgroup per CU, a multiple of 8 (items are tied to XCDs)
  const int grid = min(8 * ((cus + 7) / 8), 8 * ((total_items + 7) / 8));
  return launch("rkv_k2_compress", kern, dim3(grid), dim3(kThreads), L.total, st, p, total_items,
                rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, L);
}

}  // namespace wide

hipError_t run_k2_wide(const DenseProblem<bf16_bits>& p, int nqb, const float* rinv,
                       const float* fin, float* Z, float* dbg_R, float* dbg_I, float lam,
                       int rpg_shift, int32_t* counters, int32_t* kept, bf16_bits* K_out,
                       bf16_bits* V_out, int64_t out_stride, hipStream_t st) {
  if (counters == nullptr) return hipErrorInvalidValue;
  const WidePlan L = wide_plan_choose(p.G * p.W, nqb, p.N - p.W, p.B);
  if (L.total == 0) return hipErrorInvalidValue;
  const Finish<bf16_bits> fs{counters, counters + 8, kept, K_out, V_out, out_stride};
  const int nb128 = (p.N + 127) / 128;
  const int total_items = 8 * ((p.num_units + 7) / 8) * ((nb128 + 1) / 2);
  switch (nqb) {
    case 1: return wide::run_t<1>(p, total_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, L, st);
    case 2: return wide::run_t<2>(p, total_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, L, st);
    case 3: return wide::run_t<3>(p, total_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, L, st);
    default: return wide::run_t<4>(p, total_items, rinv, fin, Z, dbg_R, dbg_I, lam, rpg_shift, fs, L, st);
  }
}

}  // namespace rkv

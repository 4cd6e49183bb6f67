// Dense bf16 caches with units of at most 1152 candidates: the whole
// compression step of a unit in one 8-wave workgroup that reads every key
// from memory once, persistent over units, one workgroup per CU.
//
// Same arithmetic as k1_importance.hip and k2_redundancy.hip (pages and
// readings cited there): softmax of the window queries over the unit's keys
// (query r sees keys j <= N-w+r), mean over a head's w queries, max over the
// GQA group; R_j = max_{i<j} cos(k_i, k_j) on bf16 MFMA with fp32
// accumulation and the norms applied in the epilogue; Z = lambda*I -
// (1-lambda)*R; the window plus the top B-w by (Z desc, index asc),
// ascending; the kept K/V rows gathered.
//
// Shape:
//  * the unit's 128-row key tiles stream once, in order, through a ring of
//    two LDS slots filled by direct global->LDS loads (one tile in flight
//    while one is consumed; the next unit's first tile loads while a unit
//    finishes);
//  * the keys stay: global row block b (32 rows) of tiles 0..nb-2 is held by
//    wave b % 8 in registers as 16x16x32 MFMA fragments (rkv_frag16.hpp).
//    Eight waves of four blocks hold 1024 rows; the unit's last tile is never
//    needed as earlier rows of a later tile and stays in its LDS slot;
//  * when tile t lands, its keys j are the columns: every wave forms the dot
//    products of the rows it holds (i < j) with the tile's 128 keys and keeps,
//    per column, the max of dot * (1/||k_i||); a column's max is the max over
//    the lane's accumulator rows, then over the four lane quarters, then over
//    the eight waves through LDS. R_j = that max * (1/||k_j||), the same
//    products in the same order as a max of cosines;
//  * the owners of tile t's rows copy them into registers with their norms;
//    the same waves form the rows' logits against the window queries (online
//    max and sum of exponentials per query) one step later;
//  * at the end of the unit the importance of every key is formed again from
//    the held fragments (queries as MFMA rows, so a key's weights lie in one
//    lane column and reduce in-lane and over two lane exchanges), then Z,
//    the selection on Z in LDS, and the kept K rows stored from registers,
//    turned into whole rows per store through the wave's part of the V stage
//    (the last tile's from its slot); the kept V rows move during the next unit's
//    tile steps, a slice per step through an LDS stage;
//  * a step's memory instructions are spread over its column loop (one V
//    chunk per column block, the next tile's loads after the first block):
//    issued together right after the step barrier, the eight waves' loads
//    queue at the CU's vector-memory path and hold back the matrix work;
//    and only waves 0-3 load key tiles (8 KiB each): waves 4-7 share each
//    SIMD with one of them and lose the issue arbitration to it.
// Variants: without the causal window the statistics and weights mask only
// padding keys; mean pooling sums the heads' window means and divides by G.
// The symmetric R needs later keys as well and is served by k2_wide.hip.
// Under head-shared selection the kernel stops after writing Z.
#include <type_traits>

#include "rkv_launch.hpp"
#include "rkv_resident.hpp"
#include "rkv_select.hpp"

namespace rkv {
namespace resident {

using namespace frag16;

constexpr int kLoaders = 4;   // waves that load key tiles, 8 KiB each
using stream::vm_imm;

template <int kHeld>
__global__ __launch_bounds__(kThreads, 1) void k2r_kernel(
    DenseProblem<bf16_bits> p, float* __restrict__ Zdbg, float* __restrict__ Rdbg,
    float* __restrict__ Idbg, float lam, float oml, float inv_pool, int rpg_shift,
    int32_t* __restrict__ kept_all, bf16_bits* __restrict__ K_out, bf16_bits* __restrict__ V_out,
    int64_t out_stride, int score_only, ResidentPlan L) {
  static_assert(kHeld == 4, "the runs of held blocks below are written out for four");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = L.slots;
  const int N = p.N, W = p.W, G = p.G, gw = G * W, B = p.B;
  const int nb = (N + 127) / 128;
  const int nh = nb - 1;                        // tiles held in registers
  const int kv_total = (16 * B + kThreads - 1) / kThreads;   // V chunks per thread per unit
  const int kps = (kv_total + nb - 1) / nb;                  // ... per tile step (at most 4)
  const bool causal = p.causal();
  const bool mean = p.pool_mean();
  u32x2_t* const stats = reinterpret_cast<u32x2_t*>(lds + L.stats);   // (max, 1/sum) bits
  float* const sred_m = reinterpret_cast<float*>(lds + L.sred);      // [8][32]
  float* const sred_s = sred_m + 8 * 32;
  float* const rn = reinterpret_cast<float*>(lds + L.rn);            // [nb*128] 1/||k||
  int32_t* const pos = reinterpret_cast<int32_t*>(lds + L.rn);       // after scoring: output row
  float* const zs = reinterpret_cast<float*>(lds + L.zs);            // [nb*128] R, then Z
  int32_t* const ks = reinterpret_cast<int32_t*>(lds + L.ks);        // [B] kept
  float* const part = reinterpret_cast<float*>(lds + L.part);        // [2][8][128]
  float* const dpart = reinterpret_cast<float*>(lds + L.dpart);      // [4][128]
  char* const vstage = lds + L.vstage;                               // [8 waves][4][1 KiB]
  SelectLeanScratch& ssh = *reinterpret_cast<SelectLeanScratch*>(lds + L.sel);


  // Vector-memory instructions this wave has issued (vm), and the count just
  // after each ring slot's tile: waiting for a tile allows exactly the
  // instructions issued after it to stay in flight. Every instruction
  // counted here is issued unconditionally by the whole wave (stores of
  // dropped rows go past the end of their buffer, which discards them);
  // uncounted ones only lengthen a wait.
  int vm = 0, mark0 = 0, mark1 = 0;

  // ---- loader: every unit's tiles once, in order, into the ring ----
  int ld_u = blockIdx.x, ld_par = 0, ld_k = 0;
  int issued = 0, issue_slot = 0;
  // The loader runs at most one unit ahead of the consumer: the window
  // queries of two units share the two query slots.
  int ld_limit = blockIdx.x + 2 * gridDim.x;
  auto issue_next = [&]() -> bool {
    if (ld_u >= p.num_units || ld_u >= ld_limit) return false;
    int lane_v = lane;   // per call: keeps lane-derived values out of the callers' loops
    asm volatile("" : "+v"(lane_v));
    // Only waves 0-3 load tiles (waves 4-7 share each SIMD with them and
    // lose the issue arbitration to the older waves). Tile load q (0..7) of
    // wave w fills KiB 8w + q of a slot: tile row 32w + 4q + lane/16 at
    // chunk position lane % 16, fetching chunk (lane % 16) ^ (row & 15) of
    // that row (the lane offsets repeat every four loads).
    int lofs[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r16 = (4 * q + lane_v / 16) & 15;
      lofs[q] = (lane_v / 16) * kRowBytes + (((lane_v % 16) ^ r16) << 4);
    }
    if (ld_k == 0) {   // the unit's window queries, ahead of its first tile
      const char* qsrc = reinterpret_cast<const char*>(p.q(ld_u));
      const int qkb = L.qbytes / 1024;
      char* qdst = lds + L.q + ld_par * L.qbytes;
      for (int kb = wave; kb < qkb; kb += 8) {
        const int n = kb * 4 + lane_v / 16;
        const int c = (lane_v % 16) ^ (n & 15);
        load16_to_lds(qsrc + min(n, gw - 1) * kRowBytes + c * 16, qdst + kb * 1024);
        ++vm;
      }
    }
    const int t = ld_k;
    char* slot = lds + issue_slot * kTileBytes;
    if (wave < kLoaders) {
      const int row0 = t * 128 + wave * 32;   // first tile row this wave loads
      // the unit's N key rows as a buffer: the tile's row base is a scalar
      // offset, the lane's part a fixed vector offset
      const __amdgpu_buffer_rsrc_t ksrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<bf16_bits*>(p.krow(ld_u, 0)), 0, N * kRowBytes, kBufferWord3);
      if ((t + 1) * 128 <= N) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          load16_to_lds(ksrc, lofs[q & 3], slot + wave * 8192 + q * 1024, row0 * kRowBytes + q * 1024);
      } else {   // last tile of the unit: rows past N repeat row N-1
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = min(row0 + 4 * q + lane_v / 16, N - 1);
          const int chunk_ofs = lofs[q & 3] - (lane_v / 16) * kRowBytes;
          load16_to_lds(ksrc, r * kRowBytes + chunk_ofs, slot + wave * 8192 + q * 1024);
        }
      }
      vm += 8;
    }
    if (issue_slot == 0)
      mark0 = vm;
    else
      mark1 = vm;
    ++issued;
    issue_slot = issue_slot + 1 == S ? 0 : issue_slot + 1;
    if (++ld_k == nb) {
      ld_k = 0;
      ld_u += gridDim.x;
      ld_par ^= 1;
    }
    return true;
  };
  // c = the tile in use; its slot and those of the tiles after it are taken
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

  // R of the keys of tile tt from the column maxima (threads 0..127);
  // with_diag: the last tile, whose own rows left theirs in dpart
  auto finalize = [&](int tt, bool with_diag, int tid_f) {
    const int j = tt * 128 + tid_f;
    if (j < N) {
      const float* pp = part + (tt & 1) * 1024 + tid_f;
      float m = pp[0];
#pragma unroll
      for (int w = 1; w < 8; ++w) m = vmax(m, pp[w * 128]);
      if (with_diag)
        for (int r = 0; r <= (tid_f >> 5); ++r) m = vmax(m, dpart[r * 128 + tid_f]);
      zs[j] = j == 0 ? 0.f : m * rn[j];
    }
  };

  int c = 0, cons_slot = 0;
  int last_u = -1;   // the last unit whose kept V rows are still to move
  refill(0);

  int par = 0;
  for (int u = blockIdx.x; u < p.num_units; u += gridDim.x, par ^= 1) {
    // per unit: keeps lane-derived values from living across units
    int lane_u = lane, tid_u = tid;
    asm volatile("" : "+v"(lane_u), "+v"(tid_u));
    ld_limit = u + 2 * gridDim.x;
    const int64_t so = p.score_off(u);
    const char* qlds = lds + L.q + par * L.qbytes;
    float mrun[2] = {kNoLogit, kNoLogit}, srun[2] = {0.f, 0.f};
    // the kept V rows of this workgroup's previous unit move during this
    // unit's tile steps, kps 16-byte chunks per thread per step
    const int pu = u - (int)gridDim.x;
    const bool vg = !score_only && pu >= (int)blockIdx.x;
    // the previous unit's N value rows as a buffer (bounded reads)
    const __amdgpu_buffer_rsrc_t v_prev = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_bits*>(p.vrow(vg ? pu : 0, 0)), 0, N * kRowBytes, kBufferWord3);
    // (declared per unit: nothing held lives on into the next unit)
    u32x4_t A[kHeld][2][4];   // held row blocks: slot s = row block 8s + wave

    // ---------------- the tile stream: statistics, norms, R ----------------
    for (int t = 0; t < nb; ++t) {
      ensure_issued(c);
      wait_vm(vm - (cons_slot == 0 ? mark0 : mark1));
      lds_barrier();
      const char* slot = lds + cons_slot * kTileBytes;
      // a slice of the previous unit's kept V rows, into this wave's staging
      // (lane order), one chunk per column block of the pair loop below so
      // the loads enter the memory pipeline between the matrix work; stored
      // at the end of the step
      const int nv = vg ? max(0, min(kps, kv_total - t * kps)) : 0;
      auto v_chunk = [&](int j) {
        const int q = (t * kps + j) * kThreads + tid_u;
        const int r = min(q >> 4, B - 1);   // chunks past the end re-read a kept row
        load16_to_lds(v_prev, clamp_row(ks[r], N) * kRowBytes + (q & 15) * 16, vstage + (wave * 4 + j) * 1024);
      };
      vm += nv;
      if (t > 0 && tid_u < 128) finalize(t - 1, false, tid_u);

      // the owner of each of tile t's row blocks copies it into registers
      // (tiles before the last) with its norms; the logits of a held block
      // against the window queries follow one step later, when its owner is
      // not copying, so each step carries half of both
      if (t < nh && (wave >> 2) == (t & 1)) {
        const int key0 = t * 128 + (wave & 3) * 32;
#pragma unroll
        for (int s = 0; s < kHeld; ++s) {
          if (s != (t >> 1)) continue;
          load_frag(slot, (wave & 3) * 32, lane_u, A[s][0]);
          load_frag(slot, (wave & 3) * 32 + 16, lane_u, A[s][1]);
          row_norms(A[s], key0, lane_u, rn);
        }
      }

      // columns: the tile's keys against every held row before them. The
      // blocks wholly before tile t are slots 0..nfull-1, dealt as one
      // straight-line run so that one block's epilogue overlaps the next
      // block's products; the wave's own block of tile t (slot t/2) follows
      // with the diagonal mask.
      const int nfull = min(kHeld, max(0, (4 * t - wave + 7) >> 3));
      const bool has_diag = t < nh && (wave >> 2) == (t & 1);
      // per column block and half: the max over the lane's accumulator rows,
      // reduced over the lane quarters and stored once after the loop
      float cmx[4][2];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) cmx[cb][0] = cmx[cb][1] = -INFINITY;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        // the next tile's loads, after one column block of matrix work (the
        // slot freed at this step's barrier), so the step does not open with
        // every wave queueing memory instructions
        if (cb == 1) refill(c);
        if (cb < nv) v_chunk(cb);
        u32x4_t bf[2][4];
        load_frag(slot, cb * 32, lane_u, bf[0]);
        load_frag(slot, cb * 32 + 16, lane_u, bf[1]);
        float(&cm)[2] = cmx[cb];
        auto full = [&](auto sc) {
          constexpr int s = decltype(sc)::value;
          pair_max(A[s], rn + (8 * s + wave) * 32, bf, false, lane_u, cm);
        };
        switch (nfull) {
          case 4: full(std::integral_constant<int, 0>{}); full(std::integral_constant<int, 1>{});
                  full(std::integral_constant<int, 2>{}); full(std::integral_constant<int, 3>{}); break;
          case 3: full(std::integral_constant<int, 0>{}); full(std::integral_constant<int, 1>{});
                  full(std::integral_constant<int, 2>{}); break;
          case 2: full(std::integral_constant<int, 0>{}); full(std::integral_constant<int, 1>{}); break;
          case 1: full(std::integral_constant<int, 0>{}); break;
          default: break;
        }
        if (has_diag && (wave & 3) <= cb) {
#pragma unroll
          for (int s = 0; s < kHeld; ++s) {
            if (s != (t >> 1)) continue;
            pair_max(A[s], rn + (8 * s + wave) * 32, bf, (wave & 3) == cb, lane_u, cm);
          }
        }
      }
      publish_step(cmx, part + (t & 1) * 1024 + wave * 128, lane_u);
      // statistics of the block this wave copied at step t-1
      if (t >= 1 && t - 1 < nh && (wave >> 2) == ((t - 1) & 1)) {
        const int key0 = (t - 1) * 128 + (wave & 3) * 32;
#pragma unroll
        for (int s = 0; s < kHeld; ++s) {
          if (s != ((t - 1) >> 1)) continue;
          u32x4_t qf[2][4];
          load_queries<false>(qlds, lane_u, W, G, rpg_shift, qf);
          stats_update(A[s], qf, key0, N, W, G, rpg_shift, causal, lane_u, mrun, srun);
        }
      }
      if (nv > 0) {
        __builtin_amdgcn_s_waitcnt(vm_imm(0));   // the wave's V chunks have landed
        asm volatile("" ::: "memory");
        const __amdgpu_buffer_rsrc_t vo = __builtin_amdgcn_make_buffer_rsrc(
            V_out + (int64_t)pu * out_stride, 0, B * kRowBytes, kBufferWord3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j >= nv) continue;
          const int q = (t * kps + j) * kThreads + tid_u;   // chunks past B rows: dropped
          __builtin_amdgcn_raw_buffer_store_b128(ld16(vstage + (wave * 4 + j) * 1024 + lane_u * 16),
                                                 vo, q * 16, 0, kOutPolicy);
        }
        vm += nv;
      }
      if (t < nh) {
        ++c;
        cons_slot = cons_slot + 1 == S ? 0 : cons_slot + 1;
      }
    }

    // ---------------- the last tile's own rows ----------------
    // (lane ids re-materialised: offsets of the step loop do not live on)
    int lane_p = lane_u, tid_p = tid_u;
    asm volatile("" : "+v"(lane_p), "+v"(tid_p));
    const int tl = nb - 1;
    const char* lslot = lds + cons_slot * kTileBytes;
    // norms and logits: wave w takes rows 16w.. of the tile
    {
      u32x4_t kf[1][4];
      load_frag(lslot, wave * 16, lane_p, kf[0]);
      row_norms(kf, tl * 128 + wave * 16, lane_p, rn);
      u32x4_t qf[2][4];
      load_queries<false>(qlds, lane_p, W, G, rpg_shift, qf);
      stats_update(kf, qf, tl * 128 + wave * 16, N, W, G, rpg_shift, causal, lane_p, mrun, srun);
    }
    lds_barrier();
    // the tile's own pairs: row block r against column half (cb, cs) for
    // r <= cb, 20 items dealt round-robin to the 8 waves; rows past N (a copy
    // of row N-1) only meet columns before them, which the diagonal mask
    // drops, or columns past N, which are never read
    for (int it = wave; it < 20; it += 8) {
      // item -> (r, cb, cs): pairs (r, cb) in the order (0,0..3), (1,1..3), ...
      const int pr = it >> 1, cs = it & 1;
      const int r = pr < 4 ? 0 : (pr < 7 ? 1 : (pr < 9 ? 2 : 3));
      const int cb = r + pr - (r == 0 ? 0 : (r == 1 ? 4 : (r == 2 ? 7 : 9)));
      u32x4_t af[2][4], bf[4];
      load_frag(lslot, r * 32, lane_p, af[0]);
      load_frag(lslot, r * 32 + 16, lane_p, af[1]);
      load_frag(lslot, cb * 32 + cs * 16, lane_p, bf);
      float cm = -INFINITY;
      pair_max16(af, rn + tl * 128 + r * 32, bf, cs, cb == r, lane_p, cm);
      const float x = max_quarters(cm);
      if (lane_p < 16) dpart[r * 128 + cb * 32 + cs * 16 + lane_p] = x;
    }
    // statistics of the wave: merge the four lane quarters
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float m = mrun[qs], s = srun[qs];
#pragma unroll
      for (int sh = 16; sh <= 32; sh <<= 1) {
        const LanePair mp = sh == 16 ? pair16(m) : pair32(m);
        const LanePair sp = sh == 16 ? pair16(s) : pair32(s);
        const float mm = fmaxf(mp.lo, mp.hi);
        float st = 0.f;
        if (mm != -INFINITY)
          st = (mp.lo != -INFINITY ? sp.lo * fast_exp2(mp.lo - mm) : 0.f) +
               (mp.hi != -INFINITY ? sp.hi * fast_exp2(mp.hi - mm) : 0.f);
        m = mm;
        s = st;
      }
      if (lane_p < 16) {
        sred_m[wave * 32 + qs * 16 + lane_p] = m;
        sred_s[wave * 32 + qs * 16 + lane_p] = s;
      }
    }
    lds_barrier();
    if (tid_p < 128) {
      finalize(tl, true, tid_p);
    } else if (tid_p < 160) {
      const int m = tid_p - 128;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < 8; ++w) mm = fmaxf(mm, sred_m[w * 32 + m]);
      float st = 0.f;
      if (mm != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const float em = sred_m[w * 32 + m], es = sred_s[w * 32 + m];
          if (em != -INFINITY) st += es * fast_exp2(em - mm);
        }
      }
      // padding query rows (head g >= G or row r >= W) are unseen
      const bool qok = (m >> rpg_shift) < G && (m & ((1 << rpg_shift) - 1)) < W;
      const bool seen = qok && mm != -INFINITY && st > 0.f;
      stats[m] = u32x2_t{__float_as_uint(seen ? mm : 0.f), __float_as_uint(seen ? 1.0f / st : 0.f)};
    }
    lds_barrier();

    // ---------------- importance and Z ----------------
    {
      u32x4_t qf[2][4];
      load_queries(qlds, lane_p, W, G, rpg_shift, qf);
      float smax[2][4], sinv[2][4];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x2_t st = stats[qs * 16 + 4 * (lane_p >> 4) + v];
          smax[qs][v] = __uint_as_float(st.x);
          sinv[qs][v] = __uint_as_float(st.y);
        }
      // importance of every key the wave holds first (independent chains),
      // then Z over R in place
      float Ih[kHeld][2], Il[2] = {0.f, 0.f};
      const bool lown = (wave >> 2) == (tl & 1);   // owns a row block of the last tile
      const int lkey0 = tl * 128 + (wave & 3) * 32;
      // held slots 0..nheld-1, as one straight-line run
      const int nheld = min(kHeld, max(0, (4 * nh - wave + 7) >> 3));
      auto imp = [&](auto sc) {
        constexpr int s = decltype(sc)::value;
#pragma unroll
        for (int rs = 0; rs < 2; ++rs)
          Ih[s][rs] = key_importance16(A[s][rs], qf, smax, sinv, (8 * s + wave) * 32 + rs * 16, N, W,
                                       rpg_shift, causal, mean, inv_pool, lane_p);
      };
      switch (nheld) {
        case 4: imp(std::integral_constant<int, 0>{}); imp(std::integral_constant<int, 1>{});
                imp(std::integral_constant<int, 2>{}); imp(std::integral_constant<int, 3>{}); break;
        case 3: imp(std::integral_constant<int, 0>{}); imp(std::integral_constant<int, 1>{});
                imp(std::integral_constant<int, 2>{}); break;
        case 2: imp(std::integral_constant<int, 0>{}); imp(std::integral_constant<int, 1>{}); break;
        case 1: imp(std::integral_constant<int, 0>{}); break;
        default: break;
      }
      if (lown) {
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
          u32x4_t kf[4];
          load_frag(lslot, (wave & 3) * 32 + rs * 16, lane_p, kf);
          Il[rs] = key_importance16(kf, qf, smax, sinv, lkey0 + rs * 16, N, W, rpg_shift, causal,
                                    mean, inv_pool, lane_p);
        }
      }
      auto put = [&](float I, int key0) {
        const int key = key0 + (lane_p & 15);
        if (lane_p < 16 && key < N) {
          const float R = zs[key];
          const float z = lam * I - oml * R + 0.0f;   // + 0 folds -0 onto +0
          zs[key] = z;
          if (Zdbg != nullptr) Zdbg[so + key] = z;
          if (Rdbg != nullptr) Rdbg[so + key] = R;
          if (Idbg != nullptr) Idbg[so + key] = I;
        }
      };
#pragma unroll
      for (int s = 0; s < kHeld; ++s) {
        const int gb = 8 * s + wave;
        if (gb >= 4 * nh) continue;
        put(Ih[s][0], gb * 32);
        put(Ih[s][1], gb * 32 + 16);
      }
      if (lown) {
        put(Il[0], lkey0);
        put(Il[1], lkey0 + 16);
      }
    }

    // ---------------- selection and gather ----------------
    // (score_only: Z went to Zdbg; a later launch selects for groups of units)
    if (!score_only) {
      __syncthreads();
      // the kept list and every candidate's output row (-1: dropped), in the
      // norms' place
      select_block_lean<kThreads, 3>(zs, N, B, W, ks, pos, ssh);   // N <= 1152
      __syncthreads();
      int32_t* kept = kept_all + p.kept_off(u);
      for (int r = tid_u; r < B; r += kThreads) kept[r] = ks[r];
      // kept K rows held in registers. A fragment gives a row only four
      // lanes (lane quarter q has chunks q + 4*ks), so a store straight from
      // it writes 64-byte pieces of 16 rows; each 16-row half-block goes
      // through this wave's 4 KiB of the V stage instead (chunk c of row r
      // at r*256 + ((c ^ r) & 15)*16: no bank conflicts either way) and
      // leaves as four stores of four whole rows. The stage is the wave's
      // own and LDS operations of a wave run in order: no barrier. Rows
      // that are dropped store past the end of the buffer.
      const __amdgpu_buffer_rsrc_t ko = __builtin_amdgcn_make_buffer_rsrc(
          K_out + (int64_t)u * out_stride, 0, B * kRowBytes, kBufferWord3);
      const int past = B * kRowBytes;
      char* const tst = vstage + wave * 4096;
      const int fr = lane_u & 15, fq = lane_u >> 4;
#pragma unroll
      for (int s = 0; s < kHeld; ++s) {
        const int gb = 8 * s + wave;
        if (gb >= 4 * nh) continue;
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
#pragma unroll
          for (int k = 0; k < 4; ++k) st16(tst + fr * 256 + (((fq + 4 * k) ^ fr) & 15) * 16, A[s][rs][k]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rr = fq + 4 * k;   // row of the half-block; chunk fr
            const int o = pos[gb * 32 + rs * 16 + rr];
            __builtin_amdgcn_raw_buffer_store_b128(ld16(tst + rr * 256 + ((fr ^ rr) & 15) * 16), ko,
                                                   o >= 0 ? o * kRowBytes + fr * 16 : past, 0,
                                                   kOutPolicy);
          }
        }
        vm += 8;
      }
      // kept rows of the last tile, from its slot: sixteen threads per row,
      // four whole rows per store
      {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int x = k * 32 + (tid_u >> 4), ch = tid_u & 15;
          const int i = tl * 128 + x;
          const int o = i < N ? pos[i] : -1;
          __builtin_amdgcn_raw_buffer_store_b128(ld16(lslot + frag_offset<bf16_bits>(x, ch)), ko,
                                                 o >= 0 ? o * kRowBytes + ch * 16 : past, 0,
                                                 kOutPolicy);
        }
        vm += 4;
      }
      last_u = u;
    }
    // release the last tile's slot (the next unit's first barrier orders it)
    ++c;
    cons_slot = cons_slot + 1 == S ? 0 : cons_slot + 1;
  }
  // the last unit's kept V rows: no later unit carries them
  if (last_u >= 0)
    gather_rows_block<bf16_bits, kThreads>(ks, B, [&](int r) { return p.vrow(last_u, clamp_row(r, N)); },
                                           V_out + (int64_t)last_u * out_stride);
}

template <int kHeld>
static hipError_t run_t(const DenseProblem<bf16_bits>& p, float* dbg_Z, float* dbg_R, float* dbg_I,
                        float lam, int rpg_shift, int32_t* kept, bf16_bits* K_out,
                        bf16_bits* V_out, int64_t out_stride, int score_only,
                        const ResidentPlan& L, hipStream_t st) {
  auto kern = k2r_kernel<kHeld>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
  int dev = 0, cus = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = min(cus, p.num_units);   // one workgroup per CU, whole units each
  // 1 - lambda and the pooling scale as arguments: uniform values that stay in
  // scalar registers
  const float oml = 1.0f - lam;
  const float inv_pool = p.pool_mean() ? 1.0f / (float)(p.W * p.G) : 1.0f / (float)p.W;
  return launch("rkv_k2_resident", kern, dim3(grid), dim3(kThreads), L.total, st, p, dbg_Z, dbg_R,
                dbg_I, lam, oml, inv_pool, rpg_shift, kept, K_out, V_out, out_stride, score_only,
                L);
}

}  // namespace resident

bool k2_resident_fits(const DenseProblem<bf16_bits>& p, int nqb) {
  const int nb = (p.N + 127) / 128;
  return nqb == 1 && !p.symmetric() && nb - 1 <= 2 * kResidentHeld &&
         resident_plan(p.N, p.B, p.G * p.W).total > 0;
}

hipError_t run_k2_resident(const DenseProblem<bf16_bits>& p, int nqb, float* dbg_Z, float* dbg_R,
                           float* dbg_I, float lam, int rpg_shift, int32_t* kept,
                           bf16_bits* K_out, bf16_bits* V_out, int64_t out_stride, int score_only,
                           hipStream_t st) {
  if (!k2_resident_fits(p, nqb) || (score_only && dbg_Z == nullptr)) return hipErrorInvalidValue;
  const ResidentPlan L = resident_plan(p.N, p.B, p.G * p.W);
  return resident::run_t<kResidentHeld>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out,
                                        out_stride, score_only, L, st);
}

}  // namespace rkv

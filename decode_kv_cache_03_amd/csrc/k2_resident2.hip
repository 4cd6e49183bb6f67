// Dense bf16 caches with units of 1152 to 2176 candidates (the Qwen-14B
// decode event: budget 2048 + buffer 128): the whole compression step of a
// unit in one 8-wave workgroup, persistent over units, one workgroup per CU,
// with the unit's keys held in registers in two passes of 1024 rows.
//
// Same arithmetic as k2_resident.hip (pages and readings cited in
// k1_importance.hip and k2_redundancy.hip): softmax of the window queries
// over the unit's keys (query r sees keys j <= N-w+r), mean over a head's w
// queries, max over the GQA group; R_j = max_{i<j} cos(k_i, k_j) on bf16
// MFMA with fp32 accumulation and the norms applied in the epilogue;
// Z = lambda*I - (1-lambda)*R; the window plus the top B-w by (Z desc, index
// asc), ascending; the kept K/V rows gathered.
//
// A CU's registers hold 1024 key rows (8 waves x 4 blocks of 32 rows as
// 16x16x32 fragments), so a unit of up to 2176 keys takes two passes over
// its 128-row tiles, each tile streaming through a two-slot LDS ring:
//  * pass 0 holds tiles 0..7 and streams tiles 0..nb-1: the pairs of every
//    held row with every later key. Tiles 0..7 finish their R here; tiles 8..
//    leave a partial column max (rows 0..1023 only, before the 1/||k_j||
//    factor) in the score array. Pass 0 also takes every key's softmax
//    statistics: held blocks from registers one step after their copy, later
//    tiles from LDS, 32 keys per wave of waves 0-3. At its end the
//    statistics are merged and the importance and Z of rows 0..1023 are
//    formed from the fragments.
//  * pass 1 holds tiles 8..nb-2 and streams tiles 8..nb-1: the pairs of those
//    rows with every later key, merged with pass 0's partial maxima. The last
//    tile stays in its slot for its own pairs, as in the one-pass kernel.
//  * the end of the unit is the one-pass kernel's: importance and Z of the
//    rows held now and of the last tile, the selection, and K' rows stored
//    from registers (rows of pass 1, turned into whole rows per store through
//    the wave's part of the stage) and from LDS (the last tile). The kept
//    rows of pass 0 are no longer in registers: they move, with the kept V
//    rows, during the next unit's tile steps (a slice per step through an
//    LDS stage); the last unit's move after the loop.
// Pairs are formed once each (the causal triangle exactly); rows 1024.. are
// read twice, tiles 8.. of a unit within about half a unit's time of each
// other.
// Query windows of up to 48 rows (3 groups of 16: Qwen-14B's 5 query heads
// of 8 window rows) are taken one group at a time.
#include "rkv_launch.hpp"
#include "rkv_resident.hpp"
#include "rkv_select.hpp"

namespace rkv {
namespace resident {

using namespace frag16;
using stream::vm_imm;

// kFast: 8 query rows per head (windows of 5..8) and max pooling, fixed at
// compile time so the pooling steps are straight adds and maxima.
template <int NQG, bool kFast>
__global__ __launch_bounds__(kThreads, 1) void k2r2_kernel(
    DenseProblem<bf16_bits> p, float* __restrict__ Zdbg, float* __restrict__ Rdbg,
    float* __restrict__ Idbg, float lam, float oml, float inv_pool, int rpg_shift_arg,
    int32_t* __restrict__ kept_all, bf16_bits* __restrict__ K_out, bf16_bits* __restrict__ V_out,
    int64_t out_stride, int score_only, Resident2Plan L) {
  constexpr int kHeld = 4;
  constexpr int kPT = kResident2PassTiles;
  constexpr int kPR = kResident2PassRows;
  constexpr int NQ = 16 * NQG;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = L.slots;
  const int N = p.N, W = p.W, G = p.G, gw = G * W, B = p.B;
  const int nb = (N + 127) / 128;               // tiles of a unit (10..17)
  const int nh1 = nb - 1 - kPT;                 // tiles held in pass 1 (1..8)
  const int steps_u = nb + (nb - kPT);          // tile steps of a unit
  // chunks of 16 bytes per thread that move during a unit's steps: the
  // previous unit's B kept V rows and its kept K rows below row 1024
  const int kv_max = (16 * (B + min(B, kPR)) + kThreads - 1) / kThreads;
  const int kps = (kv_max + steps_u - 1) / steps_u;   // per step (at most 4)
  const bool causal = p.causal();
  const bool mean = kFast ? false : p.pool_mean();
  const int rpg_shift = kFast ? 3 : rpg_shift_arg;
  u32x2_t* const stats = reinterpret_cast<u32x2_t*>(lds + L.stats);   // (max, 1/sum) bits
  float* const sred_m = reinterpret_cast<float*>(lds + L.sred);      // [8][NQ]
  float* const sred_s = sred_m + 8 * NQ;
  float* const rn = reinterpret_cast<float*>(lds + L.rn);            // [nb*128] 1/||k||
  int32_t* const pos = reinterpret_cast<int32_t*>(lds + L.rn);       // after scoring: output row
  float* const zs = reinterpret_cast<float*>(lds + L.zs);            // [nb*128] R, then Z
  int32_t* const ks = reinterpret_cast<int32_t*>(lds + L.ks);        // [B] kept
  float* const part = reinterpret_cast<float*>(lds + L.part);        // [2][8][128]
  float* const dpart = reinterpret_cast<float*>(lds + L.dpart);      // [4][128]
  char* const vstage = lds + L.vstage;                               // [8 waves][4][1 KiB]
  int32_t* const nlow_lds = reinterpret_cast<int32_t*>(lds + L.nlow); // kept rows < 1024
  SelectLeanScratch& ssh = *reinterpret_cast<SelectLeanScratch*>(lds + L.sel);

  // Vector-memory instructions this wave has issued (vm), and the count just
  // after each ring slot's tile (as in k2_resident.hip): every counted
  // instruction is issued by the whole wave.
  int vm = 0, mark0 = 0, mark1 = 0;

  // ---- loader: every unit's tile sequence (0..nb-1, then 8..nb-1) ----
  int ld_u = blockIdx.x, ld_par = 0, ld_k = 0;
  int issued = 0, issue_slot = 0;
  int ld_limit = blockIdx.x + 2 * gridDim.x;   // at most one unit ahead (two query slots)
  auto issue_next = [&]() -> bool {
    if (ld_u >= p.num_units || ld_u >= ld_limit) return false;
    int lane_v = lane;   // per call: keeps lane-derived values out of the callers' loops
    asm volatile("" : "+v"(lane_v));
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
    const int t = ld_k < nb ? ld_k : ld_k - nb + kPT;
    char* slot = lds + issue_slot * kTileBytes;
    const int row0 = t * 128 + wave * 16;   // first tile row this wave loads
    // the unit's N key rows as a buffer: the tile's row base is a scalar
    // offset, the lane's part a fixed vector offset
    const __amdgpu_buffer_rsrc_t ksrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_bits*>(p.krow(ld_u, 0)), 0, N * kRowBytes, kBufferWord3);
    if ((t + 1) * 128 <= N) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        load16_to_lds(ksrc, lofs[q], slot + wave * 4096 + q * 1024, row0 * kRowBytes + q * 1024);
    } else {   // last tile of the unit: rows past N repeat row N-1
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = min(row0 + 4 * q + lane_v / 16, N - 1);
        const int chunk_ofs = lofs[q] - (lane_v / 16) * kRowBytes;
        load16_to_lds(ksrc, r * kRowBytes + chunk_ofs, slot + wave * 4096 + q * 1024);
      }
    }
    vm += 4;
    if (issue_slot == 0)
      mark0 = vm;
    else
      mark1 = vm;
    ++issued;
    issue_slot = issue_slot + 1 == S ? 0 : issue_slot + 1;
    if (++ld_k == steps_u) {
      ld_k = 0;
      ld_u += gridDim.x;
      ld_par ^= 1;
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

  // R of the keys of tile tt from the column maxima (threads 0..127).
  // mode 0: final (x 1/||k_j||); 1: pass 0's partial max, raw; 2: final,
  // merged with pass 0's partial. with_diag: the last tile's own pairs.
  auto finalize = [&](int tt, int mode, bool with_diag, int tid_f) {
    const int j = tt * 128 + tid_f;
    if (j < N) {
      const float* pp = part + (tt & 1) * 1024 + tid_f;
      float m = pp[0];
#pragma unroll
      for (int w = 1; w < 8; ++w) m = vmax(m, pp[w * 128]);
      if (with_diag)
        for (int r = 0; r <= (tid_f >> 5); ++r) m = vmax(m, dpart[r * 128 + tid_f]);
      if (mode == 2) m = vmax(m, zs[j]);
      zs[j] = mode == 1 ? m : (j == 0 ? 0.f : m * rn[j]);
    }
  };

  int c = 0, cons_slot = 0;
  int last_u = -1;   // the last unit whose kept rows are still to move
  refill(0);

  int par = 0;
  for (int u = blockIdx.x; u < p.num_units; u += gridDim.x, par ^= 1) {
    int lane_u = lane, tid_u = tid;   // per unit: lane-derived values do not live across units
    asm volatile("" : "+v"(lane_u), "+v"(tid_u));
    ld_limit = u + 2 * gridDim.x;
    const int64_t so = p.score_off(u);
    const char* qlds = lds + L.q + par * L.qbytes;
    float mrun[NQG], srun[NQG];
#pragma unroll
    for (int qs = 0; qs < NQG; ++qs) {
      mrun[qs] = kNoLogit;
      srun[qs] = 0.f;
    }
    // the previous unit's kept V rows, then its kept K rows below row 1024,
    // move during this unit's steps
    const int pu = u - (int)gridDim.x;
    const bool vg = !score_only && pu >= (int)blockIdx.x;
    const int nlow_prev = vg ? __builtin_amdgcn_readfirstlane(*nlow_lds) : 0;
    const int kv_total = vg ? (16 * (B + nlow_prev) + kThreads - 1) / kThreads : 0;
    const __amdgpu_buffer_rsrc_t vo_prev = __builtin_amdgcn_make_buffer_rsrc(
        V_out + (int64_t)(vg ? pu : 0) * out_stride, 0, B * kRowBytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t ko_prev = __builtin_amdgcn_make_buffer_rsrc(
        K_out + (int64_t)(vg ? pu : 0) * out_stride, 0, nlow_prev * kRowBytes, kBufferWord3);
    // the previous unit's N value and key rows as buffers (bounded reads)
    const __amdgpu_buffer_rsrc_t v_prev = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_bits*>(p.vrow(vg ? pu : 0, 0)), 0, N * kRowBytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t k_prev = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_bits*>(p.krow(vg ? pu : 0, 0)), 0, N * kRowBytes, kBufferWord3);
    u32x4_t A[kHeld][2][4];   // held row blocks: slot s = local row block 8s + wave
    int st = 0;               // tile step of the unit

#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int hb = pass * kPT;                 // first held and first streamed tile
      const int nhp = pass == 0 ? kPT : nh1;     // tiles held in this pass
      for (int t = hb; t < nb; ++t, ++st) {
        const int tl = t - hb;
        ensure_issued(c);
        wait_vm(vm - (cons_slot == 0 ? mark0 : mark1));
        lds_barrier();
        const char* slot = lds + cons_slot * kTileBytes;
        // a slice of the previous unit's rows to move, one chunk per column
        // block of the pair loop; a round of 512 chunks is 32 rows, all V
        // rows (list rows 0..B-1) or all K rows (B..), B being a multiple of
        // 32; rows past the list read a kept row again and are dropped at
        // the store
        const int nv = max(0, min(kps, kv_total - st * kps));
        auto v_chunk = [&](int j) {
          const int q = (st * kps + j) * kThreads + tid_u;
          const int r = q >> 4;
          const bool is_v = (st * kps + j) * kThreads < 16 * B;   // uniform
          const int row = is_v ? ks[r] : ks[min(r - B, max(nlow_prev - 1, 0))];
          load16_to_lds(is_v ? v_prev : k_prev, clamp_row(row, N) * kRowBytes + (q & 15) * 16,
                        vstage + (wave * 4 + j) * 1024);
        };
        vm += nv;
        if (t > hb && tid_u < 128) finalize(t - 1, pass == 1 ? 2 : (t - 1 < kPT ? 0 : 1), false, tid_u);

        // the owner of each held row block copies it into registers with its
        // norms; in pass 0 its statistics follow one step later
        const bool owner = tl < nhp && (wave >> 2) == (tl & 1);
        if (owner) {
          const int key0 = t * 128 + (wave & 3) * 32;
#pragma unroll
          for (int s = 0; s < kHeld; ++s) {
            if (s != (tl >> 1)) continue;
            load_frag(slot, (wave & 3) * 32, lane_u, A[s][0]);
            load_frag(slot, (wave & 3) * 32 + 16, lane_u, A[s][1]);
            row_norms(A[s], key0, lane_u, rn);
          }
        }

        // tiles that pass 0 does not hold: the statistics of their keys from
        // the slot, 32 keys per wave of waves 0..3, before their pair loop.
        // Waves w and w + 4 share a SIMD and the older wave w wins its matrix
        // pipe, so waves 4..7 finish their pair loops last: they start them
        // at once, alone on the pipe while waves 0..3 take the exponentials.
        if (pass == 0 && tl >= nhp && wave < 4) {
          u32x4_t kf[2][4];
          load_frag(slot, wave * 32, lane_u, kf[0]);
          load_frag(slot, wave * 32 + 16, lane_u, kf[1]);
          stats_update_groups<2, NQG>(kf, qlds, t * 128 + wave * 32, N, W, G, rpg_shift, causal,
                                      lane_u, mrun, srun);
        }

        // columns: the tile's keys against every held row before them, then
        // the wave's own block of the tile under the diagonal mask
        const int nfull = min(kHeld, max(0, (4 * min(tl, nhp) - wave + 7) >> 3));
        // per column block and half: the max over the lane's accumulator
        // rows, reduced over the lane quarters and stored once after the loop
        float cmx[4][2];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) cmx[cb][0] = cmx[cb][1] = -INFINITY;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          if (cb == 1) refill(c);
          if (cb < nv) v_chunk(cb);
          u32x4_t bf[2][4];
          load_frag(slot, cb * 32, lane_u, bf[0]);
          load_frag(slot, cb * 32 + 16, lane_u, bf[1]);
          float(&cm)[2] = cmx[cb];
          auto full = [&](auto sc) {
            constexpr int s = decltype(sc)::value;
            pair_max(A[s], rn + hb * 128 + (8 * s + wave) * 32, bf, false, lane_u, cm);
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
          if (owner && (wave & 3) <= cb) {
#pragma unroll
            for (int s = 0; s < kHeld; ++s) {
              if (s != (tl >> 1)) continue;
              pair_max(A[s], rn + hb * 128 + (8 * s + wave) * 32, bf, (wave & 3) == cb, lane_u, cm);
            }
          }
        }
        publish_step(cmx, part + (t & 1) * 1024 + wave * 128, lane_u);
        if (pass == 0) {
          // statistics of the block this wave copied at the previous step
          if (tl >= 1 && tl - 1 < nhp && (wave >> 2) == ((tl - 1) & 1)) {
            const int key0 = (t - 1) * 128 + (wave & 3) * 32;
#pragma unroll
            for (int s = 0; s < kHeld; ++s) {
              if (s != ((tl - 1) >> 1)) continue;
              stats_update_groups<2, NQG>(A[s], qlds, key0, N, W, G, rpg_shift, causal, lane_u,
                                          mrun, srun);
            }
          }
        }
        if (nv > 0) {
          __builtin_amdgcn_s_waitcnt(vm_imm(0));   // the wave's chunks have landed
          asm volatile("" ::: "memory");
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j >= nv) continue;
            const int q = (st * kps + j) * kThreads + tid_u;
            const u32x4_t d = ld16(vstage + (wave * 4 + j) * 1024 + lane_u * 16);
            if ((st * kps + j) * kThreads < 16 * B)
              __builtin_amdgcn_raw_buffer_store_b128(d, vo_prev, q * 16, 0, kOutPolicy);
            else
              __builtin_amdgcn_raw_buffer_store_b128(d, ko_prev, (q - 16 * B) * 16, 0, kOutPolicy);
          }
          vm += nv;
        }
        // release the tile: all of pass 0's; pass 1 keeps the unit's last
        if (pass == 0 || t < nb - 1) {
          ++c;
          cons_slot = cons_slot + 1 == S ? 0 : cons_slot + 1;
        }
      }

      if (pass == 0) {
        // ---------------- end of pass 0 ----------------
        int lane_p = lane_u, tid_p = tid_u;
        asm volatile("" : "+v"(lane_p), "+v"(tid_p));
        // statistics: the four lane quarters, then the eight waves
#pragma unroll
        for (int qs = 0; qs < NQG; ++qs) {
          float m = mrun[qs], s = srun[qs];
#pragma unroll
          for (int sh = 16; sh <= 32; sh <<= 1) {
            const LanePair mp = sh == 16 ? pair16(m) : pair32(m);
            const LanePair sp = sh == 16 ? pair16(s) : pair32(s);
            const float mm = fmaxf(mp.lo, mp.hi);
            float sum = 0.f;
            if (mm != -INFINITY)
              sum = (mp.lo != -INFINITY ? sp.lo * fast_exp2(mp.lo - mm) : 0.f) +
                    (mp.hi != -INFINITY ? sp.hi * fast_exp2(mp.hi - mm) : 0.f);
            m = mm;
            s = sum;
          }
          if (lane_p < 16) {
            sred_m[wave * NQ + qs * 16 + lane_p] = m;
            sred_s[wave * NQ + qs * 16 + lane_p] = s;
          }
        }
        lds_barrier();
        if (tid_p < 128) {
          finalize(nb - 1, 1, false, tid_p);   // the last tile's partial column max
        } else if (tid_p < 128 + NQ) {
          const int m = tid_p - 128;
          float mm = -INFINITY;
#pragma unroll
          for (int w = 0; w < 8; ++w) mm = fmaxf(mm, sred_m[w * NQ + m]);
          float sum = 0.f;
          if (mm != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const float em = sred_m[w * NQ + m], es = sred_s[w * NQ + m];
              if (em != -INFINITY) sum += es * fast_exp2(em - mm);
            }
          }
          // padding query rows (head g >= G or row r >= W) are unseen
          const bool qok = (m >> rpg_shift) < G && (m & ((1 << rpg_shift) - 1)) < W;
          const bool seen = qok && mm != -INFINITY && sum > 0.f;
          stats[m] = u32x2_t{__float_as_uint(seen ? mm : 0.f), __float_as_uint(seen ? 1.0f / sum : 0.f)};
        }
        lds_barrier();
        // importance and Z of rows 0..1023 (their R is final)
        float Ih[kHeld][2];
        importance_held<NQG, kHeld>(A, kHeld, 0, wave, qlds, stats, N, W, G, rpg_shift, causal, mean,
                                    inv_pool, lane_p, Ih);
#pragma unroll
        for (int s = 0; s < kHeld; ++s)
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) {
            const int key = (8 * s + wave) * 32 + rs * 16 + (lane_p & 15);
            if (lane_p < 16) {
              const float R = zs[key];
              const float z = lam * Ih[s][rs] - oml * R + 0.0f;   // + 0 folds -0 onto +0
              zs[key] = z;
              if (Zdbg != nullptr) Zdbg[so + key] = z;
              if (Rdbg != nullptr) Rdbg[so + key] = R;
              if (Idbg != nullptr) Idbg[so + key] = Ih[s][rs];
            }
          }
      }
    }

    // ---------------- the last tile's own rows ----------------
    int lane_p = lane_u, tid_p = tid_u;
    asm volatile("" : "+v"(lane_p), "+v"(tid_p));
    const int tl = nb - 1;
    const char* lslot = lds + cons_slot * kTileBytes;
    {
      u32x4_t kf[1][4];
      load_frag(lslot, wave * 16, lane_p, kf[0]);
      row_norms(kf, tl * 128 + wave * 16, lane_p, rn);
    }
    lds_barrier();
    for (int it = wave; it < 20; it += 8) {
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
    lds_barrier();
    if (tid_p < 128) finalize(tl, 2, true, tid_p);
    lds_barrier();

    // ---------------- importance and Z of rows 1024.. ----------------
    {
      const bool lown = (wave >> 2) == (tl & 1);   // takes a row block of the last tile
      const int lkey0 = tl * 128 + (wave & 3) * 32;
      auto put = [&](float I, int key0) {
        const int key = key0 + (lane_p & 15);
        if (lane_p < 16 && key < N) {
          const float R = zs[key];
          const float z = lam * I - oml * R + 0.0f;
          zs[key] = z;
          if (Zdbg != nullptr) Zdbg[so + key] = z;
          if (Rdbg != nullptr) Rdbg[so + key] = R;
          if (Idbg != nullptr) Idbg[so + key] = I;
        }
      };
      // held slots of pass 1: local row blocks 8s + wave below 4 * nh1
      const int nslots = min(kHeld, max(0, (4 * nh1 - wave + 7) >> 3));
      float Ih[kHeld][2];
      importance_held<NQG, kHeld>(A, nslots, kPR, wave, qlds, stats, N, W, G, rpg_shift, causal, mean,
                                  inv_pool, lane_p, Ih);
#pragma unroll
      for (int s = 0; s < kHeld; ++s) {
        if (s >= nslots) continue;
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) put(Ih[s][rs], kPR + (8 * s + wave) * 32 + rs * 16);
      }
      if (lown) {
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
          u32x4_t kf[4];
          load_frag(lslot, (wave & 3) * 32 + rs * 16, lane_p, kf);
          put(key_importance16_groups<NQG>(kf, qlds, stats, lkey0 + rs * 16, N, W, G, rpg_shift,
                                           causal, mean, inv_pool, lane_p),
              lkey0 + rs * 16);
        }
      }
    }

    // ---------------- selection and gather ----------------
    if (!score_only) {
      __syncthreads();
      // the kept list and every candidate's output row (-1: dropped), in the
      // norms' place
      select_block_lean<kThreads, 5>(zs, N, B, W, ks, pos, ssh);   // N <= 2176
      __syncthreads();
      int32_t* kept = kept_all + p.kept_off(u);
      for (int r = tid_u; r < B; r += kThreads) {
        const int kr = ks[r];
        kept[r] = kr;
        // the count of kept rows below 1024 (ascending; the window is above)
        if (kr < kPR && (r + 1 == B || ks[r + 1] >= kPR)) *nlow_lds = r + 1;
      }
      if (tid_u == 0 && ks[0] >= kPR) *nlow_lds = 0;
      // kept K rows of pass 1 from registers: each 16-row half-block turns
      // into whole rows through this wave's 4 KiB of the stage (chunk c of
      // row r at r*256 + ((c ^ r) & 15)*16; the wave's own, its LDS
      // operations in order: no barrier) and leaves as four stores of four
      // rows; dropped rows store past the end
      const __amdgpu_buffer_rsrc_t ko = __builtin_amdgcn_make_buffer_rsrc(
          K_out + (int64_t)u * out_stride, 0, B * kRowBytes, kBufferWord3);
      const int past = B * kRowBytes;
      char* const tst = vstage + wave * 4096;
      const int fr = lane_u & 15, fq = lane_u >> 4;
#pragma unroll
      for (int s = 0; s < kHeld; ++s) {
        const int lb = 8 * s + wave;
        if (lb >= 4 * nh1) continue;
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
#pragma unroll
          for (int k = 0; k < 4; ++k) st16(tst + fr * 256 + (((fq + 4 * k) ^ fr) & 15) * 16, A[s][rs][k]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rr = fq + 4 * k;   // row of the half-block; chunk fr
            const int o = pos[kPR + lb * 32 + rs * 16 + rr];
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
  // the last unit's kept V rows and kept K rows below 1024: no later unit
  // carries them
  if (last_u >= 0) {
    const int nl = __builtin_amdgcn_readfirstlane(*nlow_lds);
    gather_rows_block<bf16_bits, kThreads>(ks, B, [&](int r) { return p.vrow(last_u, clamp_row(r, N)); },
                                           V_out + (int64_t)last_u * out_stride);
    gather_rows_block<bf16_bits, kThreads>(ks, nl, [&](int r) { return p.krow(last_u, clamp_row(r, N)); },
                                           K_out + (int64_t)last_u * out_stride);
  }
}

template <int NQG, bool kFast>
static hipError_t run_t(const DenseProblem<bf16_bits>& p, float* dbg_Z, float* dbg_R, float* dbg_I,
                        float lam, int rpg_shift, int32_t* kept, bf16_bits* K_out,
                        bf16_bits* V_out, int64_t out_stride, int score_only,
                        const Resident2Plan& L, hipStream_t st) {
  auto kern = k2r2_kernel<NQG, kFast>;
  const void* fn = reinterpret_cast<const void*>(kern);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
  int dev = 0, cus = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = min(cus, p.num_units);   // one workgroup per CU, whole units each
  const float oml = 1.0f - lam;
  const float inv_pool = p.pool_mean() ? 1.0f / (float)(p.W * p.G) : 1.0f / (float)p.W;
  return launch("rkv_k2_resident2", kern, dim3(grid), dim3(kThreads), L.total, st, p, dbg_Z, dbg_R,
                dbg_I, lam, oml, inv_pool, rpg_shift, kept, K_out, V_out, out_stride, score_only,
                L);
}

}  // namespace resident

// Query groups of 16 window rows a unit needs (rows per head padded to
// 2^rpg_shift): 2 or 3 are served.
static int resident2_groups(const DenseProblem<bf16_bits>& p, int rpg_shift) {
  const int rows = p.G << rpg_shift;
  return rows <= 32 ? 2 : (rows <= 48 ? 3 : 0);
}

bool k2_resident2_fits(const DenseProblem<bf16_bits>& p, int rpg_shift) {
  const int nb = (p.N + 127) / 128;
  const int nqg = resident2_groups(p, rpg_shift);
  if (p.symmetric() || nqg == 0 || nb < kResident2PassTiles + 2 || nb > 2 * kResident2PassTiles + 1)
    return false;
  if (p.B % 32 != 0 || p.B >= p.N) return false;
  const int steps_u = nb + (nb - kResident2PassTiles);
  const int kv_max = (16 * (p.B + std::min(p.B, kResident2PassRows)) + 511) / 512;
  if ((kv_max + steps_u - 1) / steps_u > 4) return false;   // the V stage holds 4 chunks a thread
  return resident2_plan(p.N, p.B, p.G * p.W, 16 * nqg).total > 0;
}

hipError_t run_k2_resident2(const DenseProblem<bf16_bits>& p, float* dbg_Z, float* dbg_R,
                            float* dbg_I, float lam, int rpg_shift, int32_t* kept,
                            bf16_bits* K_out, bf16_bits* V_out, int64_t out_stride, int score_only,
                            hipStream_t st) {
  if (!k2_resident2_fits(p, rpg_shift) || (score_only && dbg_Z == nullptr)) return hipErrorInvalidValue;
  const int nqg = resident2_groups(p, rpg_shift);
  const Resident2Plan L = resident2_plan(p.N, p.B, p.G * p.W, 16 * nqg);
  const bool fast = rpg_shift == 3 && !p.pool_mean();
  if (nqg == 2)
    return fast ? resident::run_t<2, true>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out,
                                           V_out, out_stride, score_only, L, st)
                : resident::run_t<2, false>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out,
                                            V_out, out_stride, score_only, L, st);
  return fast ? resident::run_t<3, true>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out, V_out,
                                         out_stride, score_only, L, st)
              : resident::run_t<3, false>(p, dbg_Z, dbg_R, dbg_I, lam, rpg_shift, kept, K_out,
                                          V_out, out_stride, score_only, L, st);
}

}  // namespace rkv

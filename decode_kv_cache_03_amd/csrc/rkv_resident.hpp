// Building blocks of the register-resident dense bf16 kernels
// (k2_resident.hip: units of up to 1024 + 128 candidates in one pass;
// k2_resident2.hip: up to 2048 + 128 in two passes): 8 waves hold up to 1024
// key rows as 16x16x32 MFMA fragments while 128-row tiles stream past them
// through an LDS ring.
//
// Arithmetic ("R-KV: Redundancy-aware KV Cache Compression for Reasoning
// Models", atlas.scime.ai summary, "Approach"; sourcepulse summary of R-KV,
// "How It Works"): R_j = max over earlier keys i of cos(k_i, k_j), formed as
// the max of dot(k_i, k_j) * (1/||k_i||) times 1/||k_j||; the softmax
// statistics (running max and sum of exponentials) of the window queries'
// logits q.k/sqrt(128) over the keys.
#pragma once

#include "rkv_problem.hpp"
#include "rkv_stream.hpp"
#include "rkv_frag16.hpp"

namespace rkv {
namespace resident {

using namespace frag16;
using stream::vm_imm;

constexpr int kThreads = 512;
constexpr int kRowBytes = 256;                  // bf16 row of 128
constexpr int kTileBytes = 128 * kRowBytes;
// Cache policy of the K'/V' stores: streaming (non-temporal). K' and V' are
// written once and read by no later step of this call; with whole rows per
// store this measured faster than the default write-back through L2.
constexpr int kOutPolicy = kCachePolicyStream;

// Wait until at most n vector-memory instructions of this wave are in
// flight (n rounded down to a multiple of 4: never a shorter wait).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n <= 0 ? 0 : (n >= 60 ? 15 : n >> 2)) {
    case 0: __builtin_amdgcn_s_waitcnt(vm_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vm_imm(4)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vm_imm(8)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vm_imm(12)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vm_imm(16)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vm_imm(20)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vm_imm(24)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vm_imm(28)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vm_imm(32)); break;
    case 9: __builtin_amdgcn_s_waitcnt(vm_imm(36)); break;
    case 10: __builtin_amdgcn_s_waitcnt(vm_imm(40)); break;
    case 11: __builtin_amdgcn_s_waitcnt(vm_imm(44)); break;
    case 12: __builtin_amdgcn_s_waitcnt(vm_imm(48)); break;
    case 13: __builtin_amdgcn_s_waitcnt(vm_imm(52)); break;
    case 14: __builtin_amdgcn_s_waitcnt(vm_imm(56)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_imm(60)); break;
  }
}

// 1/||k|| of the 16*NK rows of NK fragments, written to rn[key0 + row]
// (rows past N are padding). ||k||^2 of a fragment's 16 rows is the
// diagonal of the fragment's product with itself (A and B fragments of the
// same rows are the same registers), four MFMA instead of a sum of squares
// per lane: lane l holds C[4q + v][l % 16] (q = l / 16), so the lanes with
// (l % 16) / 4 == q hold diagonal element l % 16 in acc[l % 4].
template <int NK>
__device__ __forceinline__ void row_norms(const u32x4_t (&f)[NK][4], int key0, int lane, float* rn) {
  asm volatile("" : "+v"(lane));   // per call: keeps lane-derived masks out of loop preheaders
  const int c = lane & 15;
  const bool on_diag = (c >> 2) == (lane >> 4);
#pragma unroll
  for (int rs = 0; rs < NK; ++rs) {
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) mma16(acc, f[rs][ks], f[rs][ks]);
    const float lo = (c & 1) ? acc[1] : acc[0], hi = (c & 1) ? acc[3] : acc[2];
    const float ss = (c & 2) ? hi : lo;
    if (on_diag) rn[key0 + rs * 16 + c] = ss > 0.f ? __frsqrt_rn(ss) : 0.f;
  }
}

// Online softmax statistics of the window queries over 16*NK keys: lane l
// owns query columns l % 16 and 16 + l % 16 (mrun/srun [qs]).
// The running softmax statistics of one query column start at (kNoLogit, 0)
// and take a block of logits lg[] (masked ones -inf) whose max is mt: the
// max moves to max(m, mt), the sum is rescaled to it and the block's
// exponentials added. kNoLogit is finite and below every logit, so the first
// block rescales a zero sum by exp2 of a very negative number (0) and
// masked logits add exp2(-inf) = 0: the same sum as starting from -inf with
// that case branched around, without a test per update. Padding query
// columns (g >= G or r >= W) accumulate zero logits here; the merge at the
// end of the unit marks them unseen.
constexpr float kNoLogit = -3.40282347e38f;   // -FLT_MAX
template <int NV>
__device__ __forceinline__ void stats_accumulate(const float (&lg)[NV], float mt, float& m, float& s) {
  const float mn = vmax(m, mt);
  float sum = s * fast_exp2(m - mn);
#pragma unroll
  for (int i = 0; i < NV; ++i) sum += fast_exp2(lg[i] - mn);
  s = sum;
  m = mn;
}

template <int NK>
__device__ __forceinline__ void stats_update(const u32x4_t (&kf)[NK][4], const u32x4_t (&qf)[2][4],
                                             int key0, int N, int W, int G, int rpg_shift,
                                             bool causal, int lane, float (&mrun)[2],
                                             float (&srun)[2]) {
  asm volatile("" : "+v"(lane));   // per call: keeps lane-derived masks out of loop preheaders
  const int rpg_mask = (1 << rpg_shift) - 1;
  f32x4_t acc[NK][2];
#pragma unroll
  for (int a = 0; a < NK; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int ksb = 0; ksb < NK; ++ksb)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) mma16(acc[ksb][qs], kf[ksb][ks], qf[qs][ks]);   // C[key][query]
  // the block holds padding or keys that some window query cannot see (a
  // block-uniform test: every other block is seen whole by every query)
  const bool edge = key0 + 16 * NK > (causal ? N - W : N);
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int r = (qs * 16 + (lane & 15)) & rpg_mask;
    const int last = causal ? N - W + r : N - 1;   // last key visible to window query r
    float lg[4 * NK];
    float mt = -INFINITY;
#pragma unroll
    for (int ksb = 0; ksb < NK; ++ksb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = key0 + ksb * 16 + 4 * (lane >> 4) + v;
        float x = acc[ksb][qs][v] * kLogitScaleLog2;
        if (edge) x = key <= last ? x : -INFINITY;
        lg[ksb * 4 + v] = x;
        mt = vmax(mt, x);
      }
    stats_accumulate<4 * NK>(lg, mt, mrun[qs], srun[qs]);
  }
}

// Column maxima of dot(k_i, k_j) * (1/||k_i||) for one 32-row block against
// 32 columns: rows are the block's fragments `af` with the 1/||k|| of the
// lane's accumulator rows in `rr`; `bf` are the columns. `diag`: rows and
// columns are the same 32 keys, and only row < column counts.
__device__ __forceinline__ void pair_max(const u32x4_t (&af)[2][4], const float* rnrow,
                                         const u32x4_t (&bf)[2][4], bool diag, int lane,
                                         float (&cm)[2]) {
  f32x4_t rr[2];
  for (int rs = 0; rs < 2; ++rs) rr[rs] = *reinterpret_cast<const f32x4_t*>(rnrow + rs * 16 + 4 * (lane >> 4));
  f32x4_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) mma16(acc[rs][cs], af[rs][ks], bf[cs][ks]);   // C[row][col]
  if (!diag) {
#pragma unroll
    for (int cs = 0; cs < 2; ++cs)
#pragma unroll
      for (int rs = 0; rs < 2; ++rs)
#pragma unroll
        for (int v = 0; v < 4; ++v) cm[cs] = fmaxf(cm[cs], acc[rs][cs][v] * rr[rs][v]);
  } else {
    int lane_v = lane;   // re-materialised: keeps the masks out of loop preheaders
    asm volatile("" : "+v"(lane_v));
    const int row0 = 4 * (lane_v >> 4), col = lane_v & 15;
#pragma unroll
    for (int cs = 0; cs < 2; ++cs)
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        if (rs > cs) continue;   // every row follows every column
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bool before = rs < cs || row0 + v < col;
          if (before) cm[cs] = vmax(cm[cs], acc[rs][cs][v] * rr[rs][v]);
        }
      }
  }
}

// As pair_max for 16 columns (column half cs of a 32-key block), with the
// row norms read from rnrow.
__device__ __forceinline__ void pair_max16(const u32x4_t (&af)[2][4], const float* rnrow,
                                           const u32x4_t (&bf)[4], int cs, bool diag, int lane,
                                           float& cm) {
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) mma16(acc[rs], af[rs][ks], bf[ks]);
  int lane_v = lane;   // re-materialised: keeps the masks out of loop preheaders
  asm volatile("" : "+v"(lane_v));
  const int row0 = 4 * (lane_v >> 4), col = lane_v & 15;
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    if (diag && rs > cs) continue;   // every row follows every column
    const f32x4_t rr = *reinterpret_cast<const f32x4_t*>(rnrow + rs * 16 + row0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const bool before = !diag || rs < cs || row0 + v < col;
      if (before) cm = vmax(cm, acc[rs][v] * rr[v]);
    }
  }
}

// The column maxima of a whole step stored at once: cm[cb][cs] holds, per
// lane, the max over its four accumulator rows of column cb*32 + cs*16 +
// l%16. A transposing butterfly reduces the eight values over the four lane
// quarters with six lane swaps: a swap of two different registers leaves
// the lower lane of each pair with both copies of the first value and the
// upper lane with both copies of the second, so each swap and max finishes
// two values and the results spread over the lanes. After the 16-lane stage
// (values 2i, 2i+1) and the 32-lane stage, lane l of quarter q holds values
// q and q + 4, the maxima of columns l and 64 + l, stored by every lane.
__device__ __forceinline__ void publish_step(const float (&cm)[4][2], float* dst, int lane) {
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // values 2i and 2i + 1: the two column halves of column block i
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(cm[i][0]), __float_as_uint(cm[i][1]),
                                                    false, false);
    r[i] = vmax(__uint_as_float(s[0]), __uint_as_float(s[1]));
  }
  float o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(r[2 * i]), __float_as_uint(r[2 * i + 1]),
                                                    false, false);
    o[i] = vmax(__uint_as_float(s[0]), __uint_as_float(s[1]));
  }
  dst[lane] = o[0];
  dst[64 + lane] = o[1];
}

// ---- query groups one at a time (windows of up to 48 query rows) ----------
// The window's query rows are MFMA columns (or rows) in groups of 16: row
// m = 16*qs + l%16 of group qs is query row r of head g with
// m = g * 2^rpg_shift + r. Loading one group at a time keeps 16 VGPRs of
// queries live instead of 16 per group.

// Fragment of query group qs: lane l takes query row 16*qs + l%16, chunks
// (l/16) + 4*ks; padding rows (g >= G or r >= W) are zero.
__device__ __forceinline__ void load_query_group(const char* qlds, int lane, int W, int G,
                                                 int rpg_shift, int qs, u32x4_t (&qf)[4]) {
  const int rpg_mask = (1 << rpg_shift) - 1;
  const int m = qs * 16 + (lane & 15);
  const int g = m >> rpg_shift, r = m & rpg_mask;
  const bool ok = g < G && r < W;
  const int n = ok ? g * W + r : 0;
  const int q = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = ok ? ld16(qlds + frag_offset<bf16_bits>(n, q + 4 * ks)) : zero16();
}

// Online softmax statistics of NQG query groups over 16*NK keys (keys as
// MFMA rows): lane l owns query column 16*qs + l%16 of group qs in
// mrun[qs], srun[qs]. Keys past N, and keys a causal window query cannot
// see, are masked.
template <int NK, int NQG>
__device__ __forceinline__ void stats_update_groups(const u32x4_t (&kf)[NK][4], const char* qlds,
                                                    int key0, int N, int W, int G, int rpg_shift,
                                                    bool causal, int lane, float (&mrun)[NQG],
                                                    float (&srun)[NQG]) {
  asm volatile("" : "+v"(lane));   // per call: keeps lane-derived masks out of loop preheaders
  const int rpg_mask = (1 << rpg_shift) - 1;
  const bool edge = key0 + 16 * NK > (causal ? N - W : N);   // as in stats_update
#pragma unroll
  for (int qs = 0; qs < NQG; ++qs) {
    u32x4_t qf[4];
    load_query_group(qlds, lane, W, G, rpg_shift, qs, qf);
    f32x4_t acc[NK];
#pragma unroll
    for (int a = 0; a < NK; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int a = 0; a < NK; ++a) mma16(acc[a], kf[a][ks], qf[ks]);   // C[key][query]
    const int r = (qs * 16 + (lane & 15)) & rpg_mask;
    const int last = causal ? N - W + r : N - 1;   // last key visible to window query r
    float lg[4 * NK];
    float mt = -INFINITY;
#pragma unroll
    for (int a = 0; a < NK; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = key0 + a * 16 + 4 * (lane >> 4) + v;
        float x = acc[a][v] * kLogitScaleLog2;
        if (edge) x = key <= last ? x : -INFINITY;
        lg[a * 4 + v] = x;
        mt = vmax(mt, x);
      }
    stats_accumulate<4 * NK>(lg, mt, mrun[qs], srun[qs]);
  }
}

// Importance of 16 keys key0 + l%16 from their fragments, the query groups
// taken one at a time: weights exp2(logit - max) / sum with the merged
// statistics `stats` ((max, 1/sum) bits per query row), summed over a head's
// rows, combined over heads by max (mean pooling: summed), times inv_pool.
// Query bit b of m = 16*qs + 4*(l/16) + v is a within-head bit when
// b < rpg_shift; groups qs (bits 4 and up) are whole heads unless
// rpg_shift = 5, when the two groups are the two halves of one head.
template <int NQG>
__device__ __forceinline__ float key_importance16_groups(const u32x4_t (&kf)[4], const char* qlds,
                                                         const u32x2_t* stats, int key0, int N,
                                                         int W, int G, int rpg_shift, bool causal,
                                                         bool mean, float inv_pool, int lane) {
  asm volatile("" : "+v"(lane));   // per call: keeps lane-derived masks out of loop preheaders
  const int rpg_mask = (1 << rpg_shift) - 1;
  const int key = key0 + (lane & 15);
  const int q = lane >> 4;
  auto comb = [&](float a, float b, int bit) { return (mean || bit < rpg_shift) ? a + b : vmax(a, b); };
  const bool all_seen = !causal || key0 + 15 <= N - W;
  float res = 0.f;
#pragma unroll
  for (int qs = 0; qs < NQG; ++qs) {
    u32x4_t qf[4];
    load_query_group(qlds, lane, W, G, rpg_shift, qs, qf);
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) mma16(acc, qf[ks], kf[ks]);   // C[query][key]
    float w[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = qs * 16 + 4 * q + v;
      const u32x2_t st = stats[m];
      const float pr = fast_exp2(acc[v] * kLogitScaleLog2 - __uint_as_float(st.x)) * __uint_as_float(st.y);
      w[v] = (all_seen || key <= N - W + (m & rpg_mask)) ? pr : 0.f;
    }
    float x = comb(comb(w[0], w[1], 0), comb(w[2], w[3], 0), 1);
    const LanePair a = pair16(x);
    const LanePair b = pair32(comb(a.lo, a.hi, 2));
    x = comb(b.lo, b.hi, 3);
    res = qs == 0 ? x : comb(res, x, 4);
  }
  return res * inv_pool;
}

// Importance of every key a wave holds: slots 0..nslots-1 of A (two 16-row
// fragments each, keys key_base + (8*s + wave)*32 + 16*rs + l%16), the
// query groups taken in the outer loop so that each group's fragment is
// loaded once and the held fragments' products are independent chains.
// Same weights and combination as key_importance16_groups; I[s][rs] of
// slots past nslots is left unset. Every weight is computed, then masked by
// a multiply, so no exponential sits behind a branch.
template <int NQG, int kHeldSlots>
__device__ __forceinline__ void importance_held(const u32x4_t (&A)[kHeldSlots][2][4], int nslots,
                                                int key_base, int wave, const char* qlds,
                                                const u32x2_t* stats, int N, int W, int G,
                                                int rpg_shift, bool causal, bool mean,
                                                float inv_pool, int lane,
                                                float (&I)[kHeldSlots][2]) {
  asm volatile("" : "+v"(lane));   // per call: keeps lane-derived masks out of loop preheaders
  const int rpg_mask = (1 << rpg_shift) - 1;
  const int q = lane >> 4;
  // 8 rows per head and max pooling: bits 0..2 of the query index are summed
  // (in-lane, then the pair16 exchange), bits 3 and up maxed
  const bool fast = !mean && rpg_shift == 3;
  auto comb = [&](float a, float b, int bit) { return (mean || bit < rpg_shift) ? a + b : vmax(a, b); };
#pragma unroll
  for (int qs = 0; qs < NQG; ++qs) {
    u32x4_t qf[4];
    load_query_group(qlds, lane, W, G, rpg_shift, qs, qf);
    float smax[4], sinv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x2_t st = stats[qs * 16 + 4 * q + v];
      smax[v] = __uint_as_float(st.x);
      sinv[v] = __uint_as_float(st.y);
    }
#pragma unroll
    for (int s = 0; s < kHeldSlots; ++s) {
      if (s >= nslots) continue;
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) mma16(acc, qf[ks], A[s][rs][ks]);   // C[query][key]
        const int key0 = key_base + (8 * s + wave) * 32 + rs * 16;
        const int key = key0 + (lane & 15);
        float w[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) w[v] = fast_exp2(acc[v] * kLogitScaleLog2 - smax[v]) * sinv[v];
        if (causal && key0 + 15 > N - W) {   // keys some window query cannot see
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = qs * 16 + 4 * q + v;
            w[v] *= key <= N - W + (m & rpg_mask) ? 1.f : 0.f;
          }
        }
        float x;
        if (fast) {
          x = (w[0] + w[1]) + (w[2] + w[3]);
          const LanePair a = pair16(x);
          const LanePair b = pair32(a.lo + a.hi);
          x = vmax(b.lo, b.hi);
        } else {
          x = comb(comb(w[0], w[1], 0), comb(w[2], w[3], 0), 1);
          const LanePair a = pair16(x);
          const LanePair b = pair32(comb(a.lo, a.hi, 2));
          x = comb(b.lo, b.hi, 3);
        }
        I[s][rs] = qs == 0 ? x : comb(I[s][rs], x, 4);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kHeldSlots; ++s)
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) I[s][rs] *= inv_pool;
}

}  // namespace resident
}  // namespace rkv

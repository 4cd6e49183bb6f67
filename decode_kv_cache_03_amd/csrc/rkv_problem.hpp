// Where a unit's rows, queries, scores and kept indices live.
//
// A unit is one (sequence, layer, KV head) whose N candidates are scored
// together. Two layouts are served by the same kernels through these
// policies:
//   Dense: unit u has rows K + u*kv_stride + t*128; all units share N and B.
//   Paged: unit u = (s, hk) with s = u / H; row t of the unit lives in page
//          page_table[s][t >> ps_shift] at slot t & (page_size-1); N and B
//          are per sequence. Work items are listed by the host.
#pragma once

#include "rkv_device.hpp"
#include "rkv_select.hpp"

namespace rkv {

constexpr int kK1Keys = 256;   // keys per importance work item (4 waves x 64)
constexpr int kK2Rows = 128;   // rows per redundancy work item (2 row groups of 64)
constexpr int kK2Cols = 128;   // columns per LDS tile of the redundancy kernel (2 groups of 64)

// LDS plan of the redundancy kernel (bytes from the start of its dynamic
// shared memory); the host checks it against the 160 KiB of a CU.
struct K2Lds {
  int tiles;     // 2 tile buffers
  int q;         // window queries of the current unit, G*w rows, swizzled like tiles
  int stats;     // (max, 1/sum) per query row, NQB*32 float2
  int imp;       // importance of the block's 128 keys
  int comb;      // row maxima of the two column-group waves: [2][128] floats
  int sel;       // selection scratch of the unit's last block, then 3 words
  int total;
};

__host__ __device__ inline K2Lds k2_lds_plan(int row_bytes, int gw, int nqb) {
  K2Lds L;
  L.tiles = 0;
  L.q = 2 * kK2Cols * row_bytes;
  const int qkb = (gw * row_bytes + 1023) / 1024;          // whole KiB per direct load
  L.stats = L.q + qkb * 1024;
  L.imp = L.stats + nqb * 32 * 8;
  L.comb = L.imp + kK2Rows * 4;
  L.sel = L.comb + 2 * kK2Rows * 4;
  L.total = L.sel + (int)((sizeof(SelectScratch) + 12 + 15) / 16 * 16);
  return L;
}

constexpr int kLdsBytesPerCU = 160 * 1024;

// LDS plan of the fused dense bf16 kernel (k2_wide.hip): a ring of `slots`
// 128-row bf16 tiles, two slots of window queries, the unit's softmax
// normalisers and their per-wave partials, the unit's 1/||k|| and Z, the
// kept indices, a block's importance and row-max exchange, and selection
// scratch.
struct FusedPlan {
  int slots, q, qbytes, stats, sred, rn, zs, ks, imp, comb, sel, total;
};

__host__ __device__ inline int round16(int64_t x) { return (int)((x + 15) / 16 * 16); }

__host__ __device__ inline FusedPlan fused_plan(int N, int B, int gw, int nqb, int slots) {
  FusedPlan L;
  L.slots = slots;
  L.q = slots * 128 * 256;
  L.qbytes = (gw * 256 + 1023) / 1024 * 1024;
  L.stats = L.q + 2 * L.qbytes;
  L.sred = L.stats + nqb * 32 * 8;
  L.rn = L.sred + 4 * nqb * 32 * 8;
  L.zs = L.rn + round16((int64_t)N * 4);
  L.ks = L.zs + round16((int64_t)N * 4);
  L.imp = L.ks + round16((int64_t)B * 4);
  L.comb = L.imp + 256 * 4;
  L.sel = L.comb + 2 * 256 * 4;
  L.total = L.sel + round16(sizeof(SelectScratch));
  return L;
}

// Deepest ring that fits in a CU's LDS; total = 0 if none does (long units:
// the item-list kernels serve them).
__host__ __device__ inline FusedPlan fused_plan_choose(int N, int B, int gw, int nqb) {
  for (int slots = 4; slots >= 2; --slots) {
    const FusedPlan L = fused_plan(N, B, gw, nqb, slots);
    if (L.total <= kLdsBytesPerCU) return L;
  }
  FusedPlan none = fused_plan(N, B, gw, nqb, 2);
  none.total = 0;
  return none;
}

// LDS plan of the register-resident dense bf16 kernel (k2_resident.hip): a
// ring of `slots` 128-row bf16 tiles, 32 KiB of staging for the previous
// unit's V rows (up to 4 KiB per wave), two slots of window queries, the
// softmax normalisers and their per-wave partials, 1/||k|| (later the output
// row of each candidate) and R then Z over the unit's padded tiles, the kept
// indices, two rounds of per-wave column maxima, the last tile's own column
// maxima, and selection scratch.
struct ResidentPlan {
  int slots, vstage, q, qbytes, stats, sred, rn, zs, ks, part, dpart, sel, total;
};

// Row blocks of 32 keys each wave holds in registers: 8 waves x 4 x 32 =
// 1024 rows, so units of up to 1024 + 128 candidates.
constexpr int kResidentHeld = 4;

__host__ __device__ inline ResidentPlan resident_plan(int N, int B, int gw) {
  ResidentPlan L;
  const int nb = (N + 127) / 128;
  L.slots = 2;
  L.vstage = L.slots * 128 * 256;
  L.q = L.vstage + 32 * 1024;
  L.qbytes = (gw * 256 + 1023) / 1024 * 1024;
  L.stats = L.q + 2 * L.qbytes;
  L.sred = L.stats + 32 * 8;
  L.rn = L.sred + 2 * 8 * 32 * 4;
  L.zs = L.rn + nb * 128 * 4;
  L.ks = L.zs + nb * 128 * 4;
  L.part = L.ks + round16((int64_t)B * 4);
  L.dpart = L.part + 2 * 8 * 128 * 4;
  L.sel = L.dpart + 4 * 128 * 4;
  L.total = L.sel + round16(sizeof(SelectLeanScratch));
  if (L.total > kLdsBytesPerCU) L.total = 0;
  return L;
}

// LDS plan of the two-pass register-resident kernel (k2_resident2.hip): as
// ResidentPlan with nq = 16 * (query groups) window rows, plus one word for
// the count of a unit's kept rows held in the first pass.
struct Resident2Plan {
  int slots, vstage, q, qbytes, stats, sred, rn, zs, ks, part, dpart, sel, nlow, total;
};

// Rows held in registers per pass, and tiles per pass.
constexpr int kResident2PassRows = 1024;
constexpr int kResident2PassTiles = 8;

__host__ __device__ inline Resident2Plan resident2_plan(int N, int B, int gw, int nq) {
  Resident2Plan L;
  const int nb = (N + 127) / 128;
  L.slots = 2;
  L.vstage = L.slots * 128 * 256;
  L.q = L.vstage + 32 * 1024;
  L.qbytes = (gw * 256 + 1023) / 1024 * 1024;
  L.stats = L.q + 2 * L.qbytes;
  L.sred = L.stats + nq * 8;
  L.rn = L.sred + 2 * 8 * nq * 4;
  L.zs = L.rn + nb * 128 * 4;
  L.ks = L.zs + nb * 128 * 4;
  L.part = L.ks + round16((int64_t)B * 4);
  L.dpart = L.part + 2 * 8 * 128 * 4;
  L.sel = L.dpart + 4 * 128 * 4;
  L.nlow = L.sel + round16(sizeof(SelectLeanScratch));
  L.total = L.nlow + 16;
  if (L.total > kLdsBytesPerCU) L.total = 0;
  return L;
}

// Reading variants of a call (bits as in rkv.h): the defaults are R over
// earlier candidates, the causal window and max pooling over the GQA heads.
constexpr uint32_t kVariantSymmetric = 1u;   // R_i over every j != i
constexpr uint32_t kVariantNoCausal = 2u;    // every window query sees all N keys
constexpr uint32_t kVariantPoolMean = 4u;    // mean over the G heads instead of max
constexpr uint32_t kVariantMask = 7u;

struct VariantBits {
  uint32_t variant = 0;
  __host__ __device__ bool symmetric() const { return (variant & kVariantSymmetric) != 0; }
  __host__ __device__ bool causal() const { return (variant & kVariantNoCausal) == 0; }
  __host__ __device__ bool pool_mean() const { return (variant & kVariantPoolMean) != 0; }
};

// Work item of the long-unit kernel (k2_long.hip): rows 512*blk .. of unit
// u, whose n candidates lie at row_base (elements) in contiguous 128-element
// rows, scores at score_off.
struct LongItem {
  int32_t u, blk, n, pad;
  int64_t row_base, score_off;
};

// LDS plan of the long-unit kernel: a ring of `slots` 128-row bf16 tiles with
// the 1/||k|| of their rows, and per item parity the window queries and the
// softmax normalisers.
struct LongPlan {
  int slots, rn, q, qbytes, stats, total;
};

__host__ __device__ inline LongPlan long_plan(int gw, int nqb, int slots) {
  LongPlan L;
  L.slots = slots;
  L.rn = slots * 128 * 256;
  L.q = L.rn + slots * 128 * 4;
  L.qbytes = (gw * 256 + 1023) / 1024 * 1024;
  L.stats = L.q + 2 * L.qbytes;
  L.total = L.stats + 2 * nqb * 32 * 8;
  return L;
}

__host__ __device__ inline LongPlan long_plan_choose(int gw, int nqb) {
  for (int slots = 4; slots >= 2; --slots) {
    const LongPlan L = long_plan(gw, nqb, slots);
    if (L.total <= 160 * 1024) return L;
  }
  LongPlan none = long_plan(gw, nqb, 2);
  none.total = 0;
  return none;
}

// LDS plan of the long-unit kernel's 1024-row form (k2_long.hip, one window
// query block, causal-order R): a ring of `slots` tiles with the 1/||k|| of
// their rows, per item parity the window queries and softmax normalisers, and
// the 1/||k|| and importance of the item's 1024 rows.
struct LongPlanR {
  int slots, rn, q, qbytes, stats, rrn, rim, total;
};

__host__ __device__ inline LongPlanR long_plan_r(int gw) {
  LongPlanR L;
  L.slots = 4;   // two tiles in use, two in flight
  L.rn = L.slots * 128 * 256;
  L.q = L.rn + L.slots * 128 * 4;
  L.qbytes = (gw * 256 + 1023) / 1024 * 1024;
  L.stats = L.q + 2 * L.qbytes;
  L.rrn = L.stats + 2 * 32 * 8;
  L.rim = L.rrn + 1024 * 4;
  L.total = L.rim + 1024 * 4;
  if (L.total > kLdsBytesPerCU) L.total = 0;
  return L;
}

// Rows per work item of the long-unit kernel: 1024 (keys held in registers)
// for one window-query block and the causal-order R, else 512.
__host__ __device__ inline int long_block_rows(int nqb, bool symmetric) {
  return (nqb == 1 && !symmetric) ? 1024 : 512;
}

template <typename T>
struct Finish {
  int32_t* queue;      // [8] items claimed per XCD; cleared by the statistics pass
  int32_t* arrive;     // [units] blocks completed; cleared by the statistics pass
  int32_t* kept;       // [units][B]
  T* K_out;
  T* V_out;
  int64_t out_stride;  // elements between units of K_out / V_out
  int select_units;    // 0: scores only (a later launch selects for groups of units)
};

template <typename T>
struct DenseProblem : VariantBits {
  static constexpr bool kRowsContiguous = true;   // rows of a unit are 128 elements apart
  static constexpr bool kFinishUnits = true;      // the redundancy kernel also selects and gathers
  const T* K;
  const T* V;
  const T* Q;              // [units][G][w][128]
  int64_t kv_stride;       // elements between units of K and V
  int num_units, N, B, G, W;
  int k1_chunks;           // ceil(N / kK1Keys)
  int k2_blocks;           // ceil(N / kK2Rows)

  __device__ int n(int) const { return N; }
  __device__ int budget(int) const { return B; }
  // Row t of unit u, unchecked: tile loads pass rows bounded by construction;
  // rows read from a kept list go through clamp_row first.
  __device__ const T* krow(int u, int t) const { return K + (int64_t)u * kv_stride + (int64_t)t * kD; }
  __device__ const T* vrow(int u, int t) const { return V + (int64_t)u * kv_stride + (int64_t)t * kD; }
  __device__ const T* q(int u) const { return Q + (int64_t)u * G * W * kD; }
  __device__ int64_t score_off(int u) const { return (int64_t)u * N; }
  __device__ int64_t kept_off(int u) const { return (int64_t)u * B; }

  // importance work item -> (unit, chunk); partial-statistics slot
  __device__ bool k1_item(int b, int& u, int& c) const {
    u = b / k1_chunks;
    c = b - u * k1_chunks;
    return u < num_units;
  }
  __device__ int64_t k1_slot(int u, int c) const { return (int64_t)u * k1_chunks + c; }
  __device__ int k1_nchunks(int) const { return k1_chunks; }

  // redundancy work item -> (unit, row block). Workgroups go to the 8 XCDs
  // round-robin by index and the persistent grid is a multiple of 8, so item
  // b runs on XCD b & 7: all blocks of a unit share one XCD and its L2, and
  // consecutive units of an XCD are worked on together by its workgroups.
  // The longest block of a unit comes first.
  __device__ bool k2_item(int b, int& u, int& blk) const {
    const int x = b & 7;
    const int k = b >> 3;
    const int hl = k / k2_blocks;
    const int ib = k - hl * k2_blocks;
    u = hl * 8 + x;
    blk = k2_blocks - 1 - ib;
    return u < num_units;
  }
  __device__ int k2_team(int) const { return k2_blocks; }   // work items of a unit
  __device__ bool select_item(int b, int& u) const {
    u = b;
    return u < num_units;
  }

  // long-unit kernel items of 1 << long_shift rows, in order of decreasing
  // work: block index descending (a block sweeps its own tiles and every tile
  // left of it)
  int long_shift = 9;
  __device__ int long_count() const { return num_units * ((N + (1 << long_shift) - 1) >> long_shift); }
  __device__ LongItem long_item(int k) const {
    const int nb5 = (N + (1 << long_shift) - 1) >> long_shift;
    LongItem it;
    it.blk = nb5 - 1 - k / num_units;
    it.u = k - (k / num_units) * num_units;
    it.n = N;
    it.pad = 0;
    it.row_base = (int64_t)it.u * kv_stride;
    it.score_off = (int64_t)it.u * N;
    return it;
  }
  __device__ const T* long_rows() const { return K; }
  __device__ T* copy_dst(int, int) const { return nullptr; }   // rows are contiguous already
};

template <typename T>
struct PagedProblem : VariantBits {
  static constexpr bool kRowsContiguous = false;
  static constexpr bool kFinishUnits = false;     // selection and in-place compaction run after
  const T* Kp;
  const T* Vp;
  const T* Q;                // [S][H][G][w][128]
  const int32_t* page_table; // [S][maxp]
  int64_t page_stride, head_stride, slot_stride;
  int maxp, num_pages, ps_shift, H, G, W;
  const int32_t* seq_len;    // device [S]
  const int32_t* bud;        // device [S]
  const int64_t* score_base; // device [S]: H * sum_{s'<s} N_s'
  const int64_t* kept_base;  // device [S]: H * sum_{s'<s} min(N_s', B_s')
  const int64_t* k1_base;    // device [S*H]: first partial-statistics slot of each unit
  const int2* k1_list;       // importance work items (unit, chunk)
  int k1_count;
  const int2* k2_list;       // redundancy work items (unit, block); unit -1 = idle
  int k2_count;
  const int32_t* unit_list;  // units with N > B (compaction)
  int unit_count;
  int all_units;             // S * H
  // long-unit kernel: the statistics pass copies each scored unit's keys to
  // contiguous rows Kc + kc_base[u]; items listed by the host in order of
  // decreasing work
  T* Kc = nullptr;
  const int64_t* kc_base = nullptr;
  const LongItem* long_list = nullptr;
  int long_cnt = 0;

  __device__ int n(int u) const { return seq_len[u / H]; }
  __device__ int budget(int u) const { return bud[u / H]; }
  __device__ const T* row_in(const T* pool, int u, int t) const {
    const int s = u / H;
    const int hk = u - s * H;
    // A row past the table reads its last column, and an out-of-range page
    // id reads page 0's slot instead: results for such inputs are undefined,
    // but memory outside the table and the pool is never touched.
    const int col = min(max(t >> ps_shift, 0), maxp - 1);
    int pg = page_table[(int64_t)s * maxp + col];
    pg = (pg >= 0 && pg < num_pages) ? pg : 0;
    return pool + (int64_t)pg * page_stride + (int64_t)hk * head_stride +
           (int64_t)(t & ((1 << ps_shift) - 1)) * slot_stride;
  }
  __device__ const T* krow(int u, int t) const { return row_in(Kp, u, t); }
  __device__ const T* vrow(int u, int t) const { return row_in(Vp, u, t); }
  __device__ const T* q(int u) const { return Q + (int64_t)u * G * W * kD; }
  __device__ int64_t score_off(int u) const {
    const int s = u / H;
    return score_base[s] + (int64_t)(u - s * H) * seq_len[s];
  }
  __device__ int64_t kept_off(int u) const {
    const int s = u / H;
    const int nb = min(seq_len[s], bud[s]);
    return kept_base[s] + (int64_t)(u - s * H) * nb;
  }
  __device__ bool k1_item(int b, int& u, int& c) const {
    if (b >= k1_count) return false;
    const int2 it = k1_list[b];
    u = it.x;
    c = it.y;
    return true;
  }
  __device__ int64_t k1_slot(int u, int c) const { return k1_base[u] + c; }
  __device__ int k1_nchunks(int u) const { return (n(u) + kK1Keys - 1) / kK1Keys; }
  __device__ int k2_team(int u) const { return (n(u) + kK2Rows - 1) / kK2Rows; }
  __device__ bool k2_item(int b, int& u, int& blk) const {
    if (b >= k2_count) return false;
    const int2 it = k2_list[b];
    u = it.x;
    blk = it.y;
    return u >= 0;
  }
  __device__ bool unit_item(int b, int& u) const {
    if (b >= unit_count) return false;
    u = unit_list[b];
    return true;
  }
  // selection visits every unit: those with N <= B get the identity
  __device__ bool select_item(int b, int& u) const {
    u = b;
    return b < all_units;
  }
  __device__ int long_count() const { return long_cnt; }
  // read through the constant address space so that a uniform index gives a
  // scalar load: a vector load here would make the long-unit kernel wait for
  // every tile load in flight
  __device__ LongItem long_item(int k) const {
    typedef const __attribute__((address_space(4))) LongItem* ConstItems;
    const ConstItems l = (ConstItems)long_list + k;
    LongItem it;
    it.u = l->u;
    it.blk = l->blk;
    it.n = l->n;
    it.pad = 0;
    it.row_base = l->row_base;
    it.score_off = l->score_off;
    return it;
  }
  __device__ const T* long_rows() const { return Kc; }
  // where the statistics pass copies row t of unit u (null: no copy)
  __device__ T* copy_dst(int u, int t) const {
    return Kc != nullptr ? Kc + kc_base[u] + (int64_t)t * kD : nullptr;
  }
};

}  // namespace rkv

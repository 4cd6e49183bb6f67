// Block-level selection and row gather, shared by the standalone selection
// kernel and the redundancy kernel, which finishes dense units itself.
//
// Selection: keep the window (last w candidates) and the B-w candidates with
// the largest Z among the other N-w, ties to the smaller index, output
// ascending ("R-KV: decoding-time KV cache compression for reasoning models",
// hysenlabs page, "What the redundancy scoring actually does at decode
// time"; sourcepulse summary of R-KV, "How It Works").
//
// A radix select on the order-preserving 32-bit image of Z (four 8-bit digit
// passes over an LDS histogram) finds the exact k-th largest key T and how
// many keys equal to T are taken; one ordered pass with two block scans then
// writes every candidate above T and the first `take` candidates equal to T,
// in index order, followed by the window. No sort and no N-sized buffer.
#pragma once

#include "rkv_device.hpp"

namespace rkv {

// Shared scratch of select_block: 256 + 16 + 2 uint32.
struct SelectScratch {
  uint32_t hist[256];
  uint32_t scan[16];   // one per wave, up to 1024 threads
  uint32_t digit, above;
};

// Reads of Z: plain loads, or agent-scope coherent loads for scores that
// other workgroups of the same launch wrote with agent-scope stores.
struct PlainLoad {
  __device__ float operator()(const float* p) const { return *p; }
};
struct AgentLoad {
  __device__ float operator()(const float* p) const {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// All NT threads of the block (NT = 256 or 512) call this with the same
// arguments. Requires N > B > W. Writes kept[0..B), and the same indices to
// kept_copy unless it is null.
template <int NT, class LoadZ = PlainLoad>
__device__ __forceinline__ void select_block(const float* __restrict__ z, int N, int B, int W,
                                             int32_t* __restrict__ kept, SelectScratch& sh,
                                             int32_t* __restrict__ kept_copy = nullptr,
                                             LoadZ ldz = LoadZ{}) {
  static_assert(NT >= 256 && NT % 64 == 0, "select_block needs at least 256 threads");
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // keeps thread-derived values from being hoisted into callers' loops
  const int cand = N - W;
  const int k = B - W;
  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cand; i += NT) {
      const uint32_t key = order_key(ldz(z + i));
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t < 256 looks at digit 255-t; inclusive count of keys with digit >= 255-t
    const uint32_t c = tid < 256 ? sh.hist[255 - tid] : 0u;
    uint32_t tot;
    const uint32_t cum = block_inclusive_scan<NT>(c, sh.scan, &tot);
    if (tid < 256 && cum >= remaining && cum - c < remaining) {
      sh.digit = 255u - (uint32_t)tid;
      sh.above = cum - c;
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= 255u << shift;
    remaining -= sh.above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t take_eq = remaining;   // keys equal to T to keep, smallest indices first

  const int per = (cand + NT - 1) / NT;
  const int lo = min(cand, tid * per), hi = min(cand, lo + per);
  uint32_t gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(ldz(z + i));
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_inclusive_scan<NT>(eq, sh.scan, &tot) - eq;
  // this thread's share of the equal keys taken (see select_block_lean on
  // why there is no conditional subtraction)
  const uint32_t take = min(eq, take_eq - min(eq_before, take_eq));
  const uint32_t cnt = gt + take;
  uint32_t pos = block_inclusive_scan<NT>(cnt, sh.scan, &tot) - cnt;
  uint32_t taken = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(ldz(z + i));
    bool keep = key > T;
    if (key == T && taken < take) {
      keep = true;
      ++taken;
    }
    if (keep) {
      kept[pos] = i;
      if (kept_copy != nullptr) kept_copy[pos] = i;
      ++pos;
    }
  }
  for (int r = tid; r < W; r += NT) {
    kept[k + r] = cand + r;
    if (kept_copy != nullptr) kept_copy[k + r] = cand + r;
  }
}

// Shared scratch of select_block_lean: three rotating histograms and the
// per-wave totals of the ordered pass's scan.
struct SelectLeanScratch {
  uint32_t hist[3][256];
  uint32_t wsum[16];
};

// The selection of select_block (same keys, same threshold and tie rule,
// same output) with one workgroup barrier per digit pass instead of six,
// for units whose candidates fit 16-bit counts (N - W < 65536) and at most
// KMAX per thread (N - W <= KMAX * NT):
//  * each thread reads its strided candidates i = wave0 + lane + j*NT once
//    and keeps their order keys in registers for the digit passes;
//  * pass p adds its keys into histogram p % 3 (the lanes of a wave that
//    share the first active lane's digit add with one atomic) and clears
//    histogram (p + 1) % 3 for the next pass, which no wave has read since
//    pass p - 2, before the barrier p; after it, EVERY wave reads the 256
//    counts (lane l: digits 255-4l .. 252-4l), scans them over its lanes and
//    finds the same digit and count above it, so nothing is broadcast;
//  * the ordered pass gives thread t the candidates [t*per, t*per + per),
//    their keys read once for its two sweeps: one block scan of
//    (keys above T) << 16 | (keys equal to T) yields both the thread's output
//    position (above-T keys before it, plus the equal keys taken before it:
//    the first take_eq in index order) and how many of its own equal keys it
//    takes.
// Writes ks[0..B) and pos[i] (output row of candidate i, or -1) for every
// i < N, both in LDS; every index written is bounded ([0, B), [0, N)). The
// caller's barrier after the call publishes them. All NT threads call it
// with the same arguments; sh.hist[0] and [1] are cleared here (one barrier).
// Requires N > B > W.
template <int NT, int KMAX>
__device__ __forceinline__ void select_block_lean(const float* __restrict__ z, int N, int B, int W,
                                                  int32_t* __restrict__ ks, int32_t* __restrict__ pos,
                                                  SelectLeanScratch& sh) {
  static_assert(NT >= 256 && NT % 64 == 0 && NT / 64 <= 16, "256..1024 threads");
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // keeps thread-derived values from being hoisted into callers' loops
  const int lane = tid & 63, wave = tid >> 6;
  const int wave0 = tid - lane;
  const int cand = N - W;
  const int k = B - W;
  uint32_t key[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int i = wave0 + j * NT + lane;
    key[j] = i < cand ? order_key(z[i]) : 0u;
  }
  if (tid < 256) {
    sh.hist[0][tid] = 0u;
    sh.hist[1][tid] = 0u;
  }
  lds_barrier();
  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* const hc = sh.hist[pass % 3];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (wave0 + j * NT >= cand) continue;   // uniform across the wave
      const int i = wave0 + j * NT + lane;
      const bool in = i < cand && (key[j] & mask) == prefix;
      const uint32_t dig = (key[j] >> shift) & 255u;
      const uint64_t act = __ballot(in);
      if (act != 0) {
        const int lead = __builtin_amdgcn_readfirstlane(__ffsll((long long)act) - 1);
        const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)dig, lead) & 255u;
        const uint64_t same = __ballot(in && dig == d0);
        if (lane == lead) atomicAdd(&hc[d0], (uint32_t)__popcll(same));
        if (in && dig != d0) atomicAdd(&hc[dig], 1u);
      }
    }
    if (pass >= 1 && pass < 3 && tid < 256) sh.hist[(pass + 1) % 3][tid] = 0u;
    lds_barrier();
    // every wave: the count of keys at or above each digit, from the top
    const u32x4_t h = *reinterpret_cast<const u32x4_t*>(hc + 252 - 4 * lane);
    const uint32_t c[4] = {h.w, h.z, h.y, h.x};
    const uint32_t sum = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_inclusive_scan(sum);
    uint32_t cum = incl - sum, dsel = 0u, abv = 0u;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!found && cum + c[j] >= remaining) {
        found = true;
        dsel = (uint32_t)(255 - 4 * lane - j);
        abv = cum;
      }
      cum += c[j];
    }
    found = found && incl - sum < remaining;
    const uint64_t fb = __ballot(found);
    const int fl = fb != 0 ? __builtin_amdgcn_readfirstlane(__ffsll((long long)fb) - 1) : 0;
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane((int)dsel, fl) & 255u;
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)abv, fl);
    prefix |= digit << shift;
    mask |= 255u << shift;
    remaining = remaining > above ? remaining - above : 0u;
  }
  const uint32_t T = prefix;
  const uint32_t take_eq = remaining;   // keys equal to T to keep, smallest indices first
  const int per = (cand + NT - 1) / NT;   // at most KMAX
  const int lo = min(cand, tid * per), hi = min(cand, lo + per);
  uint32_t ckey[KMAX];
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int i = lo + j;
    ckey[j] = i < hi ? order_key(z[i]) : 0u;
    gt += i < hi && ckey[j] > T;
    eq += i < hi && ckey[j] == T;
  }
  const uint32_t packed = (gt << 16) | eq;
  const uint32_t incl = wave_inclusive_scan(packed);
  if (lane == 63) sh.wsum[wave] = incl;
  lds_barrier();
  // the totals of the waves before this one (every wave's entry is read, the
  // later ones masked, so the reads do not wait on each other)
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) before += w < wave ? sh.wsum[w] : 0u;
  const uint32_t excl = before + incl - packed;
  // equal keys taken by the threads before this one (the first take_eq in
  // index order), then this thread's share; take_eq - taken_before cannot
  // wrap. (Written without a conditional subtraction: the optimizer turned
  // `take_eq > eq_before ? take_eq - eq_before : 0` into an unconditional
  // no-wrap subtraction and then dropped the min below as redundant.)
  const uint32_t taken_before = min(excl & 0xffffu, take_eq);
  uint32_t p = (excl >> 16) + taken_before;
  const uint32_t take = min(eq, take_eq - taken_before);
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int i = lo + j;
    if (i >= hi) continue;
    bool keep = ckey[j] > T;
    if (ckey[j] == T && taken < take) {
      keep = true;
      ++taken;
    }
    const bool ok = keep && p < (uint32_t)k;
    if (ok) ks[p] = i;
    pos[i] = ok ? (int)p : -1;
    p += keep;
  }
  for (int r = tid; r < W; r += NT) {
    ks[k + r] = cand + r;
    pos[cand + r] = k + r;
  }
}

// zs[0..n) = z[0..n) through agent-scope coherent loads, 8 in flight per
// thread (z written by other workgroups of the same launch; zs in LDS).
template <int NT>
__device__ __forceinline__ void stage_scores(const float* __restrict__ z, int n, float* zs) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const AgentLoad ld;
  for (int i0 = 0; i0 < n; i0 += NT * 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * NT + tid;
      v[j] = i < n ? ld(z + i) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * NT + tid;
      if (i < n) zs[i] = v[j];
    }
  }
}

// Copy rows kept[0..nkeep) of two row sources into consecutive output rows, as
// 16-byte chunks, in rounds of U chunks of each tensor per thread (a caller
// whose registers are free at that point takes more per round: the copy is
// bounded by the bytes a CU keeps in flight). Rounds are
// software-pipelined two deep: the loads of round r+1 are in flight while
// round r is stored. Output chunk q sits at byte 16q, so the stores are
// buffer stores with one per-thread offset and a uniform per-chunk offset:
// no per-store address registers, whose reuse would make each store wait for
// the one before. V rows and the outputs are touched once, so they are loaded
// and stored as streaming (non-temporal) accesses that do not displace cached
// keys; K rows are usually still cached from scoring and are read normally.
// Branch-free tails: chunks past the end read row kept[0] again and their
// stores fall outside the buffer range, which drops them.
template <typename T, int NT, class SrcK, class SrcV, int U = 8>
__device__ __forceinline__ void gather_rows_block(const int32_t* __restrict__ kept, int nkeep,
                                                  SrcK srck, SrcV srcv, T* __restrict__ K_out,
                                                  T* __restrict__ V_out) {
  constexpr int RC = Elem<T>::kRowChunks;
  constexpr int kRound = NT * U;   // chunks per round
  const int total = nkeep * RC;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // keeps thread-derived values from being hoisted into callers' loops
  const __amdgpu_buffer_rsrc_t ko = __builtin_amdgcn_make_buffer_rsrc(K_out, 0, total * 16, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vo = __builtin_amdgcn_make_buffer_rsrc(V_out, 0, total * 16, kBufferWord3);
  auto load_round = [&](int q0, u32x4_t (&kv)[U], u32x4_t (&vv)[U]) {
    int src[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int q = q0 + j * NT + tid;
      src[j] = kept[q < total ? q / RC : 0];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = (q0 + j * NT + tid) % RC;
      kv[j] = ld16(reinterpret_cast<const char*>(srck(src[j])) + 16 * c);
      vv[j] = ld16_stream(reinterpret_cast<const char*>(srcv(src[j])) + 16 * c);
    }
  };
  auto store_round = [&](int q0, const u32x4_t (&kv)[U], const u32x4_t (&vv)[U]) {
    const int vofs = (q0 + tid) * 16;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      __builtin_amdgcn_raw_buffer_store_b128(kv[j], ko, vofs, j * NT * 16, kCachePolicyStream);
      __builtin_amdgcn_raw_buffer_store_b128(vv[j], vo, vofs, j * NT * 16, kCachePolicyStream);
    }
  };
  u32x4_t ka[U], va[U], kb[U], vb[U];
  if (total > 0) load_round(0, ka, va);
  for (int q0 = 0; q0 < total; q0 += 2 * kRound) {
    if (q0 + kRound < total) load_round(q0 + kRound, kb, vb);
    store_round(q0, ka, va);
    if (q0 + kRound >= total) break;
    if (q0 + 2 * kRound < total) load_round(q0 + 2 * kRound, ka, va);
    store_round(q0 + kRound, kb, vb);
  }
}

// One row source: rows kept[0..nkeep) into consecutive output rows, in rounds
// of U 16-byte chunks per thread, two rounds in flight, streaming loads and
// stores, branch-free tails (as gather_rows_block).
template <typename T, int NT, class Src>
__device__ __forceinline__ void gather_rows_block(const int32_t* __restrict__ kept, int nkeep,
                                                  Src src, T* __restrict__ out) {
  constexpr int RC = Elem<T>::kRowChunks;
  constexpr int U = 8;
  constexpr int kRound = NT * U;   // chunks per round
  const int total = nkeep * RC;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // keeps thread-derived values from being hoisted into callers' loops
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(out, 0, total * 16, kBufferWord3);
  auto load_round = [&](int q0, u32x4_t (&vv)[U]) {
    int row[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int q = q0 + j * NT + tid;
      row[j] = kept[q < total ? q / RC : 0];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = (q0 + j * NT + tid) % RC;
      vv[j] = ld16_stream(reinterpret_cast<const char*>(src(row[j])) + 16 * c);
    }
  };
  auto store_round = [&](int q0, const u32x4_t (&vv)[U]) {
    const int ofs = (q0 + tid) * 16;
#pragma unroll
    for (int j = 0; j < U; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(vv[j], ro, ofs, j * NT * 16, kCachePolicyStream);
  };
  u32x4_t a[U], b[U];
  if (total > 0) load_round(0, a);
  for (int q0 = 0; q0 < total; q0 += 2 * kRound) {
    if (q0 + kRound < total) load_round(q0 + kRound, b);
    store_round(q0, a);
    if (q0 + kRound >= total) break;
    if (q0 + 2 * kRound < total) load_round(q0 + 2 * kRound, a);
    store_round(q0 + kRound, b);
  }
}

}  // namespace rkv

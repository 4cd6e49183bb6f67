// Compaction of the kept rows, and page return.
//
// Pages: the cache is physically evicted rather than masked, so the freed
// blocks go back to the allocator ("R-KV: decoding-time KV cache compression
// for reasoning models", hysenlabs page, "What the redundancy scoring actually
// does at decode time" and "How this differs from attention-sink and
// heavy-hitter eviction"); one port compacts in two phases (same page, same
// section).
//
// Dense: out of place, K_out[r] = K[kept[r]] and V_out[r] = V[kept[r]], as
// bit copies in 16-byte chunks; each workgroup moves 64 rows of K and V.
//
// Every row moved is read once and written once: loads and stores are
// streaming (non-temporal) in both.
//
// Paged: in place, one workgroup per (sequence, head). Kept indices ascend,
// so kept[r] >= r: slot r's source never lies before slot r. Slots are
// processed in chunks of 128 in ascending order, each in two phases: every
// thread first loads all of the chunk's moved rows into registers (and waits
// for them), the workgroup synchronises, then the rows are stored. Sources of
// later chunks lie at or after their slots, beyond this chunk, so no store
// ever overwrites a row that is still to be read, and no scratch buffer or
// second pass over HBM is needed. Rows with kept[r] == r are not touched.
// A separate launch then truncates the page table and appends the freed page
// ids to the free list at offsets the host computed from N_s and B_s.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"

namespace rkv {

template <typename T>
__global__ __launch_bounds__(256) void k5_gather_kernel(DenseProblem<T> p,
                                                        const int32_t* __restrict__ kept_all,
                                                        T* __restrict__ K_out, T* __restrict__ V_out,
                                                        int64_t out_stride, int nkeep, int tiles) {
  constexpr int RC = Elem<T>::kRowChunks;
  constexpr int PER = 64 * RC / 256;
  const int u = blockIdx.x / tiles;
  const int r0 = (blockIdx.x - u * tiles) * 64;
  if (u >= p.num_units) return;
  const int32_t* kept = kept_all + p.kept_off(u);
  const int tid = threadIdx.x;
  u32x4_t kv[PER], vv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = i * 256 + tid;
    const int r = r0 + q / RC, c = q % RC;
    if (r < nkeep) {
      const int src = clamp_row(kept[r], p.N);
      kv[i] = ld16_stream(reinterpret_cast<const char*>(p.krow(u, src)) + 16 * c);
      vv[i] = ld16_stream(reinterpret_cast<const char*>(p.vrow(u, src)) + 16 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = i * 256 + tid;
    const int r = r0 + q / RC, c = q % RC;
    if (r < nkeep) {
      const int64_t off = (int64_t)u * out_stride + (int64_t)r * kD;
      __builtin_nontemporal_store(kv[i], reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(K_out + off) + 16 * c));
      __builtin_nontemporal_store(vv[i], reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(V_out + off) + 16 * c));
    }
  }
}

template <typename T>
hipError_t run_k5_dense(const DenseProblem<T>& p, const int32_t* kept, T* K_out, T* V_out,
                        int64_t out_stride, int nkeep, hipStream_t st) {
  const int tiles = (nkeep + 63) / 64;
  return launch("rkv_k5_gather", k5_gather_kernel<T>, dim3(p.num_units * tiles), dim3(256), 0, st,
                p, kept, K_out, V_out, out_stride, nkeep, tiles);
}

template hipError_t run_k5_dense<bf16_bits>(const DenseProblem<bf16_bits>&, const int32_t*, bf16_bits*, bf16_bits*, int64_t, int, hipStream_t);
template hipError_t run_k5_dense<float>(const DenseProblem<float>&, const int32_t*, float*, float*, int64_t, int, hipStream_t);

// Row pointer for writing (the problem policy hands out const rows).
template <typename T>
__device__ __forceinline__ char* wrow(const PagedProblem<T>& p, T* pool, int u, int t) {
  const T* r = p.row_in(pool, u, t);
  return reinterpret_cast<char*>(pool) + (reinterpret_cast<const char*>(r) -
                                          reinterpret_cast<const char*>(pool));
}

template <typename T>
__global__ __launch_bounds__(256) void k5_paged_kernel(PagedProblem<T> p, T* Kp, T* Vp,
                                                       const int32_t* __restrict__ kept_all) {
  constexpr int RC = Elem<T>::kRowChunks;
  constexpr int CH = 128;                 // slots per chunk
  constexpr int PER = CH * RC / 256;
  int u;
  if (!p.unit_item(blockIdx.x, u)) return;
  const int N = p.n(u);
  const int B = p.budget(u);
  if (N <= B) return;
  const int32_t* kept = kept_all + p.kept_off(u);
  const int tid = threadIdx.x;
  for (int c0 = 0; c0 < B; c0 += CH) {
    u32x4_t kv[PER], vv[PER];
    int src[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = i * 256 + tid;
      const int r = c0 + q / RC, c = q % RC;
      src[i] = (r < B) ? clamp_row(kept[r], N) : r;
      if (src[i] != r) {
        kv[i] = ld16_stream(reinterpret_cast<const char*>(p.krow(u, src[i])) + 16 * c);
        vv[i] = ld16_stream(reinterpret_cast<const char*>(p.vrow(u, src[i])) + 16 * c);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);        // this chunk's loads have landed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = i * 256 + tid;
      const int r = c0 + q / RC, c = q % RC;
      if (src[i] != r) {
        __builtin_nontemporal_store(kv[i], reinterpret_cast<u32x4_t*>(wrow(p, Kp, u, r) + 16 * c));
        __builtin_nontemporal_store(vv[i], reinterpret_cast<u32x4_t*>(wrow(p, Vp, u, r) + 16 * c));
      }
    }
  }
}

template <typename T>
hipError_t run_k5_paged(const PagedProblem<T>& p, T* Kp, T* Vp, const int32_t* kept,
                        hipStream_t st) {
  return launch("rkv_k5_paged_compact", k5_paged_kernel<T>, dim3(p.unit_count), dim3(256), 0, st,
                p, Kp, Vp, kept);
}

template hipError_t run_k5_paged<bf16_bits>(const PagedProblem<bf16_bits>&, bf16_bits*, bf16_bits*, const int32_t*, hipStream_t);
template hipError_t run_k5_paged<float>(const PagedProblem<float>&, float*, float*, const int32_t*, hipStream_t);

// One workgroup per sequence: pages p in [B_s/ps, ceil(N_s/ps)) go to the
// free list, in ascending p, at free_start + free_off[s]; their table entries
// become -1.
__global__ __launch_bounds__(256) void free_pages_kernel(int32_t* __restrict__ page_table, int maxp,
                                                         const int32_t* __restrict__ seq_len,
                                                         const int32_t* __restrict__ bud,
                                                         const int32_t* __restrict__ free_off,
                                                         int ps_shift, int32_t* __restrict__ free_list,
                                                         int32_t free_start) {
  const int s = blockIdx.x;
  const int n = seq_len[s], b = bud[s];
  if (n <= b) return;
  const int ps = 1 << ps_shift;
  const int first = b >> ps_shift;
  const int end = (n + ps - 1) >> ps_shift;
  int32_t* row = page_table + (int64_t)s * maxp;
  for (int pg = first + threadIdx.x; pg < end; pg += 256) {
    free_list[free_start + free_off[s] + (pg - first)] = row[pg];
    row[pg] = -1;
  }
}

hipError_t run_free_pages(int32_t* page_table, int maxp, const int32_t* seq_len,
                          const int32_t* bud, const int32_t* free_off, int ps_shift, int num_seqs,
                          int32_t* free_list, int32_t free_start, hipStream_t st) {
  return launch("rkv_free_pages", free_pages_kernel, dim3(num_seqs), dim3(256), 0, st, page_table,
                maxp, seq_len, bud, free_off, ps_shift, free_list, free_start);
}

}  // namespace rkv

// Head-shared selection on a paged cache: the H KV heads of a sequence keep
// one token set.
//
// Pages: under tensor parallelism the ranks all-reduce their eviction scores
// so that every rank evicts the same tokens ("R-KV: decoding-time KV cache
// compression for reasoning models", hysenlabs page, "What the redundancy
// scoring actually does at decode time"). On one GPU the group is a
// sequence's H heads, which also share its pages: the sum of their Z (an
// all-reduce's default reduction), summed in head order, chooses the window
// and the B_s - w best candidates, and every head keeps those indices, so a
// kept token keeps all of its heads.
//
// One 1024-thread workgroup per sequence (a batch holds a few hundred
// sequences at most: each gets a whole CU); the selection is select_block
// (rkv_select.hpp), as for one head. Sequences with N_s <= B_s keep
// everything. The in-place compaction and the page return that follow are
// the per-head ones: each head moves its rows by its (identical) kept list.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"

namespace rkv {

constexpr int kSharedThreads = 1024;

template <typename T>
__global__ __launch_bounds__(kSharedThreads) void k4_paged_shared_kernel(
    PagedProblem<T> p, const float* __restrict__ Z, float* __restrict__ zsum,
    int32_t* __restrict__ kept_all) {
  __shared__ SelectScratch sh;
  const int s = blockIdx.x;
  const int H = p.H;
  const int u0 = s * H;
  const int N = p.n(u0), B = p.budget(u0), tid = threadIdx.x;
  if (N <= B) {   // nothing to score: every head keeps everything
    for (int h = 0; h < H; ++h) {
      int32_t* kh = kept_all + p.kept_off(u0 + h);
      for (int r = tid; r < N; r += kSharedThreads) kh[r] = r;
    }
    return;
  }
  // the sequence's sums sit at sum_{s'<s} N_s' (its score base over H)
  float* zs = zsum + p.score_base[s] / H;
  for (int i = tid; i < N - p.W; i += kSharedThreads) {
    float acc = 0.f;
    for (int h = 0; h < H; ++h) acc += Z[p.score_off(u0 + h) + i];
    zs[i] = acc + 0.0f;   // + 0 folds -0 onto +0
  }
  __syncthreads();   // the workgroup's global stores are visible to it after the barrier
  int32_t* kept0 = kept_all + p.kept_off(u0);
  select_block<kSharedThreads>(zs, N, B, p.W, kept0, sh);
  __syncthreads();
  for (int h = 1; h < H; ++h) {
    int32_t* kh = kept_all + p.kept_off(u0 + h);
    for (int r = tid; r < B; r += kSharedThreads) kh[r] = kept0[r];
  }
}

template <typename T>
hipError_t run_k4_paged_shared(const PagedProblem<T>& p, int num_seqs, const float* Z, float* zsum,
                               int32_t* kept, hipStream_t st) {
  if (num_seqs == 0) return hipSuccess;
  return launch("rkv_k4_paged_shared", k4_paged_shared_kernel<T>, dim3(num_seqs),
                dim3(kSharedThreads), 0, st, p, Z, zsum, kept);
}

template hipError_t run_k4_paged_shared<bf16_bits>(const PagedProblem<bf16_bits>&, int, const float*,
                                                   float*, int32_t*, hipStream_t);
template hipError_t run_k4_paged_shared<float>(const PagedProblem<float>&, int, const float*, float*,
                                               int32_t*, hipStream_t);

}  // namespace rkv

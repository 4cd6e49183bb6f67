// Selection: keep the window and the B-w best of the other N-w candidates.
//
// Pages: the top tokens by the joint score are retained within the budget
// (sourcepulse summary of R-KV, "How It Works"), and a recent window is exempt
// from eviction ("R-KV: decoding-time KV cache compression for reasoning
// models", hysenlabs page, "What the redundancy scoring actually does at
// decode time"). Ties go to the smaller index; output is ascending.
//
// One 256-thread workgroup per unit; the selection itself is select_block
// (rkv_select.hpp).
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"

namespace rkv {

template <class P>
__global__ __launch_bounds__(256) void k4_select_kernel(P p, const float* __restrict__ Z,
                                                        int32_t* __restrict__ kept_out,
                                                        int fill_tail) {
  __shared__ SelectScratch sh;
  int u;
  if (!p.select_item(blockIdx.x, u)) return;
  const int N = p.n(u);
  const int B = p.budget(u);
  const int tid = threadIdx.x;
  int32_t* kept = kept_out + p.kept_off(u);
  if (N <= B) {   // nothing to score: keep everything
    for (int r = tid; r < N; r += 256) kept[r] = r;
    if (fill_tail)
      for (int r = N + tid; r < B; r += 256) kept[r] = -1;
    return;
  }
  select_block<256>(Z + p.score_off(u), N, B, p.W, kept, sh);
}

template <class P>
hipError_t run_k4(const P& p, int units, const float* Z, int32_t* kept, int fill_tail,
                  hipStream_t st) {
  return launch("rkv_k4_select", k4_select_kernel<P>, dim3(units), dim3(256), 0, st, p, Z, kept,
                fill_tail);
}

// Head-shared selection [hysenlabs page, "What the redundancy scoring
// actually does at decode time": the tensor-parallel ranks all-reduce their
// eviction scores so that every rank evicts the same tokens]. One workgroup
// per group of units: Z summed over the group's units in unit order, the
// usual selection on the sum, its indices copied to every unit of the group.
template <typename T>
__global__ __launch_bounds__(256) void k4_group_select_kernel(DenseProblem<T> p, int group,
                                                              const float* __restrict__ Z,
                                                              float* __restrict__ zsum,
                                                              int32_t* __restrict__ kept_all) {
  __shared__ SelectScratch sh;
  const int grp = blockIdx.x;
  const int N = p.N, B = p.B, tid = threadIdx.x;
  const int u0 = grp * group;
  float* zs = zsum + (int64_t)grp * N;
  for (int i = tid; i < N - p.W; i += 256) {
    float s = 0.f;
    for (int h = 0; h < group; ++h) s += Z[p.score_off(u0 + h) + i];
    zs[i] = s + 0.0f;   // + 0 folds -0 onto +0
  }
  __syncthreads();   // the workgroup's global stores are visible to it after the barrier
  int32_t* kept0 = kept_all + p.kept_off(u0);
  select_block<256>(zs, N, B, p.W, kept0, sh);
  __syncthreads();
  for (int h = 1; h < group; ++h) {
    int32_t* kh = kept_all + p.kept_off(u0 + h);
    for (int r = tid; r < B; r += 256) kh[r] = kept0[r];
  }
}

template <typename T>
hipError_t run_k4_group(const DenseProblem<T>& p, int group, const float* Z, float* zsum,
                        int32_t* kept, hipStream_t st) {
  return launch("rkv_k4_group_select", k4_group_select_kernel<T>, dim3(p.num_units / group),
                dim3(256), 0, st, p, group, Z, zsum, kept);
}

template hipError_t run_k4_group<bf16_bits>(const DenseProblem<bf16_bits>&, int, const float*, float*, int32_t*, hipStream_t);
template hipError_t run_k4_group<float>(const DenseProblem<float>&, int, const float*, float*, int32_t*, hipStream_t);

template hipError_t run_k4<DenseProblem<bf16_bits>>(const DenseProblem<bf16_bits>&, int, const float*, int32_t*, int, hipStream_t);
template hipError_t run_k4<DenseProblem<float>>(const DenseProblem<float>&, int, const float*, int32_t*, int, hipStream_t);
template hipError_t run_k4<PagedProblem<bf16_bits>>(const PagedProblem<bf16_bits>&, int, const float*, int32_t*, int, hipStream_t);
template hipError_t run_k4<PagedProblem<float>>(const PagedProblem<float>&, int, const float*, int32_t*, int, hipStream_t);

}  // namespace rkv

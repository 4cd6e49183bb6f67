// Selection: keep the window and the B-w best of the other N-w candidates.
//
// Pages: the top tokens by the joint score are retained within the budget
// (sourcepulse summary of R-KV, "How It Works"), and a recent window is exempt
// from eviction ("R-KV: decoding-time KV cache compression for reasoning
// models", hysenlabs page, "What the redundancy scoring actually does at
// decode time"). Ties go to the smaller index; output is ascending.
//
// One 256-thread workgroup per unit. Radix select on the order-preserving
// 32-bit image of Z (four 8-bit digit passes over an LDS histogram) finds the
// exact k-th largest key T and how many of the keys equal to T are taken.
// Then one ordered pass with two block scans writes, in index order, every
// candidate above T and the first `take` candidates equal to T, followed by
// the window. No sort, no N-sized LDS buffer: Z is re-read from cache.
#include "rkv_problem.hpp"
#include "rkv_launch.hpp"

namespace rkv {

template <class P>
__global__ __launch_bounds__(256) void k4_select_kernel(P p, const float* __restrict__ Z,
                                                        int32_t* __restrict__ kept_out,
                                                        int fill_tail) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_tmp[4];
  __shared__ uint32_t s_digit, s_above;
  int u;
  if (!p.select_item(blockIdx.x, u)) return;
  const int N = p.n(u);
  const int B = p.budget(u);
  const int W = p.W;
  const int tid = threadIdx.x;
  int32_t* kept = kept_out + p.kept_off(u);

  if (N <= B) {   // nothing to score: keep everything
    for (int r = tid; r < N; r += 256) kept[r] = r;
    if (fill_tail)
      for (int r = N + tid; r < B; r += 256) kept[r] = -1;
    return;
  }
  const int cand = N - W;
  const int k = B - W;
  const float* z = Z + p.score_off(u);

  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cand; i += 256) {
      const uint32_t key = order_key(z[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t looks at digit 255-t; inclusive count of keys with digit >= 255-t
    const uint32_t c = hist[255 - tid];
    uint32_t tot;
    const uint32_t cum = block_inclusive_scan256(c, scan_tmp, &tot);
    if (cum >= remaining && cum - c < remaining) {
      s_digit = 255u - (uint32_t)tid;
      s_above = cum - c;
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    remaining -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t take_eq = remaining;   // keys equal to T to keep, smallest indices first

  const int per = (cand + 255) / 256;
  const int lo = min(cand, tid * per), hi = min(cand, lo + per);
  uint32_t gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(z[i]);
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_inclusive_scan256(eq, scan_tmp, &tot) - eq;
  const uint32_t take = (take_eq > eq_before) ? min(eq, take_eq - eq_before) : 0u;
  const uint32_t cnt = gt + take;
  uint32_t pos = block_inclusive_scan256(cnt, scan_tmp, &tot) - cnt;
  uint32_t taken = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(z[i]);
    bool keep = key > T;
    if (key == T && taken < take) {
      keep = true;
      ++taken;
    }
    if (keep) kept[pos++] = i;
  }
  for (int r = tid; r < W; r += 256) kept[k + r] = cand + r;
}

template <class P>
hipError_t run_k4(const P& p, int units, const float* Z, int32_t* kept, int fill_tail,
                  hipStream_t st) {
  return launch("rkv_k4_select", k4_select_kernel<P>, dim3(units), dim3(256), 0, st, p, Z, kept,
                fill_tail);
}

template hipError_t run_k4<DenseProblem<bf16_bits>>(const DenseProblem<bf16_bits>&, int, const float*, int32_t*, int, hipStream_t);
template hipError_t run_k4<DenseProblem<float>>(const DenseProblem<float>&, int, const float*, int32_t*, int, hipStream_t);
template hipError_t run_k4<PagedProblem<bf16_bits>>(const PagedProblem<bf16_bits>&, int, const float*, int32_t*, int, hipStream_t);
template hipError_t run_k4<PagedProblem<float>>(const PagedProblem<float>&, int, const float*, int32_t*, int, hipStream_t);

}  // namespace rkv

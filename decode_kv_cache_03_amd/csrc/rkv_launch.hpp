// Kernel launch helper with optional per-launch event timing, and the
// host-side entry points of each kernel family.
#pragma once

#include <hip/hip_runtime.h>

#include "rkv_problem.hpp"

namespace rkv {

struct TimingSlot;
// Returns a slot whose start event has been recorded on `st`, or nullptr when
// timing is off (or its record buffer is full).
TimingSlot* timing_begin(const char* name, hipStream_t st);
void timing_end(TimingSlot* slot, hipStream_t st);

template <typename... KArgs, typename... Args>
hipError_t launch(const char* name, void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                  hipStream_t st, Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  TimingSlot* ts = timing_begin(name, st);
  kern<<<grid, block, shmem, st>>>(args...);
  hipError_t e = hipGetLastError();
  timing_end(ts, st);
  return e;
}

// Softmax statistics of the window queries: rinv [units][N] and, per unit and
// query row, (max, 1/sum) in fin; part is per-chunk scratch. When counters
// is not null, also clears the redundancy kernel's counters: [8] per-XCD
// item claims, then [units] block arrivals (those of scored units).
template <typename T, class P>
hipError_t run_k1(const P& p, int nqb, int k1_items, int num_units, float* part, float* fin,
                  float* rinv, int32_t* counters, int rpg_shift, hipStream_t st);

// Redundancy, importance and joint score: Z [units][N] (R, I when requested).
// Dense caches (P::kFinishUnits): with select_units != 0, the last block of
// each unit to finish also selects its kept indices and gathers its kept rows
// into K_out / V_out; counters (as cleared by run_k1) must be non-null.
// Paged caches ignore the last six arguments.
template <typename T, class P>
hipError_t run_k2(const P& p, int nqb, int k2_items, const float* rinv, const float* fin, float* Z,
                  float* dbg_R, float* dbg_I, float lam, int rpg_shift, int32_t* counters,
                  int32_t* kept, T* K_out, T* V_out, int64_t out_stride, int select_units,
                  hipStream_t st);

// Dense bf16 caches whose unit fits the fused kernel's LDS plan
// (fused_plan_choose): the whole step in one launch (k2_wide.hip), no
// workspace. dbg_* may be null. With score_only the kernel writes Z (dbg_Z,
// then required) and neither selects nor gathers.
hipError_t run_k2_fused(const DenseProblem<bf16_bits>& p, int nqb, float* dbg_Z, float* dbg_R,
                        float* dbg_I, float lam, int rpg_shift, int32_t* kept, bf16_bits* K_out,
                        bf16_bits* V_out, int64_t out_stride, int score_only, hipStream_t st);

// Dense bf16 caches with at most 1024 + 128 candidates per unit, one window
// query block and the causal-order R (k2_resident_fits): the whole step in
// one launch that reads every key once (k2_resident.hip). Arguments as
// run_k2_fused.
bool k2_resident_fits(const DenseProblem<bf16_bits>& p, int nqb);
hipError_t run_k2_resident(const DenseProblem<bf16_bits>& p, int nqb, float* dbg_Z, float* dbg_R,
                           float* dbg_I, float lam, int rpg_shift, int32_t* kept,
                           bf16_bits* K_out, bf16_bits* V_out, int64_t out_stride, int score_only,
                           hipStream_t st);

// Dense bf16 caches with 1152 < N <= 2176 candidates per unit, at most 48
// window query rows, the causal-order R and a budget that is a multiple of
// 32 (k2_resident2_fits): the whole step in one launch that holds each
// unit's keys in registers in two passes of 1024 rows (k2_resident2.hip).
// Arguments as run_k2_fused.
bool k2_resident2_fits(const DenseProblem<bf16_bits>& p, int rpg_shift);
hipError_t run_k2_resident2(const DenseProblem<bf16_bits>& p, float* dbg_Z, float* dbg_R,
                            float* dbg_I, float lam, int rpg_shift, int32_t* kept,
                            bf16_bits* K_out, bf16_bits* V_out, int64_t out_stride, int score_only,
                            hipStream_t st);

// Long units (bf16): Z (R, I when requested) of every unit, one 512-row
// block per work item (k2_long.hip); `count` = p.long_count(). Needs the
// norms `rinv` and normalisers `fin` of run_k1; rows are read from
// p.long_rows().
template <class P>
hipError_t run_k2_long(const P& p, int nqb, int count, const float* rinv, const float* fin, float* Z,
                       float* dbg_R, float* dbg_I, float lam, int rpg_shift, hipStream_t st);

// Selection: kept indices per unit (ascending), from Z.
template <class P>
hipError_t run_k4(const P& p, int units, const float* Z, int32_t* kept, int fill_tail,
                  hipStream_t st);

// Head-shared selection: each run of `group` consecutive units selects once,
// on the sum of their Z (zsum: [units / group][N] scratch), and every unit of
// the run receives those kept indices.
template <typename T>
hipError_t run_k4_group(const DenseProblem<T>& p, int group, const float* Z, float* zsum,
                        int32_t* kept, hipStream_t st);

// Dense gather of the kept rows into K_out / V_out.
template <typename T>
hipError_t run_k5_dense(const DenseProblem<T>& p, const int32_t* kept, T* K_out, T* V_out,
                        int64_t out_stride, int nkeep, hipStream_t st);

// Paged in-place compaction and page return.
template <typename T>
hipError_t run_k5_paged(const PagedProblem<T>& p, T* Kp, T* Vp, const int32_t* kept,
                        hipStream_t st);
hipError_t run_free_pages(int32_t* page_table, int maxp, const int32_t* seq_len,
                          const int32_t* bud, const int32_t* free_off, int ps_shift, int num_seqs,
                          int32_t* free_list, int32_t free_start, hipStream_t st);

}  // namespace rkv

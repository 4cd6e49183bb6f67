// Device-side building blocks shared by the R-KV kernels (gfx950, wave64).
//
// Fragments. Every dense contraction here has head_dim = 128 as its inner
// dimension and runs on the 32x32 MFMA tiles of CDNA4:
//   bf16: v_mfma_f32_32x32x16_bf16, 8 bf16 of k per lane per instruction;
//   fp32: v_mfma_f32_32x32x2_f32,   1 fp32 of k per lane per instruction.
// Lane l of a 32-row operand holds row (l & 31); the two 32-lane halves hold
// two disjoint parts of k. Since a dot product may visit k in any order as
// long as both operands agree, half h (= l >> 5) of every operand takes the
// contiguous elements [64h, 64h+64) of its 128-element row, streamed as 16-byte
// chunks: chunk c of half h feeds the instruction(s) of k-step c. So a lane
// loads 128 contiguous bytes (bf16) or 256 (fp32) of one row, and A and B
// fragments are loaded by the same code.
//
// Accumulator layout of a 32x32 fp32 tile: lane l, register v holds
//   row 8*(v/4) + 4*(l/32) + (v%4),  column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

constexpr int kD = 128;        // head_dim
constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef uint16_t bf16_bits;    // storage type of a bfloat16 element

// log2(e) / sqrt(128): logits are kept in base-2 units so softmax uses exp2.
constexpr float kLogitScaleLog2 = (float)(1.4426950408889634 / 11.313708498984761);

template <typename T> struct Elem;
template <> struct Elem<bf16_bits> {
  static constexpr int kRowChunks = 16;    // 16-byte chunks per 128-element row
  static constexpr int kHalfChunks = 8;
  static constexpr int kRowBytes = 256;
};
template <> struct Elem<float> {
  static constexpr int kRowChunks = 32;
  static constexpr int kHalfChunks = 16;
  static constexpr int kRowBytes = 512;
};

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
// Streaming 16-byte load: non-temporal, for data read once.
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
// Cache-policy bits of buffer instructions: non-temporal (streaming).
constexpr int kCachePolicyStream = 2;

__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// A row index taken from a kept list, forced into [0, n): a kept list that is
// stale or only partly written then reads rows of the right unit (a wrong
// result a test reports) instead of memory outside the unit.
__device__ __forceinline__ int clamp_row(int r, int n) { return min(max(r, 0), n - 1); }
__device__ __forceinline__ u32x4_t zero16() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return z;
}

// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle;
// out-of-range accesses are dropped.
constexpr int kBufferWord3 = 0x00020000;

// 16 bytes per lane from global memory straight into LDS. The 64 lanes of the
// wave fill 1 KiB of LDS at `lds_dst` in lane order (lane l -> bytes 16l..16l+15);
// each lane's source address is free. Completion is tracked by vmcnt.
__device__ __forceinline__ void load16_to_lds(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_dst), 16, 0, 0);
}

// The same from a raw buffer resource at byte offset voffset (per lane) +
// soffset (uniform): the base stays in scalar registers (no 64-bit address
// arithmetic per lane), and an offset past the resource's size reads zeros
// instead of touching memory.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t rsrc, int voffset, char* lds_dst,
                                              int soffset = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(lds_dst), 16,
                                           voffset, soffset, 0, 0);
}

// acc += A_chunk * B_chunk over the k-values of one 16-byte chunk per lane.
template <typename T>
__device__ __forceinline__ void mma_chunk(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  if constexpr (sizeof(T) == 2) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
}

// Sum of squares of the elements in a 16-byte chunk, in fp32.
template <typename T>
__device__ __forceinline__ float sumsq_chunk(u32x4_t c) {
  float s = 0.f;
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo = __uint_as_float(w[i] << 16);
      float hi = __uint_as_float(w[i] & 0xffff0000u);
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
  } else {
    float f[4] = {__uint_as_float(c.x), __uint_as_float(c.y), __uint_as_float(c.z), __uint_as_float(c.w)};
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(f[i], f[i], s);
  }
  return s;
}

// Row of accumulator register v for lane `lane` in a 32x32 tile.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is folded onto +0 first so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float z) {
  uint32_t b = __float_as_uint(z + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Workgroup barrier for LDS written with ds_* instructions. __syncthreads()
// (and even a workgroup fence limited to LDS) makes every wave first wait for
// all of its loads in flight, direct global->LDS loads included (s_waitcnt
// vmcnt(0)), which defeats loads issued ahead. Here each wave only completes
// its own LDS instructions before the barrier; the memory clobber keeps the
// compiler from moving memory accesses across it. Data that other waves bring
// into LDS with direct global->LDS loads is visible after this barrier only if
// each of them waited for those loads (s_waitcnt vmcnt) before reaching it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive sum over lanes 0..lane of one 64-lane wave, in data-parallel
// primitive (DPP) moves instead of cross-lane permutes through the LDS unit:
// within each row of 16 lanes, the value 1, 2, 4 and 8 lanes down is added
// (lanes with no source in the row add 0); then lane 15 of rows 0 and 2 is
// added to every lane of rows 1 and 3, and lane 31 to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Inclusive scan of one uint32 per thread over a block of NT threads
// (a multiple of 64, at most 1024). `scratch` must hold NT/64 uint32 and be
// shared. Also returns the block total. All threads must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* scratch,
                                                         uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = scratch[w];
    before += w < wave ? s : 0u;
    tot += s;
  }
  *total = tot;
  __syncthreads();
  return v + before;
}

// Byte offset, inside a swizzled LDS tile of 128-element rows, of the slot
// holding 16-byte chunk `chunk` of row n: the slot at position pos holds
// chunk pos ^ (n & 15) of the row, so the 16 rows that a fragment read
// touches at one chunk position hit 16 different banks groups.
template <typename T>
__device__ __forceinline__ int frag_offset(int n, int chunk) {
  return n * Elem<T>::kRowBytes + ((chunk ^ (n & 15)) << 4);
}

// One exchange of a butterfly max-reduction of 32 values per lane across the
// 32 lanes of a half-wave: lanes whose bit W is set keep values W..2W-1 of
// the current range, the others keep 0..W-1; each receives the half it keeps
// from the partner lane l ^ W. After W = 16, 8, 4, 2, 1, lane l holds in
// val[0] the max over all lanes of value l & 31.
template <int W>
__device__ __forceinline__ void max_butterfly_step(float (&val)[32], int lane) {
  const bool upper = (lane & W) != 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const float keep = upper ? val[i + W] : val[i];
    const float send = upper ? val[i] : val[i + W];
    val[i] = fmaxf(keep, __shfl_xor(send, W, 64));
  }
}

}  // namespace rkv

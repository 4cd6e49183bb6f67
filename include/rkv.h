/*
 * rkv.h — C ABI of the R-KV decode-time KV-cache compression step for MI355X (gfx950).
 *
 * Pages this interface follows (cited by title and section):
 *   [P1] "R-KV: decoding-time KV cache compression for reasoning models"
 *        (hysenlabs project page), sections "What the redundancy scoring
 *        actually does at decode time" and "How this differs from
 *        attention-sink and heavy-hitter eviction".
 *   [P2] sourcepulse project summary of R-KV, section "How It Works".
 *   [P3] "R-KV: Redundancy-aware KV Cache Compression for Reasoning Models"
 *        (atlas.scime.ai paper summary), sections "Approach" and "Measured
 *        effects reported in the paper".
 *
 * One call compresses many independent units. A unit is one (sequence,
 * layer, KV head) with N buffered candidate tokens. For each unit:
 *   I_j  importance: softmax attention of the last w decode queries of each
 *        of the G query heads of the GQA group over the N candidates (query r
 *        of the window sees candidates j <= N-w+r; logits q.k/sqrt(d)), mean
 *        over the w queries, then max over the G heads [P2 "How It Works";
 *        P3 "Approach"; max pooling per P3 "Measured effects", last row].
 *   R_i  redundancy: max over earlier candidates j < i of cos(k_i, k_j), and
 *        R_0 = 0; a zero-norm key has cosine 0 [P2 "How It Works"; P3
 *        "Approach"; P1 "How this differs ..."].
 *   Z_i  = lambda*I_i - (1-lambda)*R_i [P3 "Approach"].
 *   The last w candidates (the window) are always kept [P1 "What the
 *   redundancy scoring ..."]; of the other N-w, the B-w with the largest Z
 *   are kept, ties going to the smaller index [P2 "How It Works"]. Kept
 *   indices are ascending. N <= B keeps every candidate.
 *   The kept K/V rows are copied out (dense) or compacted in place with the
 *   freed pages returned to a free list (paged) [P1 "What the redundancy
 *   scoring ..." on physical eviction and block return].
 *
 * Conventions for every entry point:
 *   - head_dim must be 128. dtype is RKV_BF16 or RKV_F32 for K, V and Q.
 *   - Pointers marked "device" are device memory of the current HIP device;
 *     "host" pointers are read before the call returns.
 *   - The caller owns every buffer. The library never allocates device
 *     memory; scratch comes from the caller's workspace, whose size the
 *     *_workspace_size functions return. Workspace contents need not be
 *     initialised and are garbage after the call.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and is asynchronous: outputs are valid once the stream is synchronised.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On any error nothing is written and nothing is launched, the call
 *     returns a negative status, and rkv_last_error() describes it.
 *   - Calls from different host threads are safe if they use different
 *     workspaces; error messages are per thread.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define RKV_OK 0
#define RKV_EINVAL (-1)       /* bad shape, size, pointer, aliasing or parameter */
#define RKV_EWORKSPACE (-2)   /* workspace missing or smaller than required */
#define RKV_EFREELIST (-3)    /* paged: freed pages would overflow the free list */
#define RKV_EUNSUPPORTED (-4) /* valid request outside what the kernels implement */
#define RKV_EHIP (-5)         /* a HIP runtime call or launch failed */

/* Element types of K, V and Q_win. */
#define RKV_F32 0
#define RKV_BF16 1

/* Reading variants: bits of the `variant` field of both descriptors; 0
 * selects the readings stated at the top of this file. Each replaces one
 * step the pages leave open by its alternative:
 *   RKV_VARIANT_SYMMETRIC  R_i = max over every other candidate j != i of
 *                          cos(k_i, k_j), so both copies of a duplicate score
 *                          as redundant (the plain symmetric reading; the
 *                          default follows P1's "similar to what is already
 *                          retained"). Scores the whole N x N cosine matrix:
 *                          twice the MFMA work of the default.
 *   RKV_VARIANT_NO_CAUSAL  every window query sees all N candidates.
 *   RKV_VARIANT_POOL_MEAN  I_j = mean over the G query heads instead of the
 *                          max (the pooling ablation of P3 "Measured effects
 *                          reported in the paper", last row).
 *   RKV_VARIANT_SHARED_HEADS  paged calls only: head-shared selection [P1
 *                          "What the redundancy scoring actually does at
 *                          decode time": tensor-parallel ranks all-reduce
 *                          their eviction scores so that all evict the same
 *                          tokens]. The H heads of a sequence keep one token
 *                          set: the window and the B_s - w best candidates
 *                          by the sum of their Z. Each head's Z is its own;
 *                          kept_idx holds the same list for every head. The
 *                          dense call takes select_group instead and rejects
 *                          this bit.
 * Other bits are RKV_EINVAL. */
#define RKV_VARIANT_SYMMETRIC 1u
#define RKV_VARIANT_NO_CAUSAL 2u
#define RKV_VARIANT_POOL_MEAN 4u
#define RKV_VARIANT_SHARED_HEADS 8u

/* Dense layout: unit h has K[h], V[h] = N rows of 128 contiguous elements,
 * consecutive rows 128 elements apart, consecutive units kv_head_stride
 * elements apart. */
typedef struct rkv_dense_desc {
  int32_t num_heads;       /* units in the call, >= 0 (0 = nothing to do) */
  int32_t n_cand;          /* N candidates per unit, >= 1 */
  int32_t head_dim;        /* must be 128 */
  int32_t gqa_group;       /* G query heads per KV head, >= 1 */
  int32_t window;          /* w protected recent tokens and window queries, 1..32 */
  int32_t budget;          /* B kept tokens per unit, > window */
  float mix_lambda;        /* lambda, finite */
  int32_t dtype;           /* RKV_BF16 or RKV_F32 */
  int64_t kv_head_stride;  /* elements between units in K and V; 0 means N*128 */
  int64_t out_head_stride; /* elements between units in K_out, V_out; 0 means B*128 */
  uint32_t variant;        /* RKV_VARIANT_* bits; 0 = the default readings */
  int32_t select_group;    /* 0 or 1: every unit selects its own tokens. g > 1:
                              head-shared selection: each run of g consecutive
                              units (e.g. the KV heads of one layer of one
                              sequence) keeps ONE token set, the window plus the
                              top B-w by the sum of the g units' Z, and every
                              unit of the run gathers its own rows of it. This
                              is what the eviction-score all-reduce across
                              tensor-parallel ranks does so that every rank
                              evicts the same tokens [P1 "What the redundancy
                              scoring ..."]; an all-reduce sums. num_heads must
                              be a multiple of g. Summed in unit order in fp32. */
} rkv_dense_desc;

/* Bytes of workspace rkv_compress needs for `desc` (with all debug outputs
 * NULL; supplying debug outputs never needs more). Returns 0 and sets the
 * error message if desc is invalid; a valid desc always needs > 0 bytes. */
size_t rkv_workspace_size(const rkv_dense_desc* desc);

/* Dense compression, out of place.
 *   K, V       device [num_heads][N][128] (unit stride kv_head_stride), dtype
 *   Q_win      device [num_heads][G][w][128] contiguous, dtype; row (g, r) is
 *              window query r (r = 0 oldest, w-1 newest) of query head g
 *   kept_idx   device int32 [num_heads][B]: kept candidate indices ascending
 *              (identical rows within a select_group run);
 *              when N < B, entries N..B-1 are set to -1
 *   K_out, V_out  device [num_heads][B][128] (unit stride out_head_stride);
 *              row r = row kept_idx[r] of the input; rows >= min(N, B) are
 *              not written. Must not overlap K or V.
 *   dbg_I, dbg_R, dbg_Z  device float [num_heads][N] or NULL; when given and
 *              N > B they receive each unit's own I, R and Z (window entries
 *              included; Z with -0 written as +0; not the group sum of
 *              head-shared selection). Not written when N <= B.
 *   workspace  device, >= rkv_workspace_size(desc) bytes, 256-byte aligned
 *   stream     hipStream_t
 * Returns RKV_OK or a negative status. */
int rkv_compress(const rkv_dense_desc* desc, const void* K, const void* V, const void* Q_win,
                 int32_t* kept_idx, void* K_out, void* V_out, float* dbg_I, float* dbg_R,
                 float* dbg_Z, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device scratch behind rkv_compress_static (per GPU). */
#define RKV_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* rkv_compress without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * outputs and errors as rkv_compress, minus workspace; the workspace is a
 * library-owned device array of RKV_STATIC_SCRATCH_BYTES that each GPU holds
 * from library load until the process ends. A call whose
 * rkv_workspace_size(desc) exceeds that returns RKV_EWORKSPACE (nothing
 * done). The library makes no hipMalloc/hipFree or other allocating call
 * here. Every call on one GPU shares that GPU's array and leaves its contents
 * behind (each call initialises what it reads): calls that overlap on one GPU
 * (different streams or host threads without ordering) race, so order them. */
int rkv_compress_static(const rkv_dense_desc* desc, const void* K, const void* V,
                        const void* Q_win, int32_t* kept_idx, void* K_out, void* V_out,
                        float* dbg_I, float* dbg_R, float* dbg_Z, void* stream);

/* Paged layout: a pool of num_pages pages; token t of (sequence s, KV head
 * hk) is the 128-element row at
 *   pages + page_table[s][t / page_size] * page_stride + hk * head_stride
 *         + (t % page_size) * slot_stride
 * (strides in elements; [P][H][page_size][128] contiguous is page_stride =
 * H*page_size*128, head_stride = page_size*128, slot_stride = 128). */
typedef struct rkv_paged_desc {
  int32_t num_seqs;          /* S >= 0 */
  int32_t num_kv_heads;      /* H >= 1 */
  int32_t head_dim;          /* must be 128 */
  int32_t gqa_group;         /* G >= 1 */
  int32_t window;            /* w, 1..32 */
  int32_t page_size;         /* tokens per page, a power of two, 1..4096 */
  int32_t max_pages_per_seq; /* columns of page_table */
  int32_t num_pages;         /* P, pages in the pool */
  float mix_lambda;          /* lambda, finite */
  int32_t dtype;             /* RKV_BF16 or RKV_F32 */
  int64_t page_stride;       /* elements; 0 means H*page_size*128 */
  int64_t head_stride;       /* elements; 0 means page_size*128 */
  int64_t slot_stride;       /* elements; 0 means 128 */
  uint32_t variant;          /* RKV_VARIANT_* bits; 0 = the default readings */
} rkv_paged_desc;

/* Workspace bytes for rkv_compress_paged with these host lengths/budgets;
 * 0 (with an error message) when the arguments are invalid. */
size_t rkv_paged_workspace_size(const rkv_paged_desc* desc, const int32_t* seq_len_host,
                                const int32_t* budget_host);

/* Paged compression, in place, with page return.
 *   K_pages, V_pages  device pools (layout above), updated in place: for each
 *              sequence with N_s > B_s and each head, logical slot r < B_s
 *              receives the row of kept candidate r. Other slots, and every
 *              page of a sequence with N_s <= B_s, are left unchanged.
 *   page_table device int32 [S][max_pages_per_seq], updated in place: for
 *              sequences with N_s > B_s, entries p with
 *              B_s/page_size <= p < ceil(N_s/page_size) become -1. Entries
 *              p < ceil(N_s/page_size) must be distinct valid page ids.
 *   seq_len_host, budget_host  host int32 [S]: N_s >= 1; B_s > w and a
 *              multiple of page_size; ceil(N_s/page_size) <= max_pages_per_seq.
 *   Q_win      device [S][H][G][w][128] contiguous, dtype
 *   kept_idx   device int32, ragged: sequence s, head hk occupies
 *              min(N_s, B_s) entries at offset
 *              H * sum_{s'<s} min(N_s', B_s') + hk * min(N_s, B_s)
 *   free_list  device int32 [free_capacity]: the freed page ids are written
 *              at positions *free_count_host ... in (s ascending, p
 *              ascending) order
 *   free_count_host  host in/out: entries in use before; after the call,
 *              increased by the number of freed pages
 *   dbg_Z      device float, ragged like kept_idx but with N_s entries per
 *              (s, hk) (offset H * sum_{s'<s} N_s' + hk * N_s), or NULL;
 *              written only for sequences with N_s > B_s
 *   workspace  device, >= rkv_paged_workspace_size(...) bytes
 * Returns RKV_OK, RKV_EFREELIST when *free_count_host plus the freed pages
 * exceeds free_capacity (nothing done), or another negative status. */
int rkv_compress_paged(const rkv_paged_desc* desc, void* K_pages, void* V_pages,
                       int32_t* page_table, const int32_t* seq_len_host,
                       const int32_t* budget_host, const void* Q_win, int32_t* kept_idx,
                       int32_t* free_list, int32_t free_capacity, int32_t* free_count_host,
                       float* dbg_Z, void* workspace, size_t workspace_bytes, void* stream);

/* Compression-aware admission: page accounting of a paged cache under
 * periodic compression, on the host [P1 "What the redundancy scoring
 * actually does at decode time": the serving port's scheduler admits
 * requests on the compressed footprint, and compression returns freed blocks
 * to the allocator; P3 "Approach": compression runs periodically during
 * decoding with a fixed buffer].
 *
 * A sequence that holds L tokens, with budget B and buffer divide_length D,
 * is compressed back to B tokens by the append that brings it to B + D
 * tokens; a sequence already holding more than B + D tokens (e.g. after a
 * long prompt) is compressed by the next call, at its current length. So it
 * never holds more than max(L, B + D) tokens, and a scheduler that reserves
 * that many pages per running sequence can admit new requests on the
 * remainder. Per sequence s (a sequence occupies ceil(tokens / page_size)
 * pages):
 *   pages_now      ceil(L / page_size)
 *   pages_peak     ceil(max(L, B + D) / page_size): the most it holds before
 *                  its next compression completes
 *   pages_after    B / page_size: held right after that compression
 *   pages_freed    pages_peak - pages_after: returned to the free list by it
 *                  (what rkv_compress_paged appends for s when called then)
 *   steps_to_event tokens still to append before that compression: 0 when
 *                  L >= B + D (due now), else B + D - L
 * B = 0 or D = 0 switches compression off for the sequence (the pages' "0
 * disables" convention): then pages_peak = -1 (unbounded), pages_after =
 * pages_now, pages_freed = 0 and steps_to_event = -1. Nothing here touches a
 * GPU. */
typedef struct rkv_page_plan {
  int32_t pages_now;
  int32_t pages_peak;
  int32_t pages_after;
  int32_t pages_freed;
  int32_t steps_to_event;
} rkv_page_plan;

/* Fills plan_host[s] for s < num_seqs from seq_len_host[s] (L >= 0) and
 * budget_host[s] (B = 0, or B > 0 and a multiple of page_size), with
 * page_size a power of two in [1, 4096] and divide_length >= 0. When
 * totals_host is not NULL it receives four sums over the sequences with
 * compression on: pages_now, pages_peak, pages_after and pages_freed; the
 * pages still to be claimed before the next compressions is then
 * totals[1] - totals[0]. All pointers are host memory; plan_host may be NULL
 * when only totals are wanted. Returns RKV_OK, or RKV_EINVAL (nothing
 * written) for a bad argument. */
int rkv_paged_plan(int32_t num_seqs, const int32_t* seq_len_host, const int32_t* budget_host,
                   int32_t page_size, int32_t divide_length, rkv_page_plan* plan_host,
                   int64_t* totals_host);

/* Message of the last failed call on this host thread ("" if none). The
 * pointer stays valid until the next call on this thread. */
const char* rkv_last_error(void);

/* Per-kernel timing, for benchmarks. While enabled (enable != 0), every
 * kernel the library launches is bracketed by a pair of HIP events recorded
 * on the launch stream (up to 65536 launches; later ones are not timed).
 * Enabling clears earlier records. Returns RKV_OK or RKV_EHIP. */
int rkv_timing_enable(int enable);

/* After the stream is synchronised: writes up to max_kernels entries
 * (kernel name, number of timed launches, summed milliseconds) in first-
 * launch order, returns the number of distinct kernels (which may exceed
 * max_kernels), or a negative status. Names stay valid for the process. */
int rkv_timing_read(const char** names, int32_t* launches, double* total_ms,
                    int32_t max_kernels);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */

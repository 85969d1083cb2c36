/*
 * sparse_decode.h -- C ABI of the query-adaptive sparse decode attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * One decode step, for every sequence b, query token t (T adjacent tokens per
 * sequence, usually 1) and query head h (KV group g = h / G):
 *   1. score   relevance of each chunk summary key to the query, s = q . k_g
 *              (AI Trends summary of SSA, aitrends.kr/articles/69798, sections
 *              "방법론" and "기술 상세"); for H-SSA also meta-summary scores first
 *              (same page, "핵심 기여", hierarchical gist-of-gist); or the score
 *              of every token's rank-r proxy key against the projected query
 *              (review of "Full Attention Strikes Back", section 1, 16-dim
 *              low-dimensional projection).
 *   2. select  per-head top-k chunks (SSA, "방법론"), dynamic top-p over the
 *              softmax of the scores (Full Attention Strikes Back review,
 *              section 1), or two-level top-k; then one shared selection per
 *              GQA group: the union of the group's heads, stored as an ascending
 *              compact index list (SSA, glossary "Grouped-Query Attention", and
 *              "핵심 기여", decode kernel: compact list of selected key indices).
 *   3. attend  exact softmax attention over the raw K/V of the listed chunks
 *              plus their summary K/V (the hybrid context), computed as split-K
 *              partial attention (same section).
 *   4. combine log-sum-exp merge of the split partials (same section).
 *
 * Conventions
 *   - Every pointer argument named as a tensor is DEVICE memory; the config,
 *     handle and status outputs are host memory.
 *   - The caller allocates and owns all device memory, including a workspace
 *     of the size sparse_decode_init reports (256-byte aligned). The library
 *     allocates no device memory and keeps no device state; it writes only into
 *     the workspace and the output buffers passed to it.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     compute calls only enqueue work and return; none synchronises.
 *   - Errors: every argument check runs on the host before anything is
 *     enqueued, so a call that returns an error has enqueued nothing. A failed
 *     kernel launch returns SD_EHIP. Device-side faults surface at the caller's
 *     next synchronisation. sparse_decode_last_error() gives a message for the
 *     last failing call on the calling thread. No C++ exception crosses the ABI.
 *   - A handle is immutable after init: calls with distinct workspaces may run
 *     concurrently on different streams. Calls that share one workspace must be
 *     ordered on one stream.
 *   - Call order for one step: score(0), select(0), [score(1), select(1) when
 *     sparse_decode_num_levels() == 2], attend, combine.
 */
#ifndef SPARSE_DECODE_H
#define SPARSE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sd_handle sd_handle;

typedef enum {
  SD_OK = 0,
  SD_EINVAL = 1,        /* a null, misaligned or out-of-range argument */
  SD_EUNSUPPORTED = 2,  /* a valid request the library does not implement */
  SD_EWORKSPACE = 3,    /* workspace pointer null or not 256-byte aligned */
  SD_EHIP = 4           /* a HIP runtime call failed (message has the code) */
} sd_status;

enum { SD_F32 = 0, SD_BF16 = 1 };                       /* q / K / V / summary dtype */
enum { SD_TOPK = 0, SD_TOPP = 1, SD_HIER_TOPK = 2, SD_COVERAGE = 3 };  /* selection rule */
enum { SD_ROUTE_SUMMARY = 0, SD_ROUTE_PROXY = 1 };      /* what is scored */

typedef struct {
  int32_t batch;          /* sequences B, >= 1 */
  int32_t n_queries;      /* T adjacent query tokens per sequence (0 or 1: one). With T > 1
                             (multi-query decode: speculative or batched positions; review of
                             "Hierarchical Sparse Attention Done Right", section 3 and its
                             kernel figure: adjacent queries share the union of their chunks)
                             every (token, head) selects on its own and the union per KV group
                             runs over all T x G of them; each attends that union. The T
                             queries read the same cache: it holds their past, not their own
                             keys. T x G <= 16 (8 with SD_ROUTE_PROXY). */
  int32_t kv_batch;       /* KV caches: 1 (every sequence reads cache 0) or B */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0 and G = Hq / Hkv, T x G <= 16 */
  int32_t head_dim;       /* d: 64 or 128 */
  int64_t n_ctx;          /* N tokens in the cache, 1 <= N < 2^31, N / C <= 2^24 */
  int32_t chunk_size;     /* C tokens per chunk, N % C == 0; 1 = token-level */
  int32_t seg_size;       /* SD_HIER_TOPK: chunks per segment, M % seg == 0 */
  int32_t route;          /* SD_ROUTE_SUMMARY or SD_ROUTE_PROXY (needs C == 1) */
  int32_t route_dim;      /* proxy rank r (SD_ROUTE_PROXY): 16 */
  int32_t kv_dtype;       /* SD_F32 or SD_BF16 */
  int32_t mode;           /* SD_TOPK, SD_TOPP, SD_HIER_TOPK or SD_COVERAGE */
  int32_t top_k;          /* SD_TOPK / SD_HIER_TOPK: chunks kept per head, >= 1 */
  int32_t top_k_seg;      /* SD_HIER_TOPK: segments kept per head, >= 1 */
  double top_p;           /* SD_TOPP: mass to reach, in (0, 1]; 1 keeps all */
  double select_scale;    /* SD_TOPP / SD_COVERAGE: logit = select_scale * score, > 0 */
  double tau;             /* SD_COVERAGE ([TSA] dynamic token coverage), in [0, 1): per
                             sequence, importance = the scored heads' softmax probabilities
                             summed per chunk; the ascending tail is cut until the cut mass
                             exceeds tau x total; budget = max(1, chunks - cut), and every
                             head keeps its own top-budget chunks. Summary routing, at most
                             2048 chunks per row. */
  float softmax_scale;    /* attention logit scale, > 0 (1/sqrt(d)) */
  int32_t keep_first;     /* chunks [0, keep_first) always in the union */
  int32_t keep_last;      /* chunks [M - keep_last, M) always in the union */
  int32_t sink;           /* local KV heads: tokens [0, sink) ... */
  int32_t window;         /* ... and [N - window, N); needs C == 1 */
  int32_t attend_summary; /* summary K/V in the hybrid context: 0 none, 1 the selected
                             chunks' ([SSA] technical detail), 2 every chunk's (variant:
                             the query meets all summaries) */
  int32_t attend_blocks;  /* persistent attention workgroups, each streaming an equal slice
                             of all groups' tiles; 0 = library default (256: one per CU of a
                             256-CU MI355X). See sparse_decode_attend_blocks(). */
  int32_t head_masks;     /* 0: every head of a group attends to the whole group union; 1
                             (variant): the union is still loaded once, but head h attends
                             only to its own selection plus the forced chunks (local groups
                             unmasked; summaries of unselected chunks under attend_summary 2
                             stay visible to every head) */
  const int8_t* head_mode;/* HOST array [n_kv_heads]: 0 = scored head, 1 = local head;
                             NULL = all scored. Copied at init. */
} sd_config;

/* Input tensors (device pointers) and their element strides. The last
 * dimension of every tensor is contiguous. Unused tensors may be NULL.
 *   q    [B][T][Hq][d]         kv_dtype   strides q_sb, q_st (ignored when T = 1), q_sh
 *   k, v [Bkv][Hkv][N][d]      kv_dtype   strides kv_sb (0 allowed), kv_sh, kv_st
 *   kg, vg [Bkv][Hkv][M][d]    kv_dtype   summary key / value per chunk; g_sb, g_sh, g_st
 *   kmg  [Bkv][Hkv][S][d]      kv_dtype   meta-summary key per segment; mg_sb, mg_sh, mg_st
 *   kp   [Bkv][Hkv][N][r]      fp16       proxy key per token; kp_sb, kp_sh, kp_st
 *   proj [Hkv][d][r]           fp32       contiguous projection per KV head
 *   ctx_len [B]                int32      growing cache: tokens sequence b holds this step
 *                                         (NULL: every sequence holds n_ctx)
 * Row strides (kv_st, g_st, mg_st) must keep every row 16-byte aligned, and
 * every base pointer must be 16-byte aligned.
 *
 * Growing cache (review of "Hierarchical Sparse Attention Done Right", section 3 and its kernel
 * figure: decode steps of T adjacent tokens; AI Trends summary of SSA, "주요 결과" and "관련
 * Figure": the cost per step is followed as the context grows). n_ctx is then the capacity: the
 * handle and workspace are sized for it and the tensors are allocated for it, while ctx_len[b]
 * (device memory, read by the step, values clamped to [0, n_ctx]) is the number of valid tokens
 * of sequence b at this step. Between steps the caller appends T tokens' K / V (and proxy keys)
 * and, when a chunk becomes complete, its summary K / V row, and raises ctx_len. Per sequence:
 * the complete chunks M_b = ctx_len[b] / C are scored and selected (rows past them are never
 * used); keep_first / keep_last count from 0 and from M_b; the raw tokens of the incomplete last
 * chunk [M_b C, ctx_len[b]) have no summary yet and join the group's context unselected (every
 * head attends them); local heads take [0, sink) and [ctx_len[b] - window, ctx_len[b]). The
 * lengths are read once, by the step's score call, which copies them into the workspace for the
 * later calls. Not available with SD_HIER_TOPK (SD_EUNSUPPORTED). */
typedef struct {
  const void* q;   int64_t q_sb, q_sh, q_st;
  const void* k;   const void* v;   int64_t kv_sb, kv_sh, kv_st;
  const void* kg;  const void* vg;  int64_t g_sb, g_sh, g_st;
  const void* kmg; int64_t mg_sb, mg_sh, mg_st;
  const void* kp;  int64_t kp_sb, kp_sh, kp_st;
  const float* proj;
  const int32_t* ctx_len;
} sd_tensors;

/* Device pointers into a workspace, for inspection after a step. Per-query
 * rows come T x Hq per sequence, ordered by KV group, then query token, then
 * head in the group: row g (T G) + t G + j is token t, head g G + j.
 *   scores0   fp64 [B][T Hq][len0]  level-0 scores (chunks, segments or tokens)
 *   scores1   fp64 [B][T Hq][len1]  level-1 candidate scores (two-level only)
 *   cand1     int32 [B][T Hq][len1] level-1 candidate chunk ids, ascending
 *   head_bits u32 [B][T Hq][words]  per-head selection bitmap, bit e of word e/32
 *                                 (forced and local entries are not included)
 *   list      int32 [B][Hkv][n_entries] group union, ascending; first cnt valid
 *   count     int32 [B][Hkv]      union size
 *   status    u32 [4]             internal-invariant flags, cleared by every
 *                                 step's first call: every row is resolved
 *                                 exactly for any input (near-equal and tied
 *                                 scores included), so a nonzero word after a
 *                                 step is a library defect, never an input
 *                                 condition */
typedef struct {
  const double* scores0;   int64_t len0;
  const double* scores1;   int64_t len1;
  const int32_t* cand1;
  const uint32_t* head_bits; int64_t words;
  const int32_t* list;     int64_t n_entries;
  const int32_t* count;
  const uint32_t* status;
} sd_selection_view;

/* Validate and copy `cfg`, create a handle, report the workspace size in bytes.
 * Host only: touches no GPU. Errors: SD_EINVAL (null pointer, inconsistent
 * shape or parameter), SD_EUNSUPPORTED (head_dim not 64/128, T x G > 16). */
sd_status sparse_decode_init(const sd_config* cfg, sd_handle** out, size_t* workspace_bytes);

/* 1 for flat selection, 2 for two-level (SD_HIER_TOPK). 0 for a NULL handle. */
int32_t sparse_decode_num_levels(const sd_handle* h);

/* Persistent attention workgroups the handle launches (attend_blocks, or the
 * library default when it was 0). 0 for a NULL handle. Host only. */
int32_t sparse_decode_attend_blocks(const sd_handle* h);

/* Step 1: scores of `level` (0: summary / meta-summary / proxy scores of every
 * entry; 1: chunk scores of the level-0 candidates) into the workspace. */
sd_status sparse_decode_score_chunks(const sd_handle* h, const sd_tensors* t, int level,
                                     void* ws, void* stream);

/* Step 2: per-head selection at `level`; after the last level, also the group
 * union with forced / local entries, compacted into the ascending list. */
sd_status sparse_decode_select(const sd_handle* h, int level, void* ws, void* stream);

/* Step 3: split-K partial attention over each group's list (workspace). */
sd_status sparse_decode_attend(const sd_handle* h, const sd_tensors* t, void* ws, void* stream);

/* Step 4: merge the partials into out fp32 [B][T][Hq][d] and lse_out fp32
 * [B][T][Hq] (natural log of the softmax normaliser), both contiguous device
 * buffers. */
sd_status sparse_decode_combine(const sd_handle* h, void* ws, float* out, float* lse_out,
                                void* stream);

/* One whole step -- score and select at every level, attend, combine -- on the caller's
 * workspace, in one call: the stages the SSA summary's decode kernel chains (핵심 기여), with the
 * host-side cost of one call instead of one per stage. Same arguments, layouts and results as
 * calling sparse_decode_score_chunks / sparse_decode_select per level, then sparse_decode_attend
 * and sparse_decode_combine, on `stream`; outputs out fp32 [B][T][Hq][d] and lse_out fp32
 * [B][T][Hq], contiguous device buffers (out 16-byte aligned). Errors, all from host checks with
 * nothing enqueued: SD_EINVAL (NULL handle, tensors or outputs), SD_EWORKSPACE (NULL or not
 * 256-byte aligned workspace); SD_EHIP for a failed launch. */
sd_status sparse_decode_step(const sd_handle* h, const sd_tensors* t, void* ws, float* out, float* lse_out,
                             void* stream);

/* One whole step -- score and select at every level, attend, combine -- with the library's own
 * static device scratch as the workspace. For callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the call
 * allocates nothing, on the host or the device. Outputs as sparse_decode_combine: out fp32
 * [B][T][Hq][d], lse_out fp32 [B][T][Hq], contiguous device buffers.
 *   - The scratch is a 16 MiB device array per GPU (held until the process ends); a handle whose
 *     workspace (sparse_decode_init's workspace_bytes) is larger is rejected with SD_EUNSUPPORTED
 *     before anything is enqueued (the 128K, 32K and 512K workloads fit; the 1M-token proxy
 *     workload does not).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last call's contents; each
 *     step clears what it needs zeroed (status words, arrival counters) itself. Calls that overlap
 *     on one GPU (concurrent streams, or threads) race on it: order them on one stream.
 *   - The scratch of the device current at the call is used; `stream` must belong to that device.
 *   - The per-stage inspection view is not available for this scratch.
 * Errors as the other calls: SD_EINVAL / SD_EUNSUPPORTED from host checks (nothing enqueued),
 * SD_EHIP for a failed address lookup or launch. */
sd_status sparse_decode_step_static(const sd_handle* h, const sd_tensors* t, float* out, float* lse_out,
                                    void* stream);

/* Fill `view` with device pointers into `ws` (no device access). */
sd_status sparse_decode_selection_view(const sd_handle* h, void* ws, sd_selection_view* view);

/* Message of the last failing call on this thread ("" if none). */
const char* sparse_decode_last_error(void);

/* Release a handle (host memory only). NULL is ignored. */
void sparse_decode_destroy(sd_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_DECODE_H */

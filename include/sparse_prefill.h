/*
 * sparse_prefill.h -- C ABI of the Token-Sparse prefill attention path of the
 * query-adaptive sparse attention library for AMD Instinct MI355X (gfx950).
 *
 * One prefill attention layer over a prompt of L tokens, for every sequence b and
 * query head h (KV group g = h / G), following the technical summary of "Token
 * Sparse Attention" (gist.science, paper 2602.03216), section 2:
 *   1. select   dynamic token coverage: the W most recent queries of head h attend
 *               causally to every key (a proxy attention map, fp64); head h's
 *               importance of key j is the sum of that map's column j. The heads'
 *               importances are summed per token; taken in ascending order, the low
 *               tail is cut until its mass exceeds tau of the total, and the tokens
 *               left give the budget k (at least 1). Every head then keeps its own k
 *               tokens of highest importance (equal importance: lower position
 *               first), as an ascending position list.
 *               A head routed to full attention (head_mode) keeps every position instead.
 *   2. attend   compression: the head's Q, K and V rows at its k positions form a
 *               compact sequence; causal softmax attention runs on it (compact row i
 *               attends compact rows 0..i); decompression: row i of the result is
 *               written to position S_h[i] of the output, and every other position
 *               of the head is zero (the residual stream keeps those tokens).
 *
 * Conventions are those of sparse_decode.h: tensors are DEVICE pointers, the
 * caller owns all device memory including the workspace (256-byte aligned, size
 * reported by init), calls only enqueue on `stream` and never synchronise,
 * every argument check runs on the host before anything is enqueued, and
 * sparse_decode_last_error() reports the last failing call of this thread.
 * Call order for one layer: select, then attend.
 */
#ifndef SPARSE_PREFILL_H
#define SPARSE_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#include "sparse_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sp_handle sp_handle;

typedef struct {
  int32_t batch;          /* sequences B, >= 1 */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;       /* d: 128 */
  int64_t seq_len;        /* L prompt tokens, window <= L <= 2^24 */
  int32_t window;         /* W most recent queries of the proxy map, 1 .. 64 */
  int32_t kv_dtype;       /* SD_BF16 */
  double tau;             /* coverage threshold, in [0, 1) */
  double softmax_scale;   /* logit scale of the proxy map (fp64) and of the attention (rounded
                             to fp32 there), > 0 */
} sp_config;

/* Device tensors, last dimension contiguous, element strides, 16-byte aligned rows.
 *   q         [B][Hq][L][d]   bf16   strides q_sb, q_sh, q_st
 *   k, v      [B][Hkv][L][d]  bf16   strides kv_sb, kv_sh, kv_st (k and v share them)
 *   head_mode [Hq]            int8   or NULL (every head sparse). Head-wise routing of the technical
 *             summary of "Elastic Attention" (gist.science, paper 2601.17367), sections 2.1 and 2.3:
 *             1 = full-attention head (keeps every position: plain causal attention), 0 = sparse head
 *             (the selection above). The budget is cut from the sparse heads' importances only; all
 *             heads run in the same launches. Values other than 0 count as 1. select and attend
 *             must be given the same routing. */
typedef struct {
  const void* q;  int64_t q_sb, q_sh, q_st;
  const void* k;  const void* v;  int64_t kv_sb, kv_sh, kv_st;
  const int8_t* head_mode;
} sp_tensors;

/* Device pointers into a workspace after select.
 *   importance fp64 [B][Hq][L]    head h's proxy-map column sums
 *   budget     int32 [B]          tokens kept per sparse head (unused when every head is full)
 *   head_bits  u32 [B][Hq][words] head h's positions, bit j of word j/32
 *   list       int32 [B][Hq][L]   head h's positions ascending; the first budget[b] valid
 *   status     u32 [4]            internal-invariant flags (zero after every call on any
 *                                 input; a nonzero word is a library defect) */
typedef struct {
  const double* importance;
  const int32_t* budget;
  const uint32_t* head_bits; int64_t words;
  const int32_t* list;
  const uint32_t* status;
} sp_view;

/* Validate and copy `cfg`, create a handle, report the workspace size in bytes
 * (it holds the fp64 proxy scores, B Hq W L x 8 bytes, whose region attend reuses for every
 * head's gathered K and V rows, B Hq L d x 4 bytes, and the selection state).
 * Host only. Errors: SD_EINVAL (null pointer, inconsistent shape or parameter),
 * SD_EUNSUPPORTED (head_dim != 128, kv_dtype != SD_BF16, window > 64). */
sd_status sparse_prefill_init(const sp_config* cfg, sp_handle** out, size_t* workspace_bytes);

/* Step 1: proxy map, importance, budget and every head's positions into the workspace. */
sd_status sparse_prefill_select(const sp_handle* h, const sp_tensors* t, void* ws, void* stream);

/* Step 2: compressed causal attention of every head over its positions, scattered into
 * out fp32 [B][Hq][L][d] (contiguous); positions a head did not keep are written as 0.
 * Arithmetic: q.k on bf16 inputs with fp32 accumulation; P.V in fp16 with fp32 accumulation (V
 * converted exactly under a power-of-two scale per KV head, P rounded to fp16), so an output
 * differs from exact attention by at most about 2^-11 times the head's max |v|. */
sd_status sparse_prefill_attend(const sp_handle* h, const sp_tensors* t, void* ws, float* out, void* stream);

/* Fill `view` with device pointers into `ws` (no device access). */
sd_status sparse_prefill_view(const sp_handle* h, void* ws, sp_view* view);

/* Release a handle (host memory only). NULL is ignored. */
void sparse_prefill_destroy(sp_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_PREFILL_H */

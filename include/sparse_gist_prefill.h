/*
 * sparse_gist_prefill.h -- C ABI of the gist-masked (SSA) block-sparse prefill attention of the
 * query-adaptive sparse attention library for AMD Instinct MI355X (gfx950).
 *
 * One prefill attention layer over a sequence of N raw tokens in M = N / C whole chunks, each
 * chunk followed by a gist token, following the review of "Simplified Sparse Attention"
 * (aitrends.kr, article 69798):
 *   - method / technical details: a gist token follows every chunk of C raw tokens, and the gist
 *     causal mask keeps a chunk's tokens from reaching the raw tokens of earlier chunks except
 *     through the gists. Read here as: causal in the interleaved order, and a raw key is visible
 *     only inside its own chunk. So raw token t (chunk m = t / C) attends to gists 0 .. m - 1 and
 *     raw tokens m C .. t; gist m attends to gists 0 .. m and the C raw tokens of chunk m.
 *   - contributions: the prefill kernel permutes the key columns into a block-sparse layout and
 *     skips the empty blocks. With the keys taken as [gists 0 .. M - 1 | raw tokens 0 .. N - 1]
 *     every query's visible keys are a prefix of the gists and a run of its own chunk's raw
 *     tokens; the kernel visits only the 64-key tiles that hold them.
 * Logits are softmax_scale * q . k (bf16 inputs, fp32 accumulation), softmax over the visible
 * keys, P.V in fp16 (see sparse_gist_prefill_attend), outputs fp32.
 *
 * Conventions are those of sparse_decode.h: tensors are DEVICE pointers owned by the caller,
 * calls only enqueue on `stream` and never synchronise, every argument check runs on the host
 * before anything is enqueued, and sparse_decode_last_error() reports the last failing call of
 * this thread. The attention call takes a caller-owned device workspace of the size init reports
 * (the library never allocates device memory).
 */
#ifndef SPARSE_GIST_PREFILL_H
#define SPARSE_GIST_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#include "sparse_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gp_handle gp_handle;

typedef struct {
  int32_t batch;          /* sequences B, >= 1 */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0; query head h uses KV head h / (Hq / Hkv) */
  int32_t head_dim;       /* d: 128 */
  int64_t n_tokens;       /* N raw tokens, a multiple of chunk_size, 1 .. 2^31 - 1 */
  int32_t chunk_size;     /* C >= 1 raw tokens per chunk; M = N / C gists */
  int32_t kv_dtype;       /* SD_BF16 */
  double softmax_scale;   /* logit scale, finite and > 0 (rounded to fp32) */
} gp_config;

/* Device tensors, bf16, last dimension contiguous, element strides multiple of 8 (16-byte rows).
 *   q     [B][Hq][N][d]    raw queries         strides q_sb, q_sh, q_st
 *   k, v  [B][Hkv][N][d]   raw keys / values   strides kv_sb, kv_sh, kv_st (shared)
 *   qg    [B][Hq][M][d]    gist queries        strides qg_sb, qg_sh, qg_st
 *   kg, vg [B][Hkv][M][d]  gist keys / values  strides kvg_sb, kvg_sh, kvg_st (shared) */
typedef struct {
  const void* q;  int64_t q_sb, q_sh, q_st;
  const void* k;  const void* v;  int64_t kv_sb, kv_sh, kv_st;
  const void* qg; int64_t qg_sb, qg_sh, qg_st;
  const void* kg; const void* vg; int64_t kvg_sb, kvg_sh, kvg_st;
} gp_tensors;

/* Validate and copy `cfg`, create a handle (host memory only) and report the bytes of device
 * workspace the attention call needs: an fp16 copy of every KV head's values (gists, then raw
 * tokens) scaled by a power of two, 2 (M + N) d bytes per (sequence, KV head), plus a few words
 * per head. Errors: SD_EINVAL (null pointer, inconsistent shape, n_tokens not a multiple of
 * chunk_size, bad scale), SD_EUNSUPPORTED (head_dim != 128, kv_dtype != SD_BF16). */
sd_status sparse_gist_prefill_init(const gp_config* cfg, gp_handle** out, size_t* workspace_bytes);

/* Attention of every raw and gist query over its visible keys. out fp32 [B][Hq][N][d] and
 * out_gist fp32 [B][Hq][M][d], both contiguous and 16-byte aligned, are written whole. `ws` is
 * the caller's device workspace (256-byte aligned, the size init reported; its contents on entry
 * do not matter). Arithmetic: q.k on bf16 inputs with fp32 accumulation; P.V in fp16 with fp32
 * accumulation (V converted under a power-of-two scale per KV head, exactly for every value down
 * to 2^-29 of the head's max |v|; P rounded to fp16 and the normaliser summed from the same
 * rounded values), so an output differs from exact attention by at most about 2^-11 times the
 * head's max |v|. Errors: SD_EINVAL (null or misaligned pointer, bad stride), SD_EWORKSPACE
 * (null or misaligned workspace), SD_EHIP (launch failure). */
sd_status sparse_gist_prefill_attend(const gp_handle* h, const gp_tensors* t, void* ws, float* out,
                                     float* out_gist, void* stream);

/* Release a handle (host memory only). NULL is ignored. */
void sparse_gist_prefill_destroy(gp_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_GIST_PREFILL_H */

// Host side of the C ABI: argument checks, workspace planning, dispatch.
// Every check runs before anything is enqueued; nothing here touches the GPU
// except through the launchers in sd_kernels.hip.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "sd_internal.h"
#include "sp_internal.h"
#include "gp_internal.h"

namespace {

thread_local char g_err[512] = "";

sd_status fail(sd_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sd_status ok() {
  g_err[0] = 0;
  return SD_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sd_status check_cfg(const sd_config& c) {
  if (c.batch < 1) return fail(SD_EINVAL, "batch must be >= 1 (got %d)", c.batch);
  if (c.kv_batch != 1 && c.kv_batch != c.batch)
    return fail(SD_EINVAL, "kv_batch must be 1 or batch (got %d, batch %d)", c.kv_batch, c.batch);
  if (c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_q_heads % c.n_kv_heads)
    return fail(SD_EINVAL, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", c.n_q_heads,
                c.n_kv_heads);
  if (c.n_kv_heads > sd::kMaxKvHeads)
    return fail(SD_EUNSUPPORTED, "n_kv_heads > %d", sd::kMaxKvHeads);
  if (c.n_queries < 0) return fail(SD_EINVAL, "n_queries must be >= 0 (got %d)", c.n_queries);
  {
    const int64_t T = c.n_queries > 1 ? c.n_queries : 1;
    const int64_t rows = T * (c.n_q_heads / c.n_kv_heads);
    if (rows > sd::kMaxGroup)
      return fail(SD_EUNSUPPORTED, "query rows per KV group (n_queries x group size) %lld > %d", (long long)rows,
                  sd::kMaxGroup);
    if (c.route == SD_ROUTE_PROXY && rows > sd::kMaxProxyGroup)
      return fail(SD_EUNSUPPORTED, "proxy routing: query rows per KV group %lld > %d", (long long)rows,
                  sd::kMaxProxyGroup);
  }
  if (c.head_dim != 64 && c.head_dim != 128) return fail(SD_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c.head_dim);
  if (c.kv_dtype != SD_F32 && c.kv_dtype != SD_BF16) return fail(SD_EINVAL, "kv_dtype %d unknown", c.kv_dtype);
  if (c.n_ctx < 1 || c.n_ctx >= (int64_t(1) << 31)) return fail(SD_EINVAL, "n_ctx out of range (%lld)", (long long)c.n_ctx);
  if (c.chunk_size < 1 || c.n_ctx % c.chunk_size)
    return fail(SD_EINVAL, "chunk_size %d must be >= 1 and divide n_ctx %lld", c.chunk_size, (long long)c.n_ctx);
  if (c.n_ctx / c.chunk_size > sd::kMaxRowEntries)
    return fail(SD_EUNSUPPORTED, "more than %lld selection entries (n_ctx / chunk_size) per row",
                (long long)sd::kMaxRowEntries);
  if (c.route != SD_ROUTE_SUMMARY && c.route != SD_ROUTE_PROXY) return fail(SD_EINVAL, "route %d unknown", c.route);
  if (c.mode != SD_TOPK && c.mode != SD_TOPP && c.mode != SD_HIER_TOPK && c.mode != SD_COVERAGE)
    return fail(SD_EINVAL, "mode %d unknown", c.mode);
  if (c.route == SD_ROUTE_PROXY) {
    if (c.chunk_size != 1) return fail(SD_EINVAL, "proxy routing scores tokens: chunk_size must be 1");
    if (c.route_dim != 16) return fail(SD_EUNSUPPORTED, "route_dim must be 16 (got %d)", c.route_dim);
    if (c.mode == SD_HIER_TOPK) return fail(SD_EUNSUPPORTED, "two-level selection routes on summary keys");
    if (c.attend_summary) return fail(SD_EINVAL, "token-level routing has no summary K/V to attend");
  }
  if (c.mode == SD_TOPK || c.mode == SD_HIER_TOPK) {
    if (c.top_k < 1) return fail(SD_EINVAL, "top_k must be >= 1 (got %d)", c.top_k);
  }
  if (c.mode == SD_COVERAGE) {
    if (!(c.tau >= 0.0) || !(c.tau < 1.0)) return fail(SD_EINVAL, "tau must be in [0, 1) (got %g)", c.tau);
    if (!(c.select_scale > 0.0) || !std::isfinite(c.select_scale))
      return fail(SD_EINVAL, "select_scale must be finite and > 0 (got %g)", c.select_scale);
    if (c.route != SD_ROUTE_SUMMARY) return fail(SD_EUNSUPPORTED, "the coverage budget routes on summary keys");
    if (c.n_ctx / c.chunk_size > sd::kSmallRowMax)
      return fail(SD_EUNSUPPORTED, "the coverage budget handles at most %d chunks per row", sd::kSmallRowMax);
  }
  if (c.mode == SD_TOPP) {
    if (!(c.top_p > 0.0) || !(c.top_p <= 1.0)) return fail(SD_EINVAL, "top_p must be in (0, 1] (got %g)", c.top_p);
    if (!(c.select_scale > 0.0) || !std::isfinite(c.select_scale))
      return fail(SD_EINVAL, "select_scale must be finite and > 0 (got %g)", c.select_scale);
  }
  if (c.mode == SD_HIER_TOPK) {
    const int64_t M = c.n_ctx / c.chunk_size;
    if (c.seg_size < 1 || M % c.seg_size) return fail(SD_EINVAL, "seg_size %d must divide the %lld chunks", c.seg_size, (long long)M);
    if (c.top_k_seg < 1) return fail(SD_EINVAL, "top_k_seg must be >= 1");
    const int64_t lim = sd::small_row_limit(c.n_q_heads / c.n_kv_heads);
    if (M / c.seg_size > lim) return fail(SD_EUNSUPPORTED, "more than %lld segments", (long long)lim);
    if (M > int64_t(32) * 4096) return fail(SD_EUNSUPPORTED, "two-level selection over more than %d chunks", 32 * 4096);
    if (int64_t(std::min<int64_t>(c.top_k_seg, M / c.seg_size)) * c.seg_size > lim)
      return fail(SD_EUNSUPPORTED, "top_k_seg * seg_size > %lld candidates", (long long)lim);
  }
  if (!(c.softmax_scale > 0.0f) || !std::isfinite(c.softmax_scale)) return fail(SD_EINVAL, "softmax_scale must be finite and > 0");
  if (c.keep_first < 0 || c.keep_last < 0) return fail(SD_EINVAL, "keep_first / keep_last must be >= 0");
  if (c.sink < 0 || c.window < 0) return fail(SD_EINVAL, "sink / window must be >= 0");
  if (c.attend_blocks < 0 || c.attend_blocks > 65536) return fail(SD_EINVAL, "attend_blocks must be in [0, 65536]");
  if (c.attend_summary < 0 || c.attend_summary > 2) return fail(SD_EINVAL, "attend_summary must be 0, 1 or 2");
  if (c.head_masks != 0 && c.head_masks != 1) return fail(SD_EINVAL, "head_masks must be 0 or 1");
  if (int64_t(c.batch) * c.n_kv_heads > sd::kMaxGroups)
    return fail(SD_EUNSUPPORTED, "batch * n_kv_heads > %d", sd::kMaxGroups);
  {
    const int64_t M = c.n_ctx / c.chunk_size;
    const int64_t tiles = int64_t(c.batch) * c.n_kv_heads * ((c.n_ctx + 15) / 16 + (M + 15) / 16 + 64);
    if (tiles >= (int64_t(1) << 30)) return fail(SD_EUNSUPPORTED, "too many attention tiles per call");
  }
  if (c.chunk_size & (c.chunk_size - 1)) return fail(SD_EUNSUPPORTED, "chunk_size must be a power of two (got %d)", c.chunk_size);
  bool any_local = false;
  if (c.head_mode) {
    for (int g = 0; g < c.n_kv_heads; ++g) {
      if (c.head_mode[g] != 0 && c.head_mode[g] != 1) return fail(SD_EINVAL, "head_mode[%d] = %d (must be 0 or 1)", g, c.head_mode[g]);
      any_local |= c.head_mode[g] == 1;
    }
  }
  if (any_local) {
    if (c.chunk_size != 1) return fail(SD_EINVAL, "local heads select tokens: chunk_size must be 1");
    if (c.sink + int64_t(c.window) < 1) return fail(SD_EINVAL, "local heads need sink + window >= 1");
  }
  return SD_OK;
}

void plan_workspace(sd::Plan& p) {
  const sd_config& c = p.cfg;
  const int64_t B = c.batch, Hq = c.n_q_heads, Hk = c.n_kv_heads, d = c.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  p.o_status = take(64);
  p.o_ctx = take(size_t(B) * 4);     // cache length per sequence, this step
  p.o_budget = take(size_t(B) * 4);  // coverage budget per sequence
  p.o_cmass = take(c.mode == SD_COVERAGE ? size_t(B * Hq * p.len0) * 8 : 0);  // per-head softmax masses
  p.o_cimp = take(c.mode == SD_COVERAGE ? size_t(B * p.len0) * 8 : 0);        // importance per entry
  p.o_csort = take(c.mode == SD_COVERAGE ? size_t(B * p.len0) * 8 : 0);       // importance, ascending
  p.n_arrive = int64_t(B) * Hk;
  p.o_arrive = take(size_t(p.n_arrive) * 4);
  p.o_qp = take(c.route == SD_ROUTE_PROXY ? size_t(B * Hq * 16) * 8 : 0);
  p.o_s0 = take(size_t(B * Hq * p.len0) * 8);
  p.o_s1 = take(size_t(B * Hq * p.len1) * 8);
  p.o_cand = take(size_t(B * Hq * p.len1) * 4);
  p.o_bits = take(size_t(B * Hq * p.words) * 4);
  p.o_ubits = take(size_t(B * Hk * p.words) * 4);
  p.o_rcnt = take(size_t(B * Hk * p.ranges) * 4);
  p.o_list = take(size_t(B * Hk * p.M) * 4);
  p.o_cnt = take(size_t(B * Hk) * 4);
  const size_t slots = size_t(p.attend_blocks) + size_t(B * Hk);
  p.o_gpre = take(size_t(B * Hk + 1) * 4);
  p.o_po = take(slots * p.G * d * 4);
  p.o_pl = take(slots * p.G * 4);
  const size_t rows = p.long0 ? size_t(B * Hq) : 0;
  // per-block score max / min: written by the proxy score pass, read by the long-row path
  const size_t mm_rows = (p.long0 || c.route == SD_ROUTE_PROXY) ? size_t(B * Hq) : 0;
  p.o_pmax = take(mm_rows * p.score_blocks0 * 8);
  p.o_pmin = take(mm_rows * p.score_blocks0 * 8);
  p.o_info = take(rows * sizeof(sd::RowInfo));
  p.o_h1h = take(rows * sd::kBins1 * 8);
  p.o_h1l = take(rows * sd::kBins1 * 8);
  p.o_h1c = take(rows * sd::kBins1 * 4);
  p.o_cbin = take(rows * ((p.len0 + 7) & ~int64_t(7)) * 2);
  p.o_cidx = take(rows * p.long_blocks * sd::kResolveCap * 4);
  p.o_ckey = take(rows * p.long_blocks * sd::kResolveCap * 8);
  p.o_ccnt = take(rows * p.long_blocks * 4);
  p.ws_bytes = off;
}

sd_status check_ws(const sd::Plan&, const void* ws) {
  if (!ws) return fail(SD_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SD_EWORKSPACE, "workspace not 256-byte aligned");
  return SD_OK;
}

sd_status check_tensors(const sd::Plan& p, const sd_tensors* t, bool for_score, int level) {
  const sd_config& c = p.cfg;
  if (!t) return fail(SD_EINVAL, "tensors is NULL");
  if (t->ctx_len) {
    if (reinterpret_cast<uintptr_t>(t->ctx_len) & 3u) return fail(SD_EINVAL, "ctx_len must be 4-byte aligned");
    if (c.mode == SD_HIER_TOPK)
      return fail(SD_EUNSUPPORTED, "per-sequence cache lengths (ctx_len) with two-level selection");
  }
  if (!t->q || !aligned16(t->q)) return fail(SD_EINVAL, "q must be a non-NULL 16-byte aligned pointer");
  const int es = c.kv_dtype == SD_F32 ? 4 : 2;
  auto row_ok = [&](int64_t st) { return st >= c.head_dim && (st * es) % 16 == 0; };
  if ((t->q_sh * es) % 16 || (t->q_sb * es) % 16 || t->q_sh < c.head_dim) return fail(SD_EINVAL, "q strides must keep 16-byte aligned rows");
  if (p.T > 1 && ((t->q_st * es) % 16 || t->q_st < c.head_dim)) return fail(SD_EINVAL, "q token stride must keep 16-byte aligned rows");
  if (for_score) {
    if (c.route == SD_ROUTE_PROXY) {
      if (!t->kp || !aligned16(t->kp)) return fail(SD_EINVAL, "proxy routing needs kp (16-byte aligned)");
      if (!t->proj || !aligned16(t->proj)) return fail(SD_EINVAL, "proxy routing needs proj (16-byte aligned)");
      if (t->kp_st < 16 || (t->kp_st * 2) % 16) return fail(SD_EINVAL, "kp token stride must keep 16-byte aligned rows");
    } else if (c.mode == SD_HIER_TOPK && level == 0) {
      if (!t->kmg || !aligned16(t->kmg) || !row_ok(t->mg_st)) return fail(SD_EINVAL, "two-level routing needs kmg with 16-byte aligned rows");
    } else {
      if (!t->kg || !aligned16(t->kg) || !row_ok(t->g_st)) return fail(SD_EINVAL, "summary routing needs kg with 16-byte aligned rows");
    }
  } else {
    if (!t->k || !t->v || !aligned16(t->k) || !aligned16(t->v) || !row_ok(t->kv_st))
      return fail(SD_EINVAL, "attend needs k and v with 16-byte aligned rows");
    if (c.attend_summary && (!t->kg || !t->vg || !aligned16(t->kg) || !aligned16(t->vg) || !row_ok(t->g_st)))
      return fail(SD_EINVAL, "attend_summary needs kg and vg with 16-byte aligned rows");
  }
  return SD_OK;
}

}  // namespace

extern "C" {

sd_status sparse_decode_init(const sd_config* cfg, sd_handle** out, size_t* workspace_bytes) {
  if (!cfg || !out || !workspace_bytes) return fail(SD_EINVAL, "init: NULL argument");
  *out = nullptr;
  sd_status st = check_cfg(*cfg);
  if (st != SD_OK) return st;
  sd_handle* h = new (std::nothrow) sd_handle();
  if (!h) return fail(SD_EINVAL, "init: out of host memory");
  sd::Plan& p = h->plan;
  p.cfg = *cfg;
  p.cfg.head_mode = nullptr;
  p.local_mask = 0;
  for (int g = 0; g < cfg->n_kv_heads; ++g) {
    p.head_mode[g] = cfg->head_mode ? cfg->head_mode[g] : 0;
    if (p.head_mode[g]) p.local_mask |= uint64_t(1) << g;
  }
  p.T = cfg->n_queries > 1 ? cfg->n_queries : 1;
  p.Gq = cfg->n_q_heads / cfg->n_kv_heads;
  p.Hq_user = cfg->n_q_heads;
  p.cfg.n_q_heads = p.T * cfg->n_q_heads;  // query rows per sequence (see Plan)
  const sd_config& c = p.cfg;
  p.G = c.n_q_heads / c.n_kv_heads;
  p.M = c.n_ctx / c.chunk_size;
  p.S = c.mode == SD_HIER_TOPK ? int32_t(p.M / c.seg_size) : 0;
  p.levels = c.mode == SD_HIER_TOPK ? 2 : 1;
  p.len0 = c.mode == SD_HIER_TOPK ? p.S : p.M;
  p.len1 = c.mode == SD_HIER_TOPK ? int64_t(std::min(c.top_k_seg, p.S)) * c.seg_size : 0;
  p.long0 = p.len0 > sd::small_row_limit(p.G);
  p.words = (p.M + 31) / 32;
  p.ranges = int32_t((p.words + 1023) / 1024);
  p.attend_blocks = c.attend_blocks ? c.attend_blocks : sd::kAttendBlocks;
  p.score_blocks0 = int32_t((p.len0 + sd::kMinMaxBlock - 1) / sd::kMinMaxBlock);
  p.n_scored = 0;
  for (int g = 0; g < c.n_kv_heads; ++g)
    if (!p.head_mode[g]) p.scored[p.n_scored++] = int8_t(g);
  p.long_blocks = int32_t((p.len0 + sd::kLongBlock - 1) / sd::kLongBlock);
  p.chunk_shift = 0;
  while ((int64_t(1) << p.chunk_shift) < c.chunk_size) ++p.chunk_shift;
  plan_workspace(p);
  *out = h;
  *workspace_bytes = p.ws_bytes;
  return ok();
}

int32_t sparse_decode_num_levels(const sd_handle* h) { return h ? h->plan.levels : 0; }

int32_t sparse_decode_attend_blocks(const sd_handle* h) { return h ? h->plan.attend_blocks : 0; }

sd_status sparse_decode_score_chunks(const sd_handle* h, const sd_tensors* t, int level, void* ws, void* stream) {
  if (!h) return fail(SD_EINVAL, "score: NULL handle");
  const sd::Plan& p = h->plan;
  if (level < 0 || level >= p.levels) return fail(SD_EINVAL, "score: level %d out of range [0, %d)", level, p.levels);
  sd_status st = check_ws(p, ws);
  if (st != SD_OK) return st;
  st = check_tensors(p, t, true, level);
  if (st != SD_OK) return st;
  int e = sd::launch_score(p, *t, level, static_cast<char*>(ws), stream);
  if (e) return fail(SD_EHIP, "score: HIP error %d (%s)", e, sd::hip_error_string(e));
  return ok();
}

sd_status sparse_decode_select(const sd_handle* h, int level, void* ws, void* stream) {
  if (!h) return fail(SD_EINVAL, "select: NULL handle");
  const sd::Plan& p = h->plan;
  if (level < 0 || level >= p.levels) return fail(SD_EINVAL, "select: level %d out of range [0, %d)", level, p.levels);
  sd_status st = check_ws(p, ws);
  if (st != SD_OK) return st;
  int e = sd::launch_select(p, level, static_cast<char*>(ws), stream);
  if (e) return fail(SD_EHIP, "select: HIP error %d (%s)", e, sd::hip_error_string(e));
  return ok();
}

sd_status sparse_decode_attend(const sd_handle* h, const sd_tensors* t, void* ws, void* stream) {
  if (!h) return fail(SD_EINVAL, "attend: NULL handle");
  const sd::Plan& p = h->plan;
  sd_status st = check_ws(p, ws);
  if (st != SD_OK) return st;
  st = check_tensors(p, t, false, 0);
  if (st != SD_OK) return st;
  int e = sd::launch_attend(p, *t, static_cast<char*>(ws), stream);
  if (e) return fail(SD_EHIP, "attend: HIP error %d (%s)", e, sd::hip_error_string(e));
  return ok();
}

sd_status sparse_decode_combine(const sd_handle* h, void* ws, float* out, float* lse_out, void* stream) {
  if (!h) return fail(SD_EINVAL, "combine: NULL handle");
  const sd::Plan& p = h->plan;
  sd_status st = check_ws(p, ws);
  if (st != SD_OK) return st;
  if (!out || !lse_out || !aligned16(out)) return fail(SD_EINVAL, "combine: out (16-byte aligned) and lse_out must be non-NULL");
  int e = sd::launch_combine(p, static_cast<char*>(ws), out, lse_out, stream);
  if (e) return fail(SD_EHIP, "combine: HIP error %d (%s)", e, sd::hip_error_string(e));
  return ok();
}

namespace {
// The whole step on `w`: score and select at every level, attend, combine. The tensors and outputs
// are checked first, so a rejected call enqueues nothing.
sd_status enqueue_step(const sd::Plan& p, const sd_tensors* t, char* w, float* out, float* lse_out, void* stream,
                       const char* who) {
  sd_status st;
  for (int level = 0; level < p.levels; ++level)
    if ((st = check_tensors(p, t, true, level)) != SD_OK) return st;
  if ((st = check_tensors(p, t, false, 0)) != SD_OK) return st;
  if (!out || !lse_out || !aligned16(out))
    return fail(SD_EINVAL, "%s: out (16-byte aligned) and lse_out must be non-NULL", who);
  int e = 0;
  for (int level = 0; level < p.levels && !e; ++level) {
    e = sd::launch_score(p, *t, level, w, stream);
    if (!e) e = sd::launch_select(p, level, w, stream);
  }
  if (!e) e = sd::launch_attend(p, *t, w, stream);
  if (!e) e = sd::launch_combine(p, w, out, lse_out, stream);
  if (e) return fail(SD_EHIP, "%s: HIP error %d (%s)", who, e, sd::hip_error_string(e));
  return ok();
}
}  // namespace

sd_status sparse_decode_step(const sd_handle* h, const sd_tensors* t, void* ws, float* out, float* lse_out,
                             void* stream) {
  if (!h) return fail(SD_EINVAL, "step: NULL handle");
  const sd::Plan& p = h->plan;
  sd_status st = check_ws(p, ws);
  if (st != SD_OK) return st;
  return enqueue_step(p, t, static_cast<char*>(ws), out, lse_out, stream, "step");
}

sd_status sparse_decode_step_static(const sd_handle* h, const sd_tensors* t, float* out, float* lse_out,
                                    void* stream) {
  if (!h) return fail(SD_EINVAL, "step_static: NULL handle");
  const sd::Plan& p = h->plan;
  if (p.ws_bytes > sd::kStaticScratchBytes)
    return fail(SD_EUNSUPPORTED, "step_static: the step needs a %zu-byte workspace, above the %zu-byte static scratch",
                p.ws_bytes, sd::kStaticScratchBytes);
  // the tensors are checked before the scratch address is looked up (nothing touches the GPU on a
  // rejected call)
  sd_status st;
  for (int level = 0; level < p.levels; ++level)
    if ((st = check_tensors(p, t, true, level)) != SD_OK) return st;
  if ((st = check_tensors(p, t, false, 0)) != SD_OK) return st;
  if (!out || !lse_out || !aligned16(out))
    return fail(SD_EINVAL, "step_static: out (16-byte aligned) and lse_out must be non-NULL");
  void* ws = nullptr;
  int e = sd::static_scratch(&ws);
  if (e) return fail(SD_EHIP, "step_static: static scratch address: HIP error %d (%s)", e, sd::hip_error_string(e));
  return enqueue_step(p, t, static_cast<char*>(ws), out, lse_out, stream, "step_static");
}

sd_status sparse_decode_selection_view(const sd_handle* h, void* ws, sd_selection_view* v) {
  if (!h || !v) return fail(SD_EINVAL, "selection_view: NULL argument");
  const sd::Plan& p = h->plan;
  sd_status st = check_ws(p, ws);
  if (st != SD_OK) return st;
  char* w = static_cast<char*>(ws);
  v->scores0 = reinterpret_cast<const double*>(w + p.o_s0);
  v->len0 = p.len0;
  v->scores1 = reinterpret_cast<const double*>(w + p.o_s1);
  v->len1 = p.len1;
  v->cand1 = reinterpret_cast<const int32_t*>(w + p.o_cand);
  v->head_bits = reinterpret_cast<const uint32_t*>(w + p.o_bits);
  v->words = p.words;
  v->list = reinterpret_cast<const int32_t*>(w + p.o_list);
  v->n_entries = p.M;
  v->count = reinterpret_cast<const int32_t*>(w + p.o_cnt);
  v->status = reinterpret_cast<const uint32_t*>(w + p.o_status);
  return ok();
}

// ---- Token-Sparse prefill
sd_status sparse_prefill_init(const sp_config* cfg, sp_handle** out, size_t* workspace_bytes) {
  if (!cfg || !out || !workspace_bytes) return fail(SD_EINVAL, "prefill init: NULL argument");
  *out = nullptr;
  const sp_config& c = *cfg;
  if (c.batch < 1) return fail(SD_EINVAL, "batch must be >= 1 (got %d)", c.batch);
  if (c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_q_heads % c.n_kv_heads)
    return fail(SD_EINVAL, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", c.n_q_heads, c.n_kv_heads);
  if (c.head_dim != 128) return fail(SD_EUNSUPPORTED, "prefill: head_dim must be 128 (got %d)", c.head_dim);
  if (c.kv_dtype != SD_BF16) return fail(SD_EUNSUPPORTED, "prefill: kv_dtype must be SD_BF16");
  if (c.window < 1) return fail(SD_EINVAL, "window must be >= 1 (got %d)", c.window);
  if (c.window > sd::kPfMaxWindow) return fail(SD_EUNSUPPORTED, "window must be <= %d (got %d)", sd::kPfMaxWindow, c.window);
  if (c.seq_len < c.window || c.seq_len >= (int64_t(1) << 31))
    return fail(SD_EINVAL, "seq_len must be in [window, 2^31) (got %lld)", (long long)c.seq_len);
  if (c.seq_len > sd::kMaxRowEntries)
    return fail(SD_EUNSUPPORTED, "seq_len above %lld (selection rows)", (long long)sd::kMaxRowEntries);
  if (!(c.tau >= 0.0) || !(c.tau < 1.0)) return fail(SD_EINVAL, "tau must be in [0, 1) (got %g)", c.tau);
  if (!(c.softmax_scale > 0.0) || !std::isfinite(c.softmax_scale))
    return fail(SD_EINVAL, "softmax_scale must be finite and > 0 (got %g)", c.softmax_scale);
  if (int64_t(c.batch) * c.n_q_heads * c.seq_len * c.window >= (int64_t(1) << 40))
    return fail(SD_EUNSUPPORTED, "batch x heads x seq_len x window too large");
  sp_handle* h = new (std::nothrow) sp_handle();
  if (!h) return fail(SD_EINVAL, "prefill init: out of host memory");
  sd::PrefillPlan& p = h->plan;
  p.cfg = c;
  p.G = c.n_q_heads / c.n_kv_heads;
  p.L = c.seq_len;
  p.words = (p.L + 31) / 32;
  p.nslab = int32_t((p.L + sd::kPfSlab - 1) / sd::kPfSlab);
  p.nkb = int32_t((p.L + sd::kPfKeyBlock - 1) / sd::kPfKeyBlock);
  const int64_t B = c.batch, Hq = c.n_q_heads, L = p.L, W = c.window;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  p.o_status = take(64);
  p.Lpad = (L + sd::kPfKeyTile - 1) / sd::kPfKeyTile * sd::kPfKeyTile;
  // the proxy scores are dead once the selection is made: attend gathers every head's K and V
  // rows into the same region
  p.o_S = take(std::max(size_t(B * Hq * L * W) * 8, size_t(B * Hq * p.Lpad) * size_t(c.head_dim) * 2 * 2));
  p.o_kvc = p.o_S;
  p.o_pmq = take(size_t(B * Hq * p.nkb * W) * 8);
  p.o_zb = take(size_t(B * Hq * p.nkb * W) * 8);
  p.o_M = take(size_t(B * Hq * W) * 8);
  p.o_zq = take(size_t(B * Hq * p.nslab * W) * 8);
  p.o_imp = take(size_t(B * Hq * L) * 8);
  p.o_pmax = take(size_t(B * Hq * p.nslab) * 8);
  p.o_pmin = take(size_t(B * Hq * p.nslab) * 8);
  p.o_gimp = take(size_t(B * L) * 8);
  p.o_gpmax = take(size_t(B * p.nslab) * 8);
  p.o_gpmin = take(size_t(B * p.nslab) * 8);
  p.o_long = take(sd::long_rows_scratch(B * Hq, L));
  p.o_bbits = take(size_t(B * p.words) * 4);
  p.o_budget = take(size_t(B) * 4);
  p.o_bits = take(size_t(B * Hq * p.words) * 4);
  p.o_list = take(size_t(B * Hq * L) * 4);
  p.o_vmaxp = take(size_t(B * c.n_kv_heads * p.nslab) * 4);
  p.o_vexp = take(size_t(B * Hq) * 4);
  p.ws_bytes = off;
  *out = h;
  *workspace_bytes = p.ws_bytes;
  return ok();
}

namespace {
sd_status check_prefill_tensors(const sd::PrefillPlan& p, const sp_tensors* t) {
  if (!t) return fail(SD_EINVAL, "prefill: tensors is NULL");
  if (!t->q || !t->k || !t->v || !aligned16(t->q) || !aligned16(t->k) || !aligned16(t->v))
    return fail(SD_EINVAL, "prefill: q, k and v must be non-NULL 16-byte aligned pointers");
  const int64_t d = p.cfg.head_dim;
  auto ok8 = [](int64_t x) { return x >= 0 && x % 8 == 0; };
  if (!ok8(t->q_sb) || !ok8(t->q_sh) || !ok8(t->q_st) || t->q_st < d)
    return fail(SD_EINVAL, "prefill: q strides must keep 16-byte aligned rows");
  if (!ok8(t->kv_sb) || !ok8(t->kv_sh) || !ok8(t->kv_st) || t->kv_st < d)
    return fail(SD_EINVAL, "prefill: k / v strides must keep 16-byte aligned rows");
  return SD_OK;
}
}  // namespace

sd_status sparse_prefill_select(const sp_handle* h, const sp_tensors* t, void* ws, void* stream) {
  if (!h) return fail(SD_EINVAL, "prefill select: NULL handle");
  if (!ws) return fail(SD_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SD_EWORKSPACE, "workspace not 256-byte aligned");
  sd_status st = check_prefill_tensors(h->plan, t);
  if (st != SD_OK) return st;
  int e = sd::launch_prefill_select(h->plan, *t, static_cast<char*>(ws), stream);
  if (e) return fail(SD_EHIP, "prefill select: HIP error %d (%s)", e, sd::hip_error_string(e));
  return ok();
}

sd_status sparse_prefill_attend(const sp_handle* h, const sp_tensors* t, void* ws, float* out, void* stream) {
  if (!h) return fail(SD_EINVAL, "prefill attend: NULL handle");
  if (!ws) return fail(SD_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SD_EWORKSPACE, "workspace not 256-byte aligned");
  sd_status st = check_prefill_tensors(h->plan, t);
  if (st != SD_OK) return st;
  if (!out || !aligned16(out)) return fail(SD_EINVAL, "prefill attend: out must be a non-NULL 16-byte aligned pointer");
  int e = sd::launch_prefill_attend(h->plan, *t, static_cast<char*>(ws), out, stream);
  if (e) return fail(SD_EHIP, "prefill attend: HIP error %d (%s)", e, sd::hip_error_string(e));
  return ok();
}

sd_status sparse_prefill_view(const sp_handle* h, void* ws, sp_view* v) {
  if (!h || !v) return fail(SD_EINVAL, "prefill view: NULL argument");
  if (!ws) return fail(SD_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SD_EWORKSPACE, "workspace not 256-byte aligned");
  const sd::PrefillPlan& p = h->plan;
  char* w = static_cast<char*>(ws);
  v->importance = reinterpret_cast<const double*>(w + p.o_imp);
  v->budget = reinterpret_cast<const int32_t*>(w + p.o_budget);
  v->head_bits = reinterpret_cast<const uint32_t*>(w + p.o_bits);
  v->words = p.words;
  v->list = reinterpret_cast<const int32_t*>(w + p.o_list);
  v->status = reinterpret_cast<const uint32_t*>(w + p.o_status);
  return ok();
}

void sparse_prefill_destroy(sp_handle* h) { delete h; }

// ---- gist-masked (SSA) prefill
sd_status sparse_gist_prefill_init(const gp_config* cfg, gp_handle** out, size_t* workspace_bytes) {
  if (!cfg || !out || !workspace_bytes) return fail(SD_EINVAL, "gist prefill init: NULL argument");
  *out = nullptr;
  *workspace_bytes = 0;
  const gp_config& c = *cfg;
  if (c.batch < 1) return fail(SD_EINVAL, "batch must be >= 1 (got %d)", c.batch);
  if (c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_q_heads % c.n_kv_heads)
    return fail(SD_EINVAL, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", c.n_q_heads, c.n_kv_heads);
  if (c.head_dim != 128) return fail(SD_EUNSUPPORTED, "gist prefill: head_dim must be 128 (got %d)", c.head_dim);
  if (c.kv_dtype != SD_BF16) return fail(SD_EUNSUPPORTED, "gist prefill: kv_dtype must be SD_BF16");
  if (c.chunk_size < 1) return fail(SD_EINVAL, "chunk_size must be >= 1 (got %d)", c.chunk_size);
  if (c.n_tokens < 1 || c.n_tokens >= (int64_t(1) << 31))
    return fail(SD_EINVAL, "n_tokens must be in [1, 2^31) (got %lld)", (long long)c.n_tokens);
  if (c.n_tokens % c.chunk_size)
    return fail(SD_EINVAL, "n_tokens (%lld) must be a multiple of chunk_size (%d)", (long long)c.n_tokens, c.chunk_size);
  if (!(c.softmax_scale > 0.0) || !std::isfinite(c.softmax_scale))
    return fail(SD_EINVAL, "softmax_scale must be finite and > 0 (got %g)", c.softmax_scale);
  gp_handle* h = new (std::nothrow) gp_handle();
  if (!h) return fail(SD_EINVAL, "gist prefill init: out of host memory");
  sd::GistPlan& p = h->plan;
  p.cfg = c;
  p.G = c.n_q_heads / c.n_kv_heads;
  p.M = int32_t(c.n_tokens / c.chunk_size);
  p.R = p.M + c.n_tokens;
  p.nslab = int32_t((p.R + sd::kGpSlab - 1) / sd::kGpSlab);
  const int64_t heads = int64_t(c.batch) * c.n_kv_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  p.o_vmaxp = take(size_t(heads * p.nslab) * 4);
  p.o_vexp = take(size_t(heads) * 4);
  p.o_vc = take(size_t(heads * p.R) * size_t(c.head_dim) * 2);
  p.ws_bytes = off;
  *workspace_bytes = off;
  *out = h;
  return ok();
}

sd_status sparse_gist_prefill_attend(const gp_handle* h, const gp_tensors* t, void* ws, float* out, float* out_gist,
                                     void* stream) {
  if (!h) return fail(SD_EINVAL, "gist prefill attend: NULL handle");
  if (!ws) return fail(SD_EWORKSPACE, "gist prefill attend: workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SD_EWORKSPACE, "gist prefill attend: workspace not 256-byte aligned");
  if (!t) return fail(SD_EINVAL, "gist prefill attend: tensors is NULL");
  const void* ptrs[6] = {t->q, t->k, t->v, t->qg, t->kg, t->vg};
  for (const void* ptr : ptrs)
    if (!ptr || !aligned16(ptr))
      return fail(SD_EINVAL, "gist prefill: q, k, v, qg, kg and vg must be non-NULL 16-byte aligned pointers");
  const int64_t d = h->plan.cfg.head_dim;
  auto ok8 = [](int64_t x) { return x >= 0 && x % 8 == 0; };
  auto rows_ok = [&](int64_t sb, int64_t sh, int64_t st) { return ok8(sb) && ok8(sh) && ok8(st) && st >= d; };
  if (!rows_ok(t->q_sb, t->q_sh, t->q_st) || !rows_ok(t->kv_sb, t->kv_sh, t->kv_st) ||
      !rows_ok(t->qg_sb, t->qg_sh, t->qg_st) || !rows_ok(t->kvg_sb, t->kvg_sh, t->kvg_st))
    return fail(SD_EINVAL, "gist prefill: strides must be multiples of 8 elements with rows of at least head_dim");
  if (!out || !out_gist || !aligned16(out) || !aligned16(out_gist))
    return fail(SD_EINVAL, "gist prefill attend: out and out_gist must be non-NULL 16-byte aligned pointers");
  int e = sd::launch_gist_prefill(h->plan, *t, static_cast<char*>(ws), out, out_gist, stream);
  if (e) return fail(SD_EHIP, "gist prefill attend: HIP error %d (%s)", e, sd::hip_error_string(e));
  return ok();
}

void sparse_gist_prefill_destroy(gp_handle* h) { delete h; }

const char* sparse_decode_last_error(void) { return g_err; }

void sparse_decode_destroy(sd_handle* h) { delete h; }

}  // extern "C"

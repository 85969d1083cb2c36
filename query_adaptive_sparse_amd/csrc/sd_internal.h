// Internal decode plan shared by the host API (sd_api.cpp) and the decode kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/sparse_decode.h"

namespace sd {

// Rows up to this length are selected by one workgroup sorting them in LDS;
// longer rows (token-level selection) take the histogram path.
constexpr int kSmallRowMax = 2048;
constexpr int64_t small_row_limit(int) { return kSmallRowMax; }

// Long-row path: coarse bins over the row's score range (per-slab partial histograms); the
// crossing coarse bin's entries (at most kResolveCap of them, else a fine split first) are
// resolved exactly in one workgroup.
constexpr int kBins1 = 1024;
constexpr int kBins2 = 4096;
constexpr int kResolveCap = 4096;
// Most entries in one selection row: the exact fixed-point mass sums of the selection kernels
// (2^39 and 2^40 units per weight in two 64-bit words) hold up to 2^24 weights.
constexpr int64_t kMaxRowEntries = int64_t(1) << 24;
// Entries per workgroup ("slab") in the long-row histogram and marking passes.
constexpr int kLongBlock = 32768;
// Entries per partial max / min written by the score passes of long rows.
constexpr int kMinMaxBlock = 2048;
// Attention: tokens per MFMA tile and waves per workgroup.
constexpr int kTile = 16;
constexpr int kWaves = 4;
// Query rows per KV group (T query tokens x G heads), and the limit of the proxy score kernel.
constexpr int kMaxGroup = 16;
constexpr int kMaxProxyGroup = 8;
constexpr int kMaxKvHeads = 64;
// Attention: persistent workgroups (default: one per CU of a 256-CU MI355X) and the most
// (sequence, KV group) pairs per call.
constexpr int kAttendBlocks = 256;
constexpr int kMaxGroups = 4096;

struct Plan {
  sd_config cfg;
  int8_t head_mode[kMaxKvHeads];
  uint64_t local_mask;      // bit g set: KV head g is a local (sink + window) head
  // T query tokens per sequence run as T x Hq query rows: cfg.n_q_heads holds T x Hq and G the
  // rows per KV group, T x Gq, ordered token-major inside the group (row g G + t Gq + j is token
  // t, head g Gq + j)
  int32_t G;                // query rows per KV head
  int32_t T, Gq, Hq_user;   // query tokens per sequence, heads per KV head, heads
  int64_t M;                // chunks = n_ctx / chunk_size (selection entries)
  int32_t S;                // segments (two-level)
  int32_t levels;
  int64_t len0, len1;       // row lengths of level-0 / level-1 scores
  bool long0;               // level-0 rows take the long-row (histogram) path
  int64_t words;            // bitmap words per row = ceil(M / 32)
  int32_t ranges;           // union compaction ranges per group
  int32_t attend_blocks;    // persistent attention workgroups
  int32_t score_blocks0;    // partial max / min per long row (kMinMaxBlock entries each)
  int32_t long_blocks;      // slabs per long row (kLongBlock entries each)
  int32_t n_scored;         // KV groups that are scored (not local)
  int8_t scored[kMaxKvHeads];  // their indices, ascending
  // workspace byte offsets
  size_t o_status, o_arrive, o_qp, o_s0, o_s1, o_cand, o_bits, o_ubits, o_rcnt, o_list, o_cnt;
  size_t o_gpre, o_po, o_pl, o_pmax, o_pmin, o_info, o_h1h, o_h1l, o_h1c, o_cbin, o_cidx, o_ckey, o_ccnt, o_budget, o_cmass, o_cimp, o_csort;
  size_t o_ctx;        // int32 [B]: the step's cache length per sequence (published by the score pass)
  int32_t chunk_shift; // log2(chunk_size)
  int64_t n_arrive;  // arrival counters: one per (sequence, KV group)
  size_t ws_bytes;
};

// Per-row state of the long-row selection, in the workspace.
struct RowInfo {
  double smax, smin, binscale;  // score range and coarse-bin scale
  double target;                // p * Z (top-p) or k (top-k)
  double before1;               // weight of everything ahead of the crossing coarse bin
  int32_t bin1;                 // crossing coarse bin
  int32_t all;                  // 1: the whole row is selected
  int32_t wexp;                 // masses of an `ident` row are held as value * 2^-wexp (< 1)
  int32_t pad;
};

// The static device scratch of sparse_decode_step_static (sd_static.hip): its size, and its device
// address on the current device (looked up once per device); returns hipSuccess or the error.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
int static_scratch(void** out);

// Kernel launchers (sd_score.hip, sd_select.hip, sd_attend.hip). Each returns hipSuccess or the
// launch error.
int launch_score(const Plan& p, const sd_tensors& t, int level, char* ws, void* stream);
int launch_select(const Plan& p, int level, char* ws, void* stream);
int launch_attend(const Plan& p, const sd_tensors& t, char* ws, void* stream);
int launch_combine(const Plan& p, char* ws, float* out, float* lse, void* stream);
const char* hip_error_string(int code);


}  // namespace sd

struct sd_handle {
  sd::Plan plan;
};

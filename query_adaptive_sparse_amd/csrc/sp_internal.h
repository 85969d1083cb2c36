// Internal plan of the Token-Sparse prefill path, shared by the host API (sd_api.cpp) and the
// prefill kernels (sd_prefill.hip).
#pragma once

#include "long_rows.h"
#include "../../include/sparse_prefill.h"

namespace sd {

constexpr int kPfSlab = kMinMaxBlock;  // keys per importance workgroup (and per partial max / min)
constexpr int kPfKeyBlock = 64;        // keys per proxy-score workgroup
constexpr int kPfMaxWindow = 64;
constexpr int kPfWaves = 8;            // waves per attention workgroup, 32 compact queries each
constexpr int kPfQueryBlock = 32 * kPfWaves;  // compact queries per attention workgroup
constexpr int kPfKeyTile = 64;         // compact keys per attention step (gathered rows are padded to it)

struct PrefillPlan {
  sp_config cfg;
  int32_t G;
  int64_t L, words;
  int64_t Lpad;        // L rounded up to kPfKeyTile: rows per head of the gathered K / V
  int32_t nslab, nkb;  // importance slabs, proxy-score key blocks
  size_t o_status, o_S, o_pmq, o_zb, o_M, o_zq, o_imp, o_pmax, o_pmin, o_gimp, o_gpmax, o_gpmin;
  size_t o_long, o_bbits, o_budget, o_bits, o_list;
  size_t o_kvc;    // gathered K (bf16) then V (fp16, scaled) rows [B][Hq][Lpad][d]; shares the region of S
  size_t o_vmaxp;  // float [B][Hkv][nslab]: max |v| per slab of each KV head's rows
  size_t o_vexp;   // int32 [B][Hq]: the power of two the head's gathered V rows are scaled by
  size_t ws_bytes;
};
int launch_prefill_select(const PrefillPlan& p, const sp_tensors& t, char* ws, void* stream);
int launch_prefill_attend(const PrefillPlan& p, const sp_tensors& t, char* ws, float* out, void* stream);

}  // namespace sd

struct sp_handle {
  sd::PrefillPlan plan;
};

// Internal plan of the gist-masked (SSA) prefill path, shared by the host API (sd_api.cpp) and its
// kernel (sd_gist.hip).
#pragma once

#include "sd_internal.h"
#include "../../include/sparse_gist_prefill.h"

namespace sd {

// Rows of one KV head's fp16 value copy: its M gist rows, then its N raw rows. Rows per workgroup of
// the max |v| pass (16 loads in flight per thread).
constexpr int kGpSlab = 256;

struct GistPlan {
  gp_config cfg;
  int32_t G, M;   // query heads per KV head, gists (chunks)
  int64_t R;      // rows per KV head of the value copy, M + N
  int32_t nslab;  // max |v| partials per KV head
  // workspace byte offsets: max |v| partials (fp32 [B][Hkv][nslab]), the scale exponent per KV
  // head (int32 [B][Hkv]), the scaled fp16 values ([B][Hkv][R][d])
  size_t o_vmaxp, o_vexp, o_vc, ws_bytes;
};
int launch_gist_prefill(const GistPlan& p, const gp_tensors& t, char* ws, float* out, float* out_gist, void* stream);

}  // namespace sd

struct gp_handle {
  sd::GistPlan plan;
};

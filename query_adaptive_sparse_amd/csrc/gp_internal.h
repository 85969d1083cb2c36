// Internal plan of the gist-masked (SSA) prefill path, shared by the host API (sd_api.cpp) and its
// kernel (sd_gist.hip).
#pragma once

#include "sd_internal.h"
#include "../../include/sparse_gist_prefill.h"

namespace sd {

struct GistPlan {
  gp_config cfg;
  int32_t G, M;  // query heads per KV head, gists (chunks)
};
int launch_gist_prefill(const GistPlan& p, const gp_tensors& t, float* out, float* out_gist, void* stream);

}  // namespace sd

struct gp_handle {
  sd::GistPlan plan;
};

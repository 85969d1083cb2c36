// Long-row selection over caller-given fp64 rows, used by the prefill path (sd_select.hip runs it).
#pragma once

#include "sd_internal.h"

namespace sd {

// Long-row selection (histogram passes) over caller-given fp64 rows s [B][H][len]: top-k (k, or
// kbudget[b] for every row of sequence b when non-null) with unit weights, or top-p of the
// weights exp(scale (s - smax)), or (ident) of the values themselves as masses (s >= 0).
// pmax / pmin hold each row's max / min per kMinMaxBlock entries. Writes the selection bitmaps
// bits [B][H][words] (whole words) and raises status[0] for an incomplete row.
struct LongRows {
  const double* s;
  int64_t len;
  int B, H;
  int topp, ident, k;
  int bitbins;  // values are >= 0: bin them by their bit patterns (16 bins per binade below the row max)
  const int32_t* kbudget;
  double p, scale;
  const double* pmax;
  const double* pmin;
  int nblk;
  char* scratch;  // long_rows_scratch(B * H, len) bytes, 256-byte aligned
  uint32_t* bits;
  int64_t words;
  uint32_t* status;
};
size_t long_rows_scratch(int64_t rows, int64_t len);
int launch_long_rows(const LongRows& r, void* stream);

}  // namespace sd

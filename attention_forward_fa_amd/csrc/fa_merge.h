// Internal: parameters of the partial-result merge kernel.  Plain C++ (no
// HIP types) so the host planner builds with any C++ compiler.
#pragma once

#include <stdint.h>

namespace fa {

constexpr int kMergeMaxParts = 16;

struct MergeParams {
  int32_t nparts, dv;
  int32_t nbatch, nheads, nrows;  // rows per (batch, head); TND: batch 1, rows = T
  // partial outputs (the output's dtype) and their statistics (fp32, 8 slots)
  const void* po[kMergeMaxParts];
  int64_t po_sb[kMergeMaxParts], po_ss[kMergeMaxParts], po_sh[kMergeMaxParts];
  const float* pm[kMergeMaxParts];
  const float* pl[kMergeMaxParts];
  int64_t pst_sb[kMergeMaxParts], pst_ss[kMergeMaxParts], pst_sh[kMergeMaxParts];
  // merged output and (optional) statistics
  void* o;
  int64_t o_sb, o_ss, o_sh;
  float* m;  // may be null
  float* l;  // may be null
  int64_t st_sb, st_ss, st_sh;
};

// Enqueue the merge on `stream` (a hipStream_t); returns 0 or a HIP error code.
int merge_launch(const MergeParams& mp, int32_t dtype, void* stream);

}  // namespace fa

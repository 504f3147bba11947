// Internal: per-family launchers called by phase 2.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_fwd.h"
#include "fa_params.h"

namespace fa {

hipError_t launch_mfma_bf16(const Params& p, hipStream_t s);
hipError_t launch_mfma_f16(const Params& p, hipStream_t s);
hipError_t launch_mfma_pp_bf16(const Params& p, hipStream_t s);
hipError_t launch_mfma_pp_f16(const Params& p, hipStream_t s);
hipError_t launch_generic(const Params& p, int dtype, hipStream_t s);
// merge of the key ranges of a split grid (kv_splits > 1; bf16 / fp16)
hipError_t launch_split_merge(const Params& p, int dtype, hipStream_t s);

}  // namespace fa

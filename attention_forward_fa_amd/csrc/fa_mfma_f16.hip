// fp16 instantiations of the matrix-core forward kernels.
#include "fa_mfma_dispatch.hpp"

namespace fa {

hipError_t launch_mfma_f16(const Params& p, hipStream_t s) { return launch_mfma_t<_Float16>(p, s); }
hipError_t launch_mfma_pp_f16(const Params& p, hipStream_t s) { return launch_mfma_pp_t<_Float16>(p, s); }

}  // namespace fa

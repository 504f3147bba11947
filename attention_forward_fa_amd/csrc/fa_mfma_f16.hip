// fp16 instantiations of the matrix-core forward kernel.
#include "fa_launch.h"
#include "fa_mfma.hpp"
#include "fa_mfma_pp.hpp"

namespace fa {

template <typename T>
static hipError_t launch_mfma_pp_t(const Params& p, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  const void* fn = nullptr;
  if (p.d == 128 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 128, 0>);
  else if (p.d == 128 && p.dr == 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 128, 64>);
  else if (p.d == 64 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 64, 0>);
  else if (p.d == 64 && p.dr == 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 64, 64>);
  else
    return hipErrorInvalidValue;
  return hipLaunchKernel(fn, dim3(p.num_wg), dim3(kPpThreads), args, 0, s);
}

template <typename T>
static hipError_t launch_mfma_t(const Params& p, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  const void* fn = nullptr;
  if (p.pse_lds && p.d == 128 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 128, 0, true>);
  else if (p.pse_lds && p.d == 64 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 64, 0, true>);
  else if (p.d == 128 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 128, 0>);
  else if (p.d == 128 && p.dr == 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 128, 64>);
  else if (p.d == 64 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 64, 0>);
  else if (p.d == 64 && p.dr == 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 64, 64>);
  else if (p.pse_lds && p.d == 96 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 96, 0, true>);
  else if (p.d == 96 && p.dr == 0)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 96, 0>);
  else if (p.d == 96 && p.dr == 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma<T, 96, 64>);
  else
    return hipErrorInvalidValue;
  return hipLaunchKernel(fn, dim3(p.num_wg), dim3(kMfmaThreads), args, 0, s);
}

hipError_t launch_mfma_f16(const Params& p, hipStream_t s) { return launch_mfma_t<_Float16>(p, s); }
hipError_t launch_mfma_pp_f16(const Params& p, hipStream_t s) { return launch_mfma_pp_t<_Float16>(p, s); }

}  // namespace fa

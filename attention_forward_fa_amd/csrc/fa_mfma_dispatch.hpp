// Launchers of the matrix-core forward kernels for one element type T
// (bf16 or fp16): the (D, Dr, Dv) instantiations phase 1 may plan, each
// element-type translation unit instantiating them once.
#pragma once

#include "fa_launch.h"
#include "fa_mfma.hpp"
#include "fa_mfma_pp.hpp"

namespace fa {

template <typename T>
hipError_t launch_mfma_pp_t(const Params& p, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  const void* fn = nullptr;
  if (p.d == 128 && p.dr == 0 && p.dv == 128)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 128, 0>);
  else if (p.d == 128 && p.dr == 64 && p.dv == 128)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 128, 64>);
  else if (p.d == 64 && p.dr == 0 && p.dv == 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 64, 0>);
  else if (p.d == 64 && p.dr == 64 && p.dv == 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_mfma_pp<T, 64, 64>);
  else
    return hipErrorInvalidValue;
  return hipLaunchKernel(fn, dim3(p.num_wg), dim3(kPpThreads), args, 0, s);
}

// The four-wave kernel's instantiation for (D, DR, DV, PL), or null.
template <typename T, int D, int DR, int DV>
const void* mfma_fn_if(const Params& p) {
  if (p.d != D || p.dr != DR || p.dv != DV) return nullptr;
  if constexpr (DR == 0) {
    if (p.pse_lds) return reinterpret_cast<const void*>(&fa_fwd_mfma<T, D, DR, DV, true>);
  }
  return reinterpret_cast<const void*>(&fa_fwd_mfma<T, D, DR, DV, false>);
}

template <typename T>
hipError_t launch_mfma_t(const Params& p, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  const void* fn = nullptr;
  // Dv == D, with or without 64 rope dims; without rope, D in {96, 128, 256}
  // with any smaller Dv in {64, 96, 128}
  for (const void* f : {mfma_fn_if<T, 128, 0, 128>(p), mfma_fn_if<T, 128, 64, 128>(p), mfma_fn_if<T, 64, 0, 64>(p),
                        mfma_fn_if<T, 64, 64, 64>(p), mfma_fn_if<T, 96, 0, 96>(p), mfma_fn_if<T, 96, 64, 96>(p),
                        mfma_fn_if<T, 256, 0, 256>(p), mfma_fn_if<T, 256, 0, 128>(p), mfma_fn_if<T, 256, 0, 96>(p),
                        mfma_fn_if<T, 256, 0, 64>(p), mfma_fn_if<T, 128, 0, 96>(p), mfma_fn_if<T, 128, 0, 64>(p),
                        mfma_fn_if<T, 96, 0, 64>(p)})
    if (f) fn = f;
  if (!fn) return hipErrorInvalidValue;
  return hipLaunchKernel(fn, dim3(p.num_wg), dim3(kMfmaThreads), args, 0, s);
}

}  // namespace fa

// Merge of partial forward results: one query chunk computed against several
// key chunks (an outer split along the key sequence) combined into the result
// over all keys.  With m_c, l_c the row's statistics over chunk c (natural-log
// units) and O_c its normalised output,
//
//     m = max_c m_c,   w_c = e^(m_c - m) l_c,   l = sum_c w_c,
//     O = sum_c w_c O_c / l,
//
// which follows from the definitions of softmaxMax and softmaxSum in the sink
// equations of the aclnnFlashAttentionVarLenScoreV5 page.  Chunks with no kept
// key (m_c = -inf, l_c = 0) weigh 0; a row empty in every chunk gets O = 0,
// m = -inf, l = 0.  Memory-bound: one wavefront per row, lanes along Dv.
#include <hip/hip_runtime.h>

#include "fa_device.hpp"
#include "fa_fwd.h"
#include "fa_merge.h"

namespace fa {

template <typename T>
__global__ void __launch_bounds__(256) fa_merge_kernel(const MergeParams mp) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // flat (batch, head, row)
  const int64_t per_b = (int64_t)mp.nheads * mp.nrows;
  if (r >= per_b * mp.nbatch) return;
  const int b = (int)(r / per_b);
  const int h = (int)((r - b * per_b) / mp.nrows);
  const int s = (int)(r - b * per_b - (int64_t)h * mp.nrows);

  float mc[kMergeMaxParts], lc[kMergeMaxParts];
  float m = kNegInf;
  for (int c = 0; c < mp.nparts; ++c) {
    const int64_t si = b * mp.pst_sb[c] + h * mp.pst_sh[c] + s * mp.pst_ss[c];
    mc[c] = mp.pm[c][si];
    lc[c] = mp.pl[c][si];
    m = fmaxf(m, mc[c]);
  }
  float l = 0.f;
  for (int c = 0; c < mp.nparts; ++c) {
    lc[c] = mc[c] == kNegInf ? 0.f : expf(mc[c] - m) * lc[c];  // the weight w_c
    l += lc[c];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* o = static_cast<T*>(mp.o) + b * mp.o_sb + h * mp.o_sh + s * mp.o_ss;
  for (int d = lane; d < mp.dv; d += 64) {
    float acc = 0.f;
    for (int c = 0; c < mp.nparts; ++c) {
      const T* oc = static_cast<const T*>(mp.po[c]) + b * mp.po_sb[c] + h * mp.po_sh[c] + s * mp.po_ss[c];
      acc = fmaf(lc[c], to_f32(oc[d]), acc);
    }
    o[d] = from_f32<T>(acc * inv);
  }
  if (lane < 8) {
    const int64_t so = b * mp.st_sb + h * mp.st_sh + s * mp.st_ss + lane;
    if (mp.m) mp.m[so] = m;
    if (mp.l) mp.l[so] = l;
  }
}

int merge_launch(const MergeParams& mp, int32_t dtype, void* stream) {
  const int64_t rows = (int64_t)mp.nbatch * mp.nheads * mp.nrows;
  if (rows == 0) return 0;
  void* args[] = {const_cast<MergeParams*>(&mp)};
  const void* fn = nullptr;
  switch (dtype) {
    case FA_DTYPE_F32: fn = reinterpret_cast<const void*>(&fa_merge_kernel<float>); break;
    case FA_DTYPE_F16: fn = reinterpret_cast<const void*>(&fa_merge_kernel<_Float16>); break;
    case FA_DTYPE_BF16: fn = reinterpret_cast<const void*>(&fa_merge_kernel<__bf16>); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipLaunchKernel(fn, dim3((unsigned)((rows + 3) / 4)), dim3(256), args, 0,
                              static_cast<hipStream_t>(stream));
}

}  // namespace fa

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
// m = -inf, l = 0.  Memory-bound: with 16-byte aligned rows a thread merges
// 8 consecutive output elements (one 16-byte load per part), otherwise one
// wavefront per row with lanes along Dv.
#include <hip/hip_runtime.h>

#include "fa_device.hpp"
#include "fa_fwd.h"
#include "fa_launch.h"
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

// Row weights of the parts: w_c = e^(m_c - m) l_c (0 for an empty part).
__device__ __forceinline__ void merge_weights(const MergeParams& mp, int b, int h, int s, float (&w)[kMergeMaxParts],
                                              float& m, float& l) {
  float mc[kMergeMaxParts];
  m = kNegInf;
  for (int c = 0; c < mp.nparts; ++c) {
    const int64_t si = b * mp.pst_sb[c] + h * mp.pst_sh[c] + s * mp.pst_ss[c];
    mc[c] = mp.pm[c][si];
    w[c] = mp.pl[c][si];
    m = fmaxf(m, mc[c]);
  }
  l = 0.f;
  for (int c = 0; c < mp.nparts; ++c) {
    w[c] = mc[c] == kNegInf ? 0.f : expf(mc[c] - m) * w[c];
    l += w[c];
  }
}

// 16-byte path with a fixed count of NP parts: thread = (row, 8-element
// chunk).  Every load of the thread (the NP chunks and the NP statistics
// pairs) is issued before any is used, and the output leaves with the
// non-temporal hint (nothing reads it again here).
template <typename T, int NP>
__global__ void __launch_bounds__(256) fa_merge_vec_np_kernel(const MergeParams mp) {
  const int cpr = mp.dv / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = t / cpr;
  const int chunk = (int)(t - r * cpr);
  const int64_t per_b = (int64_t)mp.nheads * mp.nrows;
  if (r >= per_b * mp.nbatch) return;
  const int b = (int)(r / per_b);
  const int h = (int)((r - b * per_b) / mp.nrows);
  const int s = (int)(r - b * per_b - (int64_t)h * mp.nrows);
  uint4 u[NP];
  float mc[NP], w[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const T* oc = static_cast<const T*>(mp.po[c]) + b * mp.po_sb[c] + h * mp.po_sh[c] + s * mp.po_ss[c] + 8 * chunk;
    u[c] = *reinterpret_cast<const uint4*>(oc);
    const int64_t si = b * mp.pst_sb[c] + h * mp.pst_sh[c] + s * mp.pst_ss[c];
    mc[c] = mp.pm[c][si];
    w[c] = mp.pl[c][si];
  }
  float m = kNegInf;
#pragma unroll
  for (int c = 0; c < NP; ++c) m = fmaxf(m, mc[c]);
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    w[c] = mc[c] == kNegInf ? 0.f : expf(mc[c] - m) * w[c];
    l += w[c];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const T* e = reinterpret_cast<const T*>(&u[c]);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[c], to_f32(e[i]), acc[i]);
  }
  T res[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) res[i] = from_f32<T>(acc[i] * inv);
  T* o = static_cast<T*>(mp.o) + b * mp.o_sb + h * mp.o_sh + s * mp.o_ss + 8 * chunk;
  nt_store16(o, *reinterpret_cast<const uint4*>(res));
  if (chunk == 0) {
    const int64_t so = b * mp.st_sb + h * mp.st_sh + s * mp.st_ss;
    if (mp.m) {
      nt_store4f(mp.m + so, m);
      nt_store4f(mp.m + so + 4, m);
    }
    if (mp.l) {
      nt_store4f(mp.l + so, l);
      nt_store4f(mp.l + so + 4, l);
    }
  }
}

// 16-byte path, any part count: thread = (row, 8-element chunk); rows of dv / 8 chunks.
template <typename T>
__global__ void __launch_bounds__(256) fa_merge_vec_kernel(const MergeParams mp) {
  const int cpr = mp.dv / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = t / cpr;
  const int chunk = (int)(t - r * cpr);
  const int64_t per_b = (int64_t)mp.nheads * mp.nrows;
  if (r >= per_b * mp.nbatch) return;
  const int b = (int)(r / per_b);
  const int h = (int)((r - b * per_b) / mp.nrows);
  const int s = (int)(r - b * per_b - (int64_t)h * mp.nrows);
  float w[kMergeMaxParts], m, l;
  merge_weights(mp, b, h, s, w, m, l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < mp.nparts; ++c) {
    const T* oc = static_cast<const T*>(mp.po[c]) + b * mp.po_sb[c] + h * mp.po_sh[c] + s * mp.po_ss[c] + 8 * chunk;
    const uint4 u = *reinterpret_cast<const uint4*>(oc);
    const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[c], to_f32(e[i]), acc[i]);
  }
  T res[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) res[i] = from_f32<T>(acc[i] * inv);
  T* o = static_cast<T*>(mp.o) + b * mp.o_sb + h * mp.o_sh + s * mp.o_ss + 8 * chunk;
  *reinterpret_cast<uint4*>(o) = *reinterpret_cast<const uint4*>(res);
  if (chunk == 0) {
    const int64_t so = b * mp.st_sb + h * mp.st_sh + s * mp.st_ss;
    if (mp.m) {
      reinterpret_cast<float4*>(mp.m + so)[0] = make_float4(m, m, m, m);
      reinterpret_cast<float4*>(mp.m + so)[1] = make_float4(m, m, m, m);
    }
    if (mp.l) {
      reinterpret_cast<float4*>(mp.l + so)[0] = make_float4(l, l, l, l);
      reinterpret_cast<float4*>(mp.l + so)[1] = make_float4(l, l, l, l);
    }
  }
}

// Whether every row the merge touches is 16-byte aligned (outputs) and the
// statistics rows are 16-byte aligned (8 fp32 slots).
template <typename T>
static bool merge_vec_ok(const MergeParams& mp) {
  if (sizeof(T) != 2 || mp.dv % 8 != 0) return false;
  auto al = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; };
  auto st = [](int64_t x) { return x % 8 == 0; };
  for (int c = 0; c < mp.nparts; ++c)
    if (!al(mp.po[c]) || !st(mp.po_sb[c]) || !st(mp.po_sh[c]) || !st(mp.po_ss[c])) return false;
  if (!al(mp.o) || !st(mp.o_sb) || !st(mp.o_sh) || !st(mp.o_ss)) return false;
  const bool stats_ok = (!mp.m || al(mp.m)) && (!mp.l || al(mp.l));
  return stats_ok && (mp.st_sb % 4 == 0) && (mp.st_sh % 4 == 0) && (mp.st_ss % 4 == 0);
}

template <typename T>
static const void* merge_vec_fn(int nparts) {
  switch (nparts) {
    case 2: return reinterpret_cast<const void*>(&fa_merge_vec_np_kernel<T, 2>);
    case 3: return reinterpret_cast<const void*>(&fa_merge_vec_np_kernel<T, 3>);
    case 4: return reinterpret_cast<const void*>(&fa_merge_vec_np_kernel<T, 4>);
    default: return reinterpret_cast<const void*>(&fa_merge_vec_kernel<T>);
  }
}

int merge_launch(const MergeParams& mp, int32_t dtype, void* stream) {
  const int64_t rows = (int64_t)mp.nbatch * mp.nheads * mp.nrows;
  if (rows == 0) return 0;
  void* args[] = {const_cast<MergeParams*>(&mp)};
  const void* fn = nullptr;
  if (dtype == FA_DTYPE_BF16 && merge_vec_ok<__bf16>(mp)) fn = merge_vec_fn<__bf16>(mp.nparts);
  if (dtype == FA_DTYPE_F16 && merge_vec_ok<_Float16>(mp)) fn = merge_vec_fn<_Float16>(mp.nparts);
  if (fn) {
    const int64_t threads = rows * (mp.dv / 8);
    return (int)hipLaunchKernel(fn, dim3((unsigned)((threads + 255) / 256)), dim3(256), args, 0,
                                static_cast<hipStream_t>(stream));
  }
  switch (dtype) {
    case FA_DTYPE_F32: fn = reinterpret_cast<const void*>(&fa_merge_kernel<float>); break;
    case FA_DTYPE_F16: fn = reinterpret_cast<const void*>(&fa_merge_kernel<_Float16>); break;
    case FA_DTYPE_BF16: fn = reinterpret_cast<const void*>(&fa_merge_kernel<__bf16>); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipLaunchKernel(fn, dim3((unsigned)((rows + 3) / 4)), dim3(256), args, 0,
                              static_cast<hipStream_t>(stream));
}

// Key-split merge of the 4-wave kernel: the same combination over the
// kv_splits fp32 partial results of each query row (workspace, rows in
// (sequence, head, row) order), written to the output in its layout and dtype
// with the statistics.  Thread = (row, 8-element chunk).
template <typename T>
__global__ void __launch_bounds__(256) fa_split_merge_kernel(const Params p) {
  const int cpr = p.dv / 8;
  const int64_t rows = (int64_t)p.nbatch * p.nq * p.sq;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = t / cpr;
  const int chunk = (int)(t - r * cpr);
  if (r >= rows) return;
  const int64_t bh = r / p.sq;
  const int s = (int)(r - bh * p.sq);
  const int b = (int)(bh / p.nq), h = (int)(bh - (int64_t)b * p.nq);
  float w[kMaxKvSplits], mc[kMaxKvSplits];
  float m = kNegInf;
#pragma unroll
  for (int c = 0; c < kMaxKvSplits; ++c) {
    if (c < p.kv_splits) {
      const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + 2 * (c * rows + r));
      mc[c] = ml.x;
      w[c] = ml.y;
      m = fmaxf(m, ml.x);
    }
  }
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxKvSplits; ++c) {
    if (c < p.kv_splits) {
      w[c] = mc[c] == kNegInf ? 0.f : expf(mc[c] - m) * w[c];
      l += w[c];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kMaxKvSplits; ++c) {
    if (c < p.kv_splits) {
      const float4* pc = reinterpret_cast<const float4*>(p.part_o + (c * rows + r) * p.dv + 8 * chunk);
      const float4 a = pc[0], e = pc[1];
      acc[0] = fmaf(w[c], a.x, acc[0]);
      acc[1] = fmaf(w[c], a.y, acc[1]);
      acc[2] = fmaf(w[c], a.z, acc[2]);
      acc[3] = fmaf(w[c], a.w, acc[3]);
      acc[4] = fmaf(w[c], e.x, acc[4]);
      acc[5] = fmaf(w[c], e.y, acc[5]);
      acc[6] = fmaf(w[c], e.z, acc[6]);
      acc[7] = fmaf(w[c], e.w, acc[7]);
    }
  }
  T res[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) res[i] = from_f32<T>(acc[i] * inv);
  T* o = static_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh + s * p.o_ss + 8 * chunk;
  *reinterpret_cast<uint4*>(o) = *reinterpret_cast<const uint4*>(res);
  if (chunk == 0) {
    const int64_t so = b * p.st_sb + h * p.st_sh + s * p.st_ss;
    if (p.smax) {
      reinterpret_cast<float4*>(p.smax + so)[0] = make_float4(m, m, m, m);
      reinterpret_cast<float4*>(p.smax + so)[1] = make_float4(m, m, m, m);
    }
    if (p.ssum) {
      reinterpret_cast<float4*>(p.ssum + so)[0] = make_float4(l, l, l, l);
      reinterpret_cast<float4*>(p.ssum + so)[1] = make_float4(l, l, l, l);
    }
  }
}

hipError_t launch_split_merge(const Params& p, int dtype, hipStream_t s) {
  const int64_t threads = (int64_t)p.nbatch * p.nq * p.sq * (p.dv / 8);
  if (threads == 0) return hipSuccess;
  void* args[] = {const_cast<Params*>(&p)};
  const void* fn = dtype == FA_DTYPE_BF16 ? reinterpret_cast<const void*>(&fa_split_merge_kernel<__bf16>)
                                          : reinterpret_cast<const void*>(&fa_split_merge_kernel<_Float16>);
  return hipLaunchKernel(fn, dim3((unsigned)((threads + 255) / 256)), dim3(256), args, 0, s);
}

}  // namespace fa

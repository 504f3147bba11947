// Phase 2 of the two-phase forward: enqueue the planned kernels on a stream.
#include <stdio.h>

#include "fa_launch.h"
#include "fa_plan.h"
#include "fa_device.hpp"

namespace fa {

// tile_prefix[b] = sum over sequences before b of ceil(rows / bm); one workgroup.
__global__ void __launch_bounds__(256) varlen_tile_prefix(const int32_t* __restrict__ cu, int total, int nbatch, int bm,
                                                         int32_t* __restrict__ prefix) {
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int per = (nbatch + 255) / 256;
  const int b0 = min(tid * per, nbatch), b1 = min(b0 + per, nbatch);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += (seq_rows(cu, b, total) + bm - 1) / bm;
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = part[i];
      part[i] = acc;
      acc += v;
    }
  }
  __syncthreads();
  int acc = part[tid];
  for (int b = b0; b < b1; ++b) {
    prefix[b] = acc;
    acc += (seq_rows(cu, b, total) + bm - 1) / bm;
  }
  if (b1 == nbatch && b0 < b1) prefix[nbatch] = acc;
  if (nbatch == 0 && tid == 0) prefix[0] = 0;
}

// pse_off[b] = sum over sequences before b of N * rows_q * rows_kv: where
// sequence b's [N, Sq_b, Skv_b] block starts in a flat TND pse.  One workgroup.
__global__ void __launch_bounds__(256) varlen_pse_prefix(const int32_t* __restrict__ cu_q,
                                                        const int32_t* __restrict__ cu_kv, int tq, int tkv,
                                                        int nbatch, int nq, int64_t* __restrict__ off) {
  __shared__ int64_t part[256];
  const int tid = threadIdx.x;
  const int per = (nbatch + 255) / 256;
  const int b0 = min(tid * per, nbatch), b1 = min(b0 + per, nbatch);
  auto size = [&](int b) { return (int64_t)nq * seq_rows(cu_q, b, tq) * seq_rows(cu_kv, b, tkv); };
  int64_t s = 0;
  for (int b = b0; b < b1; ++b) s += size(b);
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int64_t v = part[i];
      part[i] = acc;
      acc += v;
    }
  }
  __syncthreads();
  int64_t acc = part[tid];
  for (int b = b0; b < b1; ++b) {
    off[b] = acc;
    acc += size(b);
  }
  if (b1 == nbatch && b0 < b1) off[nbatch] = acc;
  if (nbatch == 0 && tid == 0) off[0] = 0;
}

}  // namespace fa

namespace {

fa_status runtime_fail(const char* what, hipError_t e) {
  char buf[256];
  snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
  fa_set_error(buf);
  return FA_ERR_RUNTIME;
}

}  // namespace

extern "C" fa_status fa_fwd(void* workspace, uint64_t workspace_size, const fa_plan* plan, void* stream) {
  if (!plan) {
    fa_set_error("plan is NULL");
    return FA_ERR_PARAM_NULLPTR;
  }
  if (plan->ws_bytes > 0 && (!workspace || workspace_size < plan->ws_bytes)) {
    char buf[128];
    snprintf(buf, sizeof(buf), "workspace needs %llu bytes, got %llu at %p", (unsigned long long)plan->ws_bytes,
             (unsigned long long)workspace_size, workspace);
    fa_set_error(buf);
    return FA_ERR_WORKSPACE;
  }
  fa::Params p = plan->p;
  if (p.varlen && p.has_pse && (reinterpret_cast<uintptr_t>(workspace) & 7u)) {
    fa_set_error("workspace must be 8-byte aligned (TND with real_shift)");
    return FA_ERR_WORKSPACE;
  }
  if (p.num_wg == 0) return FA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.varlen) {
    p.tile_prefix = static_cast<int32_t*>(workspace);
    void* args[] = {(void*)&p.cu_q, (void*)&p.tq, (void*)&p.nbatch, (void*)&plan->bm, (void*)&p.tile_prefix};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::varlen_tile_prefix), dim3(1), dim3(256), args, 0, s);
    if (e != hipSuccess) return runtime_fail("tile prefix launch", e);
    if (p.has_pse) {
      const uintptr_t o = ((uintptr_t)(p.nbatch + 1) * sizeof(int32_t) + 7) / 8 * 8;
      p.pse_off = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + o);
      void* pargs[] = {(void*)&p.cu_q, (void*)&p.cu_kv, (void*)&p.tq, (void*)&p.tkv, (void*)&p.nbatch, (void*)&p.nq,
                       (void*)&p.pse_off};
      e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::varlen_pse_prefix), dim3(1), dim3(256), pargs, 0, s);
      if (e != hipSuccess) return runtime_fail("pse prefix launch", e);
    }
  }
  hipError_t e;
  if (plan->kind == fa::KERNEL_MFMA_PP)
    e = plan->dtype == FA_DTYPE_BF16 ? fa::launch_mfma_pp_bf16(p, s) : fa::launch_mfma_pp_f16(p, s);
  else if (plan->kind == fa::KERNEL_MFMA)
    e = plan->dtype == FA_DTYPE_BF16 ? fa::launch_mfma_bf16(p, s) : fa::launch_mfma_f16(p, s);
  else
    e = fa::launch_generic(p, plan->dtype, s);
  if (e != hipSuccess) return runtime_fail("forward kernel launch", e);
  return FA_OK;
}

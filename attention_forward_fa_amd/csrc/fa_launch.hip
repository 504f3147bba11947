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
  if (p.num_wg == 0) return FA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.varlen) {
    p.tile_prefix = static_cast<int32_t*>(workspace);
    void* args[] = {(void*)&p.cu_q, (void*)&p.tq, (void*)&p.nbatch, (void*)&plan->bm, (void*)&p.tile_prefix};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::varlen_tile_prefix), dim3(1), dim3(256), args, 0, s);
    if (e != hipSuccess) return runtime_fail("tile prefix launch", e);
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

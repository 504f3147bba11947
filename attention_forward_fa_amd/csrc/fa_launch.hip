// Phase 2 of the two-phase forward: enqueue the planned kernels on a stream.
#include <stdio.h>

#include <mutex>

#include "fa_launch.h"
#include "fa_plan.h"
#include "fa_device.hpp"

namespace fa {

// tile_prefix[b] = sum over sequences before b of ceil(rows / bm), then the
// tile map built from it; one workgroup.
__global__ void __launch_bounds__(256) varlen_tile_prefix(const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_kv,
                                                         int total, int tkv, int nbatch, int bm, int tph, int reverse,
                                                         int32_t* __restrict__ prefix, int32_t* __restrict__ map) {
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int per = (nbatch + 255) / 256;
  const int b0 = min(tid * per, nbatch), b1 = min(b0 + per, nbatch);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += seq_tiles(cu, b, total, bm);
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
    acc += seq_tiles(cu, b, total, bm);
  }
  if (b1 == nbatch && b0 < b1) prefix[nbatch] = acc;
  if (nbatch == 0 && tid == 0) prefix[0] = 0;
  __syncthreads();  // the prefix is visible to the whole workgroup

  // The tile map: entry r of the grid's per-head tile index (r < tph) holds
  // the sequence b, its query tile qt and the clamped row / key ranges of the
  // tile it runs; heavier (later) tiles first when `reverse`.  Entries past
  // the total are marked invalid.
  for (int r = threadIdx.x; r < tph; r += 256) {
    int32_t e[8];
    tile_entry(prefix, cu, cu_kv, nbatch, total, tkv, reverse, r, e);
    reinterpret_cast<int4*>(map)[2 * r] = make_int4(e[0], e[1], e[2], e[3]);
    reinterpret_cast<int4*>(map)[2 * r + 1] = make_int4(e[4], e[5], e[6], e[7]);
  }
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

// Mask block classes: one workgroup per (slice, 128-row tile, 64-key block).
// A position counts when it lies inside [rows, cols); for the 2-D TND mask
// (outside_excluded) positions beyond it count as excluded by the mask, as
// the kernels read them.  With the window active (band), a position the
// window excludes is excluded whatever the mask says.  Class: EXCLUDED when
// no counted position survives both; KEPT when the mask excludes no position
// the window keeps (the block then needs no mask bytes, only the window
// tests the kernels do anyway); MIXED otherwise.
__global__ void __launch_bounds__(256) mask_classify(const uint8_t* __restrict__ mask, int64_t m_sb, int64_t m_sh,
                                                     int64_t m_sq, int64_t m_sk, int nh, int rows, int cols,
                                                     int tiles, int kblocks, int outside_excluded, int vec, int band,
                                                     int pre, int next, uint8_t* __restrict__ cls) {
  const int64_t id = blockIdx.x;
  const int kb = (int)(id % kblocks);
  const int t = (int)((id / kblocks) % tiles);
  const int64_t slice = id / ((int64_t)kblocks * tiles);
  const int mb = (int)(slice / nh), mh = (int)(slice % nh);
  const uint8_t* base = mask + mb * m_sb + mh * m_sh;
  // thread: row tid / 2 of the tile, keys 32 (tid % 2) .. +31 of the block
  const int r = t * kClsRows + (threadIdx.x >> 1);
  const int c0 = kb * kClsKeys + 32 * (threadIdx.x & 1);
  // the window keeps keys [r - pre, r + next] of row r
  const bool win_all = !band || (c0 + 31 - r <= next && r - c0 <= pre);
  const bool win_none = band && (c0 - r > next || r - (c0 + 31) > pre);
  bool alive = false, relevant = false;  // kept by both; excluded by the mask only
  if (win_none) {
    // nothing in this segment survives the window
  } else if (win_all && vec && r < rows && c0 + 32 <= cols) {
    // 32 contiguous bytes of the row: two 16-byte loads
    const uint4* src = reinterpret_cast<const uint4*>(base + (int64_t)r * m_sq + c0);
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      alive |= ((w[i] - 0x01010101u) & ~w[i] & 0x80808080u) != 0;  // some byte is 0
      relevant |= w[i] != 0;
    }
  } else {
    for (int c = c0; c < c0 + 32; ++c) {
      const bool win = !band || (c - r <= next && r - c <= pre);
      const bool inside = r < rows && c < cols;
      if (inside) {
        const bool e = base[(int64_t)r * m_sq + (int64_t)c * m_sk] != 0;
        alive |= !e && win;
        relevant |= e && win;
      } else if (outside_excluded) {
        relevant |= win;
      }
    }
  }
  const int any_alive = __syncthreads_or(alive);
  const int any_relevant = __syncthreads_or(relevant);
  if (threadIdx.x == 0) cls[id] = any_alive ? (any_relevant ? CLS_MIXED : CLS_KEPT) : CLS_EXCLUDED;
}

// Shader-clock probe: one wave reads the shader clock counter (s_memtime)
// and the constant 100 MHz counter (s_memrealtime) while it idles for `ticks`
// of the latter (or at most `cap` sleep rounds), then writes both deltas.
__global__ void __launch_bounds__(64) clock_probe(unsigned long long ticks, unsigned int cap,
                                                 unsigned long long* __restrict__ out) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r = r0;
  for (unsigned int n = 0; r - r0 < ticks && n < cap; ++n) {
    __builtin_amdgcn_s_sleep(8);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r - r0;
  }
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

namespace {

// Enqueue the planned kernels with `workspace` (at least plan->ws_bytes,
// 16-byte aligned, or unused when that is 0) as their scratch memory.
fa_status enqueue(const fa_plan* plan, void* workspace, void* stream) {
  fa::Params p = plan->p;
  if (p.num_wg == 0) return FA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.has_mask && plan->kind != fa::KERNEL_GENERIC) {  // the generic kernel reads the mask everywhere
    p.mask_cls = static_cast<uint8_t*>(workspace) + plan->ws_cls_off;
    const int64_t per_slice = (int64_t)p.cls_tiles * p.cls_kblocks;
    const int64_t blocks = (int64_t)p.cls_slices * per_slice;
    if (blocks >= ((int64_t)1 << 31)) {
      fa_set_error("mask too large to classify");
      return FA_ERR_RUNTIME;
    }
    const int rows = p.varlen ? p.m_rows : p.sq, cols = p.varlen ? p.m_cols : p.skv;
    const int outside = p.varlen;
    // rows of contiguous bytes, 16-byte aligned: vector loads
    const int vec = p.m_sk == 1 && (reinterpret_cast<uintptr_t>(p.mask) & 15u) == 0 && p.m_sq % 16 == 0 &&
                    p.m_sb % 16 == 0 && p.m_sh % 16 == 0;
    if (blocks > 0) {
      void* cargs[] = {(void*)&p.mask, (void*)&p.m_sb, (void*)&p.m_sh, (void*)&p.m_sq, (void*)&p.m_sk, (void*)&p.cls_nh,
                       (void*)&rows, (void*)&cols, (void*)&p.cls_tiles, (void*)&p.cls_kblocks, (void*)&outside,
                       (void*)&vec, (void*)&p.band, (void*)&p.pre, (void*)&p.next, (void*)&p.mask_cls};
      hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::mask_classify), dim3((unsigned)blocks),
                                     dim3(256), cargs, 0, s);
      if (e != hipSuccess) return runtime_fail("mask classification launch", e);
    }
  }
  if (p.varlen) {
    if (!p.tile_search) {
      p.tile_prefix = static_cast<int32_t*>(workspace);
      p.tile_map = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan->ws_map_off);
      void* args[] = {(void*)&p.cu_q,           (void*)&p.cu_kv,          (void*)&p.tq,      (void*)&p.tkv,
                      (void*)&p.nbatch,         (void*)&plan->bm,         (void*)&p.tiles_per_head,
                      (void*)&p.reverse_tiles,  (void*)&p.tile_prefix,    (void*)&p.tile_map};
      hipError_t e =
          hipLaunchKernel(reinterpret_cast<const void*>(&fa::varlen_tile_prefix), dim3(1), dim3(256), args, 0, s);
      if (e != hipSuccess) return runtime_fail("tile map launch", e);
    }
    if (p.has_pse) {
      p.pse_off = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + plan->ws_pse_off);
      void* pargs[] = {(void*)&p.cu_q, (void*)&p.cu_kv, (void*)&p.tq, (void*)&p.tkv, (void*)&p.nbatch, (void*)&p.nq,
                       (void*)&p.pse_off};
      hipError_t e =
          hipLaunchKernel(reinterpret_cast<const void*>(&fa::varlen_pse_prefix), dim3(1), dim3(256), pargs, 0, s);
      if (e != hipSuccess) return runtime_fail("pse prefix launch", e);
    }
  }
  if (p.kv_splits > 1) {
    p.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->ws_part_off);
    p.part_ml = p.part_o + (int64_t)p.kv_splits * p.nbatch * p.nq * p.sq * p.dv;
  }
  hipError_t e;
  if (plan->kind == fa::KERNEL_MFMA_PP)
    e = plan->dtype == FA_DTYPE_BF16 ? fa::launch_mfma_pp_bf16(p, s) : fa::launch_mfma_pp_f16(p, s);
  else if (plan->kind == fa::KERNEL_MFMA)
    e = plan->dtype == FA_DTYPE_BF16 ? fa::launch_mfma_bf16(p, s) : fa::launch_mfma_f16(p, s);
  else
    e = fa::launch_generic(p, plan->dtype, s);
  if (e != hipSuccess) return runtime_fail("forward kernel launch", e);
  if (p.kv_splits > 1) {
    e = fa::launch_split_merge(p, plan->dtype, s);
    if (e != hipSuccess) return runtime_fail("key split merge launch", e);
  }
  return FA_OK;
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
  if (plan->ws_bytes > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15u)) {
    fa_set_error("workspace must be 16-byte aligned");
    return FA_ERR_WORKSPACE;
  }
  return enqueue(plan, workspace, stream);
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: the library's own scratch array
// ---------------------------------------------------------------------------

namespace {

// Device scratch for fa_fwd_noalloc, one copy per GPU the library runs on,
// held until the process ends.  On the host this name is only a stand-in for
// the symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device (with that
// device current, as it is for the caller's stream).
fa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return runtime_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) {
    fa_set_error("device index beyond the scratch table");
    return FA_ERR_RUNTIME;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return runtime_fail("hipGetSymbolAddress(scratch)", e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" fa_status fa_fwd_noalloc(const fa_plan* plan, void* stream) {
  if (!plan) {
    fa_set_error("plan is NULL");
    return FA_ERR_PARAM_NULLPTR;
  }
  if (plan->ws_bytes > FA_NOALLOC_SCRATCH_BYTES) {
    char buf[160];
    snprintf(buf, sizeof(buf), "plan needs %llu bytes of scratch, above the %llu the no-allocation entry point holds",
             (unsigned long long)plan->ws_bytes, (unsigned long long)FA_NOALLOC_SCRATCH_BYTES);
    fa_set_error(buf);
    return FA_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  if (plan->ws_bytes > 0) {
    const fa_status st = scratch_for_current_device(&ws);
    if (st != FA_OK) return st;
  }
  return enqueue(plan, ws, stream);
}

extern "C" fa_status fa_clock_probe(uint32_t microseconds, unsigned long long* device_out, void* stream) {
  if (!device_out) {
    fa_set_error("device_out is NULL");
    return FA_ERR_PARAM_NULLPTR;
  }
  if (microseconds < 1 || microseconds > 1000000) {
    fa_set_error("microseconds must be in 1..1000000");
    return FA_ERR_UNSUPPORTED;
  }
  unsigned long long ticks = 100ull * microseconds;  // 100 MHz counter
  // one sleep round is at least 8 x 64 shader cycles (over 0.1 us at up to
  // 3 GHz), so this many rounds outlast the interval with room to spare
  unsigned int cap = 20u * microseconds + 1000u;
  void* args[] = {(void*)&ticks, (void*)&cap, (void*)&device_out};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::clock_probe), dim3(1), dim3(64), args, 0,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return runtime_fail("clock probe launch", e);
  return FA_OK;
}

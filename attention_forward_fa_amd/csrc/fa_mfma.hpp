// FlashAttention forward for bf16 / fp16 on gfx950 matrix cores.
//
// The computation is the aclnnFlashAttentionVarLenScoreV5 page's attention
// equation with its sink equations (功能说明 -> 计算公式), evaluated with the
// FlashAttention online softmax: keys are streamed in blocks of BN, and each
// query row keeps a running max m, a running denominator l and an unnormalised
// output accumulator that is rescaled by e^(m_old - m_new) when m grows.
//
// Workgroup = 4 wavefronts x 32 query rows (BM = 128), keys in steps of
// BN = 64, double-buffered through LDS.  Per wavefront and key block:
//
//   S^T[key, q]  = K[key, :] . Q[q, :]       MFMA 32x32x16, A = K from LDS,
//                                             B = Q^T held in registers
//   P^T          = exp2(S^T * c - m)          c = scale * log2(e)
//   O^T[d, q]   += V^T[d, key] . P^T[key, q]  MFMA 32x32x16, A = V^T from LDS,
//                                             B = P^T straight from registers
//
// Computing the transposed products puts one query row in each lane (lanes
// l and l+32 hold the two halves of the keys of query l%32), so the row max
// and row sum need one cross-half exchange, and the rescale factor is a
// per-lane scalar.  The accumulator layout of S^T is reused as the B operand
// of the second product without any data movement: the 16 keys of one MFMA
// k-step are {0-3, 8-11} in the low half-wave and {4-7, 12-15} in the high
// one.
//
// K and V blocks go from global memory straight into LDS (buffer loads with
// an LDS destination: no staging registers, no LDS stores), row-major as in
// memory, with the 16-byte units of each row XOR-swizzled by the row index so
// the operand reads hit distinct banks.  The V^T operand is read with the
// transposing LDS load (ds_read_tr16_b64), which hands each lane 4 keys of
// one column, so V is never transposed explicitly.
//
// A dense grid too small to fill the chip may give each query tile up to 4
// workgroups over disjoint key ranges (kv_splits); each then writes its rows'
// output over its range, normalised, in fp32 with the range's max and sum,
// and a second kernel (fa_split_merge_kernel) combines the ranges.
#pragma once

#include "fa_device.hpp"

namespace fa {

template <typename T>
__device__ __forceinline__ f32x16 mfma32(typename Vec8<T>::type a, typename Vec8<T>::type b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<__bf16>(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<_Float16>(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <typename T, int D, int DR, int DVAL>
struct MfmaCfg {
  static constexpr int BM = kMfmaBM;       // query rows per workgroup
  static constexpr int BN = kMfmaBN;       // keys per step
  static constexpr int DK = D + DR;        // score reduction length
  static constexpr int DV = DVAL;          // value / output columns
  static constexpr int KU = D / 8;         // 16-byte units per K row
  static constexpr int KRU = DR / 8;       // units per Krope row
  static constexpr int VU = DV / 8;        // units per V row
  static constexpr int K_BYTES = BN * KU * 16;
  static constexpr int KR_BYTES = BN * KRU * 16;
  static constexpr int V_BYTES = BN * VU * 16;
  static constexpr int KR_OFF = K_BYTES;             // byte offsets within a stage
  static constexpr int V_OFF = K_BYTES + KR_BYTES;
  static constexpr int STAGE_BYTES = K_BYTES + KR_BYTES + V_BYTES;
  static constexpr int K_LOADS = BN * KU / kMfmaThreads;    // 16-byte loads per thread per block
  static constexpr int KR_LOADS = BN * KRU / kMfmaThreads;
  static constexpr int V_LOADS = BN * VU / kMfmaThreads;
  static constexpr int NKS = DK / 16;                        // MFMA k-steps of the score product
  static constexpr int NDT = DV / 32;                        // 32-wide output tiles
  // Workgroups per CU: two while both stages fit in 80 KiB of LDS (the pse
  // tile, 16 KiB, comes only without rope, where a stage is at most 32 KiB);
  // wider heads (D = 256) run one, which also lets a wave hold up to 512
  // registers (the output accumulator then lives in the AGPRs).
  static constexpr int OCC = 2 * STAGE_BYTES <= 80 * 1024 ? 2 : 1;
};

// Physical 16-byte unit of logical unit u in LDS row r (the LDS serves 256
// bytes, 16 units, per cycle).  K rows: a ds_read_b128 reads one unit of 16
// consecutive rows per 16 lanes; with 256-byte rows the XOR by r & 15 puts
// them on 16 different units, with 128-byte rows (two per 256 bytes) the XOR
// by (r >> 1) & 7 does.  V rows: 32 lanes of the transposing read touch 4
// consecutive rows at 4 consecutive units (two even/odd pairs); the XOR by
// (r & 3) << 2 moves each row to its own group of 4 units.  (Measured on the
// two-group kernel at B2 S4096 N24: LDS bank-conflict cycles fell from about
// half of the LDS busy cycles to under 1%.)
// Rows of 12 units (D = 96) are not swizzled: their 192-byte stride already
// staggers consecutive rows over the banks, and no XOR stays inside 12 units.
template <int U>
__device__ __forceinline__ int k_swz(int r, int u) {
  return U % 16 == 0 ? u ^ (r & 15) : (U == 8 ? u ^ ((r >> 1) & 7) : u);
}
template <int VU>
__device__ __forceinline__ int v_swz(int r, int u) {
  return VU % 16 == 0 ? u ^ ((r & 3) << 2) : (VU == 8 ? u ^ ((r & 3) << 1) : u);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Sum / max of a value with the same lane's partner in the other half-wave
// (lane l <-> l ^ 32), one v_permlane32_swap: for (x, x) it returns the low
// half's values in lanes 32..63 of the first result and the high half's in
// lanes 0..31 of the second, so combining the two pairs every lane with its
// partner.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The reference max used in the exponentials only moves when a block's max
// exceeds it by more than 2^kLazy (in log2 units), so most blocks skip the
// rescale of the output accumulator.  Unnormalised weights stay <= 2^kLazy.
// The true running max is tracked separately for softmaxMax, and the sum is
// brought to it once at the end.
constexpr float kLazy = 8.0f;

// Epilogue through LDS.  Every lane writes its row's output values (the
// transposed accumulator: columns 32 dt + 8 g4 + 4 hh .. +3 of local row
// lrow) into an LDS tile of BM rows x DV columns whose 16-byte units are
// XOR-swizzled by the row (the lanes of one store, 32 rows at one column,
// then hit distinct banks); after a barrier the workgroup stores whole rows
// with 16-byte writes, so each row leaves as one contiguous run.  Rows at or
// past nrows are not written.  Every thread of the workgroup must call it;
// the LDS must no longer be in use (no loads in flight into it).
template <int U>
__device__ __forceinline__ int o_swz(int r, int u) {  // a permutation of [0, U) per row
  return (U & (U - 1)) == 0 ? u ^ (r % U) : (u + r) % U;
}
template <typename T, int DV, int NTHREADS>
__device__ __forceinline__ void o_tile_store(char* __restrict__ lds, const f32x16 (&oacc)[DV / 32], float inv,
                                             int lrow, int hh, T* __restrict__ obase, int64_t o_ss, int nrows) {
  constexpr int U = DV / 8;  // 16-byte units per row
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      T v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = from_f32<T>(oacc[dt][4 * g4 + e] * inv);
      const int pu = o_swz<U>(lrow, 4 * dt + g4);
      *reinterpret_cast<uint2*>(lds + (lrow * U + pu) * 16 + 8 * hh) = *reinterpret_cast<const uint2*>(v4);
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nrows * U; idx += NTHREADS) {
    const int r = idx / U, u = idx - r * U;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + (r * U + o_swz<U>(r, u)) * 16);
    nt_store16(obase + r * o_ss + 8 * u, v);
  }
}

// s_waitcnt lgkmcnt(n) (n <= 8), vector memory and export counters untouched.
__device__ __forceinline__ void lgkm_wait(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xc07f); break;
    case 1: __builtin_amdgcn_s_waitcnt(0xc17f); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xc27f); break;
    case 3: __builtin_amdgcn_s_waitcnt(0xc37f); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xc47f); break;
    case 5: __builtin_amdgcn_s_waitcnt(0xc57f); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xc67f); break;
    case 7: __builtin_amdgcn_s_waitcnt(0xc77f); break;
    default: __builtin_amdgcn_s_waitcnt(0xc87f); break;
  }
}

// One stretch of N matrix instructions that each take one LDS operand:
// operand m comes from read(m) (OPS LDS instructions) and goes to use(m, .).
// Reads run kStreamAhead instructions ahead and are issued two at a time, so
// one wait covers a pair of MFMAs; the sched_group_barrier sequence keeps the
// compiler from moving the reads back next to their use (where each pair
// would wait out the whole LDS latency).
constexpr int kStreamAhead = 4;

template <int N, int OPS, typename V8, typename Read, typename Use>
__device__ __forceinline__ void mfma_stream(Read&& read, Use&& use) {
  static_assert(N % 2 == 0 && kStreamAhead % 2 == 0, "pairs");
  constexpr int A = kStreamAhead < N ? kStreamAhead : N;
  V8 a[N];
#pragma unroll
  for (int m = 0; m < A; ++m) a[m] = read(m);
#pragma unroll
  for (int j = 0; j < N; j += 2) {
    int outstanding = 0;  // reads of MFMAs j + 2 .. j + A - 1 may still fly
#pragma unroll
    for (int m = j + 2; m < j + A && m < N; ++m) outstanding += OPS;
    lgkm_wait(outstanding);
    use(j, a[j]);
    use(j + 1, a[j + 1]);
    if (j + A < N) a[j + A] = read(j + A);
    if (j + A + 1 < N) a[j + A + 1] = read(j + A + 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, A * OPS, 0);
#pragma unroll
  for (int j = 0; j < N; j += 2) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (j + A < N) __builtin_amdgcn_sched_group_barrier(0x100, 2 * OPS, 0);
  }
}

// Per-workgroup constants of the key loop.
template <typename T>
struct LoopCtx {
  const T* kbase;
  const T* vbase;
  const T* krbase;
  int64_t krow_b, vrow_b, krrow_b;  // row strides in bytes
  const uint8_t* mrow;              // this lane's mask row (edge blocks)
  const T* pse;                     // additive bias, or null
  int64_t prow;                     // element index of this lane's pse row at key 0
  int64_t ptile;                    // element index of the tile's first pse row at key 0
  const uint8_t* cls_row;           // this tile's mask block classes (null: outside a TND mask)
  int skv, row, i0, last_row;
  int lane, wave, l32, hh;
  bool row_ok;
};

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes at
// base + voff land at dst + 16 l.  The scalar buffer descriptor covers
// [base, base + nbytes); lanes whose offset falls outside write zeros.
__device__ __forceinline__ void dma16(const void* base, int64_t nbytes, lds_void* dst, uint32_t voff) {
  const int n = (int)(nbytes < 0x7fffffff ? nbytes : 0x7fffffff);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000), dst, 16, voff, 0, 0, 0);
}

// Global -> LDS staging of the key block at row jb into stage `st`.  Scalar
// buffer descriptors based at the block's first row and sized to the rows
// left in the sequence make rows past the end arrive as zeros with no branch.
// Load n of wave w fills LDS units [64 (4n + w), +64): lane l writes unit
// 64 (4n + w) + l, i.e. row unit / U at physical unit unit % U, which holds the
// logical unit the swizzle maps there.
template <typename T, int D, int DR, int DV>
__device__ __forceinline__ void stage_block(char* __restrict__ st, int jb, const LoopCtx<T>& x) {
  using C = MfmaCfg<T, D, DR, DV>;
  const int64_t rows = min(x.skv - jb, C::BN);  // >= 1 for every visited block
  const T* kb = x.kbase + (int64_t)jb * (x.krow_b / (int64_t)sizeof(T));
#pragma unroll
  for (int n = 0; n < C::K_LOADS; ++n) {
    const int unit = 64 * (4 * n + x.wave) + x.lane;
    const int r = unit / C::KU, u = k_swz<C::KU>(r, unit % C::KU);
    dma16(kb, rows * x.krow_b, (lds_void*)(st + 1024 * (4 * n + x.wave)), (uint32_t)(r * x.krow_b + u * 16));
  }
  if constexpr (DR > 0) {
    const T* krb = x.krbase + (int64_t)jb * (x.krrow_b / (int64_t)sizeof(T));
#pragma unroll
    for (int n = 0; n < C::KR_LOADS; ++n) {
      const int unit = 64 * (4 * n + x.wave) + x.lane;
      const int r = unit / C::KRU, u = k_swz<C::KRU>(r, unit % C::KRU);
      dma16(krb, rows * x.krrow_b, (lds_void*)(st + C::KR_OFF + 1024 * (4 * n + x.wave)),
            (uint32_t)(r * x.krrow_b + u * 16));
    }
  }
  const T* vb = x.vbase + (int64_t)jb * (x.vrow_b / (int64_t)sizeof(T));
#pragma unroll
  for (int n = 0; n < C::V_LOADS; ++n) {
    const int unit = 64 * (4 * n + x.wave) + x.lane;
    const int r = unit / C::VU, u = v_swz<C::VU>(r, unit % C::VU);
    dma16(vb, rows * x.vrow_b, (lds_void*)(st + C::V_OFF + 1024 * (4 * n + x.wave)), (uint32_t)(r * x.vrow_b + u * 16));
  }
}

// Whether the block at jb needs per-element tests (window edge, sequence end,
// a mixed mask block, pse), whether it reads the mask, and whether the mask
// excludes all of it (then it is skipped).
struct BlockKind {
  bool partial, tests, read_mask, skip;
};
template <typename T>
__device__ __forceinline__ BlockKind block_kind(const Params& p, int jb, const LoopCtx<T>& x) {
  const bool tail = jb + kMfmaBN > x.skv;
  const bool edge = p.band && !(jb >= x.last_row - p.pre && jb + kMfmaBN - 1 <= x.i0 + p.next);
  const int cls = mask_class(p, x.cls_row, jb);
  const bool rm = cls == CLS_MIXED;
  const bool tests = tail || edge || rm;
  return {tests || p.has_pse, tests, rm, cls == CLS_EXCLUDED};
}

// Mask bytes of this lane's row for keys jb + 32t + 8a + 4hh + 0..3, word 4t + a
// (nonzero byte = excluded).
template <typename T>
__device__ __forceinline__ void fetch_mask(uint32_t (&mw)[8], const Params& p, int jb, const LoopCtx<T>& x) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int key = jb + 32 * (w >> 2) + 8 * (w & 3) + 4 * x.hh;
    if (p.mask_vec4) {
      mw[w] = (x.row_ok && key < x.skv) ? *reinterpret_cast<const uint32_t*>(x.mrow + key) : 0u;
    } else {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t byte = 0;
        if (x.mrow != nullptr && key + b < x.skv && (!p.varlen || key + b < p.m_cols))
          byte = x.mrow[(int64_t)(key + b) * p.m_sk];
        else if (p.varlen)
          byte = 1;  // outside the 2-D mask: excluded
        v |= (byte ? 0xffu : 0u) << (8 * b);
      }
      mw[w] = v;
    }
  }
}

// pse values of this lane's row for keys jb + 32t + 8a + 4hh + 0..3, word
// 4t + a (4 elements of T); keys past the sequence end (or outside the
// tensor) read as 0, they are excluded anyway.
template <typename T>
__device__ __forceinline__ void fetch_pse(uint2 (&pw)[8], const Params& p, int jb, const LoopCtx<T>& x) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int key = jb + 32 * (w >> 2) + 8 * (w & 3) + 4 * x.hh;
    const int64_t idx = x.prow + key;
    if (p.pse_vec4) {
      pw[w] = (x.row_ok && key < x.skv && idx + 3 < p.pse_len) ? *reinterpret_cast<const uint2*>(x.pse + idx)
                                                                : make_uint2(0, 0);
    } else {
      uint16_t e[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool ok = x.row_ok && key + b < x.skv && idx + b >= 0 && idx + b < p.pse_len;
        e[b] = ok ? __builtin_bit_cast(uint16_t, x.pse[idx + b]) : (uint16_t)0;
      }
      pw[w] = make_uint2(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16));
    }
  }
}

// Element b of pse word w as f32.
template <typename T>
__device__ __forceinline__ float pse_elem(const uint2& w, int b) {
  const uint32_t half = b < 2 ? w.x : w.y;
  const uint16_t bits = (uint16_t)(b & 1 ? half >> 16 : half & 0xffffu);
  return to_f32(__builtin_bit_cast(T, bits));
}

// pse through LDS (dense pse with 16-byte aligned rows): the tile of the
// workgroup's 128 rows x 64 keys is loaded straight into LDS with coalesced
// 16-byte loads, row-major with the 16-byte units of row r XOR-swizzled by
// (r / 2) % 8, so that the per-lane reads below (32 rows, one unit each) hit
// every bank twice at most.
constexpr int kPseTileBytes = kMfmaBM * kMfmaBN * 2;

template <typename T>
__device__ __forceinline__ void pse_stage(char* __restrict__ tile, const Params& p, int jb, const LoopCtx<T>& x) {
  const int64_t base = x.ptile + jb;  // inside the tensor: row i0 < Sq, key jb < Skv
  const T* src = x.pse + base;
  const int64_t nbytes = (p.pse_len - base) * (int64_t)sizeof(T);
#pragma unroll
  for (int n = 0; n < kPseTileBytes / 16 / kMfmaThreads; ++n) {
    const int unit = 64 * (4 * n + x.wave) + x.lane;  // physical unit
    const int r = unit >> 3, c = (unit & 7) ^ ((r >> 1) & 7);
    dma16(src, nbytes, (lds_void*)(tile + 1024 * (4 * n + x.wave)),
          (uint32_t)(((int64_t)r * p.ps_sq + 8 * c) * (int64_t)sizeof(T)));
  }
}

// This lane's pse words from the LDS tile, in fetch_pse's layout.
template <typename T>
__device__ __forceinline__ void pse_read(uint2 (&pw)[8], const char* tile, const LoopCtx<T>& x) {
  const int r = 32 * x.wave + x.l32;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int c = w ^ ((r >> 1) & 7);  // logical unit w = keys 8w .. 8w + 7
    pw[w] = *reinterpret_cast<const uint2*>(tile + (r * 8 + c) * 16 + 8 * x.hh);
  }
}

// One key block: prefetch the next block (and its mask words) into `nxt`,
// then the scores from `cur`, the softmax step and the output update.  The
// two stage pointers are restrict-qualified so the compiler knows the LDS
// reads of `cur` do not depend on the loads in flight into `nxt`.  `mw` holds
// this block's mask words on entry (fetched one block ahead) and the next
// block's on exit.
//
// Excluded positions are applied before the score product: the accumulators
// start at 0 for kept and -inf for excluded elements, and the MFMA adds K Q^T
// to them (-inf + finite = -inf).  Nothing branches after the scores.
template <typename T, int D, int DR, int DV, bool PL>
__device__ __forceinline__ void key_block(const char* __restrict__ cur, char* __restrict__ nxt,
                                          char* __restrict__ ptile, int jb, bool more, const Params& p,
                                          const LoopCtx<T>& x,
                                          const typename Vec8<T>::type (&qf)[MfmaCfg<T, D, DR, DV>::NKS],
                                          f32x16 (&oacc)[MfmaCfg<T, D, DR, DV>::NDT], float& m_ref, float& m_max,
                                          float& lsum, uint32_t (&mw)[8], uint2 (&pw)[8]) {
  using C = MfmaCfg<T, D, DR, DV>;
  using V8 = typename Vec8<T>::type;
  constexpr int BN = C::BN;
  const int l32 = x.l32, hh = x.hh, row = x.row;
  const float c = p.scale_log2;

  // ---- S^T = K Q^T (+ the exclusion bias) for 64 keys x 32 rows: two 32x32
  // tiles.  Only the first k-step differs between edge and full blocks (bias
  // or zero as the initial accumulator); it runs before the prefetch so the
  // mask words are consumed before the next block's overwrite them.
  auto kfrag = [&](int ks, int t) {
    const int r = 32 * t + l32;
    const char* src = ks < D / 16 ? cur + (r * C::KU + k_swz<C::KU>(r, 2 * ks + hh)) * 16
                                  : cur + C::KR_OFF + (r * C::KRU + k_swz<C::KRU>(r, 2 * (ks - D / 16) + hh)) * 16;
    return *reinterpret_cast<const V8*>(src);
  };
  const BlockKind bk = block_kind(p, jb, x);
  if constexpr (PL) {
    if (more) {
      // every wave has its words of this block's pse tile in registers (read
      // after the last barrier): the tile can take the next block's
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      pse_stage<T>(ptile, p, jb + BN, x);
    }
  }
  f32x16 sacc[2];
  if (!bk.skip) {  // a block the mask excludes as a whole only keeps the pipeline going
    const V8 a0 = kfrag(0, 0), a1 = kfrag(0, 1);
    if (DR == 0 && p.has_pse && !bk.tests) {  // pse only: no exclusion tests
      f32x16 bias[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) bias[t][j] = pse_elem<T>(pw[4 * t + (j >> 2)], j & 3) * p.inv_scale;
      sacc[0] = mfma32<T>(a0, qf[0], bias[0]);
      sacc[1] = mfma32<T>(a1, qf[0], bias[1]);
    } else if (bk.partial) {
      // The row keeps keys [lo, hi] (window and sequence end).  Element
      // e = 32t + 8a + b of this lane is key jb + 4hh + e, so key - lo =
      // b0 + e, kept iff unsigned(b0 + e) <= span: one add and one compare
      // per element (an empty range gets a b0 no element can bring back).
      int lo = 0, hi = x.skv - 1;
      if (p.band) {
        lo = max(lo, row - p.pre);
        hi = min(hi, row + p.next);
      }
      const uint32_t span = hi >= lo ? (uint32_t)(hi - lo) : 0u;
      const uint32_t b0 = hi >= lo ? (uint32_t)(jb + 4 * hh - lo) : 0x80000000u;
      f32x16 bias[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          bool k_ok = b0 + (uint32_t)(32 * t + 8 * (j >> 2) + (j & 3)) <= span;
          if (bk.read_mask) k_ok = k_ok && ((mw[4 * t + (j >> 2)] >> (8 * (j & 3))) & 0xffu) == 0;
          float bv = 0.f;
          if constexpr (DR == 0) {  // pse and rope do not combine
            if (p.has_pse) bv = pse_elem<T>(pw[4 * t + (j >> 2)], j & 3) * p.inv_scale;
          }
          bias[t][j] = k_ok ? bv : kNegInf;
        }
      }
      sacc[0] = mfma32<T>(a0, qf[0], bias[0]);
      sacc[1] = mfma32<T>(a1, qf[0], bias[1]);
    } else {
      sacc[0] = mfma32<T>(a0, qf[0], f32x16{});
      sacc[1] = mfma32<T>(a1, qf[0], f32x16{});
    }
  }

  if (more) {
    stage_block<T, D, DR, DV>(nxt, jb + BN, x);
    if (block_kind(p, jb + BN, x).read_mask) fetch_mask(mw, p, jb + BN, x);
    if constexpr (!PL && DR == 0) {
      if (p.has_pse) fetch_pse(pw, p, jb + BN, x);
    }
  }
  if (bk.skip) return;

  // Matrix-instruction stretches run at raised wave priority: of the two
  // workgroups on a CU, a wave feeding the matrix core then issues ahead of
  // one in its softmax, which fills the gaps (4-6% on short varlen and small
  // dense grids).
  __builtin_amdgcn_s_setprio(1);
  // k-steps 1 .. NKS - 1, the two 32-key tiles alternating
  mfma_stream<2 * (C::NKS - 1), 1, V8>([&](int m) { return kfrag(1 + (m >> 1), m & 1); },
                                       [&](int m, const V8& a) {
                                         sacc[m & 1] = mfma32<T>(a, qf[1 + (m >> 1)], sacc[m & 1]);
                                       });
  __builtin_amdgcn_s_setprio(0);

  // ---- online softmax (per lane: one query row, 32 of the block's keys)
  float mx;
  {
    // two chains of 3-input maxima (v_max3): 16 instructions for 32 values
    auto max3 = [](float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); };
    float m0 = max3(sacc[0][0], sacc[0][1], sacc[0][2]);
    float m1 = max3(sacc[1][0], sacc[1][1], sacc[1][2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) {
      m0 = max3(m0, sacc[0][j], sacc[0][j + 1]);
      m1 = max3(m1, sacc[1][j], sacc[1][j + 1]);
    }
    mx = __builtin_fmaxf(max3(m0, m1, sacc[0][15]), sacc[1][15]);
  }
  mx = xhalf_max(mx);
  const float mxc = mx * c;  // c > 0, so -inf stays -inf
  m_max = __builtin_fmaxf(m_max, mxc);
  if (mxc > m_ref + kLazy) {
    const float alpha = fast_exp2(m_ref - mxc);  // 0 when m_ref = -inf
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] *= alpha;
    m_ref = mxc;
  }
  const float m_use = m_ref == kNegInf ? 0.f : m_ref;

  V8 pk[2][2];
  float ls[4];  // four independent partial sums
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e = fast_exp2(fmaf(sacc[t][j], c, -m_use));
      if (t == 0 && j < 4) ls[j] = e;
      else ls[j & 3] += e;
      pk[t][j >> 3][j & 7] = from_f32<T>(e);
    }
  lsum += (ls[0] + ls[1]) + (ls[2] + ls[3]);

  __builtin_amdgcn_s_setprio(1);
  // ---- O^T += V^T P^T.  MFMA m: output tile dt = m % NDT, key step (t, s2) =
  // m / NDT, so consecutive MFMAs accumulate into different tiles.  V^T
  // operand: lane group q = lane / 16 covers output columns 32 dt + 16 (q & 1)
  // + 0..15 and keys kb = 32 t + 16 s2 + 4 (q >> 1) (+8 for the second read);
  // lane j of the group points at row kb + j / 4, columns 4 (j % 4) .. +3 of
  // that 16-column span.
  const int vq = x.lane >> 4, vj = x.lane & 15;
  auto vread = [&](int m) {
    const int dt = m % C::NDT, t = (m / C::NDT) >> 1, s2 = (m / C::NDT) & 1;
    const int vu = 4 * dt + 2 * (vq & 1) + ((vj & 3) >> 1);  // logical unit of this lane's 4 columns
    const int r0 = 32 * t + 16 * s2 + 4 * (vq >> 1) + (vj >> 2);
    const int r1 = r0 + 8;
    const char* a0 = cur + C::V_OFF + (r0 * C::VU + v_swz<C::VU>(r0, vu)) * 16 + 8 * (vj & 1);
    const char* a1 = cur + C::V_OFF + (r1 * C::VU + v_swz<C::VU>(r1, vu)) * 16 + 8 * (vj & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
    return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  mfma_stream<4 * C::NDT, 2, V8>(vread, [&](int m, const V8& a) {
    const int ts = m / C::NDT;
    oacc[m % C::NDT] = mfma32<T>(a, pk[ts >> 1][ts & 1], oacc[m % C::NDT]);
  });
  __builtin_amdgcn_s_setprio(0);
}

// D: score dims from q / k, DR: score dims from the rope tensors, DV: value
// and output dims.  PL: pse staged through LDS (dense pse with 16-byte
// aligned rows, no rope).
template <typename T, int D, int DR, int DV, bool PL = false>
__global__ void __launch_bounds__(kMfmaThreads, (MfmaCfg<T, D, DR, DV>::OCC)) fa_fwd_mfma(const Params p) {
  using C = MfmaCfg<T, D, DR, DV>;
  using V8 = typename Vec8<T>::type;
  constexpr int BM = C::BM, BN = C::BN;
  static_assert(!PL || DR == 0, "pse and rope do not combine");
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES + (PL ? kPseTileBytes : 0)];
  char* const ptile = smem + 2 * C::STAGE_BYTES;

  const Tile tl = map_tile(p, blockIdx.x);
  if (!tl.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int i0 = tl.qt * BM;
  const int row = i0 + wave * 32 + l32;  // this lane's query row within the sequence
  const bool row_ok = row < tl.sq;
  const int g = tl.h / p.group;

  // ---- Q^T fragments (B operand): lane holds row `row`, dims 16*ks + 8*hh .. +7
  V8 qf[C::NKS];
  {
    const int64_t qrow = tl.q_row0 + (row_ok ? row : 0);
    const T* qrowp = static_cast<const T*>(p.q) + tl.b * p.q_sb + tl.h * p.q_sh + qrow * p.q_ss;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qrowp + 16 * ks + 8 * hh) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(V8, u);
    }
    if constexpr (DR > 0) {
      const T* qrp = static_cast<const T*>(p.qr) + tl.b * p.qr_sb + tl.h * p.qr_sh + qrow * p.qr_ss;
#pragma unroll
      for (int ks = 0; ks < DR / 16; ++ks) {
        uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qrp + 16 * ks + 8 * hh) : make_uint4(0, 0, 0, 0);
        qf[D / 16 + ks] = __builtin_bit_cast(V8, u);
      }
    }
  }

  // ---- key blocks this tile visits
  const int last_row = min(i0 + BM, tl.sq) - 1;
  int kv_lo, kv_hi;
  key_range(p, i0, last_row, tl.skv, &kv_lo, &kv_hi);
  if (p.kv_splits > 1) {  // this workgroup's key range (whole key blocks)
    kv_lo = max(kv_lo, tl.split * p.split_keys);
    kv_hi = min(kv_hi, (tl.split + 1) * p.split_keys - 1);
  }
  const int jb0 = (kv_lo / BN) * BN;
  const int nblocks = (kv_hi >= kv_lo && last_row >= i0) ? (kv_hi - jb0) / BN + 1 : 0;

  // ---- running state, log2 domain: t = s * c, c = scale * log2(e)
  float m_ref = kNegInf;  // reference max of the exponentials
  float m_max = kNegInf;  // true running max (for softmaxMax)
  float lsum = 0.f;       // this half-wave's part of sum_j 2^(t_j - m_ref)
  if (p.has_sink && tl.split == 0) {  // the sink term belongs to one key range
    const float sk = p.sink[tl.h];
    if (sk > kNegInf) {
      m_ref = m_max = sk * kLog2e;
      lsum = hh == 0 ? 1.f : 0.f;  // 2^(sink - m_ref) = 1, counted once per row
    }
  }
  f32x16 oacc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] = f32x16{};

  LoopCtx<T> x;
  x.kbase = static_cast<const T*>(p.k) + tl.b * p.k_sb + g * p.k_sh + tl.kv_row0 * p.k_ss;
  x.vbase = static_cast<const T*>(p.v) + tl.b * p.v_sb + g * p.v_sh + tl.kv_row0 * p.v_ss;
  x.krbase = DR ? static_cast<const T*>(p.kr) + tl.b * p.kr_sb + g * p.kr_sh + tl.kv_row0 * p.kr_ss : nullptr;
  x.krow_b = p.k_ss * (int64_t)sizeof(T);
  x.vrow_b = p.v_ss * (int64_t)sizeof(T);
  x.krrow_b = DR ? p.kr_ss * (int64_t)sizeof(T) : 0;
  x.mrow = nullptr;
  if (p.has_mask) {  // dense: [b|0, h|0, row, :]; TND: the 2-D mask in local coordinates
    if (p.varlen)
      x.mrow = row < p.m_rows ? p.mask + (int64_t)row * p.m_sq : nullptr;
    else
      x.mrow = p.mask + tl.b * p.m_sb + tl.h * p.m_sh + (int64_t)(row_ok ? row : 0) * p.m_sq;
  }
  x.cls_row = mask_class_row(p, tl, i0);
  x.pse = static_cast<const T*>(p.pse);
  x.prow = p.has_pse && row_ok ? pse_row_index(p, tl, row) : 0;
  x.ptile = PL ? pse_row_index(p, tl, i0) : 0;
  x.skv = tl.skv;
  x.row = row;
  x.i0 = i0;
  x.last_row = last_row;
  x.lane = lane;
  x.wave = wave;
  x.l32 = l32;
  x.hh = hh;
  x.row_ok = row_ok;

  uint32_t mw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint2 pw[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) pw[w] = make_uint2(0, 0);
  if (nblocks > 0) {
    stage_block<T, D, DR, DV>(smem, jb0, x);
    if (block_kind(p, jb0, x).read_mask) fetch_mask(mw, p, jb0, x);
    if constexpr (PL) {
      pse_stage<T>(ptile, p, jb0, x);
    } else if constexpr (DR == 0) {
      if (p.has_pse) fetch_pse(pw, p, jb0, x);
    }
  }
  // Wait here once for the Q fragments, the first block and its mask words.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
  if constexpr (PL) {
    if (nblocks > 0) pse_read<T>(pw, ptile, x);
  }

  for (int it = 0; it < nblocks; ++it) {
    const int stg = it & 1;
    const bool more = it + 1 < nblocks;
    key_block<T, D, DR, DV, PL>(smem + stg * C::STAGE_BYTES, smem + (stg ^ 1) * C::STAGE_BYTES, ptile, jb0 + it * BN,
                            more, p, x, qf, oacc, m_ref, m_max, lsum, mw, pw);
    // this thread's loads of the next block landed; then everyone's, before the swap
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    if constexpr (PL) {
      if (more) pse_read<T>(pw, ptile, x);
    }
  }

  // ---- epilogue: O = O / l (through LDS, free since the loop's last
  // barrier), statistics at the true max
  const float lref = xhalf_sum(lsum);
  const float inv = lref > 0.f ? 1.f / lref : 0.f;
  if (p.kv_splits > 1) {
    // partial result over this key range, in fp32: O_c = O / l_c and the
    // range's statistics (max, sum at that max), merged by a later pass
    if (!row_ok) return;
    const int64_t prow = ((int64_t)(tl.split * p.nbatch + tl.b) * p.nq + tl.h) * p.sq + row;
    float* po = p.part_o + prow * DV;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(po + 32 * dt + 8 * g4 + 4 * hh) =
            make_float4(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv, oacc[dt][4 * g4 + 2] * inv,
                        oacc[dt][4 * g4 + 3] * inv);
    if (hh == 0) {
      const float mnat = m_max == kNegInf ? kNegInf : m_max * kLn2;
      const float ltrue = lref > 0.f ? lref * fast_exp2(m_ref - m_max) : 0.f;
      *reinterpret_cast<float2*>(p.part_ml + 2 * prow) = make_float2(mnat, ltrue);
    }
    return;
  }
  {
    T* obase = static_cast<T*>(p.o) + tl.b * p.o_sb + tl.h * p.o_sh + (tl.q_row0 + i0) * p.o_ss;
    o_tile_store<T, DV, kMfmaThreads>(smem, oacc, inv, wave * 32 + l32, hh, obase, p.o_ss, max(min(BM, tl.sq - i0), 0));
  }
  if (!row_ok) return;
  const int64_t orow = tl.q_row0 + row;
  if (p.smax || p.ssum) {
    const int64_t so = tl.b * p.st_sb + tl.h * p.st_sh + orow * p.st_ss + 4 * hh;
    const float mnat = m_max == kNegInf ? kNegInf : m_max * kLn2;
    const float ltrue = lref > 0.f ? lref * fast_exp2(m_ref - m_max) : 0.f;
    if (p.smax) nt_store4f(p.smax + so, mnat);
    if (p.ssum) nt_store4f(p.ssum + so, ltrue);
  }
}

}  // namespace fa

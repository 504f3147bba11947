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
// one.  V is stored transposed in LDS with bits 2 and 3 of the key index
// swapped, so that the same key order is one contiguous 16-byte read.
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

// Position of key k inside a 64-key block of the transposed V tile.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <typename T, int D, int DR>
struct MfmaCfg {
  static constexpr int BM = kMfmaBM;      // query rows per workgroup
  static constexpr int BN = kMfmaBN;      // keys per step
  static constexpr int DK = D + DR;       // score reduction length
  static constexpr int DV = D;
  static constexpr int KS = DK + 8;       // K row stride in LDS (elements); +16 B breaks bank aliasing
  static constexpr int VS = BN + 8;       // V^T row stride in LDS (elements)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = DV * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int KCH = BN * D / 8 / kMfmaThreads;     // 16-byte K chunks per thread
  static constexpr int KRCH = BN * DR / 8 / kMfmaThreads;    // 16-byte Krope chunks per thread
  static constexpr int VBLOCKS = (BN / 4) * (DV / 8);        // 4-key x 8-dim blocks per step
  static constexpr int NKS = DK / 16;                        // MFMA k-steps of the score product
  static constexpr int NDT = DV / 32;                        // 32-wide output tiles
};

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

template <typename T, int D, int DR>
__global__ void __launch_bounds__(kMfmaThreads, 2) fa_fwd_mfma(const Params p) {
  using C = MfmaCfg<T, D, DR>;
  using V8 = typename Vec8<T>::type;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];

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
  const int jb0 = (kv_lo / BN) * BN;
  const int nblocks = (kv_hi >= kv_lo && last_row >= i0) ? (kv_hi - jb0) / BN + 1 : 0;

  // ---- running state, log2 domain: t = s * c, c = scale * log2(e)
  const float c = p.scale_log2;
  float m_ref = kNegInf;  // reference max of the exponentials
  float m_max = kNegInf;  // true running max (for softmaxMax)
  float lsum = 0.f;       // this half-wave's part of sum_j 2^(t_j - m_ref)
  if (p.has_sink) {
    const float sk = p.sink[tl.h];
    if (sk > kNegInf) {
      m_ref = m_max = sk * kLog2e;
      lsum = hh == 0 ? 1.f : 0.f;  // 2^(sink - m_ref) = 1, counted once per row
    }
  }
  f32x16 oacc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] = f32x16{};

  // ---- global -> register staging of one key block.  Buffer loads: each
  // block gets a scalar descriptor based at its first row whose size covers
  // only the rows left in the sequence, so rows past the end read as zero with
  // no branch; the per-lane byte offsets are fixed for the whole loop.
  const T* kbase = static_cast<const T*>(p.k) + tl.b * p.k_sb + g * p.k_sh + tl.kv_row0 * p.k_ss;
  const T* vbase = static_cast<const T*>(p.v) + tl.b * p.v_sb + g * p.v_sh + tl.kv_row0 * p.v_ss;
  const T* krbase =
      DR ? static_cast<const T*>(p.kr) + tl.b * p.kr_sb + g * p.kr_sh + tl.kv_row0 * p.kr_ss : nullptr;
  const int64_t krow_b = p.k_ss * (int64_t)sizeof(T), vrow_b = p.v_ss * (int64_t)sizeof(T);
  const int64_t krrow_b = DR ? p.kr_ss * (int64_t)sizeof(T) : 0;
  uint32_t kvoff[C::KCH], kloff[C::KCH];    // K: global byte offset in the block, LDS element offset
  uint32_t krvoff[C::KRCH + 1], krloff[C::KRCH + 1];
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int ch = tid + i * kMfmaThreads;
    const int key = ch / (D / 8), col = ch % (D / 8);
    kvoff[i] = (uint32_t)(key * krow_b + col * 16);
    kloff[i] = key * C::KS + col * 8;
  }
#pragma unroll
  for (int i = 0; i < C::KRCH; ++i) {
    const int ch = tid + i * kMfmaThreads;
    const int key = ch / (DR / 8), col = ch % (DR / 8);
    krvoff[i] = (uint32_t)(key * krrow_b + col * 16);
    krloff[i] = key * C::KS + D + col * 8;
  }
  const int vkg = tid & 15, vdg = tid >> 4;  // V: keys 4*vkg..+3, dims 8*vdg..+7
  const bool v_active = tid < C::VBLOCKS;
  uint32_t vvoff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) vvoff[r] = (uint32_t)((4 * vkg + r) * vrow_b + 16 * vdg);
  const int voff = C::K_ELEMS + (8 * vdg) * C::VS + vt_pos(4 * vkg);

  auto rsrc = [](const void* base, int64_t bytes) {
    const int n = (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
  };
  uint4 kreg[C::KCH];
  uint4 krreg[C::KRCH + 1];
  uint4 vreg[4];
  auto load_block = [&](int jb) {
    const int64_t rows = min(tl.skv - jb, BN);  // >= 1 for every visited block
    const auto rk = rsrc(kbase + (int64_t)jb * p.k_ss, rows * krow_b);
#pragma unroll
    for (int i = 0; i < C::KCH; ++i)
      kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, kvoff[i], 0, 0));
    if constexpr (DR > 0) {
      const auto rkr = rsrc(krbase + (int64_t)jb * p.kr_ss, rows * krrow_b);
#pragma unroll
      for (int i = 0; i < C::KRCH; ++i)
        krreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rkr, krvoff[i], 0, 0));
    }
    if (v_active) {
      const auto rv = rsrc(vbase + (int64_t)jb * p.v_ss, rows * vrow_b);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vvoff[r], 0, 0));
    }
  };
  auto store_block = [&](int stage) {
    T* st = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) *reinterpret_cast<uint4*>(st + kloff[i]) = kreg[i];
#pragma unroll
    for (int i = 0; i < C::KRCH; ++i) *reinterpret_cast<uint4*>(st + krloff[i]) = krreg[i];
    if (v_active) {
      // 4 keys x 8 dims -> 8 dims x 4 keys (pairs of 16-bit lanes regrouped)
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
          hi = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
        } else {
          lo = (w0[w] & 0xffffu) | (w1[w] << 16);
          hi = (w2[w] & 0xffffu) | (w3[w] << 16);
        }
        *reinterpret_cast<uint2*>(st + voff + e * C::VS) = make_uint2(lo, hi);
      }
    }
  };

  // mask row of this lane (dense: [b|0, h|0, row, :]; TND: the 2-D mask in local coordinates)
  const uint8_t* mrow = nullptr;
  if (p.has_mask) {
    if (p.varlen)
      mrow = row < p.m_rows ? p.mask + (int64_t)row * p.m_sq : nullptr;
    else
      mrow = p.mask + tl.b * p.m_sb + tl.h * p.m_sh + (int64_t)(row_ok ? row : 0) * p.m_sq;
  }

  if (nblocks > 0) {
    load_block(jb0);
    store_block(0);
  }
  // Wait here once for the Q fragments (and the first block): otherwise the
  // compiler cannot prove they landed and re-waits for every outstanding load,
  // including the next block's prefetch, at the top of each iteration.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();

  for (int it = 0; it < nblocks; ++it) {
    const int jb = jb0 + it * BN;
    const int stg = it & 1;
    const bool more = it + 1 < nblocks;

    // ---- blocks crossing the window edge or the sequence end, or needing the
    // mask, test each element.  Mask bytes are fetched first so that waiting
    // for them does not also wait for the next block's prefetch.
    const bool tail = jb + BN > tl.skv;
    const bool edge = p.band && !(jb >= last_row - p.pre && jb + BN - 1 <= i0 + p.next);
    const bool read_mask = p.has_mask && (p.mask_everywhere || edge || tail);
    uint32_t mw[8];  // mask bytes of keys jb + 32t + 8a + 4hh + 0..3, word 4t + a
    if (read_mask) {
      if (p.mask_vec4) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int key = jb + 32 * (w >> 2) + 8 * (w & 3) + 4 * hh;
          mw[w] = (row_ok && key < tl.skv) ? *reinterpret_cast<const uint32_t*>(mrow + key) : 0u;
        }
      } else {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          uint32_t v = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int key = jb + 32 * (w >> 2) + 8 * (w & 3) + 4 * hh + b;
            uint32_t byte = 0;
            if (mrow != nullptr && key < tl.skv && (!p.varlen || key < p.m_cols)) byte = mrow[(int64_t)key * p.m_sk];
            else if (p.varlen) byte = 1;  // outside the 2-D mask: excluded
            v |= (byte ? 0xffu : 0u) << (8 * b);
          }
          mw[w] = v;
        }
      }
    }

    if (more) load_block(jb + BN);

    const T* ks_ = smem + stg * C::STAGE;
    const T* vs_ = ks_ + C::K_ELEMS;

    // ---- S^T = K Q^T for 64 keys x 32 rows: two 32x32 tiles
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const V8 a = *reinterpret_cast<const V8*>(ks_ + (32 * t + l32) * C::KS + 16 * ks + 8 * hh);
        sacc[t] = mfma32<T>(a, qf[ks], sacc[t]);
      }
    }

    // excluded scores become -inf (weight exactly 0 below)
    if (tail || edge || read_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = jb + 32 * t + 8 * (j >> 2) + 4 * hh + (j & 3);
          bool k_ok = key < tl.skv;
          if (p.band) k_ok = k_ok && (key - row <= p.next) && (row - key <= p.pre);
          if (read_mask) k_ok = k_ok && ((mw[4 * t + (j >> 2)] >> (8 * (j & 3))) & 0xffu) == 0;
          sacc[t][j] = k_ok ? sacc[t][j] : kNegInf;
        }
      }
    }

    // ---- online softmax (per lane: one query row, 32 of the block's keys)
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, sacc[t][j]);
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
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = fast_exp2(fmaf(sacc[t][j], c, -m_use));
        lsum += e;
        pk[t][j >> 3][j & 7] = from_f32<T>(e);
      }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const V8 a = *reinterpret_cast<const V8*>(vs_ + (32 * dt + l32) * C::VS + 32 * t + 16 * s2 + 8 * hh);
          oacc[dt] = mfma32<T>(a, pk[t][s2], oacc[dt]);
        }
      }
    }

    if (more) store_block(stg ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, statistics at the true max
  const float lref = xhalf_sum(lsum);
  if (!row_ok) return;
  const float inv = lref > 0.f ? 1.f / lref : 0.f;
  const int64_t orow = tl.q_row0 + row;
  T* op = static_cast<T*>(p.o) + tl.b * p.o_sb + tl.h * p.o_sh + orow * p.o_ss;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * dt + 8 * g4 + 4 * hh;
      T v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = from_f32<T>(oacc[dt][4 * g4 + e] * inv);
      *reinterpret_cast<uint2*>(op + d) = *reinterpret_cast<const uint2*>(v4);
    }
  }
  if (p.smax || p.ssum) {
    const int64_t so = tl.b * p.st_sb + tl.h * p.st_sh + orow * p.st_ss + 4 * hh;
    const float mnat = m_max == kNegInf ? kNegInf : m_max * kLn2;
    const float ltrue = lref > 0.f ? lref * fast_exp2(m_ref - m_max) : 0.f;
    if (p.smax) *reinterpret_cast<float4*>(p.smax + so) = make_float4(mnat, mnat, mnat, mnat);
    if (p.ssum) *reinterpret_cast<float4*>(p.ssum + so) = make_float4(ltrue, ltrue, ltrue, ltrue);
  }
}

}  // namespace fa

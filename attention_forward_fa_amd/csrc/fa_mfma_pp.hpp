// FlashAttention forward for bf16 / fp16 on gfx950: two wave groups in
// anti-phase ("ping-pong").
//
// Same arithmetic as the four-wave kernel (fa_mfma.hpp: transposed products,
// one query row per lane, lazy rescale, V^T in LDS with bits 2 and 3 of the key
// swapped), re-timed so the matrix cores and the vector ALUs of a SIMD work at
// the same time.  A workgroup has 8 wavefronts in two groups of 4; each group
// owns 128 query rows (BM = 256).  Per key block k a group runs
//
//   M phase: S_{k+1} = K_{k+1} Q^T   and   O += V_k P_k      (32 MFMA)
//   V phase: P_{k+1} = softmax step of S_{k+1}               (VALU + exp)
//
// and the groups are offset by one phase, with a workgroup barrier between
// phases: while group 0 issues matrix instructions, group 1 (one wave on every
// SIMD) does its softmax, then they swap.  Each SIMD therefore always has one
// wave feeding the matrix core and one feeding the VALU.
//
// Loads: group 0 stages K (and Krope) blocks, group 1 stages V blocks.  The
// loads for K_{k+2} and V_{k+1} are issued in phase 2k and written to LDS in
// phase 2k+1, into the buffers whose previous contents were last read in
// phase 2k-1.  Mask bytes (edge blocks only) are read in the softmax step.
#pragma once

#include "fa_mfma.hpp"

namespace fa {

// Position of key k inside a 64-key block of the transposed V tile (bits 2
// and 3 swapped, so the keys of one MFMA k-step are one 16-byte read).
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

constexpr int kPpThreads = 512;
constexpr int kPpBM = 256;

template <typename T, int D, int DR>
struct PpCfg {
  static constexpr int BN = kMfmaBN;
  static constexpr int DK = D + DR;
  static constexpr int DV = D;
  static constexpr int KS = DK + 8;
  static constexpr int VS = BN + 8;
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = DV * VS;
  static constexpr int KCH = BN * D / 8 / 256;    // K chunks per group-0 thread
  static constexpr int KRCH = BN * DR / 8 / 256;  // Krope chunks per group-0 thread
  static constexpr int VBLOCKS = (BN / 4) * (DV / 8);
  static constexpr int NKS = DK / 16;
  static constexpr int NDT = DV / 32;
};

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_s_barrier();
}

template <typename T, int D, int DR>
__global__ void __launch_bounds__(kPpThreads, 1) fa_fwd_mfma_pp(const Params p) {
  using C = PpCfg<T, D, DR>;
  using V8 = typename Vec8<T>::type;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) T smem[2 * C::K_ELEMS + 2 * C::V_ELEMS];
  T* const kbuf0 = smem;
  T* const vbuf0 = smem + 2 * C::K_ELEMS;

  const Tile tl = map_tile(p, blockIdx.x);
  if (!tl.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2;          // wave-uniform
  const int t256 = tid & 255;         // thread index within the group
  const int l32 = lane & 31, hh = lane >> 5;
  const int i0 = tl.qt * kPpBM;
  const int g_first = i0 + 128 * grp;
  const int row = g_first + (wave & 3) * 32 + l32;
  const bool row_ok = row < tl.sq;
  const int g = tl.h / p.group;

  // ---- Q^T fragments
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

  // ---- key blocks: the workgroup walks the union of both groups' ranges;
  // a group skips the blocks outside its own range (still meeting every barrier)
  const int wg_last = min(i0 + kPpBM, tl.sq) - 1;
  int kv_lo, kv_hi;
  key_range(p, i0, wg_last, tl.skv, &kv_lo, &kv_hi);
  const int jb0 = (kv_lo / BN) * BN;
  const int nblocks = (kv_hi >= kv_lo && wg_last >= i0) ? (kv_hi - jb0) / BN + 1 : 0;
  const int g_last = min(g_first + 127, tl.sq - 1);
  int glo, ghi;
  key_range(p, g_first, g_last, tl.skv, &glo, &ghi);
  const bool g_rows = g_last >= g_first && ghi >= glo;
  auto active = [&](int k) {
    const int jb = jb0 + k * BN;
    return g_rows && k < nblocks && jb <= ghi && jb + BN - 1 >= glo;
  };

  // ---- running state
  const float c = p.scale_log2;
  float m_ref = kNegInf, m_max = kNegInf, lsum = 0.f;
  if (p.has_sink) {
    const float sk = p.sink[tl.h];
    if (sk > kNegInf) {
      m_ref = m_max = sk * kLog2e;
      lsum = hh == 0 ? 1.f : 0.f;
    }
  }
  f32x16 oacc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] = f32x16{};
  f32x16 sacc[2];
  V8 pk[2][2];

  // ---- staging: group 0 loads K (+Krope), group 1 loads V
  const T* kbase = static_cast<const T*>(p.k) + tl.b * p.k_sb + g * p.k_sh + tl.kv_row0 * p.k_ss;
  const T* vbase = static_cast<const T*>(p.v) + tl.b * p.v_sb + g * p.v_sh + tl.kv_row0 * p.v_ss;
  const T* krbase =
      DR ? static_cast<const T*>(p.kr) + tl.b * p.kr_sb + g * p.kr_sh + tl.kv_row0 * p.kr_ss : nullptr;
  const int64_t krow_b = p.k_ss * (int64_t)sizeof(T), vrow_b = p.v_ss * (int64_t)sizeof(T);
  const int64_t krrow_b = DR ? p.kr_ss * (int64_t)sizeof(T) : 0;
  // chunk i of this thread: key (t256 + 256 i) / (D/8), 16-byte column (t256 + 256 i) % (D/8);
  // offsets are recomputed per use (one multiply-add) rather than held in registers
  auto k_key = [&](int i, int cols) { return (t256 + 256 * i) / cols; };
  auto k_col = [&](int i, int cols) { return (t256 + 256 * i) % cols; };
  const int vkg = t256 & 15, vdg = t256 >> 4;
  const bool v_active = t256 < C::VBLOCKS;
  const int voff = (8 * vdg) * C::VS + vt_pos(4 * vkg);

  auto rsrc = [](const void* base, int64_t bytes) {
    const int n = (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
  };
  uint4 sreg[C::KCH + C::KRCH > 4 ? C::KCH + C::KRCH : 4];  // this thread's staged chunks
  auto issue_k = [&](int k) {  // group 0
    const int jb = jb0 + k * BN;
    const int64_t rows = min(tl.skv - jb, BN);
    const auto rk = rsrc(kbase + (int64_t)jb * p.k_ss, rows * krow_b);
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const uint32_t off = (uint32_t)(k_key(i, D / 8) * krow_b + k_col(i, D / 8) * 16);
      sreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    }
    if constexpr (DR > 0) {
      const auto rkr = rsrc(krbase + (int64_t)jb * p.kr_ss, rows * krrow_b);
#pragma unroll
      for (int i = 0; i < C::KRCH; ++i) {
        const uint32_t off = (uint32_t)(k_key(i, DR / 8) * krrow_b + k_col(i, DR / 8) * 16);
        sreg[C::KCH + i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rkr, off, 0, 0));
      }
    }
  };
  auto write_k = [&](int buf) {
    T* st = kbuf0 + buf * C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i)
      *reinterpret_cast<uint4*>(st + k_key(i, D / 8) * C::KS + k_col(i, D / 8) * 8) = sreg[i];
#pragma unroll
    for (int i = 0; i < C::KRCH; ++i)
      *reinterpret_cast<uint4*>(st + k_key(i, DR / 8) * C::KS + D + k_col(i, DR / 8) * 8) = sreg[C::KCH + i];
  };
  auto issue_v = [&](int k) {  // group 1
    if (!v_active) return;
    const int jb = jb0 + k * BN;
    const int64_t rows = min(tl.skv - jb, BN);
    const auto rv = rsrc(vbase + (int64_t)jb * p.v_ss, rows * vrow_b);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = (uint32_t)((4 * vkg + r) * vrow_b + 16 * vdg);
      sreg[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto write_v = [&](int buf) {
    if (!v_active) return;
    T* st = vbuf0 + buf * C::V_ELEMS;
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&sreg[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&sreg[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&sreg[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&sreg[3]);
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
  };

  // ---- mask (edge blocks only), fetched one phase ahead of its use
  const uint8_t* mrow = nullptr;
  if (p.has_mask) {
    if (p.varlen)
      mrow = row < p.m_rows ? p.mask + (int64_t)row * p.m_sq : nullptr;
    else
      mrow = p.mask + tl.b * p.m_sb + tl.h * p.m_sh + (int64_t)(row_ok ? row : 0) * p.m_sq;
  }
  auto flags = [&](int k, bool* tail, bool* edge, bool* rmask) {
    const int jb = jb0 + k * BN;
    *tail = jb + BN > tl.skv;
    *edge = p.band && !(jb >= g_last - p.pre && jb + BN - 1 <= g_first + p.next);
    *rmask = p.has_mask && (p.mask_everywhere || *edge || *tail);
  };
  // mask bytes of keys jb + 32t + 8a + 4hh + 0..3 for this lane's row (edge blocks only)
  auto mask_word = [&](int jb, int t, int a) -> uint32_t {
    const int key = jb + 32 * t + 8 * a + 4 * hh;
    if (p.mask_vec4) return (row_ok && key < tl.skv) ? *reinterpret_cast<const uint32_t*>(mrow + key) : 0u;
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t byte = 0;
      if (mrow != nullptr && key + b < tl.skv && (!p.varlen || key + b < p.m_cols)) byte = mrow[(int64_t)(key + b) * p.m_sk];
      else if (p.varlen) byte = 1;  // outside the 2-D mask: excluded
      v |= (byte ? 0xffu : 0u) << (8 * b);
    }
    return v;
  };

  // S^T of block k from K buffer `buf`
  auto scores = [&](int buf) {
    const T* ks_ = kbuf0 + buf * C::K_ELEMS;
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const V8 a = *reinterpret_cast<const V8*>(ks_ + (32 * t + l32) * C::KS + 16 * ks + 8 * hh);
        sacc[t] = mfma32<T>(a, qf[ks], sacc[t]);
      }
    }
  };
  // O^T += V^T P^T with V buffer `buf`
  auto pv = [&](int buf) {
    const T* vs_ = vbuf0 + buf * C::V_ELEMS;
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
  };
  // softmax step of block k (scores in sacc) -> pk
  auto softmax = [&](int k) {
    const int jb = jb0 + k * BN;
    bool tail, edge, rmask;
    flags(k, &tail, &edge, &rmask);
    if (tail || edge || rmask) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint32_t mword = rmask ? mask_word(jb, t, a) : 0u;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int j = 4 * a + b;
            const int key = jb + 32 * t + 8 * a + 4 * hh + b;
            bool k_ok = key < tl.skv;
            if (p.band) k_ok = k_ok && (key - row <= p.next) && (row - key <= p.pre);
            k_ok = k_ok && ((mword >> (8 * b)) & 0xffu) == 0;
            sacc[t][j] = k_ok ? sacc[t][j] : kNegInf;
          }
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, sacc[t][j]);
    mx = xhalf_max(mx);
    const float mxc = mx * c;
    m_max = __builtin_fmaxf(m_max, mxc);
    if (mxc > m_ref + kLazy) {
      const float alpha = fast_exp2(m_ref - mxc);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] *= alpha;
      m_ref = mxc;
    }
    const float m_use = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = fast_exp2(fmaf(sacc[t][j], c, -m_use));
        lsum += e;
        pk[t][j >> 3][j & 7] = from_f32<T>(e);
      }
  };

  // ---- prologue: K_0, V_0 (and K_1) in LDS; group 0 runs the first softmax
  if (nblocks > 0) {
    if (grp == 0) {
      issue_k(0);
      __builtin_amdgcn_s_waitcnt(0x0f70);
      write_k(0);
    } else {
      issue_v(0);
      __builtin_amdgcn_s_waitcnt(0x0f70);
      write_v(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // Q fragments and the first blocks have landed
  lds_barrier();
  if (grp == 0) {
    if (nblocks > 1) {
      issue_k(1);
    }
    if (active(0)) {
      scores(0);
      softmax(0);
    }
    if (nblocks > 1) {
      __builtin_amdgcn_s_waitcnt(0x0f70);
      write_k(1);
    }
  }
  lds_barrier();

  // ---- main loop: phase 2k then phase 2k+1
  for (int k = 0; k < nblocks; ++k) {
    // phase 2k: group 0 = M_k, group 1 = softmax of block k (block 0: its scores too)
    if (grp == 0) {
      if (k + 2 < nblocks) issue_k(k + 2);
      if (active(k + 1)) scores((k + 1) & 1);
      if (active(k)) pv(k & 1);
    } else {
      if (k + 1 < nblocks) issue_v(k + 1);
      if (k == 0 && active(0)) scores(0);
      if (active(k)) softmax(k);
    }
    lds_barrier();
    // phase 2k+1: group 0 = softmax of block k+1, group 1 = M_k
    if (grp == 0) {
      if (k + 2 < nblocks) {
        __builtin_amdgcn_s_waitcnt(0x0f70);
        write_k(k & 1);
      }
      if (active(k + 1)) softmax(k + 1);
    } else {
      if (k + 1 < nblocks) {
        __builtin_amdgcn_s_waitcnt(0x0f70);
        write_v((k + 1) & 1);
      }
      if (active(k + 1)) scores((k + 1) & 1);
      if (active(k)) pv(k & 1);
    }
    lds_barrier();
  }

  // ---- epilogue
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

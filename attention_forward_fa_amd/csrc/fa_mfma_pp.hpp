// FlashAttention forward for bf16 / fp16 on gfx950: two wave groups in
// anti-phase ("ping-pong").
//
// Same arithmetic as the four-wave kernel (transposed products, one query row
// per lane, lazy rescale, K and V staged straight into LDS, V^T read with the
// transposing LDS load), re-timed so the matrix cores and the vector ALUs of a
// SIMD work at the same time.  A workgroup has 8 wavefronts in two groups of
// 4 (wave w is in group w / 4 and runs on SIMD w % 4, so every SIMD holds one
// wave of each group); each group owns 128 query rows (BM = 256) and both
// share the key / value stream, so every K / V byte staged into LDS serves
// 256 query rows.  Per key block k a group runs
//
//   M phase: S_{k+1} = K_{k+1} Q^T   and   O += P_k V_k      (matrix cores)
//   V phase: P_{k+1} = softmax step of S_{k+1}               (vector ALUs)
//
// and the groups are offset by one phase: a step starts with group 0 in its
// M phase and group 1 in its softmax, then they swap.  Only the end of a step
// has a workgroup barrier (the K / V ring needs it); within a step each SIMD's
// two waves run their phases back to back (a barrier between the phases cost
// 2-4%: its latency, and the wait for the slower group, which the next phase
// absorbs without it).  The M phase runs at raised wave priority; its LDS
// operand reads are issued kPpAhead (six) MFMAs ahead of their use, two MFMAs'
// reads at a time, so that one wait covers a pair of MFMAs.  Steps whose
// blocks are full for both groups (no window edge or sequence end, and kept
// whole by the mask's block classes) run without the per-block tests.
//
// K and V: NSLOT slots, block b in slot b % NSLOT.  In step b each group
// loads its share of block b + NSLOT - 1 during its M phase, the loads spread
// evenly between the matrix instructions (no softmax phase carries them);
// block b - 1, whose slot they fill, was read for the last time in step
// b - 1.  Every step issues the same loads (past the last block they read
// zeros into a free slot), and the end of each step waits for all but the
// newest NSLOT - 3 blocks, so block b + 2 is in LDS before step b + 1.  The
// tile's Q goes through the last slot (and the LDS past the ring) once, in the
// prologue.
//
// Masking (window edge, sequence end, explicit mask) is applied to the
// scores in the softmax step of the blocks that need it.
#pragma once

#include "fa_mfma.hpp"

namespace fa {

constexpr int kPpThreads = kMfmaPpThreads;
constexpr int kPpBM = kMfmaPpBM;

template <typename T, int D, int DR>
struct PpCfg {
  static constexpr int BN = kMfmaBN;
  static constexpr int DK = D + DR;
  static constexpr int DV = D;
  static constexpr int KU = D / 8;    // 16-byte units per K row
  static constexpr int KRU = DR / 8;  // units per Krope row
  static constexpr int VU = DV / 8;   // units per V row
  static constexpr int K_BYTES = BN * KU * 16;
  static constexpr int KR_BYTES = BN * KRU * 16;
  static constexpr int V_BYTES = BN * VU * 16;
  static constexpr int KR_OFF = K_BYTES;  // offsets within a slot
  static constexpr int V_OFF = K_BYTES + KR_BYTES;
  static constexpr int SLOT = K_BYTES + KR_BYTES + V_BYTES;
  static constexpr int NSLOT = 4 * SLOT <= 128 * 1024 ? 4 : 3;
  static constexpr int LDS_BYTES = NSLOT * SLOT;
  static constexpr int K_LOADS = BN * KU / kPpThreads;  // 16-byte loads per thread per block
  static constexpr int KR_LOADS = BN * KRU / kPpThreads;
  static constexpr int V_LOADS = BN * VU / kPpThreads;
  static constexpr int LPB = K_LOADS + KR_LOADS + V_LOADS;
  static constexpr int NKS = DK / 16;
  static constexpr int NDT = DV / 32;
};

template <typename T>
struct PpCtx {
  const T* kbase;
  const T* vbase;
  const T* krbase;
  int64_t krow_b, vrow_b, krrow_b;
  int kn, krn, vn;  // bytes of the sequence's K, Krope, V rows from its first (reads past them return zeros)
  const uint8_t* mrow;  // this lane's mask row (blocks that read the mask)
  const uint8_t* cls_row;  // this group's mask block classes (null: outside a TND mask)
  int skv, row, g_first, g_last;
  int lane, wave, l32, hh;
  int swave;  // wave index, in a scalar register: the LDS destinations of the loads are scalar
  bool row_ok;
};

// Per-lane running state of one query row.
template <typename T, int D, int DR>
struct PpState {
  typename Vec8<T>::type qf[PpCfg<T, D, DR>::NKS];  // Q^T fragments (B operand)
  f32x16 oacc[PpCfg<T, D, DR>::NDT];              // O^T accumulator
  f32x16 sacc[2];                                  // S^T of the block in flight
  typename Vec8<T>::type pk[2][2];                 // P^T of the previous block
  float m_ref, m_max, lsum;
};

// All 512 threads, load `idx` of the LPB that stage the K (+ Krope) and V of
// the block at jb into `slot`: load n of a part, from wave w, fills LDS units
// [64 (8n + w), +64) of that part.  One buffer descriptor per tensor covers
// the sequence's rows (bytes kn / krn / vn from its first row); the block
// enters only the lane's 32-bit byte offset (planning keeps those offsets, up
// to (Skv + 4 blocks) rows, under 2^31), and rows past the sequence end (or a
// block past the last) fall outside the descriptor and read as zeros.
template <typename T, int D, int DR>
__device__ __forceinline__ void pp_stage_one(char* __restrict__ slot, int jb, const PpCtx<T>& x, int idx) {
  using C = PpCfg<T, D, DR>;
  jb = __builtin_amdgcn_readfirstlane(jb);  // uniform
  // lane byte offset = the block's first row (uniform) + this lane's row and
  // unit within the block (loop-invariant); LDS destination uniform
  if (idx < C::K_LOADS) {
    const int unit = 64 * (8 * idx + x.wave) + x.lane;
    const int r = unit / C::KU, u = k_swz<C::KU>(r, unit % C::KU);
    dma16(x.kbase, x.kn, (lds_void*)(slot + 1024 * (8 * idx + x.swave)),
          (uint32_t)jb * (uint32_t)x.krow_b + ((uint32_t)r * (uint32_t)x.krow_b + u * 16));
  } else if (DR > 0 && idx < C::K_LOADS + C::KR_LOADS) {
    const int n = idx - C::K_LOADS;
    const int unit = 64 * (8 * n + x.wave) + x.lane;
    const int r = unit / C::KRU, u = k_swz<C::KRU>(r, unit % C::KRU);
    dma16(x.krbase, x.krn, (lds_void*)(slot + C::KR_OFF + 1024 * (8 * n + x.swave)),
          (uint32_t)jb * (uint32_t)x.krrow_b + ((uint32_t)r * (uint32_t)x.krrow_b + u * 16));
  } else {
    const int n = idx - C::K_LOADS - C::KR_LOADS;
    const int unit = 64 * (8 * n + x.wave) + x.lane;
    const int r = unit / C::VU, u = v_swz<C::VU>(r, unit % C::VU);
    dma16(x.vbase, x.vn, (lds_void*)(slot + C::V_OFF + 1024 * (8 * n + x.swave)),
          (uint32_t)jb * (uint32_t)x.vrow_b + ((uint32_t)r * (uint32_t)x.vrow_b + u * 16));
  }
}

// All LPB loads of the block at jb into `slot`.
template <typename T, int D, int DR>
__device__ __forceinline__ void pp_stage(char* __restrict__ slot, int jb, const PpCtx<T>& x) {
#pragma unroll
  for (int n = 0; n < PpCfg<T, D, DR>::LPB; ++n) pp_stage_one<T, D, DR>(slot, jb, x, n);
}

// S^T = K Q^T for the block in `slot` (64 keys x this wave's 32 rows).
template <typename T, int D, int DR>
__device__ __forceinline__ void pp_scores(const char* __restrict__ slot, const PpCtx<T>& x,
                                          const typename Vec8<T>::type (&qf)[PpCfg<T, D, DR>::NKS],
                                          f32x16 (&s)[2]) {
  using C = PpCfg<T, D, DR>;
  using V8 = typename Vec8<T>::type;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int kstep = 0; kstep < C::NKS; ++kstep) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 32 * t + x.l32;
      const char* src = kstep < D / 16
                            ? slot + (r * C::KU + k_swz<C::KU>(r, 2 * kstep + x.hh)) * 16
                            : slot + C::KR_OFF + (r * C::KRU + k_swz<C::KRU>(r, 2 * (kstep - D / 16) + x.hh)) * 16;
      s[t] = mfma32<T>(*reinterpret_cast<const V8*>(src), qf[kstep], s[t]);
    }
  }
}

// LDS operand reads run this many MFMAs ahead in the M phase.
constexpr int kPpAhead = 6;

// The M phase as one stream of MFMAs: the score MFMAs of the block in kslot
// (when do_s), then the P V MFMAs of the block in vslot (when do_pv), with
// every LDS operand read issued kPpAhead MFMAs ahead of its use (the
// sched_group_barrier sequence keeps the compiler from pulling them back),
// and this wave's loads of the block at jfill into slot fill spread between
// them.
template <typename T, int D, int DR>
__device__ __forceinline__ void pp_mphase(const char* __restrict__ kslot, const char* __restrict__ vslot,
                                          char* __restrict__ fill, int jfill, bool do_s, bool do_pv,
                                          const PpCtx<T>& x,
                                          const typename Vec8<T>::type (&qf)[PpCfg<T, D, DR>::NKS],
                                          const typename Vec8<T>::type (&pk)[2][2], f32x16 (&s)[2],
                                          f32x16 (&oacc)[PpCfg<T, D, DR>::NDT]) {
  using C = PpCfg<T, D, DR>;
  using V8 = typename Vec8<T>::type;
  constexpr int NS = 2 * C::NKS;  // score MFMAs
  constexpr int NP = 4 * C::NDT;  // P V MFMAs
  const char* vs = vslot + C::V_OFF;
  const int vq = x.lane >> 4, vj = x.lane & 15;
  auto kread = [&](int i) {
    const int kstep = i >> 1, t = i & 1;
    const int r = 32 * t + x.l32;
    const char* src = kstep < D / 16
                          ? kslot + (r * C::KU + k_swz<C::KU>(r, 2 * kstep + x.hh)) * 16
                          : kslot + C::KR_OFF + (r * C::KRU + k_swz<C::KRU>(r, 2 * (kstep - D / 16) + x.hh)) * 16;
    return *reinterpret_cast<const V8*>(src);
  };
  // P V MFMA i: output tile dt = i % NDT, key step (t, s2) = i / NDT, so
  // consecutive MFMAs accumulate into different tiles
  auto vread = [&](int i) {
    const int dt = i % C::NDT, t = (i / C::NDT) >> 1, s2 = (i / C::NDT) & 1;
    const int vu = 4 * dt + 2 * (vq & 1) + ((vj & 3) >> 1);
    const int r0 = 32 * t + 16 * s2 + 4 * (vq >> 1) + (vj >> 2);
    const int r1 = r0 + 8;
    const char* a0 = vs + (r0 * C::VU + v_swz<C::VU>(r0, vu)) * 16 + 8 * (vj & 1);
    const char* a1 = vs + (r1 * C::VU + v_swz<C::VU>(r1, vu)) * 16 + 8 * (vj & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
    return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  if (do_s && do_pv) {
    // MFMAs in pairs: the operand reads of a pair are issued together,
    // kPpAhead MFMAs ahead, so one LDS wait covers both MFMAs of a pair
    constexpr int NM = NS + NP;
    static_assert(NM % 2 == 0 && kPpAhead % 2 == 0, "pairs");
    auto ops = [](int m) { return m < NS ? 1 : 2; };  // LDS instructions of MFMA m's operand
    V8 a[NM];
    auto issue_read = [&](int m) {
      if (m < NS) a[m] = kread(m);
      else if (m < NM) a[m] = vread(m - NS);
    };
    auto issue_mfma = [&](int j) {
      if (j < NS) {
        s[j & 1] = mfma32<T>(a[j], qf[j >> 1], j < 2 ? f32x16{} : s[j & 1]);
      } else {
        const int q = j - NS, ts = q / C::NDT;
        oacc[q % C::NDT] = mfma32<T>(a[j], pk[ts >> 1][ts & 1], oacc[q % C::NDT]);
      }
    };
#pragma unroll
    for (int m = 0; m < kPpAhead; ++m) issue_read(m);
#pragma unroll
    for (int j = 0; j < NM; j += 2) {
      int outstanding = 0;  // reads of MFMAs j + 2 .. j + kPpAhead - 1 may still fly
#pragma unroll
      for (int m = j + 2; m < j + kPpAhead && m < NM; ++m) outstanding += ops(m);
      lgkm_wait(outstanding);
      issue_mfma(j);
      issue_mfma(j + 1);
      issue_read(j + kPpAhead);
      issue_read(j + kPpAhead + 1);
      // the next block's loads, spread evenly between the MFMA pairs
#pragma unroll
      for (int n = 0; n < C::LPB; ++n)
        if (j / 2 == (n + 1) * (NM / 2) / (C::LPB + 1)) pp_stage_one<T, D, DR>(fill, jfill, x, n);
    }
    // the same order for the scheduler: first reads, then per pair two
    // MFMAs, the next pair's reads and any load
    if (kPpAhead == 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    if (kPpAhead == 6) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int j = 0; j < NM; j += 2) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      const int n = j + kPpAhead;
      if (n < NM) {
        if (ops(n) + ops(n + 1) == 2)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (ops(n) + ops(n + 1) == 3)
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
#pragma unroll
      for (int m = 0; m < C::LPB; ++m)
        if (j / 2 == (m + 1) * (NM / 2) / (C::LPB + 1)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
    return;
  }
  pp_stage<T, D, DR>(fill, jfill, x);
  if (do_s) {
    V8 a[NS];
#pragma unroll
    for (int i = 0; i < NS + kPpAhead; ++i) {
      if (i < NS) a[i] = kread(i);
      const int j = i - kPpAhead;
      if (j >= 0) s[j & 1] = mfma32<T>(a[j], qf[j >> 1], j < 2 ? f32x16{} : s[j & 1]);
    }
  } else if (do_pv) {
    V8 a[NP];
#pragma unroll
    for (int i = 0; i < NP + kPpAhead; ++i) {
      if (i < NP) a[i] = vread(i);
      const int q = i - kPpAhead, ts = q / C::NDT;
      if (q >= 0) oacc[q % C::NDT] = mfma32<T>(a[q], pk[ts >> 1][ts & 1], oacc[q % C::NDT]);
    }
  }
}

// Mask bytes of keys jb + 32t + 8a + 4hh + 0..3 for this lane's row (nonzero = excluded).
template <typename T>
__device__ __forceinline__ uint32_t pp_mask_word(const Params& p, const PpCtx<T>& x, int jb, int t, int a) {
  const int key = jb + 32 * t + 8 * a + 4 * x.hh;
  if (p.mask_vec4) return (x.row_ok && key < x.skv) ? *reinterpret_cast<const uint32_t*>(x.mrow + key) : 0u;
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
  return v;
}

// Softmax step of the block at jb (scores in st.sacc) -> st.pk.  Blocks that
// cross the window edge or the sequence end, or whose mask block is mixed,
// first set their excluded scores to -inf.
template <typename T, int D, int DR, bool FULL = false>
__device__ __forceinline__ void pp_softmax(const Params& p, const PpCtx<T>& x, int jb, PpState<T, D, DR>& st) {
  using C = PpCfg<T, D, DR>;
  constexpr int BN = C::BN;
  const bool tail = !FULL && jb + BN > x.skv;
  const bool edge = !FULL && p.band && !(jb >= x.g_last - p.pre && jb + BN - 1 <= x.g_first + p.next);
  const bool rmask = !FULL && mask_class(p, x.cls_row, jb) == CLS_MIXED;
  if (tail || edge || rmask) {
    // the row keeps keys [lo, hi]; element (t, a, b) is key jb + 4hh + 32t +
    // 8a + b, kept iff unsigned(b0 + 32t + 8a + b) <= span with b0 = jb + 4hh - lo
    int lo = 0, hi = x.skv - 1;
    if (p.band) {
      lo = max(lo, x.row - p.pre);
      hi = min(hi, x.row + p.next);
    }
    const uint32_t span = hi >= lo ? (uint32_t)(hi - lo) : 0u;
    const uint32_t b0 = hi >= lo ? (uint32_t)(jb + 4 * x.hh - lo) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t mword = rmask ? pp_mask_word(p, x, jb, t, a) : 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int j = 4 * a + b;
          bool k_ok = b0 + (uint32_t)(32 * t + 8 * a + b) <= span;
          k_ok = k_ok && ((mword >> (8 * b)) & 0xffu) == 0;
          st.sacc[t][j] = k_ok ? st.sacc[t][j] : kNegInf;
        }
      }
    }
  }
  const float c = p.scale_log2;
  float mx;
  {
    // two chains of 3-input maxima (v_max3): 16 instructions for 32 values
    auto max3 = [](float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); };
    float m0 = max3(st.sacc[0][0], st.sacc[0][1], st.sacc[0][2]);
    float m1 = max3(st.sacc[1][0], st.sacc[1][1], st.sacc[1][2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) {
      m0 = max3(m0, st.sacc[0][j], st.sacc[0][j + 1]);
      m1 = max3(m1, st.sacc[1][j], st.sacc[1][j + 1]);
    }
    mx = __builtin_fmaxf(max3(m0, m1, st.sacc[0][15]), st.sacc[1][15]);
  }
  mx = xhalf_max(mx);
  const float mxc = mx * c;  // c > 0, so -inf stays -inf
  st.m_max = __builtin_fmaxf(st.m_max, mxc);
  if (mxc > st.m_ref + kLazy) {
    const float alpha = fast_exp2(st.m_ref - mxc);  // 0 when m_ref = -inf
    st.lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) st.oacc[dt] *= alpha;
    st.m_ref = mxc;
  }
  const float m_use = st.m_ref == kNegInf ? 0.f : st.m_ref;
  float ls[4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e = fast_exp2(fmaf(st.sacc[t][j], c, -m_use));
      if (t == 0 && j < 4) ls[j] = e;  // (no add to a zero start)
      else ls[j & 3] += e;
      st.pk[t][j >> 3][j & 7] = from_f32<T>(e);
    }
  st.lsum += (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

// One step (phases 2k and 2k + 1).  Reads slot cur (block k) and nxt (block
// k + 1); each group's M phase fills its share of slot fill with block
// k + NSLOT - 1.  The three pointers are
// restrict-qualified, so the compiler knows the operand reads do not depend
// on the loads in flight.
template <typename T, int D, int DR, bool FAST = false>
__device__ __forceinline__ void pp_step(char* __restrict__ fill, const char* __restrict__ cur,
                                        const char* __restrict__ nxt, int k, int jb0, bool act_k, bool act_k1,
                                        int grp, const Params& p, const PpCtx<T>& x, PpState<T, D, DR>& st) {
  if (FAST) act_k = act_k1 = true;
  using C = PpCfg<T, D, DR>;
  constexpr int BN = C::BN;
  const int jfill = jb0 + (k + C::NSLOT - 1) * BN;
  // phase 2k: group 0 = M phase of step k, group 1 = softmax of block k
  if (grp == 0) {
    __builtin_amdgcn_s_setprio(1);
    pp_mphase<T, D, DR>(nxt, cur, fill, jfill, act_k1, act_k, x, st.qf, st.pk, st.sacc, st.oacc);
    __builtin_amdgcn_s_setprio(0);
  } else {
    if (act_k) pp_softmax<T, D, DR, FAST>(p, x, jb0 + k * BN, st);
  }
  // (no barrier here: nothing the other group does in this step depends on
  // it, and each SIMD's two waves balance their phases themselves)
  // phase 2k + 1: group 0 = softmax of block k + 1, group 1 = M phase of step k
  if (grp == 0) {
    if (act_k1) pp_softmax<T, D, DR, FAST>(p, x, jb0 + (k + 1) * BN, st);
  } else {
    __builtin_amdgcn_s_setprio(1);
    pp_mphase<T, D, DR>(nxt, cur, fill, jfill, act_k1, act_k, x, st.qf, st.pk, st.sacc, st.oacc);
    __builtin_amdgcn_s_setprio(0);
  }
}

template <typename T, int D, int DR>
__global__ void __launch_bounds__(kPpThreads, 1) fa_fwd_mfma_pp(const Params p) {
  using C = PpCfg<T, D, DR>;
  using V8 = typename Vec8<T>::type;
  constexpr int BN = C::BN;
  constexpr int NSLOT = C::NSLOT;
  // The tile's Q goes through LDS (coalesced row loads, then one 16-byte
  // read per fragment) into the space of the last ring slot and the LDS past
  // the ring, both unused until the main loop.
  constexpr int Q_OFF = (NSLOT - 1) * C::SLOT;
  constexpr int Q_BYTES = kPpBM * D * (int)sizeof(T);
  constexpr bool kQLds = DR == 0 && Q_OFF + Q_BYTES <= 160 * 1024;
  constexpr int LDS_ALLOC = kQLds && Q_OFF + Q_BYTES > C::LDS_BYTES ? Q_OFF + Q_BYTES : C::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[LDS_ALLOC];

  const Tile tl = map_tile(p, blockIdx.x);
  if (!tl.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2;  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const int i0 = tl.qt * kPpBM;
  const int g_first = i0 + 128 * grp;
  const int row = g_first + (wave & 3) * 32 + l32;
  const bool row_ok = row < tl.sq;
  const int g = tl.h / p.group;

  PpState<T, D, DR> st;
  // ---- Q^T fragments (B operand): lane holds row `row`, dims 16*ks + 8*hh .. +7
  const int64_t q_ss_b = p.q_ss * (int64_t)sizeof(T);
  const bool q_lds = kQLds && q_ss_b >= D * (int64_t)sizeof(T) && q_ss_b * kPpBM < 0x7fffffff;  // uniform
  if (q_lds) {
    // the tile's rows [i0, i0 + BM) into LDS, KU units per row, unit u of
    // row r at k_swz(r, u): load n of wave w fills units [64 (8n + w), +64);
    // rows past the sequence end fall outside the descriptor and read zeros
    const T* qt = static_cast<const T*>(p.q) + tl.b * p.q_sb + tl.h * p.q_sh + (tl.q_row0 + i0) * p.q_ss;
    const int64_t qn = (int64_t)max(min(kPpBM, tl.sq - i0), 0) * q_ss_b;
    const int sw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int n = 0; n < kPpBM * C::KU / kPpThreads; ++n) {
      const int unit = 64 * (8 * n + wave) + lane;
      const int r = unit / C::KU, u = k_swz<C::KU>(r, unit % C::KU);
      dma16(qt, qn, (lds_void*)(smem + Q_OFF + 1024 * (8 * n + sw)), (uint32_t)r * (uint32_t)q_ss_b + u * 16);
    }
  } else {
    const int64_t qrow = tl.q_row0 + (row_ok ? row : 0);
    const T* qrowp = static_cast<const T*>(p.q) + tl.b * p.q_sb + tl.h * p.q_sh + qrow * p.q_ss;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qrowp + 16 * ks + 8 * hh) : make_uint4(0, 0, 0, 0);
      st.qf[ks] = __builtin_bit_cast(V8, u);
    }
    if constexpr (DR > 0) {
      const T* qrp = static_cast<const T*>(p.qr) + tl.b * p.qr_sb + tl.h * p.qr_sh + qrow * p.qr_ss;
#pragma unroll
      for (int ks = 0; ks < DR / 16; ++ks) {
        uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qrp + 16 * ks + 8 * hh) : make_uint4(0, 0, 0, 0);
        st.qf[D / 16 + ks] = __builtin_bit_cast(V8, u);
      }
    }
  }
  auto q_from_lds = [&]() {  // after the barrier that follows the Q loads
    if (q_lds) {
      const int r = row - i0;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        st.qf[ks] = *reinterpret_cast<const V8*>(smem + Q_OFF + (r * C::KU + k_swz<C::KU>(r, 2 * ks + hh)) * 16);
    }
  };

  // ---- key blocks: the workgroup walks the union of both groups' ranges; a
  // group skips the blocks outside its own range (still meeting every barrier)
  const int wg_last = min(i0 + kPpBM, tl.sq) - 1;
  int kv_lo, kv_hi;
  key_range(p, i0, wg_last, tl.skv, &kv_lo, &kv_hi);
  const int jb0 = (kv_lo / BN) * BN;
  const int nblocks = (kv_hi >= kv_lo && wg_last >= i0) ? (kv_hi - jb0) / BN + 1 : 0;
  const int g_last = min(g_first + 127, tl.sq - 1);
  int glo, ghi;
  key_range(p, g_first, g_last, tl.skv, &glo, &ghi);
  const bool g_rows = g_last >= g_first && ghi >= glo;
  const uint8_t* cls_row = mask_class_row(p, tl, g_first);
  auto active = [&](int k) {  // and not excluded by the mask as a whole
    const int jb = jb0 + k * BN;
    return g_rows && k < nblocks && jb <= ghi && jb + BN - 1 >= glo && mask_class(p, cls_row, jb) != CLS_EXCLUDED;
  };

  // ---- running state, log2 domain: t = s * c, c = scale * log2(e)
  st.m_ref = kNegInf;
  st.m_max = kNegInf;
  st.lsum = 0.f;
  if (p.has_sink) {
    const float sk = p.sink[tl.h];
    if (sk > kNegInf) {
      st.m_ref = st.m_max = sk * kLog2e;
      st.lsum = hh == 0 ? 1.f : 0.f;  // 2^(sink - m_ref) = 1, counted once per row
    }
  }
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) st.oacc[dt] = f32x16{};

  PpCtx<T> x;
  x.kbase = static_cast<const T*>(p.k) + tl.b * p.k_sb + g * p.k_sh + tl.kv_row0 * p.k_ss;
  x.vbase = static_cast<const T*>(p.v) + tl.b * p.v_sb + g * p.v_sh + tl.kv_row0 * p.v_ss;
  x.krbase = DR ? static_cast<const T*>(p.kr) + tl.b * p.kr_sb + g * p.kr_sh + tl.kv_row0 * p.kr_ss : nullptr;
  x.krow_b = p.k_ss * (int64_t)sizeof(T);
  x.vrow_b = p.v_ss * (int64_t)sizeof(T);
  x.krrow_b = DR ? p.kr_ss * (int64_t)sizeof(T) : 0;
  {
    auto nbytes = [&](int64_t row_b) {
      const int64_t nb = (int64_t)tl.skv * row_b;
      return (int)(nb < 0x7fffffff ? nb : 0x7fffffff);
    };
    x.kn = nbytes(x.krow_b);
    x.vn = nbytes(x.vrow_b);
    x.krn = DR ? nbytes(x.krrow_b) : 0;
  }
  x.mrow = nullptr;
  if (p.has_mask) {  // dense: [b|0, h|0, row, :]; TND: the 2-D mask in local coordinates
    if (p.varlen)
      x.mrow = row < p.m_rows ? p.mask + (int64_t)row * p.m_sq : nullptr;
    else
      x.mrow = p.mask + tl.b * p.m_sb + tl.h * p.m_sh + (int64_t)(row_ok ? row : 0) * p.m_sq;
  }
  x.cls_row = cls_row;
  x.skv = tl.skv;
  x.row = row;
  x.g_first = g_first;
  x.g_last = g_last;
  x.lane = lane;
  x.wave = wave;
  x.swave = __builtin_amdgcn_readfirstlane(wave);
  x.l32 = l32;
  x.hh = hh;
  x.row_ok = row_ok;

  auto slot = [&](int k) { return smem + (k % NSLOT) * C::SLOT; };

  // ---- prologue: blocks 0 .. NSLOT - 2 in flight; group 0 runs block 0's
  // scores and softmax while block 1 lands, group 1 block 0's scores
  if (nblocks > 0) {
#pragma unroll
    for (int b = 0; b < NSLOT - 1; ++b) pp_stage<T, D, DR>(slot(b), jb0 + b * BN, x);
    __builtin_amdgcn_s_waitcnt(0x0f70 | ((NSLOT - 2) * C::LPB));  // Q fragments and block 0
    __builtin_amdgcn_s_barrier();
    q_from_lds();
    if (active(0)) {
      if (grp == 0) {
        __builtin_amdgcn_s_setprio(1);
        pp_scores<T, D, DR>(slot(0), x, st.qf, st.sacc);
        __builtin_amdgcn_s_setprio(0);
        pp_softmax<T, D, DR>(p, x, jb0, st);
      } else {
        // group 1's scores of block 0, on the matrix cores while group 0
        // runs its softmax (group 1's softmax of block 0 opens step 0)
        pp_scores<T, D, DR>(slot(0), x, st.qf, st.sacc);
      }
    }
    // all prologue blocks: the loop's operand reads then only ever wait on
    // loads issued inside the loop, whose targets the compiler can tell apart;
    // and every Q read from LDS is done before the loop refills that space
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
  } else {
    // no key block: the Q loads still land before the epilogue reuses the LDS
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
  }

  // ---- main loop
  // Steps whose two blocks are full for both groups (inside every row's
  // window, before the sequence end, and with a mask of the kept class for
  // both groups' rows) skip the per-block tests: blocks [f0, f1] of the
  // workgroup's range are full as far as the window goes, and the run of fast
  // steps ends at the first step whose blocks the mask does not keep whole
  // (the rest run the general step).  Everything here is uniform over the
  // workgroup, so both groups run the same steps.
  int f0 = 1, f1 = 0;
  if (DR == 0 && wg_last >= i0 + 128) {
    int lo = 0, end = tl.skv;  // full blocks cover keys [lo, end) for both groups
    if (p.band) {
      lo = max(lo, wg_last - p.pre);
      end = min(end, i0 + p.next + 1);
    }
    f0 = max(0, (lo - jb0 + BN - 1) / BN);
    f1 = min(nblocks - 1, (end - jb0) / BN - 1);
  }
  int fa = max(f0, 1), fb = f1;  // fast steps k with blocks k and k + 1 in [f0, f1], k >= 1
  if (DR == 0 && p.has_mask && fb > fa) {
    // with a mask the fast steps end before the first block of [fa, fb]
    // that the mask does not keep whole for both groups: each lane checks
    // one block per pass, and a ballot finds the first such block
    static_assert(kClsKeys == BN && kClsRows == 128, "mask classes per (group, key block)");
    const uint8_t* cls_g0 = mask_class_row(p, tl, i0);
    const uint8_t* cls_g1 = mask_class_row(p, tl, i0 + 128);
    for (int c = fa; c <= fb; c += 64) {
      const int kb = c + lane;
      const int cb = jb0 / BN + kb;  // class column of block kb
      bool bad = false;
      if (kb <= fb) {
        bad = cls_g0 == nullptr || cls_g1 == nullptr || cb >= p.cls_kblocks || cls_g0[cb] != CLS_KEPT ||
              cls_g1[cb] != CLS_KEPT;
      }
      const uint64_t m = __ballot(bad);
      if (m != 0ull) {
        fb = c + __ffsll((long long)m) - 2;  // blocks [fa, fb + 1] kept whole
        break;
      }
    }
  }
  int k = 0;
  auto step_end = [&]() {
    // block k + 2 has landed (all but the newest NSLOT - 3 blocks)
    __builtin_amdgcn_s_waitcnt(0x0f70 | ((NSLOT - 3) * C::LPB));
    __builtin_amdgcn_s_barrier();
  };
  for (; k < nblocks && !(k >= fa && k < fb); ++k) {
    pp_step<T, D, DR>(slot(k + NSLOT - 1), slot(k), slot(k + 1), k, jb0, active(k), active(k + 1), grp, p, x, st);
    step_end();
  }
  if constexpr (DR == 0) {
    for (; k < fb; ++k) {
      pp_step<T, D, DR, true>(slot(k + NSLOT - 1), slot(k), slot(k + 1), k, jb0, true, true, grp, p, x, st);
      step_end();
    }
  }
  for (; k < nblocks; ++k) {
    pp_step<T, D, DR>(slot(k + NSLOT - 1), slot(k), slot(k + 1), k, jb0, active(k), active(k + 1), grp, p, x, st);
    step_end();
  }

  float& m_ref = st.m_ref;
  float& m_max = st.m_max;
  float& lsum = st.lsum;
  f32x16 (&oacc)[C::NDT] = st.oacc;
  // ---- epilogue: O = O / l (through LDS once the loads past the last block
  // have landed), statistics at the true max
  const float lref = xhalf_sum(lsum);
  const float inv = lref > 0.f ? 1.f / lref : 0.f;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
  {
    T* obase = static_cast<T*>(p.o) + tl.b * p.o_sb + tl.h * p.o_sh + (tl.q_row0 + i0) * p.o_ss;
    o_tile_store<T, D, kPpThreads>(smem, oacc, inv, row - i0, hh, obase, p.o_ss, max(min(kPpBM, tl.sq - i0), 0));
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

// FlashAttention forward, generic path: any of f32 / f16 / bf16, head dims up
// to 256, any element strides and alignment.  One wavefront per workgroup,
// one query row per lane; keys are staged 32 at a time in LDS as fp32 and
// read by all lanes at once (LDS broadcast).  Scores and the output are
// accumulated in fp32 with FMA, which is what the fp32 tolerance needs.
//
// Same computation and same readings as the matrix-core kernel: the
// aclnnFlashAttentionVarLenScoreV5 page's attention equation with its sink
// equations, online softmax over key blocks, window / mask / tail tests per
// element.
#include "fa_device.hpp"
#include "fa_launch.h"

namespace fa {

template <typename T, int MAXD>
__global__ void __launch_bounds__(kGenericThreads) fa_fwd_generic(const Params p) {
  constexpr int BM = kGenericBM, BN = kGenericBN, LD = MAXD + 1;
  __shared__ float sq_[BM * LD];
  __shared__ float sk_[BN * LD];
  __shared__ float sv_[BN * LD];
  __shared__ float sp_[BM * (BN + 1)];

  const Tile tl = map_tile(p, blockIdx.x);
  if (!tl.valid) return;
  const int lane = threadIdx.x;
  const int i0 = tl.qt * BM;
  const int row = i0 + lane;
  const bool row_ok = row < tl.sq;
  const int g = tl.h / p.group;
  const int DK = p.d + p.dr, DV = p.dv;

  const T* qp = static_cast<const T*>(p.q) + tl.b * p.q_sb + tl.h * p.q_sh + tl.q_row0 * p.q_ss;
  const T* qrp = p.dr ? static_cast<const T*>(p.qr) + tl.b * p.qr_sb + tl.h * p.qr_sh + tl.q_row0 * p.qr_ss : nullptr;
  const T* kp = static_cast<const T*>(p.k) + tl.b * p.k_sb + g * p.k_sh + tl.kv_row0 * p.k_ss;
  const T* krp = p.dr ? static_cast<const T*>(p.kr) + tl.b * p.kr_sb + g * p.kr_sh + tl.kv_row0 * p.kr_ss : nullptr;
  const T* vp = static_cast<const T*>(p.v) + tl.b * p.v_sb + g * p.v_sh + tl.kv_row0 * p.v_ss;

  // stage the tile's query rows (and rope parts) as fp32
  for (int idx = lane; idx < BM * DK; idx += kGenericThreads) {
    const int r = idx / DK, d = idx - r * DK;
    float x = 0.f;
    if (i0 + r < tl.sq) {
      const int64_t rr = i0 + r;
      x = d < p.d ? to_f32(qp[rr * p.q_ss + d]) : to_f32(qrp[rr * p.qr_ss + (d - p.d)]);
    }
    sq_[r * LD + d] = x;
  }

  const int last_row = min(i0 + BM, tl.sq) - 1;
  int kv_lo, kv_hi;
  key_range(p, i0, last_row, tl.skv, &kv_lo, &kv_hi);
  const int jb0 = (kv_lo / BN) * BN;
  const int nblocks = (kv_hi >= kv_lo && last_row >= i0) ? (kv_hi - jb0) / BN + 1 : 0;

  const float c = p.scale_log2;
  float m2 = kNegInf, l = 0.f;
  if (p.has_sink) {
    const float sk = p.sink[tl.h];
    if (sk > kNegInf) {
      m2 = sk * kLog2e;
      l = 1.f;
    }
  }
  float o[MAXD];
#pragma unroll
  for (int d = 0; d < MAXD; ++d) o[d] = 0.f;

  const uint8_t* mrow = nullptr;
  if (p.has_mask) {
    if (p.varlen)
      mrow = row < p.m_rows ? p.mask + (int64_t)row * p.m_sq : nullptr;
    else
      mrow = p.mask + tl.b * p.m_sb + tl.h * p.m_sh + (int64_t)(row_ok ? row : 0) * p.m_sq;
  }

  const T* pse = static_cast<const T*>(p.pse);
  const int64_t prow = p.has_pse && row_ok ? pse_row_index(p, tl, row) : 0;

  for (int it = 0; it < nblocks; ++it) {
    const int jb = jb0 + it * BN;
    __syncthreads();
    for (int idx = lane; idx < BN * DK; idx += kGenericThreads) {
      const int r = idx / DK, d = idx - r * DK;
      float x = 0.f;
      if (jb + r < tl.skv) {
        const int64_t rr = jb + r;
        x = d < p.d ? to_f32(kp[rr * p.k_ss + d]) : to_f32(krp[rr * p.kr_ss + (d - p.d)]);
      }
      sk_[r * LD + d] = x;
    }
    for (int idx = lane; idx < BN * MAXD; idx += kGenericThreads) {
      const int r = idx / MAXD, d = idx - r * MAXD;
      sv_[r * LD + d] = (d < DV && jb + r < tl.skv) ? to_f32(vp[(int64_t)(jb + r) * p.v_ss + d]) : 0.f;
    }
    __syncthreads();

    // logits of this lane's row against the BN staged keys in log2 units,
    // t = s * c + pse * log2(e), kept in LDS
    float* srow = sp_ + lane * (BN + 1);
    uint32_t keep = 0;
    float mx = kNegInf;
    for (int j = 0; j < BN; ++j) {
      float acc = 0.f;
      for (int d = 0; d < DK; ++d) acc = fmaf(sq_[lane * LD + d], sk_[j * LD + d], acc);
      const int key = jb + j;
      float bias = 0.f;
      if (p.has_pse && row_ok && key < tl.skv) {
        const int64_t idx = prow + key;
        if (idx >= 0 && idx < p.pse_len) bias = to_f32(pse[idx]) * kLog2e;
      }
      const float t = fmaf(acc, c, bias);
      bool ok = key < tl.skv;
      if (p.band) ok = ok && (key - row <= p.next) && (row - key <= p.pre);
      if (p.has_mask && ok) {
        if (p.varlen)
          ok = mrow != nullptr && key < p.m_cols && mrow[(int64_t)key * p.m_sk] == 0;
        else
          ok = mrow[(int64_t)key * p.m_sk] == 0;
      }
      keep |= (ok ? 1u : 0u) << j;
      if (ok) mx = fmaxf(mx, t);
      srow[j] = t;
    }
    const float m_new = fmaxf(m2, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m2 - m_use);
    m2 = m_new;
    float ps = 0.f;
    for (int j = 0; j < BN; ++j) {
      const float e = ((keep >> j) & 1u) ? exp2f(srow[j] - m_use) : 0.f;
      srow[j] = e;
      ps += e;
    }
    l = l * alpha + ps;
#pragma unroll
    for (int d = 0; d < MAXD; ++d) o[d] *= alpha;
    for (int j = 0; j < BN; ++j) {
      const float e = srow[j];
      const float* vrow = sv_ + j * LD;
#pragma unroll
      for (int d = 0; d < MAXD; ++d) o[d] = fmaf(e, vrow[d], o[d]);
    }
  }

  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = tl.q_row0 + row;
  T* op = static_cast<T*>(p.o) + tl.b * p.o_sb + tl.h * p.o_sh + orow * p.o_ss;
#pragma unroll
  for (int d = 0; d < MAXD; ++d)
    if (d < DV) op[d] = from_f32<T>(o[d] * inv);
  const int64_t so = tl.b * p.st_sb + tl.h * p.st_sh + orow * p.st_ss;
  const float mnat = m2 == kNegInf ? kNegInf : m2 * kLn2;
  for (int e = 0; e < 8; ++e) {
    if (p.smax) p.smax[so + e] = mnat;
    if (p.ssum) p.ssum[so + e] = l;
  }
}

template <typename T>
static hipError_t launch_generic_t(const Params& p, int maxd, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  const void* fn;
  if (maxd <= 64)
    fn = reinterpret_cast<const void*>(&fa_fwd_generic<T, 64>);
  else if (maxd <= 128)
    fn = reinterpret_cast<const void*>(&fa_fwd_generic<T, 128>);
  else
    fn = reinterpret_cast<const void*>(&fa_fwd_generic<T, 256>);
  return hipLaunchKernel(fn, dim3(p.num_wg), dim3(kGenericThreads), args, 0, s);
}

hipError_t launch_generic(const Params& p, int dtype, hipStream_t s) {
  const int maxd = max(p.d + p.dr, p.dv);
  switch (dtype) {
    case FA_DTYPE_F32: return launch_generic_t<float>(p, maxd, s);
    case FA_DTYPE_F16: return launch_generic_t<_Float16>(p, maxd, s);
    case FA_DTYPE_BF16: return launch_generic_t<__bf16>(p, maxd, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa

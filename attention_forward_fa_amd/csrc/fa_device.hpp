// Device-side helpers shared by the forward kernels: element types, the
// workgroup -> (sequence, head, query tile) schedule, and the window test.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_params.h"
#include "fa_tilemap.h"

namespace fa {

// The output rows and statistics (written once, read by no later tile) are
// stored with the non-temporal hint, so that they do not push out of the L2
// the K / V lines other tiles of the head read again (B4 N32 S8192 with a
// 2048-key window: 1334 MB fetched per call instead of 1635 MB, for 872 MB of
// algorithmic reads).  The Q loads keep the default policy: loaded
// non-temporally they arrive later, and short tiles wait on them (8% on
// 16 sequences of T = 8192).
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void nt_store16(void* p, uint4 u) {
  __builtin_nontemporal_store(nt_u32x4{u.x, u.y, u.z, u.w}, reinterpret_cast<nt_u32x4*>(p));
}
// four copies of a (16 bytes, 16-byte aligned)
__device__ __forceinline__ void nt_store4f(float* p, float a) {
  __builtin_nontemporal_store(nt_f32x4{a, a, a, a}, reinterpret_cast<nt_f32x4*>(p));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { typedef bf16x8 type; };
template <> struct Vec8<_Float16> { typedef f16x8 type; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }    // RNE
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }  // RNE

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One query tile of one (sequence, query head).
struct Tile {
  int b, h, qt;       // batch or sequence index, query head, tile index within the sequence
  int64_t q_row0;     // first global row of this sequence in q / o (TND), else 0
  int64_t kv_row0;    // first global row of this sequence in k / v (TND), else 0
  int sq, skv;        // rows of this sequence
  int split;          // key range of a split grid (0 otherwise)
  bool valid;
};

// Workgroups are dealt round-robin over the 8 XCDs (each with its own L2).
// Renumber them so each XCD receives one contiguous run of the linear tile
// order, in which the query tiles of one head are adjacent: a head's K/V then
// stays within one XCD's L2.
__device__ __forceinline__ int xcd_linear_id(int bid, int grid) {
  const int x = bid & 7, i = bid >> 3;
  const int per = grid >> 3, rem = grid & 7;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), with
// DPP: shifts by 1, 2, 4 and 8 within each row of 16 lanes, then lane 15 of
// a row into the next row and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 (rows 1, 3)
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 (rows 2, 3)
  return v;
}

// Entry r of the per-head TND tile list found from cu_seqlens, with no tile
// map: the same entry tile_entry reads from the prefix of seq_tiles
// (sequence b holds entries [prefix[b], prefix[b + 1]), later entries first
// when reverse_tiles).  Every wave loads the cumulative lengths of up to
// kTileSearchMaxSeqs sequences at once, lane i taking sequences i, i + 64,
// ...; per 64-sequence chunk an inclusive scan gives each sequence's first
// entry, and the one lane whose entries hold the target reports its
// sequence, tile and row spans (read into scalar registers).  Called by all
// threads of the workgroup with full waves; every value it branches on is
// wave-uniform.  Returns false past the last tile.
__device__ __forceinline__ bool search_tile(const Params& p, int r, Tile* t) {
  constexpr int NC = kTileSearchMaxSeqs / 64;
  const int lane = threadIdx.x & 63;
  const int nb = p.nbatch;
  int n[NC], incl[NC], q0[NC], q1[NC], k0[NC], k1[NC], tot[NC];
  int total = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int b = 64 * c + lane;
    int qa = 0, qe = 0, ka = 0, ke = 0;
    if (b < nb) {
      qa = p.cu_q[b];
      qe = p.cu_q[b + 1];
      ka = p.cu_kv[b];
      ke = p.cu_kv[b + 1];
    }
    clamp_span(qa, qe, p.tq, &q0[c], &q1[c]);
    clamp_span(ka, ke, p.tkv, &k0[c], &k1[c]);
    n[c] = b < nb ? (q1[c] - q0[c] + p.tile_bm - 1) / p.tile_bm : 0;
    incl[c] = 64 * c < nb ? wave_incl_scan(n[c]) : 0;
    tot[c] = __builtin_amdgcn_readlane(incl[c], 63);
    total += tot[c];
  }
  if (r >= total) return false;
  const int rr = p.reverse_tiles ? total - 1 - r : r;
  int base = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int first = base + incl[c] - n[c];
    const unsigned long long hit = __ballot(n[c] > 0 && first <= rr && rr < first + n[c]);
    if (hit != 0ull) {
      const int l = __ffsll((long long)hit) - 1;
      const int a = __builtin_amdgcn_readlane(q0[c], l), ka = __builtin_amdgcn_readlane(k0[c], l);
      t->b = 64 * c + l;
      t->qt = rr - __builtin_amdgcn_readlane(first, l);
      t->q_row0 = a;
      t->kv_row0 = ka;
      t->sq = __builtin_amdgcn_readlane(q1[c], l) - a;
      t->skv = __builtin_amdgcn_readlane(k1[c], l) - ka;
      return true;
    }
    base += tot[c];
  }
  return false;
}

__device__ __forceinline__ Tile map_tile(const Params& p, int bid) {
  Tile t;
  const int lin = xcd_linear_id(bid, p.num_wg);
  const int tph = p.tiles_per_head;
  if (!p.varlen) {
    // (sequence, head), then key range, then query tile: the tiles that
    // share one key range of one head are adjacent
    const int per_bh = tph * p.kv_splits;
    const int bh = lin / per_bh;
    int r = lin - bh * per_bh;
    t.split = r / tph;
    r -= t.split * tph;
    t.b = bh / p.nq;
    t.h = bh - t.b * p.nq;
    t.qt = p.reverse_tiles ? tph - 1 - r : r;
    t.q_row0 = 0;
    t.kv_row0 = 0;
    t.sq = p.sq;
    t.skv = p.skv;
    t.valid = true;
    return t;
  }
  t.h = lin / tph;
  t.split = 0;
  const int r = lin - t.h * tph;
  if (p.tile_search) {
    t.b = t.qt = t.sq = t.skv = 0;
    t.q_row0 = t.kv_row0 = 0;
    t.valid = search_tile(p, r, &t);
    return t;
  }
  // one 32-byte entry of the tile map (built on the device before this kernel)
  const int4* e = reinterpret_cast<const int4*>(p.tile_map) + 2 * r;
  const int4 e0 = e[0], e1 = e[1];
  t.valid = e1.z != 0;
  t.b = e0.x;
  t.qt = e0.y;
  t.q_row0 = e0.z;
  t.kv_row0 = e0.w;
  t.sq = e1.x;
  t.skv = e1.y;
  return t;
}


// Key range [lo, hi] any row of [i_first, i_last] may keep (window and length).
__device__ __forceinline__ void key_range(const Params& p, int i_first, int i_last, int skv, int* lo, int* hi) {
  int a = 0, e = skv - 1;
  if (p.band) {
    a = max(a, i_first - p.pre);
    e = min(e, i_last + p.next);
  }
  *lo = a;
  *hi = e;
}

// This tile's row of mask block classes (kClsRows query rows starting at
// row0 of the sequence), or null when the rows lie outside the 2-D TND mask.
__device__ __forceinline__ const uint8_t* mask_class_row(const Params& p, const Tile& tl, int row0) {
  if (!p.has_mask || p.mask_cls == nullptr) return nullptr;
  const int t = row0 / kClsRows;
  if (t >= p.cls_tiles) return nullptr;
  int64_t slice = 0;
  if (!p.varlen) {
    const int mb = p.m_sb != 0 ? tl.b : 0, mh = p.m_sh != 0 ? tl.h : 0;
    slice = (int64_t)mb * p.cls_nh + mh;
  }
  return p.mask_cls + (slice * p.cls_tiles + t) * p.cls_kblocks;
}

// Class of the key block starting at jb for a class row (see mask_class_row).
// The row pointer and jb are the same in every lane of a wave; the table does
// not change while a forward kernel runs, so the byte comes in through a
// scalar load of its aligned dword (the table is padded to 16 bytes), which
// leaves the vector memory counters to the key/value staging.
__device__ __forceinline__ int mask_class(const Params& p, const uint8_t* cls_row, int jb) {
  if (!p.has_mask) return CLS_KEPT;
  const int kb = jb / kClsKeys;
  if (cls_row == nullptr || kb >= p.cls_kblocks) return CLS_EXCLUDED;  // outside the 2-D TND mask
  const uint64_t a = reinterpret_cast<uint64_t>(cls_row) + (uint64_t)kb;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t au = ((uint64_t)hi << 32) | lo;
  using const_u32 = const __attribute__((address_space(4))) uint32_t;
  const uint32_t w = *reinterpret_cast<const_u32*>(au & ~(uint64_t)3);
  return (int)((w >> (8 * (lo & 3u))) & 0xffu);
}

// Element index of the pse value for (row, key 0) of this tile's (sequence,
// head): dense [B|1, N, Sq, Skv] by strides; TND from the sequence's block
// [N, Sq_b, Skv_b] in the flat tensor.  Reads add the key and stay below
// p.pse_len.
__device__ __forceinline__ int64_t pse_row_index(const Params& p, const Tile& tl, int row) {
  if (p.varlen) return p.pse_off[tl.b] + ((int64_t)tl.h * tl.sq + row) * tl.skv;
  return tl.b * p.ps_sb + tl.h * p.ps_sh + (int64_t)row * p.ps_sq;
}

}  // namespace fa

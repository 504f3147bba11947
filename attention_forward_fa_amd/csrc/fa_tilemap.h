// The varlen (TND) tile schedule: how cumulative sequence lengths become the
// per-head list of (sequence, query tile) entries a forward grid walks.
// Plain arithmetic on host-visible integers, compiled both into the device
// pre-pass and into host checks of its clamping, so that a cu_seqlens array
// that is not non-decreasing, or leaves [0, T), can only shrink the work and
// never address rows outside [0, T).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

// Rows [*start, *end) of a sequence whose cumulative lengths are a (before
// it) and e (after it): a clamped into [0, total], e into [a, total].
FA_HD inline void clamp_span(int a, int e, int total, int* start, int* end) {
  a = a < 0 ? 0 : (a > total ? total : a);
  e = e < a ? a : (e > total ? total : e);
  *start = a;
  *end = e;
}

// Rows [*start, *end) of sequence b: cu[b] and cu[b + 1] clamped.
FA_HD inline void seq_span(const int32_t* cu, int b, int total, int* start, int* end) {
  clamp_span(cu[b], cu[b + 1], total, start, end);
}

FA_HD inline int seq_rows(const int32_t* cu, int b, int total) {
  int a, e;
  seq_span(cu, b, total, &a, &e);
  return e - a;
}

// Query tiles of bm rows sequence b needs.
FA_HD inline int seq_tiles(const int32_t* cu, int b, int total, int bm) { return (seq_rows(cu, b, total) + bm - 1) / bm; }

// Entry r of the per-head tile list, given prefix[b] = tiles of the
// sequences before b (prefix[nbatch] = ntiles): the sequence, its query
// tile, the first rows of q and k, the rows of q and k, and whether the entry
// is a tile (r < ntiles); later (heavier) tiles first when `reverse`.  As
// eight int32: {b, qt, q0, k0, sq, skv, valid, 0}.
FA_HD inline void tile_entry(const int32_t* prefix, const int32_t* cu_q, const int32_t* cu_kv, int nbatch, int tq,
                             int tkv, int reverse, int r, int32_t* e) {
  for (int i = 0; i < 8; ++i) e[i] = 0;
  const int ntiles = prefix[nbatch];
  if (r >= ntiles || nbatch < 1) return;
  const int rr = reverse ? ntiles - 1 - r : r;
  // largest b with prefix[b] <= rr (prefix is non-decreasing, prefix[0] = 0)
  int lo = 0, hi = nbatch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= rr) lo = mid; else hi = mid - 1;
  }
  int q0, q1, k0, k1;
  seq_span(cu_q, lo, tq, &q0, &q1);
  seq_span(cu_kv, lo, tkv, &k0, &k1);
  e[0] = lo;
  e[1] = rr - prefix[lo];
  e[2] = q0;
  e[3] = k0;
  e[4] = q1 - q0;
  e[5] = k1 - k0;
  e[6] = 1;
}

}  // namespace fa

// Internal: the parameter block phase 1 fills and the device kernels read.
// Plain C++ (no HIP types) so the host planner builds with any C++ compiler.
#pragma once

#include <stdint.h>

namespace fa {

// Which kernel family a plan launches.
enum KernelKind : int32_t {
  KERNEL_MFMA = 0,     // bf16/fp16, MFMA 32x32x16, 4 waves, D in {64,128}, Dr in {0,64}, Dv == D
  KERNEL_GENERIC = 1,  // any dtype, one query row per lane, fp32 VALU dot products
  KERNEL_MFMA_PP = 2,  // as KERNEL_MFMA with 8 waves in two anti-phase groups (BM = 256)
};

// Mask block classes (written by a pre-pass over the mask): a block of
// kClsRows query rows x kClsKeys keys whose positions are all kept, all
// excluded, or mixed.  Only mixed blocks read the mask; excluded ones are
// skipped.
constexpr int kClsRows = 128;
constexpr int kClsKeys = 64;
enum MaskClass : uint8_t { CLS_KEPT = 0, CLS_EXCLUDED = 1, CLS_MIXED = 2 };

// Tile of the MFMA kernel: 4 wavefronts x 32 query rows, 64 keys per step.
constexpr int kMfmaBM = 128;
constexpr int kMfmaBN = 64;
constexpr int kMfmaThreads = 256;
// Key split of the 4-wave kernel: a grid with fewer workgroups than the
// chip holds at once (2 per compute unit, 256 units) gives each query tile up
// to kMaxKvSplits workgroups over disjoint key ranges of at least
// kMinSplitBlocks key blocks, then merges their partial results.
constexpr int kNumCUs = 256;
constexpr int kMaxKvSplits = 4;
constexpr int kWgSlots = 2 * kNumCUs;
constexpr int kMinSplitBlocks = 8;
// Tile of the two-group matrix-core kernel: 8 wavefronts, 256 query rows.
constexpr int kMfmaPpBM = 256;
constexpr int kMfmaPpThreads = 512;
// Tile of the generic kernel: one wavefront, one query row per lane.
constexpr int kGenericBM = 64;
constexpr int kGenericBN = 32;
constexpr int kGenericThreads = 64;
// TND with at most this many sequences: each workgroup finds its (sequence,
// query tile) from cu_seqlens_q itself (a wave scans 64 sequences at a time)
// instead of reading a tile map built by a pre-pass launch.
constexpr int kTileSearchMaxSeqs = 256;

struct Params {
  // device addresses
  const void* q;
  const void* k;
  const void* v;
  const void* qr;        // may be null
  const void* kr;        // may be null
  void* o;
  float* smax;           // may be null
  float* ssum;           // may be null
  const uint8_t* mask;   // may be null
  const float* sink;     // may be null
  const int32_t* cu_q;   // TND only
  const int32_t* cu_kv;  // TND only
  int32_t* tile_prefix;  // TND without tile_search: workspace, [nbatch + 1]
  int32_t* tile_map;     // TND without tile_search: workspace, [tiles_per_head][8] = {b, qt, q0, k0, sq, skv, valid, 0}
  const void* pse;       // may be null: additive position bias, q's element type
  int64_t* pse_off;      // TND with pse: workspace, [nbatch + 1] element offset of each sequence's block
  uint8_t* mask_cls;     // with a mask: workspace, class of every (mask slice, 128-row tile, 64-key block)
  float* part_o;         // key split: workspace, [kv_splits][nbatch * nq * sq][dv] normalised partial outputs
  float* part_ml;        // key split: workspace, [kv_splits][nbatch * nq * sq][2] = {max, sum}, natural-log units

  // element strides: batch, row (sequence position / token), head
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t qr_sb, qr_ss, qr_sh;
  int64_t kr_sb, kr_ss, kr_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t st_sb, st_ss, st_sh;           // statistics (the 8 slots are contiguous)
  int64_t m_sb, m_sh, m_sq, m_sk;        // mask (0 for broadcast dims)
  int32_t m_rows, m_cols;                // TND: extent of the 2-D mask
  int64_t ps_sb, ps_sh, ps_sq;           // dense pse: batch (0 when broadcast), head, row strides
  int64_t pse_len;                       // elements in the pse tensor; every read is bounded by it
  int32_t cls_nh, cls_tiles, cls_kblocks;  // mask classes: heads of the mask (1 or N), row tiles, key blocks
  int32_t cls_slices;                      // mask classes: (mask batch, mask head) slices; 1 for TND

  int32_t nbatch;   // B (dense) or number of sequences (TND)
  int32_t nq, nkv, group;
  int32_t sq, skv;  // dense: per-batch lengths; TND: unused (from cu_seqlens)
  int32_t tq, tkv;  // TND: total rows of q / k
  int32_t d, dr, dv;

  float scale;       // scale_value
  float scale_log2;  // scale_value * log2(e)
  int32_t pre, next; // window bounds (next already min(next,0) under causal), clamped
  int32_t band;      // window active (mask given or causal)
  int32_t has_mask, has_sink, varlen;
  int32_t mask_vec4;        // dense mask with contiguous, 4-byte aligned rows: read 4 keys at once
  int32_t has_pse;
  int32_t pse_vec4;         // dense pse whose 4-key groups are 8-byte aligned: read 4 keys at once
  int32_t pse_lds;          // dense pse with 16-byte aligned rows: staged through LDS by the matrix-core kernel
  float inv_scale;          // 1 / scale: pse enters the raw score accumulator as pse / scale

  int32_t tiles_per_head;   // dense: ceil(sq / BM); TND: ceil(tq / BM) + nbatch (upper bound)
  int32_t tile_search;      // TND: the kernel finds its tile from cu_seqlens_q (tile_prefix / tile_map unused)
  int32_t tile_bm;          // TND: query rows per tile
  int32_t num_wg;           // grid size
  int32_t reverse_tiles;    // schedule later (heavier) query tiles first
  int32_t kv_splits;        // dense, 4-wave kernel: workgroups per query tile, each over one key range (1 = off)
  int32_t split_keys;       // keys per range (a multiple of the key block); range c = [c * split_keys, +split_keys)
};

}  // namespace fa

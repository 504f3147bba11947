"""HIP forward vs the CPU oracle, element by element (needs an MI355X).

Small cases cover several tiles, ragged tails and every feature; the
full-size workloads are compared on sampled rows the oracle computes one by
one.  Tolerances are the ones stated in ``parity_util``.
"""
import math

import pytest
import torch

import synth
from attention_forward_fa_amd import _lib, api
from oracle import attention as orc

from . import parity_util as pu

pytestmark = pytest.mark.gpu

U = synth.UNBOUNDED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()  # the HIP library must be built; fails loudly otherwise
    yield


def _report(name, errs):
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.3g}" for k, v in errs.items()), flush=True)


# ---------------------------------------------------------------------------
# small cases, full comparison
# ---------------------------------------------------------------------------

def _seq_lengths(n, longest, seed):
    """n seeded sequence lengths in [0, longest], about one in eight empty."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, longest + 1, (n,), generator=g)
    lens[torch.rand(n, generator=g) < 0.125] = 0
    return lens.tolist()


SMALL = {
    "c1_fp32_bnsd": lambda: synth.workload("c1_fp32_bnsd"),
    "c2_small_bf16": lambda: synth.workload("c2_dense_bsnd", "bf16", small=True),
    "c2_small_fp16": lambda: synth.workload("c2_dense_bsnd", "fp16", small=True),
    "c3_small_causal": lambda: synth.workload("c3_causal", small=True),
    "c3_small_band": lambda: synth.workload("c3_band", small=True),
    "c4_small_varlen": lambda: synth.workload("c4_varlen_causal", small=True),
    "c5_small_sink_rope": lambda: synth.workload("c5_varlen_sink_rope", small=True),
    "c2_small_gqa_nkv4": lambda: synth.workload("c2_gqa_nkv4", small=True),
    "c2_small_mqa_fp16": lambda: synth.workload("c2_mqa", "fp16", small=True),
    "d256_small_dense": lambda: synth.workload("d256_dense_bsnd", small=True),
    "bnsd_ragged_201": lambda: synth.dense_case("x", "BNSD", 2, 2, 201, 128, "bf16", 31),
    "bsnd_d64": lambda: synth.dense_case("x", "BSND", 1, 3, 190, 64, "bf16", 32),
    "bsnd_d64_rope": lambda: synth.dense_case("x", "BSND", 1, 2, 150, 64, "bf16", 33, drope=64, causal=True),
    "fp16_rope_sink": lambda: synth.dense_case("x", "BNSD", 1, 2, 260, 128, "fp16", 34, drope=64, sink=True),
    "gqa_4_2": lambda: synth.dense_case("x", "BNSD", 2, 4, 140, 128, "bf16", 35, nkv=2, causal=True),
    "mqa_varlen": lambda: synth.varlen_case("x", [70, 0, 129, 1], 4, 128, "bf16", 36, nkv=1, causal=True),
    "sq_ne_skv": lambda: synth.dense_case("x", "BNSD", 1, 2, 100, 128, "bf16", 37, skv=300),
    "sq_ne_skv_causal": lambda: synth.dense_case("x", "BNSD", 1, 2, 300, 128, "bf16", 38, skv=100, causal=True),
    "sink_causal": lambda: synth.dense_case("x", "BSND", 1, 3, 170, 128, "bf16", 39, sink=True, causal=True),
    "band_pre5_next3_mask": lambda: _band_mask_case(40, 5, 3),
    "band_pre0_next0_mask": lambda: _band_mask_case(41, 0, 0),
    "band_neg_pre": lambda: _band_mask_case(42, -2, 9),
    "causal_flag_band": lambda: synth.dense_case("x", "BNSD", 1, 2, 333, 128, "bf16", 43, causal=True,
                                                 pre_tokens=70),
    "random_mask_4d": lambda: _random_mask_case(44, (2, 1)),
    "random_mask_bn": lambda: _random_mask_case(45, (1, 2)),
    "fp32_varlen_sink": lambda: synth.varlen_case("x", [33, 0, 90], 2, 64, "fp32", 46, sink=True, causal=True),
    "fp32_mask_band": lambda: _band_mask_case(47, 9, 0, dtype="fp32", d=64),
    "fp32_d96": lambda: synth.dense_case("x", "BSND", 1, 2, 75, 96, "fp32", 48, dv=80),
    "bf16_d96": lambda: synth.dense_case("x", "BNSD", 1, 2, 99, 96, "bf16", 49),
    "d96_causal_sink_bsnd": lambda: synth.dense_case("x", "BSND", 2, 3, 300, 96, "bf16", 58, sink=True, causal=True,
                                                     skv=333),
    "d96_fp16_band_mask": lambda: _band_mask_case(59, 17, 5, dtype="fp16", d=96),
    "d96_rope_varlen": lambda: synth.varlen_case("x", [150, 0, 61, 200], 2, 96, "bf16", 60, drope=64, sink=True,
                                                 causal=True),
    "d96_pse_lds": lambda: synth.dense_case("x", "BNSD", 1, 2, 200, 96, "bf16", 61, skv=264, pse="full",
                                            causal=True),
    "bf16_dv_lt_d": lambda: synth.dense_case("x", "BNSD", 1, 2, 99, 128, "bf16", 50, dv=64),
    "d192_dv128_causal_sink": lambda: synth.dense_case("x", "BSND", 2, 3, 260, 192, "bf16", 62, dv=128, causal=True,
                                                       sink=True),
    "d160_dv96_gqa_fp16": lambda: synth.dense_case("x", "BNSD", 1, 4, 200, 160, "fp16", 63, dv=96, nkv=2, skv=333),
    "d192_dv128_varlen": lambda: synth.varlen_case("x", [130, 0, 257, 64], 2, 192, "bf16", 64, dv=128, causal=True),
    "tnd_mask_2d": lambda: _tnd_mask_case(51),
    "scale_zero": lambda: synth.dense_case("x", "BNSD", 1, 1, 130, 128, "bf16", 52, causal=True, scale=0.0),
    "stats_same_as_input": lambda: synth.varlen_case("x", [64, 200], 2, 128, "bf16", 53, causal=True,
                                                     softmax_out_layout="same_as_input"),
    "len_1": lambda: synth.dense_case("x", "BNSD", 1, 2, 1, 128, "bf16", 54),
    "len_63_65": lambda: synth.varlen_case("x", [63, 64, 65, 127, 128, 129], 2, 128, "bf16", 55),
    # the in-kernel tile search over several 64-sequence chunks (with and
    # without reversed tiles), and the tile map beyond 256 sequences
    "seqs_70_causal": lambda: synth.varlen_case("x", _seq_lengths(70, 300, 130), 2, 128, "bf16", 131,
                                                causal=True),
    "seqs_130_dense": lambda: synth.varlen_case("x", _seq_lengths(130, 140, 132), 2, 64, "bf16", 133),
    "seqs_300_tile_map": lambda: synth.varlen_case("x", _seq_lengths(300, 20, 134), 2, 128, "bf16", 135,
                                                   causal=True),
    "sink_neg_inf": lambda: _sink_neg_inf_case(56),
    "large_logits": lambda: synth.dense_case("x", "BNSD", 1, 2, 200, 128, "bf16", 57, scale=1.0),
    # additive position bias (pse / realShift)
    "c6_small_pse": lambda: synth.workload("c6_dense_pse", small=True),
    "pse_full_bsnd_ragged": lambda: synth.dense_case("x", "BSND", 2, 3, 201, 128, "bf16", 70, pse="full"),
    "pse_bcast_causal_fp16": lambda: synth.dense_case("x", "BNSD", 2, 2, 170, 128, "fp16", 71, pse="bcast",
                                                      causal=True),
    "pse_d64_sink_band": lambda: _pse_band_mask_case(72),
    "pse_gqa": lambda: synth.dense_case("x", "BNSD", 1, 4, 140, 128, "bf16", 73, nkv=2, pse="full"),
    "pse_fp32": lambda: synth.dense_case("x", "BNSD", 1, 2, 75, 64, "fp32", 74, pse="full", causal=True),
    "pse_tnd": lambda: synth.varlen_case("x", [100, 0, 37, 140], 2, 128, "bf16", 75, causal=True, pse=True),
    "pse_tnd_sink_fp16": lambda: synth.varlen_case("x", [64, 65, 3], 3, 64, "fp16", 76, sink=True, pse=True),
    "pse_unaligned_rows": lambda: synth.dense_case("x", "BNSD", 1, 2, 130, 128, "bf16", 77, skv=131, pse="full"),
    # pse staged through LDS (rows a multiple of 8 keys, 16-byte aligned)
    "pse_lds_causal_ragged": lambda: synth.dense_case("x", "BNSD", 2, 2, 200, 128, "bf16", 90, skv=264, pse="full",
                                                      causal=True),
    "pse_lds_d64_bcast_fp16": lambda: synth.dense_case("x", "BSND", 1, 3, 300, 64, "fp16", 91, skv=256,
                                                       pse="bcast"),
    "pse_lds_band_mask_sink": lambda: _pse_lds_mask_case(92),
    "pse_lds_blocks": lambda: _block_mask_case(93, 128, 64, (1, 1), pse=True, skv=640),
    # general masks: blocks the mask keeps or excludes as a whole, and masks at odds with the window
    "mask_blocks_aligned": lambda: _block_mask_case(80, 128, 64, (2, 1)),
    "mask_blocks_unaligned": lambda: _block_mask_case(81, 96, 80, (1, 2)),
    "mask_blocks_fp16_sink": lambda: _block_mask_case(82, 128, 64, (1, 1), dtype="fp16", sink=True),
    "mask_blocks_pse": lambda: _block_mask_case(83, 128, 64, (2, 2), pse=True),
    "mask_blocks_rope_d64": lambda: _block_mask_case(84, 256, 128, (1, 1), d=64, drope=64),
    "mask_documents": lambda: _document_mask_case(85),
    "mask_inside_band": lambda: _mask_inside_band_case(86),
    "mask_outside_band": lambda: _mask_outside_band_case(87),
    "mask_causal_holes": lambda: _mask_causal_holes_case(89),
    "tnd_mask_blocks": lambda: _tnd_block_mask_case(88),
    # a 2-D TND mask smaller than the longer sequences: positions beyond it are excluded
    "tnd_mask_shorter_than_sequence": lambda: _tnd_small_mask_case(89),
    "tnd_mask_shorter_causal_sink": lambda: _tnd_small_mask_case(94, causal=True, sink=True),
    # head dim 256 (and Dv 256 or below it)
    "d256_causal_bf16": lambda: synth.dense_case("x", "BNSD", 1, 2, 200, 256, "bf16", 120, causal=True, skv=333),
    "d256_varlen_sink_fp16": lambda: synth.varlen_case("x", [130, 0, 257, 64], 2, 256, "fp16", 121, sink=True,
                                                       causal=True),
    "d256_gqa_bsnd": lambda: synth.dense_case("x", "BSND", 1, 4, 150, 256, "bf16", 122, nkv=2, skv=270),
    "d256_gqa_fp32": lambda: synth.dense_case("x", "BSND", 1, 4, 90, 256, "fp32", 123, nkv=1, causal=True),
    "d256_dv128_band_mask": lambda: _band_mask_case(124, 70, 9, d=256, dv=128),
    "d256_dv256_mask_blocks_sink": lambda: _block_mask_case(125, 128, 64, (1, 1), d=256, sink=True, skv=400),
    # Dqk > Dv on the matrix cores (the FAS page's head dims with the V5
    # page's kD >= vD): 96 -> 64, 128 -> 96 and 128 -> 64 (with pse, where the
    # rope-tail mapping does not apply), 256 -> 96 and 256 -> 64
    "d96_dv64_causal": lambda: synth.dense_case("x", "BSND", 1, 2, 190, 96, "bf16", 126, dv=64, causal=True),
    "d128_dv96_varlen_sink": lambda: synth.varlen_case("x", [130, 0, 257, 64], 2, 128, "bf16", 127, dv=96,
                                                       sink=True, causal=True),
    "d128_dv64_pse": lambda: synth.dense_case("x", "BNSD", 1, 2, 200, 128, "fp16", 128, dv=64, pse="full"),
    "d256_dv96_gqa_fp16": lambda: synth.dense_case("x", "BNSD", 1, 4, 150, 256, "fp16", 129, dv=96, nkv=2,
                                                   skv=230),
    "d256_dv64_pse_causal": lambda: synth.dense_case("x", "BNSD", 1, 2, 170, 256, "bf16", 136, dv=64, pse="full",
                                                     causal=True),
}


def _block_mask_case(seed, rb, cb, bn, *, dtype="bf16", d=128, drope=0, sink=False, pse=False, skv=650):
    """Mask of rb x cb blocks, each excluded (60%), kept (30%) or random (10%),
    plus one fully excluded row; 700 rows and skv keys."""
    c = synth.dense_case("x", "BNSD", 2, 2, 700, d, dtype, seed, skv=skv, drope=drope, sink=sink,
                         pse="full" if pse else None)
    return _add_block_mask(c, seed, rb, cb, bn, skv)


def _add_block_mask(c, seed, rb, cb, bn, skv):
    g = synth.generator(seed + 1000)
    nr, nc = -(-700 // rb), -(-skv // cb)
    kind = torch.rand(bn[0], bn[1], nr, nc, generator=g)
    blk = (kind < 0.6).repeat_interleave(rb, 2).repeat_interleave(cb, 3)[..., :700, :skv]
    rnd = (kind >= 0.9).repeat_interleave(rb, 2).repeat_interleave(cb, 3)[..., :700, :skv]
    noise = torch.rand(bn[0], bn[1], 700, skv, generator=g) < 0.5
    m = blk | (rnd & noise)
    m[..., 300, :] = True
    c.atten_mask = m.to(torch.uint8)
    return c


def _pse_lds_mask_case(seed):
    c = synth.dense_case("x", "BNSD", 1, 2, 330, 128, "bf16", seed, skv=320, sink=True, pse="full")
    i = torch.arange(330).view(-1, 1)
    j = torch.arange(320).view(1, -1)
    c.atten_mask = (((j - i) > 30) | ((i - j) > 150) | ((j % 61) == 7)).to(torch.uint8)
    c.pre_tokens, c.next_tokens = 150, 30
    return c


def _document_mask_case(seed):
    """Block-diagonal mask of documents whose boundaries differ per batch."""
    c = synth.dense_case("x", "BSND", 2, 3, 900, 128, "bf16", seed)
    m = torch.ones(2, 1, 900, 900, dtype=torch.bool)
    for b, cuts in enumerate(([0, 130, 400, 401, 900], [0, 256, 512, 700, 900])):
        for a, e in zip(cuts[:-1], cuts[1:]):
            m[b, 0, a:e, a:e] = False
    c.atten_mask = m
    return c


def _mask_inside_band_case(seed):
    """Window of 300 back and 100 ahead; the mask also drops whole blocks and
    a stripe inside it."""
    c = synth.dense_case("x", "BNSD", 1, 2, 800, 128, "bf16", seed)
    i = torch.arange(800).view(-1, 1)
    j = torch.arange(800).view(1, -1)
    band_out = ((j - i) > 100) | ((i - j) > 300)
    holes = ((i // 128) % 2 == 0) & ((j // 64) % 3 == 1)
    stripe = (j % 97) == 5
    c.atten_mask = (band_out | holes | stripe).to(torch.uint8)
    c.pre_tokens, c.next_tokens = 300, 100
    return c


def _mask_outside_band_case(seed):
    """The mask keeps positions the window excludes (the window still excludes
    them) and excludes blocks inside it."""
    c = synth.dense_case("x", "BNSD", 1, 2, 640, 128, "bf16", seed)
    i = torch.arange(640).view(-1, 1)
    j = torch.arange(640).view(1, -1)
    c.atten_mask = (((i // 128) + (j // 64)) % 4 == 0).to(torch.uint8)
    c.pre_tokens, c.next_tokens = 200, 0
    return c


def _mask_causal_holes_case(seed):
    """An explicit causal mask over 1100 rows (long runs of whole-kept blocks
    below the diagonal) with three blocks excluded inside the kept part: one
    for the first 128-row half of a 256-row tile, one for its second half, one
    for a whole row of blocks; the kept runs end there."""
    c = synth.dense_case("x", "BNSD", 1, 2, 1100, 128, "bf16", seed)
    i = torch.arange(1100).view(-1, 1)
    j = torch.arange(1100).view(1, -1)
    holes = ((i // 128 == 6) & (j // 64 == 5)) | ((i // 128 == 7) & (j // 64 == 9)) | ((j // 64 == 12) & (i >= 1024))
    c.atten_mask = ((j > i) | holes).to(torch.uint8)
    return c


def _tnd_block_mask_case(seed):
    c = synth.varlen_case("x", [300, 0, 17, 260], 2, 128, "bf16", seed)
    i = torch.arange(320).view(-1, 1)
    j = torch.arange(320).view(1, -1)
    c.atten_mask = ((((i // 128) + (j // 64)) % 3 == 0) | (j > i + 50)).to(torch.uint8)
    return c


def _pse_band_mask_case(seed):
    c = synth.dense_case("x", "BNSD", 1, 2, 230, 64, "bf16", seed, sink=True, pse="full")
    i = torch.arange(230).view(-1, 1)
    j = torch.arange(230).view(1, -1)
    c.atten_mask = (((j - i) > 4) | ((i - j) > 40)).to(torch.uint8)
    c.pre_tokens, c.next_tokens = 40, 4
    return c


def _band_mask_case(seed, pre, nxt, dtype="bf16", d=128, dv=None):
    c = synth.dense_case("x", "BNSD", 1, 2, 230, d, dtype, seed, dv=dv)
    i = torch.arange(230).view(-1, 1)
    j = torch.arange(230).view(1, -1)
    c.atten_mask = (((j - i) > nxt) | ((i - j) > pre)).to(torch.uint8)  # consistent with the window
    c.pre_tokens, c.next_tokens = pre, nxt
    return c


def _random_mask_case(seed, bn):
    c = synth.dense_case("x", "BNSD", 2, 2, 150, 128, "bf16", seed)
    g = synth.generator(seed + 1000)
    c.atten_mask = (torch.rand(bn[0], bn[1], 150, 150, generator=g) < 0.5).to(torch.bool)
    c.atten_mask[..., 7, :] = True  # a row with no kept key
    return c


def _tnd_small_mask_case(seed, causal=False, sink=False):
    """Sequences of 300, 0, 17 and 260 rows against a [200, 150] TND mask: the
    rows and keys of the long sequences beyond it are excluded."""
    c = synth.varlen_case("x", [300, 0, 17, 260], 2, 128, "bf16", seed, causal=causal, sink=sink)
    g = synth.generator(seed + 1000)
    i = torch.arange(200).view(-1, 1)
    j = torch.arange(150).view(1, -1)
    m = (torch.rand(200, 150, generator=g) < 0.2) | (((i // 128) + (j // 64)) % 3 == 1)
    m[:, 0] = False  # every row inside the mask keeps key 0
    c.atten_mask = m.to(torch.uint8)
    return c


def _tnd_mask_case(seed):
    c = synth.varlen_case("x", [100, 37, 140], 2, 128, "bf16", seed)
    g = synth.generator(seed + 1000)
    c.atten_mask = (torch.rand(160, 160, generator=g) < 0.3).to(torch.uint8)
    return c


def _sink_neg_inf_case(seed):
    c = synth.dense_case("x", "BNSD", 1, 3, 90, 128, "bf16", seed, sink=True, causal=True)
    c.sink = torch.tensor([float("-inf"), 0.5, float("-inf")])
    return c


KERNELS = ["auto", "mfma", "pp", "generic"]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_case(name, kernel):
    case = SMALL[name]()
    print(f"[parity] start {name} kernel={kernel} layout={case.layout} q={tuple(case.q.shape)} dtype={case.q.dtype}",
          flush=True)
    with pu.forced_kernel(kernel):
        try:
            errs = pu.compare_case(case)
        except _lib.FaError as e:
            if kernel != "auto" and e.code == _lib.FA_ERR_UNSUPPORTED and "FA_FWD_KERNEL" in e.message:
                pytest.skip(f"{kernel} does not cover this case")
            raise
    _report(f"{name}/{kernel}", errs)


# ---------------------------------------------------------------------------
# key split of the four-wave kernel: partial results over key ranges, merged
# ---------------------------------------------------------------------------

def _split_sink_neg_inf_case(seed):
    c = synth.dense_case("x", "BSND", 1, 3, 260, 128, "bf16", seed, skv=700, sink=True)
    c.sink = torch.tensor([float("-inf"), 1.5, -0.5])
    return c


def _split_window_case(seed):
    """A narrow window: many rows keep no key of some ranges, a few keep none
    at all (pre + next < 0 is rejected, so the empty rows come from the mask)."""
    c = synth.dense_case("x", "BNSD", 1, 2, 500, 128, "bf16", seed, skv=600, sink=True)
    i = torch.arange(500).view(-1, 1)
    j = torch.arange(600).view(1, -1)
    m = ((j - i) > 20) | ((i - j) > 90)
    m[:, :] |= (i >= 480) & (i < 490)  # ten rows with no kept key
    c.atten_mask = m.to(torch.uint8)
    c.pre_tokens, c.next_tokens = 90, 20
    return c


SPLIT = {
    "dense_ragged": lambda: synth.dense_case("x", "BNSD", 2, 3, 201, 128, "bf16", 100, skv=650),
    "sink_causal_bsnd": lambda: synth.dense_case("x", "BSND", 1, 3, 300, 128, "bf16", 101, sink=True, causal=True),
    "sink_neg_inf": lambda: _split_sink_neg_inf_case(102),
    "gqa_fp16_sq_lt_skv": lambda: synth.dense_case("x", "BNSD", 1, 4, 130, 128, "fp16", 103, nkv=2, skv=900),
    "d64_rope_causal": lambda: synth.dense_case("x", "BSND", 1, 2, 260, 64, "bf16", 104, drope=64, causal=True,
                                                skv=260),
    "d128_rope_sink": lambda: synth.dense_case("x", "BNSD", 1, 2, 200, 128, "bf16", 105, drope=64, sink=True,
                                               skv=520),
    "pse_lds_causal": lambda: synth.dense_case("x", "BNSD", 1, 2, 300, 128, "bf16", 106, skv=640, pse="full",
                                               causal=True),
    "pse_unaligned": lambda: synth.dense_case("x", "BNSD", 1, 2, 140, 128, "bf16", 107, skv=513, pse="bcast"),
    "block_mask": lambda: _block_mask_case(108, 128, 64, (1, 2)),
    "window_mask_empty_rows": lambda: _split_window_case(109),
    "sbh_layout": lambda: _split_sbh_case(110),
    "one_row_short_tail": lambda: synth.dense_case("x", "BNSD", 1, 2, 1, 128, "bf16", 112, skv=70, sink=True),
    "d96_sink_causal": lambda: synth.dense_case("x", "BNSD", 1, 3, 180, 96, "bf16", 114, skv=700, sink=True,
                                                causal=True),
    "d192_dv128_tail_rope": lambda: synth.dense_case("x", "BSND", 1, 2, 150, 192, "bf16", 115, dv=128, skv=700,
                                                     sink=True),
    "d64_gqa_band": lambda: synth.dense_case("x", "BSND", 2, 4, 190, 64, "fp16", 113, nkv=1, skv=610, causal=True,
                                             pre_tokens=200),
}


def _split_sbh_case(seed):
    base = synth.dense_case("x", "BNSD", 2, 3, 150, 128, "bf16", seed, skv=400, sink=True)
    return synth.Case(name="sbh", layout="SBH", q=orc.from_bnsd(base.q, "SBH"), k=orc.from_bnsd(base.k, "SBH"),
                      v=orc.from_bnsd(base.v, "SBH"), scale=base.scale, sink=base.sink)


@pytest.mark.parametrize("splits", ["2", "3", "4"])
@pytest.mark.parametrize("name", sorted(SPLIT))
def test_key_split(name, splits, monkeypatch):
    case = SPLIT[name]()
    print(f"[parity] start split {name} splits={splits} layout={case.layout} q={tuple(case.q.shape)}", flush=True)
    monkeypatch.setenv("FA_FWD_KV_SPLIT", splits)
    with pu.forced_kernel("mfma"):
        errs = pu.compare_case(case, heads=3 if case.layout == "SBH" else None)
    _report(f"split/{name}/{splits}", errs)


def test_key_split_chosen_for_small_grid():
    """B1 N2: four workgroups, so the plan itself splits the 2100 keys four ways."""
    case = synth.dense_case("x", "BNSD", 1, 2, 256, 128, "bf16", 111, skv=2100, sink=True)
    print("[parity] start split auto B1 N2 Sq256 Skv2100", flush=True)
    g = {k: pu.to_gpu(v, "cuda:0") for k, v in case.tensors().items()}
    out = torch.empty_like(g["q"])
    plan = api.ForwardPlan(g["q"], g["k"], g["v"], layout="BNSD", scale=case.scale, head_num=2, sink=g["sink"],
                           out=out)
    try:
        assert "kernel=mfma " in plan.describe() and "kv_splits=4" in plan.describe(), plan.describe()
    finally:
        plan.close()
    errs = pu.compare_case(case)
    _report("split/auto", errs)


@pytest.mark.parametrize("layout", ["BSH", "SBH"])
def test_hidden_layouts(layout):
    base = synth.dense_case("x", "BNSD", 2, 3, 150, 128, "bf16", 60, causal=True)
    case = synth.Case(name=layout, layout=layout, q=orc.from_bnsd(base.q, layout),
                      k=orc.from_bnsd(base.k, layout), v=orc.from_bnsd(base.v, layout), scale=base.scale,
                      causal=True)
    _report(layout, pu.compare_case(case, heads=3))


def test_noncontiguous_strides():
    """Views with padded rows and heads go through the matrix-core path unchanged."""
    g = synth.generator(61)
    big = synth.normal((1, 200, 3, 136), g, "bf16")  # pad D 128 -> 136 (multiple of 8 elements)
    q = big[..., :128]
    k = synth.normal((1, 200, 3, 136), g, "bf16")[..., :128]
    v = synth.normal((1, 200, 3, 136), g, "bf16")[..., :128]
    case = synth.Case(name="strided", layout="BSND", q=q, k=k, v=v, scale=128**-0.5, causal=True)
    qg, kg, vg = (big.cuda()[..., :128], k.contiguous().cuda(), v.contiguous().cuda())
    plan = api.attention_forward(qg, kg, vg, scale=case.scale, causal=True, return_plan=True)
    assert "kernel=mfma" in plan.describe(), plan.describe()
    torch.cuda.synchronize()
    O, _, _ = pu.run_oracle(case)
    pu.check_output(plan.out.cpu(), O, torch.bfloat16)
    plan.close()


@pytest.mark.parametrize("kernel", ["pp", "mfma"])
def test_overlapping_query_rows(kernel):
    """A query view whose rows overlap (row stride 64 elements < D = 128): the two-group kernel then loads
    each lane's fragments itself instead of staging the tile's rows through LDS."""
    B, N, S, D = 1, 2, 600, 128
    strides = (N * S * 64 + 64, S * 64 + 64, 64, 1)
    flat = synth.normal((N * S * 64 + 64 + D,), synth.generator(64), "bf16")
    q = torch.as_strided(flat, (B, N, S, D), strides)
    case = synth.dense_case("x", "BNSD", B, N, S, D, "bf16", 65)
    case.q = q
    print(f"[parity] start overlapping query rows kernel={kernel}", flush=True)
    qg = torch.as_strided(flat.cuda(), (B, N, S, D), strides)
    with pu.forced_kernel(kernel):
        plan = api.attention_forward(qg, case.k.cuda(), case.v.cuda(), layout="BNSD", scale=case.scale,
                                     return_plan=True)
    try:
        assert f"kernel={'mfma_pp' if kernel == 'pp' else 'mfma'} " in plan.describe(), plan.describe()
        torch.cuda.synchronize()
        O, _, _ = pu.run_oracle(case)
        _report(f"overlap/{kernel}", {"O": pu.check_output(plan.out.cpu(), O, torch.bfloat16)})
    finally:
        plan.close()


def test_misaligned_uses_generic_and_matches():
    g = synth.generator(62)
    flat = synth.normal((1 + 2 * 100 * 2 * 128,), g, "bf16")
    q = flat[1:].view(2, 100, 2, 128)
    case = synth.dense_case("x", "BSND", 2, 2, 100, 128, "bf16", 63)
    case.q = q
    qg = torch.empty(flat.numel(), dtype=torch.bfloat16, device="cuda")
    qg.copy_(flat.cuda())
    qg = qg[1:].view(2, 100, 2, 128)
    plan = api.attention_forward(qg, case.k.cuda(), case.v.cuda(), scale=case.scale, return_plan=True)
    assert "kernel=generic" in plan.describe()
    torch.cuda.synchronize()
    O, _, _ = pu.run_oracle(case)
    pu.check_output(plan.out.cpu(), O, torch.bfloat16)
    plan.close()


# ---------------------------------------------------------------------------
# determinism, guard bands, repeated plan execution
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", ["mfma", "pp"])
@pytest.mark.parametrize("name", ["c2_small_bf16", "c4_small_varlen", "c5_small_sink_rope"])
def test_bitwise_deterministic(name, kernel):
    case = SMALL[name]()
    with pu.forced_kernel(kernel):
        a = pu.run_gpu(case)
        b = pu.run_gpu(case)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32))


@pytest.mark.parametrize("splits", ["2", "4"])
def test_key_split_bitwise_deterministic(splits, monkeypatch):
    """The split's partials and merge use no atomics: two runs agree bit for bit."""
    monkeypatch.setenv("FA_FWD_KV_SPLIT", splits)
    case = SPLIT["d128_rope_sink"]()
    with pu.forced_kernel("mfma"):
        a = pu.run_gpu(case)
        b = pu.run_gpu(case)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32))


def test_guard_bands_untouched():
    case = synth.workload("c4_varlen_causal", small=True)
    T, N, D = case.q.shape
    pad = 4096
    poison = -12345.0
    obuf = torch.full((pad + T * N * D + pad,), poison, dtype=torch.bfloat16, device="cuda")
    out = obuf[pad:pad + T * N * D].view(T, N, D)
    sbuf = torch.full((pad + N * T * 8 + pad,), poison, dtype=torch.float32, device="cuda")
    smax = sbuf[pad:pad + N * T * 8].view(N, T, 8)
    g = {k: pu.to_gpu(v) for k, v in case.tensors().items()}
    plan = api.ForwardPlan(g["q"], g["k"], g["v"], layout="TND", scale=case.scale, head_num=N,
                           cu_seqlens_q=g["cu_seqlens_q"], cu_seqlens_kv=g["cu_seqlens_kv"], causal=True, out=out,
                           softmax_max=smax, softmax_sum=None)
    plan.run()
    torch.cuda.synchronize()
    for buf in (obuf, sbuf):
        assert bool((buf[:pad] == poison).all()) and bool((buf[-pad:] == poison).all())
    assert not bool((out == poison).any())
    O, M, _ = pu.run_oracle(case)
    pu.check_output(out.cpu(), O, torch.bfloat16)
    pu.check_stats(smax.cpu(), M, "max", torch.bfloat16)
    plan.close()


def test_guard_bands_malformed_cu_seqlens():
    """cu_seqlens that decrease and run past T: phase 2 clamps each sequence into [0, T), so the
    kernels write nothing outside O and the statistics (the rows the clamped sequences cover are
    written, the bands around the buffers stay as they were)."""
    T, N, D = 577, 2, 128
    g = synth.generator(130)
    q, k, v = (synth.normal((T, N, D), g, "bf16").cuda() for _ in range(3))
    cu = torch.tensor([0, 300, 200, 700], dtype=torch.int32, device="cuda")  # covers [0, 300) and [200, 577)
    pad, poison = 4096, -12345.0
    obuf = torch.full((pad + T * N * D + pad,), poison, dtype=torch.bfloat16, device="cuda")
    out = obuf[pad:pad + T * N * D].view(T, N, D)
    sbuf = torch.full((pad + N * T * 8 + pad,), poison, dtype=torch.float32, device="cuda")
    smax = sbuf[pad:pad + N * T * 8].view(N, T, 8)
    print("[parity] start guard bands, malformed cu_seqlens [0, 300, 200, 700] T=577", flush=True)
    plan = api.ForwardPlan(q, k, v, layout="TND", scale=D ** -0.5, head_num=N, cu_seqlens_q=cu, cu_seqlens_kv=cu,
                           causal=True, out=out, softmax_max=smax, softmax_sum=None)
    plan.run()
    pu.sync_with_deadline("forward with malformed cu_seqlens")
    plan.close()
    for buf in (obuf, sbuf):
        assert bool((buf[:pad] == poison).all()) and bool((buf[-pad:] == poison).all())
    assert not bool((out == poison).any()) and not bool((smax == poison).any())
    assert bool(torch.isfinite(out.float()).all())


def test_key_split_guard_bands_untouched(monkeypatch):
    """The split writes only its workspace and, through the merge, exactly the output and statistics rows."""
    monkeypatch.setenv("FA_FWD_KV_SPLIT", "3")
    case = SPLIT["dense_ragged"]()  # BNSD [2, 3, 201, 128], 650 keys
    B, N, S, D = case.q.shape
    pad = 4096
    poison = -12345.0
    obuf = torch.full((pad + B * N * S * D + pad,), poison, dtype=torch.bfloat16, device="cuda")
    out = obuf[pad:pad + B * N * S * D].view(B, N, S, D)
    sbuf = torch.full((pad + B * N * S * 8 + pad,), poison, dtype=torch.float32, device="cuda")
    smax = sbuf[pad:pad + B * N * S * 8].view(B, N, S, 8)
    g = {k: pu.to_gpu(v) for k, v in case.tensors().items()}
    with pu.forced_kernel("mfma"):
        plan = api.ForwardPlan(g["q"], g["k"], g["v"], layout="BNSD", scale=case.scale, head_num=N, out=out,
                               softmax_max=smax, softmax_sum=None)
    assert "kv_splits=3" in plan.describe(), plan.describe()
    plan.run()
    torch.cuda.synchronize()
    for buf in (obuf, sbuf):
        assert bool((buf[:pad] == poison).all()) and bool((buf[-pad:] == poison).all())
    assert not bool((out == poison).any()) and not bool((smax == poison).any())
    O, M, _ = pu.run_oracle(case)
    pu.check_output(out.cpu(), O, torch.bfloat16)
    pu.check_stats(smax.cpu(), M, "max", torch.bfloat16)
    plan.close()


def test_plan_reuse_and_stream():
    case = synth.workload("c2_dense_bsnd", "bf16", small=True)
    g = {k: pu.to_gpu(v) for k, v in case.tensors().items()}
    plan = api.attention_forward(g["q"], g["k"], g["v"], scale=case.scale, return_plan=True)
    first = plan.out.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan.out.zero_()
        for _ in range(3):
            plan.run()
    s.synchronize()
    assert torch.equal(first, plan.out)
    plan.close()


def test_v5_call_example_on_gpu():
    """The V5 page's call-example inputs: all-ones bf16 q/k/v + rope, sink 3.0, scale 0.088388."""
    T = 256
    ones = lambda *s: torch.ones(*s, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    out, smax, ssum = api.attention_forward_varlen(
        ones(T, 1, 128), ones(T, 1, 128), ones(T, 1, 128), cu, cu, softmax_scale=0.088388,
        q_rope=ones(T, 1, 64), k_rope=ones(T, 1, 64), sink=torch.tensor([3.0], device="cuda"),
        atten_mask=torch.zeros(T, T, dtype=torch.uint8, device="cuda"), pre_tokens=65536, next_tokens=65536,
        softmax_out_layout="same_as_input", return_softmax_stats=True)
    torch.cuda.synchronize()
    s = 0.088388 * 192
    m = max(s, 3.0)
    l = T * math.exp(s - m) + math.exp(3.0 - m)
    assert abs(float(smax[0, 0, 0]) - m) < 1e-3
    assert abs(math.log(float(ssum[0, 0, 0])) - math.log(l)) < 1e-3
    assert float((out.float() - 1.0).abs().max()) < 1e-2


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------

FULL = ["c2_bf16", "c2_fp16", "c3_causal", "c3_band", "c4_varlen_causal", "c5_varlen_sink_rope", "c6_dense_pse",
        "c2_gqa_nkv4", "c2_mqa", "d256_dense_bsnd"]


def _full_case(name):
    if name == "c2_bf16":
        return synth.workload("c2_dense_bsnd", "bf16")
    if name == "c2_fp16":
        return synth.workload("c2_dense_bsnd", "fp16")
    return synth.workload(name)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    case = _full_case(name)
    print(f"[parity] full {name} q={tuple(case.q.shape)}", flush=True)
    with pu.forced_kernel("auto"):
        # outputs start as NaN: an element no kernel writes fails the checks below
        o, smax, ssum = pu.run_gpu_poisoned(case)
    g = synth.generator(999)
    if case.layout == "TND":
        cu = case.cu_seqlens_q.tolist()
        nseq, nh = len(cu) - 1, case.q.shape[1]
        samples = []
        for b in range(nseq):
            n = cu[b + 1] - cu[b]
            for h in range(nh):
                if b in (0, nseq // 2, nseq - 1) and h in (0, nh - 1):
                    samples.append((b, h, pu.sample_rows(n, 12, g)))
                elif n > 0:  # the first and last row of every (sequence, head)
                    samples.append((b, h, torch.tensor(sorted({0, n - 1}), dtype=torch.int64)))
    else:
        B = case.q.shape[0]
        nh = case.q.shape[1] if case.layout == "BNSD" else case.q.shape[2]
        S = case.q.shape[2] if case.layout == "BNSD" else case.q.shape[1]
        samples = []
        for b in range(B):
            for h in range(nh):
                if b in (0, B - 1) and h in (0, nh // 2, nh - 1):
                    samples.append((b, h, pu.sample_rows(S, 12, g)))
                else:  # edge rows of every (batch, head): first, tile boundaries, last
                    samples.append((b, h, torch.tensor(sorted({0, 255, 256, S - 1}), dtype=torch.int64)))
    _report(name, pu.compare_sampled(case, samples, o, smax, ssum))
    # every element written (the NaN fill is gone), then properties at every row:
    # finite output, stats slots equal, l >= 1 where a key is kept
    assert not bool(torch.isnan(o.float()).any()), "output elements left unwritten"
    assert not bool(torch.isnan(smax).any()) and not bool(torch.isnan(ssum).any()), "statistics left unwritten"
    assert torch.isfinite(o.float()).all()
    assert bool((smax == smax[..., :1]).all()) and bool((ssum == ssum[..., :1]).all())
    assert bool((ssum[..., 0] >= 1.0 - 1e-6).all())


# ---------------------------------------------------------------------------
# outer split: key chunks with kv_start_idx, merged on the GPU
# ---------------------------------------------------------------------------

def _chunk_case(case, a, b):
    """The same problem restricted to keys [a, b) (BNSD)."""
    import copy
    c = copy.copy(case)
    c.k, c.v = case.k[:, :, a:b].contiguous(), case.v[:, :, a:b].contiguous()
    if case.atten_mask is not None:
        c.atten_mask = case.atten_mask[:, a:b].contiguous()
    if case.pse is not None:
        c.pse = case.pse[..., a:b].contiguous()
    return c


def _gpu_forward(case, *, q_start=None, kv_start=None, sink=True):
    g = {k: (v.to("cuda:0") if v is not None else None) for k, v in case.tensors().items()}
    res = api.attention_forward(g["q"], g["k"], g["v"], attn_mask=g["atten_mask"], scale=case.scale,
                                layout=case.layout, pre_tokens=case.pre_tokens, next_tokens=case.next_tokens,
                                sink=g["sink"] if sink else None, causal=case.causal, pse=g["pse"],
                                q_start_idx=q_start, kv_start_idx=kv_start, return_softmax_stats=True)
    return res


OUTER = {
    "causal": lambda: synth.dense_case("x", "BNSD", 1, 2, 500, 128, "bf16", 80, causal=True),
    "band_mask": lambda: _band_mask_case(81, 60, 5),
    "sink_causal_fp16": lambda: synth.dense_case("x", "BNSD", 2, 2, 300, 128, "fp16", 82, causal=True, sink=True),
    "pse_full": lambda: synth.dense_case("x", "BNSD", 1, 2, 260, 128, "bf16", 83, pse="full", causal=True),
    "fp32_causal": lambda: synth.dense_case("x", "BNSD", 1, 2, 150, 64, "fp32", 84, causal=True),
}


@pytest.mark.parametrize("kernel", ["auto", "mfma", "generic"])
@pytest.mark.parametrize("name", sorted(OUTER))
def test_outer_split_merge(name, kernel):
    case = OUTER[name]()
    if kernel == "mfma" and case.q.dtype == torch.float32:
        pytest.skip("the matrix-core kernels take f16 / bf16 only")
    S = case.k.shape[2]
    cuts = [0, S // 4 + 3, S // 4 + 4, (3 * S) // 5, S]
    print(f"[parity] outer split {name} kernel={kernel} cuts={cuts}", flush=True)
    parts = []
    with pu.forced_kernel(kernel):
        for c in range(len(cuts) - 1):
            a, b = cuts[c], cuts[c + 1]
            ch = _chunk_case(case, a, b)
            # one chunk per call; the sink goes to exactly one of them
            parts.append(_gpu_forward(ch, kv_start=a, sink=(c == 0)))
            if c == 1:  # each chunk on its own against the oracle with the same offset
                o1, m1, l1 = (x.cpu() for x in parts[-1])
                O, M, L = orc.attention_forward(ch.q, ch.k, ch.v, layout="BNSD", scale=ch.scale,
                                                atten_mask=ch.atten_mask, causal=ch.causal, pse=ch.pse,
                                                pre_tokens=ch.pre_tokens, next_tokens=ch.next_tokens,
                                                kv_start=a)
                pu.check_output(o1, O, case.q.dtype, "chunk O")
                pu.check_stats(m1, M, "max", case.q.dtype)
                pu.check_stats(l1, L, "sum", case.q.dtype)
        o, smax, ssum = api.merge_partials(parts, layout="BNSD", heads=case.q.shape[1])
        torch.cuda.synchronize()
    O, M, L = pu.run_oracle(case)
    dt = case.q.dtype
    errs = {"O": pu.check_output(o.cpu(), O, dt), "m": pu.check_stats(smax.cpu(), M, "max", dt),
            "logl": pu.check_stats(ssum.cpu(), L, "sum", dt)}
    _report(f"outer/{name}/{kernel}", errs)


@pytest.mark.parametrize("nparts", [2, 3, 5])
def test_merge_part_counts(nparts):
    """The merge's fixed-count forms (2, 3, 4 parts; 4 above) and its any-count form (5)."""
    case = OUTER["sink_causal_fp16"]()
    S = case.k.shape[2]
    cuts = [0] + [S * (c + 1) // nparts + (7 if c == 0 else 0) for c in range(nparts - 1)] + [S]
    print(f"[parity] merge parts={nparts} cuts={cuts}", flush=True)
    parts = [_gpu_forward(_chunk_case(case, a, b), kv_start=a, sink=(c == 0))
             for c, (a, b) in enumerate(zip(cuts[:-1], cuts[1:]))]
    o, smax, ssum = api.merge_partials(parts, layout="BNSD", heads=case.q.shape[1])
    torch.cuda.synchronize()
    O, M, L = pu.run_oracle(case)
    dt = case.q.dtype
    errs = {"O": pu.check_output(o.cpu(), O, dt), "m": pu.check_stats(smax.cpu(), M, "max", dt),
            "logl": pu.check_stats(ssum.cpu(), L, "sum", dt)}
    _report(f"merge/{nparts}", errs)


@pytest.mark.parametrize("kernel", ["auto", "generic"])
def test_outer_split_query_chunk(kernel):
    """Rows [r0, S) with q_start_idx = r0 against all keys equal those rows of the whole causal result."""
    case = synth.dense_case("x", "BNSD", 1, 2, 400, 128, "bf16", 85, causal=True, sink=True)
    r0 = 137
    import copy
    ch = copy.copy(case)
    ch.q = case.q[:, :, r0:].contiguous()
    with pu.forced_kernel(kernel):
        o, smax, ssum = (x.cpu() for x in _gpu_forward(ch, q_start=r0))
    O, M, L = pu.run_oracle(case)
    dt = case.q.dtype
    pu.check_output(o, O[:, :, r0:], dt, "query chunk O")
    pu.check_stats(smax, M[:, :, r0:], "max", dt)
    pu.check_stats(ssum, L[:, :, r0:], "sum", dt)

"""The benchmark's FLOP accounting, checked on the CPU against closed forms.

The workloads' throughput counts 2 (D + Dr) + 2 Dv FLOP per kept (query, key)
pair, with kept pairs counted on whole 128 x 128 blocks (the MindIE-SD
page's attention_forward example counts 4 B N S S D for a dense problem);
the exact kept-pair count is reported beside it.  Shapes only matter here,
so the stand-in cases hold meta tensors.
"""
import types

import pytest
import torch

import bench

UNBOUNDED = 2**31 - 1


def case(layout, q, k, v=None, *, causal=False, mask=False, pre=UNBOUNDED, nxt=UNBOUNDED, qr=None, cu=None):
    t = lambda s: torch.empty(s, device="meta", dtype=torch.bfloat16) if s is not None else None
    return types.SimpleNamespace(layout=layout, q=t(q), k=t(k), v=t(v or k), q_rope=t(qr), k_rope=t(qr), causal=causal,
                                 atten_mask=object() if mask else None, pre_tokens=pre, next_tokens=nxt,
                                 sink=None, pse=None,
                                 cu_seqlens_q=torch.tensor(cu) if cu else None,
                                 cu_seqlens_kv=torch.tensor(cu) if cu else None)


def test_dense_headline():
    # B2 S4096 N24 D128 BSND, no mask: every pair kept, 4 B N S^2 D
    c = case("BSND", (2, 4096, 24, 128), (2, 4096, 24, 128))
    assert bench.kept_pairs(c, block=128) == bench.kept_pairs(c) == 2 * 24 * 4096 * 4096
    assert bench.flops_per_pair(c) == 4 * 128
    assert bench.kept_pairs(c, block=128) * bench.flops_per_pair(c) == 412316860416
    # algorithmic bytes: Q, K, V read once, O written once, 2 x 8 fp32 statistics per row
    n = 2 * 4096 * 24 * 128 * 2
    assert bench.algorithmic_bytes(c) == 4 * n + 2 * (2 * 4096 * 24) * 8 * 4 == 213909504


def test_causal_and_band_blocks():
    # B4 N32 S8192 D128 with a lower-triangular mask: 64 x 65 / 2 = 2080 of the 4096 blocks of 128 x 128
    c = case("BNSD", (4, 32, 8192, 128), (4, 32, 8192, 128), mask=True, nxt=0)
    assert bench.kept_pairs(c, block=128) == 2080 * 128 * 128 * 4 * 32
    assert bench.kept_pairs(c) == 8192 * 8193 // 2 * 4 * 32
    # the same with preTokens = 2048: row-block r keeps blocks r - 16 .. r, 17 each once r >= 16
    b = case("BNSD", (4, 32, 8192, 128), (4, 32, 8192, 128), mask=True, pre=2048, nxt=0)
    blocks = sum(min(r, 16) + 1 for r in range(64))
    assert blocks == 952
    assert bench.kept_pairs(b, block=128) == blocks * 128 * 128 * 4 * 32
    exact = sum(min(i, 2048) + 1 for i in range(8192))
    assert bench.kept_pairs(b) == exact * 4 * 32


def test_varlen_rope_pairs():
    # TND T=16384 N=64, 8 causal sequences of 2048, rope 64: 640 FLOP per pair
    cu = [2048 * i for i in range(9)]
    c = case("TND", (16384, 64, 128), (16384, 64, 128), causal=True, nxt=0, qr=(16384, 64, 64), cu=cu)
    assert bench.flops_per_pair(c) == 640
    assert bench.kept_pairs(c) == 8 * 64 * (2048 * 2049 // 2)
    assert bench.kept_pairs(c, block=128) == 8 * 64 * (16 * 17 // 2) * 128 * 128


@pytest.mark.parametrize("sq,skv,pre,nxt,causal,mask", [(37, 50, 5, 3, False, True), (64, 64, UNBOUNDED, 0, True, False),
                                                        (70, 20, 10, 100, False, True), (9, 9, UNBOUNDED, UNBOUNDED,
                                                                                         False, False)])
def test_exact_pairs_brute_force(sq, skv, pre, nxt, causal, mask):
    # the window -pre <= j - i <= next (causal: next <= 0) applies with a mask or causal, else every pair
    c = case("BNSD", (1, 1, sq, 8), (1, 1, skv, 8), causal=causal, mask=mask, pre=pre, nxt=nxt)
    band = mask or causal
    n = min(nxt, 0) if causal else nxt
    want = sum(1 for i in range(sq) for j in range(skv) if not band or (-pre <= j - i <= n))
    assert bench.kept_pairs(c) == want
    # block count: whole 4 x 4 blocks that keep any pair
    blk = 4
    keep = lambda i, j: not band or (-pre <= j - i <= n)
    want_b = 0
    for ib in range(0, sq, blk):
        for jb in range(0, skv, blk):
            rows = range(ib, min(ib + blk, sq))
            cols = range(jb, min(jb + blk, skv))
            if any(keep(i, j) for i in rows for j in cols):
                want_b += len(rows) * len(cols)
    assert bench.kept_pairs(c, block=blk) == want_b

"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function takes the oracle module (normally ``oracle.attention``)
and raises AssertionError when the oracle disagrees with:
  * an independent scalar brute force (``tests/brute.py``) on tiny inputs;
  * a library routine the method reduces to in special cases
    (``torch.nn.functional.scaled_dot_product_attention`` in float64);
  * closed forms and invariants of softmax attention;
  * the call example of the aclnnFlashAttentionVarLenScoreV5 page
    (``tests/golden/v5_call_example.json``).

They are plain functions so that ``test_oracle_mutants.py`` can run them
against deliberately broken copies of the oracle and show each plausible
mistake is caught.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import torch
import torch.nn.functional as F

from . import brute

F64 = torch.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _close(a, b, what, rtol=1e-9, atol=1e-11):
    a = torch.as_tensor(a, dtype=F64)
    b = torch.as_tensor(b, dtype=F64)
    assert a.shape == b.shape, f"{what}: shape {tuple(a.shape)} vs {tuple(b.shape)}"
    torch.testing.assert_close(a, b, rtol=rtol, atol=atol, msg=lambda m: f"{what}: {m}")


def _rand(shape, g):
    return torch.randn(*shape, generator=g, dtype=F64)


# ---------------------------------------------------------------------------
# 1. Brute force over every feature combination, tiny shapes
# ---------------------------------------------------------------------------

def _brute_dense(q, k, v, scale, qr, kr, mask, causal, pre, nxt, sink):
    """BNSD tensors -> (O [B,N,Sq,Dv], m [B,N,Sq], l) by scalar loops."""
    B, N, Sq, _ = q.shape
    Nkv = k.shape[1]
    grp = N // Nkv
    O = torch.zeros(B, N, Sq, v.shape[3], dtype=F64)
    M = torch.zeros(B, N, Sq, dtype=F64)
    L = torch.zeros(B, N, Sq, dtype=F64)
    for b in range(B):
        for h in range(N):
            g = h // grp
            ms = None
            if mask is not None:
                ms = mask if mask.dim() == 2 else mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]
                ms = ms.tolist()
            o, m, l = brute.head(q[b, h].tolist(), k[b, g].tolist(), v[b, g].tolist(), scale,
                                 qr=qr[b, h].tolist() if qr is not None else None,
                                 kr=kr[b, g].tolist() if kr is not None else None,
                                 mask=ms, causal=causal, pre=pre, nxt=nxt,
                                 sink=float(sink[h]) if sink is not None else None)
            O[b, h] = torch.tensor(o, dtype=F64).view(Sq, -1)
            M[b, h] = torch.tensor(m, dtype=F64)
            L[b, h] = torch.tensor(l, dtype=F64)
    return O, M, L


def pin_brute_force_dense(orc):
    g = torch.Generator().manual_seed(11)
    B, N, Nkv, Sq, Skv, D, Dv, Dr = 2, 4, 2, 5, 7, 4, 3, 2
    q, k, v = _rand((B, N, Sq, D), g), _rand((B, Nkv, Skv, D), g), _rand((B, Nkv, Skv, Dv), g)
    qr, kr = _rand((B, N, Sq, Dr), g), _rand((B, Nkv, Skv, Dr), g)
    sink_f = _rand((N,), g) + 0.5
    masks = [None, torch.triu(torch.ones(Sq, Skv, dtype=torch.uint8), 1),
             (torch.rand(B, 1, Sq, Skv, generator=g) < 0.3).to(torch.uint8),
             (torch.rand(1, N, Sq, Skv, generator=g) < 0.3).to(torch.bool)]
    for mi, causal, pre, nxt, sk, rope in itertools.product(
            range(len(masks)), (False, True), (None, 2), (None, 1, 0), ("none", "finite", "neginf"),
            (False, True)):
        mask = masks[mi]
        sink = None if sk == "none" else (sink_f if sk == "finite" else torch.full((N,), -math.inf, dtype=F64))
        scale = 0.7
        want = _brute_dense(q, k, v, scale, qr if rope else None, kr if rope else None, mask, causal,
                            pre, nxt, sink)
        got = orc.attention_forward(q, k, v, layout="BNSD", scale=scale,
                                    q_rope=qr if rope else None, k_rope=kr if rope else None,
                                    atten_mask=mask, sink=sink, causal=causal, pre_tokens=pre,
                                    next_tokens=nxt)
        tag = f"brute dense mask={mi} causal={causal} pre={pre} next={nxt} sink={sk} rope={rope}"
        for a, b_, nm in zip(got, want, ("O", "m", "l")):
            _close(a, b_, f"{tag} {nm}")


def pin_brute_force_varlen(orc):
    g = torch.Generator().manual_seed(12)
    lq, lk = [3, 0, 5, 2, 4], [4, 1, 5, 0, 3]
    N, Nkv, D, Dv, Dr = 2, 1, 4, 4, 2
    Tq, Tk = sum(lq), sum(lk)
    q, k, v = _rand((Tq, N, D), g), _rand((Tk, Nkv, D), g), _rand((Tk, Nkv, Dv), g)
    qr, kr = _rand((Tq, N, Dr), g), _rand((Tk, Nkv, Dr), g)
    sink = _rand((N,), g)
    cq = [0] + list(itertools.accumulate(lq))
    ck = [0] + list(itertools.accumulate(lk))
    mask2d = (torch.rand(6, 6, generator=g) < 0.25).to(torch.uint8)
    for causal, rope, use_sink, pre, use_mask in itertools.product(
            (False, True), (False, True), (False, True), (None, 1), (False, True)):
        O, M, L = orc.attention_forward(q, k, v, layout="TND", scale=0.6,
                                        q_rope=qr if rope else None, k_rope=kr if rope else None,
                                        sink=sink if use_sink else None, causal=causal,
                                        atten_mask=mask2d if use_mask else None,
                                        pre_tokens=pre, next_tokens=None,
                                        cu_seqlens_q=cq, cu_seqlens_kv=ck)
        for b in range(len(lq)):
            for h in range(N):
                gh = h // (N // Nkv)
                sl_q, sl_k = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
                if lq[b] == 0:
                    continue
                ms = mask2d[:lq[b], :lk[b]].tolist() if use_mask else None
                o, m, l = brute.head(q[sl_q, h].tolist(), k[sl_k, gh].tolist(),
                                     v[sl_k, gh].tolist() if lk[b] else [], 0.6,
                                     qr=qr[sl_q, h].tolist() if rope else None,
                                     kr=kr[sl_k, gh].tolist() if rope else None,
                                     mask=ms, causal=causal, pre=pre, nxt=None,
                                     sink=float(sink[h]) if use_sink else None)
                tag = f"brute varlen b={b} h={h} causal={causal} rope={rope} sink={use_sink} pre={pre} mask={use_mask}"
                if lk[b]:
                    _close(O[sl_q, h], torch.tensor(o, dtype=F64), tag + " O")
                else:
                    _close(O[sl_q, h], torch.zeros(lq[b], Dv, dtype=F64), tag + " O")
                _close(M[h, sl_q], torch.tensor(m, dtype=F64), tag + " m")
                _close(L[h, sl_q], torch.tensor(l, dtype=F64), tag + " l")


def pin_tnd_mask_smaller_than_sequences(orc):
    """A 2-D TND mask smaller than some sequences: positions beyond its rows or
    columns are excluded (reading of the V5 parameter table, row
    attenMaskOptional).  The brute force builds each sequence's mask cell by
    cell: inside the mask it is the mask's byte, outside it is 1."""
    g = torch.Generator().manual_seed(19)
    lq, lk = [6, 2, 7, 3], [5, 4, 7, 1]
    N, D, Dv = 2, 4, 3
    Tq, Tk = sum(lq), sum(lk)
    q, k, v = _rand((Tq, N, D), g), _rand((Tk, N, D), g), _rand((Tk, N, Dv), g)
    sink = _rand((N,), g)
    cq = [0] + list(itertools.accumulate(lq))
    ck = [0] + list(itertools.accumulate(lk))
    mr, mc = 4, 3  # smaller than sequences 0 and 2 in both directions
    mask2d = (torch.rand(mr, mc, generator=g) < 0.3).to(torch.uint8)
    mask2d[0, 0] = 0  # row 0 keeps key 0 inside the mask
    ml = mask2d.tolist()
    for causal, use_sink in itertools.product((False, True), (False, True)):
        O, M, L = orc.attention_forward(q, k, v, layout="TND", scale=0.7, sink=sink if use_sink else None,
                                        causal=causal, atten_mask=mask2d, cu_seqlens_q=cq, cu_seqlens_kv=ck)
        for b in range(len(lq)):
            ms = [[ml[i][j] if (i < mr and j < mc) else 1 for j in range(lk[b])] for i in range(lq[b])]
            for h in range(N):
                sl_q, sl_k = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
                o, m, l = brute.head(q[sl_q, h].tolist(), k[sl_k, h].tolist(), v[sl_k, h].tolist(), 0.7,
                                     mask=ms, causal=causal, sink=float(sink[h]) if use_sink else None)
                tag = f"tnd small mask b={b} h={h} causal={causal} sink={use_sink}"
                _close(O[sl_q, h], torch.tensor(o, dtype=F64), tag + " O")
                _close(M[h, sl_q], torch.tensor(m, dtype=F64), tag + " m")
                _close(L[h, sl_q], torch.tensor(l, dtype=F64), tag + " l")
        # rows past the mask's extent keep no key: O = 0 and, without a sink, m = -inf and l = 0
        if not use_sink:
            assert bool((M[:, cq[0] + mr:cq[1]] == float("-inf")).all()), "rows beyond the mask must be empty"
            assert bool((O[cq[0] + mr:cq[1]] == 0).all())


# ---------------------------------------------------------------------------
# 2. Reductions to torch's scaled_dot_product_attention (float64, CPU)
# ---------------------------------------------------------------------------

def pin_sdpa(orc):
    g = torch.Generator().manual_seed(13)
    B, N, S, D = 2, 3, 37, 16
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    sc = 0.31
    # no mask
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=sc)
    _close(O, F.scaled_dot_product_attention(q, k, v, scale=sc), "sdpa plain")
    # causal flag
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, causal=True)
    _close(O, F.scaled_dot_product_attention(q, k, v, scale=sc, is_causal=True), "sdpa causal")
    # explicit mask (1 = excluded) vs SDPA's boolean (True = attend); keep the diagonal
    m = (torch.rand(B, N, S, S, generator=g) < 0.4)
    m &= ~torch.eye(S, dtype=torch.bool)
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, atten_mask=m.to(torch.uint8))
    _close(O, F.scaled_dot_product_attention(q, k, v, attn_mask=~m, scale=sc), "sdpa mask")
    # GQA: Nq = 6 query heads over Nkv = 2, heads grouped contiguously
    q6 = _rand((B, 6, S, D), g)
    O, _, _ = orc.attention_forward(q6, k[:, :2], v[:, :2], layout="BNSD", scale=sc)
    kk = k[:, :2].repeat_interleave(3, dim=1)
    vv = v[:, :2].repeat_interleave(3, dim=1)
    _close(O, F.scaled_dot_product_attention(q6, kk, vv, scale=sc), "sdpa gqa")
    # band with mask given: pre = 4, next = 2 -> keep -4 <= j - i <= 2
    zero = torch.zeros(S, S, dtype=torch.uint8)
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, atten_mask=zero,
                                    pre_tokens=4, next_tokens=2)
    i = torch.arange(S).view(-1, 1)
    j = torch.arange(S).view(1, -1)
    allow = ((j - i) <= 2) & ((i - j) <= 4)
    _close(O, F.scaled_dot_product_attention(q, k, v, attn_mask=allow, scale=sc), "sdpa band")


def pin_sink_extra_key(orc):
    """Sink == one extra key with logit sink_h and a zero value row (the sink equations)."""
    g = torch.Generator().manual_seed(14)
    B, N, S, D = 1, 3, 20, 8
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    sink = torch.tensor([0.5, -2.0, 4.0], dtype=F64)
    sc = 0.4
    for causal in (False, True):
        O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, sink=sink, causal=causal)
        k2 = torch.cat([k, torch.zeros(B, N, 1, D, dtype=F64)], 2)
        v2 = torch.cat([v, torch.zeros(B, N, 1, D, dtype=F64)], 2)
        bias = torch.zeros(B, N, S, S + 1, dtype=F64)
        if causal:
            bias[..., :S] = torch.triu(torch.full((S, S), -math.inf, dtype=F64), 1)
        bias[..., S] = sink.view(1, N, 1)
        _close(O, F.scaled_dot_product_attention(q, k2, v2, attn_mask=bias, scale=sc), f"sink extra key causal={causal}")
        logits = sc * q @ k2.transpose(-1, -2) + bias
        _close(M + torch.log(L), torch.logsumexp(logits, -1), f"sink logsumexp causal={causal}")
        _close(M, logits.amax(-1), f"sink max causal={causal}")


def pin_rope_linearity(orc):
    """scale*(Q K^T + Qr Kr^T) == scale*[Q|Qr][K|Kr]^T: the split equals the concatenation."""
    g = torch.Generator().manual_seed(15)
    B, N, S, D, Dr = 1, 2, 19, 8, 4
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    qr, kr = _rand((B, N, S, Dr), g), _rand((B, N, S, Dr), g)
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=0.3, q_rope=qr, k_rope=kr, causal=True)
    b = orc.attention_forward(torch.cat([q, qr], -1), torch.cat([k, kr], -1), v, layout="BNSD",
                              scale=0.3, causal=True)
    for x, y, nm in zip(a, b, "Oml"):
        _close(x, y, f"rope linearity {nm}")
    # and against SDPA on the concatenation
    _close(a[0], F.scaled_dot_product_attention(torch.cat([q, qr], -1), torch.cat([k, kr], -1), v,
                                                scale=0.3, is_causal=True), "rope sdpa")


def pin_varlen_block_diagonal(orc):
    """Per-sequence TND == one dense call over the packed rows with a block-diagonal mask."""
    g = torch.Generator().manual_seed(16)
    lens = [7, 1, 12, 5]
    T, N, D = sum(lens), 2, 8
    q, k, v = _rand((T, N, D), g), _rand((T, N, D), g), _rand((T, N, D), g)
    cu = [0] + list(itertools.accumulate(lens))
    seq = torch.repeat_interleave(torch.arange(len(lens)), torch.tensor(lens))
    pos = torch.cat([torch.arange(n) for n in lens])
    for causal in (False, True):
        O, M, L = orc.attention_forward(q, k, v, layout="TND", scale=0.5, causal=causal,
                                        cu_seqlens_q=cu, cu_seqlens_kv=cu)
        allow = seq.view(-1, 1) == seq.view(1, -1)
        if causal:
            allow &= pos.view(1, -1) <= pos.view(-1, 1)
        qd, kd, vd = (x.permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
        want = F.scaled_dot_product_attention(qd, kd, vd, attn_mask=allow, scale=0.5)[0].permute(1, 0, 2)
        _close(O, want, f"varlen block-diagonal causal={causal}")
        logits = 0.5 * qd[0] @ kd[0].transpose(-1, -2)
        logits = logits.masked_fill(~allow, -math.inf)
        _close(M + torch.log(L), torch.logsumexp(logits, -1), f"varlen logsumexp causal={causal}")


def pin_layouts(orc):
    """BSND / BSH / SBH / TND are relabelings of BNSD: outputs permute the same way."""
    g = torch.Generator().manual_seed(17)
    B, N, S, D = 2, 3, 11, 4
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    base = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True)
    bsnd = orc.attention_forward(*(x.permute(0, 2, 1, 3) for x in (q, k, v)), layout="BSND",
                                 scale=0.5, causal=True)
    _close(bsnd[0], base[0].permute(0, 2, 1, 3), "layout BSND O")
    _close(bsnd[1], base[1], "layout BSND m")
    bsh = orc.attention_forward(*(x.permute(0, 2, 1, 3).reshape(B, S, N * D) for x in (q, k, v)),
                                layout="BSH", heads=N, scale=0.5, causal=True)
    _close(bsh[0], base[0].permute(0, 2, 1, 3).reshape(B, S, N * D), "layout BSH O")
    sbh = orc.attention_forward(*(x.permute(2, 0, 1, 3).reshape(S, B, N * D) for x in (q, k, v)),
                                layout="SBH", heads=N, scale=0.5, causal=True)
    _close(sbh[0], base[0].permute(2, 0, 1, 3).reshape(S, B, N * D), "layout SBH O")
    tnd = orc.attention_forward(*(x.permute(0, 2, 1, 3).reshape(B * S, N, D) for x in (q, k, v)),
                                layout="TND", scale=0.5, causal=True, cu_seqlens_q=[0, S, 2 * S],
                                cu_seqlens_kv=[0, S, 2 * S])
    _close(tnd[0], base[0].permute(0, 2, 1, 3).reshape(B * S, N, D), "layout TND O")
    _close(tnd[1], base[1].permute(1, 0, 2).reshape(N, B * S), "layout TND m")


def pin_logsumexp(orc):
    """m + log l equals logsumexp of the kept logits; m equals their max."""
    g = torch.Generator().manual_seed(18)
    B, N, S, D = 1, 2, 23, 8
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    mask = torch.triu(torch.ones(S, S, dtype=torch.uint8), 1)
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=0.9, atten_mask=mask, pre_tokens=5,
                                    next_tokens=0)
    i = torch.arange(S).view(-1, 1)
    j = torch.arange(S).view(1, -1)
    allow = (j <= i) & (i - j <= 5)
    logits = (0.9 * q @ k.transpose(-1, -2)).masked_fill(~allow, -math.inf)
    _close(M, logits.amax(-1), "stats max")
    _close(M + torch.log(L), torch.logsumexp(logits, -1), "stats logsumexp")


# ---------------------------------------------------------------------------
# 3. Invariants and closed forms
# ---------------------------------------------------------------------------

def pin_rows_sum_to_one(orc):
    """With V = I the output row is the probability row; with a sink the rest is p_sink."""
    g = torch.Generator().manual_seed(19)
    S, D = 9, 5
    q, k = _rand((1, 1, S, D), g), _rand((1, 1, S, D), g)
    eye = torch.eye(S, dtype=F64).view(1, 1, S, S)
    for sink in (None, torch.tensor([1.3], dtype=F64)):
        O, M, L = orc.attention_forward(q, k, eye, layout="BNSD", scale=0.8, causal=True, sink=sink)
        tot = O.sum(-1)
        if sink is not None:
            tot = tot + torch.exp(sink[0] - M) / L
        _close(tot, torch.ones_like(tot), f"rows sum to one sink={sink is not None}")
        assert bool((O >= 0).all()), "probabilities must be non-negative"
        _close(O.triu(1), torch.zeros_like(O), "causal probabilities above the diagonal are zero")


def pin_single_key(orc):
    g = torch.Generator().manual_seed(20)
    q, k, v = _rand((1, 2, 6, 4), g), _rand((1, 2, 1, 4), g), _rand((1, 2, 1, 3), g)
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5)
    _close(O, v.expand(1, 2, 6, 3), "one key returns V")
    _close(L, torch.ones_like(L), "one key: l = 1")
    _close(M, 0.5 * (q @ k.transpose(-1, -2))[..., 0], "one key: m = s")


def pin_constant_v(orc):
    g = torch.Generator().manual_seed(21)
    S = 10
    q, k = _rand((1, 2, S, 4), g), _rand((1, 2, S, 4), g)
    row = torch.tensor([1.5, -2.0, 0.25], dtype=F64)
    v = row.expand(1, 2, S, 3).clone()
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True)
    _close(O, v, "constant V returns V")
    sink = torch.tensor([0.7, -1.1], dtype=F64)
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True, sink=sink)
    p_sink = torch.exp(sink.view(1, 2, 1) - M) / L
    _close(O, v * (1 - p_sink).unsqueeze(-1), "constant V with sink returns V*(1-p_sink)")


def pin_sink_neg_inf(orc):
    g = torch.Generator().manual_seed(22)
    q, k, v = _rand((1, 2, 8, 4), g), _rand((1, 2, 8, 4), g), _rand((1, 2, 8, 4), g)
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True)
    b = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True,
                              sink=torch.full((2,), -math.inf, dtype=F64))
    for x, y, nm in zip(a, b, "Oml"):
        _close(x, y, f"sink -inf equals no sink ({nm})")


def pin_causal_row0(orc):
    g = torch.Generator().manual_seed(23)
    q, k, v = _rand((1, 1, 7, 4), g), _rand((1, 1, 7, 4), g), _rand((1, 1, 7, 3), g)
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True)
    _close(O[0, 0, 0], v[0, 0, 0], "causal row 0 returns V_0")
    _close(M[0, 0, 0], 0.5 * float(q[0, 0, 0] @ k[0, 0, 0]), "causal row 0: m = s_00")
    _close(L[0, 0, 0], 1.0, "causal row 0: l = 1")


def pin_band_closed_form(orc):
    """pre/next direction: the window keeps -pre <= j - i <= next."""
    g = torch.Generator().manual_seed(24)
    S = 8
    q, k, v = _rand((1, 1, S, 4), g), _rand((1, 1, S, 4), g), _rand((1, 1, S, 3), g)
    zero = torch.zeros(S, S, dtype=torch.uint8)
    s = 0.5 * (q @ k.transpose(-1, -2))[0, 0]
    # pre = next = 0 -> only the diagonal
    O, M, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, atten_mask=zero, pre_tokens=0,
                                    next_tokens=0)
    _close(O[0, 0], v[0, 0], "band 0/0 returns V_i")
    _close(M[0, 0], torch.diagonal(s), "band 0/0 m = s_ii")
    # pre = 1, next = 0 -> keys {i-1, i}
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, atten_mask=zero, pre_tokens=1,
                                    next_tokens=0)
    for i in range(1, S):
        w = 1.0 / (1.0 + math.exp(float(s[i, i] - s[i, i - 1])))
        _close(O[0, 0, i], w * v[0, 0, i - 1] + (1 - w) * v[0, 0, i], f"band pre=1 row {i}")
    # pre = 0, next = 1 -> keys {i, i+1}
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, atten_mask=zero, pre_tokens=0,
                                    next_tokens=1)
    for i in range(S - 1):
        w = 1.0 / (1.0 + math.exp(float(s[i, i] - s[i, i + 1])))
        _close(O[0, 0, i], w * v[0, 0, i + 1] + (1 - w) * v[0, 0, i], f"band next=1 row {i}")
    # without a mask and without causal the band is ignored
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, pre_tokens=0, next_tokens=0)
    b = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5)
    _close(a[0], b[0], "band ignored without mask or causal")


def pin_shift_invariance(orc):
    """Adding c_i to every logit of row i (via one extra rope column) leaves O and l unchanged."""
    g = torch.Generator().manual_seed(25)
    S = 9
    q, k, v = _rand((1, 1, S, 4), g), _rand((1, 1, S, 4), g), _rand((1, 1, S, 3), g)
    c = _rand((S,), g) * 3
    sc = 0.5
    qr = (c / sc).view(1, 1, S, 1)
    kr = torch.ones(1, 1, S, 1, dtype=F64)
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, causal=True)
    b = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, causal=True, q_rope=qr, k_rope=kr)
    _close(b[0], a[0], "row shift leaves O unchanged")
    _close(b[2], a[2], "row shift leaves l unchanged")
    _close(b[1], a[1] + c.view(1, 1, S), "row shift moves m by c")


def pin_key_permutation(orc):
    g = torch.Generator().manual_seed(26)
    S = 12
    q, k, v = _rand((1, 2, S, 4), g), _rand((1, 2, S, 4), g), _rand((1, 2, S, 3), g)
    perm = torch.randperm(S, generator=g)
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5)
    b = orc.attention_forward(q, k[:, :, perm], v[:, :, perm], layout="BNSD", scale=0.5)
    for x, y, nm in zip(a, b, "Oml"):
        _close(x, y, f"key permutation ({nm})")


def pin_scale_zero(orc):
    g = torch.Generator().manual_seed(27)
    S = 10
    q, k, v = _rand((1, 1, S, 4), g), _rand((1, 1, S, 4), g), _rand((1, 1, S, 3), g)
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=0.0, causal=True)
    csum = torch.cumsum(v[0, 0], 0) / torch.arange(1, S + 1, dtype=F64).view(-1, 1)
    _close(O[0, 0], csum, "scale 0 gives the running mean of V")
    _close(L[0, 0], torch.arange(1, S + 1, dtype=F64), "scale 0: l counts kept keys")


def pin_fully_masked_rows(orc):
    """Rows with no kept key: O = 0; (m, l) = (-inf, 0), or (sink, 1) with a sink."""
    g = torch.Generator().manual_seed(28)
    S = 6
    q, k, v = _rand((1, 2, S, 4), g), _rand((1, 2, S, 4), g), _rand((1, 2, S, 3), g)
    mask = torch.zeros(S, S, dtype=torch.uint8)
    mask[2] = 1
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, atten_mask=mask)
    _close(O[0, :, 2], torch.zeros(2, 3, dtype=F64), "empty row O = 0")
    assert bool(torch.isneginf(M[0, :, 2]).all()) and float(L[0, :, 2].abs().max()) == 0.0
    sink = torch.tensor([0.25, -3.0], dtype=F64)
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, atten_mask=mask, sink=sink)
    _close(O[0, :, 2], torch.zeros(2, 3, dtype=F64), "empty row with sink O = 0")
    _close(M[0, :, 2], sink, "empty row with sink m = sink")
    _close(L[0, :, 2], torch.ones(2, dtype=F64), "empty row with sink l = 1")


# ---------------------------------------------------------------------------
# 4. The V5 page's call example
# ---------------------------------------------------------------------------

def pin_v5_call_example(orc):
    """Inputs of the call example (all-ones q/k/v and rope parts, sink 3.0) and the
    values the attention and sink equations give for them in closed form."""
    with open(os.path.join(GOLDEN, "v5_call_example.json")) as f:
        ex = json.load(f)
    T, N = ex["T"], ex["N"]
    D, Dr, Dv = ex["D"], ex["D_rope"], ex["D_v"]
    ones = lambda *s: torch.ones(*s, dtype=torch.bfloat16)
    O, M, L = orc.attention_forward(
        ones(T, N, D), ones(T, N, D), ones(T, N, Dv), layout="TND", scale=ex["scale"],
        q_rope=ones(T, N, Dr), k_rope=ones(T, N, Dr),
        atten_mask=torch.zeros(*ex["atten_mask_shape"], dtype=torch.uint8),
        sink=torch.tensor(ex["sink"], dtype=torch.float32), pre_tokens=ex["pre_tokens"],
        next_tokens=ex["next_tokens"], cu_seqlens_q=[0, T], cu_seqlens_kv=[0, T])
    # closed form: every logit equals s = scale * (D + Dr)
    s = ex["scale"] * (D + Dr)
    sink = float(torch.tensor(ex["sink"][0], dtype=torch.float32))
    m = max(s, sink)
    l = T * math.exp(s - m) + math.exp(sink - m)
    o = T * math.exp(s - m) / l
    _close(M, torch.full((N, T), m, dtype=F64), "v5 example softmaxMax")
    _close(L, torch.full((N, T), l, dtype=F64), "v5 example softmaxSum")
    _close(O, torch.full((T, N, Dv), o, dtype=F64), "v5 example output")
    # the page's actualSeqQLen form (cumulative, no leading 0) describes the same single sequence
    assert ex["actual_seq_q_len"] == [T] and ex["actual_seq_kv_len"] == [T]



# ---------------------------------------------------------------------------
# pse (realShift): the additive bias of the attention equation, after the scale
# ---------------------------------------------------------------------------

def pin_pse_brute_force(orc):
    """Dense and TND pse against the scalar brute force, with masks, causal, sink and GQA."""
    g = torch.Generator().manual_seed(21)
    B, N, Nkv, Sq, Skv, D = 2, 4, 2, 5, 6, 4
    q, k, v = _rand((B, N, Sq, D), g), _rand((B, Nkv, Skv, D), g), _rand((B, Nkv, Skv, D), g)
    sink = _rand((N,), g)
    pses = [_rand((B, N, Sq, Skv), g), _rand((1, N, Sq, Skv), g)]
    mask = (torch.rand(B, 1, Sq, Skv, generator=g) < 0.3).to(torch.uint8)
    for pi, causal, use_mask, use_sink in itertools.product(range(2), (False, True), (False, True), (False, True)):
        pse = pses[pi]
        got = orc.attention_forward(q, k, v, layout="BNSD", scale=0.45, pse=pse, causal=causal,
                                    atten_mask=mask if use_mask else None, sink=sink if use_sink else None)
        for b in range(B):
            for h in range(N):
                gh = h // (N // Nkv)
                o, m, l = brute.head(q[b, h].tolist(), k[b, gh].tolist(), v[b, gh].tolist(), 0.45,
                                     mask=mask[b, 0].tolist() if use_mask else None, causal=causal,
                                     sink=float(sink[h]) if use_sink else None,
                                     pse=pse[b if pse.shape[0] > 1 else 0, h].tolist())
                tag = f"pse brute dense pse={pi} causal={causal} mask={use_mask} sink={use_sink} b={b} h={h}"
                _close(got[0][b, h], torch.tensor(o, dtype=F64), tag + " O")
                _close(got[1][b, h], torch.tensor(m, dtype=F64), tag + " m")
                _close(got[2][b, h], torch.tensor(l, dtype=F64), tag + " l")
    # TND: one flat pse, an [N, Sq_i, Skv_i] block per sequence
    lq, lk = [3, 4, 2], [2, 4, 5]
    Nt = 2
    cq = [0] + list(itertools.accumulate(lq))
    ck = [0] + list(itertools.accumulate(lk))
    qt, kt, vt = _rand((cq[-1], Nt, D), g), _rand((ck[-1], Nt, D), g), _rand((ck[-1], Nt, D), g)
    flat = _rand((sum(Nt * a * b_ for a, b_ in zip(lq, lk)),), g)
    O, M, L = orc.attention_forward(qt, kt, vt, layout="TND", scale=0.45, pse=flat, causal=True,
                                    cu_seqlens_q=cq, cu_seqlens_kv=ck)
    off = 0
    for bi in range(len(lq)):
        blk = flat[off:off + Nt * lq[bi] * lk[bi]].view(Nt, lq[bi], lk[bi])
        off += Nt * lq[bi] * lk[bi]
        for h in range(Nt):
            o, m, l = brute.head(qt[cq[bi]:cq[bi + 1], h].tolist(), kt[ck[bi]:ck[bi + 1], h].tolist(),
                                 vt[ck[bi]:ck[bi + 1], h].tolist(), 0.45, causal=True, pse=blk[h].tolist())
            tag = f"pse brute TND seq={bi} h={h}"
            _close(O[cq[bi]:cq[bi + 1], h], torch.tensor(o, dtype=F64), tag + " O")
            _close(M[h, cq[bi]:cq[bi + 1]], torch.tensor(m, dtype=F64), tag + " m")
            _close(L[h, cq[bi]:cq[bi + 1]], torch.tensor(l, dtype=F64), tag + " l")


def pin_pse_sdpa(orc):
    """SDPA adds a float attn_mask to the scaled scores: exactly the equation's + pse."""
    g = torch.Generator().manual_seed(22)
    B, N, S, D = 2, 3, 29, 8
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    pse = 2.0 * _rand((1, N, S, S), g)
    sc = 0.37
    O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, pse=pse)
    _close(O, F.scaled_dot_product_attention(q, k, v, attn_mask=pse, scale=sc), "pse sdpa")
    logits = sc * q @ k.transpose(-1, -2) + pse
    _close(M + torch.log(L), torch.logsumexp(logits, -1), "pse logsumexp")
    _close(M, logits.amax(-1), "pse max")
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, pse=pse, causal=True)
    causal_bias = torch.triu(torch.full((S, S), -math.inf, dtype=F64), 1)
    _close(O, F.scaled_dot_product_attention(q, k, v, attn_mask=pse + causal_bias, scale=sc), "pse sdpa causal")


def pin_pse_row_shift_and_neg_inf(orc):
    """A per-row constant in pse shifts m and leaves O, l alone; pse = -inf acts as the mask."""
    g = torch.Generator().manual_seed(23)
    B, N, S, D = 1, 2, 17, 8
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    pse = _rand((B, N, S, S), g)
    c = _rand((B, N, S, 1), g) * 3
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, pse=pse)
    b = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, pse=pse + c)
    _close(b[0], a[0], "pse row shift O")
    _close(b[1], a[1] + c[..., 0], "pse row shift m")
    _close(b[2], a[2], "pse row shift l")
    mask = (torch.rand(B, N, S, S, generator=g) < 0.4)
    mask &= ~torch.eye(S, dtype=torch.bool)
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, atten_mask=mask.to(torch.uint8))
    b = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5,
                              pse=torch.zeros(B, N, S, S, dtype=F64).masked_fill(mask, -math.inf))
    for x, y, nm in zip(a, b, "Oml"):
        _close(y, x, f"pse -inf as mask {nm}")


# ---------------------------------------------------------------------------
# Outer split: qStartIdx / kvStartIdx offsets and the merge of partial results
# ---------------------------------------------------------------------------

def pin_outer_split_offsets(orc):
    """A query / key chunk with global offsets equals SDPA with the global-position causal or band mask."""
    g = torch.Generator().manual_seed(31)
    B, N, D = 1, 2, 8
    q, k, v = _rand((B, N, 23, D), g), _rand((B, N, 17, D), g), _rand((B, N, 17, D), g)
    sc = 0.4
    for qs, ks, causal, pre, nxt in [(30, 20, True, None, None), (5, 25, True, None, None),
                                     (40, 30, False, 6, 3), (0, 0, True, None, None), (12, 3, True, 8, 0)]:
        mask = None if causal else torch.zeros(23, 17, dtype=torch.uint8)
        O, M, L = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, causal=causal, atten_mask=mask,
                                        pre_tokens=pre, next_tokens=nxt, q_start=qs, kv_start=ks)
        ig = torch.arange(23).view(-1, 1) + qs
        jg = torch.arange(17).view(1, -1) + ks
        allow = torch.ones(23, 17, dtype=torch.bool)
        if causal:
            allow &= jg <= ig
        if pre is not None:
            allow &= (ig - jg) <= pre
        if nxt is not None:
            allow &= (jg - ig) <= nxt
        logits = (sc * q @ k.transpose(-1, -2)).masked_fill(~allow, -math.inf)
        rows = allow.any(-1)
        want = F.scaled_dot_product_attention(q, k, v, attn_mask=allow | ~rows.view(-1, 1), scale=sc)
        want = torch.where(rows.view(1, 1, -1, 1), want, torch.zeros_like(want))
        tag = f"outer split q_start={qs} kv_start={ks} causal={causal} pre={pre} next={nxt}"
        _close(O, want, tag + " O")
        lse = torch.logsumexp(logits, -1)
        _close(torch.where(rows.view(1, 1, -1), M + torch.log(L), lse), lse, tag + " lse")
    # an explicit mask stays in the chunk's own coordinates
    rm = torch.rand(23, 17, generator=g) < 0.3
    O, _, _ = orc.attention_forward(q, k, v, layout="BNSD", scale=sc, causal=True, atten_mask=rm.to(torch.uint8),
                                    q_start=30, kv_start=20)
    allow = ~rm & ((torch.arange(17).view(1, -1) + 20) <= (torch.arange(23).view(-1, 1) + 30))
    rows = allow.any(-1)
    want = F.scaled_dot_product_attention(q, k, v, attn_mask=allow | ~rows.view(-1, 1), scale=sc)
    want = torch.where(rows.view(1, 1, -1, 1), want, torch.zeros_like(want))
    _close(O, want, "outer split with a chunk-local mask")


def pin_outer_split_merge(orc):
    """Key chunks with kv_start offsets, merged, equal the unsplit call (causal, band, sink in one chunk)."""
    g = torch.Generator().manual_seed(32)
    B, N, S, D = 2, 2, 29, 8
    q, k, v = _rand((B, N, S, D), g), _rand((B, N, S, D), g), _rand((B, N, S, D), g)
    sink = _rand((N,), g)
    cuts = [0, 6, 7, 19, 29]
    for causal, band, use_sink in itertools.product((False, True), (False, True), (False, True)):
        kw = dict(layout="BNSD", scale=0.5, causal=causal)
        if band:
            kw.update(atten_mask=torch.zeros(S, S, dtype=torch.uint8), pre_tokens=5, next_tokens=2)
        whole = orc.attention_forward(q, k, v, sink=sink if use_sink else None, **kw)
        parts = []
        for c in range(len(cuts) - 1):
            a, b_ = cuts[c], cuts[c + 1]
            kwc = dict(kw)
            if band:
                kwc["atten_mask"] = torch.zeros(S, b_ - a, dtype=torch.uint8)
            parts.append(orc.attention_forward(q, k[:, :, a:b_], v[:, :, a:b_], kv_start=a,
                                               sink=sink if (use_sink and c == 1) else None, **kwc))
        merged = orc.merge_partials(parts)
        tag = f"merge causal={causal} band={band} sink={use_sink}"
        for x, y, nm in zip(merged, whole, "Oml"):
            _close(x, y, f"{tag} {nm}")


def pin_offsets_relative_only(orc):
    """Equal offsets on both sides change nothing: only relative positions enter the window."""
    g = torch.Generator().manual_seed(33)
    q, k, v = _rand((1, 2, 21, 8), g), _rand((1, 2, 21, 8), g), _rand((1, 2, 21, 8), g)
    a = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True, pre_tokens=4)
    b = orc.attention_forward(q, k, v, layout="BNSD", scale=0.5, causal=True, pre_tokens=4, q_start=9, kv_start=9)
    for x, y, nm in zip(a, b, "Oml"):
        _close(y, x, f"offsets relative {nm}")

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

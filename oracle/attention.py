"""CPU float64 oracle for the FlashAttention forward score-and-output computation.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path (the
HIP library and its Python binding) never does.  It shares no code with the
HIP path: it computes the plain definition with whole-row softmax, no tiling,
no online rescaling, no exp2, no block skipping.

What it computes (aclnnFlashAttentionVarLenScoreV5 page, 功能说明 → 计算公式,
the attention equation and the three sink equations below it):

    s_ij = scale * ( q_i . k_j  +  qrope_i . krope_j )  +  pse_ij
    masked(i, j)  ->  s_ij = -inf
    m_i  = max( max_j s_ij , sink_h )                  (sink term only if given)
    l_i  = sum_j e^(s_ij - m_i)  +  e^(sink_h - m_i)
    O_i  = sum_j e^(s_ij - m_i) v_j / l_i

and it reports ``softmaxMax = m_i`` and ``softmaxSum = l_i`` per query row
(the same page's parameter table, rows softmaxMaxOut / softmaxSumOut, which
says the sink changes both).

Readings where the pages are silent or garbled (each one also listed with its
reason in the design notes):
  * The mask marks EXCLUDED positions with 1/True (V5 parameter table, row
    attenMaskOptional; aclnnFlashAttentionScore page, parameter attenMask) and
    an excluded logit is -inf, so its weight is exactly 0.
  * preTokens / nextTokens (V5 parameter table, rows preTokens / nextTokens)
    bound a window: key j is kept for row i iff -pre <= j - i <= next, both
    ends inclusive.  The window only acts when a mask is given or the causal
    flag is set (V5 约束说明: without attenMaskOptional the band parameters do
    not take effect).  Mask, causal and band restrict by union.
  * causal (MindIE-SD attention_forward_varlen page, 参数说明 row causal)
    excludes j > i with positions counted from the start of each sequence
    (top-left alignment).
  * In TND each sequence is its own problem: positions are local to the
    sequence and a query never sees another sequence's keys (V5 约束说明 on
    TND: T is B and S packed tightly).  A mask given with TND is one 2-D
    [S1, S2] matrix read in sequence-local coordinates (the V5 call example
    passes a [256, 256] mask with TND); a position of a sequence that lies
    beyond the mask's rows or columns counts as excluded.
  * The sink is in logit units: it is neither scaled nor biased.  A sink of
    -inf contributes nothing (it must equal "no sink").
  * A row with no kept key has O = 0, m = -inf, l = 0 without a sink, and
    O = 0, m = sink, l = 1 with a finite sink.
  * GQA: query head h reads key/value head h // (Nq / Nkv) (V5 约束说明 on
    Nq / Nkv); the sink is indexed by the query head.
  * The value head dim Dv may be smaller than Dqk; O has Dv columns.
  * pse (realShift) is added after the scale, as the attention equation
    writes it (that order is pseType 1 on the V5 page; the other pseType
    values are not defined there).  Dense: [B or 1, N, Sq, Skv].  TND: one
    flat tensor holding, sequence after sequence, an [N, Sq_i, Skv_i] block
    (V5 约束说明 on realShiftOptional with TND).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import torch

NEG_INF = float("-inf")
ROW_CHUNK = 1024  # rows per fp64 score block, bounds the memory of one step

__all__ = ["keep_matrix", "head_attention", "attention_forward", "to_bnsd", "from_bnsd",
           "expand_stats", "merge_partials", "NEG_INF"]


def keep_matrix(rows: torch.Tensor, skv: int, *, mask: Optional[torch.Tensor], causal: bool,
                pre_tokens: Optional[int], next_tokens: Optional[int], q_start: int = 0,
                kv_start: int = 0) -> torch.Tensor:
    """Boolean [R, skv]: True where key j is KEPT for query row ``rows[r]``.

    ``mask`` is the [Sq, Skv] slice for this (batch, head), nonzero = excluded,
    in the chunk's own coordinates.  ``q_start`` / ``kv_start`` place the
    chunk's rows and keys in the whole sequence (the V5 page's qStartIdx /
    kvStartIdx for an outer split): causal and band tests use the global
    positions i + q_start and j + kv_start.  Follows the mask / causal / band
    readings stated in the module docstring.
    """
    il = rows.to(torch.int64).view(-1, 1)
    jl = torch.arange(skv, dtype=torch.int64).view(1, -1)
    i = il + int(q_start)
    j = jl + int(kv_start)
    keep = torch.ones(il.shape[0], skv, dtype=torch.bool)
    if mask is not None:
        keep &= mask.index_select(0, rows.to(torch.int64)) == 0
    if causal:
        keep &= j <= i
    if mask is not None or causal:
        if pre_tokens is not None:
            keep &= (i - j) <= int(pre_tokens)
        if next_tokens is not None:
            keep &= (j - i) <= int(next_tokens)
    return keep


def head_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: float,
                   q_rope: Optional[torch.Tensor] = None, k_rope: Optional[torch.Tensor] = None,
                   mask: Optional[torch.Tensor] = None, causal: bool = False,
                   pre_tokens: Optional[int] = None, next_tokens: Optional[int] = None,
                   sink: Optional[float] = None, rows: Optional[torch.Tensor] = None,
                   pse: Optional[torch.Tensor] = None, q_start: int = 0, kv_start: int = 0
                   ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Attention for one (sequence, query head): q [Sq,D], k [Skv,D], v [Skv,Dv].

    ``pse`` is this head's [Sq, Skv] additive position bias (or None).

    Returns (O [R, Dv], m [R], l [R]) in float64 for the query rows ``rows``
    (all rows by default).  This is the V5 page's attention equation with its
    sink equations, evaluated row block by row block.
    """
    q = q.to(torch.float64)
    k = k.to(torch.float64)
    v = v.to(torch.float64)
    qr = q_rope.to(torch.float64) if q_rope is not None else None
    kr = k_rope.to(torch.float64) if k_rope is not None else None
    sq, skv, dv = q.shape[0], k.shape[0], v.shape[1]
    if rows is None:
        rows = torch.arange(sq, dtype=torch.int64)
    rows = rows.to(torch.int64)
    use_sink = sink is not None and not (math.isinf(sink) and sink < 0)
    outs, ms, ls = [], [], []
    for c0 in range(0, rows.numel(), ROW_CHUNK):
        r = rows[c0:c0 + ROW_CHUNK]
        # scores: scale * (Q K^T + Qrope Krope^T)
        s = q.index_select(0, r) @ k.T
        if qr is not None:
            s = s + qr.index_select(0, r) @ kr.T
        s = scale * s
        if pse is not None:
            s = s + pse.index_select(0, r).to(torch.float64)
        keep = keep_matrix(r, skv, mask=mask, causal=causal, pre_tokens=pre_tokens,
                           next_tokens=next_tokens, q_start=q_start, kv_start=kv_start)
        s = s.masked_fill(~keep, NEG_INF)
        # m = max(sink, max_j s_ij)
        m = s.amax(dim=1) if skv > 0 else torch.full((r.numel(),), NEG_INF, dtype=torch.float64)
        if use_sink:
            m = torch.clamp(m, min=float(sink))
        finite = torch.isfinite(m)
        m_safe = torch.where(finite, m, torch.zeros_like(m))
        p = torch.exp(s - m_safe.view(-1, 1))          # exp(-inf) = 0 for excluded keys
        l = p.sum(dim=1)
        if use_sink:
            l = l + torch.exp(float(sink) - m_safe)
        num = p @ v if skv > 0 else torch.zeros(r.numel(), dv, dtype=torch.float64)
        o = torch.where((l > 0).view(-1, 1), num / torch.where(l > 0, l, torch.ones_like(l)).view(-1, 1),
                        torch.zeros_like(num))
        outs.append(o)
        ms.append(m)
        ls.append(l)
    if not outs:
        return (torch.zeros(0, dv, dtype=torch.float64), torch.zeros(0, dtype=torch.float64),
                torch.zeros(0, dtype=torch.float64))
    return torch.cat(outs), torch.cat(ms), torch.cat(ls)


# ---------------------------------------------------------------------------
# Layouts (aclnnFlashAttentionScore page, parameter inputLayout: BSH, SBH,
# BSND, BNSD with D = H / N; V5 page: TND).  Dense layouts are brought to a
# canonical [B, N, S, D] view by a permutation or a reshape only.
# ---------------------------------------------------------------------------

def to_bnsd(x: torch.Tensor, layout: str, heads: int) -> torch.Tensor:
    if layout == "BNSD":
        return x
    if layout == "BSND":
        return x.permute(0, 2, 1, 3)
    if layout == "BSH":
        b, s, h = x.shape
        return x.reshape(b, s, heads, h // heads).permute(0, 2, 1, 3)
    if layout == "SBH":
        s, b, h = x.shape
        return x.reshape(s, b, heads, h // heads).permute(1, 2, 0, 3)
    raise ValueError(f"not a dense layout: {layout}")


def from_bnsd(x: torch.Tensor, layout: str) -> torch.Tensor:
    if layout == "BNSD":
        return x.contiguous()
    if layout == "BSND":
        return x.permute(0, 2, 1, 3).contiguous()
    if layout == "BSH":
        b, n, s, d = x.shape
        return x.permute(0, 2, 1, 3).reshape(b, s, n * d).contiguous()
    if layout == "SBH":
        b, n, s, d = x.shape
        return x.permute(2, 0, 1, 3).reshape(s, b, n * d).contiguous()
    raise ValueError(f"not a dense layout: {layout}")


def _mask_slice(mask: Optional[torch.Tensor], b: int, h: int) -> Optional[torch.Tensor]:
    """[Sq,Skv] slice of a mask shaped [B,N,Sq,Skv], [B,1,..], [1,1,..] or [Sq,Skv]."""
    if mask is None:
        return None
    if mask.dim() == 2:
        return mask
    bb = b if mask.shape[0] > 1 else 0
    hh = h if mask.shape[1] > 1 else 0
    return mask[bb, hh]


def attention_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, layout: str,
                      scale: float, heads: Optional[int] = None, kv_heads: Optional[int] = None,
                      q_rope: Optional[torch.Tensor] = None, k_rope: Optional[torch.Tensor] = None,
                      atten_mask: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
                      causal: bool = False, pre_tokens: Optional[int] = None,
                      next_tokens: Optional[int] = None,
                      cu_seqlens_q: Optional[Sequence[int] | torch.Tensor] = None,
                      cu_seqlens_kv: Optional[Sequence[int] | torch.Tensor] = None,
                      samples: Optional[Sequence[Tuple[int, int, torch.Tensor]]] = None,
                      pse: Optional[torch.Tensor] = None, q_start: int = 0, kv_start: int = 0):
    """Whole-problem oracle in the caller's layout.

    Dense layouts return ``(O, m, l)`` with O in the input layout (last dim Dv)
    and m, l shaped [B, N, Sq].  TND returns O [T, N, Dv] and m, l shaped
    [N, T] (one value per query row; the ABI's trailing 8 copies are checked
    separately).  With ``samples`` = [(b, h, rows), ...] only those rows are
    evaluated and a list of (O [R,Dv], m [R], l [R]) is returned instead; for
    TND, ``b`` is the sequence index and ``rows`` are local to it.
    """
    if layout == "TND":
        return _forward_tnd(q, k, v, scale=scale, q_rope=q_rope, k_rope=k_rope, atten_mask=atten_mask,
                            sink=sink, causal=causal, pre_tokens=pre_tokens, next_tokens=next_tokens,
                            cu_q=cu_seqlens_q, cu_kv=cu_seqlens_kv, samples=samples, pse=pse,
                            q_start=q_start, kv_start=kv_start)
    if layout in ("BSH", "SBH"):
        if heads is None:
            raise ValueError("BSH/SBH need the query head count")
        kv_heads = heads if kv_heads is None else kv_heads
    else:
        heads = q.shape[1] if layout == "BNSD" else q.shape[2]
        kv_heads = k.shape[1] if layout == "BNSD" else k.shape[2]
    qc, kc, vc = to_bnsd(q, layout, heads), to_bnsd(k, layout, kv_heads), to_bnsd(v, layout, kv_heads)
    qrc = to_bnsd(q_rope, layout, heads) if q_rope is not None else None
    krc = to_bnsd(k_rope, layout, kv_heads) if k_rope is not None else None
    B, N, Sq, _ = qc.shape
    Nkv = kc.shape[1]
    if N % Nkv:
        raise ValueError("Nq must be a multiple of Nkv")
    group = N // Nkv

    def one(b, h, rows=None):
        g = h // group
        return head_attention(qc[b, h], kc[b, g], vc[b, g], scale=scale,
                              q_rope=qrc[b, h] if qrc is not None else None,
                              k_rope=krc[b, g] if krc is not None else None,
                              mask=_mask_slice(atten_mask, b, h), causal=causal,
                              pre_tokens=pre_tokens, next_tokens=next_tokens,
                              sink=float(sink[h]) if sink is not None else None, rows=rows,
                              pse=pse[b if pse.shape[0] > 1 else 0, h] if pse is not None else None,
                              q_start=q_start, kv_start=kv_start)

    if samples is not None:
        return [one(b, h, torch.as_tensor(rows)) for (b, h, rows) in samples]
    Dv = vc.shape[3]
    O = torch.zeros(B, N, Sq, Dv, dtype=torch.float64)
    M = torch.zeros(B, N, Sq, dtype=torch.float64)
    L = torch.zeros(B, N, Sq, dtype=torch.float64)
    for b in range(B):
        for h in range(N):
            O[b, h], M[b, h], L[b, h] = one(b, h)
    return from_bnsd(O, layout), M, L


def _tnd_mask(atten_mask: torch.Tensor, lq: int, lk: int) -> torch.Tensor:
    """The 2-D TND mask as seen by one sequence of lq rows and lk keys.

    Sequence-local position (i, j) reads atten_mask[i, j]; where the sequence
    is longer than the mask in either direction, the positions outside it are
    excluded (the reading of the V5 parameter table, row attenMaskOptional,
    for a [S1, S2] mask smaller than a sequence).
    """
    out = torch.ones(lq, lk, dtype=atten_mask.dtype)
    r, c = min(lq, atten_mask.shape[0]), min(lk, atten_mask.shape[1])
    out[:r, :c] = atten_mask[:r, :c]
    return out


def _as_list(cu) -> list:
    return [int(x) for x in (cu.tolist() if isinstance(cu, torch.Tensor) else cu)]


def _forward_tnd(q, k, v, *, scale, q_rope, k_rope, atten_mask, sink, causal, pre_tokens,
                 next_tokens, cu_q, cu_kv, samples, pse=None, q_start=0, kv_start=0):
    if atten_mask is not None and atten_mask.dim() != 2:
        raise NotImplementedError("with TND only a 2-D [Sq, Skv] mask in sequence-local coordinates")
    cq, ck = _as_list(cu_q), _as_list(cu_kv)
    if len(cq) != len(ck):
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    T, N, _ = q.shape
    Nkv = k.shape[1]
    group = N // Nkv
    # start of each sequence's [N, Sq_i, Skv_i] block in the flat pse
    pse_off = [0]
    for bi in range(len(cq) - 1):
        pse_off.append(pse_off[-1] + N * (cq[bi + 1] - cq[bi]) * (ck[bi + 1] - ck[bi]))
    if pse is not None and pse.numel() != pse_off[-1]:
        raise ValueError(f"TND pse must hold {pse_off[-1]} values, got {pse.numel()}")

    def pse_block(bi, h):
        if pse is None:
            return None
        lq, lk = cq[bi + 1] - cq[bi], ck[bi + 1] - ck[bi]
        return pse.reshape(-1)[pse_off[bi]:pse_off[bi + 1]].view(N, lq, lk)[h]

    def one(bi, h, rows=None):
        q0, q1, k0, k1 = cq[bi], cq[bi + 1], ck[bi], ck[bi + 1]
        g = h // group
        return head_attention(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], scale=scale,
                              q_rope=q_rope[q0:q1, h] if q_rope is not None else None,
                              k_rope=k_rope[k0:k1, g] if k_rope is not None else None,
                              mask=_tnd_mask(atten_mask, q1 - q0, k1 - k0) if atten_mask is not None else None,
                              causal=causal, pre_tokens=pre_tokens, next_tokens=next_tokens,
                              sink=float(sink[h]) if sink is not None else None, rows=rows,
                              pse=pse_block(bi, h), q_start=q_start, kv_start=kv_start)

    if samples is not None:
        return [one(bi, h, torch.as_tensor(rows)) for (bi, h, rows) in samples]
    Dv = v.shape[2]
    O = torch.zeros(T, N, Dv, dtype=torch.float64)
    M = torch.full((N, T), NEG_INF, dtype=torch.float64)
    L = torch.zeros(N, T, dtype=torch.float64)
    for bi in range(len(cq) - 1):
        q0, q1 = cq[bi], cq[bi + 1]
        if q1 <= q0:
            continue
        for h in range(N):
            O[q0:q1, h], M[h, q0:q1], L[h, q0:q1] = one(bi, h)
    return O, M, L


def expand_stats(x: torch.Tensor, layout: str, softmax_out_layout: str = "") -> torch.Tensor:
    """Lay per-row statistics out as the ABI writes them: 8 equal trailing slots.

    Dense: [B, N, Sq] -> [B, N, Sq, 8].  TND: [N, T] -> [N, T, 8] for the
    empty layout string, [T, N, 8] for "same_as_input" (V5 parameter table,
    row softmaxOutLayout).
    """
    if layout == "TND" and softmax_out_layout == "same_as_input":
        x = x.transpose(0, 1)
    return x.unsqueeze(-1).expand(*x.shape, 8).contiguous()


def merge_partials(parts: Sequence[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]]
                   ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Combine the results of one query chunk against several key chunks.

    Each part is (O_c [..., Dv], m_c [...], l_c [...]) for the same rows, with
    m_c and l_c the row's max logit and sum of e^(s - m_c) over that chunk's
    keys (so O_c = sum e^(s - m_c) v / l_c).  Over the union of the chunks the
    max is m = max_c m_c and, from the definitions of m and l in the sink
    equations, l = sum_c e^(m_c - m) l_c and O = sum_c e^(m_c - m) l_c O_c / l.
    Chunks with no kept key (m_c = -inf, l_c = 0) contribute nothing; a row
    empty in every chunk gets O = 0, m = -inf, l = 0.
    """
    Os = [p[0].to(torch.float64) for p in parts]
    ms = torch.stack([p[1].to(torch.float64) for p in parts])
    ls = torch.stack([p[2].to(torch.float64) for p in parts])
    m = ms.amax(dim=0)
    m_safe = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    w = torch.where(torch.isfinite(ms), torch.exp(ms - m_safe) * ls, torch.zeros_like(ls))
    l = w.sum(dim=0)
    num = sum(w[c].unsqueeze(-1) * Os[c] for c in range(len(Os)))
    o = torch.where((l > 0).unsqueeze(-1), num / torch.where(l > 0, l, torch.ones_like(l)).unsqueeze(-1),
                    torch.zeros_like(num))
    return o, m, l

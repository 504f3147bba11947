"""Scalar brute force of the attention forward, used only to pin the oracle.

Written independently of ``oracle/attention.py``: pure Python loops over
nested lists, ``math.exp`` and ``math.fsum`` (exactly rounded sums), no torch
arithmetic.  It evaluates the aclnnFlashAttentionVarLenScoreV5 page's
attention equation with its sink equations (功能说明 → 计算公式) entry by entry,
for tiny shapes only.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

NEG_INF = float("-inf")


def _kept(i: int, j: int, mask, causal: bool, pre: Optional[int], nxt: Optional[int]) -> bool:
    if mask is not None and mask[i][j]:
        return False
    if causal and j > i:
        return False
    if mask is not None or causal:
        if pre is not None and i - j > pre:
            return False
        if nxt is not None and j - i > nxt:
            return False
    return True


def head(q: Sequence[Sequence[float]], k, v, scale: float, *, qr=None, kr=None, mask=None,
         causal=False, pre=None, nxt=None, sink: Optional[float] = None, pse=None):
    """One (sequence, head): lists q [Sq][D], k [Skv][D], v [Skv][Dv]; optional pse [Sq][Skv]
    added to the scaled logits.  Returns (O, m, l) lists."""
    sq, skv = len(q), len(k)
    dv = len(v[0]) if skv else 0
    O: List[List[float]] = []
    M: List[float] = []
    L: List[float] = []
    for i in range(sq):
        logits = []
        for j in range(skv):
            if not _kept(i, j, mask, causal, pre, nxt):
                continue
            terms = [q[i][d] * k[j][d] for d in range(len(q[i]))]
            if qr is not None:
                terms += [qr[i][d] * kr[j][d] for d in range(len(qr[i]))]
            x = scale * math.fsum(terms)
            if pse is not None:
                x = x + pse[i][j]
            logits.append((x, j))
        cands = [x for x, _ in logits]
        has_sink = sink is not None and sink != NEG_INF
        if has_sink:
            cands.append(sink)
        if not cands:
            O.append([0.0] * dv)
            M.append(NEG_INF)
            L.append(0.0)
            continue
        m = max(cands)
        w = [(math.exp(x - m), j) for x, j in logits]
        parts = [x for x, _ in w] + ([math.exp(sink - m)] if has_sink else [])
        l = math.fsum(parts)
        O.append([math.fsum(wj * v[j][d] for wj, j in w) / l for d in range(dv)])
        M.append(m)
        L.append(l)
    return O, M, L

"""Seeded synthetic inputs for the FlashAttention forward workloads.

This module is shared by the CPU oracle side and the HIP side of the tests and
the benchmark.  It holds only random-number draws and input *structure*
(shapes, sequence-length mixes, mask patterns); none of the attention
arithmetic lives here, so neither side borrows the other's computation.

Recipe (all workloads):
  * ``g = torch.Generator("cpu").manual_seed(seed)``;
  * tensors are drawn in the order Q, K, V, Qrope, Krope, sink as
    ``torch.randn(shape, generator=g, dtype=float32)`` and then rounded once to
    the working dtype; the rounded values are what both sides see;
  * the varlen length mix draws ``u = 64 + 960*rand(n, float64)``, rescales it
    to sum to ``T``, floors, and hands the remainder out one by one to the
    largest fractional parts (ties by lower index).

The shapes follow the workloads the pages illustrate: the dense example of the
MindIE-SD ``attention_forward`` page (B=2, S=4096, N=24, D=128, BSND), its
varlen example (T=8192, N=24, D=128), and the sink + rope example of the
``aclnnFlashAttentionVarLenScoreV5`` page (TND, D=128 plus 64 rope dims,
per-head fp32 sink).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import torch

DTYPES = {
    "fp32": torch.float32,
    "fp16": torch.float16,
    "bf16": torch.bfloat16,
}

UNBOUNDED = 2**31 - 1  # "no limit" value for preTokens / nextTokens


@dataclasses.dataclass
class Case:
    """One attention problem, as CPU tensors plus the scalar attributes."""

    name: str
    layout: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float
    q_rope: Optional[torch.Tensor] = None
    k_rope: Optional[torch.Tensor] = None
    atten_mask: Optional[torch.Tensor] = None
    sink: Optional[torch.Tensor] = None
    causal: bool = False
    pre_tokens: int = UNBOUNDED
    next_tokens: int = UNBOUNDED
    cu_seqlens_q: Optional[torch.Tensor] = None
    cu_seqlens_kv: Optional[torch.Tensor] = None
    softmax_out_layout: str = ""
    pse: Optional[torch.Tensor] = None

    def tensors(self) -> Dict[str, Optional[torch.Tensor]]:
        return {
            "q": self.q, "k": self.k, "v": self.v, "q_rope": self.q_rope,
            "k_rope": self.k_rope, "atten_mask": self.atten_mask, "sink": self.sink,
            "cu_seqlens_q": self.cu_seqlens_q, "cu_seqlens_kv": self.cu_seqlens_kv, "pse": self.pse,
        }


def generator(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(int(seed))


def normal(shape: Sequence[int], g: torch.Generator, dtype: str | torch.dtype) -> torch.Tensor:
    """iid N(0,1) drawn in float32, then rounded once to ``dtype``."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(dt)


def uniform_lengths(n: int, total: int, g: torch.Generator, lo: float = 64.0, hi: float = 1024.0) -> List[int]:
    """Integer lengths drawn uniform in [lo, hi] and rescaled to sum exactly to ``total``."""
    u = lo + (hi - lo) * torch.rand(n, generator=g, dtype=torch.float64)
    x = u * (total / float(u.sum()))
    base = torch.floor(x).to(torch.int64)
    rem = int(total - int(base.sum()))
    frac = (x - base.to(torch.float64)).tolist()
    order = sorted(range(n), key=lambda i: (-frac[i], i))
    out = base.tolist()
    for i in order[:rem]:
        out[i] += 1
    return [int(v) for v in out]


def cu_from_lengths(lengths: Sequence[int]) -> torch.Tensor:
    """Cumulative lengths with a leading 0, int32 (the MindIE-SD ``cu_seqlens`` form)."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def lower_triangular_mask(sq: int, skv: int) -> torch.Tensor:
    """uint8 [sq, skv] with 1 (= excluded) strictly above the diagonal."""
    return torch.triu(torch.ones(sq, skv, dtype=torch.uint8), diagonal=1)


def _shape(layout: str, b: int, n: int, s: int, d: int, t: int = 0) -> tuple:
    if layout == "BNSD":
        return (b, n, s, d)
    if layout == "BSND":
        return (b, s, n, d)
    if layout == "BSH":
        return (b, s, n * d)
    if layout == "SBH":
        return (s, b, n * d)
    if layout == "TND":
        return (t, n, d)
    raise ValueError(layout)


def dense_case(name: str, layout: str, b: int, nq: int, sq: int, d: int, dtype: str, seed: int, *,
               skv: Optional[int] = None, nkv: Optional[int] = None, dv: Optional[int] = None,
               drope: int = 0, sink: bool = False, causal: bool = False, mask: bool = False,
               pre_tokens: int = UNBOUNDED, next_tokens: int = UNBOUNDED,
               scale: Optional[float] = None, pse: Optional[str] = None) -> Case:
    """A dense (BNSD / BSND / BSH / SBH) problem with seeded iid N(0,1) tensors.

    ``pse``: None, "full" ([B, N, Sq, Skv]) or "bcast" ([1, N, Sq, Skv]); drawn
    after every other tensor, in the working dtype."""
    skv = sq if skv is None else skv
    nkv = nq if nkv is None else nkv
    dv = d if dv is None else dv
    g = generator(seed)
    q = normal(_shape(layout, b, nq, sq, d), g, dtype)
    k = normal(_shape(layout, b, nkv, skv, d), g, dtype)
    v = normal(_shape(layout, b, nkv, skv, dv), g, dtype)
    rope_dt = dtype if dtype != "fp32" else "bf16"
    qr = normal(_shape(layout, b, nq, sq, drope), g, rope_dt) if drope else None
    kr = normal(_shape(layout, b, nkv, skv, drope), g, rope_dt) if drope else None
    sk = normal((nq,), g, torch.float32) if sink else None
    am = lower_triangular_mask(sq, skv) if mask else None
    ps = normal((b if pse == "full" else 1, nq, sq, skv), g, dtype) if pse else None
    return Case(name=name, layout=layout, q=q, k=k, v=v, q_rope=qr, k_rope=kr,
                scale=(d ** -0.5) if scale is None else scale, atten_mask=am, sink=sk,
                causal=causal, pre_tokens=pre_tokens, next_tokens=next_tokens, pse=ps)


def varlen_case(name: str, lengths_q: Sequence[int], nq: int, d: int, dtype: str, seed: int, *,
                lengths_kv: Optional[Sequence[int]] = None, nkv: Optional[int] = None,
                dv: Optional[int] = None, drope: int = 0, sink: bool = False, causal: bool = False,
                pre_tokens: int = UNBOUNDED, next_tokens: int = UNBOUNDED,
                scale: Optional[float] = None, softmax_out_layout: str = "", pse: bool = False) -> Case:
    """A TND problem: sequences packed along T, described by int32 cumulative lengths.

    ``pse``: draw a flat bias holding an [N, Sq_i, Skv_i] block per sequence."""
    lengths_kv = list(lengths_q) if lengths_kv is None else list(lengths_kv)
    nkv = nq if nkv is None else nkv
    dv = d if dv is None else dv
    tq, tkv = int(sum(lengths_q)), int(sum(lengths_kv))
    g = generator(seed)
    q = normal((tq, nq, d), g, dtype)
    k = normal((tkv, nkv, d), g, dtype)
    v = normal((tkv, nkv, dv), g, dtype)
    rope_dt = dtype if dtype != "fp32" else "bf16"
    qr = normal((tq, nq, drope), g, rope_dt) if drope else None
    kr = normal((tkv, nkv, drope), g, rope_dt) if drope else None
    sk = normal((nq,), g, torch.float32) if sink else None
    npse = sum(nq * a * b for a, b in zip(lengths_q, lengths_kv))
    ps = normal((npse,), g, dtype) if pse else None
    return Case(name=name, layout="TND", q=q, k=k, v=v, q_rope=qr, k_rope=kr,
                scale=(d ** -0.5) if scale is None else scale, sink=sk, causal=causal,
                pre_tokens=pre_tokens, next_tokens=next_tokens,
                cu_seqlens_q=cu_from_lengths(lengths_q), cu_seqlens_kv=cu_from_lengths(lengths_kv),
                softmax_out_layout=softmax_out_layout, pse=ps)


# ---------------------------------------------------------------------------
# The five named workloads.  ``small=True`` shrinks the long ones so the CPU
# oracle finishes in seconds while keeping their structure (several tiles and
# a ragged tail where the full size has one).
# ---------------------------------------------------------------------------

WORKLOADS = ("c1_fp32_bnsd", "c2_dense_bsnd", "c3_causal", "c3_band", "c4_varlen_causal",
             "c5_varlen_sink_rope", "c6_dense_pse", "c7_outer_split", "c2_gqa_nkv4", "c2_mqa",
             "d256_dense_bsnd")

# The c7 workload runs the c2 problem as an outer split: its keys in these
# chunks, one forward call per chunk (with its kv start), then the merge.
C7_CUTS = (0, 2048, 4096)


def c4_lengths(seed: int = 4, n: int = 16, total: int = 8192) -> List[int]:
    return uniform_lengths(n, total, generator(seed))


def workload(name: str, dtype: str = "bf16", small: bool = False) -> Case:
    if name == "c1_fp32_bnsd":
        return dense_case(name, "BNSD", 1, 2, 128, 64, "fp32", seed=1)
    if name == "c2_dense_bsnd":
        s = 4096 if not small else 320
        return dense_case(name, "BSND", 2, 24 if not small else 3, s, 128, dtype, seed=2)
    if name in ("c3_causal", "c3_band"):
        b, n, s = (4, 32, 8192) if not small else (1, 2, 400)
        pre = UNBOUNDED if name == "c3_causal" else (2048 if not small else 130)
        return dense_case(name, "BNSD", b, n, s, 128, "bf16", seed=3, mask=True,
                          pre_tokens=pre, next_tokens=0)
    if name == "c4_varlen_causal":
        if small:
            lens = uniform_lengths(5, 700, generator(4))
            return varlen_case(name, lens, 3, 128, "bf16", seed=4, causal=True)
        return varlen_case(name, c4_lengths(), 24, 128, "bf16", seed=4, causal=True)
    if name == "c5_varlen_sink_rope":
        if small:
            return varlen_case(name, [200, 0, 77, 160], 4, 128, "bf16", seed=5, drope=64,
                               sink=True, causal=True, scale=128 ** -0.5)
        return varlen_case(name, [2048] * 8, 64, 128, "bf16", seed=5, drope=64, sink=True,
                           causal=True, scale=128 ** -0.5)
    if name == "c7_outer_split":
        s = 4096 if not small else 320
        return dense_case(name, "BSND", 2, 24 if not small else 3, s, 128, "bf16", seed=2)
    if name in ("c2_gqa_nkv4", "c2_mqa"):
        # the headline shape with grouped key / value heads: 24 query heads over 4 or 1 kv heads
        s = 4096 if not small else 320
        n = 24 if not small else 4
        return dense_case(name, "BSND", 2, n, s, 128, dtype, seed=8, nkv=(4 if name == "c2_gqa_nkv4" else 1)
                          if not small else (2 if name == "c2_gqa_nkv4" else 1))
    if name == "d256_dense_bsnd":
        # head dim 256 at the headline's FLOP count: B2 S4096 N12
        s = 4096 if not small else 320
        return dense_case(name, "BSND", 2, 12 if not small else 2, s, 256, dtype, seed=9)
    if name == "c6_dense_pse":
        # the additive bias term: a full [B, N, S, S] pse makes the pass HBM-bound
        s = 4096 if not small else 300
        return dense_case(name, "BNSD", 1, 8 if not small else 2, s, 128, "bf16", seed=6, pse="full")
    raise KeyError(name)

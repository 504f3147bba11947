"""Python entry points over the C ABI.

``attention_forward`` and ``attention_forward_varlen`` take the argument
shapes of the MindIE-SD pages (attention_forward: 4-D [B,S,N,D] or [B,N,S,D];
attention_forward_varlen: [T,N,D] with int32 ``cu_seqlens`` of B+1 entries),
plus the Ascend operator's extra inputs (sink, rope parts, mask, window).
They allocate the outputs with torch (device memory only), run phase 1 and
phase 2 of ``libfa_fwd.so`` on torch's current stream, and return the output.
All arithmetic happens in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

UNBOUNDED = 2**31 - 1


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_device(*ts: Optional[torch.Tensor]) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


class ForwardPlan:
    """A planned forward: the library plan, its workspace and its outputs.

    ``run()`` enqueues phase 2 on the current stream (or ``stream``) and may be
    called repeatedly; the plan keeps references to every tensor it reads or
    writes so their memory stays valid.
    """

    def __init__(self, query, key, value, *, layout: str, scale: float, head_num: int,
                 query_rope=None, key_rope=None, atten_mask=None, sink=None, cu_seqlens_q=None,
                 cu_seqlens_kv=None, causal: bool = False, pre_tokens: int = UNBOUNDED,
                 next_tokens: int = UNBOUNDED, softmax_out_layout: str = "", out=None,
                 softmax_max=None, softmax_sum=None, inner_precise: int = 0, real_shift=None,
                 q_start_idx: Optional[int] = None, kv_start_idx: Optional[int] = None):
        self.device = _check_device(query, key, value, query_rope, key_rope, atten_mask, sink, cu_seqlens_q,
                                    cu_seqlens_kv, out, softmax_max, softmax_sum, real_shift)
        self._keep = (query, key, value, query_rope, key_rope, atten_mask, sink, cu_seqlens_q, cu_seqlens_kv,
                      real_shift)
        self.out, self.softmax_max, self.softmax_sum = out, softmax_max, softmax_sum
        self.plan = None
        ws, plan = _lib.fa_fwd_get_workspace_size(
            query, query_rope, key, key_rope, value, real_shift, atten_mask, sink, cu_seqlens_q, cu_seqlens_kv,
            q_start_idx, kv_start_idx, scale, 1.0, pre_tokens, next_tokens, head_num, layout, inner_precise, 0, causal,
            softmax_out_layout, softmax_max, softmax_sum, out)
        self.plan = plan
        self.workspace_size = ws
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device) if ws > 0 else None

    def describe(self) -> str:
        return _lib.fa_plan_describe(self.plan)

    def run(self, stream: Optional[int] = None) -> None:
        if stream is None:
            stream = _stream_handle(self.device)
        _lib.fa_fwd(self.workspace, self.workspace_size, self.plan, stream)

    def close(self) -> None:
        if self.plan is not None:
            _lib.fa_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dense_dims(t: torch.Tensor, layout: str, heads: Optional[int]) -> Tuple[int, int, int, int]:
    """(B, S, N, D) of a dense-layout tensor."""
    if layout == "BNSD":
        b, n, s, d = t.shape
    elif layout == "BSND":
        b, s, n, d = t.shape
    elif layout in ("BSH", "SBH"):
        if heads is None:
            raise ValueError(f"{layout} needs the head count")
        if layout == "BSH":
            b, s, h = t.shape
        else:
            s, b, h = t.shape
        n, d = heads, h // heads
    else:
        raise ValueError(f"unknown layout {layout}")
    return b, s, n, d


def _out_like(query: torch.Tensor, layout: str, dv: int, heads: int) -> torch.Tensor:
    shp = list(query.shape)
    shp[-1] = heads * dv if layout in ("BSH", "SBH") else dv
    return torch.empty(shp, dtype=query.dtype, device=query.device)


def attention_forward(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                      attn_mask: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                      head_first: bool = False, *, layout: Optional[str] = None, heads: Optional[int] = None,
                      kv_heads: Optional[int] = None, pre_tokens: int = UNBOUNDED, next_tokens: int = UNBOUNDED,
                      sink: Optional[torch.Tensor] = None, query_rope: Optional[torch.Tensor] = None,
                      key_rope: Optional[torch.Tensor] = None, causal: bool = False,
                      pse: Optional[torch.Tensor] = None, q_start_idx: Optional[int] = None,
                      kv_start_idx: Optional[int] = None,
                      return_softmax_stats: bool = False, return_plan: bool = False):
    """Dense attention forward.

    ``layout`` defaults to "BNSD" when ``head_first`` else "BSND"; "BSH" and
    "SBH" need ``heads``.  ``attn_mask``: u8/bool, nonzero = excluded.
    ``pse``: optional additive bias [B|1, N, Sq, Skv] in the query's dtype,
    added after the scale (the realShift input).  ``q_start_idx`` /
    ``kv_start_idx``: where these query / key rows start in the whole sequence
    (outer split); causal and window tests then use global positions.
    ``scale`` defaults to D**-0.5 with D the non-rope head dim.  Returns the
    output, plus (softmax_max, softmax_sum) shaped [B,N,Sq,8] when
    ``return_softmax_stats``.
    """
    layout = layout or ("BNSD" if head_first else "BSND")
    b, s, n, d = _dense_dims(query, layout, heads)
    if layout in ("BSH", "SBH"):
        nk = kv_heads if kv_heads is not None else key.shape[-1] // d
        dv = value.shape[-1] // nk
    else:
        dv = value.shape[-1]
    if scale is None:
        scale = d ** -0.5
    out = _out_like(query, layout, dv, n)
    smax = ssum = None
    if return_softmax_stats:
        smax = torch.empty(b, n, s, 8, dtype=torch.float32, device=query.device)
        ssum = torch.empty_like(smax)
    plan = ForwardPlan(query, key, value, layout=layout, scale=scale, head_num=n, query_rope=query_rope,
                       key_rope=key_rope, atten_mask=attn_mask, sink=sink, causal=causal, pre_tokens=pre_tokens,
                       next_tokens=next_tokens, out=out, softmax_max=smax, softmax_sum=ssum, real_shift=pse,
                       q_start_idx=q_start_idx, kv_start_idx=kv_start_idx)
    plan.run()
    if return_plan:
        return plan
    plan.close()
    if return_softmax_stats:
        return out, smax, ssum
    return out


def attention_forward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                             cu_seqlens_k: torch.Tensor, max_seqlen_q=None, max_seqlen_k=None, dropout_p: float = 0.0,
                             softmax_scale: Optional[float] = None, causal: bool = False, window_size=None,
                             softcap=None, alibi_slopes=None, deterministic=None, return_attn_probs=None,
                             block_table=None, *, sink: Optional[torch.Tensor] = None,
                             q_rope: Optional[torch.Tensor] = None, k_rope: Optional[torch.Tensor] = None,
                             atten_mask: Optional[torch.Tensor] = None, pre_tokens: int = UNBOUNDED,
                             next_tokens: int = UNBOUNDED, softmax_out_layout: str = "",
                             pse: Optional[torch.Tensor] = None, q_start_idx: Optional[int] = None,
                             kv_start_idx: Optional[int] = None,
                             return_softmax_stats: bool = False, return_plan: bool = False):
    """Varlen (TND) attention forward over sequences packed along T.

    ``pse``: optional additive bias, one flat tensor holding an
    [N, Sq_i, Skv_i] block per sequence, in sequence order.

    ``cu_seqlens_*``: int32 [B+1] on the GPU, leading 0.  ``max_seqlen_*`` and
    ``deterministic`` are accepted and unused (the kernel never needs them;
    results are always bitwise repeatable).  ``window_size``, ``softcap``,
    ``alibi_slopes``, ``return_attn_probs`` and ``block_table`` must be left
    unset; ``dropout_p`` must be 0.
    """
    for name, val in (("window_size", window_size), ("softcap", softcap), ("alibi_slopes", alibi_slopes),
                      ("return_attn_probs", return_attn_probs), ("block_table", block_table)):
        if val not in (None, False):
            raise NotImplementedError(f"{name} is not supported")
    if dropout_p != 0.0:
        raise NotImplementedError("dropout_p must be 0.0")
    t, n, d = q.shape
    dv = v.shape[-1]
    scale = d ** -0.5 if softmax_scale is None else softmax_scale
    out = torch.empty(t, n, dv, dtype=q.dtype, device=q.device)
    smax = ssum = None
    if return_softmax_stats:
        shp = (t, n, 8) if softmax_out_layout == "same_as_input" else (n, t, 8)
        smax = torch.empty(shp, dtype=torch.float32, device=q.device)
        ssum = torch.empty_like(smax)
    plan = ForwardPlan(q, k, v, layout="TND", scale=scale, head_num=n, query_rope=q_rope, key_rope=k_rope,
                       atten_mask=atten_mask, sink=sink, cu_seqlens_q=cu_seqlens_q, cu_seqlens_kv=cu_seqlens_k,
                       causal=causal, pre_tokens=pre_tokens, next_tokens=next_tokens,
                       softmax_out_layout=softmax_out_layout, out=out, softmax_max=smax, softmax_sum=ssum,
                       real_shift=pse, q_start_idx=q_start_idx, kv_start_idx=kv_start_idx)
    plan.run()
    if return_plan:
        return plan
    plan.close()
    if return_softmax_stats:
        return out, smax, ssum
    return out


def merge_partials(parts, *, layout: str, heads: int, softmax_out_layout: str = ""):
    """Merge [(out, softmax_max, softmax_sum), ...] of one query chunk over several key
    chunks into (out, softmax_max, softmax_sum) over all keys (``fa_fwd_merge``)."""
    o0, m0, _ = parts[0]
    out = torch.empty_like(o0)
    smax = torch.empty_like(m0)
    ssum = torch.empty_like(m0)
    _lib.fa_fwd_merge([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts], layout, heads,
                      softmax_out_layout, out, smax, ssum, _stream_handle(out.device))
    return out, smax, ssum


def cu_from_actual_seq_len(actual) -> list:
    """The V5 page's cumulative lengths without a leading 0 -> the cu_seqlens form with one."""
    vals = [int(x) for x in actual]
    return [0] + vals

"""Helpers for comparing the HIP forward with the CPU oracle on one Case.

Tolerances (written here, used by every parity test):
  * fp32 inputs: max |O_gpu - O_ref| <= 1e-5; |m| and |log l| within 1e-5.
  * fp16 / bf16 inputs: |O_gpu - O_ref| <= 1e-2 + half an ulp of the output
    dtype at |O_ref|: the output is rounded to that dtype, which alone costs
    up to half an ulp (0.0078 for |O| in [2, 4) in bf16), on top of the
    kernel's own error (P is rounded to the input dtype before the P V
    product).  Each comparison also counts the elements above 1e-2 and the
    smallest |O_ref| among them (reported as "over1e-2" and "over_min_abs").
    |m| and |log l| within 1e-3.
  * Rows with no kept key: O exactly 0, m exactly -inf (or the sink), l
    exactly 0 (or 1).
  * All 8 trailing statistics slots hold the same value.
"""
from __future__ import annotations

import contextlib
import math
import os
import time
from typing import Dict, Optional

import torch

import synth
from attention_forward_fa_amd import api
from oracle import attention as orc


@contextlib.contextmanager
def forced_kernel(kind: str):
    """Force the library's kernel family (FA_FWD_KERNEL) for the calls inside; 'auto' = the plan's choice."""
    old = os.environ.get("FA_FWD_KERNEL")
    if kind == "auto":
        os.environ.pop("FA_FWD_KERNEL", None)
    else:
        os.environ["FA_FWD_KERNEL"] = kind
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("FA_FWD_KERNEL", None)
        else:
            os.environ["FA_FWD_KERNEL"] = old


# Stream watchdog: the GPU work a test enqueues must finish within this many
# seconds, else the test fails with a TimeoutError naming what it waited for
# (instead of blocking the whole run inside a synchronize).
GPU_DEADLINE_S = float(os.environ.get("FA_TEST_GPU_DEADLINE_S", "120"))


def sync_with_deadline(what: str = "GPU work", seconds: Optional[float] = None) -> None:
    """Wait for everything enqueued on the current stream, polling an event, up to a deadline."""
    limit = GPU_DEADLINE_S if seconds is None else seconds
    ev = torch.cuda.Event()
    ev.record()
    t0 = time.monotonic()
    while not ev.query():
        if time.monotonic() - t0 > limit:
            raise TimeoutError(f"{what} did not finish within {limit:.0f} s")
        time.sleep(0.0005)
    torch.cuda.synchronize()


def to_gpu(t: Optional[torch.Tensor], dev="cuda:0"):
    return None if t is None else t.to(dev)


def run_gpu_poisoned(case: synth.Case, dev="cuda:0"):
    """Run the library on the case with O and both statistics pre-filled with NaN,
    so that an element the kernels never write stays NaN; returns CPU tensors
    (O, softmax_max, softmax_sum)."""
    g = {k: to_gpu(v, dev) for k, v in case.tensors().items()}
    q = g["q"]
    out = torch.full(q.shape[:-1] + (case.v.shape[-1],), float("nan"), dtype=q.dtype, device=dev)
    if case.layout == "TND":
        T, N = q.shape[0], q.shape[1]
        shp = (T, N, 8) if case.softmax_out_layout == "same_as_input" else (N, T, 8)
        N_ = N
    else:
        B = q.shape[0]
        N_ = q.shape[1] if case.layout == "BNSD" else q.shape[2]
        S = q.shape[2] if case.layout == "BNSD" else q.shape[1]
        shp = (B, N_, S, 8)
    smax = torch.full(shp, float("nan"), dtype=torch.float32, device=dev)
    ssum = torch.full(shp, float("nan"), dtype=torch.float32, device=dev)
    plan = api.ForwardPlan(q, g["k"], g["v"], layout=case.layout, scale=case.scale, head_num=N_,
                           query_rope=g["q_rope"], key_rope=g["k_rope"], atten_mask=g["atten_mask"], sink=g["sink"],
                           cu_seqlens_q=g["cu_seqlens_q"], cu_seqlens_kv=g["cu_seqlens_kv"], causal=case.causal,
                           pre_tokens=case.pre_tokens, next_tokens=case.next_tokens,
                           softmax_out_layout=case.softmax_out_layout, out=out, softmax_max=smax, softmax_sum=ssum,
                           real_shift=g["pse"])
    try:
        plan.run()
        sync_with_deadline(f"forward on {case.layout} q={tuple(case.q.shape)}")
    finally:
        plan.close()
    return out.cpu(), smax.cpu(), ssum.cpu()


def run_gpu(case: synth.Case, *, stats: bool = True, layout_heads: Optional[int] = None, dev="cuda:0"):
    """Run the library on the case; returns CPU tensors (O, softmax_max, softmax_sum)."""
    g = {k: to_gpu(v, dev) for k, v in case.tensors().items()}
    if case.layout == "TND":
        res = api.attention_forward_varlen(
            g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_kv"], softmax_scale=case.scale,
            causal=case.causal, sink=g["sink"], q_rope=g["q_rope"], k_rope=g["k_rope"], atten_mask=g["atten_mask"],
            pre_tokens=case.pre_tokens, next_tokens=case.next_tokens, softmax_out_layout=case.softmax_out_layout,
            pse=g["pse"], return_softmax_stats=stats)
    else:
        res = api.attention_forward(
            g["q"], g["k"], g["v"], attn_mask=g["atten_mask"], scale=case.scale, layout=case.layout,
            heads=layout_heads, pre_tokens=case.pre_tokens, next_tokens=case.next_tokens, sink=g["sink"],
            query_rope=g["q_rope"], key_rope=g["k_rope"], causal=case.causal, pse=g["pse"],
            return_softmax_stats=stats)
    sync_with_deadline(f"forward on {case.layout} q={tuple(case.q.shape)}")
    if stats:
        return tuple(x.cpu() for x in res)
    return res.cpu(), None, None


def run_oracle(case: synth.Case, heads: Optional[int] = None):
    """Oracle (O, m, l) with m, l laid out like the ABI's stats minus the 8 slots."""
    O, M, L = orc.attention_forward(
        case.q, case.k, case.v, layout=case.layout, scale=case.scale, heads=heads, q_rope=case.q_rope,
        k_rope=case.k_rope, atten_mask=case.atten_mask, sink=case.sink, causal=case.causal,
        pre_tokens=case.pre_tokens, next_tokens=case.next_tokens, cu_seqlens_q=case.cu_seqlens_q,
        cu_seqlens_kv=case.cu_seqlens_kv, pse=case.pse)
    if case.layout == "TND" and case.softmax_out_layout == "same_as_input":
        M, L = M.transpose(0, 1), L.transpose(0, 1)
    return O, M, L


def ulp_half(ref: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """Half a unit in the last place of `dtype` at |ref| (normal range)."""
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    a = ref.abs().clamp_min(2.0**-14)
    return torch.exp2(torch.floor(torch.log2(a)) - mant) / 2


# elements above 1e-2 in the checks since the last reset (bf16 / fp16
# outputs), and the smallest |O_ref| among them
OVER_1E2 = [0, math.inf]


def check_output(o_gpu: torch.Tensor, o_ref: torch.Tensor, dtype: torch.dtype, what: str = "O") -> float:
    o_gpu = o_gpu.to(torch.float64)
    assert o_gpu.shape == o_ref.shape, f"{what}: shape {tuple(o_gpu.shape)} vs {tuple(o_ref.shape)}"
    assert torch.isfinite(o_gpu).all(), f"{what}: non-finite output"
    err = (o_gpu - o_ref).abs()
    if dtype == torch.float32:
        tol = torch.full_like(o_ref, 1e-5)
    else:
        tol = 1e-2 + ulp_half(o_ref, dtype)
        over = err > 1e-2
        if over.any():
            OVER_1E2[0] += int(over.sum())
            OVER_1E2[1] = min(OVER_1E2[1], float(o_ref.abs()[over].min()))
    bad = err > tol
    if bad.any():
        idx = tuple(int(i) for i in bad.nonzero()[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.numel()} outside tolerance; max err "
                             f"{float(err.max()):.3g}; first at {idx}: gpu {float(o_gpu[idx]):.6g} ref "
                             f"{float(o_ref[idx]):.6g}")
    return float(err.max()) if err.numel() else 0.0


def check_stats(s_gpu: torch.Tensor, ref: torch.Tensor, kind: str, dtype: torch.dtype) -> float:
    """s_gpu [..., 8] fp32 vs ref [...] fp64; kind 'max' compares m, 'sum' compares log l."""
    assert s_gpu.shape[-1] == 8 and tuple(s_gpu.shape[:-1]) == tuple(ref.shape), (s_gpu.shape, ref.shape)
    s0 = s_gpu[..., 0]
    assert bool((s_gpu == s0.unsqueeze(-1)).all() | (torch.isnan(s_gpu).all())), f"{kind}: 8 slots differ"
    s0 = s0.to(torch.float64)
    tol = 1e-5 if dtype == torch.float32 else 1e-3
    if kind == "max":
        inf = torch.isinf(ref)
        assert bool((s0[inf] == ref[inf]).all()), f"max: -inf rows differ"
        err = (s0[~inf] - ref[~inf]).abs()
    else:
        zero = ref == 0
        assert bool((s0[zero] == 0).all()), "sum: empty rows must be 0"
        assert bool((s0[~zero] > 0).all()), "sum: non-positive sum"
        err = (torch.log(s0[~zero]) - torch.log(ref[~zero])).abs()
    if err.numel() and float(err.max()) > tol:
        i = int(err.argmax())
        raise AssertionError(f"{kind}: max err {float(err.max()):.3g} > {tol} at flat index {i}")
    return float(err.max()) if err.numel() else 0.0


def compare_case(case: synth.Case, *, heads: Optional[int] = None) -> Dict[str, float]:
    """Full comparison of one case (GPU vs oracle); returns the max errors."""
    o, smax, ssum = run_gpu(case, layout_heads=heads)
    O, M, L = run_oracle(case, heads=heads)
    dt = case.q.dtype
    OVER_1E2[0], OVER_1E2[1] = 0, math.inf
    errs = {"O": check_output(o, O, dt), "m": check_stats(smax, M, "max", dt),
            "logl": check_stats(ssum, L, "sum", dt)}
    errs["over1e-2"] = OVER_1E2[0]
    errs["over_min_abs"] = OVER_1E2[1]
    return errs


def sample_rows(n: int, count: int, g: torch.Generator) -> torch.Tensor:
    """Edges plus random interior rows of a sequence of n rows."""
    fixed = [r for r in (0, 1, 63, 64, 127, 128, 129, n // 2, n - 2, n - 1) if 0 <= r < n]
    rnd = torch.randint(0, max(n, 1), (count,), generator=g).tolist() if n > 0 else []
    return torch.tensor(sorted(set(fixed + rnd)), dtype=torch.int64)


def compare_sampled(case: synth.Case, samples, o, smax, ssum):
    """Compare the GPU's full-size output with the oracle on sampled (b, h, rows)."""
    res = orc.attention_forward(
        case.q, case.k, case.v, layout=case.layout, scale=case.scale, q_rope=case.q_rope, k_rope=case.k_rope,
        atten_mask=case.atten_mask, sink=case.sink, causal=case.causal, pre_tokens=case.pre_tokens,
        next_tokens=case.next_tokens, cu_seqlens_q=case.cu_seqlens_q, cu_seqlens_kv=case.cu_seqlens_kv,
        samples=samples, pse=case.pse)
    dt = case.q.dtype
    errs = {"O": 0.0, "m": 0.0, "logl": 0.0}
    OVER_1E2[0], OVER_1E2[1] = 0, math.inf
    for (b, h, rows), (Or, Mr, Lr) in zip(samples, res):
        if case.layout == "TND":
            r0 = int(case.cu_seqlens_q[b])
            g_rows = rows + r0
            og = o[g_rows, h]
            if case.softmax_out_layout == "same_as_input":
                mg, lg = smax[g_rows, h], ssum[g_rows, h]
            else:
                mg, lg = smax[h, g_rows], ssum[h, g_rows]
        elif case.layout == "BNSD":
            og, mg, lg = o[b, h, rows], smax[b, h, rows], ssum[b, h, rows]
        elif case.layout == "BSND":
            og, mg, lg = o[b, rows, h], smax[b, h, rows], ssum[b, h, rows]
        else:
            raise ValueError(case.layout)
        errs["O"] = max(errs["O"], check_output(og, Or, dt, f"O b={b} h={h}"))
        errs["m"] = max(errs["m"], check_stats(mg, Mr, "max", dt))
        errs["logl"] = max(errs["logl"], check_stats(lg, Lr, "sum", dt))
    errs["over1e-2"] = OVER_1E2[0]
    errs["over_min_abs"] = OVER_1E2[1]
    return errs

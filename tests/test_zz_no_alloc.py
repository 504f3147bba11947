"""fa_fwd_noalloc: the same results as fa_fwd, with the library's own scratch array (needs an MI355X).

Each case needs scratch memory: a varlen call over more than 256 sequences
(tile prefix and map), a masked dense call (mask block classes) and a small
dense grid that splits its keys (fp32 partial results).  The outputs of fa_fwd_noalloc must equal those of
fa_fwd bit for bit; two calls in a row, the second on a smaller input, check
that what the first left in the array does not leak into the second.
"""
import pytest
import torch

import synth
from attention_forward_fa_amd import _lib, api

from . import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    yield


def _outputs(case, dev="cuda:0"):
    g = {k: pu.to_gpu(v, dev) for k, v in case.tensors().items()}
    q = g["q"]
    nh = q.shape[1] if case.layout in ("BNSD", "TND") else q.shape[2]
    out = torch.full(q.shape[:-1] + (case.v.shape[-1],), float("nan"), dtype=q.dtype, device=dev)
    if case.layout == "TND":
        shp = (nh, q.shape[0], 8)
    else:
        S = q.shape[2] if case.layout == "BNSD" else q.shape[1]
        shp = (q.shape[0], nh, S, 8)
    smax = torch.full(shp, float("nan"), dtype=torch.float32, device=dev)
    ssum = torch.full(shp, float("nan"), dtype=torch.float32, device=dev)
    plan = api.ForwardPlan(q, g["k"], g["v"], layout=case.layout, scale=case.scale, head_num=nh,
                           query_rope=g["q_rope"], key_rope=g["k_rope"], atten_mask=g["atten_mask"], sink=g["sink"],
                           cu_seqlens_q=g["cu_seqlens_q"], cu_seqlens_kv=g["cu_seqlens_kv"], causal=case.causal,
                           pre_tokens=case.pre_tokens, next_tokens=case.next_tokens, out=out, softmax_max=smax,
                           softmax_sum=ssum)
    return plan, (out, smax, ssum)


def _run_both(case):
    """(outputs of fa_fwd, outputs of fa_fwd_noalloc, workspace bytes) for one case."""
    plan_a, outs_a = _outputs(case)
    plan_b, outs_b = _outputs(case)
    try:
        assert plan_a.workspace_size > 0, "the case must use scratch memory"
        plan_a.run()
        _lib.fa_fwd_noalloc(plan_b.plan, torch.cuda.current_stream().cuda_stream)
        pu.sync_with_deadline("fa_fwd / fa_fwd_noalloc")
        return outs_a, outs_b, plan_a.workspace_size
    finally:
        plan_a.close()
        plan_b.close()


def _same(a, b):
    for x, y in zip(a, b):
        xi = x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)
        yi = y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32)
        assert torch.equal(xi, yi)


def _lengths(n, longest, seed):
    """n seeded sequence lengths in [0, longest]."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, longest + 1, (n,), generator=g).tolist()


CASES = [
    # varlen with more sequences than the kernels' own tile search takes,
    # causal, sink: tile prefix and tile map in the scratch
    ("varlen_big_then_small", lambda: synth.varlen_case("x", _lengths(300, 40, 140), 4, 128, "bf16", 140, sink=True,
                                                       causal=True),
     lambda: synth.varlen_case("x", _lengths(260, 10, 141), 2, 128, "bf16", 141, causal=True)),
    # masked dense: mask block classes in the scratch
    ("mask_big_then_small", lambda: synth.dense_case("x", "BNSD", 2, 2, 640, 128, "bf16", 142, mask=True,
                                                     pre_tokens=300, next_tokens=0),
     lambda: synth.dense_case("x", "BNSD", 1, 1, 200, 64, "fp16", 143, mask=True)),
    # small dense grid: the key split's fp32 partials in the scratch
    ("split_big_then_small", lambda: synth.dense_case("x", "BNSD", 1, 2, 300, 128, "bf16", 144, skv=2100, sink=True),
     lambda: synth.dense_case("x", "BNSD", 1, 1, 130, 128, "bf16", 145, skv=1030)),
]


@pytest.mark.parametrize("name,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_fa_fwd(name, big, small):
    print(f"[no-alloc] {name}: first call", flush=True)
    a, b, ws1 = _run_both(big())
    _same(a, b)
    print(f"[no-alloc] {name}: second, smaller call", flush=True)
    a2, b2, ws2 = _run_both(small())
    assert ws2 < ws1
    _same(a2, b2)
    assert not bool(torch.isnan(b2[0].float()).any())


def test_noalloc_rejects_plans_above_its_scratch():
    # B1 N8 S4096 Dv128, keys split: kv_splits x 32768 rows x 130 floats > 32 MiB
    q = torch.empty(1, 8, 4096, 128, dtype=torch.bfloat16, device="cuda")
    plan = api.ForwardPlan(q, q, q, layout="BNSD", scale=0.1, head_num=8, out=torch.empty_like(q))
    try:
        assert plan.workspace_size > (32 << 20), plan.describe()
        with pytest.raises(_lib.FaError) as ei:
            _lib.fa_fwd_noalloc(plan.plan, torch.cuda.current_stream().cuda_stream)
        assert ei.value.code == _lib.FA_ERR_UNSUPPORTED and "scratch" in ei.value.message
    finally:
        plan.close()

"""The C ABI on the CPU: the library loads, exports what the header declares,
and phase 1 validates and plans without touching a GPU.

Phase 1 reads only descriptors, so these tests hand it fabricated (aligned,
never dereferenced) device addresses.  Phase 2 is called only on paths that
return before any launch (NULL plan, missing workspace).
"""
import ctypes
import os
import re

import pytest

from attention_forward_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_fwd.h")

F32, F16, BF16, U8, BOOL, I32, I64 = range(7)
ADDR = 0x7F0000000000  # fake, 256-byte aligned


def desc(shape, dtype=BF16, strides=None, addr=ADDR):
    t = _lib.FaTensor()
    t.data = addr
    t.dtype = dtype
    t.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        t.shape[i] = s
        t.stride[i] = st
    return t


def plan(q, k, v, o, *, qr=None, kr=None, pse=None, mask=None, sink=None, cuq=None, cuk=None, scale=0.088,
         keep=1.0, pre=2**31 - 1, nxt=2**31 - 1, heads=None, layout=b"BSND", inner=0, sparse=0, causal=0,
         sol=b"", smax=None, ssum=None, qs=None, ks=None):
    L = _lib.lib()
    ws = ctypes.c_uint64(123)
    pl = ctypes.c_void_p(None)
    r = lambda d: ctypes.byref(d) if d is not None else None
    if heads is None:
        axis = {b"BNSD": 1, b"BSND": 2, b"TND": 1}.get(layout)
        heads = q.shape[axis] if (q is not None and axis is not None) else 24
    qsv = ctypes.c_int64(qs) if qs is not None else None
    ksv = ctypes.c_int64(ks) if ks is not None else None
    st = L.fa_fwd_get_workspace_size(r(q), r(qr), r(k), r(kr), r(v), r(pse), r(mask), r(sink), r(cuq), r(cuk),
                                     r(qsv), r(ksv),
                                     scale, keep, pre, nxt, heads, layout, inner, sparse, causal, sol, r(smax),
                                     r(ssum), r(o), ctypes.byref(ws), ctypes.byref(pl))
    return st, ws.value, pl.value


def describe(pl):
    return _lib.fa_plan_describe(pl)


def c2(dtype=BF16):
    s = [2, 4096, 24, 128]
    return desc(s, dtype), desc(s, dtype), desc(s, dtype), desc(s, dtype)


def test_header_symbols_exported():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:fa_status|void|int32_t|const char\*)\s+(fa_\w+)\s*\(", text, re.M))
    assert declared == set(_lib.EXPORTED), declared
    L = _lib.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name in ("FA_OK", "FA_ERR_PARAM_NULLPTR", "FA_ERR_PARAM_INVALID", "FA_ERR_UNSUPPORTED",
                 "FA_ERR_WORKSPACE", "FA_ERR_RUNTIME"):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == getattr(_lib, name)


def test_dense_headline_plan():
    q, k, v, o = c2()
    smax = desc([2, 24, 4096, 8], F32)
    ssum = desc([2, 24, 4096, 8], F32)
    st, ws, pl = plan(q, k, v, o, smax=smax, ssum=ssum)
    assert st == 0, _lib.last_error_message()
    try:
        assert ws == 0
        d = describe(pl)
        # long dense sequences, D = 128, no rope: the two-group kernel (256-row tiles)
        assert "kernel=mfma_pp " in d and "grid=768" in d and "block=512" in d and "dtype=bf16" in d, d
    finally:
        _lib.fa_plan_destroy(pl)


def test_varlen_plan_workspace():
    T, N = 8192, 24
    q = desc([T, N, 128])
    cu = desc([17], I32)
    smax = desc([N, T, 8], F32)
    st, ws, pl = plan(q, q, q, q, cuq=cu, cuk=cu, layout=b"TND", causal=1, smax=smax, ssum=smax)
    assert st == 0, _lib.last_error_message()
    # 16 sequences: each workgroup finds its tile from cu_seqlens, no tile map in the workspace
    assert ws == 0
    d = describe(pl)
    assert "varlen=1" in d and "grid=1920" in d and "reverse=1" in d, d  # (64 + 16) 128-row tiles x 24 heads
    assert "tile_search=1" in d, d
    _lib.fa_plan_destroy(pl)


def test_varlen_plan_tile_map_beyond_search_limit():
    """More sequences than the in-kernel search takes: the tile prefix and the
    map (a 32-byte entry per tile) come back in the workspace."""
    T, N, B = 8192, 4, 300
    q = desc([T, N, 128])
    cu = desc([B + 1], I32)
    st, ws, pl = plan(q, q, q, q, cuq=cu, cuk=cu, layout=b"TND", causal=1)
    assert st == 0, _lib.last_error_message()
    tiles = -(-T // 128) + B
    assert ws == ((B + 1) * 4 + 15) // 16 * 16 + tiles * 32
    d = describe(pl)
    assert "tile_search=0" in d and f"grid={tiles * N}" in d, d
    _lib.fa_plan_destroy(pl)
    cu = desc([257], I32)  # 256 sequences: still searched
    st, ws, pl = plan(q, q, q, q, cuq=cu, cuk=cu, layout=b"TND", causal=1)
    assert st == 0 and ws == 0 and "tile_search=1" in describe(pl)
    _lib.fa_plan_destroy(pl)


def test_fp32_uses_generic_kernel():
    s = [1, 2, 128, 64]
    st, ws, pl = plan(desc(s, F32), desc(s, F32), desc(s, F32), desc(s, F32), layout=b"BNSD")
    assert st == 0
    assert "kernel=generic" in describe(pl)
    _lib.fa_plan_destroy(pl)


def test_misaligned_falls_back_to_generic():
    q, k, v, o = c2()
    q.data = ADDR + 2
    st, ws, pl = plan(q, k, v, o)
    assert st == 0 and "kernel=generic" in describe(pl)
    _lib.fa_plan_destroy(pl)


def test_bsh_sbh_and_gqa_plan():
    q = desc([2, 100, 8 * 64])
    k = desc([2, 100, 2 * 64])
    st, ws, pl = plan(q, k, k, q, layout=b"BSH", heads=8)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "nq=8 nkv=2" in d and "d=64" in d
    _lib.fa_plan_destroy(pl)
    qs = desc([100, 2, 8 * 64])
    ks = desc([100, 2, 2 * 64])
    st, ws, pl = plan(qs, ks, ks, qs, layout=b"SBH", heads=8)
    assert st == 0
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("which", ["query", "key", "value", "out"])
def test_null_required_tensor(which):
    q, k, v, o = c2()
    args = dict(q=q, k=k, v=v, o=o)
    args[{"query": "q", "key": "k", "value": "v", "out": "o"}[which]] = None
    st, ws, pl = plan(args["q"], args["k"], args["v"], args["o"])
    assert st == 161001 and pl is None
    assert which in _lib.last_error_message() or "NULL" in _lib.last_error_message()


def test_null_layout_and_outputs():
    q, k, v, o = c2()
    L = _lib.lib()
    ws = ctypes.c_uint64(0)
    pl = ctypes.c_void_p(None)
    r = ctypes.byref
    st = L.fa_fwd_get_workspace_size(r(q), None, r(k), None, r(v), None, None, None, None, None, None, None, 0.1,
                                     1.0, 0, 0, 24, None, 0, 0, 0, b"", None, None, r(o), r(ws), r(pl))
    assert st == 161001
    st = L.fa_fwd_get_workspace_size(r(q), None, r(k), None, r(v), None, None, None, None, None, None, None, 0.1,
                                     1.0, 0, 0, 24, b"BSND", 0, 0, 0, b"", None, None, r(o), None, r(pl))
    assert st == 161001


def test_rope_pairing():
    q, k, v, o = c2()
    st, _, _ = plan(q, k, v, o, qr=desc([2, 4096, 24, 64]))
    assert st == 161001


@pytest.mark.parametrize("case", ["layout", "dtype_mismatch", "out_dtype", "int_q", "rope_f32", "rope_dtype",
                                  "mask_dtype", "sink_dtype", "stats_dtype", "sol", "ndim", "cu_dtype"])
def test_invalid_formats(case):
    q, k, v, o = c2()
    kw = {}
    if case == "layout":
        kw["layout"] = b"NSD"
    elif case == "dtype_mismatch":
        k = desc([2, 4096, 24, 128], F16)
    elif case == "out_dtype":
        o = desc([2, 4096, 24, 128], F32)
    elif case == "int_q":
        q = desc([2, 4096, 24, 128], I32)
    elif case == "rope_f32":
        q, k, v, o = c2(F32)
        kw.update(qr=desc([2, 4096, 24, 64], F32), kr=desc([2, 4096, 24, 64], F32))
    elif case == "rope_dtype":
        kw.update(qr=desc([2, 4096, 24, 64], F16), kr=desc([2, 4096, 24, 64], F16))
    elif case == "mask_dtype":
        kw["mask"] = desc([4096, 4096], F16)
    elif case == "sink_dtype":
        kw["sink"] = desc([24], BF16)
    elif case == "stats_dtype":
        kw["smax"] = desc([2, 24, 4096, 8], F16)
    elif case == "sol":
        kw["sol"] = b"NTD"
    elif case == "ndim":
        q = desc([2, 4096, 24 * 128])
        kw["heads"] = 24
    elif case == "cu_dtype":
        q = desc([100, 24, 128])
        kw.update(layout=b"TND", cuq=desc([3], I64), cuk=desc([3], I64))
        k = v = o = q
    st, _, pl = plan(q, k, v, o, **kw)
    assert st == 161002, (case, st, _lib.last_error_message())
    assert pl is None


@pytest.mark.parametrize("case", ["keep_prob", "sparse", "pse_compressed", "inner", "scale_neg", "scale_nan", "heads",
                                  "gqa_ratio", "d_mismatch", "dv_gt_d", "batch", "kv_rows", "out_shape",
                                  "mask_shape", "sink_shape", "stats_shape", "window_empty", "cu_dense",
                                  "tnd_mask_4d", "big_d", "cu_len"])
def test_unsupported(case):
    q, k, v, o = c2()
    kw = {}
    if case == "keep_prob":
        kw["keep"] = 0.9
    elif case == "sparse":
        kw["sparse"] = 2
    elif case == "pse_compressed":  # the last-1024-rows alibi form is not supported
        kw["pse"] = desc([2, 24, 1024, 4096])
    elif case == "inner":
        kw["inner"] = 3
    elif case == "scale_neg":
        kw["scale"] = -0.1
    elif case == "scale_nan":
        kw["scale"] = float("nan")
    elif case == "heads":
        kw["heads"] = 12
    elif case == "gqa_ratio":
        k = desc([2, 4096, 5, 128])
        v = desc([2, 4096, 5, 128])
    elif case == "d_mismatch":
        k = desc([2, 4096, 24, 64])
    elif case == "dv_gt_d":
        v = desc([2, 4096, 24, 256])
    elif case == "batch":
        k = desc([3, 4096, 24, 128])
    elif case == "kv_rows":
        v = desc([2, 4000, 24, 128])
    elif case == "out_shape":
        o = desc([2, 4096, 24, 64])
    elif case == "mask_shape":
        kw["mask"] = desc([4096, 4000], U8)
    elif case == "sink_shape":
        kw["sink"] = desc([23], F32)
    elif case == "stats_shape":
        kw["smax"] = desc([2, 24, 4096, 4], F32)
    elif case == "window_empty":
        kw.update(mask=desc([4096, 4096], U8), pre=-5, nxt=2)
    elif case == "cu_dense":
        kw.update(cuq=desc([3], I32), cuk=desc([3], I32))
    elif case == "tnd_mask_4d":
        q = desc([100, 24, 128])
        k = v = o = q
        kw.update(layout=b"TND", cuq=desc([3], I32), cuk=desc([3], I32), mask=desc([1, 1, 100, 100], U8))
    elif case == "big_d":
        q, k, v, o = (desc([2, 64, 24, 320]) for _ in range(4))
    elif case == "cu_len":
        q = desc([100, 24, 128])
        k = v = o = q
        kw.update(layout=b"TND", cuq=desc([3], I32), cuk=desc([4], I32))
    st, _, pl = plan(q, k, v, o, **kw)
    assert st == 561103, (case, st, _lib.last_error_message())
    assert pl is None


def test_tnd_requires_cu_seqlens():
    q = desc([100, 24, 128])
    st, _, _ = plan(q, q, q, q, layout=b"TND")
    assert st == 161001


def test_window_with_causal_needs_pre_plus_min_next_nonnegative():
    q, k, v, o = c2()
    # causal caps next at 0: pre = -1 leaves no key for any row
    st, _, _ = plan(q, k, v, o, causal=1, pre=-1, nxt=5)
    assert st == 561103
    st, _, pl = plan(q, k, v, o, causal=1, pre=0, nxt=5)
    assert st == 0
    assert "next=0" in describe(pl)
    _lib.fa_plan_destroy(pl)


def test_band_ignored_without_mask_or_causal():
    q, k, v, o = c2()
    st, _, pl = plan(q, k, v, o, pre=-5, nxt=2)  # would be empty, but no mask and no causal -> inactive
    assert st == 0 and "band=0" in describe(pl)
    _lib.fa_plan_destroy(pl)


def test_mask_class_table_in_workspace():
    """With a mask the workspace holds one class byte per (mask slice, 128-row
    tile, 64-key block), padded to 16 bytes; TND puts it after the tile prefix."""
    q, k, v, o = c2()
    cases = [([4096, 4096], 32 * 64), ([2, 1, 4096, 4096], 2 * 32 * 64), ([1, 24, 4096, 4096], 24 * 32 * 64),
             ([1, 1, 4096, 4096], 32 * 64)]
    for shape, want in cases:
        st, ws, pl = plan(q, k, v, o, mask=desc(shape, U8))
        assert st == 0, _lib.last_error_message()
        assert ws == want, (shape, ws)
        _lib.fa_plan_destroy(pl)
    # an odd key count: ceil(4000 / 64) = 63 blocks, ceil(4000 / 128) = 32 tiles
    s = [1, 4000, 2, 128]
    qq = desc(s)
    st, ws, pl = plan(qq, qq, qq, qq, mask=desc([4000, 4000], U8))
    # (64 workgroups: the keys split in 4 ranges, whose fp32 partials follow the table)
    assert st == 0 and "kv_splits=4" in describe(pl)
    assert ws == (32 * 63 + 15) // 16 * 16 + 4 * 2 * 4000 * 130 * 4, ws
    _lib.fa_plan_destroy(pl)
    # TND with 5 sequences (tiles found in the kernel, no map): only the 2-D mask's
    # table (8 x 11 -> 96)
    T, N = 1000, 4
    qt = desc([T, N, 128])
    cu = desc([6], I32)
    st, ws, pl = plan(qt, qt, qt, qt, cuq=cu, cuk=cu, layout=b"TND", mask=desc([1000, 700], U8))
    assert st == 0, _lib.last_error_message()
    assert ws == 96, ws  # 5 sequences: no tile map
    _lib.fa_plan_destroy(pl)
    # no mask: no table
    st, ws, pl = plan(q, k, v, o)
    assert st == 0 and ws == 0
    _lib.fa_plan_destroy(pl)


def test_phase2_argument_errors_without_launch():
    L = _lib.lib()
    assert L.fa_fwd(None, 0, None, None) == 161001
    T, N = 1000, 4
    q = desc([T, N, 128])
    cu = desc([301], I32)  # 300 sequences: a tile map in the workspace
    st, ws, pl = plan(q, q, q, q, cuq=cu, cuk=cu, layout=b"TND")
    assert st == 0 and ws == 1216 + (8 + 300) * 32  # tile prefix (301 int32 -> 1216 bytes) + map (308 tiles)
    assert L.fa_fwd(None, 0, pl, None) == 561201
    assert L.fa_fwd(ctypes.c_void_p(ADDR), ws - 1, pl, None) == 561201
    assert "workspace" in _lib.last_error_message()
    _lib.fa_plan_destroy(pl)


def test_plan_is_not_consumed_by_phase2():
    """Phase 2 leaves the plan alive (reusable plans; the caller releases it with fa_plan_destroy):
    the same plan answers several phase-2 calls and still describes itself afterwards."""
    L = _lib.lib()
    q = desc([300, 2, 128])
    cu = desc([301], I32)
    st, ws, pl = plan(q, q, q, q, cuq=cu, cuk=cu, layout=b"TND")
    assert st == 0 and ws > 0
    before = describe(pl)
    for _ in range(3):
        assert L.fa_fwd(ctypes.c_void_p(ADDR), ws - 16, pl, None) == 561201  # returns before any launch
    assert describe(pl) == before
    _lib.fa_plan_destroy(pl)
    header = open(HEADER).read()
    assert "The plan is not consumed" in header and "调用示例" in header


def test_clock_probe_argument_errors_without_launch():
    L = _lib.lib()
    assert L.fa_clock_probe(1000, None, None) == 161001
    assert L.fa_clock_probe(0, ctypes.c_void_p(ADDR), None) == 561103
    assert L.fa_clock_probe(1000001, ctypes.c_void_p(ADDR), None) == 561103


def test_fa_log_prints_the_plan(monkeypatch, capfd):
    q, k, v, o = c2()
    monkeypatch.setenv("FA_LOG", "1")
    st, _, pl = plan(q, k, v, o)
    assert st == 0
    _lib.fa_plan_destroy(pl)
    err = capfd.readouterr().err
    assert "[fa_fwd] plan kernel=mfma_pp " in err and "layout=BSND" in err, err
    monkeypatch.setenv("FA_LOG", "0")
    st, _, pl = plan(q, k, v, o)
    _lib.fa_plan_destroy(pl)
    assert "[fa_fwd]" not in capfd.readouterr().err


def test_noalloc_argument_errors_without_launch():
    L = _lib.lib()
    assert L.fa_fwd_noalloc(None, None) == 161001
    # B1 N8 S4096 D128: the small grid splits its keys in two, whose fp32 partials need more scratch
    # than the no-allocation entry point holds (32 MiB): refused before any device call
    s = [1, 8, 4096, 128]
    st, ws, pl = plan(desc(s), desc(s), desc(s), desc(s), layout=b"BNSD")
    assert st == 0 and ws > (32 << 20), describe(pl)
    assert L.fa_fwd_noalloc(ctypes.c_void_p(pl), None) == 561103
    assert "scratch" in _lib.last_error_message()
    _lib.fa_plan_destroy(pl)


def test_plan_destroy_null_and_describe_null():
    L = _lib.lib()
    L.fa_plan_destroy(None)
    assert L.fa_plan_describe(None, None, 0) == -1


def test_describe_truncates_safely():
    q, k, v, o = c2()
    st, _, pl = plan(q, k, v, o)
    L = _lib.lib()
    buf = ctypes.create_string_buffer(8)
    n = L.fa_plan_describe(pl, buf, 8)
    assert n > 8 and len(buf.value) == 7
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("case,family", [
    ("causal", "mfma_pp"),      # the window cuts only the causal side
    ("band", "mfma"),           # narrow sliding window: the four-wave kernel
    ("wide_band", "mfma_pp"),   # a window of 2048 + 1 keys: the two-group kernel
    ("rope", "mfma"),
    ("d64", "mfma"),
])
def test_family_policy(case, family):
    S, N = 4096, 16  # 256 two-group workgroups: one per compute unit
    q = desc([1, N, S, 128 if case != "d64" else 64])
    kw = dict(layout=b"BNSD")
    if case in ("causal", "band", "wide_band"):
        kw.update(causal=1, pre={"causal": 2**31 - 1, "band": 1024, "wide_band": 2048}[case], nxt=0)
    if case == "rope":
        r = desc([1, N, S, 64])
        kw.update(qr=r, kr=r)
    st, ws, pl = plan(q, q, q, q, **kw)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert f"kernel={family} " in d, d
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("causal", [0, 1])
def test_small_dense_grid_splits_keys(causal):
    # B1 N8 S4096: 128 two-group workgroups would leave half the compute units
    # idle; 256 four-wave workgroups fill half the slots, so two key ranges
    # (with pse there is no split: test_no_key_split_with_pse)
    B, N, S, D = 1, 8, 4096, 128
    q = desc([B, N, S, D])
    kw = dict(layout=b"BNSD", causal=causal, nxt=0 if causal else 2**31 - 1)
    st, ws, pl = plan(q, q, q, q, **kw)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "kernel=mfma " in d and "kv_splits=2" in d and "grid=512" in d, d
    assert ws == 2 * B * N * S * (D + 2) * 4  # fp32 partial outputs and {max, sum}
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("force,skv,splits,grid", [("1", 4096, 1, 256), ("3", 1000, 3, 768), ("4", 4096, 4, 1024),
                                                   ("2", 100, 2, 512), ("4", 100, 2, 512)])
def test_forced_key_split(monkeypatch, force, skv, splits, grid):
    monkeypatch.setenv("FA_FWD_KV_SPLIT", force)
    B, N, S, D = 1, 8, 4096, 128
    q, k = desc([B, N, S, D]), desc([B, N, skv, D])
    st, ws, pl = plan(q, k, k, q, layout=b"BNSD")
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "kernel=mfma " in d and f"kv_splits={splits} " in d + " " and f"grid={grid} " in d, d
    assert ws == (splits * B * N * S * (D + 2) * 4 if splits > 1 else 0)
    _lib.fa_plan_destroy(pl)


def test_key_split_limits(monkeypatch):
    # keys shorter than 8 blocks per range, a full grid, TND and the two-group
    # kernel never split on their own; bad forced counts are rejected
    s = [1, 8, 600, 128]
    st, ws, pl = plan(desc(s), desc(s), desc(s), desc(s), layout=b"BNSD")
    assert st == 0 and "kv_splits=1" in describe(pl) and ws == 0
    _lib.fa_plan_destroy(pl)
    q, k, v, o = c2()
    monkeypatch.setenv("FA_FWD_KERNEL", "mfma")
    st, ws, pl = plan(q, k, v, o)
    assert st == 0 and "kv_splits=1" in describe(pl) and "grid=1536" in describe(pl)
    _lib.fa_plan_destroy(pl)
    monkeypatch.setenv("FA_FWD_KERNEL", "pp")
    monkeypatch.setenv("FA_FWD_KV_SPLIT", "2")
    st, ws, pl = plan(q, k, v, o)
    assert st == 0 and "kv_splits=1" in describe(pl) and "kernel=mfma_pp" in describe(pl)
    _lib.fa_plan_destroy(pl)
    monkeypatch.delenv("FA_FWD_KERNEL")
    T = 4096
    t3 = desc([T, 2, 128])
    cu = desc([2], I32)
    st, ws, pl = plan(t3, t3, t3, t3, cuq=cu, cuk=cu, layout=b"TND", causal=1, nxt=0)
    assert st == 0, _lib.last_error_message()
    assert "kv_splits=1" in describe(pl)
    _lib.fa_plan_destroy(pl)
    for bad in ["0", "5", "two", "-1"]:
        monkeypatch.setenv("FA_FWD_KV_SPLIT", bad)
        st, _, pl = plan(desc([1, 8, 4096, 128]), desc([1, 8, 4096, 128]), desc([1, 8, 4096, 128]),
                         desc([1, 8, 4096, 128]), layout=b"BNSD")
        assert st == 561103 and pl is None and "FA_FWD_KV_SPLIT" in _lib.last_error_message()


def test_two_group_kernel_needs_32bit_row_offsets(monkeypatch):
    # BSND N128 D128: 32 KiB per key row; 65536 keys (+ 4 blocks) span 2 GiB, past the two-group kernel's
    # 32-bit offsets, so the four-wave kernel takes the call (and forcing the two-group one is refused)
    s = [1, 65536, 128, 128]
    st, ws, pl = plan(desc(s), desc(s), desc(s), desc(s))
    assert st == 0, _lib.last_error_message()
    assert "kernel=mfma " in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    s2 = [1, 65536 - 8192, 128, 128]  # (57344 + 256) rows x 32 KiB < 2 GiB
    st, ws, pl = plan(desc(s2), desc(s2), desc(s2), desc(s2))
    assert st == 0 and "kernel=mfma_pp " in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    monkeypatch.setenv("FA_FWD_KERNEL", "pp")
    st, _, pl = plan(desc(s), desc(s), desc(s), desc(s))
    assert st == 561103 and pl is None and "2 GiB" in _lib.last_error_message()


def test_four_wave_kernel_needs_32bit_block_offsets(monkeypatch):
    # the four-wave kernel stages a 64-row key block with 32-bit byte offsets: 64 x the row stride in bytes
    # must stay below 2^31; a strided K with 2^25-byte rows reaches it, one 8-element step less does not
    q = desc([1, 256, 2, 128])
    far = desc([1, 256, 2, 128], strides=[2**25, 2**24, 128, 1])          # 2^24 elements = 2^25 bytes per row
    near = desc([1, 256, 2, 128], strides=[2**25, 2**24 - 8, 128, 1])
    st, _, pl = plan(q, far, q, q)
    assert st == 0, _lib.last_error_message()
    assert "kernel=generic" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    st, _, pl = plan(q, near, q, q)
    assert st == 0 and "kernel=mfma " in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    st, _, pl = plan(q, q, far, q)  # the same bound holds for V
    assert st == 0 and "kernel=generic" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    monkeypatch.setenv("FA_FWD_KERNEL", "mfma")
    st, _, pl = plan(q, far, q, q)
    assert st == 561103 and pl is None and "32-bit block offsets" in _lib.last_error_message()


def test_pse_lds_needs_32bit_tile_offsets():
    # the pse tile (128 rows) is read with 32-bit byte offsets: 128 x the row stride in bytes below 2^31
    B, N, S, D = 1, 2, 256, 128
    q = desc([B, N, S, D])
    ok = desc([B, N, S, S], strides=[N * S * (2**23 - 8), S * (2**23 - 8), 2**23 - 8, 1])
    far = desc([B, N, S, S], strides=[N * S * 2**23, S * 2**23, 2**23, 1])
    st, _, pl = plan(q, q, q, q, pse=ok, layout=b"BNSD")
    assert st == 0 and "pse_lds=1" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    st, _, pl = plan(q, q, q, q, pse=far, layout=b"BNSD")
    assert st == 0 and "pse_lds=0" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("dr", [0, 64])
def test_d96_on_matrix_cores(dr, monkeypatch):
    s = [2, 1024, 8, 96]
    kw = dict(qr=desc([2, 1024, 8, 64]), kr=desc([2, 1024, 8, 64])) if dr else {}
    st, ws, pl = plan(desc(s), desc(s), desc(s), desc(s), **kw)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "kernel=mfma " in d and "d=96 " in d and f"dr={dr} " in d, d
    _lib.fa_plan_destroy(pl)
    monkeypatch.setenv("FA_FWD_KERNEL", "pp")  # the two-group kernel has no D = 96
    st, _, pl = plan(desc(s), desc(s), desc(s), desc(s), **kw)
    assert st == 561103 and pl is None and "D = Dv = 64 or 128" in _lib.last_error_message()


@pytest.mark.parametrize("dqk,dv,want", [(192, 128, "d=128 dr=64"), (128, 64, "d=64 dr=64"), (160, 96, "d=96 dr=64")])
def test_dqk_above_dv_on_matrix_cores(dqk, dv, want):
    # no rope inputs: the last 64 dims of q and k become the rope part of the matrix-core kernels
    q, v = desc([1, 512, 4, dqk]), desc([1, 512, 4, dv])
    st, ws, pl = plan(q, q, v, v)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "kernel=mfma " in d and want in d and f"dv={dv} " in d, d
    _lib.fa_plan_destroy(pl)
    # with pse (which the rope kernels do not take) the pair stays as it is: on the matrix cores for
    # Dqk in {96, 128, 256}, else on the generic kernel
    st, ws, pl = plan(q, q, v, v, pse=desc([1, 4, 512, 512]), layout=b"BSND")
    fam = "kernel=mfma " if dqk in (96, 128, 256) else "kernel=generic"
    assert st == 0 and fam in describe(pl) and f"d={dqk} dr=0" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("dqk,dv", [(96, 64), (128, 96), (256, 96), (256, 64)])
def test_dqk_above_dv_without_rope_tail(dqk, dv):
    """Dqk > Dv with Dqk - Dv != 64: the four-wave kernel's own (Dqk, 0, Dv) instantiations, with and
    without pse; fp32 stays on the generic kernel."""
    q, v = desc([1, 512, 4, dqk]), desc([1, 512, 4, dv])
    for pse in (None, desc([1, 4, 512, 512])):
        st, ws, pl = plan(q, q, v, v, pse=pse, layout=b"BSND")
        assert st == 0, _lib.last_error_message()
        d = describe(pl)
        assert "kernel=mfma " in d and f"d={dqk} dr=0 dv={dv} " in d, d
        _lib.fa_plan_destroy(pl)
    qf, vf = desc([1, 512, 4, dqk], F32), desc([1, 512, 4, dv], F32)
    st, ws, pl = plan(qf, qf, vf, vf)
    assert st == 0 and "kernel=generic" in describe(pl)
    _lib.fa_plan_destroy(pl)
    # a pair outside the instantiated set (Dv above 128 but below Dqk) stays on the generic kernel
    q2, v2 = desc([1, 512, 4, 256]), desc([1, 512, 4, 192])
    st, ws, pl = plan(q2, q2, v2, v2)
    assert st == 0 and "kernel=generic" in describe(pl)
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("dv", [256, 128])
def test_d256_on_matrix_cores(dv, monkeypatch):
    # head dim 256 (the largest the aclnnFlashAttentionScore page lists) runs the four-wave kernel, one
    # workgroup per CU (its two LDS stages take 128 KiB); Dv = 256 or 128
    q, v = desc([2, 4096, 16, 256]), desc([2, 4096, 16, dv])
    st, ws, pl = plan(q, q, v, v)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "kernel=mfma " in d and "d=256 dr=0 " in d and f"dv={dv} " in d and "kv_splits=1" in d, d
    _lib.fa_plan_destroy(pl)
    # a small grid splits the keys against one workgroup slot per CU: 16 tiles x 2 heads = 32 workgroups
    q2, v2 = desc([1, 2048, 2, 256]), desc([1, 2048, 2, dv])
    st, ws, pl = plan(q2, q2, v2, v2)
    assert st == 0 and "kv_splits=4" in describe(pl) and ws > 0, describe(pl)
    _lib.fa_plan_destroy(pl)
    monkeypatch.setenv("FA_FWD_KERNEL", "pp")
    st, _, pl = plan(q, q, v, v)
    assert st == 561103 and pl is None and "two-group" in _lib.last_error_message()


def test_small_grid_uses_four_wave_kernel():
    s = [1, 300, 2, 128]
    st, ws, pl = plan(desc(s), desc(s), desc(s), desc(s))
    assert st == 0
    d = describe(pl)
    assert "kernel=mfma " in d and "bm=128" in d and "grid=6" in d, d
    _lib.fa_plan_destroy(pl)


@pytest.mark.parametrize("force,expect", [("mfma", "kernel=mfma grid=1536"), ("pp", "kernel=mfma_pp grid=768"),
                                          ("generic", "kernel=generic"), ("", "kernel=mfma_pp grid=768")])
def test_forced_kernel_family(monkeypatch, force, expect):
    monkeypatch.setenv("FA_FWD_KERNEL", force)
    q, k, v, o = c2()
    st, ws, pl = plan(q, k, v, o)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    for part in expect.split():
        assert part in d.split(), d
    _lib.fa_plan_destroy(pl)


def test_forced_kernel_errors(monkeypatch):
    monkeypatch.setenv("FA_FWD_KERNEL", "mfma")
    s = [1, 2, 128, 64]
    st, _, pl = plan(desc(s, F32), desc(s, F32), desc(s, F32), desc(s, F32), layout=b"BNSD")
    assert st == 561103 and pl is None and "FA_FWD_KERNEL" in _lib.last_error_message()
    monkeypatch.setenv("FA_FWD_KERNEL", "fastest")
    q, k, v, o = c2()
    st, _, pl = plan(q, k, v, o)
    assert st == 561103 and pl is None


# ---------------------------------------------------------------------------
# pse (real_shift)
# ---------------------------------------------------------------------------

def test_pse_plan_and_validation():
    B, N, S, D = 2, 4, 512, 128
    q = desc([B, N, S, D])
    ok = desc([B, N, S, S])
    st, ws, pl = plan(q, q, q, q, pse=ok, layout=b"BNSD")
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "pse=1" in d and "kernel=mfma " in d and "pse_lds=1" in d, d
    _lib.fa_plan_destroy(pl)
    # rows that are not a multiple of 8 keys, or a base off 16 bytes: per-lane reads
    odd = desc([B, N, S, S + 4])
    st, _, pl = plan(q, desc([B, N, S + 4, D]), desc([B, N, S + 4, D]), q, pse=odd, layout=b"BNSD")
    assert st == 0 and "pse_lds=0" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    st, _, pl = plan(q, q, q, q, pse=desc([B, N, S, S], addr=ADDR + 8), layout=b"BNSD")
    assert st == 0 and "pse_lds=0" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    # pse with the rope term is not combined
    qr = desc([B, N, S, 64])
    st, _, pl = plan(q, q, q, q, qr=qr, kr=qr, pse=ok, layout=b"BNSD")
    assert st == 561103 and pl is None and "rope" in _lib.last_error_message()
    st, _, pl = plan(q, q, q, q, pse=desc([1, N, S, S]), layout=b"BNSD")  # broadcast over batch
    assert st == 0, _lib.last_error_message()
    _lib.fa_plan_destroy(pl)
    # long dense D=128 would pick the two-group kernel, which takes no pse
    q4 = desc([1, N, 4096, D])
    st, _, pl = plan(q4, q4, q4, q4, pse=desc([1, N, 4096, 4096]), layout=b"BNSD")
    assert st == 0 and "kernel=mfma " in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    bad = [
        (dict(pse=desc([B, N, S, S], F16)), 161002),            # dtype differs from query's
        (dict(pse=desc([B, N, S])), 561103),                    # rank
        (dict(pse=desc([B, 1, S, S])), 561103),                 # heads must be N
        (dict(pse=desc([B, N, 1024 if S > 1024 else S - 1, S])), 561103),  # not Sq rows
        (dict(pse=ok, qr=desc([B, N, S, 64]), kr=desc([B, N, S, 64])), 561103),  # with rope
    ]
    for kw, code in bad:
        st, _, pl = plan(q, q, q, q, layout=b"BNSD", **kw)
        assert st == code and pl is None, (kw, st, _lib.last_error_message())


def test_pse_forced_pp_rejected(monkeypatch):
    monkeypatch.setenv("FA_FWD_KERNEL", "pp")
    q = desc([1, 2, 256, 128])
    st, _, pl = plan(q, q, q, q, pse=desc([1, 2, 256, 256]), layout=b"BNSD")
    assert st == 561103 and pl is None and "FA_FWD_KERNEL" in _lib.last_error_message()


def test_pse_tnd_workspace():
    T, N = 1000, 2
    q = desc([T, N, 128])
    cu = desc([6], I32)
    st, ws, pl = plan(q, q, q, q, cuq=cu, cuk=cu, layout=b"TND", pse=desc([12345]))
    assert st == 0, _lib.last_error_message()
    assert ws == 8 * 6  # 5 sequences, no tile map: the 6 int64 pse block offsets
    _lib.fa_plan_destroy(pl)
    st, _, pl = plan(q, q, q, q, cuq=cu, cuk=cu, layout=b"TND", pse=desc([10, 10]))
    assert st == 561103 and pl is None


# ---------------------------------------------------------------------------
# outer split (q_start_idx / kv_start_idx) and the merge entry point
# ---------------------------------------------------------------------------

def test_outer_split_moves_the_window():
    q = desc([1, 2, 512, 128])
    # causal chunk whose keys all precede its rows: the window no longer cuts
    st, _, pl = plan(q, q, q, q, layout=b"BNSD", causal=1, qs=4096, ks=0)
    assert st == 0, _lib.last_error_message()
    d = describe(pl)
    assert "pre=268431360" in d and "next=4096" in d and "reverse=0" in d, d
    _lib.fa_plan_destroy(pl)
    st, _, pl = plan(q, q, q, q, layout=b"BNSD", causal=1, pre=100, qs=1000, ks=1200)
    assert st == 0 and "pre=300 " in describe(pl) and "next=-200 " in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    st, _, pl = plan(q, q, q, q, layout=b"BNSD", causal=1, qs=-1)
    assert st == 561103 and pl is None


def _merge_call(parts, out, smax=None, ssum=None, layout=b"BNSD", heads=2, sol=b""):
    L = _lib.lib()
    n = len(parts)
    arr = lambda i: (_lib.FaTensor * n)(*[p[i] for p in parts])
    r = lambda d: ctypes.byref(d) if d is not None else None
    return L.fa_fwd_merge(n, arr(0), arr(1), arr(2), layout, heads, sol, r(out), r(smax), r(ssum), None)


def test_merge_validation():
    o = desc([1, 2, 64, 128])
    st_ = desc([1, 2, 64, 8], F32)
    part = (o, st_, st_)
    assert _merge_call([part] * 17, o) == 561103                       # too many parts
    assert _merge_call([(desc([1, 2, 63, 128]), st_, st_)], o) == 561103  # shape differs
    assert _merge_call([(o, desc([1, 2, 64, 4], F32), st_)], o) == 561103  # stats shape
    assert _merge_call([(o, desc([1, 2, 64, 8], BF16), st_)], o) == 161002  # stats dtype
    assert _merge_call([(desc([1, 2, 64, 128], F16), st_, st_)], o) == 161002  # out dtype differs
    assert _merge_call([part], o, layout=b"XYZ") == 161002

def test_no_key_split_with_pse(monkeypatch):
    """A dense grid too small for the chip splits its keys, except with pse, whose bias dominates the
    HBM bytes (the split's fp32 partials would add a fifth); FA_FWD_KV_SPLIT still forces a split."""
    q = desc([1, 8, 4096, 128])
    st, ws, pl = plan(q, q, q, q, layout=b"BNSD")
    assert st == 0 and "kv_splits=2" in describe(pl), describe(pl)
    _lib.fa_plan_destroy(pl)
    pse = desc([1, 8, 4096, 4096])
    st, ws, pl = plan(q, q, q, q, pse=pse, layout=b"BNSD")
    assert st == 0 and "kv_splits=1" in describe(pl) and "pse_lds=1" in describe(pl) and ws == 0, describe(pl)
    _lib.fa_plan_destroy(pl)
    monkeypatch.setenv("FA_FWD_KV_SPLIT", "2")
    st, ws, pl = plan(q, q, q, q, pse=pse, layout=b"BNSD")
    assert st == 0 and "kv_splits=2" in describe(pl) and ws > 0, describe(pl)
    _lib.fa_plan_destroy(pl)

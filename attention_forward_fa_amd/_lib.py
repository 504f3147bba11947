"""ctypes binding of ``libfa_fwd.so`` (declared in ``include/fa_fwd.h``).

Argument marshalling only: torch tensors become ``fa_tensor`` descriptors of
their device memory, and the C entry points are called with the same names.
Every step of the forward runs in the library's HIP kernels; there is no
other code path, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

# FA_FWD_LIB names another build of the same C ABI (the tests use it for a host-only
# AddressSanitizer build of phase 1); by default the in-tree library.
LIB_PATH = os.environ.get("FA_FWD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_fwd.so")

FA_OK = 0
FA_ERR_PARAM_NULLPTR = 161001
FA_ERR_PARAM_INVALID = 161002
FA_ERR_UNSUPPORTED = 561103
FA_ERR_WORKSPACE = 561201
FA_ERR_RUNTIME = 561202

FA_DTYPE = {
    torch.float32: 0,
    torch.float16: 1,
    torch.bfloat16: 2,
    torch.uint8: 3,
    torch.bool: 4,
    torch.int32: 5,
    torch.int64: 6,
}

EXPORTED = ("fa_fwd_get_workspace_size", "fa_fwd", "fa_fwd_merge", "fa_plan_destroy", "fa_plan_describe",
            "fa_last_error_message", "fa_clock_probe", "fa_fwd_noalloc")


class FaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class FaError(RuntimeError):
    """A non-zero status from the library, with its message."""

    def __init__(self, code: int, where: str, message: str):
        super().__init__(f"{where} failed with status {code}: {message}")
        self.code = code
        self.message = message


_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m attention_forward_fa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        T = P(FaTensor)
        L.fa_fwd_get_workspace_size.restype = ctypes.c_int32
        L.fa_fwd_get_workspace_size.argtypes = [
            T, T, T, T, T, T, T, T, T, T, P(ctypes.c_int64), P(ctypes.c_int64),
            ctypes.c_double, ctypes.c_double, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_char_p,
            T, T, T, P(ctypes.c_uint64), P(ctypes.c_void_p),
        ]
        L.fa_fwd.restype = ctypes.c_int32
        L.fa_fwd.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        L.fa_plan_destroy.restype = None
        L.fa_plan_destroy.argtypes = [ctypes.c_void_p]
        L.fa_plan_describe.restype = ctypes.c_int32
        L.fa_plan_describe.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_size_t]
        L.fa_fwd_merge.restype = ctypes.c_int32
        L.fa_fwd_merge.argtypes = [ctypes.c_int32, T, T, T, ctypes.c_char_p, ctypes.c_int64, ctypes.c_char_p,
                                   T, T, T, ctypes.c_void_p]
        L.fa_fwd_noalloc.restype = ctypes.c_int32
        L.fa_fwd_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.fa_clock_probe.restype = ctypes.c_int32
        L.fa_clock_probe.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
        L.fa_last_error_message.restype = ctypes.c_char_p
        L.fa_last_error_message.argtypes = []
        _lib = L
        return L


def describe_tensor(t: Optional[torch.Tensor], *, device_required: bool = True) -> Optional[FaTensor]:
    """fa_tensor for a torch tensor's memory (None -> None)."""
    if t is None:
        return None
    if t.dtype not in FA_DTYPE:
        raise TypeError(f"dtype {t.dtype} has no fa_dtype")
    if t.dim() < 1 or t.dim() > 4:
        raise ValueError(f"tensors must have 1..4 dims, got {t.dim()}")
    if device_required and not t.is_cuda:
        raise ValueError("tensor must live in GPU memory")
    d = FaTensor()
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = FA_DTYPE[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d: Optional[FaTensor]):
    return ctypes.byref(d) if d is not None else None


def last_error_message() -> str:
    return lib().fa_last_error_message().decode()


def fa_fwd_get_workspace_size(query, query_rope, key, key_rope, value, real_shift, atten_mask, sink,
                              cu_seqlens_q, cu_seqlens_kv, q_start_idx: Optional[int], kv_start_idx: Optional[int],
                              scale_value: float, keep_prob: float,
                              pre_tokens: int, next_tokens: int, head_num: int, input_layout: str,
                              inner_precise: int, sparse_mode: int, causal: bool,
                              softmax_out_layout: str, softmax_max, softmax_sum, attention_out,
                              *, device_required: bool = True):
    """Phase 1.  Tensor arguments are torch tensors or None; the start indices
    are ints or None.  Returns (workspace_bytes, plan handle)."""
    L = lib()
    ds = [describe_tensor(t, device_required=device_required) for t in
          (query, query_rope, key, key_rope, value, real_shift, atten_mask, sink, cu_seqlens_q, cu_seqlens_kv,
           softmax_max, softmax_sum, attention_out)]
    qs = ctypes.c_int64(int(q_start_idx)) if q_start_idx is not None else None
    ks = ctypes.c_int64(int(kv_start_idx)) if kv_start_idx is not None else None
    ws = ctypes.c_uint64(0)
    plan = ctypes.c_void_p(None)
    st = L.fa_fwd_get_workspace_size(
        *(_ref(d) for d in ds[:10]), _ref(qs), _ref(ks),
        float(scale_value), float(keep_prob), int(pre_tokens), int(next_tokens),
        int(head_num), input_layout.encode() if input_layout is not None else None, int(inner_precise),
        int(sparse_mode), 1 if causal else 0,
        softmax_out_layout.encode() if softmax_out_layout is not None else None,
        *(_ref(d) for d in ds[10:]), ctypes.byref(ws), ctypes.byref(plan))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_get_workspace_size", last_error_message())
    return int(ws.value), plan.value


def fa_fwd(workspace: Optional[torch.Tensor], workspace_size: int, plan, stream: int) -> None:
    """Phase 2: enqueue on ``stream`` (a hipStream_t handle as int)."""
    L = lib()
    ptr = workspace.data_ptr() if workspace is not None and workspace.numel() > 0 else None
    st = L.fa_fwd(ptr, int(workspace_size), plan, stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd", last_error_message())


def fa_fwd_noalloc(plan, stream: int) -> None:
    """Phase 2 with the library's own scratch array instead of a workspace (allocates nothing)."""
    st = lib().fa_fwd_noalloc(plan, stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_noalloc", last_error_message())


def fa_fwd_merge(part_out, part_max, part_sum, input_layout: str, head_num: int, softmax_out_layout: str,
                 attention_out, softmax_max, softmax_sum, stream: int) -> None:
    """Merge partial results (lists of torch tensors) into attention_out / the stats (enqueued on ``stream``)."""
    L = lib()
    n = len(part_out)
    if not (len(part_max) == len(part_sum) == n):
        raise ValueError("part lists differ in length")
    arr = lambda ts: (FaTensor * max(n, 1))(*[describe_tensor(t) for t in ts])
    po, pm, pl = arr(part_out), arr(part_max), arr(part_sum)
    st = L.fa_fwd_merge(n, po, pm, pl, input_layout.encode(), int(head_num),
                        softmax_out_layout.encode() if softmax_out_layout is not None else None,
                        _ref(describe_tensor(attention_out)), _ref(describe_tensor(softmax_max)),
                        _ref(describe_tensor(softmax_sum)), stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_merge", last_error_message())


def fa_plan_destroy(plan) -> None:
    lib().fa_plan_destroy(plan)


def fa_plan_describe(plan) -> str:
    L = lib()
    n = L.fa_plan_describe(plan, ctypes.create_string_buffer(1), 1)
    buf = ctypes.create_string_buffer(n + 1)
    L.fa_plan_describe(plan, buf, n + 1)
    return buf.value.decode()


def fa_clock_probe(microseconds: int, device_out: torch.Tensor, stream: int) -> None:
    """Enqueue the shader-clock probe; ``device_out`` is a GPU int64 tensor of 2 elements."""
    if device_out.dtype != torch.int64 or device_out.numel() < 2 or not device_out.is_cuda:
        raise ValueError("device_out must be a GPU int64 tensor with 2 elements")
    st = lib().fa_clock_probe(int(microseconds), device_out.data_ptr(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_clock_probe", last_error_message())

"""FlashAttention forward for MI355X (gfx950): a C-ABI library of HIP kernels
(``libfa_fwd.so``, declared in ``include/fa_fwd.h``) and its Python binding."""
from ._lib import (FA_ERR_PARAM_INVALID, FA_ERR_PARAM_NULLPTR, FA_ERR_RUNTIME, FA_ERR_UNSUPPORTED,
                   FA_ERR_WORKSPACE, FA_OK, FaError, fa_fwd, fa_fwd_get_workspace_size, fa_plan_describe,
                   fa_plan_destroy)
from .api import (ForwardPlan, attention_forward, attention_forward_varlen, cu_from_actual_seq_len)

__all__ = ["FA_OK", "FA_ERR_PARAM_NULLPTR", "FA_ERR_PARAM_INVALID", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE",
           "FA_ERR_RUNTIME", "FaError", "fa_fwd_get_workspace_size", "fa_fwd", "fa_plan_destroy",
           "fa_plan_describe", "ForwardPlan", "attention_forward", "attention_forward_varlen",
           "cu_from_actual_seq_len"]

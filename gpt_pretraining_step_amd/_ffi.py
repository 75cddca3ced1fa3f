"""ctypes declarations of include/gpt2.h (libgpt2hip.so).

Argument marshalling only: every computation happens in the library's HIP
kernels.  Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes as ct
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2hip.so")

GPT2_OK = 0
GPT2_WARN_NO_TARGETS = 1
GPT2_ERR_ARG = -1
GPT2_ERR_SHAPE = -2
GPT2_ERR_HIP = -3
GPT2_ERR_UNBOUND = -4
GPT2_ERR_BAD_ID = -5
GPT2_ERR_NONFINITE = -6

PRECISION_FP32 = 0
PRECISION_BF16 = 1

EPI_STORE = 0
EPI_RESIDUAL = 1
EPI_GELU = 2
EPI_DGELU = 3
EPI_ACCUMULATE = 4
EPI_GELU_GRAD = 5
EPI_MUL = 6
EPI_ROPE = 7
EPI_SWIGLU = 8
EPI_SWIGLU_BWD = 9

ARCH_GPT2 = 0
ARCH_ROTARY = 1


class Config(ct.Structure):
    _fields_ = [(n, ct.c_int32) for n in (
        "vocab_size", "block_size", "n_layer", "n_head", "n_embd", "mlp_hidden", "max_batch", "precision", "arch",
        "n_kv_head")]


class Sizes(ct.Structure):
    _fields_ = [
        ("n_params", ct.c_size_t), ("n_elems", ct.c_size_t), ("n_tensors", ct.c_int32), ("n_decayed", ct.c_int32),
        ("params_bytes", ct.c_size_t), ("grads_bytes", ct.c_size_t), ("adam_m_bytes", ct.c_size_t),
        ("adam_v_bytes", ct.c_size_t), ("shadow_bytes", ct.c_size_t), ("activations_bytes", ct.c_size_t),
        ("scratch_bytes", ct.c_size_t),
    ]


class Buffers(ct.Structure):
    _fields_ = [(n, ct.c_void_p) for n in ("params", "grads", "adam_m", "adam_v", "shadow", "activations", "scratch")]


class AdamW(ct.Structure):
    _fields_ = [(n, ct.c_float) for n in ("lr", "beta1", "beta2", "eps", "weight_decay", "max_norm")]


class ParamDesc(ct.Structure):
    _fields_ = [("name", ct.c_char * 64), ("offset", ct.c_size_t), ("ndim", ct.c_int32), ("shape", ct.c_int32 * 2),
                ("decayed", ct.c_int32)]


class GemmArgs(ct.Structure):
    _fields_ = [
        ("M", ct.c_int32), ("N", ct.c_int32), ("K", ct.c_int32), ("dtype", ct.c_int32),
        ("a_kmajor", ct.c_int32), ("b_kmajor", ct.c_int32),
        ("lda", ct.c_int64), ("ldb", ct.c_int64), ("ldc", ct.c_int64),
        ("A", ct.c_void_p), ("B", ct.c_void_p), ("C", ct.c_void_p), ("C2", ct.c_void_p), ("R", ct.c_void_p),
        ("U", ct.c_void_p), ("bias", ct.c_void_p), ("alpha", ct.c_float), ("epilogue", ct.c_int32),
        ("out_bf16", ct.c_int32), ("rope", ct.c_void_p), ("rope_period", ct.c_int32), ("rope_cols", ct.c_int32),
        ("ld2", ct.c_int64),
    ]


# name -> (restype, argtypes)
SIGNATURES = {
    "gpt2_query_sizes": (ct.c_int, [ct.POINTER(Config), ct.POINTER(Sizes)]),
    "gpt2_param_info": (ct.c_int, [ct.POINTER(Config), ct.c_int, ct.POINTER(ParamDesc)]),
    "gpt2_create": (ct.c_int, [ct.POINTER(Config), ct.POINTER(Buffers), ct.c_void_p, ct.POINTER(ct.c_void_p)]),
    "gpt2_destroy": (ct.c_int, [ct.c_void_p]),
    "gpt2_set_stream": (ct.c_int, [ct.c_void_p, ct.c_void_p]),
    "gpt2_set_doc_mask": (ct.c_int, [ct.c_void_p, ct.c_int]),
    "gpt2_init_params": (ct.c_int, [ct.c_void_p, ct.c_uint64]),
    "gpt2_sync_shadow": (ct.c_int, [ct.c_void_p]),
    "gpt2_zero_grad": (ct.c_int, [ct.c_void_p]),
    "gpt2_fwd_bwd": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_float, ct.c_void_p,
                                ct.c_void_p]),
    "gpt2_graph_capture": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_float,
                                      ct.c_void_p]),
    "gpt2_graph_launch": (ct.c_int, [ct.c_void_p]),
    "gpt2_clip_adamw_step": (ct.c_int, [ct.c_void_p, ct.POINTER(AdamW), ct.c_void_p]),
    "gpt2_lr_at": (ct.c_double, [ct.c_int64, ct.c_double, ct.c_double, ct.c_int64, ct.c_int64]),
    "gpt2_get_step": (ct.c_int, [ct.c_void_p, ct.POINTER(ct.c_int64)]),
    "gpt2_set_step": (ct.c_int, [ct.c_void_p, ct.c_int64]),
    "gpt2_get_status": (ct.c_int, [ct.c_void_p]),
    "gpt2_strerror": (ct.c_char_p, [ct.c_int]),
    "gpt2_lmhead_ce_scratch_bytes": (ct.c_size_t, [ct.c_int, ct.c_int, ct.c_int]),
    "gpt2_lmhead_ce": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_int,
                                  ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p]),
    "gpt2_op_gemm": (ct.c_int, [ct.c_void_p, ct.POINTER(GemmArgs)]),
    "gpt2_gemm_grouped_workspace_bytes": (ct.c_size_t, [ct.POINTER(GemmArgs), ct.c_int]),
    "gpt2_op_gemm_grouped": (ct.c_int, [ct.c_void_p, ct.POINTER(GemmArgs), ct.c_int, ct.POINTER(ct.c_void_p),
                                        ct.c_void_p]),
    "gpt2_op_colsum": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_int64, ct.c_void_p]),
    "gpt2_op_layernorm_fwd": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int,
                                         ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int]),
    "gpt2_op_layernorm_bwd": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int] + [ct.c_void_p] * 8 + [ct.c_int, ct.c_int]),
    "gpt2_op_attention_fwd": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_int, ct.c_int, ct.c_int,
                                         ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p]),
    "gpt2_attention_bwd_scratch_bytes": (ct.c_size_t, [ct.c_int, ct.c_int, ct.c_int]),
    "gpt2_op_attention_bwd": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_int, ct.c_int, ct.c_int,
                                         ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                         ct.c_void_p, ct.c_void_p, ct.c_void_p]),
    "gpt2_noalloc_scratch_bytes": (ct.c_size_t, []),
    "gpt2_op_attention_bwd_noalloc": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_int, ct.c_int,
                                                 ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                 ct.c_void_p, ct.c_void_p, ct.c_void_p]),
    "gpt2_embedding_bwd_scratch_bytes": (ct.c_size_t, [ct.c_int, ct.c_int]),
    "gpt2_op_embedding_bwd": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int,
                                         ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p]),
    "gpt2_op_segment_starts": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "gpt2_profile_enable": (ct.c_int, [ct.c_void_p, ct.c_int]),
    "gpt2_profile_only": (ct.c_int, [ct.c_void_p, ct.c_char_p]),
    "gpt2_profile_mark": (ct.c_int, [ct.c_void_p, ct.c_int]),
    "gpt2_op_marker": (ct.c_int, [ct.c_void_p]),
    "gpt2_op_rmsnorm_fwd": (ct.c_int, [ct.c_void_p] * 5 + [ct.c_int, ct.c_int]),
    "gpt2_op_rmsnorm_bwd": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int] + [ct.c_void_p] * 6 + [ct.c_int, ct.c_int]),
    "gpt2_op_rope_table": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_double, ct.c_void_p]),
    "gpt2_op_rope_bwd": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int64, ct.c_int, ct.c_int, ct.c_void_p]),
    "gpt2_profile_reset": (ct.c_int, [ct.c_void_p]),
    "gpt2_profile_count": (ct.c_int, [ct.c_void_p]),
    "gpt2_profile_entry": (ct.c_int, [ct.c_void_p, ct.c_int, ct.POINTER(ct.c_char_p), ct.POINTER(ct.c_int64),
                                      ct.POINTER(ct.c_double)]),
}

_LIB = None


def lib() -> ct.CDLL:
    """The loaded library.  Raises if it has not been built: there is no
    fallback implementation."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gpt_pretraining_step_amd.build`")
        L = ct.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class GPT2Error(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        msg = lib().gpt2_strerror(status).decode()
        super().__init__(f"{where}: {msg} (status {status})" if where else f"{msg} (status {status})")


def check(status: int, where: str = "") -> int:
    if status < 0:
        raise GPT2Error(status, where)
    return status

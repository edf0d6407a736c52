"""ctypes binding of include/llama_mi355x.h -- argument marshalling only.

Every function here has the name and meaning of the C entry point it wraps; device
buffers and streams are passed as integer addresses (torch's data_ptr() / cuda_stream).
All computation happens in libllama_mi355x.so; if it is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllama_mi355x.so")

LLAMA_OK = 0
LLAMA_ERR_INVALID_ARG = -1
LLAMA_ERR_UNSUPPORTED = -2
LLAMA_ERR_WORKSPACE = -3
LLAMA_ERR_HIP = -4
LLAMA_BF16 = 0
LLAMA_FP32 = 1
LLAMA_FP16 = 2
DTYPES = {"bf16": LLAMA_BF16, "fp32": LLAMA_FP32, "fp16": LLAMA_FP16}

# Every symbol include/llama_mi355x.h declares.
EXPORTED = ("llama_check_args", "llama_workspace_bytes", "llama_init", "llama_prefill",
            "llama_decode_step", "llama_decode_step_noalloc", "llama_argmax", "llama_sample_top_p", "llama_select_next", "llama_destroy",
            "llama_status_str", "llama_profile_select", "llama_profile_read")

# Kernel classes for llama_profile_select (llama_kernel_class in the header).
KERNEL_CLASSES = {"none": 0, "gemv_qkv": 1, "attn_decode": 2, "gemv_wo": 3, "gemv_w13": 4,
                  "gemv_w2": 5, "gemv_out": 6, "gemm_qkv": 7, "attn_prefill": 8, "gemm_wo": 9,
                  "gemm_w13": 10, "gemm_w2": 11, "rmsnorm": 12}


class llama_args(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("vocab_size", ctypes.c_int32), ("hidden_dim", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_batch_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class llama_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w2", "w3")]


class llama_weights(ctypes.Structure):
    _fields_ = [("tok_embeddings", ctypes.c_void_p), ("norm", ctypes.c_void_p),
                ("output", ctypes.c_void_p), ("layers", ctypes.POINTER(llama_layer_weights))]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decoder_only_transformer_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        A = ctypes.POINTER(llama_args)
        L.llama_check_args.argtypes = [A]
        L.llama_check_args.restype = ctypes.c_int
        L.llama_workspace_bytes.argtypes = [A]
        L.llama_workspace_bytes.restype = SZ
        L.llama_init.argtypes = [A, ctypes.POINTER(llama_weights), P, SZ, P, ctypes.POINTER(P)]
        L.llama_init.restype = ctypes.c_int
        L.llama_prefill.argtypes = [P, P, I64, I32, I32, I32, P, I32, P]
        L.llama_prefill.restype = ctypes.c_int
        L.llama_decode_step.argtypes = [P, P, I64, I32, I32, P, P]
        L.llama_decode_step.restype = ctypes.c_int
        L.llama_decode_step_noalloc.argtypes = [P, P, I64, I32, I32, P, P]
        L.llama_decode_step_noalloc.restype = ctypes.c_int
        L.llama_argmax.argtypes = [P, I32, I32, I64, P, P]
        L.llama_argmax.restype = ctypes.c_int
        L.llama_sample_top_p.argtypes = [P, I32, I32, I64, ctypes.c_float, ctypes.c_float, P, P, P, P]
        L.llama_sample_top_p.restype = ctypes.c_int
        L.llama_select_next.argtypes = [P, P, I64, I32, P, I32, P]
        L.llama_select_next.restype = ctypes.c_int
        L.llama_destroy.argtypes = [P]
        L.llama_destroy.restype = None
        L.llama_profile_select.argtypes = [P, I32]
        L.llama_profile_select.restype = ctypes.c_int
        L.llama_profile_read.argtypes = [P, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_double)]
        L.llama_profile_read.restype = ctypes.c_int
        L.llama_status_str.argtypes = [ctypes.c_int]
        L.llama_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def llama_check_args(args: llama_args) -> int:
    return lib().llama_check_args(ctypes.byref(args))


def llama_workspace_bytes(args: llama_args) -> int:
    return lib().llama_workspace_bytes(ctypes.byref(args))


def llama_init(args: llama_args, weights: llama_weights, d_workspace: int, workspace_bytes: int,
               stream: int) -> Tuple[int, Optional[int]]:
    ctx = ctypes.c_void_p()
    st = lib().llama_init(ctypes.byref(args), ctypes.byref(weights), d_workspace, workspace_bytes,
                          stream, ctypes.byref(ctx))
    return st, ctx.value


def llama_prefill(ctx: int, d_tokens: int, ld_tokens: int, bsz: int, seqlen: int,
                  start_pos: int, d_logits: int, all_positions: int, stream: int) -> int:
    return lib().llama_prefill(ctx, d_tokens, ld_tokens, bsz, seqlen, start_pos, d_logits,
                               all_positions, stream)


def llama_decode_step(ctx: int, d_tokens: int, ld_tokens: int, bsz: int, start_pos: int,
                      d_logits: int, stream: int) -> int:
    return lib().llama_decode_step(ctx, d_tokens, ld_tokens, bsz, start_pos, d_logits, stream)


def llama_decode_step_noalloc(ctx: int, d_tokens: int, ld_tokens: int, bsz: int, start_pos: int,
                              d_logits: int, stream: int) -> int:
    return lib().llama_decode_step_noalloc(ctx, d_tokens, ld_tokens, bsz, start_pos, d_logits, stream)


def llama_argmax(d_logits: int, bsz: int, vocab: int, row_stride: int, d_out: int,
                 stream: int) -> int:
    return lib().llama_argmax(d_logits, bsz, vocab, row_stride, d_out, stream)


def llama_sample_top_p(d_logits: int, bsz: int, vocab: int, row_stride: int, temperature: float,
                       top_p: float, d_uniform: int, d_out: int, d_logprob: int, stream: int) -> int:
    return lib().llama_sample_top_p(d_logits, bsz, vocab, row_stride, temperature, top_p, d_uniform, d_out,
                                    d_logprob, stream)


def llama_select_next(d_next: int, d_tokens: int, ld_tokens: int, cur_pos: int,
                      d_prompt_len: int, bsz: int, stream: int) -> int:
    return lib().llama_select_next(d_next, d_tokens, ld_tokens, cur_pos, d_prompt_len, bsz, stream)


def llama_destroy(ctx: int) -> None:
    lib().llama_destroy(ctx)


def llama_status_str(st: int) -> str:
    return lib().llama_status_str(st).decode()


def llama_profile_select(ctx: int, kernel_class: int) -> int:
    return lib().llama_profile_select(ctx, kernel_class)


def llama_profile_read(ctx: int) -> Tuple[int, int, float]:
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    st = lib().llama_profile_read(ctx, ctypes.byref(n), ctypes.byref(ms))
    return st, n.value, ms.value

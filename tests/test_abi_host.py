"""The C-ABI library without a GPU: it loads, exports every declared symbol, and rejects
bad arguments on the host before any device call."""
import ctypes
import os
import re

import pytest

from decoder_only_transformer_amd import abi
from decoder_only_transformer_amd.runtime import make_args

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "llama_mi355x.h")


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:llama_status|size_t|void|const char)\s*\*?\s*(llama_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(abi.LIB_PATH):
        pytest.skip("library not built")
    return abi.lib()


def tiny(**kw):
    base = dict(dim=256, n_layers=4, n_heads=8, n_kv_heads=2, vocab_size=512, hidden_dim=768,
                norm_eps=1e-5, rope_theta=10000.0, max_batch_size=2, max_seq_len=128, dtype="fp32")
    base.update(kw)
    return make_args(**base)


def test_exports_every_header_symbol(lib):
    syms = header_symbols()
    assert set(syms) == set(abi.EXPORTED)
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings(lib):
    assert abi.llama_status_str(abi.LLAMA_OK) == "LLAMA_OK"
    assert abi.llama_status_str(abi.LLAMA_ERR_WORKSPACE) == "LLAMA_ERR_WORKSPACE"
    assert abi.llama_status_str(-99) == "LLAMA_STATUS_UNKNOWN"


@pytest.mark.parametrize("kw,expect", [
    (dict(), abi.LLAMA_OK),
    (dict(dtype="bf16"), abi.LLAMA_OK),
    (dict(dtype="fp16"), abi.LLAMA_OK),
    (dict(n_kv_heads=3), abi.LLAMA_ERR_INVALID_ARG),          # n_heads % n_kv_heads
    (dict(dim=250), abi.LLAMA_ERR_INVALID_ARG),               # dim % n_heads
    (dict(n_heads=16, n_kv_heads=1), abi.LLAMA_ERR_UNSUPPORTED),  # head_dim 16, n_rep 16
    (dict(n_heads=2, n_kv_heads=2), abi.LLAMA_OK),            # head_dim 128, MHA
    (dict(n_heads=4, n_kv_heads=4, dim=1024), abi.LLAMA_ERR_UNSUPPORTED),  # head_dim 256
    (dict(max_batch_size=0), abi.LLAMA_ERR_INVALID_ARG),
    (dict(max_seq_len=-1), abi.LLAMA_ERR_INVALID_ARG),
    (dict(vocab_size=511), abi.LLAMA_ERR_UNSUPPORTED),
    (dict(hidden_dim=700), abi.LLAMA_ERR_UNSUPPORTED),
    (dict(max_seq_len=70000), abi.LLAMA_ERR_UNSUPPORTED),
])
def test_check_args(lib, kw, expect):
    a = tiny(**kw)
    assert abi.llama_check_args(a) == expect
    assert (abi.llama_workspace_bytes(a) > 0) == (expect == abi.LLAMA_OK)


def test_fp16_models_take_the_bf16_workspace_layout(lib):
    """An fp16 model runs the bf16 model's kernels (MFMA prefill, 16-bit operands, split-K
    partials) with the other 16-bit type, so its workspace is the bf16 one byte for byte; the
    fp32 model keeps fp32 activations for every prefill row and a 4-byte cache instead."""
    f32 = abi.llama_workspace_bytes(tiny(dtype="fp32"))
    f16 = abi.llama_workspace_bytes(tiny(dtype="fp16"))
    b16 = abi.llama_workspace_bytes(tiny(dtype="bf16"))
    assert f16 == b16 and f16 != f32 and f16 > 0
    bad = tiny()
    bad.dtype = 3
    assert abi.llama_check_args(bad) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_workspace_bytes(bad) == 0


def test_workspace_holds_kv_cache_of_pages_example(lib):
    """7B shape, batch 4, seq 2048, 2-byte cache: 64 MiB per tensor per layer, K and V over
    32 layers = 4 GiB, plus activation scratch."""
    a = make_args(4096, 32, 32, 32, 32000, 11008, 1e-5, 10000.0, 4, 2048, "bf16")
    kv = 2 * 32 * 4 * 2048 * 32 * 128 * 2
    assert kv == 4 * 2 ** 30
    ws = abi.llama_workspace_bytes(a)
    assert ws >= kv and ws < kv + 8 * 2 ** 30


def test_init_rejects_bad_arguments_without_touching_the_device(lib):
    a = tiny()
    layers = (abi.llama_layer_weights * 4)(*[abi.llama_layer_weights(*([16] * 9)) for _ in range(4)])
    w = abi.llama_weights(16, 16, 16, ctypes.cast(layers, ctypes.POINTER(abi.llama_layer_weights)))
    need = abi.llama_workspace_bytes(a)
    st, ctx = abi.llama_init(a, w, 256, need - 1, 0)
    assert st == abi.LLAMA_ERR_WORKSPACE and ctx is None
    st, ctx = abi.llama_init(a, w, 0, need, 0)
    assert st == abi.LLAMA_ERR_WORKSPACE
    st, ctx = abi.llama_init(a, w, 100, need, 0)           # misaligned workspace
    assert st == abi.LLAMA_ERR_WORKSPACE
    bad = (abi.llama_layer_weights * 4)(*[abi.llama_layer_weights(*([16] * 8 + [0])) for _ in range(4)])
    wb = abi.llama_weights(16, 16, 16, ctypes.cast(bad, ctypes.POINTER(abi.llama_layer_weights)))
    st, _ = abi.llama_init(a, wb, 256, need, 0)
    assert st == abi.LLAMA_ERR_INVALID_ARG
    st, _ = abi.llama_init(tiny(n_kv_heads=3), w, 256, need, 0)
    assert st == abi.LLAMA_ERR_INVALID_ARG
    for i in range(3):                                      # misaligned embeddings / norm / output
        ptrs = [16, 16, 16]
        ptrs[i] = 18
        wm = abi.llama_weights(*ptrs, ctypes.cast(layers, ctypes.POINTER(abi.llama_layer_weights)))
        st, _ = abi.llama_init(a, wm, 256, need, 0)
        assert st == abi.LLAMA_ERR_INVALID_ARG


def test_calls_reject_bad_arguments(lib):
    assert abi.llama_prefill(None, 16, 16, 1, 1, 0, 16, 0, 0) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_decode_step(None, 16, 1, 1, 0, 16, 0) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_argmax(16, 0, 10, 10, 16, 0) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_argmax(16, 1, 10, 9, 16, 0) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_argmax(0, 1, 10, 10, 16, 0) == abi.LLAMA_ERR_INVALID_ARG
    # sampling: every host-checkable precondition, before anything is launched
    for args in [(0, 2, 10, 10, 0.8, 0.9, 16, 16, 0, 0),           # NULL logits
                 (16, 0, 10, 10, 0.8, 0.9, 16, 16, 0, 0),          # bsz < 1
                 (16, 2, 0, 10, 0.8, 0.9, 16, 16, 0, 0),           # vocab < 1
                 (16, 2, 10, 9, 0.8, 0.9, 16, 16, 0, 0),           # row_stride < vocab
                 (16, 2, 10, 10, 0.0, 0.9, 16, 16, 0, 0),          # temperature 0 (argmax's case)
                 (16, 2, 10, 10, float("inf"), 0.9, 16, 16, 0, 0), # temperature not finite
                 (16, 2, 10, 10, 0.8, -0.5, 16, 16, 0, 0),         # top_p < 0
                 (16, 2, 10, 10, 0.8, float("nan"), 16, 16, 0, 0), # top_p NaN
                 (16, 2, 10, 10, 0.8, 0.9, 0, 16, 0, 0),           # NULL uniforms
                 (16, 2, 10, 10, 0.8, 0.9, 16, 0, 0, 0)]:          # NULL out
        assert abi.llama_sample_top_p(*args) == abi.LLAMA_ERR_INVALID_ARG, args
    assert abi.llama_sample_top_p(16, 2, 40000, 40000, 0.8, 0.9, 16, 16, 0, 0) == abi.LLAMA_ERR_UNSUPPORTED
    assert abi.llama_select_next(16, 16, 8, 8, 16, 1, 0) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_select_next(16, 16, 8, -1, 16, 1, 0) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_select_next(16, 16, 8, 3, 0, 1, 0) == abi.LLAMA_ERR_INVALID_ARG


def test_profile_calls_reject_null(lib):
    assert abi.llama_profile_select(None, 1) == abi.LLAMA_ERR_INVALID_ARG
    st, n, ms = abi.llama_profile_read(None)
    assert st == abi.LLAMA_ERR_INVALID_ARG

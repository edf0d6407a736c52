"""Checked mode (LLAMA_MI355X_CHECK_TOKENS=1 at llama_init): token ids outside [0, vocab) are
detected on the device and the call returns LLAMA_ERR_INVALID_ARG; in-range calls are unchanged
(bit-identical logits to the unchecked ctx); without the mode the ids are clamped."""
import os

import numpy as np
import pytest
import torch

import synth
from decoder_only_transformer_amd import abi, runtime

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.lib()
    return True


def make(wl, checked):
    old = os.environ.get("LLAMA_MI355X_CHECK_TOKENS")
    os.environ["LLAMA_MI355X_CHECK_TOKENS"] = "1" if checked else "0"
    try:
        W = synth.gen_weights(wl, device="cuda")
        args = runtime.make_args(wl.dim, wl.n_layers, wl.n_heads, wl.n_kv_heads, wl.vocab_size, wl.hidden_dim,
                                 wl.norm_eps, wl.rope_theta, wl.batch, wl.max_seq_len, wl.dtype)
        return runtime.LlamaModel(args, W)
    finally:
        if old is None:
            os.environ.pop("LLAMA_MI355X_CHECK_TOKENS")
        else:
            os.environ["LLAMA_MI355X_CHECK_TOKENS"] = old


@pytest.mark.parametrize("dtype,batch", [("fp32", 2), ("bf16", 2), ("bf16", 6)])
def test_checked_mode_flags_out_of_range_tokens(dtype, batch):
    wl = synth.WORKLOADS["tiny_fp32"].with_(name="checked", dtype=dtype, batch=batch, max_seq_len=32)
    plain, checked = make(wl, False), make(wl, True)
    V = wl.vocab_size
    rng = np.random.default_rng(3)
    tok = torch.from_numpy(rng.integers(3, V, size=(batch, 8)).astype(np.int32)).cuda()
    s = runtime.stream_handle()
    outs = []
    for m in (plain, checked):
        lg = torch.empty((batch, V), device="cuda")
        assert abi.llama_prefill(m.ctx, tok.data_ptr(), 8, batch, 6, 0, lg.data_ptr(), 0, s) == abi.LLAMA_OK
        d = torch.empty((batch, V), device="cuda")
        assert abi.llama_decode_step(m.ctx, tok.data_ptr() + 4 * 6, 8, batch, 6, d.data_ptr(), s) == abi.LLAMA_OK
        n = torch.empty((batch, V), device="cuda")
        assert abi.llama_decode_step_noalloc(m.ctx, tok.data_ptr() + 4 * 6, 8, batch, 6, n.data_ptr(), s) == abi.LLAMA_OK
        torch.cuda.synchronize()
        outs.append((lg, d, n))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    bad = tok.clone()
    bad[batch - 1, 2] = V            # one past the end, in the prefill
    bad[0, 7] = -5                   # negative, at the decode position
    lg = torch.empty((batch, V), device="cuda")
    assert abi.llama_prefill(checked.ctx, bad.data_ptr(), 8, batch, 6, 0, lg.data_ptr(), 0, s) == \
        abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_prefill(plain.ctx, bad.data_ptr(), 8, batch, 6, 0, lg.data_ptr(), 0, s) == abi.LLAMA_OK
    d = torch.empty((batch, V), device="cuda")
    assert abi.llama_decode_step(checked.ctx, bad.data_ptr() + 4 * 7, 8, batch, 7, d.data_ptr(), s) == \
        abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_decode_step_noalloc(checked.ctx, bad.data_ptr() + 4 * 7, 8, batch, 7, d.data_ptr(), s) == \
        abi.LLAMA_ERR_INVALID_ARG
    # the flag is cleared per call: an in-range call afterwards succeeds
    assert abi.llama_decode_step(checked.ctx, tok.data_ptr() + 4 * 7, 8, batch, 7, d.data_ptr(), s) == abi.LLAMA_OK
    torch.cuda.synchronize()
    assert torch.isfinite(d).all()
    plain.close()
    checked.close()

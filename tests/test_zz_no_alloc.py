"""llama_decode_step_noalloc (the decode step whose scratch is the library's static device
array) against llama_decode_step through the C ABI: same kernels, same arithmetic, so the
logits must be bit-identical; two calls in a row, the second with a smaller batch (another
kernel path and a smaller scratch carve-up)."""
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


def model_of(wl, max_batch, weights=None):
    W = weights if weights is not None else synth.gen_weights(wl, device="cuda")
    args = runtime.make_args(wl.dim, wl.n_layers, wl.n_heads, wl.n_kv_heads, wl.vocab_size, wl.hidden_dim,
                             wl.norm_eps, wl.rope_theta, max_batch, wl.max_seq_len, wl.dtype)
    return runtime.LlamaModel(args, W)


@pytest.mark.parametrize("dtype,batches", [("bf16", (20, 3)), ("bf16", (32, 6)), ("fp16", (24, 5)), ("fp32", (2, 1))])
def test_noalloc_decode_equals_decode_step(dtype, batches):
    """Prefill the batch, then at the next two positions: llama_decode_step, then
    llama_decode_step_noalloc on the same tokens and position (it rewrites the same K/V),
    bit-identical logits; the second position with fewer rows."""
    wl = synth.WORKLOADS["tiny_fp32"].with_(name="noalloc", dtype=dtype, n_heads=8, n_kv_heads=2, dim=1024,
                                            hidden_dim=2816, vocab_size=2000, n_layers=3, max_seq_len=64,
                                            weight_seed=31, prompt_seed=131)
    B = batches[0]
    model = model_of(wl, B)
    rng = np.random.default_rng(7)
    S = 24
    tok = torch.from_numpy(rng.integers(3, wl.vocab_size, size=(B, S + 2)).astype(np.int32)).cuda()
    pre = torch.empty((B, wl.vocab_size), device="cuda")
    model.prefill(tok, B, S, 0, pre)
    for j, bsz in enumerate(batches):
        pos = S + j
        ref = torch.full((bsz, wl.vocab_size), float("nan"), device="cuda")
        got = torch.full((bsz, wl.vocab_size), float("nan"), device="cuda")
        model.decode_step(tok, bsz, pos, pos, ref)
        st = model.decode_step_noalloc(tok, bsz, pos, pos, got)
        assert st == abi.LLAMA_OK, abi.llama_status_str(st)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref), (got - ref).abs().max().item()
        print(f"  {dtype} position {pos}, {bsz} rows: bit-identical", flush=True)
    model.close()


def test_noalloc_decode_rejects_what_it_cannot_serve():
    wl = synth.WORKLOADS["tiny_fp32"].with_(name="noalloc_err", dtype="bf16", n_layers=1, max_seq_len=16,
                                            weight_seed=32)
    model = model_of(wl, 40)
    tok = torch.zeros((40, 4), dtype=torch.int32, device="cuda")
    out = torch.empty((40, wl.vocab_size), device="cuda")
    s = runtime.stream_handle()
    assert abi.llama_decode_step_noalloc(model.ctx, tok.data_ptr(), 4, 33, 0, out.data_ptr(), s) == \
        abi.LLAMA_ERR_UNSUPPORTED
    assert abi.llama_decode_step_noalloc(model.ctx, tok.data_ptr(), 4, 41, 0, out.data_ptr(), s) == \
        abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_decode_step_noalloc(model.ctx, 0, 4, 2, 0, out.data_ptr(), s) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_decode_step_noalloc(model.ctx, tok.data_ptr(), 4, 2, 16, out.data_ptr(), s) == \
        abi.LLAMA_ERR_INVALID_ARG
    model.close()
    # a step whose scratch passes the 32 MiB array: 32 rows x 196608 hidden units of fp32 gate
    # activations alone are 24 MiB, their bf16 copy 12 MiB (weights never read: rejected first)
    big = synth.WORKLOADS["tiny_fp32"].with_(name="noalloc_big", dtype="bf16", dim=512, n_heads=4, n_kv_heads=4,
                                             hidden_dim=196608, n_layers=1, vocab_size=512, max_seq_len=8)
    e = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    W = {"tok_embeddings": e(512, 512), "norm": e(512), "output": e(512, 512),
         "layers": [{"attention_norm": e(512), "wq": e(512, 512), "wk": e(512, 512), "wv": e(512, 512),
                     "wo": e(512, 512), "ffn_norm": e(512), "w1": e(196608, 512), "w2": e(512, 196608),
                     "w3": e(196608, 512)}]}
    m2 = model_of(big, 32, W)
    tok2 = torch.zeros((32, 2), dtype=torch.int32, device="cuda")
    out2 = torch.empty((32, 512), device="cuda")
    assert abi.llama_decode_step_noalloc(m2.ctx, tok2.data_ptr(), 2, 32, 0, out2.data_ptr(), s) == \
        abi.LLAMA_ERR_WORKSPACE
    m2.close()

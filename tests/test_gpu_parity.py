"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.

The oracle is run teacher-forced on the GPU's own token sequence (one causal pass, layer by
layer), which by the causal mask gives the logits every generate call should have produced,
including after a legitimate low-margin divergence.

fp32 models: max |d logit| <= 1e-4 against the plain oracle in fp64.

16-bit models (bf16; fp16 with the bar scaled by the ulp ratio): the stated bars are max
|d logit| <= 3e-2 and cosine >= 0.999 per position, and the greedy token must be the
oracle's wherever the oracle's top-1/top-2 margin exceeds 0.1.  Each result is compared
with three oracle evaluations on the same tokens:
  ref    the oracle in its 16-bit storage mode (fp32 arithmetic, the tensors the method
         stores in 16 bits rounded where they are produced);
  alt    the same, on an equivalent model whose model and FFN dimensions are permuted
         consistently (the same function; every fp32 sum in another order): a second
         correct evaluation of the method;
  plain  the plain fp32 oracle (no storage rounding).
Where a second correct evaluation meets the stated bars (small shapes, one layer at the 7B
widths), the GPU must meet them too.  At depth it does not: two correct bf16 evaluations
of the 7B shape differ by ~0.15 at single logits, and the bf16-storage oracle itself sits
at cosine 0.9987 from the plain one (rounding the K/V cache alone moves the logits by
0.15; measured in test_llama2_7b_b1_generate_matches_oracle).  There the GPU must be as
close to ref and to plain as a correct evaluation is, within a factor 1 + DELTA, on the
pooled RMS and 99.9th percentile of |d logit|, the worst position's RMS and the maximum
(tests/parity_stats.py), and greedy tokens must match where no correct evaluation could
flip them, with band mismatches within what a correct evaluation's noise explains.
"""
import os
import sys

import time

import numpy as np
import pytest
import torch

import oracle
import parity_stats as ps
import synth
from decoder_only_transformer_amd import abi, runtime

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4
BF16_TOL = 3e-2
COS_MIN = 0.999
MARGIN = 0.1
# Allowance over a second correct evaluation.  Correct evaluations (fp32 with permuted sums,
# fp64) differ from one another by up to 3% in the pooled statistics and 7% in the extreme
# ones (worst position, maximum) at the 7B widths; the GPU's arithmetic perturbs the stored
# values in more places than a summation order does (P carried as bf16 high + low parts in
# the attention, fp32 RoPE table, exp2-based softmax), each at the same ~1e-6 relative level.
DELTA = 0.2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.lib()   # fail loudly if the library is missing
    return True


def args_of(wl, max_batch=None):
    return runtime.make_args(wl.dim, wl.n_layers, wl.n_heads, wl.n_kv_heads, wl.vocab_size,
                             wl.hidden_dim, wl.norm_eps, wl.rope_theta,
                             max_batch or wl.batch, wl.max_seq_len, wl.dtype)


class HostWeights:
    """Oracle weights: the generator's device tensors as host fp32 arrays (the generator's
    device output is bit-identical to its CPU output), one layer at a time.  Each tensor is
    widened on the device (exact) and copied into a pinned host buffer that the next layer's
    tensor of the same name reuses; the oracle touches a layer's weights only while it
    computes that layer.

    perm_seed: the model with its dim and hidden axes permuted consistently (the same
    function, every fp32 sum over them in another order); the gathers are torch indexing on
    the device (data movement only)."""

    def __init__(self, W, dim, hidden, perm_seed=None):
        self.W = W
        self.bufs = {}
        self.cache = {}
        self.layer = None
        self.pd = self.ph = None
        if perm_seed is not None:
            rng = np.random.default_rng(perm_seed)
            dev = W["output"].device
            self.pd = torch.from_numpy(rng.permutation(dim)).to(dev)
            self.ph = torch.from_numpy(rng.permutation(hidden)).to(dev)

    def _permute(self, name, w):
        pd, ph = self.pd, self.ph
        if name in ("tok_embeddings", "output", "wq", "wk", "wv"):
            return w[:, pd]
        if name in ("norm", "attention_norm", "ffn_norm", "wo"):
            return w[pd]
        if name in ("w1", "w3"):
            return w[ph][:, pd]
        if name == "w2":
            return w[pd][:, ph]
        raise KeyError(name)

    def __call__(self, name, layer):
        key = (name, layer)
        if key in self.cache:
            return self.cache[key]
        if layer >= 0 and layer != self.layer:
            for k in [k for k in self.cache if k[1] >= 0]:
                del self.cache[k]
            self.layer = layer
        w = self.W[name] if layer < 0 else self.W["layers"][layer][name]
        if self.pd is not None:
            w = self._permute(name, w)
        bkey = (name, layer < 0)
        buf = self.bufs.get(bkey)
        if buf is None or buf.shape != w.shape:
            buf = torch.empty(w.shape, dtype=torch.float32, pin_memory=True)
            self.bufs[bkey] = buf
        buf.copy_(w.float())
        self.cache[key] = buf.numpy()
        return self.cache[key]


def host_weights(wl, W):
    return HostWeights(W, wl.dim, wl.hidden_dim)


def oracle_pass(wl, W, tokens, kind, storage="bf16", dtype=np.float32):
    """Teacher-forced oracle logits (B, T, V) for tokens (B, T): kind "ref" (storage mode),
    "alt" (storage mode, permuted model), "plain" (no storage rounding) or "kv" (only the
    K/V cache rounded to bf16)."""
    a = oracle.args_from_workload(wl)
    prov = HostWeights(W, wl.dim, wl.hidden_dim, perm_seed=7 if kind == "alt" else None)
    st = {"ref": storage, "alt": storage, "plain": None, "kv": "bf16_kv"}[kind]
    t0 = time.perf_counter()
    out = oracle.teacher_forced_logits(a, prov, tokens, dtype, storage=st)
    say(f"    oracle pass {kind:5s} over {tokens.shape[0]} x {tokens.shape[1]} positions: "
        f"{time.perf_counter() - t0:.1f} s")
    return out


def gpu_generate(wl, weights, prompts, keep_logits=True):
    model = runtime.LlamaModel(args_of(wl, len(prompts)), weights)
    run = runtime.GreedyRun(model, prompts, wl.gen_steps, keep_logits=keep_logits)
    run.run()
    torch.cuda.synchronize()
    out = run.tokens.cpu().numpy().astype(np.int64), run.logits.cpu().numpy(), run
    model.close()
    return out


def check_logits(gpu, ref, alt, plain, stated=BF16_TOL):
    """ps.check_depth with this file's bars; returns the distances."""
    return ps.check_depth(gpu, ref, alt, plain, DELTA, say=say, stated_max=stated, stated_cos=COS_MIN)


def forced_margin(dist, stated=BF16_TOL):
    """Oracle margin above which the greedy token is forced: the stated 0.1 where a second
    correct evaluation stays within the stated bar, else twice the largest logit error the
    GPU is allowed (no correct evaluation can flip such a pick)."""
    a = dist["alt_ref"].max_all
    return MARGIN if a <= stated else max(MARGIN, 2.0 * (1.0 + DELTA) * a)


def check_generate_rows(wl, W, prompts, tokens, call_logits, rows, storage="bf16", stated=BF16_TOL,
                        plain=True, min_len=None, extra_kinds=()):
    """The generate run's logits of batch rows `rows` against the oracle passes on those rows
    (teacher-forced on the GPU's tokens), pooled over rows and calls; greedy tokens against
    the reference's.  Call i produced the logits of position min_len - 1 + i (min_len: the
    shortest prompt of the whole batch).  Returns the oracle passes."""
    rows = list(rows)
    if min_len is None:
        min_len = min(len(p) for p in prompts)
    n_calls = call_logits.shape[0]
    sel = np.arange(min_len - 1, min_len - 1 + n_calls)
    tb = tokens[rows, :-1]
    passes = {k: oracle_pass(wl, W, tb, k, storage) for k in ("ref", "alt") + (("plain",) if plain else ())
              + tuple(extra_kinds)}

    def pooled(x):   # (rows, calls, V) -> (rows * calls, V)
        return x.reshape(-1, x.shape[-1])
    G = pooled(np.transpose(call_logits[:, rows], (1, 0, 2)))
    assert np.isfinite(G).all(), "non-finite GPU logits"
    S, P = pooled(passes["ref"][:, sel]), pooled(passes["alt"][:, sel])
    X = pooled(passes["plain"][:, sel]) if plain else None
    dist = check_logits(G, S, P, X, stated)
    # greedy tokens at the positions generated (not prompt tokens kept by the select)
    free = np.array([[sel[i] + 1 >= len(prompts[b]) for i in range(n_calls)] for b in rows]).reshape(-1)
    nxt = np.array([[tokens[b, sel[i] + 1] for i in range(n_calls)] for b in rows]).reshape(-1)
    rep = ps.greedy_check(nxt[free], G[free], S[free], P[free], forced_margin(dist, stated))
    say(f"    {rep.line()}")
    for b in rows:
        assert tokens[b, :len(prompts[b])].tolist() == list(prompts[b]), "prompt overwritten"
    passes["sel"] = sel
    return passes


def check_positions(wl, W, tokens, gpu_logits, storage="bf16", stated=BF16_TOL, plain=True):
    """All-positions logits (B, T, V) of a prefill (or a sequence of calls covering every
    position) against the oracle passes over the same tokens (B, T)."""
    passes = {k: oracle_pass(wl, W, tokens, k, storage) for k in ("ref", "alt") + (("plain",) if plain else ())}
    V = gpu_logits.shape[-1]
    return check_logits(gpu_logits.reshape(-1, V), passes["ref"].reshape(-1, V), passes["alt"].reshape(-1, V),
                        passes["plain"].reshape(-1, V) if plain else None, stated)


def verify_fp32_generate(prompts, tokens, call_logits, tf_logits, min_len=None):
    """fp32 models: every call's logits within 1e-4 of the fp64 plain oracle; greedy tokens
    equal wherever the oracle's margin exceeds 0.1."""
    if min_len is None:
        min_len = min(len(p) for p in prompts)
    worst, checked = 0.0, 0
    for i in range(call_logits.shape[0]):
        p = min_len - 1 + i
        g = call_logits[i].astype(np.float64)
        o = tf_logits[:, p].astype(np.float64)
        assert np.isfinite(g).all(), f"non-finite GPU logits at call {i}"
        worst = max(worst, np.abs(g - o).max())
        top, margin = ps.top2(o)
        for b in range(len(prompts)):
            if p + 1 >= len(prompts[b]) and margin[b] > MARGIN:
                assert tokens[b, p + 1] == top[b], f"greedy token differs at row {b} pos {p + 1}"
                checked += 1
    say(f"  max|dlogit|={worst:.3e} greedy tokens checked={checked}")
    assert worst <= FP32_TOL, worst
    for b, p in enumerate(prompts):
        assert tokens[b, :len(p)].tolist() == list(p), "prompt overwritten"
    return worst


# ----------------------------------------------------------------------------- tiny fp32

def test_tiny_fp32_generate_matches_oracle():
    wl = synth.WORKLOADS["tiny_fp32"]
    say(f"case tiny_fp32 generate {wl}")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    a = oracle.args_from_workload(wl)
    tf = oracle.teacher_forced_logits(a, host_weights(wl, W), tokens[:, :-1], np.float64)
    verify_fp32_generate(prompts, tokens, logits, tf)
    # free-running oracle generate gives the same tokens (all margins are checked above)
    ref_tokens, _ = oracle.greedy_generate(oracle.Oracle(a, host_weights(wl, W), wl.batch, np.float64),
                                           prompts, wl.gen_steps)
    assert (ref_tokens == tokens).all()


def test_tiny_fp32_prefill_all_positions_and_chunked():
    wl = synth.WORKLOADS["tiny_fp32"]
    say("case tiny_fp32 prefill all positions, chunked at 10")
    W = synth.gen_weights(wl, device="cuda")
    tok = np.array(synth.prompts(wl), dtype=np.int32)
    B, S = tok.shape
    model = runtime.LlamaModel(args_of(wl), W)
    dtok = torch.from_numpy(tok).cuda()
    full = torch.empty((B, S, wl.vocab_size), device="cuda")
    model.prefill(dtok, B, S, 0, full, all_positions=True)
    a = torch.empty((B, 10, wl.vocab_size), device="cuda")
    b = torch.empty((B, S - 10, wl.vocab_size), device="cuda")
    model.prefill(dtok, B, 10, 0, a, all_positions=True)
    model.prefill(dtok, B, S - 10, 10, b, all_positions=True, col=10)
    last = torch.empty((B, wl.vocab_size), device="cuda")
    model.prefill(dtok, B, S, 0, last)
    torch.cuda.synchronize()
    ref = oracle.Oracle(oracle.args_from_workload(wl), host_weights(wl, W), B, np.float64).forward(tok, 0)
    assert np.abs(full.cpu().numpy() - ref).max() <= FP32_TOL
    chunked = np.concatenate([a.cpu().numpy(), b.cpu().numpy()], 1)
    assert np.abs(chunked - ref).max() <= FP32_TOL
    assert np.abs(last.cpu().numpy() - ref[:, -1]).max() <= FP32_TOL
    model.close()


def test_tiny_fp32_prefill_equals_token_by_token_decode():
    wl = synth.WORKLOADS["tiny_fp32"]
    say("case tiny_fp32 prefill vs decode")
    W = synth.gen_weights(wl, device="cuda")
    tok = torch.tensor(synth.prompts(wl), dtype=torch.int32).cuda()
    B, S = tok.shape
    model = runtime.LlamaModel(args_of(wl), W)
    full = torch.empty((B, S, wl.vocab_size), device="cuda")
    model.prefill(tok, B, S, 0, full, all_positions=True)
    steps = torch.empty((S, B, wl.vocab_size), device="cuda")
    for j in range(S):
        model.decode_step(tok, B, j, j, steps[j])
    torch.cuda.synchronize()
    d = (steps.transpose(0, 1) - full).abs().max().item()
    assert d <= FP32_TOL, d
    model.close()


# ----------------------------------------------------------------------------- small bf16 shapes

SMALL_BF16 = {
    "mha": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_mha", dtype="bf16", n_heads=4,
                                              n_kv_heads=4, dim=512, hidden_dim=1536, vocab_size=1024,
                                              batch=3, prompt_len=0, prompt_len_range=(20, 70),
                                              gen_steps=24, weight_seed=11, prompt_seed=111),
    "gqa8": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_gqa8", dtype="bf16", n_heads=16,
                                               n_kv_heads=2, dim=1024, hidden_dim=2816, vocab_size=2048,
                                               batch=2, prompt_len=0, prompt_len_range=(33, 150),
                                               gen_steps=40, weight_seed=12, prompt_seed=112, max_seq_len=256),
    "hd64": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_hd64", dtype="bf16", n_heads=8,
                                               n_kv_heads=4, dim=512, hidden_dim=1536, vocab_size=1000,
                                               batch=4, prompt_len=17, gen_steps=20, weight_seed=13,
                                               prompt_seed=113),
    # decode batches above 4 take the skinny MFMA products (split over K at these widths):
    # 6 rows (one 16-column tile, rows past the batch clamped) and 32 (two full tiles)
    "b6": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_b6", dtype="bf16", n_heads=16,
                                             n_kv_heads=2, dim=1024, hidden_dim=2816, vocab_size=2048,
                                             batch=6, prompt_len=0, prompt_len_range=(20, 60),
                                             gen_steps=16, weight_seed=15, prompt_seed=115, max_seq_len=128),
    "b32": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_b32", dtype="bf16", n_heads=8,
                                              n_kv_heads=8, dim=1024, hidden_dim=2816, vocab_size=1000,
                                              batch=32, prompt_len=0, prompt_len_range=(12, 40),
                                              gen_steps=12, weight_seed=16, prompt_seed=116, max_seq_len=96),
    # head_dim 32 with GQA 4:1 (prefill on the row attention kernel, decode on the MFMA GQA
    # kernel at its narrowest head) and 17 decode rows: the skinny products' second 16-row tile
    # holds one live row
    "hd32": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_hd32", dtype="bf16", n_heads=8,
                                               n_kv_heads=2, dim=256, hidden_dim=768, vocab_size=512,
                                               batch=17, prompt_len=0, prompt_len_range=(10, 50),
                                               gen_steps=12, weight_seed=18, prompt_seed=118, max_seq_len=96),
    # 20 decode rows at a width where wo and w2 split K in two: the split partials of a second
    # row tile with 4 live rows, added by the RMSNorm that follows
    "b20": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_b20", dtype="bf16", n_heads=8,
                                              n_kv_heads=8, dim=1024, hidden_dim=2816, vocab_size=1000,
                                              batch=20, prompt_len=0, prompt_len_range=(10, 30),
                                              gen_steps=12, weight_seed=21, prompt_seed=121, max_seq_len=64),
    # RoPE base 500000 instead of 10000 (theta is an argument of the ABI, not a constant)
    "theta": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_theta", dtype="bf16", n_heads=8,
                                                n_kv_heads=2, dim=512, hidden_dim=1536, vocab_size=1000,
                                                batch=2, prompt_len=0, prompt_len_range=(40, 180),
                                                gen_steps=20, weight_seed=17, prompt_seed=117,
                                                max_seq_len=256, rope_theta=500000.0),
    # widths that are not whole 128-column tiles: dim 576 (9 heads of 64), so q/k/v (1728 rows)
    # and wo / w2 (576) end in half tiles of the 128 x 128 short-prefill kernel, and the
    # 80..126 prompt rows a partial 128-row tile (also the first, partial, query tile of the
    # attention)
    "ragged_n": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_ragged_n", dtype="bf16", n_heads=9,
                                                   n_kv_heads=9, dim=576, hidden_dim=1600, vocab_size=1000,
                                                   batch=2, prompt_len=0, prompt_len_range=(40, 63),
                                                   gen_steps=16, weight_seed=24, prompt_seed=124, max_seq_len=128),
    # long prompts: 4 x 600 = 2400 prefill rows take the 256x256 GEMM path (ragged tiles)
    # with its fused RoPE / cache-append epilogue
    "long": synth.WORKLOADS["tiny_fp32"].with_(name="small_bf16_long", dtype="bf16", n_heads=4,
                                               n_kv_heads=4, dim=512, hidden_dim=1536, vocab_size=1024,
                                               batch=4, prompt_len=600, gen_steps=6, weight_seed=14,
                                               prompt_seed=114, max_seq_len=640),
}


# ----------------------------------------------------------------------------- fp16 models

# fp16 (the reference's dtype) takes the same kernels as bf16 (vector path at decode batch <= 4,
# skinny MFMA products at 5..32 rows, MFMA GEMMs for prefill and above 32 rows; only the GQA
# decode attention stays on the vector kernel) with every 16-bit storage point rounded to
# binary16.  Its 11 significant bits are 3 more than bf16's, so the bar is the stated bf16 bar
# scaled by the ulp ratio, 2^-3.
FP16_TOL = BF16_TOL / 8

FP16 = {
    "gqa": synth.WORKLOADS["tiny_fp32"].with_(name="tiny_fp16_gqa", dtype="fp16", batch=3,
                                              prompt_len=0, prompt_len_range=(8, 40), gen_steps=16,
                                              weight_seed=19, prompt_seed=119, max_seq_len=96),
    # 6 decode rows on the skinny fp16 MFMA products, MHA with head_dim 64
    "mha_b6": synth.WORKLOADS["tiny_fp32"].with_(name="tiny_fp16_mha_b6", dtype="fp16", n_heads=8,
                                                 n_kv_heads=8, dim=512, hidden_dim=1536, vocab_size=1000,
                                                 batch=6, prompt_len=0, prompt_len_range=(12, 50),
                                                 gen_steps=12, weight_seed=20, prompt_seed=120, max_seq_len=96),
    # 20 decode rows with wo and w2 split over K (the partials of a second, 4-row tile added by
    # the next RMSNorm), GQA 8:1 with head_dim 128 on the vector decode attention
    "b20": synth.WORKLOADS["tiny_fp32"].with_(name="tiny_fp16_b20", dtype="fp16", n_heads=8,
                                              n_kv_heads=1, dim=1024, hidden_dim=2816, vocab_size=1000,
                                              batch=20, prompt_len=0, prompt_len_range=(10, 30),
                                              gen_steps=10, weight_seed=22, prompt_seed=122, max_seq_len=64),
    # 40 decode rows: more than the skinny kernels take, so decode runs the prefill GEMMs with
    # the decode attention (and its key splits merged into fp16 operands)
    "b40": synth.WORKLOADS["tiny_fp32"].with_(name="tiny_fp16_b40", dtype="fp16", n_heads=8,
                                              n_kv_heads=4, dim=512, hidden_dim=1536, vocab_size=1000,
                                              batch=40, prompt_len=0, prompt_len_range=(8, 24),
                                              gen_steps=8, weight_seed=23, prompt_seed=123, max_seq_len=48),
}


@pytest.mark.parametrize("name", list(FP16))
def test_fp16_generate_matches_oracle(name):
    wl = FP16[name]
    say(f"case {wl}")
    W = synth.gen_weights(wl, device="cuda")
    assert W["layers"][0]["wq"].dtype == torch.float16
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    check_generate_rows(wl, W, prompts, tokens, logits, range(len(prompts)), storage="fp16", stated=FP16_TOL)


@pytest.mark.timeout(600)
def test_llama2_7b_b1_fp16_generate_matches_oracle():
    """The 7B fp16 workload at full depth in the launch configuration bench.py times: batch 1
    on the vector path (the one-row fp16 GEMV, w2 over three K segments), prefill four rows
    at a time, 128 greedy decode calls."""
    wl = synth.WORKLOADS["llama2_7b_b1_fp16"]
    say(f"case {wl.name}")
    W = synth.gen_weights(wl, device="cuda")
    assert W["layers"][0]["wq"].dtype == torch.float16
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    check_generate_rows(wl, W, prompts, tokens, logits, [0], storage="fp16", stated=FP16_TOL)


@pytest.mark.parametrize("widths,batch", [("llama2_7b_b1_fp16", 2), ("llama2_7b_b1_fp16", 8), ("llama2_13b_b16", 1)])
def test_fp16_full_width_one_layer_generate_matches_oracle(widths, batch):
    """One fp16 layer at full width: 7B at two rows (the two-row GEMV) and at eight (the skinny
    fp16 MFMA products, wo and w2 split over K), 13B at one row (dim 5120 > one 4096-element
    segment: the fused norm's statistics take a pass of their own)."""
    plen, gen = (96, 24) if batch <= 4 else (48, 12)
    wl = synth.WORKLOADS[widths].with_(name=f"{widths}_fp16_one_layer_b{batch}", dtype="fp16", n_layers=1,
                                       batch=batch, prompt_len=plen, gen_steps=gen, prompt_seed=140 + batch)
    say(f"case {wl.name}")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    check_generate_rows(wl, W, prompts, tokens, logits, range(batch), storage="fp16", stated=FP16_TOL)


def test_fp16_prefill_all_positions_chunked_and_decode():
    """Prefill of every position (whole, and in two chunks the second at start_pos > 0)
    against the oracle's fp16-storage forward, and token-by-token decode against prefill."""
    wl = FP16["gqa"]
    say("case tiny_fp16_gqa: prefill all positions, chunked, decode")
    W = synth.gen_weights(wl, device="cuda")
    P = synth.prompts(wl)
    S = min(len(p) for p in P)
    tok = np.array([p[:S] for p in P], dtype=np.int32)
    B = tok.shape[0]
    c = S // 2
    model = runtime.LlamaModel(args_of(wl), W)
    dtok = torch.from_numpy(tok).cuda()
    full = torch.empty((B, S, wl.vocab_size), device="cuda")
    model.prefill(dtok, B, S, 0, full, all_positions=True)
    a = torch.empty((B, c, wl.vocab_size), device="cuda")
    b = torch.empty((B, S - c, wl.vocab_size), device="cuda")
    model.prefill(dtok, B, c, 0, a, all_positions=True)
    model.prefill(dtok, B, S - c, c, b, all_positions=True, col=c)
    steps = torch.empty((S, B, wl.vocab_size), device="cuda")
    for j in range(S):
        model.decode_step(dtok, B, j, j, steps[j])
    torch.cuda.synchronize()
    ref = oracle.Oracle(oracle.args_from_workload(wl), host_weights(wl, W), B, np.float32,
                        storage="fp16").forward(tok, 0)
    d_full = np.abs(full.cpu().numpy() - ref).max()
    d_chunk = np.abs(np.concatenate([a.cpu().numpy(), b.cpu().numpy()], 1) - ref).max()
    d_dec = (steps.transpose(0, 1) - full).abs().max().item()
    say(f"  max|dlogit| prefill {d_full:.3e} chunked {d_chunk:.3e} decode-vs-prefill {d_dec:.3e}")
    assert d_full <= FP16_TOL and d_chunk <= FP16_TOL and d_dec <= FP16_TOL
    model.close()


@pytest.mark.parametrize("name", list(SMALL_BF16))
def test_small_bf16_generate_matches_oracle(name):
    wl = SMALL_BF16[name]
    say(f"case {wl}")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    check_generate_rows(wl, W, prompts, tokens, logits, range(len(prompts)))


def test_small_bf16_cache_filled_to_max_seq_len_with_one_token_prompt():
    """Edge cases of the schedule: one prompt of a single token (the prefill covers one
    position), the others up to 40, and total_len = max_seq_len (the last decode call writes
    and attends to the cache's last position and reads the RoPE table's last row), at a batch
    that takes the skinny decode products."""
    wl = SMALL_BF16["gqa8"].with_(name="small_bf16_edge", batch=8, max_seq_len=64, gen_steps=30,
                                  weight_seed=22, prompt_seed=122)
    rng = np.random.default_rng(122)
    prompts = [[int(rng.integers(3, wl.vocab_size))]] + \
              [rng.integers(3, wl.vocab_size, size=int(n)).tolist() for n in rng.integers(2, 41, size=7)]
    total_len = min(wl.max_seq_len, wl.gen_steps + max(len(p) for p in prompts))
    assert total_len == wl.max_seq_len
    say(f"case {wl.name}: prompt lengths {[len(p) for p in prompts]}, total_len {total_len}")
    W = synth.gen_weights(wl, device="cuda")
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    assert tokens.shape[1] == wl.max_seq_len and logits.shape[0] == wl.max_seq_len - 1
    check_generate_rows(wl, W, prompts, tokens, logits, range(len(prompts)))


def test_small_bf16_prefill_equals_token_by_token_decode():
    wl = SMALL_BF16["gqa8"]
    say("case small bf16 gqa8: prefill (MFMA path) vs decode (GEMV path)")
    W = synth.gen_weights(wl, device="cuda")
    tok = torch.tensor([p[:33] for p in synth.prompts(wl)], dtype=torch.int32).cuda()
    B, S = tok.shape
    model = runtime.LlamaModel(args_of(wl), W)
    full = torch.empty((B, S, wl.vocab_size), device="cuda")
    model.prefill(tok, B, S, 0, full, all_positions=True)
    steps = torch.empty((S, B, wl.vocab_size), device="cuda")
    for j in range(S):
        model.decode_step(tok, B, j, j, steps[j])
    torch.cuda.synchronize()
    d = (steps.transpose(0, 1) - full).abs().max().item()
    say(f"  max|prefill - decode| = {d:.3e}")
    assert d <= BF16_TOL, d
    model.close()


@pytest.mark.parametrize("name", ["gqa8", "mha", "theta", "hd32"])
def test_small_bf16_chunked_prefill_all_positions(name):
    """Prefill in two chunks (the second at start_pos > 0, ragged against the 64-row tiles)
    against the oracle's full forward, every position."""
    wl = SMALL_BF16[name]
    say(f"case {wl.name}: chunked prefill")
    W = synth.gen_weights(wl, device="cuda")
    P = synth.prompts(wl)
    S = min(len(p) for p in P)
    tok = np.array([p[:S] for p in P], dtype=np.int32)
    B = tok.shape[0]
    c = min(37, S - 7)
    model = runtime.LlamaModel(args_of(wl), W)
    dtok = torch.from_numpy(tok).cuda()
    a = torch.empty((B, c, wl.vocab_size), device="cuda")
    b = torch.empty((B, S - c, wl.vocab_size), device="cuda")
    model.prefill(dtok, B, c, 0, a, all_positions=True)
    model.prefill(dtok, B, S - c, c, b, all_positions=True, col=c)
    torch.cuda.synchronize()
    got = np.concatenate([a.cpu().numpy(), b.cpu().numpy()], 1)
    model.close()
    check_positions(wl, W, tok, got)


@pytest.mark.timeout(600)
def test_llama2_7b_widths_one_layer_chunked_prefill_all_positions():
    """Chunked prefill at the 7B widths: 3 x 1536 tokens in a chunk of 1024 (3072 rows: the
    256x256 GEMM) and a chunk of 512 at start_pos 1024 (flash attention over a cached prefix
    twice the chunk), every position against the oracle's full forward (one layer: 3e-2)."""
    wl = synth.WORKLOADS["llama2_7b_b1"].with_(name="llama2_7b_chunked_one_layer", n_layers=1, batch=3,
                                               prompt_len=1536, gen_steps=1)
    say(f"case {wl.name}")
    W = synth.gen_weights(wl, device="cuda")
    P = synth.prompts(wl)
    tok = np.array(P, dtype=np.int32)
    B, S = tok.shape
    c = 1024
    model = runtime.LlamaModel(args_of(wl), W)
    dtok = torch.from_numpy(tok).cuda()
    a = torch.empty((B, c, wl.vocab_size), device="cuda")
    b = torch.empty((B, S - c, wl.vocab_size), device="cuda")
    model.prefill(dtok, B, c, 0, a, all_positions=True)
    model.prefill(dtok, B, S - c, c, b, all_positions=True, col=c)
    torch.cuda.synchronize()
    got = np.concatenate([a.cpu().numpy(), b.cpu().numpy()], 1)
    del a, b
    model.close()
    V = wl.vocab_size
    passes = {k: oracle_pass(wl, W, tok, k) for k in ("ref", "alt", "plain")}
    for name, sl in (("first chunk (positions 0-1023)", slice(0, c)), ("second chunk (1024-1535)", slice(c, S))):
        g, r, p = (x[:, sl].reshape(-1, V) for x in (got, passes["ref"], passes["alt"]))
        say(f"  {name}: GPU - ref {ps.distance(g, r).line()}; alt - ref {ps.distance(p, r).line()}")
    check_logits(got.reshape(-1, V), passes["ref"].reshape(-1, V), passes["alt"].reshape(-1, V),
                 passes["plain"].reshape(-1, V))


@pytest.mark.parametrize("name", ["gqa8", "mha", "b6", "b20", "fp16_mha_b6", "fp16_b20", "tiny_fp32"])
def test_decode_graph_replays_match_eager_launches(name):
    """Decode steps replay one captured graph per split count; the generate loop puts eager
    work (argmax, select, step-state writes) between replays.  Every replay's logits must
    equal the eagerly launched step bit for bit (same kernels, same arithmetic).  Cases: bf16
    on the vector and skinny paths (b20: with the wo/w2 K split), fp16 on the skinny path, and
    fp32 models."""
    if name in SMALL_BF16:
        wl = SMALL_BF16[name]
    elif name.startswith("fp16_"):
        wl = FP16[name[len("fp16_"):]]
    else:
        wl = synth.WORKLOADS[name]
    say(f"case {wl.name}: graph replays vs eager launches")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    old = os.environ.get("LLAMA_MI355X_GRAPHS")
    try:
        os.environ["LLAMA_MI355X_GRAPHS"] = "0"
        t_eager, l_eager, _ = gpu_generate(wl, W, prompts)
        os.environ["LLAMA_MI355X_GRAPHS"] = "1"
        t_graph, l_graph, _ = gpu_generate(wl, W, prompts)
    finally:
        if old is None:
            os.environ.pop("LLAMA_MI355X_GRAPHS", None)
        else:
            os.environ["LLAMA_MI355X_GRAPHS"] = old
    assert np.array_equal(t_eager, t_graph)
    assert np.array_equal(l_eager, l_graph), np.abs(l_eager - l_graph).max()
    say(f"  {l_graph.shape[0] - 1} graph replays identical to eager launches")


def test_generator_bit_identical_on_gpu_and_cpu():
    wl = synth.WORKLOADS["llama2_7b_b1"]
    g = synth.gen_tensor(wl, "w2", 7, device="cuda").cpu()
    c = synth.gen_tensor(wl, "w2", 7, device="cpu")
    assert torch.equal(g, c)


# ----------------------------------------------------------------------------- argmax / select

def test_argmax_ties_nan_and_select():
    say("case argmax/select")
    V = 32000
    x = torch.randn(5, V + 7, device="cuda")
    x[0, 100] = 50.0
    x[0, 9000] = 50.0                     # tie -> lowest index
    x[1, :] = -1.0                        # all equal -> 0
    x[2, 5] = float("nan")
    x[2, 31999] = 99.0
    x[3, 0] = float("inf")
    out = torch.full((5,), -7, dtype=torch.int32, device="cuda")
    runtime.check("argmax", abi.llama_argmax(x.data_ptr(), 5, V, x.stride(0), out.data_ptr(),
                                             runtime.stream_handle()))
    torch.cuda.synchronize()
    xs = x[:, :V].cpu().numpy()
    got = out.cpu().numpy()
    assert got[0] == 100 and got[1] == 0 and got[2] == 31999 and got[3] == 0
    assert got[4] == int(np.argmax(xs[4]))
    tokens = torch.arange(12, dtype=torch.int32, device="cuda").view(3, 4).contiguous()
    plen = torch.tensor([2, 3, 4], dtype=torch.int32, device="cuda")
    nxt = torch.tensor([70, 71, 72], dtype=torch.int32, device="cuda")
    runtime.select_next(nxt, tokens, 2, plen)
    torch.cuda.synchronize()
    assert tokens.cpu().tolist() == [[0, 1, 70, 3], [4, 5, 6, 7], [8, 9, 10, 11]]


# ----------------------------------------------------------------------------- 7B shape, batch 1

@pytest.mark.timeout(600)
def test_llama2_7b_widths_one_layer_generate_matches_oracle():
    base = synth.WORKLOADS["llama2_7b_b1"]
    wl = base.with_(n_layers=1)
    say(f"case llama2_7b_b1 widths, 1 layer")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    check_generate_rows(wl, W, prompts, tokens, logits, [0])


@pytest.mark.timeout(600)
def test_llama2_7b_widths_one_layer_tail_rows_match_oracle():
    """33 x 256 prefill rows at the 7B widths: the 256x256 tiles of the first 8192 rows fill
    whole rounds of one tile per CU, so the last 256 rows of every projection (q/k/v with
    RoPE and the cache append, wo and w2 with the residual add, the SiLU gate) run on the
    split-K path with its reduce passes (a product launched in two row ranges adds its results
    itself rather than leaving partials for the next norm).  The first and the last batch row
    (all of whose prompt rows are in that tail) are checked against the oracle."""
    wl = synth.WORKLOADS["llama2_7b_b1"].with_(name="llama2_7b_b33_one_layer", n_layers=1, batch=33,
                                               prompt_len=256, gen_steps=4)
    say(f"case {wl.name}")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    assert len(prompts) * min(len(p) for p in prompts) == 33 * 256
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    check_generate_rows(wl, W, prompts, tokens, logits, [0, 32])


@pytest.mark.timeout(600)
def test_llama2_7b_widths_one_layer_128_row_tail_matches_oracle():
    """65 x 128 prefill rows at the 7B widths: after 32 whole rounds of 256-row tiles, the last
    128 rows of every projection run as a second launch on the 128 x 128 short-prefill tile
    (row offset into the q / cache rows, the residual and the gated output; q/k/v and wo / w2
    split over K with their reduce passes, the gate unsplit).  The first row and the last
    (whose whole prompt is in that tail) are checked against the oracle."""
    wl = synth.WORKLOADS["llama2_7b_b1"].with_(name="llama2_7b_b65_one_layer", n_layers=1, batch=65,
                                               prompt_len=128, gen_steps=4)
    say(f"case {wl.name}")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    assert len(prompts) * min(len(p) for p in prompts) == 65 * 128
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    check_generate_rows(wl, W, prompts, tokens, logits, [0, 64])


@pytest.mark.timeout(900)
def test_llama2_7b_b1_generate_matches_oracle():
    """The 7B batch-1 workload at full depth, in the launch configuration bench.py times.
    Besides the checks of every depth case, this measures the floor the bf16 format sets
    against the plain fp32 oracle on the same tokens: rounding only the K/V cache (the
    layout the method fixes) already moves single logits by more than three times the
    stated 3e-2, and the full bf16-storage method sits below the stated cosine."""
    wl = synth.WORKLOADS["llama2_7b_b1"]
    say(f"case {wl.name}: generating weights")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    say("  gpu generate")
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    passes = check_generate_rows(wl, W, prompts, tokens, logits, [0], extra_kinds=("kv",))
    sel = passes["sel"]
    kv = ps.distance(passes["kv"][0, sel], passes["plain"][0, sel])
    st = ps.distance(passes["ref"][0, sel], passes["plain"][0, sel])
    say(f"  floor: K/V cache alone in bf16 - plain: {kv.line()}")
    say(f"  floor: bf16 storage - plain:            {st.line()}")
    assert kv.max_all > 3 * BF16_TOL
    assert st.cos.min() < COS_MIN and st.rms_all > kv.rms_all


# ----------------------------------------------------------------------------- other workloads
#
# The oracle's cost grows with batch x depth x length, so the larger workloads are checked
# on sampled rows: the GPU runs the whole batch (the launch configuration of a real
# generate), the oracle follows selected rows teacher-forced.  Batch rows are independent in
# the forward (no cross-row term), so a row subset is exact for those rows.

@pytest.mark.timeout(900)
def test_llama2_7b_b32_ragged_generate_rows_match_oracle():
    """Full batch, ragged prompts, full depth; the oracle follows the first and last row of
    each of the skinny decode products' two 16-row tiles."""
    wl = synth.WORKLOADS["llama2_7b_b32_ragged"]
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    lens = [len(p) for p in prompts]
    rows = [0, 15, 16, 31]
    say(f"case {wl.name}: full batch, ragged prompts {min(lens)}-{max(lens)}, full depth; oracle rows {rows}")
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    assert np.isfinite(logits).all()
    check_generate_rows(wl, W, prompts, tokens, logits, rows)


@pytest.mark.timeout(900)
def test_llama2_13b_b16_generate_rows_match_oracle():
    """The 13B workload at full depth (40 layers), full batch and prompt, full generate; the
    oracle follows the first and the last row."""
    wl = synth.WORKLOADS["llama2_13b_b16"]
    say(f"case {wl.name}: full batch {wl.batch} x {wl.prompt_len}, {wl.gen_steps} steps, full depth")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    assert np.isfinite(logits).all()
    check_generate_rows(wl, W, prompts, tokens, logits, [0, wl.batch - 1], plain=False)


@pytest.mark.timeout(900)
def test_llama2_70b_b8_full_depth_prefix_rows_match_oracle():
    """The 70B workload (GQA 8:1) at full depth (80 layers), full batch of 8, on a causal
    prefix: a 512-token prefill with every position's logits, then 16 single-token decode
    calls feeding the prompt's next tokens (the skinny decode products and the MFMA GQA
    decode attention over 513-528 keys).  By the causal mask the logits of these positions
    are those of the full-length run's; the oracle follows rows 0 and 7."""
    wl = synth.WORKLOADS["llama2_70b_b8"]
    n_pre, n_dec = 512, 16
    say(f"case {wl.name}: full depth, batch {wl.batch}, {n_pre}-token prefix + {n_dec} decode calls")
    W = synth.gen_weights(wl, device="cuda")
    tok = np.array([p[:n_pre + n_dec] for p in synth.prompts(wl)], dtype=np.int32)
    B, V = wl.batch, wl.vocab_size
    model = runtime.LlamaModel(args_of(wl), W)
    dtok = torch.from_numpy(tok).cuda()
    pre = torch.empty((B, n_pre, V), device="cuda")
    model.prefill(dtok, B, n_pre, 0, pre, all_positions=True)
    dec = torch.empty((n_dec, B, V), device="cuda")
    for j in range(n_dec):
        model.decode_step(dtok, B, n_pre + j, n_pre + j, dec[j])
    torch.cuda.synchronize()
    rows = [0, B - 1]
    got = np.concatenate([pre.cpu().numpy()[rows], np.transpose(dec.cpu().numpy(), (1, 0, 2))[rows]], 1)
    del pre, dec
    model.close()
    assert np.isfinite(got).all()
    check_positions(wl, W, tok[rows], got, plain=False)


@pytest.mark.timeout(900)
def test_llama2_70b_b8_first_layers_full_length_generate_rows_match_oracle():
    """The 70B workload cut to its first 2 layers at full width: the whole batch, the whole
    3584-token prompts and all 512 greedy decode calls (the cache filled to max_seq_len);
    the oracle follows rows 0 and 7."""
    wl = synth.WORKLOADS["llama2_70b_b8"].with_(n_layers=2)
    say(f"case {wl.name} cut to 2 layers: full batch {wl.batch} x {wl.prompt_len}, {wl.gen_steps} steps")
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    tokens, logits, _ = gpu_generate(wl, W, prompts)
    assert np.isfinite(logits).all()
    check_generate_rows(wl, W, prompts, tokens, logits, [0, wl.batch - 1])


# ----------------------------------------------------------------------------- sampling

def _draw_ok(logits64, temperature, top_p, u, tok, tol):
    """The GPU's draw equals the oracle's for top_p and u each moved by at most tol (the GPU
    sums in fp32, so a draw point or cutoff within ~1e-6 of a boundary may fall either way)."""
    for dp in (0.0, -tol, tol):
        for du in (0.0, -tol, tol):
            uu = np.clip(np.array([u + du]), 0.0, 1.0 - 1e-12)
            if oracle.sample_top_p(logits64[None], temperature, max(0.0, top_p + dp), uu)[0][0] == tok:
                return True
    return False


@pytest.mark.parametrize("vocab", [7, 1000, 32000])
def test_sample_top_p_matches_oracle(vocab):
    """llama_sample_top_p against the oracle, with the same uniforms.  Logits are a shuffled
    evenly spaced grid (no two probabilities within fp32 rounding of each other), plus a row
    of exactly equal logits (ties sort by index) and a row with one dominant token."""
    rng = np.random.default_rng(60 + vocab)
    B = 16
    grid = np.linspace(-6.0, 6.0, vocab)
    logits = np.stack([rng.permutation(grid) for _ in range(B)]).astype(np.float32)
    logits[0, :] = 0.5
    logits[1, rng.integers(vocab)] = 40.0
    L = torch.from_numpy(logits).cuda()
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    n_exact = n_near = 0
    for temperature, top_p in [(1.0, 0.9), (0.7, 0.5), (1.5, 1.0), (1.0, 0.0), (2.0, 0.95), (0.3, 0.99)]:
        u = rng.random(B).astype(np.float32)
        U = torch.from_numpy(u).cuda()
        runtime.sample_top_p(L, temperature, top_p, U, out, lp)
        torch.cuda.synchronize()
        g_tok, g_lp = out.cpu().numpy(), lp.cpu().numpy()
        r_tok, r_lp = oracle.sample_top_p(logits.astype(np.float64), temperature, top_p, u.astype(np.float64))
        for b in range(B):
            if g_tok[b] == r_tok[b]:
                n_exact += 1
            else:
                assert _draw_ok(logits[b].astype(np.float64), temperature, top_p, float(u[b]), g_tok[b], 2e-5), \
                    (temperature, top_p, b, g_tok[b], r_tok[b])
                n_near += 1
            assert abs(g_lp[b] - r_lp[b]) <= 1e-4 * max(1.0, abs(r_lp[b])), (b, g_lp[b], r_lp[b])
        if top_p == 0.0:
            assert (g_tok == np.argmax(logits, -1)).all()
    say(f"  vocab {vocab}: {n_exact} draws equal to the oracle's, {n_near} at a boundary within 2e-5")
    # every other draw was checked above; fp32 sums over up to 32768 terms put a few draws
    # per hundred within 2e-5 of a boundary when single probabilities are ~1e-4
    assert n_near <= 0.1 * (n_exact + n_near)


def test_sample_top_p_timing_and_errors():
    B, V = 32, 32000
    rng = np.random.default_rng(5)
    L = torch.from_numpy(rng.normal(0.0, 3.0, size=(B, V)).astype(np.float32)).cuda()
    U = torch.from_numpy(rng.random(B).astype(np.float32)).cuda()
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    for _ in range(3):
        runtime.sample_top_p(L, 0.8, 0.9, U, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        runtime.sample_top_p(L, 0.8, 0.9, U, out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 20 * 1e3
    import time
    host = L.cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    oracle.sample_top_p(host, 0.8, 0.9, U.cpu().numpy().astype(np.float64))
    ms_oracle = (time.perf_counter() - t0) * 1e3
    say(f"  llama_sample_top_p {B} x {V}: {us:.1f} us per call; oracle (fp64 NumPy, one host thread "
        f"for the sorts): {ms_oracle:.1f} ms")
    s = runtime.stream_handle()
    p = L.data_ptr()
    assert abi.llama_sample_top_p(p, B, V, V, 0.0, 0.9, U.data_ptr(), out.data_ptr(), 0, s) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_sample_top_p(p, B, V, V, 0.8, -0.1, U.data_ptr(), out.data_ptr(), 0, s) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_sample_top_p(p, B, V, V - 1, 0.8, 0.9, U.data_ptr(), out.data_ptr(), 0, s) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_sample_top_p(p, B, V, V, 0.8, 0.9, 0, out.data_ptr(), 0, s) == abi.LLAMA_ERR_INVALID_ARG
    assert abi.llama_sample_top_p(p, 1, 40000, 40000, 0.8, 0.9, U.data_ptr(), out.data_ptr(), 0, s) == \
        abi.LLAMA_ERR_UNSUPPORTED


def test_tiny_fp32_sampled_generate_matches_oracle():
    """Generate with temperature 0.8 and top_p 0.9 on the tiny workload: every drawn token is
    the oracle's draw (teacher-forced logits on the GPU's tokens, the same uniforms), up to
    boundary cases within the fp32 logit tolerance; log-probs agree."""
    wl = synth.WORKLOADS["tiny_fp32"]
    W = synth.gen_weights(wl, device="cuda")
    prompts = synth.prompts(wl)
    model = runtime.LlamaModel(args_of(wl, len(prompts)), W)
    run = runtime.GreedyRun(model, prompts, wl.gen_steps, temperature=0.8, top_p=0.9, seed=11)
    run.run()
    torch.cuda.synchronize()
    tokens = run.tokens.cpu().numpy().astype(np.int64)
    u = run.uniforms.cpu().numpy().astype(np.float64)
    g_lp = run.logprobs.cpu().numpy()
    model.close()
    a = oracle.args_from_workload(wl)
    tf = oracle.teacher_forced_logits(a, host_weights(wl, W), tokens[:, :-1], np.float64)
    min_len = min(len(p) for p in prompts)
    checked = near = 0
    for i in range(run.n_calls):
        pos = min_len - 1 + i
        for b in range(len(prompts)):
            if pos + 1 < len(prompts[b]):
                continue
            tok = tokens[b, pos + 1]
            r_tok, r_lp = oracle.sample_top_p(tf[b, pos][None], 0.8, 0.9, u[i, b:b + 1])
            if r_tok[0] != tok:
                assert _draw_ok(tf[b, pos], 0.8, 0.9, u[i, b], tok, 1e-3), (i, b)
                near += 1
            assert abs(g_lp[i, b] - r_lp[0]) <= 1e-3, (i, b, g_lp[i, b], r_lp[0])
            checked += 1
    say(f"  sampled tokens checked={checked} (at a boundary: {near})")
    assert checked > 0 and near <= 2
    for b, p in enumerate(prompts):
        assert tokens[b, :len(p)].tolist() == list(p)

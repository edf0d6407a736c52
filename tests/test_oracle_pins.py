"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test pins one part of oracle/llama.py against a closed form, an invariant the pages
state, a library routine the special case reduces to (torch / scipy CPU ops), or a number
the pages print (tests/golden/pages_worked_examples.json).  Together they are meant to make
a plausible slip anywhere in the oracle fail: a dropped eps or residual, a wrong RoPE sign
or pairing, a wrong attention scale, mask offset or GQA head map, swapped or transposed
weights, a wrong SiLU.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import ModelArgs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.json")


def small_args(**kw):
    base = dict(dim=64, n_layers=2, n_heads=4, n_kv_heads=2, vocab_size=97,
                hidden_dim=oracle.ffn_hidden_dim(64), norm_eps=1e-5, rope_theta=10000.0,
                max_seq_len=40)
    base.update(kw)
    return ModelArgs(**base)


def random_weights(a: ModelArgs, seed=0, scale=0.08, dtype=np.float64):
    rng = np.random.default_rng(seed)
    hd = a.head_dim

    def m(r, c):
        return (rng.standard_normal((r, c)) * scale).astype(dtype)

    def v(n):
        return (1.0 + 0.1 * rng.standard_normal(n)).astype(dtype)
    layers = []
    for _ in range(a.n_layers):
        layers.append(dict(attention_norm=v(a.dim), wq=m(a.n_heads * hd, a.dim),
                           wk=m(a.kv_heads * hd, a.dim), wv=m(a.kv_heads * hd, a.dim),
                           wo=m(a.dim, a.n_heads * hd), ffn_norm=v(a.dim),
                           w1=m(a.hidden_dim, a.dim), w2=m(a.dim, a.hidden_dim),
                           w3=m(a.hidden_dim, a.dim)))
    return dict(tok_embeddings=m(a.vocab_size, a.dim) * 10, norm=v(a.dim),
                output=m(a.vocab_size, a.dim), layers=layers)


# ----------------------------------------------------------------------------- pages' numbers

def test_ffn_hidden_rule_matches_pages_cases():
    g = json.load(open(GOLDEN))["ffn_hidden_rule"]
    for case in g["cases"]:
        assert oracle.ffn_hidden_dim(case["dim"]) == case["hidden"]
    # the rule rounds up, never down, and lands on the multiple
    for dim in (100, 333, 4096, 8192):
        h = oracle.ffn_hidden_dim(dim, multiple_of=256)
        assert h % 256 == 0 and h >= int(8 * dim / 3) and h - int(8 * dim / 3) < 256


def test_kv_cache_footprint_worked_example():
    g = json.load(open(GOLDEN))["kv_cache_7b_example"]
    per = oracle.kv_cache_bytes(g["max_batch_size"], g["max_seq_len"], g["n_kv_heads"],
                                g["head_dim"], g["bytes_per_element"])
    assert per == 64 * 2 ** 20
    assert abs(per - g["per_tensor_per_layer_bytes_approx"]) / per < 0.05
    total = per * g["n_layers"] * 2
    assert total == 4 * 2 ** 30
    assert abs(total - g["total_k_and_v_bytes_approx"]) / total < 0.08


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    eps = 1e-5
    for c in (1e-3, 0.5, 3.0, -2.0):
        x = np.full((3, 16), c, dtype=np.float64)
        w = np.linspace(0.5, 1.5, 16)
        y = oracle.rms_norm(x, w, eps)
        np.testing.assert_allclose(y, np.broadcast_to(c / math.sqrt(c * c + eps) * w, y.shape), rtol=1e-14)


def test_rmsnorm_matches_torch_library():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 48))
    w = rng.standard_normal(48)
    ref = F.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-5), ref, rtol=1e-12, atol=1e-14)


def test_rmsnorm_fp32_mean_is_the_correctly_rounded_mean():
    """In float32 the mean of squares is the correctly rounded one (math.fsum of the exact
    squares), so the result does not depend on the order of the row's elements."""
    rng = np.random.default_rng(8)
    eps = 1e-5
    for n in (4096, 5120, 768):
        x = (rng.standard_normal((64, n)) * 0.02).astype(np.float32)
        got = oracle.rms_norm(x, np.float32(1.0), eps)
        for r in range(x.shape[0]):
            sq = [float(v) * float(v) for v in x[r]]          # exact in binary64
            ms = np.float32(math.fsum(sq) / n)
            np.testing.assert_array_equal(got[r], x[r] / np.sqrt(ms + np.float32(eps)))
        perm = rng.permutation(n)
        np.testing.assert_array_equal(oracle.rms_norm(x[:, perm], np.float32(1.0), eps), got[:, perm])


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 64))
    ones = np.ones(64)
    y = oracle.rms_norm(x, ones, 0.0)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, ones, 0.0), y, rtol=1e-13)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)


# ----------------------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    x = np.random.default_rng(3).standard_normal((2, 1, 3, 16))
    np.testing.assert_array_equal(oracle.apply_rope(x, [0], 10000.0), x)


def test_rope_head_dim_2_is_plane_rotation_by_t():
    x = np.random.default_rng(4).standard_normal((1, 5, 1, 2))
    pos = [0, 1, 2, 7, 100]
    y = oracle.apply_rope(x, pos, 10000.0)
    for s, t in enumerate(pos):
        z = complex(x[0, s, 0, 0], x[0, s, 0, 1]) * complex(math.cos(t), math.sin(t))
        assert abs(y[0, s, 0, 0] - z.real) < 1e-12 and abs(y[0, s, 0, 1] - z.imag) < 1e-12


def test_rope_is_complex_multiplication_of_adjacent_pairs():
    """The pages: view q, k as pairs of reals, multiply as complex numbers by e^{i t f}."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 6, 3, 32))
    pos = list(range(9, 15))
    ang = torch.from_numpy(oracle.rope_angles(32, pos, 10000.0))
    table = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]
    xc = torch.view_as_complex(torch.from_numpy(x).reshape(2, 6, 3, 16, 2).contiguous())
    ref = torch.view_as_real(xc * table).reshape(2, 6, 3, 32).numpy()
    np.testing.assert_allclose(oracle.apply_rope(x, pos, 10000.0), ref, atol=1e-13)


def test_rope_preserves_norms_and_dot_depends_on_offset_only():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 1, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    for t in (0, 5, 3000):
        qr = oracle.apply_rope(q, [t], 10000.0)
        pair_norm = np.hypot(qr[..., 0::2], qr[..., 1::2])
        np.testing.assert_allclose(pair_norm, np.hypot(q[..., 0::2], q[..., 1::2]), rtol=1e-12)
    d = []
    for shift in (0, 17, 1000):
        a = oracle.apply_rope(q, [10 + shift], 10000.0)
        b = oracle.apply_rope(k, [3 + shift], 10000.0)
        d.append(float(np.sum(a * b)))
    np.testing.assert_allclose(d, d[0], rtol=1e-9)
    # and it does depend on the offset
    e = float(np.sum(oracle.apply_rope(q, [11], 10000.0) * oracle.apply_rope(k, [3], 10000.0)))
    assert abs(e - d[0]) > 1e-6


@pytest.mark.parametrize("hd,theta", [(32, 10000.0), (64, 10000.0), (128, 10000.0), (128, 500000.0)])
def test_rope_schedule_matches_transformers_llama_rotary_embedding(hd, theta):
    """Reading R1 (pair i of a head turns at theta^(-2i/head_dim)) against an independent
    implementation of the same model family: transformers' LlamaRotaryEmbedding and
    apply_rotary_pos_emb.  That implementation pairs element i with element i + head_dim/2
    ("rotate half") where the pages pair adjacent elements (2i, 2i+1), so a head is compared
    through the permutation that maps adjacent pair i to (i, i + head_dim/2).  Its tables are
    fp32 (the frequencies, then angles t * f rounded once), hence the tolerances."""
    transformers = pytest.importorskip("transformers")
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    cfg = transformers.LlamaConfig(hidden_size=4 * hd, num_attention_heads=4, rope_theta=theta,
                                   max_position_embeddings=4096)
    emb = LlamaRotaryEmbedding(config=cfg)
    # the frequency schedule itself
    np.testing.assert_allclose(emb.inv_freq.double().numpy(), oracle.rope_frequencies(hd, theta), rtol=2e-7)
    # the rotation of whole heads at a few positions
    rng = np.random.default_rng(hd)
    pos = np.array([0, 1, 2, 5, 17, 64, 100])
    x = rng.standard_normal((1, len(pos), 3, hd))                    # (B, S, H, hd), adjacent pairs
    perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])
    xt = torch.from_numpy(x[..., perm]).float().transpose(1, 2)      # (B, H, S, hd), rotate-half layout
    cos, sin = emb(xt, torch.from_numpy(pos)[None])
    q, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    y_lib = q.transpose(1, 2).double().numpy()
    y = oracle.apply_rope(x, pos, theta)[..., perm]
    np.testing.assert_allclose(y, y_lib, atol=1e-4, rtol=1e-4)
    # a sign slip or a pairing slip would be far outside that: the other rotation direction
    y_wrong = oracle.apply_rope(x, -pos, theta)[..., perm]
    assert np.abs(y_wrong - y_lib).max() > 0.1


# ----------------------------------------------------------------------------- attention

def _sdpa(q, k, v, start_pos):
    """torch's scaled_dot_product_attention with its repeat-interleave GQA."""
    S, ctx = q.shape[1], k.shape[1]
    allowed = torch.arange(ctx)[None, :] <= (start_pos + torch.arange(S))[:, None]
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3)  # noqa: E731
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=allowed, enable_gqa=True)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("H,KVH,S,start", [(4, 4, 7, 0), (8, 2, 5, 3), (8, 1, 1, 12), (6, 3, 9, 0)])
def test_attention_matches_torch_sdpa(H, KVH, S, start):
    rng = np.random.default_rng(7)
    hd = 16
    q = rng.standard_normal((2, S, H, hd))
    k = rng.standard_normal((2, start + S, KVH, hd))
    v = rng.standard_normal((2, start + S, KVH, hd))
    out = oracle.attention(q, k, v, start, H // KVH)
    np.testing.assert_allclose(out, _sdpa(q, k, v, start), rtol=1e-11, atol=1e-12)


def test_attention_single_visible_key_returns_its_value():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 3, 2, 8))
    k = rng.standard_normal((1, 3, 2, 8))
    v = rng.standard_normal((1, 3, 2, 8))
    out = oracle.attention(q, k, v, 0, 1)
    np.testing.assert_allclose(out[:, 0], v[:, 0], rtol=1e-14)


def test_attention_zero_query_averages_visible_values():
    rng = np.random.default_rng(9)
    S, start = 4, 2
    q = np.zeros((1, S, 2, 8))
    k = rng.standard_normal((1, start + S, 1, 8))
    v = rng.standard_normal((1, start + S, 1, 8))
    out = oracle.attention(q, k, v, start, 2)
    for i in range(S):
        np.testing.assert_allclose(out[0, i, 0], v[0, :start + i + 1, 0].mean(0), rtol=1e-12)


def test_mask_shape_and_entries():
    m = oracle.causal_mask(3, 2)
    assert m.shape == (3, 5)
    assert np.isneginf(m[0, 3]) and m[0, 2] == 0 and m[2, 4] == 0
    assert (m[:, :2] == 0).all()


# ----------------------------------------------------------------------------- SwiGLU

def test_silu_matches_library_routines():
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(oracle.silu(x), x * scipy.special.expit(x), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(oracle.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-12, atol=1e-14)
    assert oracle.silu(np.array([-200.0], dtype=np.float32))[0] == 0.0


def test_feed_forward_gate_zero_and_linear_orientation():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3, 16))
    w1, w3 = rng.standard_normal((24, 16)), rng.standard_normal((24, 16))
    w2 = rng.standard_normal((16, 24))
    assert np.all(oracle.feed_forward(x, w1, w2, np.zeros_like(w3)) == 0)
    X, W1, W2, W3 = map(torch.from_numpy, (x, w1, w2, w3))
    ref = F.linear(F.silu(F.linear(X, W1)) * F.linear(X, W3), W2).numpy()
    np.testing.assert_allclose(oracle.feed_forward(x, w1, w2, w3), ref, rtol=1e-12)


# ----------------------------------------------------------------------------- whole model

def torch_model_forward(a: ModelArgs, W: dict, tokens: np.ndarray, act=None, kv=None) -> np.ndarray:
    """The pre-norm block of the pages composed from torch library routines (F.embedding,
    F.rms_norm, F.linear, complex RoPE via torch.polar, SDPA with repeat-interleave GQA,
    F.silu), fp64, one causal pass from position 0.

    act / kv: optional storage roundings (numpy functions) applied to the stored activations
    (normalised operands, q after RoPE, attention output, gated FFN activation) and to the
    cached k (after RoPE) and v, the points the 16-bit method stores."""
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))  # noqa: E731
    keep = lambda x: x  # noqa: E731
    ra = (lambda x: torch.from_numpy(act(x.numpy()))) if act else keep  # noqa: E731
    rk = (lambda x: torch.from_numpy(kv(x.numpy()))) if kv else keep  # noqa: E731
    B, S = tokens.shape
    hd = a.head_dim
    freqs = 1.0 / (a.rope_theta ** (torch.arange(0, hd, 2, dtype=torch.float64) / hd))
    ang = torch.outer(torch.arange(S, dtype=torch.float64), freqs)
    cis = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

    def rope(x):
        xc = torch.view_as_complex(x.reshape(*x.shape[:-1], -1, 2).contiguous())
        return torch.view_as_real(xc * cis).reshape(x.shape)
    h = F.embedding(torch.from_numpy(tokens), t(W["tok_embeddings"]))
    for L in W["layers"]:
        x = ra(F.rms_norm(h, (a.dim,), t(L["attention_norm"]), eps=a.norm_eps))
        q = ra(rope(F.linear(x, t(L["wq"])).view(B, S, a.n_heads, hd)))
        k = rk(rope(F.linear(x, t(L["wk"])).view(B, S, a.kv_heads, hd)))
        v = rk(F.linear(x, t(L["wv"])).view(B, S, a.kv_heads, hd))
        o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                           is_causal=True, enable_gqa=True)
        h = h + F.linear(ra(o.transpose(1, 2).reshape(B, S, -1)), t(L["wo"]))
        x = ra(F.rms_norm(h, (a.dim,), t(L["ffn_norm"]), eps=a.norm_eps))
        h = h + F.linear(ra(F.silu(F.linear(x, t(L["w1"]))) * F.linear(x, t(L["w3"]))), t(L["w2"]))
    x = ra(F.rms_norm(h, (a.dim,), t(W["norm"]), eps=a.norm_eps))
    return F.linear(x, t(W["output"])).numpy()


@pytest.mark.parametrize("kvh", [4, 2, 1])
def test_model_matches_torch_library_composition(kvh):
    a = small_args(n_kv_heads=kvh)
    W = random_weights(a, seed=11)
    tokens = np.random.default_rng(12).integers(0, a.vocab_size, size=(2, 9))
    ref = torch_model_forward(a, W, tokens)
    got = oracle.Oracle(a, W, 2, dtype=np.float64).forward(tokens, 0)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(oracle.teacher_forced_logits(a, W, tokens, np.float64), ref,
                               rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("kvh", [4, 2])
def test_model_matches_transformers_llama(kvh):
    """The whole forward against an independent implementation of the same model family:
    transformers' LlamaForCausalLM (eager attention) with the same weights.  Its RoPE pairs
    element i with i + head_dim/2 where the pages pair adjacent elements, so the rows of
    wq and wk are permuted within each head (adjacent pair i -> rows i and i + head_dim/2);
    the scores, and everything after them, are unchanged by that relabelling.  Its RMSNorm
    and RoPE tables run in fp32 whatever the model dtype, hence the tolerance."""
    transformers = pytest.importorskip("transformers")
    a = small_args(n_kv_heads=kvh)
    W = random_weights(a, seed=21)
    hd = a.head_dim
    cfg = transformers.LlamaConfig(vocab_size=a.vocab_size, hidden_size=a.dim, intermediate_size=a.hidden_dim,
                                   num_hidden_layers=a.n_layers, num_attention_heads=a.n_heads,
                                   num_key_value_heads=a.kv_heads, rms_norm_eps=a.norm_eps,
                                   rope_theta=a.rope_theta, max_position_embeddings=64,
                                   tie_word_embeddings=False, attention_bias=False, mlp_bias=False)
    cfg._attn_implementation = "eager"
    model = transformers.LlamaForCausalLM(cfg).double().eval()
    perm_head = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])

    def heads(w, n):   # rows of each head reordered from adjacent pairs to rotate-half
        return np.concatenate([w[h * hd:(h + 1) * hd][perm_head] for h in range(n)])
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))  # noqa: E731
    with torch.no_grad():
        model.model.embed_tokens.weight.copy_(t(W["tok_embeddings"]))
        for L, layer in zip(W["layers"], model.model.layers):
            layer.input_layernorm.weight.copy_(t(L["attention_norm"]))
            layer.self_attn.q_proj.weight.copy_(t(heads(L["wq"], a.n_heads)))
            layer.self_attn.k_proj.weight.copy_(t(heads(L["wk"], a.kv_heads)))
            layer.self_attn.v_proj.weight.copy_(t(L["wv"]))
            layer.self_attn.o_proj.weight.copy_(t(L["wo"]))
            layer.post_attention_layernorm.weight.copy_(t(L["ffn_norm"]))
            layer.mlp.gate_proj.weight.copy_(t(L["w1"]))
            layer.mlp.up_proj.weight.copy_(t(L["w3"]))
            layer.mlp.down_proj.weight.copy_(t(L["w2"]))
        model.model.norm.weight.copy_(t(W["norm"]))
        model.lm_head.weight.copy_(t(W["output"]))
        tokens = np.random.default_rng(22).integers(0, a.vocab_size, size=(2, 11))
        ref = model(torch.from_numpy(tokens)).logits.numpy()
    got = oracle.Oracle(a, W, 2, dtype=np.float64).forward(tokens, 0)
    scale = np.abs(ref).max()
    assert scale > 0.5
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6 * scale)   # measured 1.3e-7 * scale


@pytest.mark.parametrize("storage", ["bf16", "bf16_kv", "fp16"])
def test_storage_modes_round_exactly_at_the_stated_points(storage):
    """The storage modes against the torch composition with the roundings placed by hand at
    the points each mode names (bf16 / fp16: every stored activation and the cache; bf16_kv:
    the cache only).  The rounding functions themselves are pinned against torch's bf16 and
    numpy's float16 conversions below; this pins where they are applied."""
    a = small_args()
    W = random_weights(a, seed=36)
    tokens = np.random.default_rng(37).integers(0, a.vocab_size, size=(2, 11))
    r = oracle.round_fp16 if storage == "fp16" else oracle.round_bf16
    ref = torch_model_forward(a, W, tokens, act=None if storage == "bf16_kv" else r, kv=r)
    got = oracle.Oracle(a, W, 2, dtype=np.float64, storage=storage).forward(tokens, 0)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(oracle.teacher_forced_logits(a, W, tokens, np.float64, storage=storage),
                               ref, rtol=1e-10, atol=1e-10)
    # and the rounding is not a no-op: the plain model differs
    assert np.abs(ref - torch_model_forward(a, W, tokens)).max() > 1e-7


def test_identity_blocks_closed_form():
    """wo = w2 = 0 makes each block the identity: logits = Wout (rmsnorm(E[tok]) * w_norm)."""
    a = small_args()
    W = random_weights(a, seed=13)
    for L in W["layers"]:
        L["wo"][:] = 0
        L["w2"][:] = 0
    tokens = np.array([[3, 50, 7, 7]])
    E, wn, Wout = W["tok_embeddings"], W["norm"], W["output"]
    x = E[tokens]
    expect = (x / np.sqrt(np.mean(x * x, -1, keepdims=True) + a.norm_eps) * wn) @ Wout.T
    got = oracle.Oracle(a, W, 1, dtype=np.float64).forward(tokens, 0)
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_with_repeat_interleaved_kv_weights():
    a = small_args(n_kv_heads=2)
    W = random_weights(a, seed=14)
    m = small_args(n_kv_heads=4)
    Wm = {k: v for k, v in W.items() if k != "layers"}
    Wm["layers"] = []
    hd, n_rep = a.head_dim, a.n_rep
    for L in W["layers"]:
        L2 = dict(L)
        for n in ("wk", "wv"):
            blocks = L[n].reshape(a.kv_heads, hd, a.dim)
            L2[n] = np.repeat(blocks, n_rep, axis=0).reshape(a.n_heads * hd, a.dim)
        Wm["layers"].append(L2)
    tokens = np.random.default_rng(15).integers(0, a.vocab_size, size=(2, 6))
    g = oracle.Oracle(a, W, 2, dtype=np.float64).forward(tokens, 0)
    h = oracle.Oracle(m, Wm, 2, dtype=np.float64).forward(tokens, 0)
    np.testing.assert_allclose(g, h, rtol=1e-12, atol=1e-12)


def test_prefill_equals_incremental_decode_and_chunked_prefill():
    """The mask's (seqlen, start_pos+seqlen) form is what lets the cache stream: the same
    tokens give the same logits whether fed at once, in chunks, or one by one."""
    a = small_args()
    W = random_weights(a, seed=16)
    tokens = np.random.default_rng(17).integers(0, a.vocab_size, size=(2, 12))
    full = oracle.Oracle(a, W, 2, dtype=np.float64).forward(tokens, 0)
    inc = oracle.Oracle(a, W, 2, dtype=np.float64)
    steps = [inc.forward(tokens[:, j:j + 1], j)[:, 0] for j in range(12)]
    np.testing.assert_allclose(np.stack(steps, 1), full, rtol=1e-9, atol=1e-9)
    ch = oracle.Oracle(a, W, 2, dtype=np.float64)
    parts = [ch.forward(tokens[:, 0:5], 0), ch.forward(tokens[:, 5:12], 5)]
    np.testing.assert_allclose(np.concatenate(parts, 1), full, rtol=1e-9, atol=1e-9)


def test_causality_and_batch_row_independence():
    a = small_args()
    W = random_weights(a, seed=18)
    rng = np.random.default_rng(19)
    tokens = rng.integers(0, a.vocab_size, size=(3, 8))
    base = oracle.Oracle(a, W, 3, dtype=np.float64).forward(tokens, 0)
    t2 = tokens.copy()
    t2[:, 5:] = (t2[:, 5:] + 1) % a.vocab_size
    pert = oracle.Oracle(a, W, 3, dtype=np.float64).forward(t2, 0)
    np.testing.assert_allclose(pert[:, :5], base[:, :5], rtol=1e-13, atol=1e-13)
    assert np.abs(pert[:, 5:] - base[:, 5:]).max() > 1e-6
    alone = oracle.Oracle(a, W, 1, dtype=np.float64).forward(tokens[1:2], 0)
    np.testing.assert_allclose(alone[0], base[1], rtol=1e-12, atol=1e-12)


def test_fp32_oracle_close_to_fp64_on_tiny_workload():
    import synth
    wl = synth.WORKLOADS["tiny_fp32"]
    a = oracle.args_from_workload(wl)
    W = synth.gen_weights(wl)
    pr = synth.prompts(wl)
    tokens = np.array(pr)
    l32 = oracle.teacher_forced_logits(a, W, tokens, np.float32)
    l64 = oracle.teacher_forced_logits(a, W, tokens, np.float64)
    assert np.abs(l32 - l64).max() < 1e-5


# ----------------------------------------------------------------------------- greedy / generate

def test_argmax_ties_go_to_lowest_index_and_nan_rejected():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]])
    assert oracle.argmax_lowest(x).tolist() == [1, 0]
    with pytest.raises(ValueError):
        oracle.argmax_lowest(np.array([1.0, np.nan]))


def test_generate_keeps_prompts_and_matches_teacher_forcing():
    a = small_args()
    W = random_weights(a, seed=20)
    prompts = [[5, 9, 11, 2, 40, 41, 42], [7, 8, 9]]
    model = oracle.Oracle(a, W, 2, dtype=np.float64)
    tokens, step_logits = oracle.greedy_generate(model, prompts, max_gen_len=6)
    total = min(a.max_seq_len, 6 + 7)
    assert tokens.shape == (2, total)
    assert tokens[0, :7].tolist() == prompts[0] and tokens[1, :3].tolist() == prompts[1]
    assert len(step_logits) == total - 3
    tf = oracle.teacher_forced_logits(a, W, tokens[:, :-1], np.float64)
    for i, cur in enumerate(range(3, total)):
        np.testing.assert_allclose(step_logits[i], tf[:, cur - 1], rtol=1e-9, atol=1e-9)
        expect = np.argmax(tf[:, cur - 1], -1)
        for b, p in enumerate(prompts):
            if cur >= len(p):
                assert tokens[b, cur] == expect[b]


def test_generate_stops_when_every_row_hit_eos():
    a = small_args()
    W = random_weights(a, seed=21)
    model = oracle.Oracle(a, W, 1, dtype=np.float64)
    tokens, _ = oracle.greedy_generate(model, [[1, 2, 3]], max_gen_len=8)
    first = int(tokens[0, 3])
    model = oracle.Oracle(a, W, 1, dtype=np.float64)
    tokens2, logits2 = oracle.greedy_generate(model, [[1, 2, 3]], max_gen_len=8, eos_id=first)
    assert len(logits2) == 1 and tokens2[0, 3] == first


# ----------------------------------------------------------------------------- bf16 storage mode

def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(30)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # exact ties: values halfway between two bf16 numbers, both parities
    base = torch.tensor(rng.standard_normal(1000), dtype=torch.float32).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1.0, -3.5], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # float64 input: result is a bf16 value within half a bf16 ulp, and idempotent
    y = rng.standard_normal(10000) * 3
    r = oracle.round_bf16(y)
    assert np.array_equal(oracle.round_bf16(r), r)
    assert np.array_equal(r.astype(np.float32), torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).float().numpy())
    m, e = np.frexp(y)
    assert np.all(np.abs(r - y) <= np.ldexp(1.0 / 512, e) * (1 + 1e-12))


def test_working_precision_is_the_dtype_argument_whatever_the_provider_hands_over():
    """A weight callable that returns fp32 arrays must not lower a float64 oracle's precision:
    the result equals the one from float64 arrays of the same values, bit for bit."""
    a = small_args()
    W = random_weights(a, seed=36)
    def getter(dt):
        return lambda n, l: np.asarray(W[n] if l < 0 else W["layers"][l][n], dtype=np.float32).astype(dt)
    tokens = np.random.default_rng(37).integers(0, a.vocab_size, size=(2, 9))
    r32 = oracle.Oracle(a, getter(np.float32), 2, dtype=np.float64).forward(tokens, 0)
    r64 = oracle.Oracle(a, getter(np.float64), 2, dtype=np.float64).forward(tokens, 0)
    assert r32.dtype == np.float64 and np.array_equal(r32, r64)
    t32 = oracle.teacher_forced_logits(a, getter(np.float32), tokens, np.float64)
    t64 = oracle.teacher_forced_logits(a, getter(np.float64), tokens, np.float64)
    assert np.array_equal(t32, t64)
    # and the other way round: a float32 oracle computes in float32 from float64 arrays
    assert oracle.teacher_forced_logits(a, getter(np.float64), tokens, np.float32).dtype == np.float32


def test_round_fp16_matches_numpy_binary16():
    """The binary16 rounding written from the format's definition against numpy's float16
    conversion (a library routine): normals, subnormals, exact ties of both parities,
    overflow to infinity, signed zeros."""
    rng = np.random.default_rng(33)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-22, 12, 200000))).astype(np.float32)
    # exact ties between two binary16 neighbours: a binary16 value plus half its spacing
    h = rng.standard_normal(2000).astype(np.float16)
    h = h[np.isfinite(h) & (h != 0)].astype(np.float64)
    _, e = np.frexp(h)
    spacing = np.where(e < -13, 2.0 ** -24, np.ldexp(1.0, e - 11))
    ties = (h + spacing / 2).astype(np.float32)
    edge = np.array([0.0, -0.0, 1.0, 65504.0, 65519.0, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
                     1.5 * 2.0 ** -24, 2.0 ** -14, 3.0 * 2.0 ** -26], dtype=np.float32)
    x = np.concatenate([x, ties, edge])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float32)
    got = oracle.round_fp16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # worked values: ties to even at 1 + 2^-11 (down to 1) and 1 + 3 * 2^-11 (up to 1 + 2^-9)
    w = oracle.round_fp16(np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65520.0, 0.5 * 2.0 ** -24]))
    assert w[0] == 1.0 and w[1] == 1 + 2.0 ** -9 and np.isinf(w[2]) and w[3] == 0.0


def test_fp16_storage_keeps_prefill_equal_to_decode_and_cache_in_fp16():
    a = small_args()
    W = random_weights(a, seed=34)
    tokens = np.random.default_rng(35).integers(0, a.vocab_size, size=(2, 10))
    full = oracle.Oracle(a, W, 2, dtype=np.float64, storage="fp16")
    lf = full.forward(tokens, 0)
    inc = oracle.Oracle(a, W, 2, dtype=np.float64, storage="fp16")
    steps = np.stack([inc.forward(tokens[:, j:j + 1], j)[:, 0] for j in range(10)], 1)
    np.testing.assert_allclose(steps, lf, rtol=1e-9, atol=1e-9)
    kv = full.cache_k[:, :, :10]
    assert np.array_equal(kv.astype(np.float16).astype(np.float64), kv)
    plain = oracle.Oracle(a, W, 2, dtype=np.float64).forward(tokens, 0)
    bf = oracle.Oracle(a, W, 2, dtype=np.float64, storage="bf16").forward(tokens, 0)
    # binary16 keeps 3 more significant bits than bf16: its rounding moves the logits less
    assert 0 < np.abs(plain - lf).max() < np.abs(plain - bf).max()


def test_bf16_storage_keeps_prefill_equal_to_decode_and_cache_in_bf16():
    a = small_args()
    W = random_weights(a, seed=31)
    tokens = np.random.default_rng(32).integers(0, a.vocab_size, size=(2, 10))
    full = oracle.Oracle(a, W, 2, dtype=np.float64, storage="bf16")
    lf = full.forward(tokens, 0)
    inc = oracle.Oracle(a, W, 2, dtype=np.float64, storage="bf16")
    steps = np.stack([inc.forward(tokens[:, j:j + 1], j)[:, 0] for j in range(10)], 1)
    np.testing.assert_allclose(steps, lf, rtol=1e-9, atol=1e-9)
    kv = full.cache_k[:, :, :10]
    assert np.array_equal(oracle.round_bf16(kv), kv)
    tf = oracle.teacher_forced_logits(a, W, tokens, np.float64, storage="bf16")
    np.testing.assert_allclose(tf, lf, rtol=1e-9, atol=1e-9)
    plain = oracle.Oracle(a, W, 2, dtype=np.float64).forward(tokens, 0)
    d = np.abs(plain - lf).max()
    assert 1e-6 < d < 5e-2     # rounding changes the logits, a little


# ----------------------------------------------------------------------------- sampling
# [AG] 8.5 (temperature > 0 branch), 6.3 and [ST] "Sampling, Stopping, and the Chat Template";
# the cases [AG] 8.9 lists for sample_top_p (greedy threshold, threshold below the largest
# single mass), hand-derived draws on a known distribution, and closed forms.

def test_sample_top_p_known_distribution_hand_derived():
    # p = [0.1, 0.4, 0.2, 0.3]; sorted 0.4 (t1), 0.3 (t3), 0.2 (t2), 0.1 (t0) with mass before
    # 0, 0.4, 0.7, 0.9; top_p = 0.6 keeps t1 and t3, renormalised 4/7 and 3/7
    logits = np.log(np.array([[0.1, 0.4, 0.2, 0.3]]))
    for u, want in [(0.0, 1), (0.5, 1), (4 / 7 - 1e-9, 1), (4 / 7 + 1e-9, 3), (0.999999, 3)]:
        tok, _ = oracle.sample_top_p(logits, 1.0, 0.6, np.array([u]))
        assert tok[0] == want, (u, tok)
    # top_p = 0.75 also keeps t2 (mass before it 0.7 <= 0.75): 4/9, 3/9, 2/9
    for u, want in [(0.44, 1), (0.45, 3), (0.77, 3), (0.78, 2)]:
        tok, _ = oracle.sample_top_p(logits, 1.0, 0.75, np.array([u]))
        assert tok[0] == want, (u, tok)


def test_sample_top_p_threshold_below_largest_mass_and_greedy():
    rng = np.random.default_rng(7)
    logits = rng.normal(0.0, 2.0, size=(6, 50))
    top = np.argmax(logits, axis=-1)
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    for top_p in (0.0, float(p.max(-1).min()) * 0.99):
        for u in (0.0, 0.3, 0.999):
            tok, _ = oracle.sample_top_p(logits, 1.0, top_p, np.full(6, u))
            assert (tok == top).all()


def test_sample_top_p_draw_frequencies_are_the_distribution():
    # evenly spaced u: each token is drawn for a fraction of u equal to its probability
    logits = np.log(np.array([[0.05, 0.25, 0.1, 0.35, 0.25]]))
    n = 20000
    u = (np.arange(n) + 0.5) / n
    toks = np.array([oracle.sample_top_p(logits, 1.0, 1.0, u[i:i + 1])[0][0] for i in range(0, n, 1)])
    freq = np.bincount(toks, minlength=5) / n
    assert np.allclose(freq, [0.05, 0.25, 0.1, 0.35, 0.25], atol=2.0 / n)
    # ties sort by token index: t1 and t4 both 0.25, t1 first (cdf 0.35 -> 0.6 -> 0.85)
    assert oracle.sample_top_p(logits, 1.0, 1.0, np.array([0.61]))[0][0] == 4
    assert oracle.sample_top_p(logits, 1.0, 1.0, np.array([0.59]))[0][0] == 1


def test_sample_top_p_temperature_closed_form_and_logprob():
    p1 = np.array([0.1, 0.4, 0.2, 0.3])
    logits = np.log(p1)[None] + 3.0          # shift: softmax and log_softmax unchanged
    # temperature 2 -> probabilities proportional to sqrt(p1)
    q = np.sqrt(p1) / np.sqrt(p1).sum()
    n = 8000
    u = (np.arange(n) + 0.5) / n
    toks = np.array([oracle.sample_top_p(logits, 2.0, 1.0, u[i:i + 1])[0][0] for i in range(n)])
    assert np.allclose(np.bincount(toks, minlength=4) / n, q, atol=2.0 / n)
    # the log-prob is of the untempered softmax
    tok, lp = oracle.sample_top_p(logits, 2.0, 1.0, np.array([0.0]))
    assert abs(lp[0] - np.log(p1[tok[0]])) < 1e-12


@pytest.mark.parametrize("temperature,top_p", [(0.7, 0.8), (1.0, 0.5), (0.6, 0.95), (1.3, 0.3)])
def test_sample_top_p_distribution_matches_transformers_warpers(temperature, top_p):
    """Readings R20 and R22 (which tokens top-p keeps, the renormalised draw) against an
    independent implementation: transformers' TemperatureLogitsWarper + TopPLogitsWarper.
    The oracle's inverse-CDF draw at the uniforms (k + 1/2) / N, k < N, takes each kept
    token for its share of N within 1, so the draw counts give the renormalised kept
    distribution, which must equal the softmax of the warped logits (tokens the library drops
    never drawn).  Random logits, so no two cumulative masses tie with top_p."""
    transformers = pytest.importorskip("transformers")
    from transformers.generation.logits_process import TemperatureLogitsWarper, TopPLogitsWarper
    rng = np.random.default_rng(int(top_p * 100))
    V, N = 50, 4000
    logits = rng.standard_normal(V)
    warped = TopPLogitsWarper(top_p)(None, TemperatureLogitsWarper(temperature)(None, torch.from_numpy(logits)[None]))
    p_lib = torch.softmax(warped, dim=-1)[0].numpy()
    u = (np.arange(N) + 0.5) / N
    tok, _ = oracle.sample_top_p(np.repeat(logits[None], N, axis=0), temperature, top_p, u)
    freq = np.bincount(tok, minlength=V) / N
    assert set(np.flatnonzero(freq)) <= set(np.flatnonzero(p_lib > 0))
    np.testing.assert_allclose(freq, p_lib, atol=2.0 / N)
    assert 1 < (p_lib > 0).sum() < V     # the case keeps some tokens and drops others

"""Plain, slow, obviously correct CPU reference of the Llama 2 decoder forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg; never by the product path.  NumPy only, no blocking or fusion beyond
what each definition states; default precision float32 (the model's storage precision for
the tiny workload), float64 for self-checks.

Sources (cited by page title and section):
  [AG] "Llama 2 Reference Implementation -- Administrator & Developer Guide"
       section 8.4 "The model architecture in detail", 8.5 "The generation loop in
       detail", 6.2 "KV cache footprint", 3.3 "ModelArgs".
  [ST] the pyshine.com source tour of meta-llama/llama, sections "One model.py, Four
       Ideas" and "Sampling, Stopping, and the Chat Template".

Readings taken where the pages leave a step open:
  R1  RoPE frequency of pair i is theta**(-2i/head_dim)  (the pages fix only theta and
      "one frequency per pair"; pinned against transformers' LlamaRotaryEmbedding, an
      independent implementation of the same model family, in tests/test_oracle_pins.py).
  R2  RoPE pairs are adjacent elements (2i, 2i+1) of each head = (real, imag).
  R4  grouped-query head h reads kv head floor(h / n_rep) (repeat-interleave).
  R5  softmax in the working precision with max subtraction.
  R11 prompts are left-aligned in the token rectangle, pads after (generate's layout).
  R12 total_len = min(max_seq_len, max_gen_len + max_prompt_len).
  R16 argmax ties go to the lowest index.
  R18 storage precision: with storage="bf16" the tensors the bf16 method stores in 16 bits
      -- the normalised GEMM operands, q, the cached k and v, the attention output and the
      gated FFN activation -- are rounded to bf16 (round-to-nearest-even) where they are
      produced; every operation still computes in the working precision.  The pages run
      the reference with 16-bit activations throughout (fp16, [AG] 6.4 and the loader
      description in [ST]); the bf16 method keeps the residual stream and all accumulation
      in fp32 and rounds only at these points.  storage="fp16" rounds at the same points to
      IEEE binary16 (the fp16 model).  storage="bf16_kv" rounds only the cached k and v
      to bf16 (the cache format alone, everything else exact): it measures what the 16-bit
      cache by itself costs.  storage=None is the plain definition.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class ModelArgs:
    """Structural config ([AG] 3.3 and 8.4, ModelArgs).  n_kv_heads=None means n_heads."""
    dim: int
    n_layers: int
    n_heads: int
    vocab_size: int
    hidden_dim: int
    n_kv_heads: Optional[int] = None
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0
    max_seq_len: int = 2048

    @property
    def kv_heads(self) -> int:
        return self.n_heads if self.n_kv_heads is None else self.n_kv_heads

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    @property
    def n_rep(self) -> int:
        return self.n_heads // self.kv_heads


def ffn_hidden_dim(dim: int, multiple_of: int = 256,
                   ffn_dim_multiplier: Optional[float] = None) -> int:
    """SwiGLU hidden size ([AG] 8.4 FeedForward): start from 4*dim, take int(2/3 of it),
    optionally scale by ffn_dim_multiplier, then round up to a multiple of multiple_of."""
    hidden = int(2 * (4 * dim) / 3)
    if ffn_dim_multiplier is not None:
        hidden = int(ffn_dim_multiplier * hidden)
    return multiple_of * ((hidden + multiple_of - 1) // multiple_of)


def kv_cache_bytes(max_batch_size: int, max_seq_len: int, n_kv_heads: int, head_dim: int,
                   bytes_per_element: int) -> int:
    """Size of one cache tensor of one layer ([AG] 6.2): the cache is a dense
    (max_batch_size, max_seq_len, n_kv_heads, head_dim) array allocated up front."""
    return max_batch_size * max_seq_len * n_kv_heads * head_dim * bytes_per_element


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits, ties to even), kept in x's
    dtype.  Written from the format's definition: with x = m * 2^e, 0.5 <= |m| < 1, keep
    m to 8 bits."""
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0) / 256.0, e).astype(x.dtype, copy=False)


def round_fp16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest IEEE binary16 value, kept in x's dtype.  Written from the format's
    definition: 11 significant bits, so with x = m * 2^e (0.5 <= |m| < 1) the spacing is
    2^(e - 11); below 2^-14 (subnormals) the spacing stays 2^-24; ties go to even; a result
    above the largest finite value 65504 is infinity."""
    x64 = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x64)
    q = np.where(e < -13, 2.0 ** -24, np.ldexp(1.0, e - 11))
    r = np.round(x64 / q) * q
    r = np.where(np.abs(r) > 65504.0, np.copysign(np.inf, x64), r)
    return r.astype(np.asarray(x).dtype, copy=False)


def _storage_fns(storage: Optional[str]):
    """(rounding of the activations the method stores in 16 bits, rounding of the cached k
    and v) for a storage mode."""
    keep = lambda x: x  # noqa: E731
    if storage is None:
        return keep, keep
    if storage == "bf16":
        return round_bf16, round_bf16
    if storage == "fp16":
        return round_fp16, round_fp16
    if storage == "bf16_kv":
        return keep, round_bf16
    raise ValueError(storage)


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm ([AG] 8.4 RMSNorm; [ST] RMSNorm): x * rsqrt(mean(x^2) + eps) * weight over
    the last axis.  No mean subtraction, no bias.  The mean of squares is taken in float64
    (every square of a float32 is exact there) and then held in the working precision: in
    float32 it is the correctly rounded mean, which any other summation order reproduces."""
    ms = np.mean(np.square(x, dtype=np.float64), axis=-1, keepdims=True).astype(x.dtype)
    return (x / np.sqrt(ms + x.dtype.type(eps))) * weight


def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """One rotation frequency per pair of a head (reading R1), float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope_angles(head_dim: int, positions: Sequence[int], theta: float) -> np.ndarray:
    """Angle t * freq_i for every position t and pair i ([AG] 8.4 precompute_freqs_cis:
    the table holds e^{i t freq}); float64, shape (len(positions), head_dim // 2)."""
    return np.outer(np.asarray(positions, dtype=np.float64), rope_frequencies(head_dim, theta))


def apply_rope(x: np.ndarray, positions: Sequence[int], theta: float) -> np.ndarray:
    """Rotary embedding ([AG] 8.4 apply_rotary_emb; [ST] "One model.py"): view each head as
    head_dim/2 complex numbers (x[2i] + j x[2i+1]) and multiply the one at position t by
    e^{j t freq_i}.  x has shape (..., S, n_heads, head_dim) with S = len(positions)."""
    ang = rope_angles(x.shape[-1], positions, theta)          # (S, hd/2)
    c = np.cos(ang).astype(x.dtype)[:, None, :]
    s = np.sin(ang).astype(x.dtype)[:, None, :]
    re, im = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


def causal_mask(seqlen: int, start_pos: int, dtype=np.float32) -> np.ndarray:
    """(seqlen, start_pos + seqlen) additive mask ([AG] 8.4 note on the mask): query i sits
    at absolute position start_pos + i and may not see keys after it."""
    q = start_pos + np.arange(seqlen)[:, None]
    k = np.arange(start_pos + seqlen)[None, :]
    m = np.zeros((seqlen, start_pos + seqlen), dtype=dtype)
    m[k > q] = -np.inf
    return m


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """Softmax with max subtraction (reading R5)."""
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, start_pos: int,
              n_rep: int) -> np.ndarray:
    """Causal grouped-query attention ([AG] 8.4 Attention, steps 5-7).

    q: (B, S, H, hd) queries at positions start_pos..start_pos+S-1.
    keys, values: (B, start_pos+S, KVH, hd), the whole visible cache.
    Each kv head serves n_rep consecutive query heads (repeat_kv, reading R4); scores are
    q.k / sqrt(hd) plus the causal mask, softmax over keys, then a weighted sum of values.
    Returns (B, S, H, hd)."""
    B, S, H, hd = q.shape
    kv_of_head = np.arange(H) // n_rep
    k = keys[:, :, kv_of_head, :].transpose(0, 2, 3, 1)        # (B, H, hd, ctx)
    v = values[:, :, kv_of_head, :].transpose(0, 2, 1, 3)      # (B, H, ctx, hd)
    qh = q.transpose(0, 2, 1, 3)                               # (B, H, S, hd)
    scores = np.matmul(qh, k) / q.dtype.type(math.sqrt(hd))
    scores = scores + causal_mask(S, start_pos, q.dtype)
    p = softmax(scores, axis=-1)
    return np.matmul(p, v).transpose(0, 2, 1, 3)


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU: x * sigmoid(x)."""
    with np.errstate(over="ignore"):
        return x / (x.dtype.type(1) + np.exp(-x))


def feed_forward(x: np.ndarray, w1: np.ndarray, w2: np.ndarray, w3: np.ndarray) -> np.ndarray:
    """SwiGLU FFN ([AG] 8.4 FeedForward; [ST] FeedForward): w2(silu(w1 x) * w3 x), bias-free
    linears in nn.Linear orientation (y = x W^T)."""
    return (silu(x @ w1.T) * (x @ w3.T)) @ w2.T


WeightFn = Callable[[str, int], np.ndarray]


def _dense_weights(weights: dict, dtype) -> WeightFn:
    cache: Dict[Tuple[str, int], np.ndarray] = {}

    def get(name: str, layer: int) -> np.ndarray:
        key = (name, layer)
        if key not in cache:
            t = weights[name] if layer < 0 else weights["layers"][layer][name]
            cache[key] = _to_numpy(t, dtype)
        return cache[key]
    return get


def _to_numpy(t, dtype) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(dtype, copy=False)
    import torch
    return t.detach().to("cpu", torch.float64 if dtype == np.float64 else torch.float32).numpy().astype(dtype, copy=False)


class Oracle:
    """Transformer.forward(tokens, start_pos) with a persistent KV cache ([AG] 8.4
    Transformer and Attention; the cache is written at [start_pos, start_pos+seqlen) and
    read over [0, start_pos+seqlen)).

    `weights` is the dict layout of synth.gen_weights (torch or numpy arrays), or a
    callable (name, layer) -> array with layer = -1 for the global tensors."""

    def __init__(self, args: ModelArgs, weights, max_batch_size: int, dtype=np.float32,
                 storage: Optional[str] = None):
        self.args = args
        self.dtype = dtype
        self.st, self.st_kv = _storage_fns(storage)
        # every weight in the working precision: arrays a callable hands over in another dtype
        # (fp32 copies of the device tensors) would otherwise set the precision of the sums
        self.w: WeightFn = ((lambda n, l: np.asarray(weights(n, l)).astype(dtype, copy=False))
                            if callable(weights) else _dense_weights(weights, dtype))
        shape = (args.n_layers, max_batch_size, args.max_seq_len, args.kv_heads, args.head_dim)
        self.cache_k = np.zeros(shape, dtype=dtype)
        self.cache_v = np.zeros(shape, dtype=dtype)

    def forward(self, tokens: np.ndarray, start_pos: int) -> np.ndarray:
        """tokens (B, S) int -> fp logits (B, S, vocab) for every position."""
        a = self.args
        tokens = np.asarray(tokens)
        B, S = tokens.shape
        assert start_pos + S <= a.max_seq_len and B <= self.cache_k.shape[1]
        hd, H, KVH = a.head_dim, a.n_heads, a.kv_heads
        positions = list(range(start_pos, start_pos + S))
        st, st_kv = self.st, self.st_kv
        h = self.w("tok_embeddings", -1)[tokens]                       # (B, S, D)
        for l in range(a.n_layers):
            w = lambda n: self.w(n, l)  # noqa: E731
            x = st(rms_norm(h, w("attention_norm"), a.norm_eps))
            q = (x @ w("wq").T).reshape(B, S, H, hd)
            k = (x @ w("wk").T).reshape(B, S, KVH, hd)
            v = (x @ w("wv").T).reshape(B, S, KVH, hd)
            q = st(apply_rope(q, positions, a.rope_theta))
            k = st_kv(apply_rope(k, positions, a.rope_theta))
            self.cache_k[l, :B, start_pos:start_pos + S] = k
            self.cache_v[l, :B, start_pos:start_pos + S] = st_kv(v)
            keys = self.cache_k[l, :B, :start_pos + S]
            vals = self.cache_v[l, :B, :start_pos + S]
            o = st(attention(q, keys, vals, start_pos, a.n_rep).reshape(B, S, H * hd))
            h = h + o @ w("wo").T
            x = st(rms_norm(h, w("ffn_norm"), a.norm_eps))
            g = st(silu(x @ w("w1").T) * (x @ w("w3").T))
            h = h + g @ w("w2").T
        x = st(rms_norm(h, self.w("norm", -1), a.norm_eps))
        return x @ self.w("output", -1).T


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Greedy pick over the last axis ([AG] 8.5, temperature == 0); ties -> lowest index
    (reading R16).  NaN is an error."""
    if np.isnan(logits).any():
        raise ValueError("NaN logit")
    return np.argmax(logits, axis=-1)   # numpy returns the first maximal index


def sample_top_p(logits: np.ndarray, temperature: float, top_p: float, u: np.ndarray):
    """Temperature + nucleus sampling of one token per row ([AG] 8.5, temperature > 0: softmax
    of logits / temperature, then sample_top_p; [AG] 6.3 and [ST] "Sampling, Stopping, and the
    Chat Template": sort the probabilities descending, zero the tokens beyond the cumulative
    top-p mass, renormalise, draw one token from the multinomial).  float64 throughout.

    Readings: R20 a token is beyond the top-p mass when the mass of the tokens sorted before
    it exceeds top_p (so the first token always stays; top_p >= 1 keeps every token); R21 equal
    probabilities sort by lower token index first; R22 the draw is the inverse CDF of the
    renormalised kept distribution in sorted order at the caller's uniform u[b] in [0, 1),
    i.e. the first sorted token whose cumulative mass exceeds u[b]; R23 the returned log-prob
    is log_softmax of the raw (untempered) logits at the drawn token.

    logits: (B, V); u: (B,).  Returns (tokens int64 (B,), logprobs float64 (B,))."""
    x = np.asarray(logits, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("non-finite logit")
    B, V = x.shape
    z = x / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=-1, keepdims=True)
    lse = np.log(np.exp(x - x.max(axis=-1, keepdims=True)).sum(axis=-1)) + x.max(axis=-1)
    tokens = np.empty(B, dtype=np.int64)
    logprobs = np.empty(B, dtype=np.float64)
    for b in range(B):
        order = np.lexsort((np.arange(V), -p[b]))          # descending p, then lower index
        ps = p[b][order]
        before = np.cumsum(ps) - ps                          # mass sorted before each token
        kept = ps.copy()
        if top_p < 1.0:
            kept[before > top_p] = 0.0
        kept = kept / kept.sum()
        cdf = np.cumsum(kept)
        n_kept = int((kept > 0).sum()) if top_p < 1.0 else V
        i = int(np.searchsorted(cdf, float(u[b]), side="right"))   # first cdf > u
        i = min(i, n_kept - 1)
        tokens[b] = order[i]
        logprobs[b] = x[b, order[i]] - lse[b]
    return tokens, logprobs


def greedy_generate(model: Oracle, prompts: List[List[int]], max_gen_len: int,
                    eos_id: int = -1, pad_id: int = -1):
    """Llama.generate at temperature 0 ([AG] 8.5; [ST] "Sampling, Stopping"): prompts sit
    left-aligned in a pad-filled (bsz, total_len) rectangle; the first call covers
    [0, min_prompt_len), later calls one position each; rows still inside their prompt keep
    their prompt token; the loop stops early only when every row has emitted eos.

    Returns (tokens (bsz, total_len), list of per-call last-position logits (bsz, V))."""
    bsz = len(prompts)
    min_len = min(len(p) for p in prompts)
    max_len = max(len(p) for p in prompts)
    total_len = min(model.args.max_seq_len, max_gen_len + max_len)
    tokens = np.full((bsz, total_len), pad_id, dtype=np.int64)
    for b, p in enumerate(prompts):
        tokens[b, :len(p)] = p
    in_prompt = tokens != pad_id
    eos_reached = np.zeros(bsz, dtype=bool)
    prev = 0
    step_logits = []
    for cur in range(min_len, total_len):
        logits = model.forward(tokens[:, prev:cur], prev)[:, -1]
        step_logits.append(logits)
        nxt = argmax_lowest(logits)
        nxt = np.where(in_prompt[:, cur], tokens[:, cur], nxt)
        tokens[:, cur] = nxt
        eos_reached |= (~in_prompt[:, cur]) & (nxt == eos_id)
        prev = cur
        if eos_reached.all():
            break
    return tokens, step_logits


def teacher_forced_logits(args: ModelArgs, weights, tokens: np.ndarray,
                          dtype=np.float32, layer_hook: Optional[Callable[[int], None]] = None,
                          storage: Optional[str] = None) -> np.ndarray:
    """Logits at every position of a fixed token sequence in one causal pass from position 0,
    computed layer by layer (each layer's weights are touched once).  By the causal mask
    ([AG] 8.4 note), position j's logits equal what an incremental run would emit at the
    call that ends at j.  tokens (B, T) -> logits (B, T, vocab)."""
    wf: WeightFn = ((lambda n, l: np.asarray(weights(n, l)).astype(dtype, copy=False))
                    if callable(weights) else _dense_weights(weights, dtype))
    st, st_kv = _storage_fns(storage)
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    hd, H, KVH = args.head_dim, args.n_heads, args.kv_heads
    positions = list(range(T))
    h = wf("tok_embeddings", -1)[tokens].astype(dtype)
    for l in range(args.n_layers):
        if layer_hook is not None:
            layer_hook(l)
        w = lambda n: wf(n, l)  # noqa: E731
        x = st(rms_norm(h, w("attention_norm"), args.norm_eps))
        q = st(apply_rope((x @ w("wq").T).reshape(B, T, H, hd), positions, args.rope_theta))
        k = st_kv(apply_rope((x @ w("wk").T).reshape(B, T, KVH, hd), positions, args.rope_theta))
        v = st_kv((x @ w("wv").T).reshape(B, T, KVH, hd))
        o = st(attention(q, k, v, 0, args.n_rep).reshape(B, T, H * hd))
        h = h + o @ w("wo").T
        x = st(rms_norm(h, w("ffn_norm"), args.norm_eps))
        g = st(silu(x @ w("w1").T) * (x @ w("w3").T))
        h = h + g @ w("w2").T
    x = st(rms_norm(h, wf("norm", -1), args.norm_eps))
    return x @ wf("output", -1).T


def args_from_workload(wl) -> ModelArgs:
    """ModelArgs for a synth.Workload (shape fields only)."""
    return ModelArgs(dim=wl.dim, n_layers=wl.n_layers, n_heads=wl.n_heads,
                     vocab_size=wl.vocab_size, hidden_dim=wl.hidden_dim,
                     n_kv_heads=wl.n_kv_heads, norm_eps=wl.norm_eps,
                     rope_theta=wl.rope_theta, max_seq_len=wl.max_seq_len)


def workload_weights(wl, dtype=np.float32, device="cpu") -> WeightFn:
    """Weight provider drawing each tensor from the shared seeded generator on demand and
    keeping only the most recent layer (the layer-major passes touch each layer once)."""
    import synth
    state: Dict[str, object] = {"layer": None, "tensors": {}}
    glob: Dict[str, np.ndarray] = {}

    def get(name: str, layer: int) -> np.ndarray:
        if layer < 0:
            if name not in glob:
                glob[name] = _to_numpy(synth.gen_tensor(wl, name, 0, device), dtype)
            return glob[name]
        if state["layer"] != layer:
            state["layer"] = layer
            state["tensors"] = {}
        t = state["tensors"]
        if name not in t:
            t[name] = _to_numpy(synth.gen_tensor(wl, name, layer, device), dtype)
        return t[name]
    return get

"""Seeded synthetic inputs for the Llama 2 decoder forward: weights, prompts, workload shapes.

This module is shared by the CPU oracle side and the HIP side and holds none of the
model's arithmetic: it only produces numbers to feed both.

Weights.  Every matrix is drawn from N(0, 0.02) as a stand-in for a trained checkpoint
(none is available).  Generation must be fast for 7B-70B shapes and bit-identical on CPU
and GPU, so it is counter based and integer only:

    idx  = flat element index (int64)
    u    = mix32(mix32(idx + k1) ^ k2)          # k1, k2 from (seed, tensor id)
    q    = u >> 16                               # 16-bit uniform index
    w    = TABLE[q]                              # TABLE[i] = 0.02 * Phi^-1((i + 0.5) / 65536)

TABLE is built once on the host in float64 (scipy's ndtri), rounded to float32 and, for
bf16 models, rounded to bf16 with round-to-nearest-even by torch.  The draw is therefore a
65536-level quantisation of the normal distribution (truncated at 4.3 sigma), finer than
bf16's 8-bit mantissa.  mix32 is the two-round xor-shift-multiply integer hash with
multiplier 0x045D9F3B; every product stays below 2**63, so torch int64 arithmetic gives the
same bits on every device.

RMSNorm weights are 1.0 in every workload (a norm weight drawn from N(0, 0.02) would shrink
every logit about fifty-fold, and no greedy token would ever have a clear margin).

Prompts.  Token ids are uniform in [3, vocab) (ids 0-2 are the tokenizer's special ids),
drawn with numpy's PCG64 from the workload's prompt seed; ragged lengths are uniform
integers in the stated closed range.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

M32 = 0xFFFFFFFF
_MULT = 0x045D9F3B
_TABLE_BITS = 16
_CHUNK = 1 << 24


@dataclasses.dataclass(frozen=True)
class Workload:
    """A model shape plus the batch it is run on (prefill of the prompts, then greedy decode)."""
    name: str
    dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    hidden_dim: int
    vocab_size: int
    norm_eps: float
    rope_theta: float
    max_seq_len: int
    batch: int
    prompt_len: int                      # fixed prompt length (0 when ragged)
    prompt_len_range: Optional[tuple]    # (lo, hi) inclusive, for ragged prompts
    gen_steps: int                       # max_gen_len of the greedy generate schedule
    dtype: str                           # "bf16", "fp16" or "fp32"
    weight_seed: int
    prompt_seed: int

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_fp32", 256, 4, 8, 2, 768, 512, 1e-5, 10000.0, 128,
                 2, 16, None, 16, "fp32", 1, 1001),
        Workload("llama2_7b_b1", 4096, 32, 32, 32, 11008, 32000, 1e-5, 10000.0, 4096,
                 1, 128, None, 128, "bf16", 2, 1002),
        # the 7B batch-1 workload with fp16 weights and cache (the reference's dtype; the
        # vector-ALU path)
        Workload("llama2_7b_b1_fp16", 4096, 32, 32, 32, 11008, 32000, 1e-5, 10000.0, 4096,
                 1, 128, None, 128, "fp16", 2, 1002),
        Workload("llama2_7b_b32_ragged", 4096, 32, 32, 32, 11008, 32000, 1e-5, 10000.0, 4096,
                 32, 0, (256, 512), 256, "bf16", 3, 1003),
        Workload("llama2_13b_b16", 5120, 40, 40, 40, 13824, 32000, 1e-5, 10000.0, 4096,
                 16, 2048, None, 128, "bf16", 4, 1004),
        Workload("llama2_70b_b8", 8192, 80, 64, 8, 28672, 32000, 1e-5, 10000.0, 4096,
                 8, 3584, None, 512, "bf16", 5, 1005),
    ]
}

LAYER_TENSORS = ("attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w2", "w3")
GLOBAL_TENSORS = ("tok_embeddings", "norm", "output")
NORM_TENSORS = ("attention_norm", "ffn_norm", "norm")


def tensor_shape(w: Workload, name: str) -> tuple:
    """nn.Linear orientation: [out_features][in_features], row-major."""
    hd = w.head_dim
    return {
        "tok_embeddings": (w.vocab_size, w.dim),
        "norm": (w.dim,),
        "output": (w.vocab_size, w.dim),
        "attention_norm": (w.dim,),
        "ffn_norm": (w.dim,),
        "wq": (w.n_heads * hd, w.dim),
        "wk": (w.n_kv_heads * hd, w.dim),
        "wv": (w.n_kv_heads * hd, w.dim),
        "wo": (w.dim, w.n_heads * hd),
        "w1": (w.hidden_dim, w.dim),
        "w2": (w.dim, w.hidden_dim),
        "w3": (w.hidden_dim, w.dim),
    }[name]


def tensor_id(name: str, layer: int) -> int:
    if name in GLOBAL_TENSORS:
        return GLOBAL_TENSORS.index(name)
    return len(GLOBAL_TENSORS) + layer * len(LAYER_TENSORS) + LAYER_TENSORS.index(name)


def _mix32_int(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * _MULT) & M32
    x ^= x >> 16
    x = (x * _MULT) & M32
    x ^= x >> 16
    return x


def _mix32_(x: torch.Tensor, t: torch.Tensor) -> torch.Tensor:
    """In-place mix32 of x (int64 values in [0, 2**32)); t is a work buffer of x's size."""
    for _ in range(2):
        torch.bitwise_right_shift(x, 16, out=t)
        x.bitwise_xor_(t)
        x.mul_(_MULT).bitwise_and_(M32)
    torch.bitwise_right_shift(x, 16, out=t)
    x.bitwise_xor_(t)
    return x


_WORK: Dict[str, tuple] = {}


def _work_buffers(device) -> tuple:
    key = str(device)
    if key not in _WORK:
        _WORK[key] = tuple(torch.empty(_CHUNK, dtype=torch.int64, device=device) for _ in range(2))
    return _WORK[key]


_TABLES: Dict[tuple, torch.Tensor] = {}


def quantile_table(dtype: str, device="cpu") -> torch.Tensor:
    """65536 equiprobable N(0, 0.02) levels (midpoint quantiles), in the storage dtype."""
    key = (dtype, str(device))
    if key not in _TABLES:
        from scipy.special import ndtri
        p = (np.arange(1 << _TABLE_BITS, dtype=np.float64) + 0.5) / float(1 << _TABLE_BITS)
        t32 = torch.from_numpy((0.02 * ndtri(p)).astype(np.float32))
        t = t32.to(torch_dtype(dtype))
        _TABLES[key] = t.to(device)
    return _TABLES[key]


def torch_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]


def gen_tensor(w: Workload, name: str, layer: int = 0, device="cpu",
               rows: Optional[slice] = None) -> torch.Tensor:
    """One weight tensor of workload `w`, bit-identical on any device.

    `rows` optionally restricts a matrix to a row range (same values as the full tensor)."""
    shape = tensor_shape(w, name)
    dt = torch_dtype(w.dtype)
    if name in NORM_TENSORS:
        return torch.ones(shape, dtype=dt, device=device)
    ncols = shape[1]
    r0, r1 = 0, shape[0]
    if rows is not None:
        r0, r1 = rows.start or 0, shape[0] if rows.stop is None else rows.stop
    out = torch.empty(((r1 - r0) * ncols,), dtype=dt, device=device)
    tid = tensor_id(name, layer)
    k1 = _mix32_int(w.weight_seed * 0x9E3779B1 + tid * 0x85EBCA77 + 0x27D4EB2F)
    k2 = _mix32_int(k1 ^ 0x165667B1)
    table = quantile_table(w.dtype, device)
    n = out.numel()
    base = r0 * ncols
    ubuf, tbuf = _work_buffers(device)
    for s in range(0, n, _CHUNK):
        m = min(n, s + _CHUNK) - s
        u, t = ubuf[:m], tbuf[:m]
        torch.arange(base + s, base + s + m, dtype=torch.int64, out=u)
        u.add_(k1).bitwise_and_(M32)
        _mix32_(u, t)
        u.bitwise_xor_(k2)
        _mix32_(u, t)
        u.bitwise_right_shift_(16)
        torch.index_select(table, 0, u, out=out[s:s + m])
    return out.view(r1 - r0, ncols)


def gen_weights(w: Workload, device="cpu", layers: Optional[Sequence[int]] = None) -> dict:
    """{"tok_embeddings", "norm", "output", "layers": [ {name: tensor} ... ]}."""
    layers = range(w.n_layers) if layers is None else layers
    d = {n: gen_tensor(w, n, 0, device) for n in GLOBAL_TENSORS}
    d["layers"] = [{n: gen_tensor(w, n, l, device) for n in LAYER_TENSORS} for l in layers]
    return d


def prompts(w: Workload) -> List[List[int]]:
    """The workload's prompt token ids (ids uniform in [3, vocab))."""
    rng = np.random.Generator(np.random.PCG64(w.prompt_seed))
    if w.prompt_len_range is not None:
        lo, hi = w.prompt_len_range
        lens = rng.integers(lo, hi + 1, size=w.batch)
    else:
        lens = np.full(w.batch, w.prompt_len)
    return [rng.integers(3, w.vocab_size, size=int(n)).tolist() for n in lens]


def tensor_digest(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's bytes (manifest entry)."""
    return hashlib.sha256(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()

"""Statistics the GPU parity tests compare logits with.  Pure NumPy; no model arithmetic.

Two sets of logits over the same positions, shape (positions, vocab), are compared by
  - per position: RMS of the difference over the vocabulary, its 99.9th percentile of
    |difference|, its maximum and the cosine of the two logit vectors;
  - pooled over every checked logit: the same RMS, 99.9th percentile and maximum.

At the 7B depths two correct evaluations of the same bf16-storage method already differ by
more than the stated 3e-2 (an fp32 summation order flips some bf16 roundings and each flip
moves a stored value by a whole bf16 unit), so a GPU result is held to what a second
correct evaluation of the method shows: the oracle on an equivalent model whose model and
FFN dimensions are permuted consistently (same function, every fp32 sum in another order).

Greedy tokens: at a position where the reference's top-1/top-2 margin m exceeds what a
correct evaluation's errors can reach, the token must be the reference's; in the band
below, a mismatch is legitimate, and the number of mismatches is held against what a
correct evaluation's noise makes likely: the logit difference of the two candidates moves
by a Gaussian of standard deviation sqrt(2) * rms (the per-position RMS of the correct
evaluation's difference), so position j flips with probability p_j = Phi(-m_j / (sqrt(2)
rms_j)); the count over the band is Poisson-binomial(p), and the GPU's count must not pass
its 0.999 quantile.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np


@dataclasses.dataclass
class Dist:
    """Distance between two logit sets over the same positions."""
    rms: np.ndarray      # per position
    p999: np.ndarray     # per position, 99.9th percentile of |d|
    max: np.ndarray      # per position
    cos: np.ndarray      # per position
    rms_all: float       # pooled over every logit
    p999_all: float
    max_all: float

    def line(self) -> str:
        return (f"rms {self.rms_all:.4e} p99.9 {self.p999_all:.4e} max {self.max_all:.4e} "
                f"worst-position rms {self.rms.max():.4e} min cos {self.cos.min():.6f}")


def distance(a: np.ndarray, b: np.ndarray) -> Dist:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape and a.ndim == 2, (a.shape, b.shape)
    d = a - b
    ad = np.abs(d)
    rms = np.sqrt(np.mean(d * d, axis=-1))
    k = max(0, int(math.ceil(0.999 * a.shape[1])) - 1)
    p999 = np.partition(ad, k, axis=-1)[:, k]
    mx = ad.max(axis=-1)
    cos = (a * b).sum(-1) / (np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1))
    flat = ad.ravel()
    kk = max(0, int(math.ceil(0.999 * flat.size)) - 1)
    return Dist(rms=rms, p999=p999, max=mx, cos=cos,
                rms_all=float(np.sqrt(np.mean(d * d))),
                p999_all=float(np.partition(flat, kk)[kk]),
                max_all=float(mx.max()))


def poisson_binomial_quantile(p: Sequence[float], q: float) -> int:
    """Smallest k with P(N <= k) >= q for N the number of successes of independent
    Bernoulli trials with probabilities p (exact, by dynamic programming)."""
    p = np.clip(np.asarray(p, dtype=np.float64), 0.0, 1.0)
    dist = np.zeros(len(p) + 1)
    dist[0] = 1.0
    for i, pi in enumerate(p):
        dist[1:i + 2] = dist[1:i + 2] * (1.0 - pi) + dist[0:i + 1] * pi
        dist[0] *= 1.0 - pi
    cdf = np.cumsum(dist)
    return int(np.searchsorted(cdf, q - 1e-12))


def normal_tail(x: np.ndarray) -> np.ndarray:
    """Phi(-x) for x >= 0."""
    return 0.5 * np.array([math.erfc(v / math.sqrt(2.0)) for v in np.ravel(x)]).reshape(np.shape(x))


def top2(logits: np.ndarray):
    """(argmax with ties to the lowest index, top-1 minus top-2 margin) per row."""
    x = np.asarray(logits, dtype=np.float64)
    top = np.argmax(x, axis=-1)
    srt = np.sort(x, axis=-1)
    return top, srt[:, -1] - srt[:, -2]


@dataclasses.dataclass
class GreedyReport:
    checked: int          # positions with a free (generated) token
    forced: int           # of them, margin above the forced threshold (must match)
    band: int             # margin in (0.1, forced threshold]
    band_mismatch: int    # GPU tokens that differ from the reference's in the band
    band_expected: float  # expected mismatches under a correct evaluation's noise
    band_limit: int       # 0.999 quantile of that count
    alt_mismatch: int     # the correct evaluation's own mismatches in the band

    def line(self) -> str:
        return (f"greedy: {self.checked} tokens, {self.forced} forced (all equal), band "
                f"{self.band}: GPU {self.band_mismatch} mismatches, a correct evaluation "
                f"{self.alt_mismatch}, expected {self.band_expected:.2f}, limit {self.band_limit}")


def greedy_check(tokens_next: np.ndarray, gpu_logits: np.ndarray, ref: np.ndarray,
                 alt: np.ndarray, forced_margin: float, min_margin: float = 0.1) -> GreedyReport:
    """tokens_next[j]: the token the GPU emitted after position j (only free positions are
    passed); gpu_logits / ref / alt: (positions, vocab) logits of the GPU, the reference and a
    second correct evaluation.  Asserts (a) every token is the argmax of the GPU's own logits,
    (b) tokens equal the reference's where its margin exceeds forced_margin, (c) the band's
    mismatch count is within the 0.999 quantile of the count a correct evaluation's noise
    gives."""
    tokens_next = np.asarray(tokens_next)
    g_top, _ = top2(gpu_logits)
    assert np.array_equal(tokens_next, g_top), \
        f"emitted token is not the argmax of the GPU's own logits at {np.nonzero(tokens_next != g_top)[0][:8]}"
    r_top, margin = top2(ref)
    a_top, _ = top2(alt)
    forced = margin > forced_margin
    bad = np.nonzero(forced & (tokens_next != r_top))[0]
    assert bad.size == 0, f"greedy token differs at forced positions {bad[:8]} (margins {margin[bad[:8]]})"
    band = (margin > min_margin) & ~forced
    sigma = np.sqrt(2.0) * np.sqrt(np.mean((np.asarray(alt, np.float64) - np.asarray(ref, np.float64)) ** 2, axis=-1))
    p = normal_tail(margin[band] / np.maximum(sigma[band], 1e-30)) if band.any() else np.zeros(0)
    rep = GreedyReport(checked=int(tokens_next.size), forced=int(forced.sum()), band=int(band.sum()),
                       band_mismatch=int((band & (tokens_next != r_top)).sum()),
                       band_expected=float(p.sum()),
                       band_limit=poisson_binomial_quantile(p, 0.999) if p.size else 0,
                       alt_mismatch=int((band & (a_top != r_top)).sum()))
    assert rep.band_mismatch <= rep.band_limit, rep.line()
    return rep


def check_depth(gpu: np.ndarray, ref: np.ndarray, alt: np.ndarray, plain: Optional[np.ndarray],
                delta: float, say=print, stated_max: float = 3e-2, stated_cos: float = 0.999):
    """Logit checks of a GPU result against the 16-bit-storage oracle `ref`, with `alt` a
    second correct evaluation of it and `plain` the plain fp32 oracle (all (positions, vocab)).

    Against ref: where alt meets the stated bars (max |d| <= stated_max, cosine >=
    stated_cos at every position), the GPU must meet them; where it does not, the GPU's
    pooled RMS and 99.9th percentile of |GPU - ref|, its worst position's RMS and its maximum
    must each be at most (1 + delta) times alt's.
    Against plain: where ref and alt both meet the stated bars against plain, the GPU must
    too; where they do not, the GPU must be no farther from plain than a correct 16-bit
    evaluation is: pooled RMS and 99.9th percentile at most (1 + delta) times the larger of
    ref's and alt's, and the smallest cosine at least what that RMS allowance admits
    (1 - cos ~ rms(d)^2 / (2 rms(x)^2)).  Returns the distances."""
    k = 1.0 + delta
    fails = []

    def meets(d: Dist) -> bool:
        return d.max_all <= stated_max and d.cos.min() >= stated_cos

    g_r, a_r = distance(gpu, ref), distance(alt, ref)
    say(f"    GPU - oracle(16-bit storage):    {g_r.line()}")
    say(f"    permuted oracle - oracle:        {a_r.line()}")
    if meets(a_r):
        if not meets(g_r):
            fails.append(f"vs storage oracle: max {g_r.max_all:.4e} / min cos {g_r.cos.min():.6f} "
                         f"outside the stated {stated_max} / {stated_cos}")
    else:
        for what, g, a in (("pooled rms", g_r.rms_all, a_r.rms_all), ("pooled p99.9", g_r.p999_all, a_r.p999_all),
                           ("worst-position rms", g_r.rms.max(), a_r.rms.max()), ("max", g_r.max_all, a_r.max_all)):
            if not g <= k * a:
                fails.append(f"vs storage oracle: {what} {g:.4e} > {k:.2f} x {a:.4e}")
    out = {"gpu_ref": g_r, "alt_ref": a_r}
    if plain is not None:
        g_p, r_p, a_p = distance(gpu, plain), distance(ref, plain), distance(alt, plain)
        say(f"    GPU - plain fp32 oracle:         {g_p.line()}")
        say(f"    oracle(16-bit storage) - plain:  {r_p.line()}")
        say(f"    permuted oracle - plain:         {a_p.line()}")
        if meets(r_p) and meets(a_p):
            if not meets(g_p):
                fails.append(f"vs plain oracle: max {g_p.max_all:.4e} / min cos {g_p.cos.min():.6f} "
                             f"outside the stated {stated_max} / {stated_cos}")
        else:
            for what, g, r, a in (("pooled rms", g_p.rms_all, r_p.rms_all, a_p.rms_all),
                                  ("pooled p99.9", g_p.p999_all, r_p.p999_all, a_p.p999_all)):
                if not g <= k * max(r, a):
                    fails.append(f"vs plain oracle: {what} {g:.4e} > {k:.2f} x {max(r, a):.4e}")
            cos_floor = 1.0 - k * k * (1.0 - min(r_p.cos.min(), a_p.cos.min()))
            if not g_p.cos.min() >= min(stated_cos, cos_floor):
                fails.append(f"vs plain oracle: min cos {g_p.cos.min():.6f} < {min(stated_cos, cos_floor):.6f}")
        out.update(gpu_plain=g_p, ref_plain=r_p, alt_plain=a_p)
    assert not fails, "; ".join(fails)
    return out

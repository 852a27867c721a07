"""Seeded synthetic inputs for the attention-KL path.

This module holds random-number generation and dtype rounding only: none of the
method's arithmetic.  Both the HIP path (through the tests and the bench) and the
CPU oracle consume what it returns.

Every tensor of every (batch, head) slice comes from its own generator,
``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, b, h])))``, so a
single head can be regenerated alone, at any size, without drawing the rest.

Tensor ids: 0 teacher Q, 1 teacher K, 2 student Q (or its noise), 3 student K
(or its noise), 4 the key subset that is scaled in the peaky recipe, 5 the
per-row upstream gradient g.

Values are drawn in float32; bf16 inputs are rounded to nearest-even from those
float32 draws, and the student of the ``noise`` recipe is
``round(teacher_f32 + sigma * noise_f32)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

TID_QT, TID_KT, TID_QS, TID_KS, TID_PEAK, TID_G = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem: shapes, dtype and the recipe for the values."""

    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d_t: int
    d_s: int
    causal: bool
    dtype: str  # "fp32" or "bf16"
    recipe: str  # "noise": student = teacher + sigma*N(0,1); "independent"
    sigma: float = 0.0
    peak_frac: float = 0.0  # fraction of teacher keys scaled by peak_scale
    peak_scale: float = 1.0
    seed: int = 0

    @property
    def scale_t(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d_t)))

    @property
    def scale_s(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d_s)))

    @property
    def rows(self) -> int:
        return self.B * self.H * self.Nq

    def pairs_per_head(self) -> int:
        """Allowed (query, key) pairs of one head (bottom-right causal alignment)."""
        if not self.causal:
            return self.Nq * self.Nk
        return _causal_pairs(self.Nq, self.Nk)

    def fwd_flops(self) -> float:
        return 2.0 * self.pairs_per_head() * (self.d_t + self.d_s) * self.B * self.H

    def bwd_flops(self, teacher: bool = False) -> float:
        f = 2.0 * self.pairs_per_head() * (self.d_t + 3 * self.d_s) * self.B * self.H
        if teacher:
            f += 4.0 * self.pairs_per_head() * self.d_t * self.B * self.H
        return f


def _causal_pairs(nq: int, nk: int) -> int:
    """Pairs under bottom-right causal alignment: row i sees keys 0..i+(nk-nq) (needs nq <= nk)."""
    off = nk - nq
    return nq * (off + 1) + nq * (nq - 1) // 2


# The five synthetic configurations of the attention-KL workload, smallest first.
WORKLOADS: Dict[int, Workload] = {
    1: Workload("b1h2n128d64-fp32", 1, 2, 128, 128, 64, 64, False, "fp32", "noise", sigma=0.3, seed=1),
    2: Workload("b2h16n2048d128-causal", 2, 16, 2048, 2048, 128, 128, True, "bf16", "noise", sigma=0.1, seed=2),
    3: Workload("b1h32n32768d128-causal-peaky", 1, 32, 32768, 32768, 128, 128, True, "bf16", "independent",
                peak_frac=0.01, peak_scale=4.0, seed=3),
    4: Workload("b4h8n8192-dt128-ds64", 4, 8, 8192, 8192, 128, 64, False, "bf16", "independent", seed=4),
    5: Workload("b1h8n131072d128-causal", 1, 8, 131072, 131072, 128, 128, True, "bf16", "noise", sigma=0.2, seed=5),
}


def custom(B, H, Nq, Nk, d_t, d_s, causal, dtype="bf16", recipe="noise", sigma=0.3, seed=100,
           peak_frac=0.0, peak_scale=1.0) -> Workload:
    return Workload(f"b{B}h{H}q{Nq}k{Nk}dt{d_t}ds{d_s}{'-causal' if causal else ''}-{dtype}",
                    B, H, Nq, Nk, d_t, d_s, causal, dtype, recipe, sigma, peak_frac, peak_scale, seed)


def length_mix(total: int, seed: int, lo: int = 256, hi: int = 8192) -> list:
    """Segment lengths of a packed batch: log-uniform in [lo, hi], drawn until they fill `total` rows
    (the last one cut to fit).  Seeded: PCG64(SeedSequence([seed, 6]))."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 6])))
    out, left = [], total
    while left > 0:
        n = int(round(math.exp(g.uniform(math.log(lo), math.log(hi)))))
        out.append(min(n, left))
        left -= out[-1]
    return out


def _rng(seed: int, tid: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b, h])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_f32(w: Workload, b: int, h: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """The four float32 input slices of one (b, h) head, already rounded to w.dtype."""
    qt = _rng(w.seed, TID_QT, b, h).standard_normal((w.Nq, w.d_t), dtype=np.float32)
    kt = _rng(w.seed, TID_KT, b, h).standard_normal((w.Nk, w.d_t), dtype=np.float32)
    if w.peak_frac > 0:
        npk = int(math.floor(w.peak_frac * w.Nk))
        idx = _rng(w.seed, TID_PEAK, b, h).choice(w.Nk, size=npk, replace=False)
        kt[idx] *= np.float32(w.peak_scale)
    if w.recipe == "noise":
        assert w.d_t == w.d_s, "the noise recipe needs equal head dims"
        qs = qt + np.float32(w.sigma) * _rng(w.seed, TID_QS, b, h).standard_normal(qt.shape, dtype=np.float32)
        ks = kt + np.float32(w.sigma) * _rng(w.seed, TID_KS, b, h).standard_normal(kt.shape, dtype=np.float32)
    elif w.recipe == "independent":
        qs = _rng(w.seed, TID_QS, b, h).standard_normal((w.Nq, w.d_s), dtype=np.float32)
        ks = _rng(w.seed, TID_KS, b, h).standard_normal((w.Nk, w.d_s), dtype=np.float32)
    elif w.recipe == "same":  # student identical to teacher
        assert w.d_t == w.d_s
        qs, ks = qt.copy(), kt.copy()
    elif w.recipe == "uniform_teacher":  # teacher queries all zero
        qt[:] = 0
        qs = _rng(w.seed, TID_QS, b, h).standard_normal((w.Nq, w.d_s), dtype=np.float32)
        ks = _rng(w.seed, TID_KS, b, h).standard_normal((w.Nk, w.d_s), dtype=np.float32)
    else:
        raise ValueError(w.recipe)
    if w.dtype == "bf16":
        qt, kt, qs, ks = (bf16_bits_to_f32(f32_to_bf16_bits(a)) for a in (qt, kt, qs, ks))
    return qt, kt, qs, ks


def head_f64(w: Workload, b: int, h: int):
    """One head's inputs as float64 (exact: every bf16/fp32 value is a float64)."""
    return tuple(a.astype(np.float64) for a in head_f32(w, b, h))


def head_g(w: Workload, b: int, h: int) -> np.ndarray:
    """Per-row upstream gradient g ~ U[0.5, 1.5] (float32) for one head."""
    return _rng(w.seed, TID_G, b, h).uniform(0.5, 1.5, size=w.Nq).astype(np.float32)


def full_f32(w: Workload, heads: Optional[list] = None):
    """All four inputs as float32 arrays [B, H, N, d] (values already rounded to w.dtype)."""
    qt = np.empty((w.B, w.H, w.Nq, w.d_t), np.float32)
    kt = np.empty((w.B, w.H, w.Nk, w.d_t), np.float32)
    qs = np.empty((w.B, w.H, w.Nq, w.d_s), np.float32)
    ks = np.empty((w.B, w.H, w.Nk, w.d_s), np.float32)
    for b in range(w.B):
        for h in range(w.H):
            qt[b, h], kt[b, h], qs[b, h], ks[b, h] = head_f32(w, b, h)
    return qt, kt, qs, ks


def full_g(w: Workload) -> np.ndarray:
    g = np.empty((w.B, w.H, w.Nq), np.float32)
    for b in range(w.B):
        for h in range(w.H):
            g[b, h] = head_g(w, b, h)
    return g


def full_bf16_bits(w: Workload):
    """All four inputs as uint16 bf16 bit arrays [B, H, N, d]; built head by head to bound memory."""
    assert w.dtype == "bf16"
    out = [np.empty((w.B, w.H, n, d), np.uint16)
           for n, d in ((w.Nq, w.d_t), (w.Nk, w.d_t), (w.Nq, w.d_s), (w.Nk, w.d_s))]
    for b in range(w.B):
        for h in range(w.H):
            for o, a in zip(out, head_f32(w, b, h)):
                o[b, h] = f32_to_bf16_bits(a)  # exact: a already holds bf16 values
    return tuple(out)

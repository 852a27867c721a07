"""The bounds on |dS| that the backward's fp16 gradient product scales by, checked on random and
adversarial rows in float64 (no GPU).

Per row, with P_t = softmax(a), P_s = softmax(b), KL = KL(P_t || P_s):
  KL student gradients    dS = P_s - P_t                                  |dS| <= 1
  KL teacher gradients    dS = P_t ((a - LSE_t) - (b - LSE_s) - KL)       |dS| <= 2 KL + 3/e
  JS, either half (log2)  dS = P (log2(P / M) - KL(P || M) log2 e)        |dS| <= 1.34
The kernel keeps the scaled |dS| below 2^14 from these (2^13 for the first and third, 2^(14 - e) with
2^e above the second); a bound that failed would overflow fp16 and send the workgroup to the exact
path, or worse, if it failed by less than the headroom, lose nothing but that headroom.
"""
import math

import numpy as np
import pytest
from scipy.special import log_softmax


def _rows(rng, n_rows, n_keys):
    """Logit pairs of several kinds: independent, close, far apart, one-sided extremes."""
    out = []
    for _ in range(n_rows):
        kind = rng.integers(0, 5)
        a = rng.standard_normal(n_keys) * rng.uniform(0.1, 8.0)
        if kind == 0:
            b = rng.standard_normal(n_keys) * rng.uniform(0.1, 8.0)
        elif kind == 1:
            b = a + 0.01 * rng.standard_normal(n_keys)
        elif kind == 2:
            b = -a * rng.uniform(1.0, 20.0)
        elif kind == 3:  # the student gives almost nothing to a key the teacher favours
            b = a.copy()
            j = int(np.argmax(a))
            b[j] -= rng.uniform(10.0, 1000.0)
        else:  # the teacher splits its mass over two keys, the student sees only one of them
            a = np.full(n_keys, -50.0)
            a[:2] = 0.0
            b = np.full(n_keys, -50.0)
            b[1] = 0.0
            b[0] = -rng.uniform(10.0, 1000.0)
        out.append((a, b))
    return out


def test_ds_bounds_hold_on_random_and_adversarial_rows():
    rng = np.random.default_rng(91)
    worst = {"student": 0.0, "teacher": 0.0, "js": 0.0}
    for n_keys in (2, 7, 64, 1000):
        for a, b in _rows(rng, 300, n_keys):
            lpt, lps = log_softmax(a), log_softmax(b)
            pt, ps = np.exp(lpt), np.exp(lps)
            kl = float(np.sum(pt * (lpt - lps)))
            worst["student"] = max(worst["student"], float(np.abs(ps - pt).max()))
            ds_t = pt * (lpt - lps - kl)
            worst["teacher"] = max(worst["teacher"], float(np.abs(ds_t).max() / (2.0 * kl + 3.0 / math.e)))
            lm = np.logaddexp(lpt, lps) - math.log(2.0)
            for lp, p in ((lpt, pt), (lps, ps)):
                half = float(np.sum(p * (lp - lm)))
                ds = p * ((lp - lm) / math.log(2.0) - half / math.log(2.0))
                worst["js"] = max(worst["js"], float(np.abs(ds).max()))
    assert worst["student"] <= 1.0
    assert worst["teacher"] <= 1.0, worst
    assert worst["js"] <= 1.34, worst


@pytest.mark.parametrize("p", [0.05, 0.3, 0.5, 0.9, 0.999])
def test_teacher_bound_as_a_student_logit_vanishes(p):
    """Teacher mass p on a key whose student logit falls by `drop`: there dS ~ p (1 - p) drop grows
    with the KL (~ p drop), and stays below 2 KL + 3/e however far the logit falls."""
    for drop in (10.0, 100.0, 1000.0):
        a = np.array([math.log(p), math.log(1.0 - p)])
        b = np.array([-drop, 0.0])
        lpt, lps = log_softmax(a), log_softmax(b)
        pt = np.exp(lpt)
        kl = float(np.sum(pt * (lpt - lps)))
        ds = pt * (lpt - lps - kl)
        assert np.abs(ds).max() <= 2.0 * kl + 3.0 / math.e

"""Pins for the oracle's Jensen-Shannon functions: each test ties them to something other than
the oracle itself (scipy's jensenshannon and rel_entr, a closed form, bounds and symmetry, torch
autograd of the entropy form H(M) - H(P_t)/2 - H(P_s)/2, finite differences, causal special rows).
"""
import math

import numpy as np
import pytest
import scipy.spatial.distance as ssd
import scipy.special as sps
import torch

from oracle import js_backward_head, js_forward_head


def rand_head(rng, nq, nk, dt, ds, scale=1.0):
    return (rng.standard_normal((nq, dt)) * scale, rng.standard_normal((nk, dt)) * scale,
            rng.standard_normal((nq, ds)) * scale, rng.standard_normal((nk, ds)) * scale)


def _rows(qt, kt, qs, ks, st, ss, causal):
    """Each row's allowed teacher / student distributions, via scipy's softmax."""
    nq, nk = qt.shape[0], kt.shape[0]
    a, b = st * qt @ kt.T, ss * qs @ ks.T
    for i in range(nq):
        n = min(nk, i + nk - nq + 1) if causal else nk
        yield sps.softmax(a[i, :n]), sps.softmax(b[i, :n])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(7, 7, 5, 5), (5, 9, 4, 3), (16, 16, 8, 8)])
def test_js_matches_scipy(causal, shape):
    nq, nk, dt, ds = shape
    qt, kt, qs, ks = rand_head(np.random.default_rng(21), nq, nk, dt, ds, 1.2)
    st, ss = 0.6, 0.5
    js, ht, hs, lt, ls = js_forward_head(qt, kt, qs, ks, st, ss, causal)
    for i, (p, q) in enumerate(_rows(qt, kt, qs, ks, st, ss, causal)):
        m = 0.5 * (p + q)
        assert js[i] == pytest.approx(ssd.jensenshannon(p, q) ** 2, rel=1e-9, abs=1e-15)
        assert ht[i] == pytest.approx(sps.rel_entr(p, m).sum(), rel=1e-10, abs=1e-15)
        assert hs[i] == pytest.approx(sps.rel_entr(q, m).sum(), rel=1e-10, abs=1e-15)
        n = len(p)
        assert lt[i] == pytest.approx(sps.logsumexp(st * qt[i] @ kt[:n].T), rel=1e-12)
        assert ls[i] == pytest.approx(sps.logsumexp(ss * qs[i] @ ks[:n].T), rel=1e-12)


def test_js_two_key_closed_form():
    # teacher logits (0, 0): P_t = (1/2, 1/2); student logits (ln 3, 0): P_s = (3/4, 1/4); M = (5/8, 3/8)
    qt, kt = np.array([[1.0]]), np.array([[0.0], [0.0]])
    qs, ks = np.array([[1.0]]), np.array([[math.log(3.0)], [0.0]])
    js, ht, hs, _, _ = js_forward_head(qt, kt, qs, ks, 1.0, 1.0, False)
    kl_tm = 0.5 * math.log(0.5 / 0.625) + 0.5 * math.log(0.5 / 0.375)
    kl_sm = 0.75 * math.log(0.75 / 0.625) + 0.25 * math.log(0.25 / 0.375)
    assert ht[0] == pytest.approx(kl_tm, rel=1e-13)
    assert hs[0] == pytest.approx(kl_sm, rel=1e-13)
    assert js[0] == pytest.approx(0.5 * (kl_tm + kl_sm), rel=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_js_identity_bounds_and_symmetry(causal):
    qt, kt, qs, ks = rand_head(np.random.default_rng(22), 12, 12, 6, 6, 3.0)
    js, ht, hs, _, _ = js_forward_head(qt, kt, qt, kt, 0.5, 0.5, causal)
    np.testing.assert_array_equal(js, 0.0)
    js, ht, hs, _, _ = js_forward_head(qt, kt, qs, ks, 0.5, 0.5, causal)
    assert np.all(js >= 0.0) and np.all(js <= math.log(2.0))
    js2, ht2, hs2, _, _ = js_forward_head(qs, ks, qt, kt, 0.5, 0.5, causal)  # sides exchanged
    np.testing.assert_allclose(js2, js, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(ht2, hs, rtol=1e-13, atol=1e-16)
    # very different sharp distributions approach the bound ln 2
    big = 40.0
    qa, ka = np.array([[big]]), np.array([[1.0], [-1.0]])
    js_far, _, _, _, _ = js_forward_head(qa, ka, -qa, ka, 1.0, 1.0, False)
    assert js_far[0] == pytest.approx(math.log(2.0), rel=1e-12)


def _torch_js(qt, kt, qs, ks, st, ss, causal, g):
    """sum_i g_i JS_i written as entropies, H(M) - H(P_t)/2 - H(P_s)/2, for torch autograd."""
    nq, nk = qt.shape[0], kt.shape[0]
    a, b = st * qt @ kt.T, ss * qs @ ks.T
    i = torch.arange(nq)[:, None]
    j = torch.arange(nk)[None, :]
    allowed = (j <= i + nk - nq) if causal else torch.ones(nq, nk, dtype=torch.bool)
    pa = torch.softmax(a.masked_fill(~allowed, -math.inf), -1)
    pb = torch.softmax(b.masked_fill(~allowed, -math.inf), -1)
    pm = 0.5 * (pa + pb)

    def ent(p):
        return -(torch.where(p > 0, p * torch.log(torch.where(p > 0, p, torch.ones_like(p))), torch.zeros_like(p))).sum(-1)
    return (g * (ent(pm) - 0.5 * ent(pa) - 0.5 * ent(pb))).sum()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(6, 6, 4, 4), (4, 7, 3, 5)])
def test_js_gradients_match_torch_autograd_of_the_entropy_form(causal, shape):
    nq, nk, dt, ds = shape
    arrs = rand_head(np.random.default_rng(23), nq, nk, dt, ds, 1.1)
    g = np.random.default_rng(24).uniform(-1.0, 1.5, nq)
    st, ss = 0.8, 0.55
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in arrs]
    _torch_js(*ts, st, ss, causal, torch.tensor(g)).backward()
    r = js_backward_head(*arrs, st, ss, causal, g, teacher=True)
    for name, t in zip(("dq_t", "dk_t", "dq_s", "dk_s"), ts):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-12, err_msg=name)


def test_js_gradients_match_finite_differences():
    qt, kt, qs, ks = rand_head(np.random.default_rng(25), 4, 5, 3, 3, 0.9)
    g = np.array([0.7, -1.2, 1.5, 0.4])
    st, ss = 0.9, 0.6

    def loss(qt_, kt_, qs_, ks_):
        return float((g * js_forward_head(qt_, kt_, qs_, ks_, st, ss, False)[0]).sum())
    r = js_backward_head(qt, kt, qs, ks, st, ss, False, g, teacher=True)
    h = 1e-6
    arrs = [qt, kt, qs, ks]
    for idx, name in enumerate(("dq_t", "dk_t", "dq_s", "dk_s")):
        num = np.zeros_like(arrs[idx])
        for pos in np.ndindex(arrs[idx].shape):
            hi = [x.copy() for x in arrs]
            lo = [x.copy() for x in arrs]
            hi[idx][pos] += h
            lo[idx][pos] -= h
            num[pos] = (loss(*hi) - loss(*lo)) / (2 * h)
        np.testing.assert_allclose(r[name], num, rtol=1e-6, atol=1e-9, err_msg=name)


def test_js_causal_single_key_rows_are_zero():
    # causal with N_Q = N_K: row 0 sees one key, so both distributions are (1) and JS = 0 with no gradient
    qt, kt, qs, ks = rand_head(np.random.default_rng(26), 5, 5, 4, 4, 2.0)
    js, _, _, _, _ = js_forward_head(qt, kt, qs, ks, 0.5, 0.5, True)
    assert js[0] == 0.0 and js[1] > 0.0
    g = np.zeros(5)
    g[0] = 1.0
    r = js_backward_head(qt, kt, qs, ks, 0.5, 0.5, True, g, teacher=True)
    for v in r.values():
        np.testing.assert_array_equal(v, 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_js_row_blocking_and_subsets_agree(causal):
    """Row blocks and row/key subsets (what the full-size GPU checks ask for) give the full result's
    rows and keys."""
    rng = np.random.default_rng(26)
    nq, nk = 37, 45
    arrs = rand_head(rng, nq, nk, 4, 4)
    g = rng.uniform(0.5, 1.5, nq)
    f1 = js_forward_head(*arrs, 0.5, 0.5, causal, block=1000)
    f2 = js_forward_head(*arrs, 0.5, 0.5, causal, block=5)
    rows = [0, 3, 36, 20]
    f3 = js_forward_head(*arrs, 0.5, 0.5, causal, rows=rows)
    for x, y, z in zip(f1, f2, f3):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(x[rows], z, rtol=1e-13, atol=1e-16)
    b1 = js_backward_head(*arrs, 0.5, 0.5, causal, g, teacher=True, block=1000)
    b2 = js_backward_head(*arrs, 0.5, 0.5, causal, g, teacher=True, block=7)
    keys = [44, 0, 30]
    b3 = js_backward_head(*arrs, 0.5, 0.5, causal, g, teacher=True, rows=rows, keys=keys, block=6)
    for k in b1:
        np.testing.assert_allclose(b1[k], b2[k], rtol=1e-11, atol=1e-14)
    for k in ("dq_s", "dq_t"):
        np.testing.assert_allclose(b3[k], b1[k][rows], rtol=1e-11, atol=1e-14)
    for k in ("dk_s", "dk_t"):
        np.testing.assert_allclose(b3[k], b1[k][keys], rtol=1e-11, atol=1e-14)

"""Pins for the CPU oracle: each test ties it to something other than itself.

Closed forms, library routines (scipy, torch autograd), a 50-digit brute force,
finite differences, invariants and hand-derived worked examples.  A dropped
term, a wrong sign, a swapped KL direction, a transposed operand or a shifted
causal diagonal in the oracle fails at least one of these.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special as sps
import torch

from oracle import backward_head, forward_head

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_head(rng, nq, nk, dt, ds, scale=1.0):
    return (rng.standard_normal((nq, dt)) * scale, rng.standard_normal((nk, dt)) * scale,
            rng.standard_normal((nq, ds)) * scale, rng.standard_normal((nk, ds)) * scale)


def _eval(expr):
    if isinstance(expr, (int, float)):
        return float(expr)
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log}))


# ---------------------------------------------------------------- worked examples
def test_worked_examples_closed_form():
    ex = json.load(open(os.path.join(HERE, "golden", "worked_examples.json")))["examples"]
    for e in ex:
        arr = {k: np.array([[_eval(v) for v in row] for row in e[k]]) for k in ("q_t", "k_t", "q_s", "k_s")}
        kl, lt, ls = forward_head(arr["q_t"], arr["k_t"], arr["q_s"], arr["k_s"], e["scale_t"], e["scale_s"],
                                  e["causal"])
        np.testing.assert_allclose(kl, [_eval(x) for x in e["kl"]], rtol=1e-12, atol=1e-14, err_msg=e["name"])
        np.testing.assert_allclose(lt, [_eval(x) for x in e["lse_t"]], rtol=1e-12, err_msg=e["name"])
        np.testing.assert_allclose(ls, [_eval(x) for x in e["lse_s"]], rtol=1e-12, err_msg=e["name"])
        gr = backward_head(arr["q_t"], arr["k_t"], arr["q_s"], arr["k_s"], e["scale_t"], e["scale_s"],
                           e["causal"], np.array(e["g"]), teacher=True)
        for key in ("dq_s", "dk_s", "dq_t", "dk_t"):
            if key in e:
                exp = np.array([[_eval(v) for v in row] for row in e[key]])
                np.testing.assert_allclose(gr[key], exp, rtol=1e-12, atol=1e-14, err_msg=f"{e['name']} {key}")


# ---------------------------------------------------------------- library routines
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(7, 7, 5, 5), (5, 9, 4, 3), (16, 16, 8, 8), (1, 4, 3, 3)])
def test_kl_matches_scipy_rel_entr_and_torch_kl_div(causal, shape):
    nq, nk, dt, ds = shape
    rng = np.random.default_rng(11)
    qt, kt, qs, ks = rand_head(rng, nq, nk, dt, ds, 1.3)
    st, ss = 0.7, 0.45
    kl, lt, ls = forward_head(qt, kt, qs, ks, st, ss, causal)
    # independent route: build each row's key list explicitly, then scipy softmax + rel_entr
    for i in range(nq):
        last = nk - 1 if not causal else i + (nk - nq)
        keys = np.arange(last + 1)
        a = st * np.array([np.dot(qt[i], kt[j]) for j in keys])
        b = ss * np.array([np.dot(qs[i], ks[j]) for j in keys])
        pt, ps = sps.softmax(a), sps.softmax(b)
        assert kl[i] == pytest.approx(sps.rel_entr(pt, ps).sum(), rel=1e-10, abs=1e-13)
        assert lt[i] == pytest.approx(sps.logsumexp(a), rel=1e-13)
        assert ls[i] == pytest.approx(sps.logsumexp(b), rel=1e-13)
        tk = torch.nn.functional.kl_div(torch.log_softmax(torch.tensor(b), 0), torch.log_softmax(torch.tensor(a), 0),
                                        reduction="sum", log_target=True)
        assert kl[i] == pytest.approx(float(tk), rel=1e-10, abs=1e-13)


def test_kl_brute_force_50_digits():
    """Direct definition with Decimal arithmetic at 50 digits, explicit loops, no numpy."""
    getcontext().prec = 50
    rng = np.random.default_rng(5)
    nq, nk, dt, ds = 4, 6, 3, 2
    qt, kt, qs, ks = rand_head(rng, nq, nk, dt, ds)
    st, ss = 0.5, 0.8
    for causal in (False, True):
        kl, lt, ls = forward_head(qt, kt, qs, ks, st, ss, causal)
        for i in range(nq):
            keys = range(nk) if not causal else range(i + (nk - nq) + 1)
            a = [Decimal(st) * sum(Decimal(qt[i, c]) * Decimal(kt[j, c]) for c in range(dt)) for j in keys]
            b = [Decimal(ss) * sum(Decimal(qs[i, c]) * Decimal(ks[j, c]) for c in range(ds)) for j in keys]
            za = sum(x.exp() for x in a)
            zb = sum(x.exp() for x in b)
            p = [x.exp() / za for x in a]
            q = [x.exp() / zb for x in b]
            ref = sum(pi * (pi / qi).ln() for pi, qi in zip(p, q))
            assert abs(kl[i] - float(ref)) <= 1e-13 * max(1.0, abs(float(ref)))
            assert lt[i] == pytest.approx(float(za.ln()), rel=1e-14)
            assert ls[i] == pytest.approx(float(zb.ln()), rel=1e-14)


# ---------------------------------------------------------------- closed forms / special cases
@pytest.mark.parametrize("causal", [False, True])
def test_teacher_equals_student_gives_zero(causal):
    rng = np.random.default_rng(3)
    qt, kt, _, _ = rand_head(rng, 12, 12, 6, 6)
    kl, lt, ls = forward_head(qt, kt, qt, kt, 0.4, 0.4, causal)
    assert np.all(np.abs(kl) < 1e-14)
    np.testing.assert_array_equal(lt, ls)
    gr = backward_head(qt, kt, qt, kt, 0.4, 0.4, causal, np.ones(12), teacher=True)
    for v in gr.values():
        assert np.abs(v).max() < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_gibbs_nonnegative(causal):
    rng = np.random.default_rng(4)
    for trial in range(5):
        qt, kt, qs, ks = rand_head(rng, 20, 24, 4, 7, 2.0 + trial)
        kl, _, _ = forward_head(qt, kt, qs, ks, 1.0, 1.0, causal)
        assert np.all(kl >= -1e-12)
        if trial == 0:  # moderate logits: no row collapses to a shared one-hot, so strictly positive
            assert np.all(kl > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_teacher_closed_form(causal):
    """Q_t = 0: P_t uniform over A_i, so KL_i = LSE_s,i - mean_{A_i} b_ij - ln|A_i|."""
    rng = np.random.default_rng(6)
    nq, nk = 9, 13
    _, kt, qs, ks = rand_head(rng, nq, nk, 5, 4)
    qt = np.zeros((nq, 5))
    kl, lt, ls = forward_head(qt, kt, qs, ks, 0.9, 0.6, causal)
    for i in range(nq):
        n = nk if not causal else i + (nk - nq) + 1
        b = 0.6 * ks[:n] @ qs[i]
        assert kl[i] == pytest.approx(ls[i] - b.mean() - math.log(n), rel=1e-11, abs=1e-13)
        assert lt[i] == pytest.approx(math.log(n), rel=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_student_closed_form(causal):
    """Q_s = 0: P_s uniform, so KL_i = sum P_t a - LSE_t,i + ln|A_i| (= ln|A_i| - entropy(P_t))."""
    rng = np.random.default_rng(7)
    nq, nk = 9, 13
    qt, kt, _, ks = rand_head(rng, nq, nk, 5, 4)
    qs = np.zeros((nq, 4))
    kl, lt, ls = forward_head(qt, kt, qs, ks, 0.9, 0.6, causal)
    for i in range(nq):
        n = nk if not causal else i + (nk - nq) + 1
        a = 0.9 * kt[:n] @ qt[i]
        p = np.exp(a - a.max())
        p /= p.sum()
        entropy = -(p * np.log(p)).sum()
        assert kl[i] == pytest.approx(math.log(n) - entropy, rel=1e-11, abs=1e-13)


def test_causal_rows_zero_and_one():
    """|A_0| = 1 gives KL 0; |A_1| = 2 gives the Bernoulli KL of two sigmoids."""
    rng = np.random.default_rng(8)
    n = 6
    qt, kt, qs, ks = rand_head(rng, n, n, 3, 3)
    kl, _, _ = forward_head(qt, kt, qs, ks, 1.0, 1.0, True)
    assert kl[0] == 0.0
    a = kt[:2] @ qt[1]
    b = ks[:2] @ qs[1]
    p = 1 / (1 + math.exp(-(a[1] - a[0])))
    q = 1 / (1 + math.exp(-(b[1] - b[0])))
    bern = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
    assert kl[1] == pytest.approx(bern, rel=1e-11)
    gr = backward_head(qt, kt, qs, ks, 1.0, 1.0, True, np.ones(n))
    assert np.abs(gr["dq_s"][0]).max() == 0.0


def test_causal_row_equals_truncated_noncausal():
    """Row i of a causal (bottom-right) problem = a non-causal one-row problem on keys 0..i+Nk-Nq."""
    rng = np.random.default_rng(9)
    nq, nk = 6, 10
    qt, kt, qs, ks = rand_head(rng, nq, nk, 4, 4)
    kl, lt, ls = forward_head(qt, kt, qs, ks, 0.5, 0.5, True)
    for i in range(nq):
        last = i + nk - nq
        r = forward_head(qt[i:i + 1], kt[:last + 1], qs[i:i + 1], ks[:last + 1], 0.5, 0.5, False)
        assert (kl[i], lt[i], ls[i]) == pytest.approx((r[0][0], r[1][0], r[2][0]), rel=1e-13, abs=1e-15)


def test_key_permutation_invariance_and_query_equivariance():
    rng = np.random.default_rng(10)
    nq, nk = 8, 11
    qt, kt, qs, ks = rand_head(rng, nq, nk, 4, 3)
    kl, lt, ls = forward_head(qt, kt, qs, ks, 0.7, 0.7, False)
    pk = rng.permutation(nk)
    kl2, lt2, ls2 = forward_head(qt, kt[pk], qs, ks[pk], 0.7, 0.7, False)
    np.testing.assert_allclose(kl2, kl, rtol=1e-12)
    pq = rng.permutation(nq)
    kl3, _, _ = forward_head(qt[pq], kt, qs[pq], ks, 0.7, 0.7, False)
    np.testing.assert_allclose(kl3, kl[pq], rtol=1e-12)
    g = rng.uniform(0.5, 1.5, nq)
    g1 = backward_head(qt, kt, qs, ks, 0.7, 0.7, False, g)
    g2 = backward_head(qt, kt[pk], qs, ks[pk], 0.7, 0.7, False, g)
    np.testing.assert_allclose(g2["dk_s"], g1["dk_s"][pk], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(g2["dq_s"], g1["dq_s"], rtol=1e-11, atol=1e-14)


def test_all_student_keys_equal_gives_zero_dq():
    """Equal student keys make P_s uniform and dQ_s = s sum_j dS_ij k = k s sum_j dS_ij = 0."""
    rng = np.random.default_rng(12)
    qt, kt, qs, _ = rand_head(rng, 7, 9, 4, 5)
    ks = np.tile(rng.standard_normal(5), (9, 1))
    for causal in (False, True):
        gr = backward_head(qt, kt, qs, ks, 0.6, 0.6, causal, np.ones(7))
        assert np.abs(gr["dq_s"]).max() < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identity_q_dot_dq_equals_k_dot_dk(causal):
    """sum_i q_i . dQ_i = s sum_ij dS_ij (q_i . k_j) = sum_j k_j . dK_j, for either side."""
    rng = np.random.default_rng(13)
    qt, kt, qs, ks = rand_head(rng, 10, 14, 4, 6)
    g = rng.uniform(0.5, 1.5, 10)
    gr = backward_head(qt, kt, qs, ks, 0.8, 0.3, causal, g, teacher=True)
    assert (qs * gr["dq_s"]).sum() == pytest.approx((ks * gr["dk_s"]).sum(), rel=1e-11, abs=1e-14)
    assert (qt * gr["dq_t"]).sum() == pytest.approx((kt * gr["dk_t"]).sum(), rel=1e-11, abs=1e-14)


# ---------------------------------------------------------------- gradients
def _torch_loss(qt, kt, qs, ks, st, ss, causal, g):
    """sum_i g_i KL_i built row by row over each row's allowed keys only (no masking needed)."""
    nq, nk = qt.shape[0], kt.shape[0]
    total = 0
    for i in range(nq):
        n = nk if not causal else i + (nk - nq) + 1
        la = torch.log_softmax(st * (kt[:n] @ qt[i]), 0)
        lb = torch.log_softmax(ss * (ks[:n] @ qs[i]), 0)
        total = total + g[i] * torch.nn.functional.kl_div(lb, la, reduction="sum", log_target=True)
    return total


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(6, 6, 4, 4), (5, 8, 6, 3), (12, 12, 8, 8)])
def test_gradients_match_torch_autograd(causal, shape):
    nq, nk, dt, ds = shape
    rng = np.random.default_rng(14)
    arrs = rand_head(rng, nq, nk, dt, ds)
    g = rng.uniform(0.5, 1.5, nq)
    st, ss = 0.55, 0.8
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in arrs]
    _torch_loss(*ts, st, ss, causal, torch.tensor(g)).backward()
    gr = backward_head(*arrs, st, ss, causal, g, teacher=True)
    for name, t in zip(("dq_t", "dk_t", "dq_s", "dk_s"), ts):
        np.testing.assert_allclose(gr[name], t.grad.numpy(), rtol=1e-10, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_finite_differences(causal):
    nq, nk, dt, ds = 5, 7, 3, 4
    rng = np.random.default_rng(15)
    arrs = [x.copy() for x in rand_head(rng, nq, nk, dt, ds)]
    g = rng.uniform(0.5, 1.5, nq)
    st, ss = 0.9, 0.6
    gr = backward_head(*arrs, st, ss, causal, g, teacher=True)
    h = 1e-5

    def loss():
        return float(g @ forward_head(*arrs, st, ss, causal)[0])

    for ti, name in enumerate(("dq_t", "dk_t", "dq_s", "dk_s")):
        x = arrs[ti]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(gr[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


# ---------------------------------------------------------------- internal consistency of the oracle's blocking
@pytest.mark.parametrize("causal", [False, True])
def test_row_blocking_and_subsets_agree(causal):
    rng = np.random.default_rng(16)
    nq, nk = 37, 45
    arrs = rand_head(rng, nq, nk, 4, 4)
    g = rng.uniform(0.5, 1.5, nq)
    f1 = forward_head(*arrs, 0.5, 0.5, causal, block=1000)
    f2 = forward_head(*arrs, 0.5, 0.5, causal, block=5)
    for x, y in zip(f1, f2):
        np.testing.assert_allclose(x, y, rtol=1e-13)
    rows = [0, 3, 36, 20]
    f3 = forward_head(*arrs, 0.5, 0.5, causal, rows=rows)
    for x, y in zip(f1, f3):
        np.testing.assert_allclose(x[rows], y, rtol=1e-13)
    b1 = backward_head(*arrs, 0.5, 0.5, causal, g, teacher=True, block=1000)
    b2 = backward_head(*arrs, 0.5, 0.5, causal, g, teacher=True, block=7)
    keys = [44, 0, 30]
    b3 = backward_head(*arrs, 0.5, 0.5, causal, g, teacher=True, rows=rows, keys=keys, block=6)
    for k in b1:
        np.testing.assert_allclose(b1[k], b2[k], rtol=1e-11, atol=1e-14)
    for k in ("dq_s", "dq_t"):
        np.testing.assert_allclose(b3[k], b1[k][rows], rtol=1e-11, atol=1e-14)
    for k in ("dk_s", "dk_t"):
        np.testing.assert_allclose(b3[k], b1[k][keys], rtol=1e-11, atol=1e-14)


def test_scale_folding_invariance():
    """(alpha Q, scale/alpha) gives the same logits, so the same KL and LSEs."""
    rng = np.random.default_rng(17)
    qt, kt, qs, ks = rand_head(rng, 6, 6, 4, 4)
    r1 = forward_head(qt, kt, qs, ks, 0.5, 0.25, True)
    r2 = forward_head(qt * 2, kt, qs * 4, ks, 0.25, 0.0625, True)
    for x, y in zip(r1, r2):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- the row-window runner of the GPU tests
@pytest.mark.parametrize("nq,nk,causal,r0,teacher,js", [
    (300, 300, True, 0, True, False),
    (300, 300, True, 130, False, False),
    (257, 400, True, 64, True, False),      # bottom-right alignment with more keys than queries
    (200, 150, False, 0, True, False),
    (300, 300, True, 0, True, True),
    (220, 300, True, 100, False, True),
])
def test_row_window_runner_reassembles_the_whole_head(nq, nk, causal, r0, teacher, js):
    """The full-size GPU tests run the oracle on row blocks of a head in threads (each block a
    problem of its own rows and their keys) and sum the dK partials; here the result must equal the
    oracle on the whole head to float64 rounding, for every row of the window and every key whose dK
    the window completes."""
    import oracle
    from parity import oracle_window
    rng = np.random.default_rng(nq + nk + r0)
    head = rand_head(rng, nq, nk, 16, 8)
    g = rng.uniform(0.5, 1.5, nq)
    st, ss = 0.3, 0.4
    win = oracle_window(head, st, ss, causal, g, r0=r0, teacher=teacher, js=js, block=48, workers=3)
    rows = np.arange(r0, nq)
    if js:
        ref_f = oracle.js_forward_head(*head, st, ss, causal)
        names = ("js", "js_t", "js_s", "lse_t", "lse_s")
        ref_b = oracle.js_backward_head(*head, st, ss, causal, g, teacher=teacher)
    else:
        ref_f = oracle.forward_head(*head, st, ss, causal)
        names = ("kl", "lse_t", "lse_s")
        ref_b = backward_head(*head, st, ss, causal, g, teacher=teacher)
    for n, v in zip(names, ref_f):
        np.testing.assert_allclose(win[n], v[rows], rtol=1e-12, atol=1e-13)
    k0 = win["k0"]
    assert k0 == (r0 + nk - nq if causal else 0)
    for sd in (("s", "t") if teacher else ("s",)):
        np.testing.assert_allclose(win["dq_" + sd], ref_b["dq_" + sd][rows], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(win["dk_" + sd], ref_b["dk_" + sd][k0:], rtol=1e-11, atol=1e-13)

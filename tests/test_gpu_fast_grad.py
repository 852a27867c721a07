"""GPU parity of the backward's fast (fp16) gradient product at the edges of its range.

For bf16 inputs the backward rounds dS once to fp16 (scaled by a power of two below a bound on |dS|:
1 for the student, 2 KL_i + 3/e per row for KL teacher gradients, times |g| for the key owner) and
converts the streamed operand (K for dQ, Q for dK) to fp16.  A workgroup that meets a streamed value
of magnitude 2^16 or more, or a run of values all below 2^-8 and not all zero, redoes its work with
the bf16 hi + lo product.  Each case below sits at one of those edges and is compared with the
float64 oracle under the usual criteria (rtol 2e-3 for bf16).  Queries and keys of a side are
multiplied by c and its scale divided by c^2, so the logits, and with them P and the KL, stay
ordinary while the streamed values move.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import all_pass, grad_floor, ratio_kl, ratio_rows, report

pytestmark = pytest.mark.gpu


def _run(host, scale_t, scale_s, causal, g, name, teacher=False):
    dev = [torch.from_numpy(a.astype(np.float32)).cuda().to(torch.bfloat16) for a in host]
    h64 = [x.float().cpu().numpy().astype(np.float64) for x in dev]  # the values the kernels see
    print(f"case {name}", flush=True)
    kl, lt, ls = S.fwd(*dev, causal=causal, scale_t=scale_t, scale_s=scale_s)
    dq, dk, dqt, dkt = S.bwd(*dev, lt, ls, torch.from_numpy(g.astype(np.float32)).cuda(), causal=causal,
                             kl=kl, teacher_grads=teacher, scale_t=scale_t, scale_s=scale_s)
    torch.cuda.synchronize()
    rkl, _, _ = oracle.forward(*h64, scale_t, scale_s, causal)
    rg = oracle.backward(*h64, scale_t, scale_s, causal, g.astype(np.float64), teacher=teacher)
    c = lambda x: x.cpu().numpy()
    ag = np.abs(g)
    r = dict(kl=ratio_kl(c(kl), rkl, 2e-3),
             dq_s=ratio_rows(c(dq), rg["dq_s"], 2e-3, grad_floor(scale_s, ag, h64[3])),
             dk_s=ratio_rows(c(dk), rg["dk_s"], 2e-3, grad_floor(scale_s, ag, h64[2])))
    if teacher:
        r.update(dq_t=ratio_rows(c(dqt), rg["dq_t"], 2e-3, grad_floor(scale_t, ag, h64[1])),
                 dk_t=ratio_rows(c(dkt), rg["dk_t"], 2e-3, grad_floor(scale_t, ag, h64[0])))
        assert np.all(np.isfinite(c(dqt))) and np.all(np.isfinite(c(dkt)))
    msg = report(name, **r)
    print(msg, flush=True)
    assert np.all(np.isfinite(c(dq))) and np.all(np.isfinite(c(dk)))
    assert all_pass(r), msg


@pytest.mark.parametrize("c", [2.0e4, 1.0e-3, 3.0e-6], ids=["large", "small", "subnormal"])
@pytest.mark.parametrize("d", [128, 64])
def test_streamed_values_at_the_edges_of_fp16(c, d):
    """c = 2e4: streamed values reach 2^16 and beyond (fp16 overflow, so the exact product);
    c = 1e-3: every value below 2^-8 (the exact product); c = 3e-6: values on the fp16 subnormal grid."""
    w = wl.custom(1, 2, 300, 300, d, d, True, recipe="independent", seed=81)
    host = [a.astype(np.float64) for a in wl.full_f32(w)]
    host[2] = host[2] * c
    host[3] = host[3] * c
    _run(host, w.scale_t, w.scale_s / (c * c), True, wl.full_g(w), f"{w.name} c={c:g}")


def test_tiny_rows_among_ordinary_ones():
    """A tenth of the student's key and query rows scaled by 1e-4 (their chunks fall below 2^-8)."""
    w = wl.custom(1, 2, 257, 257, 128, 128, True, recipe="independent", seed=82)
    host = [a.astype(np.float64) for a in wl.full_f32(w)]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([82, 1])))
    for i in (2, 3):
        rows = rng.choice(w.Nq, w.Nq // 10, replace=False)
        host[i][:, :, rows] *= 1e-4
    _run(host, w.scale_t, w.scale_s, True, wl.full_g(w), f"{w.name} tiny rows")


@pytest.mark.parametrize("kind", ["spread", "tiny", "large"])
def test_row_weights_over_many_orders_of_magnitude(kind):
    """The key owner scales dS by the largest |g| it streams: g spread over ten decades (signed),
    uniformly tiny (a mean over a million rows), or large."""
    w = wl.custom(1, 2, 260, 260, 128, 128, False, recipe="independent", seed=83)
    host = [a.astype(np.float64) for a in wl.full_f32(w)]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([83, 2])))
    shape = (w.B, w.H, w.Nq)
    if kind == "spread":
        g = 10.0 ** rng.uniform(-7.0, 3.0, shape) * np.where(rng.random(shape) < 0.3, -1.0, 1.0)
    elif kind == "tiny":
        g = np.full(shape, 1.0e-6) * rng.uniform(0.5, 1.5, shape)
    else:
        g = rng.uniform(1.0e3, 3.0e3, shape)
    _run(host, w.scale_t, w.scale_s, False, g.astype(np.float32).astype(np.float64), f"{w.name} g {kind}")


def test_nearly_equal_long_rows():
    """Student within 0.3% of the teacher over 3000 keys: dS entries near 2^-20, far below fp16's
    normal range unless scaled."""
    w = wl.custom(1, 1, 3000, 3000, 128, 128, True, sigma=0.003, seed=84)
    host = [a.astype(np.float64) for a in wl.full_f32(w)]
    _run(host, w.scale_t, w.scale_s, True, wl.full_g(w), f"{w.name} sigma 0.003")


@pytest.mark.parametrize("c", [1.0, 2.0e4, 1.0e-3], ids=["ordinary", "large", "small"])
def test_teacher_gradients_at_the_edges(c):
    """Teacher gradients take the fast product too (dS per row below 2 KL + 3/e); the teacher's
    queries and keys scaled by c move its streamed values across the fp16 edges."""
    w = wl.custom(1, 2, 300, 300, 128, 64, True, recipe="independent", seed=85)
    host = [a.astype(np.float64) for a in wl.full_f32(w)]
    host[0] = host[0] * c
    host[1] = host[1] * c
    _run(host, w.scale_t / (c * c), w.scale_s, True, wl.full_g(w), f"{w.name} teacher c={c:g}", teacher=True)


@pytest.mark.parametrize("spread", [3.0, 12.0])
def test_teacher_gradients_of_rows_far_apart(spread):
    """Student logits far from the teacher's (KL of several nats, dS of the teacher up to ~2 KL):
    the per-row bound scales dS without overflow.  Signed g over five decades for the key owner."""
    w = wl.custom(1, 2, 257, 257, 64, 128, False, recipe="independent", seed=86)
    host = [a.astype(np.float64) for a in wl.full_f32(w)]
    host[2] = host[2] * spread
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([86, int(spread)])))
    shape = (w.B, w.H, w.Nq)
    g = 10.0 ** rng.uniform(-3.0, 2.0, shape) * np.where(rng.random(shape) < 0.3, -1.0, 1.0)
    _run(host, w.scale_t, w.scale_s, False, g.astype(np.float32).astype(np.float64),
         f"{w.name} teacher spread {spread:g}", teacher=True)

"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Small and ragged problems are compared element by element over every output; the
full-size workloads run in the same launch configuration the bench times and are
compared on sampled rows / keys that the oracle computes one by one, plus
properties that hold at any size.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import (device_inputs, device_inputs_bf16_bits, grad_floor, ratio_kl, ratio_lse, ratio_rows, report,
                    rtol_of)

pytestmark = pytest.mark.gpu


def _run_gpu(w, dev_in, teacher=False):
    qt, kt, qs, ks = dev_in
    kl, lt, ls = S.fwd(qt, kt, qs, ks, causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    g = torch.from_numpy(wl.full_g(w)).cuda()
    grads = S.bwd(qt, kt, qs, ks, lt, ls, g, causal=w.causal, kl=kl, teacher_grads=teacher,
                  scale_t=w.scale_t, scale_s=w.scale_s)
    torch.cuda.synchronize()
    return (kl.cpu().numpy(), lt.cpu().numpy(), ls.cpu().numpy()), [x.cpu().numpy() for x in grads if x is not None]


def _check_full(w, teacher=False):
    """Every output of a small problem against the oracle."""
    print(f"case {w.name} teacher={teacher}", flush=True)
    dev_in, host = device_inputs(w)
    (kl, lt, ls), grads = _run_gpu(w, dev_in, teacher)
    h64 = [a.astype(np.float64) for a in host]
    rkl, rlt, rls = oracle.forward(*h64, w.scale_t, w.scale_s, w.causal)
    rg = oracle.backward(*h64, w.scale_t, w.scale_s, w.causal, wl.full_g(w), teacher=teacher)
    rt = rtol_of(w)
    g = wl.full_g(w)
    qt_h, kt_h, qs_h, ks_h = host
    r = dict(kl=ratio_kl(kl, rkl, rt), lse_t=ratio_lse(lt, rlt, rt), lse_s=ratio_lse(ls, rls, rt),
             dq_s=ratio_rows(grads[0], rg["dq_s"], rt, grad_floor(w.scale_s, g, ks_h)),
             dk_s=ratio_rows(grads[1], rg["dk_s"], rt, grad_floor(w.scale_s, g, qs_h)))
    if teacher:
        r.update(dq_t=ratio_rows(grads[2], rg["dq_t"], rt, grad_floor(w.scale_t, g, kt_h)),
                 dk_t=ratio_rows(grads[3], rg["dk_t"], rt, grad_floor(w.scale_t, g, qt_h)))
    msg = report(w.name, **r)
    print(msg, flush=True)
    assert max(r.values()) <= 1.0, msg
    assert np.all(np.isfinite(kl)) and all(np.all(np.isfinite(g)) for g in grads)


SMALL = [
    wl.WORKLOADS[1],
    wl.custom(1, 2, 1, 1, 64, 64, True),
    wl.custom(1, 1, 2, 2, 128, 128, False),
    wl.custom(1, 1, 3, 3, 128, 128, True),
    wl.custom(1, 2, 17, 17, 128, 64, True, recipe="independent"),
    wl.custom(1, 1, 127, 127, 64, 128, False, recipe="independent"),
    wl.custom(2, 1, 129, 129, 128, 128, True),
    wl.custom(1, 3, 255, 255, 128, 128, True, sigma=1.0),
    wl.custom(1, 1, 100, 300, 128, 128, True),
    wl.custom(1, 1, 300, 100, 64, 64, False),
    wl.custom(1, 1, 257, 513, 128, 64, True, recipe="independent"),
    wl.custom(1, 1, 17, 33, 64, 128, True, dtype="fp32", recipe="independent"),
    wl.custom(1, 2, 129, 129, 128, 128, False, dtype="fp32"),
    wl.custom(1, 1, 200, 200, 128, 128, True, recipe="independent", peak_frac=0.02, peak_scale=4.0),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_and_ragged(w):
    _check_full(w)


@pytest.mark.parametrize("w", [wl.custom(1, 2, 129, 129, 128, 128, True, recipe="independent"),
                               wl.custom(1, 1, 70, 70, 128, 64, False, recipe="independent"),
                               wl.custom(1, 1, 33, 33, 64, 64, True, dtype="fp32")], ids=lambda w: w.name)
def test_teacher_gradients(w):
    _check_full(w, teacher=True)


def test_b2h16n2048_causal_small_kl_full():
    """b2h16n2048d128 causal, student = teacher + 0.1 N(0,1): the small-KL cancellation regime."""
    w = wl.WORKLOADS[2]
    print(f"case {w.name}", flush=True)
    dev_in, host = device_inputs(w)
    (kl, lt, ls), grads = _run_gpu(w, dev_in)
    rt = rtol_of(w)
    g = wl.full_g(w)
    worst = {}
    for b in range(w.B):
        for h in range(w.H):
            hh = [a[b, h].astype(np.float64) for a in host]
            rkl, rlt, rls = oracle.forward_head(*hh, w.scale_t, w.scale_s, w.causal)
            worst["kl"] = max(worst.get("kl", 0), ratio_kl(kl[b, h], rkl, rt))
            worst["lse"] = max(worst.get("lse", 0), ratio_lse(lt[b, h], rlt, rt), ratio_lse(ls[b, h], rls, rt))
            if (b * w.H + h) % 8 == 0:  # gradients on 4 of the 32 heads
                rg = oracle.backward_head(*hh, w.scale_t, w.scale_s, w.causal, g[b, h])
                worst["dq_s"] = max(worst.get("dq_s", 0), ratio_rows(grads[0][b, h], rg["dq_s"], rt))
                worst["dk_s"] = max(worst.get("dk_s", 0), ratio_rows(grads[1][b, h], rg["dk_s"], rt))
    msg = report(w.name, **worst)
    print(msg, flush=True)
    assert max(worst.values()) <= 1.0, msg


@pytest.mark.parametrize("causal", [False, True])
def test_teacher_equals_student_is_exactly_zero(causal):
    w = wl.custom(1, 2, 200, 200, 128, 128, causal, recipe="same")
    print(f"case {w.name}", flush=True)
    dev_in, _ = device_inputs(w)
    (kl, lt, ls), grads = _run_gpu(w, dev_in, teacher=True)
    assert np.all(kl == 0.0)
    np.testing.assert_array_equal(lt, ls)
    for gr in grads:
        assert np.all(gr == 0.0)


def test_deterministic_and_strided_layout():
    """Bitwise-repeatable results; a [B, N, H, d] memory layout gives the same bits as [B, H, N, d]."""
    w = wl.custom(2, 3, 190, 250, 128, 64, True, recipe="independent")
    print(f"case {w.name}", flush=True)
    dev_in, _ = device_inputs(w)
    a1, g1 = _run_gpu(w, dev_in, teacher=True)
    a2, g2 = _run_gpu(w, dev_in, teacher=True)
    for x, y in zip(list(a1) + g1, list(a2) + g2):
        np.testing.assert_array_equal(x, y)
    perm = tuple(t.transpose(1, 2).contiguous().transpose(1, 2) for t in dev_in)  # strides (N*H*d, d, H*d, 1)
    assert perm[0].stride(1) != dev_in[0].stride(1)
    a3, g3 = _run_gpu(w, perm, teacher=True)
    for x, y in zip(list(a1) + g1, list(a3) + g3):
        np.testing.assert_array_equal(x, y)


def test_library_allocates_nothing():
    """Extra HBM: the only memory the path adds is the caller's 12 bytes per row (KL, LSE_t, LSE_s)."""
    w = wl.custom(1, 4, 4096, 4096, 128, 128, True)
    dev_in = device_inputs_bf16_bits(w)
    outs = tuple(torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda") for _ in range(3))
    g = torch.ones((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    dq = torch.empty((w.B, w.H, w.Nq, w.d_s), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.B, w.H, w.Nk, w.d_s), dtype=torch.float32, device="cuda")
    S.fwd(*dev_in, causal=True, out=outs)  # first launches load the code objects
    S.bwd(*dev_in, outs[1], outs[2], g, causal=True, out=[dq, dk])
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    S.fwd(*dev_in, causal=True, out=outs)
    S.bwd(*dev_in, outs[1], outs[2], g, causal=True, out=[dq, dk])
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    assert torch.cuda.memory_allocated() == alloc0
    assert sum(o.numel() * 4 for o in outs) == 12 * w.B * w.H * w.Nq


# ------------------------------------------------------------------ full-size workloads, sampled
def _sampled(w, heads, rows, keys, teacher=False):
    """teacher: the teacher pair alone (dq_t, dk_t from one streamkl_bwd call), else the student pair."""
    print(f"case {w.name} (full size, sampled) teacher={teacher}", flush=True)
    dev_in = device_inputs_bf16_bits(w)
    qt, kt, qs, ks = dev_in
    kl, lt, ls = S.fwd(qt, kt, qs, ks, causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    g = torch.from_numpy(wl.full_g(w)).cuda()
    grads = S.bwd(qt, kt, qs, ks, lt, ls, g, causal=w.causal, kl=kl, teacher_grads=teacher, student_grads=not teacher,
                  scale_t=w.scale_t, scale_s=w.scale_s)
    dq, dk = (grads[2], grads[3]) if teacher else (grads[0], grads[1])
    assert (grads[0] is None) == teacher and (grads[2] is None) != teacher
    xq, xk = (qt, kt) if teacher else (qs, ks)  # the side being differentiated
    side = "t" if teacher else "s"
    torch.cuda.synchronize()
    rt = rtol_of(w)
    # properties over every row
    klc = kl.cpu().numpy()
    assert np.all(np.isfinite(klc)) and np.all(torch.isfinite(dq).cpu().numpy()) and bool(torch.isfinite(dk).all())
    assert klc.min() >= -1e-4
    if w.causal:
        assert np.abs(klc[:, :, 0]).max() <= 1e-5  # one allowed key: KL = 0
    # sum_i q_i . dQ_i = sum_j k_j . dK_j (= scale sum_ij dS_ij q_i.k_j) per head
    lhs = (xq.double() * dq.double()).sum(dim=(2, 3))
    rhs = (xk.double() * dk.double()).sum(dim=(2, 3))
    norm = (xq.double().norm(dim=3) * dq.double().norm(dim=3)).sum(dim=2) + \
        (xk.double().norm(dim=3) * dk.double().norm(dim=3)).sum(dim=2)
    assert float(((lhs - rhs).abs() / norm).max()) <= rt
    worst = {}
    gh = wl.full_g(w)
    for (b, h) in heads:
        hh = wl.head_f64(w, b, h)
        rkl, rlt, rls = oracle.forward_head(*hh, w.scale_t, w.scale_s, w.causal, rows=rows)
        worst["kl"] = max(worst.get("kl", 0), ratio_kl(klc[b, h, rows], rkl, rt))
        worst["lse"] = max(worst.get("lse", 0), ratio_lse(lt[b, h, rows].cpu().numpy(), rlt, rt),
                           ratio_lse(ls[b, h, rows].cpu().numpy(), rls, rt))
        rg = oracle.backward_head(*hh, w.scale_t, w.scale_s, w.causal, gh[b, h], teacher=teacher, rows=rows,
                                  keys=keys)
        worst["dq_" + side] = max(worst.get("dq_" + side, 0),
                                  ratio_rows(dq[b, h, rows].cpu().numpy(), rg["dq_" + side], rt))
        worst["dk_" + side] = max(worst.get("dk_" + side, 0),
                                  ratio_rows(dk[b, h, keys].cpu().numpy(), rg["dk_" + side], rt))
    msg = report(w.name, **worst)
    print(msg, flush=True)
    assert max(worst.values()) <= 1.0, msg


def _rows(n, seed):
    r = np.random.default_rng(seed).choice(n, 12, replace=False)
    return sorted(set([0, 1, 2, 31, 32, 63, 64, 127, 128, n // 2, n - 2, n - 1] + list(r)))


def test_b1h32n32768_causal_full_size_sampled():
    w = wl.WORKLOADS[3]
    n = w.Nq
    _sampled(w, [(0, 0), (0, 17), (0, 31)], _rows(n, 3), [n - 1, n - 2, n - 31, n - 32, n - 64, n - 65, n - 130])


def test_b1h32n32768_causal_teacher_gradients_full_size_sampled():
    """The teacher pair at the bench size, launched as the bench's teacher-gradient step launches it."""
    w = wl.WORKLOADS[3]
    n = w.Nq
    _sampled(w, [(0, 3), (0, 30)], _rows(n, 6), [n - 1, n - 2, n - 31, n - 32, n - 64, n - 65, n - 130], teacher=True)


def test_b4h8n8192_two_head_dims_full_size_sampled():
    w = wl.WORKLOADS[4]
    n = w.Nk
    _sampled(w, [(0, 0), (3, 7)], _rows(w.Nq, 4), [0, 1, 63, 64, 4095, n - 1])


def test_b1h8n131072_causal_full_size_sampled():
    w = wl.WORKLOADS[5]
    n = w.Nq
    _sampled(w, [(0, 0), (0, 5)], _rows(n, 5), [n - 1, n - 2, n - 33, n - 100])


@pytest.mark.parametrize("w", [wl.custom(1, 2, 300, 300, 128, 128, True, recipe="independent", seed=41),
                               wl.custom(2, 1, 129, 200, 128, 64, False, recipe="independent", seed=42),
                               wl.custom(1, 2, 100, 100, 64, 64, True, dtype="fp32", recipe="independent", seed=43)],
                         ids=lambda w: w.name)
def test_signed_and_zero_row_weights(w):
    """g of either sign, with exact zeros: the key owner folds |g| into its statistics and applies the
    sign per tile, so tiles with and without negative weights both occur here (every 4th row is zero,
    and a whole 32-row tile of each head has only positive weights)."""
    print(f"case {w.name} signed g", flush=True)
    dev_in, host = device_inputs(w)
    qt, kt, qs, ks = dev_in
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 7])))
    g = rng.standard_normal((w.B, w.H, w.Nq)).astype(np.float32)
    g[..., ::4] = 0.0
    g[..., 32:64] = np.abs(g[..., 32:64]) + 0.1
    kl, lt, ls = S.fwd(qt, kt, qs, ks, causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    grads = S.bwd(qt, kt, qs, ks, lt, ls, torch.from_numpy(g).cuda(), causal=w.causal, kl=kl, teacher_grads=True,
                  scale_t=w.scale_t, scale_s=w.scale_s)
    torch.cuda.synchronize()
    h64 = [a.astype(np.float64) for a in host]
    rg = oracle.backward(*h64, w.scale_t, w.scale_s, w.causal, g.astype(np.float64), teacher=True)
    rt = rtol_of(w)
    ag = np.abs(g)
    r = {}
    for name, x, other, sc in (("dq_s", grads[0], h64[3], w.scale_s), ("dk_s", grads[1], h64[2], w.scale_s),
                               ("dq_t", grads[2], h64[1], w.scale_t), ("dk_t", grads[3], h64[0], w.scale_t)):
        r[name] = ratio_rows(x.cpu().numpy(), rg[name], rt, grad_floor(sc, ag, other))
    msg = report(w.name + " signed g", **r)
    print(msg, flush=True)
    assert max(r.values()) <= 1.0, msg


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["overflow", "underflow"])
def test_extreme_logits_take_the_exact_path(dtype, kind):
    """Rows whose logits leave the range of the forward's power-of-two references: logits of several
    hundred nats (unit scale, inputs of scale 4) overflow a sum taken against 2^0, and rows whose every
    logit is near -1000 (queries opposite to clustered keys) underflow it.  The kernel must notice
    and redo the workgroup with running maxima; the oracle works in float64 at any magnitude.  The
    gradients are compared for the overflow rows only: in the underflow construction the keys cluster
    around one direction u and sum_j dS_ij = 0, so dQ = sum_j dS_ij k_j cancels the u component about
    twentyfold, which magnifies the float32 rounding of the recomputed logits (of order L sqrt(d) 2^-24
    at |logit| L ~ 640) past the tolerance; that is a property of float32 at these magnitudes, not of
    the forward under test."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([71, kind == "overflow", dtype == "fp32"])))
    B, H, N, d = 1, 2, 160, 64
    if kind == "overflow":
        arrs = [4.0 * rng.standard_normal((B, H, N, d)) for _ in range(4)]
    else:
        u = rng.standard_normal((B, H, 1, d))
        k = u + 0.05 * rng.standard_normal((B, H, N, d))
        q = -10.0 * u + 0.05 * rng.standard_normal((B, H, N, d))
        q[:, :, ::3] = rng.standard_normal((B, H, (N + 2) // 3, d))  # ordinary rows in the same workgroups
        arrs = [q, k, q + 0.1 * rng.standard_normal((B, H, N, d)), k]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = [torch.from_numpy(a.astype(np.float32)).cuda().to(tdt) for a in arrs]
    host = [x.float().cpu().numpy().astype(np.float64) for x in dev]  # the values the kernels see
    print(f"case extreme logits {kind} {dtype}", flush=True)
    kl, lt, ls = S.fwd(*dev, causal=True, scale_t=1.0, scale_s=1.0)
    g = torch.ones_like(kl)
    dq, dk, _, _ = S.bwd(*dev, lt, ls, g, causal=True, scale_t=1.0, scale_s=1.0)
    torch.cuda.synchronize()
    rkl, rlt, rls = oracle.forward(*host, 1.0, 1.0, True)
    rg = oracle.backward(*host, 1.0, 1.0, True, np.ones((B, H, N)))
    rt = {"bf16": 2e-3, "fp32": 1e-5}[dtype]
    # float32 limit at these magnitudes: every logit is a float32 sum of d products whose partial sums
    # reach L = max |logit|, so it carries an absolute rounding error of order L sqrt(d) 2^-24 (the
    # fp32 products accumulate in d/2 steps).  KL, a P-weighted difference of two logits, inherits
    # that absolute error (bounded here by 4 L sqrt(d) 2^-24), and P = exp(a - LSE) with the
    # gradients the relative one; both are added to the usual criteria.
    L = max(float(np.abs(host[0] @ host[1].transpose(0, 1, 3, 2)).max()),
            float(np.abs(host[2] @ host[3].transpose(0, 1, 3, 2)).max()))
    kl_abs = 4.0 * L * math.sqrt(d) * 2.0 ** -24
    rt_g = max(rt, L * math.sqrt(d) * 2.0 ** -22)
    c = lambda x: x.cpu().numpy()
    assert np.all(np.isfinite(c(kl))) and np.all(np.isfinite(c(lt))) and np.all(np.isfinite(c(ls)))
    rms = np.maximum(np.sqrt((rkl ** 2).mean(axis=-1, keepdims=True)), 1e-3)
    kl_ratio = float((np.abs(c(kl) - rkl) / (rt * np.abs(rkl) + rt * rms + kl_abs)).max())
    r = dict(kl=kl_ratio, lse_t=ratio_lse(c(lt), rlt, max(rt, rt_g)), lse_s=ratio_lse(c(ls), rls, max(rt, rt_g)))
    if kind == "overflow":
        r.update(dq=ratio_rows(c(dq), rg["dq_s"], rt_g, grad_floor(1.0, np.ones((B, H, N)), host[3])),
                 dk=ratio_rows(c(dk), rg["dk_s"], rt_g, grad_floor(1.0, np.ones((B, H, N)), host[2])))
    else:
        assert np.all(np.isfinite(c(dq))) and np.all(np.isfinite(c(dk)))
    msg = report(f"extreme {kind} {dtype}", **r)
    print(msg, flush=True)
    assert max(r.values()) <= 1.0, msg

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

from parity import (all_pass, oracle_window, worst_of, device_inputs, device_inputs_bf16_bits, grad_floor, ratio_kl, ratio_lse, ratio_rows, report,
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
    assert all_pass(r), msg
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


# Mid-size problems in full (512 to 1300 keys, a few workgroups): ragged tile counts, unequal head dims
# (no difference chain), more keys than queries under the causal mask, the small-KL regime, logits
# with a few large peaks.
MID = [
    wl.custom(1, 2, 600, 600, 128, 128, True, recipe="independent"),
    wl.custom(1, 1, 1030, 1030, 128, 64, False, recipe="independent"),
    wl.custom(2, 2, 520, 1300, 128, 128, True, recipe="independent"),
    wl.custom(1, 2, 700, 700, 128, 128, True, sigma=0.1),
    wl.custom(1, 1, 800, 800, 128, 128, True, recipe="independent", peak_frac=0.02, peak_scale=4.0),
]


@pytest.mark.parametrize("w", MID, ids=lambda w: w.name)
def test_mid_size(w):
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
    assert all_pass(worst), msg


@pytest.mark.parametrize("n", [200, 700])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_teacher_equals_student_gives_zero(causal, dtype, n):
    """Identical teacher and student (KL = 0, every gradient 0).  fp32 inputs form both sides' logits
    with the same instructions: bitwise-equal statistics, exact zeros.  The bf16 forward with equal
    scales takes the logit difference from a second MFMA chain that starts from the finished teacher
    logits, so for identical rows it is a few float32 roundings of the partial sums instead of 0: KL
    and the gap between the two log-sum-exps stay within 1e-6 (absolute, and relative to the LSE),
    and the gradients, which the backward forms from those statistics, within 1e-5 of their natural
    size scale * max |g| * max row norm."""
    w = wl.custom(1, 2, n, n, 128, 128, causal, dtype=dtype, recipe="same")
    print(f"case {w.name}", flush=True)
    dev_in, host = device_inputs(w)
    (kl, lt, ls), grads = _run_gpu(w, dev_in, teacher=True)
    if dtype == "fp32":
        assert np.all(kl == 0.0)
        np.testing.assert_array_equal(lt, ls)
        for gr in grads:
            assert np.all(gr == 0.0)
        return
    assert np.abs(kl).max() <= 1e-6
    assert np.all(np.abs(lt - ls) <= 1e-6 * np.maximum(1.0, np.abs(lt)))
    gmax = float(np.abs(wl.full_g(w)).max())
    for gr, other in zip(grads, (host[3], host[2], host[1], host[0])):  # dq_s, dk_s, dq_t, dk_t
        natural = w.scale_s * gmax * float(np.linalg.norm(other, axis=-1).max())
        assert np.linalg.norm(gr, axis=-1).max() <= 1e-5 * natural


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


# ------------------------------------------------------------------ full-size workloads
def _full_size(w, teacher=False, whole=(), window=(), r0=None, lead=0, sampled=(), rows=(), keys=(),
               check_alloc=False):
    """One full-size workload run as the bench runs it (streamkl_fwd, then streamkl_bwd_dk and
    streamkl_bwd_dq; teacher: the teacher pair alone from one streamkl_bwd call, as the bench's
    teacher step), then compared with the oracle:
      whole:   heads compared over every row (KL, LSE_t, LSE_s, dQ) and every key (dK);
      window:  heads compared over rows r0 .. Nq-1 and keys r0 + Nk - Nq .. Nk-1 (causal: every row that
               sees those keys lies in the window, so their dK is complete), plus, when lead > 0, the
               forward and dQ of rows 0 .. lead-1;
      sampled: heads compared on the given rows and keys;
    and properties checked over every row of every head.  check_alloc: the calls allocate no device
    memory (outputs preallocated; the path's extra HBM is the 12 bytes per row of KL, LSE_t, LSE_s)."""
    print(f"case {w.name} (full size) teacher={teacher} whole={whole} window={window} r0={r0}", flush=True)
    dev_in = device_inputs_bf16_bits(w)
    qt, kt, qs, ks = dev_in
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    gh = wl.full_g(w)
    g = torch.from_numpy(gh).cuda()
    side = "t" if teacher else "s"
    dx = w.d_t if teacher else w.d_s
    kl, lt, ls = (torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda") for _ in range(3))
    dq = torch.empty((w.B, w.H, w.Nq, dx), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.B, w.H, w.Nk, dx), dtype=torch.float32, device="cuda")
    if check_alloc:  # the same kernels once at a small size: code objects and the runtime's per-kernel
        # private memory are set up before the measurement
        sm = tuple(x[:, :1, :256].contiguous() for x in dev_in)
        kls, lts, lss = S.fwd(*sm, **kw)
        S.bwd(*sm, lts, lss, g[:, :1, :256].contiguous(), kl=kls, teacher_grads=teacher, student_grads=not teacher,
              **kw)
        torch.cuda.synchronize()
        free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    S.fwd(qt, kt, qs, ks, out=(kl, lt, ls), **kw)
    if teacher:
        S.bwd(qt, kt, qs, ks, lt, ls, g, kl=kl, teacher_grads=True, student_grads=False, out=[None, None, dq, dk], **kw)
    else:
        S.bwd_dk(qt, kt, qs, ks, lt, ls, g, out=dk, **kw)
        S.bwd_dq(qt, kt, qs, ks, lt, ls, g, out=dq, **kw)
    torch.cuda.synchronize()
    if check_alloc:
        assert torch.cuda.mem_get_info()[0] == free0, "the path allocated device memory"
        assert torch.cuda.memory_allocated() == alloc0
        assert sum(x.numel() * x.element_size() for x in (kl, lt, ls)) == 12 * w.B * w.H * w.Nq
    xq, xk = (qt, kt) if teacher else (qs, ks)  # the side being differentiated
    rt = rtol_of(w)
    # properties over every row
    klc = kl.cpu().numpy()
    assert np.all(np.isfinite(klc)) and bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all())
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
    c = lambda x: x.cpu().numpy()

    def compare(tag, b, h, r, k, ref):
        worst_of(worst, "kl" + tag, ratio_kl(klc[b, h, r], ref["kl"], rt))
        worst_of(worst, "lse" + tag, ratio_lse(c(lt[b, h, r]), ref["lse_t"], rt), ratio_lse(c(ls[b, h, r]), ref["lse_s"], rt))
        worst_of(worst, "dq_" + side + tag, ratio_rows(c(dq[b, h, r]), ref["dq_" + side], rt))
        if k is not None:
            worst_of(worst, "dk_" + side + tag, ratio_rows(c(dk[b, h, k]), ref["dk_" + side], rt))

    for (b, h) in whole:
        hh = wl.head_f64(w, b, h)
        ref = oracle_window(hh, w.scale_t, w.scale_s, w.causal, gh[b, h], teacher=teacher)
        compare("(whole)", b, h, slice(None), slice(None), ref)
    for (b, h) in window:
        hh = wl.head_f64(w, b, h)
        ref = oracle_window(hh, w.scale_t, w.scale_s, w.causal, gh[b, h], r0=r0, teacher=teacher)
        compare(f"(rows {r0}:)", b, h, slice(r0, None), slice(ref["k0"], None), ref)
        if lead:
            ref = oracle_window(tuple(x[:lead] for x in hh), w.scale_t, w.scale_s, w.causal, gh[b, h, :lead],
                                teacher=teacher)
            compare(f"(rows :{lead})", b, h, slice(0, lead), None, ref)
    for (b, h) in sampled:
        hh = wl.head_f64(w, b, h)
        rkl, rlt, rls = oracle.forward_head(*hh, w.scale_t, w.scale_s, w.causal, rows=rows)
        rg = oracle.backward_head(*hh, w.scale_t, w.scale_s, w.causal, gh[b, h], teacher=teacher, rows=rows,
                                  keys=keys)
        compare("(sampled)", b, h, rows, keys, dict(kl=rkl, lse_t=rlt, lse_s=rls, **rg))
    msg = report(w.name, **worst)
    print(msg, flush=True)
    assert all_pass(worst), msg


def _rows(n, seed):
    r = np.random.default_rng(seed).choice(n, 12, replace=False)
    return sorted(set([0, 1, 2, 31, 32, 63, 64, 127, 128, n // 2, n - 2, n - 1] + list(r)))


def test_b1h32n32768_causal_whole_head():
    """The bench workload: head 0 over all 32768 rows and keys (key j's dK sums a causal stream of
    32768 - j query rows, up to 1024 tiles), and sampled rows and keys of two more heads."""
    w = wl.WORKLOADS[3]
    n = w.Nq
    _full_size(w, whole=[(0, 0)], sampled=[(0, 17), (0, 31)], rows=_rows(n, 3),
               keys=[0, 1, 31, 32, n // 4, n // 2, n - 130, n - 1])


def test_b1h32n32768_causal_teacher_gradients_whole_head():
    """The teacher pair at the bench size, launched as the bench's teacher-gradient step launches it:
    head 3 over every row and key."""
    w = wl.WORKLOADS[3]
    _full_size(w, teacher=True, whole=[(0, 3)])


def test_b4h8n8192_two_head_dims_whole_heads():
    """Teacher d = 128, student d = 64, not causal: two whole heads (every key sees all 8192 rows)."""
    w = wl.WORKLOADS[4]
    _full_size(w, whole=[(0, 0), (3, 7)])


def test_b1h8n131072_causal_long_streams_and_no_allocation():
    """The 131072-row workload as the bench runs it, with no device allocation by the path: head 5
    over its last 16384 rows and keys (dK of key 131072 - 16384 sums a stream of 16384 rows, 512
    tiles; every dQ row there streams over 114688 or more keys) and its first 1024 rows."""
    w = wl.WORKLOADS[5]
    _full_size(w, window=[(0, 5)], r0=w.Nq - 16384, lead=1024, check_alloc=True)


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
    assert all_pass(r), msg


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
    assert all_pass(r), msg


@pytest.mark.parametrize("alpha,beta,N", [(8.0, 8.0, 160), (2.0, 2.0, 160), (8.0, -0.5, 160), (8.0, 8.0, 640),
                                          (7.0, 7.0, 90)])
def test_teacher_and_student_logits_far_apart(alpha, beta, N):
    """bf16 with equal scales takes the forward's difference chain, whose two sides share one
    power-of-two reference.  Rows whose teacher logits sit near +alpha * 8 nats and student logits
    near -beta * 8 nats (keys clustered around one direction u, teacher queries along +u, student
    queries along -u): at (8, 8) the student's sum sinks about 180 binades below the teacher's, which
    the kernel must notice and rerun with separate running maxima; (2, 2) and (8, -0.5) stay on the fast
    path; (8, 8) at 640 rows takes the rerun over rows of up to 20 tiles.  (7, 7) at 90 rows puts one head's gap between the two log-sum-exps at 137-141
    binades: after the only renormalisation of a three-tile row the student's sum against the shared
    reference is a denormal, not zero, which must also send the row to the rerun (it gave -inf
    before each lane half's smaller sum was checked against the shared reference).  Against the float64 oracle, with the float32 rounding of logits of this size
    added to the criteria as in test_extreme_logits_take_the_exact_path.

    The keys cluster around u, so a gradient row sum_j dS_ij k_j cancels its u component about
    tenfold and the relative criterion does not apply to it: the bf16 backward rounds dS once to fp16
    (2^-11 relative per element), an error bound of 2^-11 scale sum_j |dS_ij| |k_j| per row whatever the
    cancellation.  The gradients are held to 2^-10 times that sum (plus the relative term), computed
    here in float64 from the two softmaxes of the definition."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([72, int(alpha * 10), int(beta * 10) + 50] + ([N] if N != 160 else []))))
    B, H, d = 1, 2, 64
    u = rng.standard_normal((B, H, 1, d))
    k = u + 0.1 * rng.standard_normal((B, H, N, d))
    qt = alpha * u + 0.3 * rng.standard_normal((B, H, N, d))
    qs = -beta * u + 0.3 * rng.standard_normal((B, H, N, d))
    dev = [torch.from_numpy(a.astype(np.float32)).cuda().to(torch.bfloat16) for a in (qt, k, qs, k)]
    host = [x.float().cpu().numpy().astype(np.float64) for x in dev]
    print(f"case logits far apart alpha={alpha} beta={beta}", flush=True)
    sc = 0.125
    kl, lt, ls = S.fwd(*dev, causal=True, scale_t=sc, scale_s=sc)
    g = torch.ones_like(kl)
    dq, dk, _, _ = S.bwd(*dev, lt, ls, g, causal=True, scale_t=sc, scale_s=sc)
    torch.cuda.synchronize()
    rkl, rlt, rls = oracle.forward(*host, sc, sc, True)
    rg = oracle.backward(*host, sc, sc, True, np.ones((B, H, N)))
    rt = 2e-3
    L = max(float(np.abs(host[0] @ host[1].transpose(0, 1, 3, 2)).max()),
            float(np.abs(host[2] @ host[3].transpose(0, 1, 3, 2)).max()))  # largest raw logit
    kl_abs = 4.0 * sc * L * math.sqrt(d) * 2.0 ** -24
    rt_g = max(rt, sc * L * math.sqrt(d) * 2.0 ** -22)
    c = lambda x: x.cpu().numpy()
    for x in (kl, lt, ls, dq, dk):
        assert np.all(np.isfinite(c(x)))
    rms = np.maximum(np.sqrt((rkl ** 2).mean(axis=-1, keepdims=True)), 1e-3)
    kl_ratio = float((np.abs(c(kl) - rkl) / (rt * np.abs(rkl) + rt * rms + kl_abs)).max())
    # |dS| of the definition (g = 1): softmaxes of the causal rows in float64
    mask = np.tril(np.ones((N, N), bool))
    def softmax(q, kk):
        a = np.where(mask, sc * q @ kk.transpose(0, 1, 3, 2), -np.inf)
        a = a - a.max(-1, keepdims=True)
        e = np.exp(a)
        return e / e.sum(-1, keepdims=True)
    ads = np.abs(softmax(host[2], host[3]) - softmax(host[0], host[1]))
    kn, qn = np.linalg.norm(host[3], axis=-1), np.linalg.norm(host[2], axis=-1)
    bound_q = 2.0 ** -10 * sc * (ads * kn[:, :, None, :]).sum(-1)   # per query row
    bound_k = 2.0 ** -10 * sc * (ads * qn[:, :, :, None]).sum(-2)   # per key row

    def ratio_bound(got, ref, bound, floor):
        # the usual per-row criterion (relative to the row and to the head's rms row) plus the bound
        err = np.linalg.norm(got - ref, axis=-1)
        rn = np.linalg.norm(ref, axis=-1)
        rms = np.maximum(np.sqrt((rn ** 2).mean(axis=-1, keepdims=True)), floor)
        return float((err / (rt_g * rn + rt_g * rms + bound + 1e-30)).max())
    ones = np.ones((B, H, N))
    r = dict(kl=kl_ratio, lse_t=ratio_lse(c(lt), rlt, rt_g), lse_s=ratio_lse(c(ls), rls, rt_g),
             dq=ratio_bound(c(dq), rg["dq_s"], bound_q, grad_floor(sc, ones, host[3])),
             dk=ratio_bound(c(dk), rg["dk_s"], bound_k, grad_floor(sc, ones, host[2])))
    msg = report(f"logits far apart {alpha} {beta} N={N}", **r)
    print(msg, flush=True)
    assert all_pass(r), msg

"""GPU parity of the Jensen-Shannon kernels (streamkl_js_fwd / streamkl_js_bwd) against the float64
oracle's js_forward / js_backward, with the tolerances and criteria of the KL parity tests.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import loss as L
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import (all_pass, oracle_window, worst_of, device_inputs, device_inputs_bf16_bits, grad_floor, ratio_kl, ratio_lse, ratio_rows, report,
                    rtol_of)

pytestmark = pytest.mark.gpu


def _check(w, teacher, g=None):
    print(f"case {w.name} js teacher={teacher}", flush=True)
    dev_in, host = device_inputs(w)
    qt, kt, qs, ks = dev_in
    g = wl.full_g(w) if g is None else g
    js, lt, ls, ht = S.js_fwd(qt, kt, qs, ks, causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    grads = S.js_bwd(qt, kt, qs, ks, lt, ls, js, ht, torch.from_numpy(g).cuda(), causal=w.causal,
                     teacher_grads=teacher, scale_t=w.scale_t, scale_s=w.scale_s)
    torch.cuda.synchronize()
    for x in (js, ht, lt, ls, *grads):
        assert x is None or bool(torch.isfinite(x).all()), "non-finite output"
    h64 = [a.astype(np.float64) for a in host]
    rjs, rht, _, rlt, rls = oracle.js_forward(*h64, w.scale_t, w.scale_s, w.causal)
    rg = oracle.js_backward(*h64, w.scale_t, w.scale_s, w.causal, g.astype(np.float64), teacher=teacher)
    rt = rtol_of(w)
    ag = np.abs(g)
    c = lambda x: x.cpu().numpy()
    r = dict(js=ratio_kl(c(js), rjs, rt), js_t=ratio_kl(c(ht), rht, rt), lse_t=ratio_lse(c(lt), rlt, rt),
             lse_s=ratio_lse(c(ls), rls, rt),
             dq_s=ratio_rows(c(grads[0]), rg["dq_s"], rt, grad_floor(0.5 * w.scale_s, ag, h64[3])),
             dk_s=ratio_rows(c(grads[1]), rg["dk_s"], rt, grad_floor(0.5 * w.scale_s, ag, h64[2])))
    if teacher:
        r.update(dq_t=ratio_rows(c(grads[2]), rg["dq_t"], rt, grad_floor(0.5 * w.scale_t, ag, h64[1])),
                 dk_t=ratio_rows(c(grads[3]), rg["dk_t"], rt, grad_floor(0.5 * w.scale_t, ag, h64[0])))
    msg = report(w.name + " js", **r)
    print(msg, flush=True)
    assert all_pass(r), msg
    jsv = c(js)
    assert np.all(jsv >= -1e-6) and np.all(jsv <= math.log(2.0) + 1e-6)


CASES = [
    wl.custom(1, 2, 129, 129, 128, 128, True, seed=51),
    wl.custom(1, 1, 3, 3, 64, 64, True, seed=52),
    wl.custom(2, 1, 200, 257, 128, 64, True, recipe="independent", seed=53),
    wl.custom(1, 2, 70, 300, 64, 128, False, recipe="independent", seed=54),
    wl.custom(1, 2, 255, 255, 128, 128, True, sigma=0.1, seed=55),          # nearly equal rows: small JS
    wl.custom(1, 1, 200, 200, 128, 128, True, recipe="independent", peak_frac=0.02, peak_scale=4.0, seed=56),
    wl.custom(1, 2, 100, 100, 64, 64, True, dtype="fp32", recipe="independent", seed=57),
    wl.custom(1, 1, 33, 90, 128, 64, False, dtype="fp32", recipe="independent", seed=58),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_js_matches_the_oracle(w):
    _check(w, teacher=True)


def test_js_signed_row_weights():
    w = wl.custom(1, 2, 160, 160, 128, 128, True, recipe="independent", seed=59)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 7])))
    g = rng.standard_normal((w.B, w.H, w.Nq)).astype(np.float32)
    g[..., ::5] = 0.0
    _check(w, teacher=True, g=g)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_js_zero_row_weights_stay_finite(dtype):
    """Rows with g = 0 (a masked or sliced reduction): the key owner folds log2|g| into the streamed
    queries' exponents, and for such rows both probabilities must come out as exact zeros without
    an inf - inf in the JS log-ratio.  Whole 32-row tiles of zeros, single zero rows and signed
    weights in one problem; every gradient finite and equal to the oracle's."""
    w = wl.custom(1, 2, 200, 200, 128, 64, True, dtype=dtype, recipe="independent", seed=67)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 8])))
    g = rng.uniform(0.5, 1.5, (w.B, w.H, w.Nq)).astype(np.float32)
    g[..., 32:96] = 0.0
    g[..., ::7] = 0.0
    g[..., 150:160] *= -1.0
    _check(w, teacher=True, g=g)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_rows_give_exact_zeros(causal):
    w = wl.custom(1, 2, 150, 150, 128, 128, causal, recipe="same", seed=60)
    print(f"case {w.name} js same", flush=True)
    dev_in, _ = device_inputs(w)
    js, lt, ls, ht = S.js_fwd(*dev_in, causal=causal)
    grads = S.js_bwd(*dev_in, lt, ls, js, ht, torch.ones_like(js), causal=causal, teacher_grads=True)
    torch.cuda.synchronize()
    assert torch.all(js == 0.0) and torch.all(ht == 0.0)
    for x in grads:
        assert torch.all(x == 0.0)


def test_js_on_packed_and_grouped_inputs():
    """One packed batch with grouped student keys, each segment against the oracle on its own."""
    H, hk_s = 4, 2
    lens = [90, 1, 257]
    segs = [wl.custom(1, H, n, n, 128, 128, True, recipe="independent", seed=61 + i) for i, n in enumerate(lens)]
    print(f"case packed js {lens} hk_s={hk_s}", flush=True)
    hosts = [[a.astype(np.float64) for a in wl.full_f32(w)] for w in segs]
    for h in hosts:
        h[3] = h[3][:, ::H // hk_s]

    def pack(i):
        cat = np.concatenate([h[i][0] for h in hosts], axis=1)  # [heads, N, d]
        return torch.from_numpy(np.ascontiguousarray(cat.transpose(1, 0, 2))).float().to(torch.bfloat16).cuda()
    qt, kt, qs, ks = (pack(i) for i in range(4))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32).cuda()
    seg = dict(cu_seqlens_q=cu, cu_seqlens_k=cu)
    js, lt, ls, ht = S.js_fwd(qt, kt, qs, ks, causal=True, **seg)
    g = torch.from_numpy(np.concatenate([wl.full_g(w)[0] for w in segs], axis=1)).cuda()
    dq, dk, _, _ = S.js_bwd(qt, kt, qs, ks, lt, ls, js, ht, g, causal=True, **seg)
    torch.cuda.synchronize()
    js, dq, dk = js.cpu().numpy(), dq.cpu().numpy(), dk.cpu().numpy()
    q0 = 0
    worst = {}
    for w, h, n in zip(segs, hosts, lens):
        eks = np.repeat(h[3], H // hk_s, axis=1)
        rjs = oracle.js_forward(h[0], h[1], h[2], eks, w.scale_t, w.scale_s, True)[0]
        gw = wl.full_g(w)
        rg = oracle.js_backward(h[0], h[1], h[2], eks, w.scale_t, w.scale_s, True, gw)
        rdk = rg["dk_s"].reshape(1, hk_s, H // hk_s, n, -1).sum(axis=2)
        r = dict(js=ratio_kl(js[None, :, q0:q0 + n], rjs, 2e-3),
                 dq=ratio_rows(dq[None, :, q0:q0 + n], rg["dq_s"], 2e-3, grad_floor(0.5 * w.scale_s, gw, eks)),
                 dk=ratio_rows(dk[None, :, q0:q0 + n], rdk, 2e-3, grad_floor(0.5 * w.scale_s, gw, h[2])))
        for k, v in r.items():
            worst[k] = max(worst.get(k, 0.0), v)
        q0 += n
    msg = report("packed js", **worst)
    print(msg, flush=True)
    assert all_pass(worst), msg


def test_autograd_js_direction():
    w = wl.custom(1, 2, 96, 96, 128, 128, True, recipe="independent", seed=65)
    print(f"case {w.name} autograd js", flush=True)
    dev_in, host = device_inputs(w)
    ins = [x.clone().requires_grad_(True) for x in dev_in]
    out = L.attention_kl(*ins, causal=True, scale_t=w.scale_t, scale_s=w.scale_s, direction="js", reduction="sum")
    out.backward()
    torch.cuda.synchronize()
    h64 = [a.astype(np.float64) for a in host]
    rjs = oracle.js_forward(*h64, w.scale_t, w.scale_s, True)[0]
    ones = np.ones((w.B, w.H, w.Nq))
    rg = oracle.js_backward(*h64, w.scale_t, w.scale_s, True, ones, teacher=True)
    assert abs(out.item() - rjs.sum()) <= 2e-3 * abs(rjs.sum())
    rt = 2e-3 + 2.0 ** -9  # bf16 gradients
    for x, name, other, sc in ((ins[0], "dq_t", h64[1], w.scale_t), (ins[1], "dk_t", h64[0], w.scale_t),
                               (ins[2], "dq_s", h64[3], w.scale_s), (ins[3], "dk_s", h64[2], w.scale_s)):
        assert ratio_rows(x.grad.float().cpu().numpy(), rg[name], rt, grad_floor(0.5 * sc, ones, other)) <= 1.0, name


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_js_grouped_keys_with_teacher_gradients(dtype):
    """Grouped keys on both sides (teacher 2 key heads, student 1) with both gradient pairs: the
    key-owner kernels make one pass per query head of the group; the oracle runs on keys expanded to
    every query head, the expanded heads' dK summed per group."""
    H, hk_t, hk_s = 4, 2, 1
    w = wl.custom(1, H, 150, 150, 64, 64, True, dtype=dtype, recipe="independent", seed=66)
    print(f"case {w.name} js hk_t={hk_t} hk_s={hk_s}", flush=True)
    dev_in, host = device_inputs(w)
    qt, kt, qs, ks = dev_in
    kt, ks = kt[:, ::H // hk_t], ks[:, ::H // hk_s]
    h64 = [a.astype(np.float64) for a in host]
    ekt = np.repeat(h64[1][:, ::H // hk_t], H // hk_t, axis=1)
    eks = np.repeat(h64[3][:, ::H // hk_s], H // hk_s, axis=1)
    g = wl.full_g(w)
    js, lt, ls, ht = S.js_fwd(qt, kt, qs, ks, causal=True)
    grads = S.js_bwd(qt, kt, qs, ks, lt, ls, js, ht, torch.from_numpy(g).cuda(), causal=True, teacher_grads=True)
    torch.cuda.synchronize()
    rjs = oracle.js_forward(h64[0], ekt, h64[2], eks, w.scale_t, w.scale_s, True)[0]
    rg = oracle.js_backward(h64[0], ekt, h64[2], eks, w.scale_t, w.scale_s, True, g, teacher=True)
    rt = rtol_of(w)

    def sumg(x, hk):
        return x.reshape(1, hk, H // hk, w.Nk, -1).sum(axis=2)
    c = lambda x: x.cpu().numpy()
    r = dict(js=ratio_kl(c(js), rjs, rt),
             dq_s=ratio_rows(c(grads[0]), rg["dq_s"], rt, grad_floor(0.5 * w.scale_s, g, eks)),
             dk_s=ratio_rows(c(grads[1]), sumg(rg["dk_s"], hk_s), rt, grad_floor(0.5 * w.scale_s, g, h64[2])),
             dq_t=ratio_rows(c(grads[2]), rg["dq_t"], rt, grad_floor(0.5 * w.scale_t, g, ekt)),
             dk_t=ratio_rows(c(grads[3]), sumg(rg["dk_t"], hk_t), rt, grad_floor(0.5 * w.scale_t, g, h64[0])))
    msg = report(f"js grouped {dtype}", **r)
    print(msg, flush=True)
    assert all_pass(r), msg


def test_js_b1h32n32768_causal_full_size():
    """The Jensen-Shannon step at the bench size, launched as `bench.py --divergence js` launches it:
    properties over every row and head, head 0 against the oracle over every row and key, and
    sampled rows and keys (early and late) of head 21."""
    w = wl.WORKLOADS[3]
    n = w.Nq
    print(f"case {w.name} js (full size)", flush=True)
    qt, kt, qs, ks = device_inputs_bf16_bits(w)
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    js, lt, ls, ht = S.js_fwd(qt, kt, qs, ks, **kw)
    gh = wl.full_g(w)
    dq, dk, _, _ = S.js_bwd(qt, kt, qs, ks, lt, ls, js, ht, torch.from_numpy(gh).cuda(), **kw)
    torch.cuda.synchronize()
    rt = rtol_of(w)
    jsv, htv = js.cpu().numpy(), ht.cpu().numpy()
    assert np.all(np.isfinite(jsv)) and bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all())
    assert jsv.min() >= -1e-6 and jsv.max() <= math.log(2.0) + 1e-6
    assert np.abs(jsv[:, :, 0]).max() <= 1e-6  # one allowed key: both rows are that key, JS = 0
    # each half KL(P || M) lies in [0, ln 2] and JS is their mean, so the teacher half is at most 2 JS
    assert htv.min() >= -1e-6 and np.all(htv <= 2.0 * jsv + 1e-5)
    # sum_i q_i . dQ_i = sum_j k_j . dK_j per head (both are s_s sum_ij dS_ij q_i . k_j)
    lhs = (qs.double() * dq.double()).sum(dim=(2, 3))
    rhs = (ks.double() * dk.double()).sum(dim=(2, 3))
    norm = (qs.double().norm(dim=3) * dq.double().norm(dim=3)).sum(dim=2) + \
        (ks.double().norm(dim=3) * dk.double().norm(dim=3)).sum(dim=2)
    assert float(((lhs - rhs).abs() / norm).max()) <= rt
    extra = np.random.default_rng(7).choice(n, 12, replace=False)
    rows = sorted(set([0, 1, 2, 31, 32, 63, 64, 127, 128, n // 2, n - 2, n - 1] + list(extra)))
    keys = [0, 1, n // 4, n // 2, n - 1, n - 2, n - 31, n - 32, n - 64, n - 65, n - 130]
    worst = {}
    c = lambda x: x.cpu().numpy()
    # head 0 whole: every row and every key (key 0's dK sums all 32768 rows)
    ref = oracle_window(wl.head_f64(w, 0, 0), w.scale_t, w.scale_s, w.causal, gh[0, 0], js=True)
    worst_of(worst, "js(whole)", ratio_kl(jsv[0, 0], ref["js"], rt))
    worst_of(worst, "js_t(whole)", ratio_kl(htv[0, 0], ref["js_t"], rt))
    worst_of(worst, "lse(whole)", ratio_lse(c(lt[0, 0]), ref["lse_t"], rt), ratio_lse(c(ls[0, 0]), ref["lse_s"], rt))
    worst_of(worst, "dq_s(whole)", ratio_rows(c(dq[0, 0]), ref["dq_s"], rt))
    worst_of(worst, "dk_s(whole)", ratio_rows(c(dk[0, 0]), ref["dk_s"], rt))
    for (b, h) in [(0, 21)]:
        hh = wl.head_f64(w, b, h)
        rjs, rht, _, rlt, rls = oracle.js_forward_head(*hh, w.scale_t, w.scale_s, w.causal, rows=rows)
        worst_of(worst, "js", ratio_kl(jsv[b, h, rows], rjs, rt))
        worst_of(worst, "js_t", ratio_kl(htv[b, h, rows], rht, rt))
        worst_of(worst, "lse", ratio_lse(lt[b, h, rows].cpu().numpy(), rlt, rt),
                 ratio_lse(ls[b, h, rows].cpu().numpy(), rls, rt))
        rg = oracle.js_backward_head(*hh, w.scale_t, w.scale_s, w.causal, gh[b, h], rows=rows, keys=keys)
        worst_of(worst, "dq_s", ratio_rows(dq[b, h, rows].cpu().numpy(), rg["dq_s"], rt))
        worst_of(worst, "dk_s", ratio_rows(dk[b, h, keys].cpu().numpy(), rg["dk_s"], rt))
    msg = report(w.name + " js", **worst)
    print(msg, flush=True)
    assert all_pass(worst), msg

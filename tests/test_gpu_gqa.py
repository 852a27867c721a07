"""GPU parity of grouped key heads: query head h reads key head h // (H // Hk) of each side.

The oracle knows nothing of key heads.  It runs on the keys expanded to one head per query head,
and the gradient of a shared key head is the sum of the expanded heads' gradients: that is the
chain rule for one input used by several heads, applied here in the test, outside the oracle.
Inputs: the usual seeded workload with H heads; key head j of a side is that side's generated
head j * (H // Hk), passed to the library as a strided view (head stride (H // Hk) * Nk * d).
Tolerances and criteria are those of the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import loss as L
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import all_pass, oracle_window, worst_of, device_inputs, grad_floor, ratio_kl, ratio_lse, ratio_rows, report, rtol_of

pytestmark = pytest.mark.gpu


def _grouped_inputs(w, hk_t, hk_s):
    dev_in, host = device_inputs(w)
    gt, gs = w.H // hk_t, w.H // hk_s
    qt, kt, qs, ks = dev_in
    dev = (qt, kt[:, ::gt], qs, ks[:, ::gs])
    h64 = [a.astype(np.float64) for a in host]
    kt_g, ks_g = h64[1][:, ::gt], h64[3][:, ::gs]
    expanded = (h64[0], np.repeat(kt_g, gt, axis=1), h64[2], np.repeat(ks_g, gs, axis=1))
    return dev, expanded, (gt, gs)


def _sum_groups(dk, g):
    B, H, N, d = dk.shape
    return dk.reshape(B, H // g, g, N, d).sum(axis=2)


CASES = [
    # (workload, Hk_t, Hk_s, teacher gradients)
    (wl.custom(1, 4, 129, 129, 128, 128, True, seed=31), 2, 1, False),
    (wl.custom(2, 4, 70, 200, 128, 64, True, recipe="independent", seed=32), 4, 2, True),
    (wl.custom(1, 6, 100, 100, 64, 64, False, dtype="fp32", recipe="independent", seed=33), 3, 2, True),
    (wl.custom(1, 8, 257, 257, 64, 128, False, recipe="independent", seed=34), 1, 8, True),
    (wl.custom(1, 2, 33, 300, 128, 128, True, recipe="independent", seed=35), 1, 1, True),
]


@pytest.mark.parametrize("w,hk_t,hk_s,teacher", CASES,
                         ids=[f"{c[0].name}-hkt{c[1]}-hks{c[2]}" for c in CASES])
def test_grouped_key_heads_match_the_expanded_oracle(w, hk_t, hk_s, teacher):
    print(f"case {w.name} Hk_t={hk_t} Hk_s={hk_s} teacher={teacher}", flush=True)
    (qt, kt, qs, ks), h64, (gt, gs) = _grouped_inputs(w, hk_t, hk_s)
    assert kt.shape[1] == hk_t and ks.shape[1] == hk_s
    kl, lt, ls = S.fwd(qt, kt, qs, ks, causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    g = wl.full_g(w)
    grads = S.bwd(qt, kt, qs, ks, lt, ls, torch.from_numpy(g).cuda(), causal=w.causal, kl=kl, teacher_grads=teacher,
                  scale_t=w.scale_t, scale_s=w.scale_s)
    torch.cuda.synchronize()
    assert grads[1].shape == (w.B, hk_s, w.Nk, w.d_s)
    rkl, rlt, rls = oracle.forward(*h64, w.scale_t, w.scale_s, w.causal)
    rg = oracle.backward(*h64, w.scale_t, w.scale_s, w.causal, g, teacher=teacher)
    rt = rtol_of(w)
    cpu = [x.cpu().numpy() if x is not None else None for x in grads]
    r = dict(kl=ratio_kl(kl.cpu().numpy(), rkl, rt), lse_t=ratio_lse(lt.cpu().numpy(), rlt, rt),
             lse_s=ratio_lse(ls.cpu().numpy(), rls, rt),
             dq_s=ratio_rows(cpu[0], rg["dq_s"], rt, grad_floor(w.scale_s, g, h64[3])),
             dk_s=ratio_rows(cpu[1], _sum_groups(rg["dk_s"], gs), rt, grad_floor(w.scale_s, g, h64[2])))
    if teacher:
        assert cpu[3].shape == (w.B, hk_t, w.Nk, w.d_t)
        r.update(dq_t=ratio_rows(cpu[2], rg["dq_t"], rt, grad_floor(w.scale_t, g, h64[1])),
                 dk_t=ratio_rows(cpu[3], _sum_groups(rg["dk_t"], gt), rt, grad_floor(w.scale_t, g, h64[0])))
    msg = report(w.name, **r)
    print(msg, flush=True)
    assert all_pass(r), msg


def test_grouped_keys_equal_explicitly_repeated_keys_in_the_forward():
    """The forward reads key head h // G: the same bits as the keys repeated to H heads."""
    w = wl.custom(2, 4, 190, 190, 128, 128, True, recipe="independent", seed=36)
    print(f"case {w.name}", flush=True)
    (qt, kt, qs, ks), _, (gt, gs) = _grouped_inputs(w, 2, 1)
    a = S.fwd(qt, kt, qs, ks, causal=True)
    b = S.fwd(qt, kt.repeat_interleave(gt, dim=1), qs, ks.repeat_interleave(gs, dim=1), causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_with_grouped_student_keys():
    """The loss wrapper passes grouped keys through: k_s.grad has the key heads' shape."""
    w = wl.custom(1, 4, 64, 64, 128, 128, True, recipe="independent", seed=37)
    print(f"case {w.name}", flush=True)
    (qt, kt, qs, ks), h64, (gt, gs) = _grouped_inputs(w, 4, 2)
    qs = qs.clone().requires_grad_()
    ks = ks.clone().requires_grad_()
    L.attention_kl(qt, kt, qs, ks, causal=True, scale_t=w.scale_t, scale_s=w.scale_s, reduction="sum").backward()
    torch.cuda.synchronize()
    assert ks.grad.shape == ks.shape
    rg = oracle.backward(*h64, w.scale_t, w.scale_s, True, np.ones((w.B, w.H, w.Nq)))
    rt = 2e-3 + 2.0 ** -9  # bf16 gradients come back rounded to bf16
    ones = np.ones((w.B, w.H, w.Nq))
    assert ratio_rows(ks.grad.float().cpu().numpy(), _sum_groups(rg["dk_s"], gs), rt,
                      grad_floor(w.scale_s, ones, h64[2])) <= 1.0
    assert ratio_rows(qs.grad.float().cpu().numpy(), rg["dq_s"], rt, grad_floor(w.scale_s, ones, h64[3])) <= 1.0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_workspace_arrangements_agree_and_repeat_bitwise(dtype):
    """The three key-owner arrangements for grouped keys, through the raw ABI: a full workspace (the
    ungrouped kernel over every query head, then the group sums), a workspace of four partial dK (each
    group's passes split four ways), and none (one workgroup per group).  Each gives the same bits on
    every run; they agree with each other to within float32 summation order, and with the oracle."""
    import ctypes
    w = wl.custom(1, 8, 300, 300, 128, 128, True, dtype=dtype, recipe="independent", seed=38)
    print(f"case {w.name} workspace arrangements", flush=True)
    (qt, kt, qs, ks), h64, (gt, gs) = _grouped_inputs(w, 8, 1)
    kl, lt, ls = S.fwd(qt, kt, qs, ks, causal=True)
    g = torch.from_numpy(wl.full_g(w)).cuda()
    p = S.make_problem(qt, kt, qs, ks, True)
    part = 1 * 1 * 300 * 128                     # one key head's dK
    assert S.lib().streamkl_workspace_floats(ctypes.byref(p)) == 8 * part  # an ungrouped dK (8 heads)

    def run(n_ws):
        dk = torch.empty(1, 1, 300, 128, device="cuda")
        ws = torch.empty(max(n_ws, 1), device="cuda")
        p.workspace, p.workspace_floats = (ws.data_ptr(), n_ws) if n_ws else (None, 0)
        st = S.lib().streamkl_bwd_dk(ctypes.byref(p), qt.data_ptr(), kt.data_ptr(), qs.data_ptr(), ks.data_ptr(),
                                     lt.data_ptr(), ls.data_ptr(), g.data_ptr(), dk.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        assert st == S.OK
        torch.cuda.synchronize()
        return dk.cpu().numpy()
    full, full2 = run(8 * part), run(8 * part)
    split, split2 = run(4 * part), run(4 * part)
    none = run(0)
    np.testing.assert_array_equal(full, full2)
    np.testing.assert_array_equal(split, split2)
    rg = oracle.backward(*h64, w.scale_t, w.scale_s, True, wl.full_g(w))
    ref = rg["dk_s"].reshape(1, 1, 8, 300, 128).sum(axis=2)
    rt = rtol_of(w)
    floor = grad_floor(w.scale_s, wl.full_g(w), h64[2])
    for x in (full, split, none):
        assert ratio_rows(x, ref, rt, floor) <= 1.0
        assert np.abs(x - none).max() <= 1e-5 * np.abs(none).max()  # float32 summation order only


@pytest.mark.parametrize("hk_s", [8, 1])
def test_grouped_student_keys_full_size(hk_s):
    """The bench workload with K student key heads, as `bench.py --student-key-heads K` launches it
    (key head j = the workload's student head j H/K, a strided view; the binding's workspace):
    a window of the last rows of every query head of one group, and the dK of those keys of its key
    head summed over the whole group."""
    from parity import device_inputs_bf16_bits
    w = wl.WORKLOADS[3]
    n, G = w.Nq, w.H // hk_s
    print(f"case {w.name} Hk_s={hk_s} (full size)", flush=True)
    qt, kt, qs, ks = device_inputs_bf16_bits(w)
    ks = ks[:, ::G]
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    kl, lt, ls = S.fwd(qt, kt, qs, ks, **kw)
    gh = wl.full_g(w)
    dq, dk, _, _ = S.bwd(qt, kt, qs, ks, lt, ls, torch.from_numpy(gh).cuda(), **kw)
    torch.cuda.synchronize()
    assert dk.shape == (1, hk_s, n, w.d_s)
    assert bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all()) and bool(torch.isfinite(kl).all())
    rt = rtol_of(w)
    # rows r0 .. n-1 of every query head of the last key head's group: their forward and dQ, and dK of
    # keys r0 .. n-1 of that key head summed over the group (complete: causal, every row that sees
    # those keys is in the window).  Eight query heads' windows of 8192 rows for K = 8 (four per
    # group: streams of up to 256 tiles), 1024 rows of all 32 for K = 1.
    r0 = n - (8192 if G <= 4 else 1024)
    j = hk_s - 1  # the last key head: query heads j G .. j G + G - 1
    ks_j = wl.head_f64(w, 0, j * G)[3]
    worst, rdk = {}, 0.0
    c = lambda x: x.cpu().numpy()
    for h in range(j * G, j * G + G):
        qt_h, kt_h, qs_h, _ = wl.head_f64(w, 0, h)
        ref = oracle_window((qt_h, kt_h, qs_h, ks_j), w.scale_t, w.scale_s, w.causal, gh[0, h], r0=r0)
        rdk = rdk + ref["dk_s"]
        worst_of(worst, "kl", ratio_kl(c(kl[0, h, r0:]), ref["kl"], rt))
        worst_of(worst, "lse", ratio_lse(c(lt[0, h, r0:]), ref["lse_t"], rt), ratio_lse(c(ls[0, h, r0:]), ref["lse_s"], rt))
        worst_of(worst, "dq_s", ratio_rows(c(dq[0, h, r0:]), ref["dq_s"], rt))
    worst_of(worst, "dk_s", ratio_rows(c(dk[0, j, r0:]), rdk, rt))
    msg = report(f"{w.name} Hk_s={hk_s}", **worst)
    print(msg, flush=True)
    assert all_pass(worst), msg

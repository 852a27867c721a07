"""GPU: the autograd loss (attention_kl_amd.loss) on the HIP library against the float64 oracle.

Directions, reductions and gradient combinations run through torch autograd on the real kernels.
References: the oracle's KL(P_t || P_s) and its gradients; the reverse direction is the same
definition with the two sides exchanged (so its student gradients are the exchanged problem's
teacher gradients).  Tolerances as in the parity tests (2e-3 bf16, 1e-5 fp32, same floors); bf16
inputs get bf16 gradients from autograd, so their gradient check adds bf16's half-ulp, 2^-9.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import loss as L
from attention_kl_amd import workloads as wl

from parity import device_inputs, grad_floor, ratio_kl, ratio_rows

pytestmark = pytest.mark.gpu

CASES = [
    wl.custom(1, 2, 70, 96, 64, 128, True, dtype="fp32", recipe="independent", seed=11),
    wl.custom(2, 1, 129, 129, 128, 128, True, dtype="bf16", recipe="noise", sigma=0.3, seed=12),
    wl.custom(1, 2, 64, 64, 128, 64, False, dtype="bf16", recipe="independent", seed=13),
]


def _ref(h64, w, direction, gw):
    """Oracle KL per row and the gradients of sum(gw * KL) for each input (None if absent)."""
    qt, kt, qs, ks = h64
    fwd = lambda a, b, c, d, sa, sb: oracle.forward(a, b, c, d, sa, sb, w.causal)[0]
    bwd = lambda a, b, c, d, sa, sb: oracle.backward(a, b, c, d, sa, sb, w.causal, gw, teacher=True)
    kl = 0.0
    grads = [0.0, 0.0, 0.0, 0.0]
    if direction in ("forward", "symmetric"):
        kl = kl + fwd(qt, kt, qs, ks, w.scale_t, w.scale_s)
        r = bwd(qt, kt, qs, ks, w.scale_t, w.scale_s)
        grads = [grads[0] + r["dq_t"], grads[1] + r["dk_t"], grads[2] + r["dq_s"], grads[3] + r["dk_s"]]
    if direction in ("reverse", "symmetric"):
        kl = kl + fwd(qs, ks, qt, kt, w.scale_s, w.scale_t)
        r = bwd(qs, ks, qt, kt, w.scale_s, w.scale_t)
        grads = [grads[0] + r["dq_s"], grads[1] + r["dk_s"], grads[2] + r["dq_t"], grads[3] + r["dk_t"]]
    return kl, grads


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("direction,reduction,train_teacher", [
    ("forward", "sum", False), ("forward", "mean", True), ("reverse", "batchmean", False),
    ("reverse", "none", True), ("symmetric", "sum", True)])
def test_autograd_loss_matches_oracle(w, direction, reduction, train_teacher):
    print(f"case {w.name} {direction} {reduction} teacher={train_teacher}", flush=True)
    dev_in, host = device_inputs(w)
    ins = [x.clone().requires_grad_(train_teacher if i < 2 else True) for i, x in enumerate(dev_in)]
    out = L.attention_kl(*ins, causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s, direction=direction,
                         reduction=reduction)
    n_rows = w.B * w.H * w.Nq
    weights = {"sum": 1.0, "mean": 1.0 / n_rows, "batchmean": 1.0 / w.B}
    if reduction == "none":
        gw = wl.full_g(w)  # a non-uniform row weighting through torch
        (out * torch.from_numpy(gw).cuda()).sum().backward()
    else:
        gw = np.full((w.B, w.H, w.Nq), weights[reduction])
        out.backward()
    torch.cuda.synchronize()
    h64 = [a.astype(np.float64) for a in host]
    rkl, rgrads = _ref(h64, w, direction, gw)
    rt = 2e-3 if w.dtype == "bf16" else 1e-5
    if reduction == "none":
        assert ratio_kl(out.detach().cpu().numpy(), rkl, rt) <= 1.0
    else:
        # the per-row criterion of the parity tests, summed over the rows the reduction adds up
        red = float((weights[reduction] * rkl).sum())
        rms = max(float(np.sqrt((rkl ** 2).mean())), 1e-3)
        allowed = weights[reduction] * (rt * np.abs(rkl).sum() + rt * n_rows * rms)
        assert abs(out.item() - red) <= allowed
    grt = rt + (2.0 ** -9 if w.dtype == "bf16" else 0.0)
    names = ["q_t", "k_t", "q_s", "k_s"]
    others = [h64[1], h64[0], h64[3], h64[2]]
    scales = [w.scale_t, w.scale_t, w.scale_s, w.scale_s]
    for i, x in enumerate(ins):
        if not x.requires_grad:
            assert x.grad is None
            continue
        assert x.grad is not None and x.grad.dtype == x.dtype, names[i]
        fl = grad_floor(max(scales), gw, others[i]) * (2 if direction == "symmetric" else 1)
        r = ratio_rows(x.grad.float().cpu().numpy(), rgrads[i], grt, fl)
        print(f"  d{names[i]} worst ratio {r:.3f}", flush=True)
        assert r <= 1.0, names[i]

"""GPU parity over a seeded sweep of option combinations: batch, heads, grouped student keys,
ragged lengths, both head dims, causal or not, bf16 or fp32, KL or Jensen-Shannon, student or both
gradient pairs.  Each case is drawn from its own seed and compared with the float64 oracle (grouped
keys expanded to every query head, their gradients summed per group) under the criteria of the other
parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import all_pass, device_inputs, grad_floor, ratio_kl, ratio_lse, ratio_rows, report, rtol_of

pytestmark = pytest.mark.gpu


def _draw(seed):
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 9])))
    B = int(r.integers(1, 3))
    H = int(r.choice([1, 2, 4]))
    hk_s = int(r.choice([h for h in (1, 2, 4) if H % h == 0]))
    causal = bool(r.integers(0, 2))
    nq = int(r.integers(1, 300))
    nk = int(r.integers(nq, 320)) if causal else int(r.integers(1, 320))
    d_t, d_s = int(r.choice([64, 128])), int(r.choice([64, 128]))
    dtype = "bf16" if r.random() < 0.7 else "fp32"
    teacher = bool(r.integers(0, 2))
    js = bool(r.random() < 0.4)
    w = wl.custom(B, H, nq, nk, d_t, d_s, causal, dtype=dtype, recipe="independent", seed=1000 + seed)
    return w, hk_s, teacher, js


SEEDS = list(range(20))


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_matches_the_oracle(seed):
    w, hk_s, teacher, js = _draw(seed)
    print(f"case seed {seed}: {w.name} Hk_s={hk_s} teacher={teacher} js={js}", flush=True)
    (qt, kt, qs, ks), host = device_inputs(w)
    gs = w.H // hk_s
    ks = ks[:, ::gs]
    h64 = [a.astype(np.float64) for a in host]
    eks = np.repeat(h64[3][:, ::gs], gs, axis=1)  # the keys each query head reads
    g = wl.full_g(w)
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    if js:
        out, lt, ls, ht = S.js_fwd(qt, kt, qs, ks, **kw)
        grads = S.js_bwd(qt, kt, qs, ks, lt, ls, out, ht, torch.from_numpy(g).cuda(), teacher_grads=teacher, **kw)
        rout, _, _, rlt, rls = oracle.js_forward(h64[0], h64[1], h64[2], eks, w.scale_t, w.scale_s, w.causal)
        rg = oracle.js_backward(h64[0], h64[1], h64[2], eks, w.scale_t, w.scale_s, w.causal, g, teacher=teacher)
        fs = 0.5  # the JS gradients carry a 1/2 per half
    else:
        out, lt, ls = S.fwd(qt, kt, qs, ks, **kw)
        grads = S.bwd(qt, kt, qs, ks, lt, ls, torch.from_numpy(g).cuda(), kl=out, teacher_grads=teacher, **kw)
        rout, rlt, rls = oracle.forward(h64[0], h64[1], h64[2], eks, w.scale_t, w.scale_s, w.causal)
        rg = oracle.backward(h64[0], h64[1], h64[2], eks, w.scale_t, w.scale_s, w.causal, g, teacher=teacher)
        fs = 1.0
    torch.cuda.synchronize()
    c = lambda x: x.cpu().numpy()
    rt = rtol_of(w)
    ag = np.abs(g)
    rdk_s = rg["dk_s"].reshape(w.B, hk_s, gs, w.Nk, -1).sum(axis=2)
    r = dict(out=ratio_kl(c(out), rout, rt), lse_t=ratio_lse(c(lt), rlt, rt), lse_s=ratio_lse(c(ls), rls, rt),
             dq_s=ratio_rows(c(grads[0]), rg["dq_s"], rt, grad_floor(fs * w.scale_s, ag, eks)),
             dk_s=ratio_rows(c(grads[1]), rdk_s, rt, grad_floor(fs * w.scale_s, ag, h64[2])))
    assert grads[1].shape == (w.B, hk_s, w.Nk, w.d_s)
    if teacher:
        r.update(dq_t=ratio_rows(c(grads[2]), rg["dq_t"], rt, grad_floor(fs * w.scale_t, ag, h64[1])),
                 dk_t=ratio_rows(c(grads[3]), rg["dk_t"], rt, grad_floor(fs * w.scale_t, ag, h64[0])))
    msg = report(f"seed {seed} {w.name}", **r)
    print(msg, flush=True)
    assert all_pass(r), msg

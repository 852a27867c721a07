"""The allocation-free backward (streamkl_bwd_noalloc) through the C ABI: the same results as
streamkl_bwd with a caller workspace, on two calls in a row (the second on a smaller problem, so
the scratch holds the first call's values when it starts), no device memory allocated by the calls,
and problems that need more scratch than the static array rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import all_pass, device_inputs, grad_floor, ratio_rows, report, rtol_of

pytestmark = pytest.mark.gpu


def _grouped(w, hk_t, hk_s):
    dev_in, host = device_inputs(w)
    qt, kt, qs, ks = dev_in
    return (qt, kt[:, ::w.H // hk_t].contiguous(), qs, ks[:, ::w.H // hk_s].contiguous()), host


def _case(w, hk_t, hk_s):
    print(f"case {w.name} hk_t={hk_t} hk_s={hk_s} noalloc", flush=True)
    (qt, kt, qs, ks), host = _grouped(w, hk_t, hk_s)
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    kl, lt, ls = S.fwd(qt, kt, qs, ks, **kw)
    g = torch.from_numpy(wl.full_g(w)).cuda()
    p = S.make_problem(qt, kt, qs, ks, w.causal, w.scale_t, w.scale_s)
    need = S.lib().streamkl_workspace_floats(ctypes.byref(p))
    assert 0 < need <= S.NOALLOC_SCRATCH_FLOATS  # a grouped problem that uses the scratch
    # the existing entry point, with the workspace the binding attaches
    ref = S.bwd(qt, kt, qs, ks, lt, ls, g, kl=kl, teacher_grads=True, **kw)
    torch.cuda.synchronize()
    out = [torch.full_like(x, float("nan")) for x in ref]
    torch.cuda.synchronize()
    free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    S.bwd_noalloc(qt, kt, qs, ks, lt, ls, g, kl=kl, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "the call allocated device memory"
    assert torch.cuda.memory_allocated() == alloc0
    for name, a, b in zip(("dq_s", "dk_s", "dq_t", "dk_t"), out, ref):
        assert torch.equal(a, b), f"{name}: streamkl_bwd_noalloc differs from streamkl_bwd"
    # and both at the parity bar against the oracle (keys expanded to every query head, the expanded
    # heads' dK summed over each key head's group)
    h64 = [a.astype(np.float64) for a in host]
    ekt = np.repeat(h64[1][:, ::w.H // hk_t], w.H // hk_t, axis=1)
    eks = np.repeat(h64[3][:, ::w.H // hk_s], w.H // hk_s, axis=1)
    gh = wl.full_g(w)
    rg = oracle.backward(h64[0], ekt, h64[2], eks, w.scale_t, w.scale_s, w.causal, gh, teacher=True)
    rt = rtol_of(w)

    def sumg(x, hk):
        return x.reshape(w.B, hk, w.H // hk, w.Nk, -1).sum(axis=2)
    c = lambda x: x.cpu().numpy()
    r = dict(dq_s=ratio_rows(c(out[0]), rg["dq_s"], rt, grad_floor(w.scale_s, gh, eks)),
             dk_s=ratio_rows(c(out[1]), sumg(rg["dk_s"], hk_s), rt, grad_floor(w.scale_s, gh, h64[2])),
             dq_t=ratio_rows(c(out[2]), rg["dq_t"], rt, grad_floor(w.scale_t, gh, ekt)),
             dk_t=ratio_rows(c(out[3]), sumg(rg["dk_t"], hk_t), rt, grad_floor(w.scale_t, gh, h64[0])))
    msg = report(w.name + " noalloc", **r)
    print(msg, flush=True)
    assert all_pass(r), msg


def _setup():
    """One call on a small grouped problem: the first call on a device resolves the scratch array's
    device address (and the runtime may load the code object that holds it, with the array); what
    the later calls allocate is measured against that state."""
    w = wl.custom(1, 2, 40, 40, 64, 64, True, recipe="independent", seed=80)
    (qt, kt, qs, ks), _ = _grouped(w, 2, 1)
    kl, lt, ls = S.fwd(qt, kt, qs, ks, causal=True)
    out = [torch.empty(2, 40, 64, device="cuda")[None], torch.empty(1, 40, 64, device="cuda")[None]]
    S.bwd_noalloc(qt, kt, qs, ks, lt, ls, torch.ones_like(kl), causal=True, out=out)
    torch.cuda.synchronize()


def test_noalloc_matches_the_workspace_entry_point_twice():
    """Two calls in a row: a bf16 problem, then a smaller fp32 one."""
    _setup()
    _case(wl.custom(1, 8, 700, 700, 128, 128, True, recipe="independent", seed=81), hk_t=4, hk_s=2)
    _case(wl.custom(2, 4, 300, 300, 64, 64, True, dtype="fp32", recipe="independent", seed=82), hk_t=2, hk_s=1)


def test_noalloc_rejects_what_does_not_fit():
    """Checked on the host before any launch (fake, aligned device addresses are never touched)."""
    L = S.lib()
    p = S.Problem()
    p.B, p.H, p.Nq, p.Nk, p.d_t, p.d_s = 1, 32, 32768, 32768, 128, 128
    p.scale_t = p.scale_s = 0.0883883
    p.causal, p.dtype = 1, S.BF16
    for f in ("stride_qt", "stride_kt", "stride_qs", "stride_ks"):
        getattr(p, f)[:] = [32 * 32768 * 128, 32768 * 128, 128]
    p.Hk_s = 1  # one student key head: the per-query-head dK needs 32 x 32768 x 128 floats
    a = 0x10000
    ptrs = [a + 0x1000 * i for i in range(12)]
    need = L.streamkl_workspace_floats(ctypes.byref(p))
    assert need > S.NOALLOC_SCRATCH_FLOATS
    args = (ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], ptrs[5], None, ptrs[6], ptrs[7], ptrs[8], None, None, None)
    assert L.streamkl_bwd_noalloc(ctypes.byref(p), *args) == S.ERR_SCRATCH
    assert "scratch" in S.status_string(S.ERR_SCRATCH)
    p.workspace, p.workspace_floats = ptrs[9], 1024  # a caller workspace is not taken here
    assert L.streamkl_bwd_noalloc(ctypes.byref(p), *args) == S.ERR_INVALID

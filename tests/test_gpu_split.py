"""The forward of a small causal problem given a workspace splits the key tiles of the later half of each
head's query blocks over two workgroups, and a second kernel merges their row states (streamkl_fwd with
a workspace of streamkl_workspace_floats(p)).  Checked here through the C ABI: the split path writes its
row states (the workspace, filled with NaN first, is written), agrees with the oracle as closely as the
unsplit forward (no workspace), and repeats its bits."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import all_pass, device_inputs, ratio_kl, ratio_lse, report, rtol_of

pytestmark = pytest.mark.gpu

CASES = [
    wl.custom(1, 3, 1100, 1100, 128, 128, True, recipe="independent"),  # 9 query blocks, 5 of them split
    wl.custom(2, 2, 1024, 1500, 128, 128, True, recipe="independent"),  # more keys than queries, 8 blocks
    wl.custom(1, 2, 700, 700, 128, 128, True, sigma=0.1),               # the small-KL regime
    wl.custom(1, 1, 200, 200, 128, 64, True, recipe="independent"),     # two blocks (one split), unequal dims
]


def _fwd(w, x, split):
    """The forward through the C ABI, with (split) or without a workspace; returns host outputs and the
    workspace after the call (None without)."""
    p = S.make_problem(*x, w.causal, w.scale_t, w.scale_s)
    ws = None
    if split:
        n = S.lib().streamkl_workspace_floats(ctypes.byref(p))
        assert n > 0, "a small causal problem asks for the forward's workspace"
        ws = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        p.workspace, p.workspace_floats = ws.data_ptr(), n
    out = [torch.full(p.stat_shape(), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    st = S.lib().streamkl_fwd(ctypes.byref(p), *(t.data_ptr() for t in x), *(o.data_ptr() for o in out),
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == S.OK, S.status_string(st)
    return [o.cpu().numpy() for o in out], (None if ws is None else ws.cpu().numpy())


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_split_forward(w):
    print(f"case split forward {w.name}", flush=True)
    x, host = device_inputs(w)
    (kl, lt, ls), ws = _fwd(w, x, True)
    (kl0, lt0, ls0), _ = _fwd(w, x, False)
    (kl2, lt2, ls2), _ = _fwd(w, x, True)
    # the split blocks' rows went through the workspace: five floats for each of their rows per half
    nqb = (w.Nq + 127) // 128
    nsb = nqb - nqb // 2
    rows = w.B * w.H * nsb * 2 * 5 * 128
    written = np.isfinite(ws[:rows]).reshape(w.B * w.H * nsb, 2, 5, 128)
    last_rows = w.Nq - (nqb - 1) * 128  # the last block may be ragged
    assert written[..., :last_rows].all()
    h64 = [a.astype(np.float64) for a in host]
    rkl, rlt, rls = oracle.forward(*h64, w.scale_t, w.scale_s, w.causal)
    rt = rtol_of(w)
    r = dict(kl=ratio_kl(kl, rkl, rt), lse_t=ratio_lse(lt, rlt, rt), lse_s=ratio_lse(ls, rls, rt),
             kl_unsplit=ratio_kl(kl0, rkl, rt), lse_t_unsplit=ratio_lse(lt0, rlt, rt))
    msg = report(w.name, **r)
    print(msg, flush=True)
    assert all_pass(r), msg
    for a, b in ((kl, kl2), (lt, lt2), (ls, ls2)):  # the same bits again
        assert np.array_equal(a.view(np.int32), b.view(np.int32))

"""Host-side checks of the C ABI: the library loads, exports what the header declares,
and rejects bad arguments before any HIP call (no GPU needed: nothing is launched)."""
import ctypes
import os
import subprocess

import pytest

from attention_kl_amd import streamkl as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    declared = S.declared_symbols()
    assert {"streamkl_fwd", "streamkl_bwd", "streamkl_bwd_dq", "streamkl_bwd_dk", "streamkl_js_fwd", "streamkl_js_bwd",
            "streamkl_status_string",
            "streamkl_version"} <= set(declared)
    L = S.lib()
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported
    assert S.version() == 10700


def test_status_strings():
    for st in (S.OK, S.ERR_INVALID, S.ERR_UNSUPPORTED, S.ERR_LAUNCH, S.ERR_SCRATCH, 99):
        assert S.status_string(st).startswith("STREAMKL")


def _problem(**kw):
    p = S.Problem()
    p.B, p.H, p.Nq, p.Nk, p.d_t, p.d_s = 1, 1, 128, 128, 128, 128
    p.scale_t = p.scale_s = 0.125
    p.causal, p.dtype = 1, S.BF16
    for f in ("stride_qt", "stride_kt", "stride_qs", "stride_ks"):
        getattr(p, f)[:] = [128 * 128, 128 * 128, 128]
    for k, v in kw.items():
        if k.startswith("stride"):
            getattr(p, k)[:] = v
        else:
            setattr(p, k, v)
    return p


# 16-byte aligned fake device addresses: argument checks never dereference them
A = 0x10000
PTRS = [A, A + 0x1000, A + 0x2000, A + 0x3000]
OUTS = [A + 0x4000, A + 0x5000, A + 0x6000]


def fwd_status(p, ptrs=PTRS, outs=OUTS):
    return S.lib().streamkl_fwd(ctypes.byref(p) if p is not None else None, *ptrs, *outs, None)


@pytest.mark.parametrize("kw,expected", [
    (dict(d_t=96), S.ERR_UNSUPPORTED),
    (dict(d_s=32), S.ERR_UNSUPPORTED),
    (dict(dtype=7), S.ERR_UNSUPPORTED),
    (dict(Nq=-1), S.ERR_INVALID),
    (dict(Nq=200, Nk=100), S.ERR_INVALID),  # causal needs Nq <= Nk
    (dict(Nk=0), S.ERR_INVALID),
    (dict(causal=2), S.ERR_INVALID),
    (dict(scale_t=0.0), S.ERR_INVALID),
    (dict(scale_s=float("nan")), S.ERR_INVALID),
    (dict(scale_t=float("inf")), S.ERR_INVALID),
    (dict(stride_qt=[1, 1, 3]), S.ERR_UNSUPPORTED),  # 6-byte row stride breaks 16-byte alignment
    (dict(stride_ks=[-128, 128, 128]), S.ERR_INVALID),
    (dict(H=4, Hk_t=3), S.ERR_INVALID),  # key heads must divide the query heads
    (dict(H=4, Hk_s=8), S.ERR_INVALID),
    (dict(H=4, Hk_s=-1), S.ERR_INVALID),
    (dict(H=4, Hk_t=2, Hk_s=1, stride_qt=[1, 1, 3]), S.ERR_UNSUPPORTED),  # valid grouping: later checks run
])
def test_fwd_rejects_bad_problems(kw, expected):
    assert fwd_status(_problem(**kw)) == expected


def test_fwd_rejects_null_and_misaligned_pointers():
    assert fwd_status(None) == S.ERR_INVALID
    assert fwd_status(_problem(), ptrs=[A, 0, A, A]) == S.ERR_INVALID
    assert fwd_status(_problem(), ptrs=[A + 2, A, A, A]) == S.ERR_UNSUPPORTED
    assert fwd_status(_problem(), outs=[A, 0, A]) == S.ERR_INVALID
    assert fwd_status(_problem(), outs=[A + 1, A, A]) == S.ERR_UNSUPPORTED


def test_empty_problems_are_noops():
    for kw in (dict(B=0), dict(H=0), dict(Nq=0), dict(Nq=0, Nk=0)):
        assert fwd_status(_problem(**kw), ptrs=[0, 0, 0, 0], outs=[0, 0, 0]) == S.OK


def test_bwd_argument_rules():
    L = S.lib()
    p = _problem()
    st = [A + 0x7000, A + 0x8000, A + 0x9000, A + 0xA000]  # lse_t, lse_s, kl, g
    # only one teacher output given
    assert L.streamkl_bwd(ctypes.byref(p), *PTRS, *st, A + 0xB000, A + 0xC000, A + 0xD000, None, None) == \
        S.ERR_INVALID
    # teacher gradients need kl
    assert L.streamkl_bwd(ctypes.byref(p), *PTRS, st[0], st[1], None, st[3], A + 0xB000, A + 0xC000, A + 0xD000,
                          A + 0xE000, None) == S.ERR_INVALID
    # missing g
    assert L.streamkl_bwd(ctypes.byref(p), *PTRS, st[0], st[1], None, None, A + 0xB000, A + 0xC000, None, None,
                          None) == S.ERR_INVALID
    # only one student output given; no gradient asked for at all
    assert L.streamkl_bwd(ctypes.byref(p), *PTRS, st[0], st[1], None, st[3], A + 0xB000, None, None, None,
                          None) == S.ERR_INVALID
    assert L.streamkl_bwd(ctypes.byref(p), *PTRS, st[0], st[1], None, st[3], None, None, None, None,
                          None) == S.ERR_INVALID
    # teacher gradients alone still need kl
    assert L.streamkl_bwd(ctypes.byref(p), *PTRS, st[0], st[1], None, st[3], None, None, A + 0xB000, A + 0xC000,
                          None) == S.ERR_INVALID
    assert L.streamkl_bwd_dq(ctypes.byref(p), *PTRS, st[0], st[1], st[3], None, None) == S.ERR_INVALID
    assert L.streamkl_bwd_dk(ctypes.byref(_problem(d_s=48)), *PTRS, st[0], st[1], st[3], A, None) == \
        S.ERR_UNSUPPORTED
    assert L.streamkl_bwd(ctypes.byref(_problem(B=0)), *([0] * 12), None) == S.OK


def test_problem_struct_layout_matches_the_header(tmp_path):
    """The ctypes mirror has the C struct's size and field offsets (compiled from include/streamkl.h)."""
    fields = [f[0] for f in S.Problem._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "streamkl.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(streamkl_problem_t));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(streamkl_problem_t, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(S.Problem)
    assert got[1:] == [getattr(S.Problem, f).offset for f in fields]


def test_grouped_key_heads_are_accepted_and_described():
    # every divisor of H (0 meaning H) passes the problem checks: the misaligned pointer checked after
    # them is what the call reports; a non-divisor stops at the problem checks
    for hk_t, hk_s in ((0, 0), (1, 4), (2, 1), (4, 2)):
        assert fwd_status(_problem(H=4, Hk_t=hk_t, Hk_s=hk_s), ptrs=[A + 2, A, A, A]) == S.ERR_UNSUPPORTED
    assert fwd_status(_problem(H=4, Hk_t=3), ptrs=[A + 2, A, A, A]) == S.ERR_INVALID
    torch = pytest.importorskip("torch")
    q = torch.zeros(2, 8, 4, 64)
    p = S.make_problem(q, torch.zeros(2, 2, 6, 64), torch.zeros(2, 8, 4, 128), torch.zeros(2, 1, 6, 128), True)
    assert (p.H, p.Hk_t, p.Hk_s, p.Nk, p.d_s) == (8, 2, 1, 6, 128)
    with pytest.raises(ValueError):  # 3 key heads cannot serve 8 query heads
        S.make_problem(q, torch.zeros(2, 3, 6, 64), q, torch.zeros(2, 8, 6, 64), False)
    with pytest.raises(ValueError):  # key heads of the student's own dimension
        S.make_problem(q, torch.zeros(2, 2, 6, 64), q, torch.zeros(2, 2, 6, 128), False)


def test_python_binding_validates_shapes():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        S.make_problem(q, torch.zeros(1, 1, 4, 32), q, q, False)
    with pytest.raises(ValueError):
        S.make_problem(q, q, q.double(), q, False)
    p = S.make_problem(q, torch.zeros(1, 1, 6, 64), q, torch.zeros(1, 1, 6, 64), True)
    assert (p.Nq, p.Nk, p.d_t, p.causal, p.dtype) == (4, 6, 64, 1, S.FP32)
    assert abs(p.scale_t - 0.125) < 1e-9


def test_product_path_has_no_fallback():
    """The binding never imports the oracle and never computes on the host."""
    src = open(os.path.join(ROOT, "attention_kl_amd", "streamkl.py")).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "numpy" not in src


def test_packed_batch_argument_rules():
    # packed problem: 3 segments over 300 packed rows; fake device addresses for the offsets
    cu_q, cu_k = A + 0x8000, A + 0x9000
    ok = dict(B=3, Nq=300, Nk=300, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=128, max_seqlen_k=128)
    bad_ptr = [A + 2, A, A, A]  # checked after the problem: UNSUPPORTED means the problem passed
    assert fwd_status(_problem(**ok), ptrs=bad_ptr) == S.ERR_UNSUPPORTED
    # causal with more packed query rows than key rows is a per-segment matter, not rejected here
    assert fwd_status(_problem(**{**ok, "Nq": 400, "max_seqlen_q": 200}), ptrs=bad_ptr) == S.ERR_UNSUPPORTED
    for kw in (dict(cu_seqlens_k=None), dict(cu_seqlens_q=None), dict(max_seqlen_q=301), dict(max_seqlen_k=-1)):
        assert fwd_status(_problem(**{**ok, **kw}), ptrs=bad_ptr) == S.ERR_INVALID, kw
    assert fwd_status(_problem(**{**ok, "cu_seqlens_q": cu_q + 2}), ptrs=bad_ptr) == S.ERR_UNSUPPORTED
    # nothing to do: no rows in any segment
    assert fwd_status(_problem(**{**ok, "max_seqlen_q": 0}), ptrs=[0] * 4, outs=[0] * 3) == S.OK


def test_python_binding_describes_a_packed_batch():
    torch = pytest.importorskip("torch")
    q = torch.zeros(300, 4, 64)    # [N, H, d]
    k = torch.zeros(350, 2, 64)    # [N, Hk, d]
    cu_q = torch.tensor([0, 100, 100, 300], dtype=torch.int32)
    cu_k = torch.tensor([0, 150, 170, 350], dtype=torch.int32)
    p = S.make_problem(q, k, q, k, False, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    assert (p.B, p.H, p.Nq, p.Nk, p.Hk_t) == (3, 4, 300, 350, 2)
    assert (p.max_seqlen_q, p.max_seqlen_k) == (200, 180)
    assert list(p.stride_qt)[1:] == [64, 4 * 64]  # head and row strides of [N, H, d] (the b stride is unused)
    assert p.packed and p.stat_shape() == (4, 300) and p.dk_shape(2, 64) == (2, 350, 64)
    with pytest.raises(ValueError):  # both offset vectors or neither
        S.make_problem(q, k, q, k, True, cu_seqlens_q=cu_q)
    with pytest.raises(ValueError):  # int32 offsets only
        S.make_problem(q, k, q, k, True, cu_seqlens_q=cu_q.long(), cu_seqlens_k=cu_k)
    with pytest.raises(ValueError):  # packed inputs are [N, heads, d]
        S.make_problem(q[None], k[None], q[None], k[None], True, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)


def test_python_binding_rejects_invalid_offsets():
    """Offsets that break the packed-batch rules raise in the binding, before any launch (CPU
    tensors here: the check is the read-back the binding makes anyway)."""
    torch = pytest.importorskip("torch")
    q = torch.zeros(300, 2, 64)
    k = torch.zeros(350, 2, 64)
    t = lambda v: torch.tensor(v, dtype=torch.int32)
    good_q, good_k = t([0, 100, 100, 300]), t([0, 150, 150, 350])
    S.make_problem(q, k, q, k, True, cu_seqlens_q=good_q, cu_seqlens_k=good_k)
    bad = [
        (t([-1, 100, 100, 300]), good_k, {}),     # negative start
        (t([0, 100, 90, 300]), good_k, {}),       # decreasing
        (good_q, t([0, 150, 170, 351]), {}),      # past the packed key rows
        (t([0, 100, 100, 301]), good_k, {}),      # past the packed query rows
        (t([0, 100, 110, 300]), t([0, 150, 150, 350]), {}),  # a segment with queries and no keys
        (t([0, 100, 100, 300]), t([0, 99, 170, 350]), {}),   # causal: fewer keys than queries
        (good_q, good_k, dict(max_seqlen_q=150)),  # the grid would miss rows of the longest segment
    ]
    for cq, ck, kw in bad:
        with pytest.raises(ValueError):
            S.make_problem(q, k, q, k, True, cu_seqlens_q=cq, cu_seqlens_k=ck, **kw)
        with pytest.raises(ValueError):
            S.fwd(q, k, q, k, causal=True, cu_seqlens_q=cq, cu_seqlens_k=ck, **kw)
    # not causal: fewer keys than queries is a valid segment
    S.make_problem(q, k, q, k, False, cu_seqlens_q=t([0, 100, 100, 300]), cu_seqlens_k=t([0, 99, 170, 350]))
    with pytest.raises(ValueError):  # skipping the read-back needs the maxima
        S.make_problem(q, k, q, k, True, cu_seqlens_q=good_q, cu_seqlens_k=good_k, validate=False)
    p = S.make_problem(q, k, q, k, True, cu_seqlens_q=good_q, cu_seqlens_k=good_k, validate=False,
                       max_seqlen_q=200, max_seqlen_k=180)
    assert (p.max_seqlen_q, p.max_seqlen_k) == (200, 180)


def test_js_argument_rules():
    L = S.lib()
    p = _problem()
    outs = [A + 0x4000, A + 0x5000, A + 0x6000, A + 0x7000]  # js, lse_t, lse_s, js_t
    assert L.streamkl_js_fwd(ctypes.byref(p), *PTRS, *outs[:3], None, None) == S.ERR_INVALID  # js_t missing
    assert L.streamkl_js_fwd(ctypes.byref(p), *PTRS, outs[0] + 2, *outs[1:], None) == S.ERR_UNSUPPORTED
    assert L.streamkl_js_fwd(ctypes.byref(_problem(B=0)), *([0] * 8), None) == S.OK
    st = [A + 0x8000, A + 0x9000, A + 0xA000, A + 0xB000, A + 0xC000]  # lse_t, lse_s, js, js_t, g
    pair_s, pair_t = [A + 0xD000, A + 0xE000], [A + 0xF000, A + 0x10000]
    assert L.streamkl_js_bwd(ctypes.byref(p), *PTRS, *st, None, None, None, None, None) == S.ERR_INVALID  # nothing asked
    assert L.streamkl_js_bwd(ctypes.byref(p), *PTRS, *st, pair_s[0], None, None, None, None) == S.ERR_INVALID  # half pair
    assert L.streamkl_js_bwd(ctypes.byref(p), *PTRS, st[0], st[1], None, st[3], st[4], *pair_s, None, None,
                             None) == S.ERR_INVALID  # js missing
    assert L.streamkl_js_bwd(ctypes.byref(p), *PTRS, st[0], st[1], st[2], None, st[4], None, None, *pair_t,
                             None) == S.ERR_INVALID  # js_t missing
    assert L.streamkl_js_bwd(ctypes.byref(p), *PTRS, *st[:4], None, *pair_s, None, None, None) == S.ERR_INVALID  # g
    assert L.streamkl_js_bwd(ctypes.byref(_problem(d_t=96)), *PTRS, *st, *pair_s, None, None, None) == \
        S.ERR_UNSUPPORTED


def test_workspace_size_and_checks():
    L = S.lib()
    q = lambda **kw: L.streamkl_workspace_floats(ctypes.byref(_problem(**kw)))
    big = dict(B=1, H=32, Nq=32768, Nk=32768, stride_qt=[32 * 32768 * 128, 32768 * 128, 128],
               stride_kt=[32 * 32768 * 128, 32768 * 128, 128], stride_qs=[32 * 32768 * 128, 32768 * 128, 128],
               stride_ks=[32 * 32768 * 128, 32768 * 128, 128])
    assert q(**big) == 0                          # one key head per query head: no workspace
    dk_full = 32 * 32768 * 128                    # an ungrouped dK of the workload: 32 query heads
    assert q(**big, Hk_s=8) == dk_full            # each query head's contribution, then the group sums
    assert q(**big, Hk_s=1) == dk_full
    assert q(**big, Hk_t=2, Hk_s=1) == dk_full    # the larger of the two sides (both ungrouped dK here)
    assert q(**big, Hk_s=1, dtype=S.FP32) == dk_full
    assert q(H=4, Hk_s=1) == 4 * 128 * 128
    assert q(B=0, H=4, Hk_s=1) == 0 and L.streamkl_workspace_floats(None) == 0
    bad_ptr = [A + 2, A, A, A]
    assert fwd_status(_problem(H=4, Hk_s=1, workspace=A + 8, workspace_floats=100), ptrs=bad_ptr) == \
        S.ERR_UNSUPPORTED  # 8-byte aligned workspace
    assert fwd_status(_problem(H=4, Hk_s=1, workspace=A + 0x100, workspace_floats=-1), ptrs=bad_ptr) == \
        S.ERR_INVALID
    assert fwd_status(_problem(H=4, Hk_s=1, workspace=A + 0x100, workspace_floats=100), ptrs=bad_ptr) == \
        S.ERR_UNSUPPORTED  # a valid workspace: the problem checks pass

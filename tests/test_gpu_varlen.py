"""GPU parity of packed variable-length batches against the float64 oracle, segment by segment.

Each segment is generated as a workload of its own (one batch entry, its own seed) and the
segments are packed one after another along the row axis, as [N, heads, d] tensors with int32
offsets cu_seqlens.  The oracle sees each segment alone, as an ordinary one-entry problem: a
packed batch is defined as the independent problems of its segments.  Statistics and gradients
come back in the library's packed layout ([H, N_Q], [H, N_Q, d], [Hk, N_K, d]) and are compared on
each segment's columns.  Tolerances and criteria are those of the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import loss as L
from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

from parity import all_pass, RTOL, grad_floor, ratio_kl, ratio_lse, ratio_rows, report

pytestmark = pytest.mark.gpu


def _segments(H, lens_q, lens_k, d_t, d_s, causal, dtype, recipe, seed, hk_t=None, hk_s=None):
    """Per-segment float64 host arrays (key heads subsampled as in the grouped tests) and the packed device inputs."""
    hk_t, hk_s = hk_t or H, hk_s or H
    segs = []
    for i, (nq, nk) in enumerate(zip(lens_q, lens_k)):
        w = wl.custom(1, H, nq, nk, d_t, d_s, causal, dtype=dtype, recipe=recipe, seed=seed + i)
        qt, kt, qs, ks = (a.astype(np.float64) for a in wl.full_f32(w)) if nq and nk else (
            np.zeros((1, H, nq, d_t)), np.zeros((1, H, nk, d_t)), np.zeros((1, H, nq, d_s)), np.zeros((1, H, nk, d_s)))
        kt, ks = kt[:, ::H // hk_t], ks[:, ::H // hk_s]
        g = wl.full_g(w) if nq else np.zeros((1, H, 0))
        segs.append(dict(w=w, qt=qt, kt=kt, qs=qs, ks=ks, g=g))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def pack(key):  # [1, heads, n, d] per segment -> [sum n, heads, d] on the device
        cat = np.concatenate([s[key][0] for s in segs], axis=1)  # [heads, N, d]
        return torch.from_numpy(np.ascontiguousarray(cat.transpose(1, 0, 2))).to(torch.float32).to(tdt).cuda()

    dev = tuple(pack(k) for k in ("qt", "kt", "qs", "ks"))
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lens_q)]), dtype=torch.int32).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens_k)]), dtype=torch.int32).cuda()
    g = torch.from_numpy(np.ascontiguousarray(np.concatenate([s["g"][0] for s in segs], axis=1))).float().cuda()
    return segs, dev, cu_q, cu_k, g


CASES = [
    # H, lens_q, lens_k, d_t, d_s, causal, dtype, recipe, teacher, hk_t, hk_s
    (2, [37, 0, 300, 1, 129, 64], [37, 0, 300, 1, 129, 64], 128, 128, True, "bf16", "noise", False, None, None),
    (2, [50, 3, 200, 7, 129], [60, 40, 257, 7, 400], 128, 64, True, "bf16", "independent", True, None, None),
    (3, [17, 100, 0, 33], [5, 100, 9, 250], 64, 64, False, "fp32", "independent", True, None, None),
    (4, [256, 31, 300], [256, 31, 520], 64, 128, False, "bf16", "independent", True, 2, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[f"h{c[0]}-{len(c[1])}seg-{'causal' if c[5] else 'full'}-{c[6]}"
                                             f"{'-teacher' if c[8] else ''}{'-gqa' if c[9] else ''}" for c in CASES])
def test_packed_segments_match_the_oracle_segment_by_segment(case):
    H, lq, lk, d_t, d_s, causal, dtype, recipe, teacher, hk_t, hk_s = case
    print(f"case packed H={H} q={lq} k={lk} causal={causal} {dtype} teacher={teacher} hk={hk_t},{hk_s}", flush=True)
    segs, (qt, kt, qs, ks), cu_q, cu_k, g = _segments(H, lq, lk, d_t, d_s, causal, dtype, recipe, 500, hk_t, hk_s)
    sc_t, sc_s = segs[0]["w"].scale_t, segs[0]["w"].scale_s
    seg = dict(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    kl, lt, ls = S.fwd(qt, kt, qs, ks, causal=causal, **seg)
    grads = S.bwd(qt, kt, qs, ks, lt, ls, g, causal=causal, kl=kl, teacher_grads=teacher, **seg)
    torch.cuda.synchronize()
    assert kl.shape == (H, sum(lq)) and grads[1].shape == (ks.shape[1], sum(lk), d_s)
    kl, lt, ls = (x.cpu().numpy() for x in (kl, lt, ls))
    gr = [None if x is None else x.cpu().numpy() for x in grads]
    rt = RTOL[dtype]
    worst = {}
    q0 = k0 = 0
    for s, nq, nk in zip(segs, lq, lk):
        if nq:
            ekt = np.repeat(s["kt"], H // s["kt"].shape[1], axis=1)
            eks = np.repeat(s["ks"], H // s["ks"].shape[1], axis=1)
            h64 = (s["qt"], ekt, s["qs"], eks)
            rkl, rlt, rls = oracle.forward(*h64, sc_t, sc_s, causal)
            rg = oracle.backward(*h64, sc_t, sc_s, causal, s["g"], teacher=teacher)

            def sumg(x, hk):  # dK of the expanded heads, summed over each key head's group
                return x.reshape(1, hk, H // hk, nk, x.shape[-1]).sum(axis=2)
            sl = slice(q0, q0 + nq)
            r = dict(kl=ratio_kl(kl[None, :, sl], rkl, rt), lse_t=ratio_lse(lt[:, sl], rlt[0], rt),
                     lse_s=ratio_lse(ls[:, sl], rls[0], rt),
                     dq_s=ratio_rows(gr[0][None, :, sl], rg["dq_s"], rt, grad_floor(sc_s, s["g"], eks)),
                     dk_s=ratio_rows(gr[1][None, :, k0:k0 + nk], sumg(rg["dk_s"], s["ks"].shape[1]), rt,
                                     grad_floor(sc_s, s["g"], s["qs"])))
            if teacher:
                r.update(dq_t=ratio_rows(gr[2][None, :, sl], rg["dq_t"], rt, grad_floor(sc_t, s["g"], ekt)),
                         dk_t=ratio_rows(gr[3][None, :, k0:k0 + nk], sumg(rg["dk_t"], s["kt"].shape[1]), rt,
                                         grad_floor(sc_t, s["g"], s["qt"])))
            for k, v in r.items():
                worst[k] = max(worst.get(k, 0.0), v)
        elif nk:
            # keys that no query reads: their gradient is exactly zero
            assert np.all(gr[1][:, k0:k0 + nk] == 0.0)
            if teacher:
                assert np.all(gr[3][:, k0:k0 + nk] == 0.0)
        q0 += nq
        k0 += nk
    msg = report(f"packed {lq}", **worst)
    print(msg, flush=True)
    assert all_pass(worst), msg


def test_equal_segments_give_the_dense_batch_bit_for_bit():
    """B segments of one length, packed, against the same rows as a dense [B, H, N, d] batch."""
    w = wl.custom(3, 2, 190, 190, 128, 128, True, recipe="independent", seed=77)
    print(f"case {w.name} packed vs dense", flush=True)
    host = wl.full_f32(w)
    dense = tuple(torch.from_numpy(a).cuda().to(torch.bfloat16) for a in host)
    # [B, H, N, d] -> packed [B*N, H, d]
    packed = tuple(x.permute(0, 2, 1, 3).reshape(w.B * w.Nq, w.H, x.shape[-1]).contiguous() for x in dense)
    cu = torch.arange(0, w.B * w.Nq + 1, w.Nq, dtype=torch.int32).cuda()
    g = torch.from_numpy(wl.full_g(w)).cuda()
    a = S.fwd(*dense, causal=True, split=False)  # a packed batch never splits its query blocks' keys
    b = S.fwd(*packed, causal=True, cu_seqlens_q=cu, cu_seqlens_k=cu)
    ga = S.bwd(*dense, a[1], a[2], g, causal=True, kl=a[0], teacher_grads=True)
    gp = g.permute(1, 0, 2).reshape(w.H, w.B * w.Nq).contiguous()  # [B, H, N] -> [H, B*N]
    gb = S.bwd(*packed, b[1], b[2], gp, causal=True, kl=b[0], teacher_grads=True, cu_seqlens_q=cu, cu_seqlens_k=cu)
    torch.cuda.synchronize()
    for x, y in zip(a, b):  # [B, H, N] vs [H, B*N]
        assert torch.equal(x.permute(1, 0, 2).reshape(w.H, -1), y)
    for x, y in zip(ga, gb):  # [B, H, N, d] vs [H, B*N, d]
        assert torch.equal(x.permute(1, 0, 2, 3).reshape(w.H, w.B * w.Nq, -1), y)


def test_autograd_on_a_packed_batch():
    """The loss wrapper on packed inputs: gradients come back as [N, heads, d] like the inputs."""
    lq = [70, 5, 128]
    segs, (qt, kt, qs, ks), cu_q, cu_k, _ = _segments(2, lq, lq, 128, 128, True, "bf16", "independent", 900)
    print(f"case packed autograd {lq}", flush=True)
    qs = qs.clone().requires_grad_()
    ks = ks.clone().requires_grad_()
    loss = L.attention_kl(qt, kt, qs, ks, causal=True, reduction="batchmean", cu_seqlens_q=cu_q, cu_seqlens_k=cu_q)
    loss.backward()
    torch.cuda.synchronize()
    assert qs.grad.shape == qs.shape and ks.grad.shape == ks.shape
    sc = segs[0]["w"].scale_s
    total = 0.0
    rt = 2e-3 + 2.0 ** -9  # bf16 gradients come back rounded to bf16
    q0 = 0
    for s, n in zip(segs, lq):
        h64 = (s["qt"], s["kt"], s["qs"], s["ks"])
        gw = np.full((1, 2, n), 1.0 / len(lq))
        total += float(oracle.forward(*h64, segs[0]["w"].scale_t, sc, True)[0].sum()) / len(lq)
        rg = oracle.backward(*h64, segs[0]["w"].scale_t, sc, True, gw)
        dq = qs.grad[q0:q0 + n].float().permute(1, 0, 2).cpu().numpy()[None]
        dk = ks.grad[q0:q0 + n].float().permute(1, 0, 2).cpu().numpy()[None]
        assert ratio_rows(dq, rg["dq_s"], rt, grad_floor(sc, gw, s["ks"])) <= 1.0
        assert ratio_rows(dk, rg["dk_s"], rt, grad_floor(sc, gw, s["qs"])) <= 1.0
        q0 += n
    assert abs(loss.item() - total) <= 2e-3 * max(abs(total), 1e-3) * 4


def test_packed_length_mix_full_size():
    """The bench workload's 32768 rows cut into the seeded length mix, as `bench.py --packed-mix 1`
    launches it (the workload's generated tensors viewed as [N, H, d]): each segment is the problem
    of its own rows and keys, checked over every row and key of three segments (the longest, the
    shortest, the last) in two heads."""
    from parity import device_inputs_bf16_bits, rtol_of
    w = wl.WORKLOADS[3]
    lens = wl.length_mix(w.Nq, 1)
    cu_h = np.concatenate([[0], np.cumsum(lens)])
    print(f"case {w.name} packed mix 1: {len(lens)} segments (full size)", flush=True)
    qt, kt, qs, ks = (x[0].permute(1, 0, 2) for x in device_inputs_bf16_bits(w))
    cu = torch.tensor(cu_h, dtype=torch.int32, device="cuda")
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s, cu_seqlens_q=cu, cu_seqlens_k=cu,
              max_seqlen_q=max(lens), max_seqlen_k=max(lens))
    kl, lt, ls = S.fwd(qt, kt, qs, ks, **kw)
    gh = wl.full_g(w)
    dq, dk, _, _ = S.bwd(qt, kt, qs, ks, lt, ls, torch.from_numpy(gh[0]).cuda(), **kw)
    torch.cuda.synchronize()
    assert kl.shape == (w.H, w.Nq) and dq.shape == (w.H, w.Nq, w.d_s)
    assert bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all()) and bool(torch.isfinite(kl).all())
    klc = kl.cpu().numpy()
    assert np.abs(klc[:, cu_h[:-1]]).max() <= 1e-5  # each segment's first row sees one key: KL = 0
    rt = rtol_of(w)
    worst = {}
    c = lambda x: x.cpu().numpy()
    from parity import oracle_window, worst_of
    for s in sorted({int(np.argmax(lens)), int(np.argmin(lens)), len(lens) - 1}):
        a, m = int(cu_h[s]), int(lens[s])
        for h in (0, 19):  # the whole segment: every row and key
            hh = tuple(x[a:a + m] for x in wl.head_f64(w, 0, h))
            ref = oracle_window(hh, w.scale_t, w.scale_s, w.causal, gh[0, h, a:a + m])
            worst_of(worst, "kl", ratio_kl(klc[h, a:a + m], ref["kl"], rt))
            worst_of(worst, "lse", ratio_lse(c(lt[h, a:a + m]), ref["lse_t"], rt), ratio_lse(c(ls[h, a:a + m]), ref["lse_s"], rt))
            worst_of(worst, "dq_s", ratio_rows(c(dq[h, a:a + m]), ref["dq_s"], rt))
            worst_of(worst, "dk_s", ratio_rows(c(dk[h, a:a + m]), ref["dk_s"], rt))
    msg = report(f"{w.name} packed mix 1", **worst)
    print(msg, flush=True)
    assert all_pass(worst), msg

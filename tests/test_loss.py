"""Host logic of attention_kl_amd.loss (the autograd glue), on the CPU.

The binding's fwd/bwd are swapped for fakes backed by the float64 oracle, so these tests exercise
only the wrapper's own work: which side goes where for each direction, which gradient path feeds
which input, which gradients are asked for, the reductions (they reach the backward as g), and the
dtype of the returned gradients.  The reference is torch autograd through the plain definition
(two log-softmaxes and the KL sum) in float64, which shares nothing with the oracle's backward.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_kl_amd import loss as L
from attention_kl_amd import streamkl as S

CALLS = []


def _np(t):
    return t.detach().cpu().numpy().astype(np.float64)


def _fake_fwd(qt, kt, qs, ks, *, causal, scale_t=None, scale_s=None, out=None, stream=None):
    st = 1.0 / math.sqrt(qt.shape[-1]) if scale_t is None else scale_t
    ss = 1.0 / math.sqrt(qs.shape[-1]) if scale_s is None else scale_s
    kl, lt, ls = oracle.forward(_np(qt), _np(kt), _np(qs), _np(ks), st, ss, causal)
    return tuple(torch.from_numpy(x) for x in (kl, lt, ls))


def _fake_bwd(qt, kt, qs, ks, lse_t, lse_s, g, *, causal, kl=None, teacher_grads=False, student_grads=True,
              scale_t=None, scale_s=None, out=None, stream=None):
    CALLS.append(dict(teacher=teacher_grads, student=student_grads, g_dtype=g.dtype, g_contig=g.is_contiguous(),
                      kl_given=kl is not None))
    st = 1.0 / math.sqrt(qt.shape[-1]) if scale_t is None else scale_t
    ss = 1.0 / math.sqrt(qs.shape[-1]) if scale_s is None else scale_s
    r = oracle.backward(_np(qt), _np(kt), _np(qs), _np(ks), st, ss, causal, _np(g), teacher=teacher_grads)
    t = {k: torch.from_numpy(v) for k, v in r.items()}
    return (t["dq_s"] if student_grads else None, t["dk_s"] if student_grads else None,
            t.get("dq_t") if teacher_grads else None, t.get("dk_t") if teacher_grads else None)


def _fake_js_fwd(qt, kt, qs, ks, *, causal, scale_t=None, scale_s=None, out=None, stream=None):
    st = 1.0 / math.sqrt(qt.shape[-1]) if scale_t is None else scale_t
    ss = 1.0 / math.sqrt(qs.shape[-1]) if scale_s is None else scale_s
    js, ht, _, lt, ls = oracle.js_forward(_np(qt), _np(kt), _np(qs), _np(ks), st, ss, causal)
    return tuple(torch.from_numpy(x) for x in (js, lt, ls, ht))


def _fake_js_bwd(qt, kt, qs, ks, lse_t, lse_s, js, js_t, g, *, causal, teacher_grads=False, student_grads=True,
                 scale_t=None, scale_s=None, out=None, stream=None):
    CALLS.append(dict(teacher=teacher_grads, student=student_grads, g_dtype=g.dtype, g_contig=g.is_contiguous(),
                      kl_given=True))
    st = 1.0 / math.sqrt(qt.shape[-1]) if scale_t is None else scale_t
    ss = 1.0 / math.sqrt(qs.shape[-1]) if scale_s is None else scale_s
    r = oracle.js_backward(_np(qt), _np(kt), _np(qs), _np(ks), st, ss, causal, _np(g), teacher=teacher_grads)
    t = {k: torch.from_numpy(v) for k, v in r.items()}
    return (t["dq_s"] if student_grads else None, t["dk_s"] if student_grads else None,
            t.get("dq_t") if teacher_grads else None, t.get("dk_t") if teacher_grads else None)


@pytest.fixture
def fake_backend(monkeypatch):
    monkeypatch.setattr(S, "fwd", _fake_fwd)
    monkeypatch.setattr(S, "bwd", _fake_bwd)
    monkeypatch.setattr(S, "js_fwd", _fake_js_fwd)
    monkeypatch.setattr(S, "js_bwd", _fake_js_bwd)
    CALLS.clear()
    yield


def _ref_kl(qt, kt, qs, ks, causal, direction):
    """Per-row divergence from the definition, differentiable by torch (float64)."""
    def one(qa, ka, qb, kb):
        sa, sb = 1.0 / math.sqrt(qa.shape[-1]), 1.0 / math.sqrt(qb.shape[-1])
        a = sa * qa @ ka.transpose(-1, -2)
        b = sb * qb @ kb.transpose(-1, -2)
        nq, nk = a.shape[-2], a.shape[-1]
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        allowed = (j <= i + nk - nq) if causal else torch.ones(nq, nk, dtype=torch.bool)
        # a finite fill (not -inf) keeps every masked term exactly 0 and its gradient exactly 0
        a = a.masked_fill(~allowed, -1e9)
        b = b.masked_fill(~allowed, -1e9)
        la, lb = torch.log_softmax(a, -1), torch.log_softmax(b, -1)
        if direction == "js":  # masked entries have P = 0 exactly and finite logs, so they add 0
            lm = torch.logaddexp(la, lb) - math.log(2.0)
            return 0.5 * (la.exp() * (la - lm)).sum(-1) + 0.5 * (lb.exp() * (lb - lm)).sum(-1)
        return (la.exp() * (la - lb)).sum(-1)
    if direction in ("forward", "js"):
        return one(qt, kt, qs, ks)
    if direction == "reverse":
        return one(qs, ks, qt, kt)
    return one(qt, kt, qs, ks) + one(qs, ks, qt, kt)


def _inputs(seed, causal):
    gen = torch.Generator().manual_seed(seed)
    B, H, nq, nk, dt, ds = 2, 2, 5, 7 if causal else 6, 8, 4
    f = lambda *s: torch.randn(*s, generator=gen, dtype=torch.float64)
    qt, kt, qs, ks = f(B, H, nq, dt), f(B, H, nk, dt), f(B, H, nq, ds), f(B, H, nk, ds)
    return qt, kt, qs, ks


REDUCE = {"none": lambda x: (x * torch.linspace(0.5, 1.5, x.numel(), dtype=x.dtype).view_as(x)).sum(),
          "sum": lambda x: x, "mean": lambda x: x, "batchmean": lambda x: x}


@pytest.mark.parametrize("direction", L.DIRECTIONS)
@pytest.mark.parametrize("reduction", L.REDUCTIONS)
@pytest.mark.parametrize("causal", [False, True])
def test_values_and_gradients_match_autograd_of_the_definition(fake_backend, direction, reduction, causal):
    qt, kt, qs, ks = _inputs(L.DIRECTIONS.index(direction) * 10 + L.REDUCTIONS.index(reduction) * 2 + causal, causal)
    ins = [x.clone().requires_grad_(True) for x in (qt, kt, qs, ks)]
    refs = [x.clone().requires_grad_(True) for x in (qt, kt, qs, ks)]
    out = L.attention_kl(*ins, causal=causal, direction=direction, reduction=reduction)
    rkl = _ref_kl(*refs, causal, direction)
    ref = {"none": rkl, "sum": rkl.sum(), "mean": rkl.mean(), "batchmean": rkl.sum() / rkl.shape[0]}[reduction]
    assert out.shape == ref.shape
    assert torch.allclose(out, ref, rtol=1e-9, atol=1e-12)
    # a non-uniform weighting for "none", so a row-indexing slip in g shows
    REDUCE[reduction](out).backward()
    REDUCE[reduction](ref).backward()
    for a, b in zip(ins, refs):
        # g passes through float32 in the wrapper (the ABI's g is float32): an error of ~1e-7 of the
        # tensor's scale, not of each element
        assert (a.grad - b.grad).abs().max() <= 1e-6 * b.grad.abs().max(), (direction, reduction)


def test_only_the_gradients_asked_for_are_computed(fake_backend):
    qt, kt, qs, ks = _inputs(1, True)
    # student trains, teacher frozen: forward KL uses the student path only
    L.attention_kl(qt, kt, qs.requires_grad_(), ks.requires_grad_(), causal=True, reduction="sum").backward()
    assert CALLS[-1] == dict(teacher=False, student=True, g_dtype=torch.float32, g_contig=True, kl_given=False)
    # reverse KL with a frozen teacher: the student sits in the teacher slot, and only that path runs
    qs.grad = ks.grad = None
    L.attention_kl(qt, kt, qs, ks, causal=True, direction="reverse", reduction="mean").backward()
    assert CALLS[-1] == dict(teacher=True, student=False, g_dtype=torch.float32, g_contig=True, kl_given=True)
    assert qs.grad is not None and ks.grad is not None
    # nothing requires grad: no backward call at all
    n = len(CALLS)
    with torch.no_grad():
        L.attention_kl(qt, kt, qs.detach(), ks.detach(), causal=True)
    assert len(CALLS) == n


def test_gradients_come_back_in_the_input_dtype(fake_backend):
    qt, kt, qs, ks = (x.float() for x in _inputs(2, False))
    qs.requires_grad_()
    ks.requires_grad_()
    L.attention_kl(qt, kt, qs, ks, reduction="sum").backward()
    assert qs.grad.dtype == torch.float32 and ks.grad.dtype == torch.float32


def test_bad_arguments_are_rejected_before_any_call(fake_backend):
    qt, kt, qs, ks = _inputs(3, False)
    with pytest.raises(ValueError):
        L.attention_kl(qt, kt, qs, ks, direction="total_variation")
    with pytest.raises(ValueError):
        L.attention_kl(qt, kt, qs, ks, reduction="max")
    assert CALLS == []


def test_loss_module_never_touches_the_oracle():
    import os
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "attention_kl_amd",
                            "loss.py")).read()
    assert "oracle" not in src and "numpy" not in src

"""Attention-KL distillation loss on the StreamKL primitive, with torch autograd.

StreamKL abstract (arXiv 2026), S1: attention distillation trains one attention
distribution to match another by minimising their KL divergence; S3: the
primitive is meant to sit inside such a training loop.  This module is that
glue, and only glue: the forward calls ``streamkl_fwd``, the backward calls
``streamkl_bwd``; every number is computed by the library's kernels.

The primitive returns the per-query-row divergence KL_i (float32 [B, H, N_Q]).
Whatever reduction the caller applies to it with torch operations (a sum, a
mean, a weighted sum, ...) reaches the backward as the per-row weight
g_i = dL/dKL_i, which is exactly the ``g`` of the C ABI, so every loss that is
a function of the rows is supported without special cases.

Directions (the pages fix none, S1):
  "forward"    KL(P_t || P_s)  teacher first, the primitive as defined
  "reverse"    KL(P_s || P_t)  the primitive with the two sides exchanged; the
               gradients of the student then come from the primitive's
               teacher-gradient path
  "symmetric"  KL(P_t || P_s) + KL(P_s || P_t)
  "js"         Jensen-Shannon: KL(P_t || M)/2 + KL(P_s || M)/2 with M = (P_t + P_s)/2, symmetric and at
               most ln 2 (streamkl_js_fwd / streamkl_js_bwd)

Packed variable-length batches (inputs [N, heads, d], segments given by cu_seqlens_q /
cu_seqlens_k) give the per-row KL as [H, N_Q]; "batchmean" then divides by the number of
sequences.

Gradients with respect to the teacher inputs are computed only when one of them
requires grad.  The library returns float32 gradients; autograd needs them in
the dtype of the input, so bf16 inputs receive bf16-rounded gradients (a relative
rounding of at most 2^-9 per element, on top of the kernels' own error).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import streamkl as S

DIRECTIONS = ("forward", "reverse", "symmetric", "js")
REDUCTIONS = ("none", "sum", "mean", "batchmean")


class StreamKLFunction(torch.autograd.Function):
    """Per-row KL(P_t || P_s) (js=True: Jensen-Shannon divergence) with its backward on the library.
    Inputs [B, H, N, d], or [N, H, d] with packed = (cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
    max_seqlen_k) for a packed batch."""

    @staticmethod
    def forward(ctx, qt, kt, qs, ks, causal: bool, scale_t: Optional[float], scale_s: Optional[float],
                packed: Optional[tuple] = None, js: bool = False):
        seg = _seg_kwargs(packed)
        kw = dict(causal=causal, scale_t=scale_t, scale_s=scale_s, **seg)
        if js:
            div, lse_t, lse_s, half_t = S.js_fwd(qt, kt, qs, ks, **kw)
            ctx.save_for_backward(qt, kt, qs, ks, div, lse_t, lse_s, half_t)
        else:
            div, lse_t, lse_s = S.fwd(qt, kt, qs, ks, **kw)
            ctx.save_for_backward(qt, kt, qs, ks, div, lse_t, lse_s)
        ctx.cfg = (bool(causal), scale_t, scale_s, bool(js))
        ctx.packed = packed
        return div

    @staticmethod
    def backward(ctx, g):
        qt, kt, qs, ks, div, lse_t, lse_s = ctx.saved_tensors[:7]
        causal, scale_t, scale_s, js = ctx.cfg
        need_t = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        need_s = ctx.needs_input_grad[2] or ctx.needs_input_grad[3]
        if not (need_t or need_s):
            return (None,) * 9
        g = g.to(torch.float32).contiguous()  # the upstream gradient may be a broadcast view
        kw = dict(causal=causal, teacher_grads=need_t, student_grads=need_s, scale_t=scale_t, scale_s=scale_s,
                  **_seg_kwargs(ctx.packed))
        if js:
            grads = S.js_bwd(qt, kt, qs, ks, lse_t, lse_s, div, ctx.saved_tensors[7], g, **kw)
        else:
            grads = S.bwd(qt, kt, qs, ks, lse_t, lse_s, g, kl=div if need_t else None, **kw)
        if ctx.packed is not None:  # the library's packed layout [heads, N, d] -> the inputs' [N, heads, d]
            grads = tuple(None if x is None else x.transpose(0, 1) for x in grads)
        dq_s, dk_s, dq_t, dk_t = grads

        def cast(grad, like, needed):
            return grad.to(like.dtype) if (needed and grad is not None) else None

        return (cast(dq_t, qt, ctx.needs_input_grad[0]), cast(dk_t, kt, ctx.needs_input_grad[1]),
                cast(dq_s, qs, ctx.needs_input_grad[2]), cast(dk_s, ks, ctx.needs_input_grad[3]),
                None, None, None, None, None)


def _seg_kwargs(packed):
    if packed is None:
        return {}
    cu_q, cu_k, mq, mk = packed
    return dict(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=mq, max_seqlen_k=mk)


def attention_kl(qt, kt, qs, ks, *, causal: bool = False, scale_t: Optional[float] = None,
                 scale_s: Optional[float] = None, direction: str = "forward", reduction: str = "none",
                 cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: Optional[int] = None,
                 max_seqlen_k: Optional[int] = None):
    """Attention-KL divergence between teacher (qt, kt) and student (qs, ks) attention rows.

    Shapes [B, H, N_Q, d_t], [B, Hk_t, N_K, d_t], [B, H, N_Q, d_s], [B, Hk_s, N_K, d_s] (Hk dividing
    H: grouped key heads), bf16 or float32, d unit-stride.  Softmax scales default to 1/sqrt(d) per
    side.  Packed variable-length batch: [N_Q, H, d] / [N_K, Hk, d] inputs and int32 device
    cu_seqlens_q, cu_seqlens_k of B + 1 segment offsets (max_seqlen_* default to the longest
    segment, read back from the device once).

    reduction: "none" -> per-row float32 [B, H, N_Q] ([H, N_Q] packed); "sum" -> sum over rows;
    "mean" -> mean over all rows; "batchmean" -> sum divided by B (per-sample divergence summed
    over heads and rows).
    """
    if direction not in DIRECTIONS:
        raise ValueError(f"direction must be one of {DIRECTIONS}, got {direction!r}")
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {REDUCTIONS}, got {reduction!r}")
    packed = None
    n_batch = qt.shape[0]
    if cu_seqlens_q is not None or cu_seqlens_k is not None:
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise ValueError("a packed batch needs both cu_seqlens_q and cu_seqlens_k")

        def longest(c):
            return int((c[1:] - c[:-1]).max().item()) if c.numel() > 1 else 0
        mq = longest(cu_seqlens_q) if max_seqlen_q is None else int(max_seqlen_q)
        mk = longest(cu_seqlens_k) if max_seqlen_k is None else int(max_seqlen_k)
        packed = (cu_seqlens_q, cu_seqlens_k, mq, mk)
        n_batch = cu_seqlens_q.numel() - 1
    if direction == "js":
        kl = StreamKLFunction.apply(qt, kt, qs, ks, causal, scale_t, scale_s, packed, True)
    elif direction == "forward":
        kl = StreamKLFunction.apply(qt, kt, qs, ks, causal, scale_t, scale_s, packed)
    elif direction == "reverse":
        kl = StreamKLFunction.apply(qs, ks, qt, kt, causal, scale_s, scale_t, packed)
    else:
        kl = (StreamKLFunction.apply(qt, kt, qs, ks, causal, scale_t, scale_s, packed)
              + StreamKLFunction.apply(qs, ks, qt, kt, causal, scale_s, scale_t, packed))
    if reduction == "none":
        return kl
    if reduction == "sum":
        return kl.sum()
    if reduction == "mean":
        return kl.mean()
    return kl.sum() / n_batch

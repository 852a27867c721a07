"""CPU oracle for the attention-KL path (float64, materialising). TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import this
module; the product path never calls it.  It shares no code with the HIP path.

What it computes (the plain definition, written out):
the StreamKL abstract ("StreamKL: Fast and Memory-Efficient KL Divergence for
Boosting Attention Distillation", arXiv 2026; sentences numbered S1..S8 in
reading order) describes attention distillation as fitting one attention
distribution to another by minimising their KL divergence (S1), and describes the
existing approach as forming both attention distributions in full and then
reducing the KL over them (S2).  This oracle is exactly that existing approach:

  a_ij = s_t q_t,i . k_t,j      b_ij = s_s q_s,i . k_s,j
  allowed keys of row i: A_i = { j < N_K : not causal  or  j <= i + N_K - N_Q }
  log P_t = a - logsumexp_{A_i}(a)      log P_s = b - logsumexp_{A_i}(b)
  KL_i = sum_{j in A_i} P_t,ij (log P_t,ij - log P_s,ij)        (teacher || student)

and, for the backward (S5 names only the recompute; the gradients are the
calculus of the line above, with per-row upstream weights g_i):

  dS_s = g_i (P_s - P_t)                          dQ_s = s_s dS_s K_s,  dK_s = s_s dS_s^T Q_s
  dS_t = g_i P_t ((a - b) - sum_k P_t,ik (a_ik - b_ik))   dQ_t = s_t dS_t K_t,  dK_t = s_t dS_t^T Q_t

Readings taken where the pages are silent: KL direction teacher || student; the
output is one KL per query row (the caller reduces over rows through g); the
scale is per side (1/sqrt(d_t), 1/sqrt(d_s) by default); causal masks are
bottom-right aligned and need N_Q <= N_K; masked pairs contribute nothing.

The only blocking is over query rows, to bound memory at long N: each block of
rows forms its full rows of both distributions over every allowed key.
Everything is float64 numpy.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Tuple

import numpy as np

ROW_BLOCK = 1024


def allowed_mask(rows: np.ndarray, nq: int, nk: int, causal: bool, ncols: Optional[int] = None) -> np.ndarray:
    """Boolean [len(rows), ncols] mask of allowed keys j < ncols for the given query rows."""
    ncols = nk if ncols is None else ncols
    cols = np.arange(ncols)
    m = np.broadcast_to(cols[None, :] < nk, (len(rows), ncols))
    if causal:
        m = m & (cols[None, :] <= (np.asarray(rows)[:, None] + (nk - nq)))
    return np.array(m)


def _masked_log_softmax(x: np.ndarray, mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row log-softmax over the allowed entries; returns (log-probabilities with -inf where masked, lse)."""
    xm = np.where(mask, x, -np.inf)
    mx = xm.max(axis=1, keepdims=True)
    lse = mx + np.log(np.exp(xm - mx).sum(axis=1, keepdims=True))
    return xm - lse, lse[:, 0]


def _check(qt, kt, qs, ks, causal):
    nq, nk = qt.shape[0], kt.shape[0]
    assert qs.shape[0] == nq and ks.shape[0] == nk
    assert qt.shape[1] == kt.shape[1] and qs.shape[1] == ks.shape[1]
    assert nk >= 1, "softmax over an empty key set is undefined"
    if causal:
        assert nq <= nk, "causal (bottom-right aligned) needs N_Q <= N_K"
    return nq, nk


def _row_blocks(rows: np.ndarray, block: int):
    for s in range(0, len(rows), block):
        yield rows[s:s + block]


def _block_terms(qt, kt, qs, ks, s_t, s_s, causal, r):
    """Both log-distributions (and logits) of the query rows r, over keys 0..last allowed key of r."""
    nq, nk = qt.shape[0], kt.shape[0]
    kmax = nk if not causal else min(nk, int(r.max()) + (nk - nq) + 1)
    a = s_t * (qt[r] @ kt[:kmax].T)
    b = s_s * (qs[r] @ ks[:kmax].T)
    mask = allowed_mask(r, nq, nk, causal, kmax)
    la, lse_t = _masked_log_softmax(a, mask)
    lb, lse_s = _masked_log_softmax(b, mask)
    return a, b, mask, la, lb, lse_t, lse_s, kmax


def forward_head(qt, kt, qs, ks, scale_t, scale_s, causal, rows: Optional[Iterable[int]] = None,
                 block: int = ROW_BLOCK) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per-row KL(P_t || P_s), LSE_t, LSE_s (float64) of one head, for `rows` (default: all)."""
    qt, kt, qs, ks = (np.asarray(x, np.float64) for x in (qt, kt, qs, ks))
    nq, nk = _check(qt, kt, qs, ks, causal)
    rows = np.arange(nq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    s_t, s_s = float(scale_t), float(scale_s)
    kl = np.empty(len(rows))
    lt = np.empty(len(rows))
    ls = np.empty(len(rows))
    pos = 0
    for r in _row_blocks(rows, block):
        _, _, mask, la, lb, lse_t, lse_s, _ = _block_terms(qt, kt, qs, ks, s_t, s_s, causal, r)
        pt = np.where(mask, np.exp(la), 0.0)
        # masked terms are excluded from the sum (never 0 * (-inf - -inf))
        log_ratio = np.where(mask, la, 0.0) - np.where(mask, lb, 0.0)
        kl[pos:pos + len(r)] = (pt * log_ratio).sum(axis=1)
        lt[pos:pos + len(r)] = lse_t
        ls[pos:pos + len(r)] = lse_s
        pos += len(r)
    return kl, lt, ls


def backward_head(qt, kt, qs, ks, scale_t, scale_s, causal, g, teacher: bool = False,
                  rows: Optional[Iterable[int]] = None, keys: Optional[Iterable[int]] = None,
                  block: int = ROW_BLOCK) -> Dict[str, np.ndarray]:
    """Gradients of sum_i g_i KL_i for one head.

    Returns dq_s (for `rows`, default all) and dk_s (for `keys`, default all), plus dq_t and dk_t
    when `teacher`.  dK of a key sums over every query row that may attend to it, so the rows
    visited are all rows that see any requested key, whatever `rows` asks for.
    """
    qt, kt, qs, ks = (np.asarray(x, np.float64) for x in (qt, kt, qs, ks))
    g = np.asarray(g, np.float64)
    nq, nk = _check(qt, kt, qs, ks, causal)
    s_t, s_s = float(scale_t), float(scale_s)
    qrows = np.arange(nq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    kcols = np.arange(nk) if keys is None else np.asarray(list(keys), dtype=np.int64)
    off = nk - nq
    visit = np.zeros(nq, bool)
    visit[qrows] = True
    if len(kcols):
        first = max(0, int(kcols.min()) - off) if causal else 0
        visit[first:] = True
    qpos = {int(r): i for i, r in enumerate(qrows)}
    out = {"dq_s": np.zeros((len(qrows), qs.shape[1])), "dk_s": np.zeros((len(kcols), ks.shape[1]))}
    if teacher:
        out["dq_t"] = np.zeros((len(qrows), qt.shape[1]))
        out["dk_t"] = np.zeros((len(kcols), kt.shape[1]))
    for r in _row_blocks(np.nonzero(visit)[0], block):
        a, b, mask, la, lb, _, _, kmax = _block_terms(qt, kt, qs, ks, s_t, s_s, causal, r)
        pt = np.where(mask, np.exp(la), 0.0)
        ps = np.where(mask, np.exp(lb), 0.0)
        gr = g[r][:, None]
        ds_s = gr * (ps - pt)
        if teacher:
            diff = np.where(mask, a - b, 0.0)
            mean_diff = (pt * diff).sum(axis=1, keepdims=True)
            ds_t = gr * pt * (diff - mean_diff)
        sel = np.array([qpos.get(int(i), -1) for i in r])
        hit = sel >= 0
        if hit.any():
            out["dq_s"][sel[hit]] = s_s * (ds_s[hit] @ ks[:kmax])
            if teacher:
                out["dq_t"][sel[hit]] = s_t * (ds_t[hit] @ kt[:kmax])
        kin = kcols < kmax
        if kin.any():
            out["dk_s"][kin] += s_s * (ds_s[:, kcols[kin]].T @ qs[r])
            if teacher:
                out["dk_t"][kin] += s_t * (ds_t[:, kcols[kin]].T @ qt[r])
    return out


def forward(qt, kt, qs, ks, scale_t, scale_s, causal, block: int = ROW_BLOCK):
    """All heads: inputs [B, H, N, d]; returns KL, LSE_t, LSE_s as float64 [B, H, N_Q]."""
    B, H, nq = qt.shape[:3]
    kl, lt, ls = (np.empty((B, H, nq)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            kl[b, h], lt[b, h], ls[b, h] = forward_head(qt[b, h], kt[b, h], qs[b, h], ks[b, h],
                                                        scale_t, scale_s, causal, block=block)
    return kl, lt, ls


def backward(qt, kt, qs, ks, scale_t, scale_s, causal, g, teacher: bool = False, block: int = ROW_BLOCK):
    """All heads: gradients of sum g*KL; returns a dict of float64 [B, H, N, d] arrays."""
    B, H = qt.shape[:2]
    res = None
    for b in range(B):
        for h in range(H):
            o = backward_head(qt[b, h], kt[b, h], qs[b, h], ks[b, h], scale_t, scale_s, causal, g[b, h],
                              teacher=teacher, block=block)
            if res is None:
                res = {k: np.empty((B, H) + v.shape) for k, v in o.items()}
            for k, v in o.items():
                res[k][b, h] = v
    return res


# ------------------------------------------------------------------------------------------------
# Jensen-Shannon divergence between the same two attention rows.  The pages name only KL (S1); the
# JS variant is the symmetric, bounded relative commonly used in distillation, defined here as
#
#   M = (P_t + P_s) / 2,   JS_i = 1/2 KL(P_t || M)_i + 1/2 KL(P_s || M)_i      (natural log, <= ln 2)
#
# and, with per-row weights g_i, the gradient of sum_i g_i JS_i with respect to the logits (the
# softmax chain rule applied to d JS / d P = 1/2 log(P / M) on each side):
#
#   dS_t = g_i 1/2 P_t (log(P_t / M) - KL(P_t || M)_i)     dQ_t = s_t dS_t K_t,  dK_t = s_t dS_t^T Q_t
#   dS_s = g_i 1/2 P_s (log(P_s / M) - KL(P_s || M)_i)     dQ_s = s_s dS_s K_s,  dK_s = s_s dS_s^T Q_s

def _js_terms(la, lb, mask):
    """log(P_t/M), log(P_s/M) over the allowed entries (0 where masked) and P_t, P_s."""
    lm = np.logaddexp(np.where(mask, la, 0.0), np.where(mask, lb, 0.0)) - np.log(2.0)
    pt = np.where(mask, np.exp(la), 0.0)
    ps = np.where(mask, np.exp(lb), 0.0)
    return np.where(mask, la - lm, 0.0), np.where(mask, lb - lm, 0.0), pt, ps


def js_forward_head(qt, kt, qs, ks, scale_t, scale_s, causal, rows: Optional[Iterable[int]] = None,
                    block: int = ROW_BLOCK):
    """Per-row JS, KL(P_t || M), KL(P_s || M), LSE_t, LSE_s (float64) of one head, for `rows`
    (default: all)."""
    qt, kt, qs, ks = (np.asarray(x, np.float64) for x in (qt, kt, qs, ks))
    nq, _ = _check(qt, kt, qs, ks, causal)
    rows = np.arange(nq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    out = [np.empty(len(rows)) for _ in range(5)]
    pos = 0
    for r in _row_blocks(rows, block):
        _, _, mask, la, lb, lse_t, lse_s, _ = _block_terms(qt, kt, qs, ks, float(scale_t), float(scale_s), causal, r)
        lrt, lrs, pt, ps = _js_terms(la, lb, mask)
        kt_m = (pt * lrt).sum(axis=1)
        ks_m = (ps * lrs).sum(axis=1)
        for o, v in zip(out, (0.5 * (kt_m + ks_m), kt_m, ks_m, lse_t, lse_s)):
            o[pos:pos + len(r)] = v
        pos += len(r)
    return tuple(out)


def js_backward_head(qt, kt, qs, ks, scale_t, scale_s, causal, g, teacher: bool = False,
                     rows: Optional[Iterable[int]] = None, keys: Optional[Iterable[int]] = None,
                     block: int = ROW_BLOCK) -> Dict[str, np.ndarray]:
    """Gradients of sum_i g_i JS_i for one head: dq_s for `rows` and dk_s for `keys` (default all),
    and dq_t, dk_t when `teacher`.  As in backward_head, every row that sees a requested key is
    visited, since dK sums over them."""
    qt, kt, qs, ks = (np.asarray(x, np.float64) for x in (qt, kt, qs, ks))
    g = np.asarray(g, np.float64)
    nq, nk = _check(qt, kt, qs, ks, causal)
    s_t, s_s = float(scale_t), float(scale_s)
    qrows = np.arange(nq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    kcols = np.arange(nk) if keys is None else np.asarray(list(keys), dtype=np.int64)
    visit = np.zeros(nq, bool)
    visit[qrows] = True
    if len(kcols):
        visit[max(0, int(kcols.min()) - (nk - nq)) if causal else 0:] = True
    qpos = {int(r): i for i, r in enumerate(qrows)}
    out = {"dq_s": np.zeros((len(qrows), qs.shape[1])), "dk_s": np.zeros((len(kcols), ks.shape[1]))}
    if teacher:
        out["dq_t"] = np.zeros((len(qrows), qt.shape[1]))
        out["dk_t"] = np.zeros((len(kcols), kt.shape[1]))
    for r in _row_blocks(np.nonzero(visit)[0], block):
        _, _, mask, la, lb, _, _, kmax = _block_terms(qt, kt, qs, ks, s_t, s_s, causal, r)
        lrt, lrs, pt, ps = _js_terms(la, lb, mask)
        gr = g[r][:, None]
        sides = [("s", gr * 0.5 * ps * (lrs - (ps * lrs).sum(axis=1, keepdims=True)), s_s, ks, qs)]
        if teacher:
            sides.append(("t", gr * 0.5 * pt * (lrt - (pt * lrt).sum(axis=1, keepdims=True)), s_t, kt, qt))
        sel = np.array([qpos.get(int(i), -1) for i in r])
        hit = sel >= 0
        kin = kcols < kmax
        for side, ds, sc, kx, qx in sides:
            if hit.any():
                out["dq_" + side][sel[hit]] = sc * (ds[hit] @ kx[:kmax])
            if kin.any():
                out["dk_" + side][kin] += sc * (ds[:, kcols[kin]].T @ qx[r])
    return out


def js_forward(qt, kt, qs, ks, scale_t, scale_s, causal, block: int = ROW_BLOCK):
    """All heads: inputs [B, H, N, d]; returns JS, KL(P_t||M), KL(P_s||M), LSE_t, LSE_s, float64 [B, H, N_Q]."""
    B, H, nq = qt.shape[:3]
    res = [np.empty((B, H, nq)) for _ in range(5)]
    for b in range(B):
        for h in range(H):
            for o, v in zip(res, js_forward_head(qt[b, h], kt[b, h], qs[b, h], ks[b, h], scale_t, scale_s, causal,
                                                 block=block)):
                o[b, h] = v
    return tuple(res)


def js_backward(qt, kt, qs, ks, scale_t, scale_s, causal, g, teacher: bool = False, block: int = ROW_BLOCK):
    """All heads: gradients of sum g*JS; returns a dict of float64 [B, H, N, d] arrays."""
    B, H = qt.shape[:2]
    res = None
    for b in range(B):
        for h in range(H):
            o = js_backward_head(qt[b, h], kt[b, h], qs[b, h], ks[b, h], scale_t, scale_s, causal, g[b, h],
                                 teacher=teacher, block=block)
            if res is None:
                res = {k: np.empty((B, H) + v.shape) for k, v in o.items()}
            for k, v in o.items():
                res[k][b, h] = v
    return res

"""Shared helpers of the GPU parity tests: inputs on the device, the tolerance criterion.

Tolerance (relative, written out in every comparison): 2e-3 for bf16 inputs, 1e-5 for
fp32 inputs.  Near-zero references (causal row 0 has KL = 0 exactly, small-KL rows
~1e-4) make a pure relative test meaningless, so each criterion adds the same rtol
times the typical magnitude of its group:
  KL       |d_i| <= rtol |ref_i| + rtol max(rms_head(ref), 1e-3)
  LSE      |d_i| <= rtol max(1, |ref_i|)
  grads    ||d_r|| <= rtol ||ref_r|| + rtol max(rms_head(||ref_r||), floor)     (r = one output row)
The floors (1e-3 nats; 1e-3 of a gradient row's natural size, see grad_floor) only matter for
heads whose exact result is zero or nearly so, where a relative test has no meaning.
"""
from __future__ import annotations

import os

import numpy as np
import torch

from attention_kl_amd import workloads as wl

RTOL = {"bf16": 2e-3, "fp32": 1e-5}


def rtol_of(w: wl.Workload) -> float:
    return RTOL[w.dtype]


def device_inputs(w: wl.Workload, dev="cuda"):
    """The four inputs as device tensors of w.dtype (bf16 or fp32) plus their float32 host copies."""
    host = wl.full_f32(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    devt = tuple(torch.from_numpy(a).to(dev).to(tdt) for a in host)  # exact: host values are already of tdt
    return devt, host


def device_inputs_bf16_bits(w: wl.Workload, dev="cuda"):
    """Large bf16 problems: ship bf16 bit patterns (half the host memory of float32)."""
    bits = wl.full_bf16_bits(w)
    return tuple(torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in bits)


KL_FLOOR = 1e-3  # nats: lower bound of the per-head KL magnitude used in the criterion


def _worst(ratio: np.ndarray) -> float:
    """Largest ratio; inf when any entry is not finite (a NaN or inf output fails every criterion,
    and np.max / Python's max would otherwise let a NaN through or drop it)."""
    ratio = np.asarray(ratio, np.float64)
    if ratio.size == 0:
        return 0.0
    if not np.all(np.isfinite(ratio)):
        return float("inf")
    return float(ratio.max())


def ratio_kl(gpu: np.ndarray, ref: np.ndarray, rtol: float) -> float:
    """Worst |d| / allowed over the last axis groups (heads); <= 1 passes."""
    gpu = np.asarray(gpu, np.float64).reshape(-1, gpu.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    rms = np.maximum(np.sqrt((ref ** 2).mean(axis=1, keepdims=True)), KL_FLOOR)
    allowed = rtol * np.abs(ref) + rtol * rms + 1e-30
    return _worst(np.abs(gpu - ref) / allowed)


def ratio_lse(gpu, ref, rtol) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return _worst(np.abs(gpu - ref) / (rtol * np.maximum(1.0, np.abs(ref))))


def grad_floor(scale: float, g: np.ndarray, other: np.ndarray) -> float:
    """1e-3 of a gradient row's natural size, scale * mean(g) * rms row norm of the operand it sums over.

    Used only as a lower bound of the per-head rms in the gradient criterion, for heads whose exact
    gradient is zero or nearly so (a row with one allowed key has P_s = P_t = 1 and dS = 0).
    """
    rn = np.linalg.norm(np.asarray(other, np.float64).reshape(-1, other.shape[-1]), axis=1)
    return 1e-3 * scale * float(np.mean(g)) * float(np.sqrt((rn ** 2).mean()))


def ratio_rows(gpu, ref, rtol, floor: float = 0.0) -> float:
    """Rows are the second-to-last axis; heads are everything before it."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    g2 = gpu.reshape(-1, gpu.shape[-2], gpu.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-2], ref.shape[-1])
    dn = np.linalg.norm(g2 - r2, axis=-1)
    rn = np.linalg.norm(r2, axis=-1)
    rms = np.maximum(np.sqrt((rn ** 2).mean(axis=1, keepdims=True)), floor)
    return _worst(dn / (rtol * rn + rtol * rms + 1e-30))


def worst_of(acc: dict, key: str, *values: float) -> None:
    """acc[key] = the largest of its old value and `values`, inf if any is not finite."""
    vals = [acc.get(key, 0.0), *values]
    acc[key] = float("inf") if not all(np.isfinite(v) for v in vals) else max(vals)


def all_pass(ratios: dict) -> bool:
    """Every ratio finite and <= 1."""
    return all(np.isfinite(v) and v <= 1.0 for v in ratios.values())


def report(name: str, **ratios) -> str:
    return name + " " + " ".join(f"{k}={v:.3g}" for k, v in ratios.items())


# ------------------------------------------------------------------ whole heads of the large workloads
def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_window(head, scale_t, scale_s, causal, g, r0=0, teacher=False, js=False, block=512, workers=None):
    """The float64 oracle on query rows r0 .. Nq-1 of one head, run as row-block sub-problems in threads.

    head = (qt, kt, qs, ks) float64 arrays of one head.  Rows [s, e) of a head form a problem of their
    own with keys [0, e + Nk - Nq) (causal: bottom-right alignment then gives each row exactly its keys
    in the whole head; not causal: all Nk keys), so each sub-problem's KL, LSE and dQ rows are those of
    the whole head and its dK is the contribution of its rows; the dK partials are summed.  With
    causal masking every row that sees a key j >= r0 + Nk - Nq lies in the window, so dK of those keys
    is complete; without it, dK is complete only for r0 = 0.  (tests/test_oracle.py pins that this
    reassembles the whole-head oracle.)

    Returns a dict: "rows" (the row indices), forward outputs for them ("kl", or "js" and "js_t"; "lse_t",
    "lse_s"), "dq_s" (and "dq_t"), "k0" (first key with a complete dK) and "dk_s" (and "dk_t") for keys
    k0 .. Nk-1."""
    import concurrent.futures as cf

    import oracle
    from threadpoolctl import threadpool_limits

    qt, kt, qs, ks = head
    nq, nk = qt.shape[0], kt.shape[0]
    off = nk - nq
    assert causal or r0 == 0, "without causal masking only the whole head gives complete dK"
    g = np.asarray(g, np.float64)
    blocks = [(s, min(s + block, nq)) for s in range(r0, nq, block)]
    sides = ("s", "t") if teacher else ("s",)
    out = {"rows": np.arange(r0, nq)}
    fwd_names = ("js", "js_t", "js_s", "lse_t", "lse_s") if js else ("kl", "lse_t", "lse_s")
    for n in fwd_names:
        out[n] = np.empty(nq - r0)
    for sd in sides:
        out["dq_" + sd] = np.empty((nq - r0, (qs if sd == "s" else qt).shape[1]))
        out["dk_" + sd] = np.zeros((nk, (ks if sd == "s" else kt).shape[1]))

    def run(blk):
        s, e = blk
        kend = e + off if causal else nk
        sub = (qt[s:e], kt[:kend], qs[s:e], ks[:kend])
        if js:
            f = oracle.js_forward_head(*sub, scale_t, scale_s, causal)
            b = oracle.js_backward_head(*sub, scale_t, scale_s, causal, g[s:e], teacher=teacher)
        else:
            f = oracle.forward_head(*sub, scale_t, scale_s, causal)
            b = oracle.backward_head(*sub, scale_t, scale_s, causal, g[s:e], teacher=teacher)
        return s, e, kend, f, b

    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers or _workers()) as ex:
            futs = [ex.submit(run, blk) for blk in blocks[::-1]]  # longest rows first
            for fu in cf.as_completed(futs):
                s, e, kend, f, b = fu.result()
                for n, v in zip(fwd_names, f):
                    out[n][s - r0:e - r0] = v
                for sd in sides:
                    out["dq_" + sd][s - r0:e - r0] = b["dq_" + sd]
                    out["dk_" + sd][:kend] += b["dk_" + sd]
    k0 = r0 + off if causal else 0
    out["k0"] = k0
    for sd in sides:
        out["dk_" + sd] = out["dk_" + sd][k0:]
    return out

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


def ratio_kl(gpu: np.ndarray, ref: np.ndarray, rtol: float) -> float:
    """Worst |d| / allowed over the last axis groups (heads); <= 1 passes."""
    gpu = np.asarray(gpu, np.float64).reshape(-1, gpu.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    rms = np.maximum(np.sqrt((ref ** 2).mean(axis=1, keepdims=True)), KL_FLOOR)
    allowed = rtol * np.abs(ref) + rtol * rms + 1e-30
    return float((np.abs(gpu - ref) / allowed).max())


def ratio_lse(gpu, ref, rtol) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float((np.abs(gpu - ref) / (rtol * np.maximum(1.0, np.abs(ref)))).max())


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
    return float((dn / (rtol * rn + rtol * rms + 1e-30)).max())


def report(name: str, **ratios) -> str:
    return name + " " + " ".join(f"{k}={v:.3g}" for k, v in ratios.items())

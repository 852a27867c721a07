"""Benchmark of the attention-KL hot path on one MI355X.

One step = the whole path on one batch: the forward (per-row KL + both LSEs) and
the student backward (dK_s then dQ_s), on the b1h32n32768d128 causal workload
(teacher keys 1% scaled x4, independent student), bf16 inputs already resident in
HBM.  Prints ONE JSON line; its `configs` object adds the same step timed on each
of the five synthetic workloads.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]
                  [--no-configs] [--copy-calibrate]

Work is counted as the method's algorithmic MFMA flops, each product once: the forward
2 (d_t + d_s) per allowed pair (both logit products), the backward 2 (d_t + 3 d_s) (the two
logit products, dQ_s and dK_s).  The two backward kernels each recompute both logit
products; that repeat is overhead and shows as `issued_tflops` per kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_PEAK_BF16_TFLOPS = 2516.6  # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
MI355X_PEAK_FP32_MFMA_TFLOPS = 157.3
MI355X_HBM_GBS = 8000.0
METRIC = "attention-KL fwd/bwd TFLOP/s and ms at N=32K, % of MFMA peak, extra HBM bytes"
_C = "attention_kl_amd/csrc/"
KERNEL_SOURCES = {"fwd": [_C + "skl_fwd.hip", _C + "skl_fwd_impl.hpp"],
                  "bwd_dq": [_C + "skl_bwd.hip", _C + "skl_bwd_impl.hpp"],
                  "bwd_dk": [_C + "skl_bwd.hip", _C + "skl_bwd_impl.hpp"]}


def source_sha(kernel: str) -> str:
    """Hash of the sources a kernel is built from (its template, launchers and the shared headers)."""
    paths = KERNEL_SOURCES[kernel] + [_C + "skl_device.hpp", _C + "skl_kernels.hpp"]
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def kernel_flops(w, kernel: str, pairs=None) -> float:
    """MFMA flops one launch issues for the allowed pairs (its `issued_tflops`).

    fwd:    both logit products, 2 (d_t + d_s) per allowed pair.
    bwd_dq: both logit products (the kernel has no other source of the logits) + dQ_s,
            2 (d_t + 2 d_s) per pair.   bwd_dk: the same with dK_s.
    bwd_teacher: both teacher kernels (dQ_t and dK_t), each 2 (2 d_t + d_s) per pair.
    Masked-tile work, and the second gradient product of the hi + lo form (taken only by inputs outside
    the fp16 product's range), are not counted.  The method's own (algorithmic) count, which the
    roofline fractions use, counts each product once: see step_flops.
    """
    pairs = w.pairs_per_head() * w.B * w.H if pairs is None else pairs
    if kernel == "fwd":
        return 2.0 * pairs * (w.d_t + w.d_s)
    if kernel == "js_fwd":  # Jensen-Shannon: the KL pass for the log-sum-exps, then the JS pass
        return 4.0 * pairs * (w.d_t + w.d_s)
    if kernel == "js_bwd":  # both backward kernels of the student side
        return 4.0 * pairs * (w.d_t + 2 * w.d_s)
    if kernel == "bwd_teacher":
        return 4.0 * pairs * (2 * w.d_t + w.d_s)
    return 2.0 * pairs * (w.d_t + 2 * w.d_s)


def step_flops(w, pairs=None, js=False, teacher=False):
    """Algorithmic MFMA flops of one step, each product counted once: forward 2 (d_t + d_s) per allowed
    pair (JS: twice, a streaming JS needs both log-sum-exps before its pass), backward 2 (d_t + 3 d_s)
    (two logit products, dQ_s, dK_s), plus 4 d_t for dQ_t and dK_t with teacher gradients."""
    P = w.pairs_per_head() * w.B * w.H if pairs is None else pairs
    fwd = (4.0 if js else 2.0) * P * (w.d_t + w.d_s)
    bwd = 2.0 * P * (w.d_t + 3 * w.d_s) + (4.0 * P * w.d_t if teacher else 0.0)
    return fwd, bwd


def host_info():
    """CPU model and BLAS library of the host (for the CPU baseline)."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return model, blas


def cpu_baseline(w, budget_rows: int):
    """The float64 oracle timed on the host on a bounded sample of the same workload.

    Sample: the last `budget_rows` query rows of head (0, 0) (each sees ~N keys), forward for
    those rows and backward for the same rows with dK for the last `budget_rows` keys.
    """
    import numpy as np

    import oracle
    from attention_kl_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    hh = wl.head_f64(w, 0, 0)
    g = wl.head_g(w, 0, 0)
    rows = np.arange(w.Nq - budget_rows, w.Nq)
    keys = np.arange(w.Nk - budget_rows, w.Nk)
    t0 = time.perf_counter()
    oracle.forward_head(*hh, w.scale_t, w.scale_s, w.causal, rows=rows)
    t1 = time.perf_counter()
    oracle.backward_head(*hh, w.scale_t, w.scale_s, w.causal, g, rows=rows, keys=keys)
    t2 = time.perf_counter()
    off = w.Nk - w.Nq
    row_pairs = int(sum(min(w.Nk, i + off + 1) if w.causal else w.Nk for i in rows))
    # pairs (i, j) with i in rows, j in keys, j allowed for i
    rk = sum(max(0, min(w.Nk, i + off + 1) - keys[0]) if w.causal else len(keys) for i in rows)
    fl_fwd = 2.0 * row_pairs * (w.d_t + w.d_s)
    fl_bwd = 2.0 * row_pairs * (w.d_t + 2 * w.d_s) + 2.0 * rk * w.d_s
    secs = t2 - t0
    model, blas = host_info()
    return {"value": (fl_fwd + fl_bwd) / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "blas": blas,
            "sample": f"float64 oracle on head (0,0): forward of the last {budget_rows} query rows, backward "
                      f"(dQ_s of those rows, dK_s of the last {budget_rows} keys); {secs:.2f} s "
                      f"(fwd {t1 - t0:.2f} s, bwd {t2 - t1:.2f} s)",
            "seconds": secs}


def load_traffic(kernel: str, workload: str):
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(workload, {}).get(kernel)
        if not e or e.get("source_sha") != source_sha(kernel):
            return None  # counters were taken on a different kernel
        return float(e["hbm_bytes_per_launch"])
    except Exception:
        return None


def _kernel_class(name: str):
    """Map a rocprofv3 kernel name to fwd / bwd_dq / bwd_dk / copy (None for anything else)."""
    if "fwd_kernel" in name:
        return "fwd"
    if "bwd_kernel" in name:
        # template arguments <T, DT, DS, CAUSAL, TEACHER, OWN_Q, GRP>: OWN_Q picks the query owner (dQ)
        m = re.search(r"bwd_kernel<([^>]*)>", name)
        if m:
            own_q = m.group(1).split(",")[5].strip() in ("true", "1")
        else:  # mangled: the four bool arguments are Lb0E / Lb1E
            own_q = re.findall(r"Lb([01])E", name)[2] == "1"
        return "bwd_dq" if own_q else "bwd_dk"
    if "copy" in name.lower():
        return "copy"
    return None


def _pmc_means(csv_path: str, counter: str):
    """Mean per-dispatch value of one counter for each kernel class in a rocprofv3 counter CSV, over
    the dispatches of that class with the largest grid (the workload's own launches, not the small
    warm-up calls the bench makes first)."""
    import csv
    import collections
    per = collections.defaultdict(float)
    cls, grid = {}, {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        k = _kernel_class(r["Kernel_Name"])
        if k is None:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        cls[r["Dispatch_Id"]] = k
        grid[r["Dispatch_Id"]] = int(r.get("Grid_Size") or 0)
    top = collections.defaultdict(int)
    for d, k in cls.items():
        top[k] = max(top[k], grid[d])
    out = collections.defaultdict(list)
    for d, v in per.items():
        if grid[d] == top[cls[d]]:
            out[cls[d]].append(v)
    return {k: sum(v) / len(v) for k, v in out.items()}


def ingest_pmc(fetch_csv: str, write_csv: str, workload: str, copy_bytes: int = 1 << 30):
    """Turn FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) into HBM bytes per launch.

    Each counter is scaled by copy_bytes / (what it reads for the plain device copy of copy_bytes
    bytes run in the same process), and the result is stored with a hash of each kernel's source so
    that bench.py reports it only while the kernel is unchanged.
    """
    f = _pmc_means(fetch_csv, "FETCH_SIZE")
    w = _pmc_means(write_csv, "WRITE_SIZE")
    ff = copy_bytes / (f["copy"] * 1024.0)
    fw = copy_bytes / (w["copy"] * 1024.0)
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    d = json.load(open(p)) if os.path.exists(p) else {}
    ent = {"copy_calibration": {"bytes": copy_bytes, "fetch_kib": f["copy"], "write_kib": w["copy"],
                                "fetch_factor": ff, "write_factor": fw}}
    for k in ("fwd", "bwd_dq", "bwd_dk"):
        if k in f and k in w:
            ent[k] = {"fetch_kib": f[k], "write_kib": w[k],
                      "hbm_bytes_per_launch": f[k] * 1024.0 * ff + w[k] * 1024.0 * fw,
                      "source_sha": source_sha(k)}
    d[workload] = ent
    json.dump(d, open(p, "w"), indent=1)
    return ent


def autograd_step(w, qt, kt, qs, ks, g, raw_ms: float, steps: int = 3, seg=None, direction="kl"):
    """The same step (forward, student dQ and dK) through torch autograd: sum_i g_i KL_i .backward().

    Beyond the raw kernels it pays for autograd bookkeeping, output allocation and the cast of
    the float32 gradients to the bf16 dtype of the inputs.
    """
    import torch
    from attention_kl_amd.loss import attention_kl
    qs_ = qs.detach().requires_grad_(True)
    ks_ = ks.detach().requires_grad_(True)

    def run():
        qs_.grad = ks_.grad = None
        kl = attention_kl(qt, kt, qs_, ks_, causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s,
                          direction="js" if direction == "js" else "forward", **(seg or {}))
        (kl * g).sum().backward()

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"ms_per_step": round(ms, 4), "overhead_ms": round(ms - raw_ms, 4), "steps": steps,
            "what": "attention_kl(...) then (kl * g).sum().backward(), bf16 gradients into q_s, k_s"}


def _f32_or_bf16_inputs(w, dev):
    """The workload's four inputs on the device (bf16 bit patterns shipped as int16, or float32)."""
    import numpy as np
    import torch
    from attention_kl_amd import workloads as wl
    if w.dtype == "bf16":
        bits = wl.full_bf16_bits(w)
        return tuple(torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in bits)
    return tuple(torch.from_numpy(a).to(dev) for a in wl.full_f32(w))


def warm_library(dev, w):
    """Tiny forwards and backwards with workload w's head dims, dtype and mask, so that loading the
    kernels' code (device memory of the runtime's own, taken at a kernel's first launch) falls
    outside every measurement of what the path allocates."""
    import torch
    from attention_kl_amd import streamkl as S
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    xt = torch.zeros((1, 1, 64, w.d_t), dtype=dt, device=dev)
    xs = torch.zeros((1, 1, 64, w.d_s), dtype=dt, device=dev)
    x = (xt, xt, xs, xs)
    kl, lt, ls = S.fwd(*x, causal=w.causal)
    S.bwd(*x, lt, ls, torch.ones_like(kl), causal=w.causal, kl=kl, teacher_grads=True)
    S.bwd_dq(*x, lt, ls, torch.ones_like(kl), causal=w.causal)
    S.bwd_dk(*x, lt, ls, torch.ones_like(kl), causal=w.causal)
    js, lt, ls, ht = S.js_fwd(*x, causal=w.causal)
    S.js_bwd(*x, lt, ls, js, ht, torch.ones_like(kl), causal=w.causal)
    torch.cuda.synchronize()


def measured_peak(dev, iters: int = 4000, nblocks: int = 4096):
    """Dense bf16 MFMA rate this GPU sustains (register operands, no memory traffic) and the shader
    clock meanwhile, from the library's probe (include/streamkl_probe.h)."""
    import ctypes
    import numpy as np
    import torch
    from attention_kl_amd import streamkl as S
    sink = torch.empty(nblocks * 256, dtype=torch.float32, device=dev)
    clk = torch.empty(2 * nblocks, dtype=torch.int64, device=dev)
    khz = ctypes.c_double(0.0)
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(2):  # the first launch warms the clock up
        assert S.lib().streamkl_probe_mfma(nblocks, iters, sink.data_ptr(), clk.data_ptr(), ctypes.byref(khz), s) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    assert S.lib().streamkl_probe_mfma(nblocks, iters, sink.data_ptr(), clk.data_ptr(), ctypes.byref(khz), s) == 0
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = nblocks * 4 * 4 * iters * 32768.0
    c = clk.view(-1, 2).cpu().numpy().astype(np.float64)
    ok = c[:, 1] > 0
    ghz = float(np.median(c[ok, 0] / c[ok, 1]) * khz.value / 1e6) if ok.any() else None
    return {"tflops": round(flops / ms / 1e9, 1), "clock_ghz": None if ghz is None else round(ghz, 3),
            "published_tflops": MI355X_PEAK_BF16_TFLOPS,
            "what": f"{nblocks} workgroups x 4 waves, 4 independent v_mfma_f32_32x32x16_bf16 chains of {iters} "
                    "each on register operands; clock = shader-clock counter / constant-rate counter"}


def alloc_outside_torch(free0: int, reserved0: int) -> int:
    """Device bytes taken since free0 (hipMemGetInfo) that torch's caching allocator does not hold:
    what the library allocated by itself.  The caller workspace the binding attaches for some paths is
    a torch tensor (reported as workspace_bytes), so a segment the allocator reserves for it is not
    counted here."""
    import torch
    return max(0, (free0 - torch.cuda.mem_get_info()[0]) - (torch.cuda.memory_reserved() - reserved0))


def time_step(w, dev, steps: int, warmup: int):
    """Forward, dK_s, dQ_s of workload w, each launch timed with HIP events on the launch stream.

    Returns per-kernel mean ms, the step's mean ms, what the library path allocated on its first call
    and the floats of the workspace the binding attaches (small causal forwards, grouped keys)."""
    import ctypes
    import numpy as np
    import torch
    from attention_kl_amd import streamkl as S
    from attention_kl_amd import workloads as wl
    qt, kt, qs, ks = _f32_or_bf16_inputs(w, dev)
    ws_floats = int(S.lib().streamkl_workspace_floats(ctypes.byref(
        S.make_problem(qt, kt, qs, ks, w.causal, w.scale_t, w.scale_s))))
    g = torch.from_numpy(wl.full_g(w)).to(dev)
    kl = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    lt, ls = torch.empty_like(kl), torch.empty_like(kl)
    dq = torch.empty((w.B, w.H, w.Nq, w.d_s), dtype=torch.float32, device=dev)
    dk = torch.empty((w.B, w.H, w.Nk, w.d_s), dtype=torch.float32, device=dev)
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)

    def step(ev=None):
        ev and ev[0].record()
        S.fwd(qt, kt, qs, ks, out=(kl, lt, ls), **kw)
        ev and ev[1].record()
        S.bwd_dk(qt, kt, qs, ks, lt, ls, g, out=dk, **kw)
        ev and ev[2].record()
        S.bwd_dq(qt, kt, qs, ks, lt, ls, g, out=dq, **kw)
        ev and ev[3].record()

    torch.cuda.synchronize()
    free0, res0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_reserved()
    step()  # the first call: whatever the library allocates shows here
    torch.cuda.synchronize()
    lib_alloc = alloc_outside_torch(free0, res0)
    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms = {k: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, k in
          enumerate(("fwd", "bwd_dk", "bwd_dq"))}
    step_ms = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))

    # the backward as one streamkl_bwd call, as the autograd wrapper makes it: for small problems its
    # two kernels run side by side on two streams, so only the call as a whole is timed
    def step_call(ev=None):
        ev and ev[0].record()
        S.fwd(qt, kt, qs, ks, out=(kl, lt, ls), **kw)
        ev and ev[1].record()
        S.bwd(qt, kt, qs, ks, lt, ls, g, out=[dq, dk], **kw)
        ev and ev[2].record()

    for _ in range(warmup + 1):
        step_call()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        step_call(e)
    torch.cuda.synchronize()
    ms["bwd_call"] = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms["step_call"] = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
    del qt, kt, qs, ks, g, kl, lt, ls, dq, dk
    torch.cuda.empty_cache()
    return ms, step_ms, int(lib_alloc), ws_floats


def config_entry(w, ms, step_ms, lib_alloc, peak=None, workspace_floats=0):
    """The bench line's record of one workload: ms and algorithmic TFLOP/s of the forward, the backward
    pair and the step, with their fractions of the published (and measured) peak."""
    fwd_fl, bwd_fl = step_flops(w)
    bwd_ms = ms["bwd_dk"] + ms["bwd_dq"]
    mp = MI355X_PEAK_BF16_TFLOPS if w.dtype == "bf16" else MI355X_PEAK_FP32_MFMA_TFLOPS
    e = {"fwd_ms": round(ms["fwd"], 4), "bwd_dk_ms": round(ms["bwd_dk"], 4), "bwd_dq_ms": round(ms["bwd_dq"], 4),
         "bwd_ms": round(bwd_ms, 4), "step_ms": round(step_ms, 4),
         "fwd_tflops": round(fwd_fl / ms["fwd"] / 1e9, 2), "bwd_tflops": round(bwd_fl / bwd_ms / 1e9, 2),
         "step_tflops": round((fwd_fl + bwd_fl) / step_ms / 1e9, 2),
         "fwd_frac": round(fwd_fl / ms["fwd"] / 1e9 / mp, 4), "bwd_frac": round(bwd_fl / bwd_ms / 1e9 / mp, 4),
         "peak_tflops": mp, "dtype": w.dtype,
         **({"bwd_call_ms": round(ms["bwd_call"], 4), "step_call_ms": round(ms["step_call"], 4),
             "step_call_tflops": round((fwd_fl + bwd_fl) / ms["step_call"] / 1e9, 2)} if "bwd_call" in ms else {}),
         "extra_hbm_bytes": 12 * w.B * w.H * w.Nq + 4 * int(workspace_floats),
         "workspace_bytes": 4 * int(workspace_floats), "library_alloc_bytes": lib_alloc}
    if peak and w.dtype == "bf16":
        e["fwd_frac_of_measured_peak"] = round(fwd_fl / ms["fwd"] / 1e9 / peak["tflops"], 4)
        e["bwd_frac_of_measured_peak"] = round(bwd_fl / bwd_ms / 1e9 / peak["tflops"], 4)
    return e


def power_profile(w, dev, seconds: float = 6.0):
    """Board power and shader clocks while each kernel of workload w (and the MFMA probe) runs back to
    back for `seconds`: `amd-smi metric -p -c --json` sampled every 0.5 s; medians of the samples
    taken after the first second.  None where amd-smi is missing or reports no socket power."""
    import ctypes
    import shutil
    import statistics
    import subprocess
    import threading
    import torch
    from attention_kl_amd import streamkl as S
    from attention_kl_amd import workloads as wl
    if shutil.which("amd-smi") is None:
        return None
    qt, kt, qs, ks = _f32_or_bf16_inputs(w, dev)
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s)
    kl, lt, ls = S.fwd(qt, kt, qs, ks, **kw)
    g = torch.from_numpy(wl.full_g(w)).to(dev)
    dq = torch.empty((w.B, w.H, w.Nq, w.d_s), dtype=torch.float32, device=dev)
    dk = torch.empty((w.B, w.H, w.Nk, w.d_s), dtype=torch.float32, device=dev)
    psink = torch.empty(4096 * 256, dtype=torch.float32, device=dev)
    pclk = torch.empty(2 * 4096, dtype=torch.int64, device=dev)
    khz = ctypes.c_double(0.0)
    launches = {
        "mfma_probe": lambda: S.lib().streamkl_probe_mfma(4096, 4000, psink.data_ptr(), pclk.data_ptr(),
                                                          ctypes.byref(khz), torch.cuda.current_stream().cuda_stream),
        "fwd": lambda: S.fwd(qt, kt, qs, ks, out=(kl, lt, ls), **kw),
        "bwd_dk": lambda: S.bwd_dk(qt, kt, qs, ks, lt, ls, g, out=dk, **kw),
        "bwd_dq": lambda: S.bwd_dq(qt, kt, qs, ks, lt, ls, g, out=dq, **kw),
    }

    def sample():
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        d = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = [v["clk"]["value"] for k, v in d["clock"].items() if k.startswith("gfx_") and isinstance(v, dict)]
        return float(d["power"]["socket_power"]["value"]), [float(c) for c in clk]

    out = {}
    for name, fn in launches.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        samples, stop = [], threading.Event()

        def sampler():
            t0 = time.perf_counter()
            while not stop.is_set():
                try:
                    p_w, clk = sample()
                    if time.perf_counter() - t0 > 1.0:
                        samples.append((p_w, clk))
                except Exception:
                    pass
                stop.wait(0.5)
        th = threading.Thread(target=sampler)
        th.start()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                fn()
                n += 1
            torch.cuda.synchronize()
        el = time.perf_counter() - t0
        stop.set()
        th.join()
        if not samples:
            return None
        nx = len(samples[0][1])
        out[name] = {"socket_power_w": statistics.median(p for p, _ in samples),
                     "gfx_clock_mhz_per_xcd": [statistics.median(c[i] for _, c in samples) for i in range(nx)],
                     "ms_per_launch": round(el * 1e3 / n, 3), "samples": len(samples)}
    del qt, kt, qs, ks, g, kl, lt, ls, dq, dk, psink, pclk
    torch.cuda.empty_cache()
    out["what"] = (f"each kernel of {w.name} (and the MFMA probe) launched back to back for {seconds:.0f} s; "
                   "amd-smi socket power and per-XCD gfx clocks every 0.5 s, medians after the first second")
    return out


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--ingest-pmc":
        # python bench.py --ingest-pmc <fetch counter csv> <write counter csv> [workload id]
        from attention_kl_amd import workloads as wl
        w = wl.WORKLOADS[int(sys.argv[4]) if len(sys.argv) > 4 else 3]
        print(json.dumps(ingest_pmc(sys.argv[2], sys.argv[3], w.name), indent=1))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="synthetic workload id in workloads.WORKLOADS (3 = b1h32n32768d128 causal)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other synthetic workloads (the line's `configs` object)")
    ap.add_argument("--no-peak", action="store_true", help="skip the measured MFMA peak and clock")
    ap.add_argument("--cpu-rows", type=int, default=12288)
    ap.add_argument("--no-autograd", action="store_true",
                    help="skip timing the same step through the torch autograd wrapper (attention_kl_amd.loss)")
    ap.add_argument("--student-key-heads", type=int, default=None,
                    help="grouped student keys: K key heads shared by the H query heads (K divides H); key head j "
                         "is the workload's head j*H/K.  Default: one key head per query head")
    ap.add_argument("--teacher-grads", action="store_true",
                    help="KL step with the teacher's gradients too (two more backward kernels, timed together)")
    ap.add_argument("--divergence", choices=("kl", "js"), default="kl",
                    help="kl (default): KL(P_t || P_s); js: the Jensen-Shannon step (streamkl_js_fwd + streamkl_js_bwd)")
    ap.add_argument("--packed-mix", type=int, default=None, metavar="SEED",
                    help="packed variable-length batch: the workload's rows cut into segments of a seeded "
                         "log-uniform length mix (256..8192 rows), each its own (causal) problem")
    ap.add_argument("--power", action="store_true",
                    help="also sample board power and per-XCD clocks while each kernel runs back to back (amd-smi)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; the path shards by heads with no exchange in the "
              "forward, but no multi-GPU run is implemented or measured here.", file=sys.stderr)
        sys.exit(2)

    import ctypes

    import numpy as np
    import torch

    from attention_kl_amd import streamkl as S
    from attention_kl_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S.lib()  # fail loudly if the library is missing
    warm_library(dev, w)
    qt, kt, qs, ks = _f32_or_bf16_inputs(w, dev)
    g = torch.from_numpy(wl.full_g(w)).to(dev)
    B, H = w.B, w.H
    hk_s = H if args.student_key_heads is None else args.student_key_heads
    if hk_s < 1 or H % hk_s != 0:
        print(f"bench.py: --student-key-heads must divide H = {H}", file=sys.stderr)
        sys.exit(2)
    ks = ks[:, ::H // hk_s]
    seg = {}
    pairs = None  # allowed pairs of the whole step (None: the workload's own)
    if args.packed_mix is not None:
        if B != 1 or hk_s != H:
            print("bench.py: --packed-mix needs a one-entry workload and no key grouping", file=sys.stderr)
            sys.exit(2)
        lens = wl.length_mix(w.Nq, args.packed_mix)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        # offsets built here, checked once below: the timed calls skip the binding's read-back
        S.make_problem(*(x[0].permute(1, 0, 2) for x in (qt, kt, qs, ks)), w.causal, cu_seqlens_q=cu, cu_seqlens_k=cu)
        seg = dict(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=max(lens), max_seqlen_k=max(lens), validate=False)
        qt, kt, qs, ks = (x[0].permute(1, 0, 2) for x in (qt, kt, qs, ks))  # [N, H, d] views, same memory
        g = g[0]
        per_seg = [(n * (n + 1) // 2) if w.causal else n * n for n in lens]
        pairs = sum(per_seg) * H
    lead = () if seg else (B,)  # a packed batch takes the one-entry layout [H, N...]
    kl = torch.empty(lead + (H, w.Nq), dtype=torch.float32, device=dev)
    lt = torch.empty_like(kl)
    ls = torch.empty_like(kl)
    dq = torch.empty(lead + (H, w.Nq, w.d_s), dtype=torch.float32, device=dev)
    dk = torch.empty(lead + (hk_s, w.Nk, w.d_s), dtype=torch.float32, device=dev)
    kw = dict(causal=w.causal, scale_t=w.scale_t, scale_s=w.scale_s, **seg)
    js = args.divergence == "js"
    ht = torch.empty_like(kl)  # JS: the teacher half KL(P_t || M)
    teacher = args.teacher_grads
    if teacher and (js or seg or hk_s != H):
        print("bench.py: --teacher-grads goes with the dense KL step", file=sys.stderr)
        sys.exit(2)
    dqt = torch.empty(lead + (H, w.Nq, w.d_t), dtype=torch.float32, device=dev) if teacher else None
    dkt = torch.empty(lead + (H, w.Nk, w.d_t), dtype=torch.float32, device=dev) if teacher else None
    # the caller workspace the binding attaches for grouped keys (part of the path's extra HBM)
    prob = S.make_problem(qt, kt, qs, ks, w.causal, w.scale_t, w.scale_s,
                          **{k: v for k, v in seg.items()})
    ws_floats = int(S.lib().streamkl_workspace_floats(ctypes.byref(prob)))

    def step(ev=None):
        if js:  # forward (two launches), then both student backward kernels
            if ev is not None:
                ev[0].record()
            S.js_fwd(qt, kt, qs, ks, out=(kl, lt, ls, ht), **kw)
            if ev is not None:
                ev[1].record()
            S.js_bwd(qt, kt, qs, ks, lt, ls, kl, ht, g, out=[dq, dk], **kw)
            if ev is not None:
                ev[2].record()
                ev[3].record()
            return
        if ev is not None:
            ev[0].record()
        S.fwd(qt, kt, qs, ks, out=(kl, lt, ls), **kw)
        if ev is not None:
            ev[1].record()
        S.bwd_dk(qt, kt, qs, ks, lt, ls, g, out=dk, **kw)
        if ev is not None:
            ev[2].record()
        S.bwd_dq(qt, kt, qs, ks, lt, ls, g, out=dq, **kw)
        if ev is not None:
            ev[3].record()
        if teacher:
            S.bwd(qt, kt, qs, ks, lt, ls, g, kl=kl, teacher_grads=True, student_grads=False,
                  out=[None, None, dqt, dkt], **kw)
            if ev is not None:
                ev[4].record()

    # what the library itself allocates: device memory taken around the first call beyond what torch's
    # caching allocator reserves (it grows by the binding's workspace here, if any, and keeps it)
    torch.cuda.synchronize()
    free0, res0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_reserved()
    step()
    torch.cuda.synchronize()
    first_call_alloc = alloc_outside_torch(free0, res0)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibrate:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    free0, res0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_reserved()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5 if teacher else 4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steady_alloc = alloc_outside_torch(free0, res0)
    per = {"js_fwd": [], "js_bwd": []} if js else {"fwd": [], "bwd_dk": [], "bwd_dq": []}
    if teacher:
        per["bwd_teacher"] = []
    for e in evs:
        if js:
            per["js_fwd"].append(e[0].elapsed_time(e[1]))
            per["js_bwd"].append(e[1].elapsed_time(e[2]))
            continue
        per["fwd"].append(e[0].elapsed_time(e[1]))
        per["bwd_dk"].append(e[1].elapsed_time(e[2]))
        per["bwd_dq"].append(e[2].elapsed_time(e[3]))
        if teacher:
            per["bwd_teacher"].append(e[3].elapsed_time(e[4]))
    step_ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))
    kern = {}
    for k, v in per.items():
        ms = float(np.mean(v))
        fl = kernel_flops(w, k, pairs)
        kern[k] = {"ms": round(ms, 4), "issued_tflops": round(fl / ms / 1e9, 2),
                   "issued_frac_of_bf16_peak": round(fl / ms / 1e9 / MI355X_PEAK_BF16_TFLOPS, 4)}
    P = pairs if pairs is not None else w.pairs_per_head() * B * H
    fwd_fl, bwd_fl = step_flops(w, P, js=js, teacher=teacher)
    fwd_ms = kern["js_fwd" if js else "fwd"]["ms"]
    bwd_ms = kern["js_bwd"]["ms"] if js else kern["bwd_dk"]["ms"] + kern["bwd_dq"]["ms"]
    if teacher:
        bwd_ms += kern["bwd_teacher"]["ms"]
    plain = hk_s == H and not seg and not js and not teacher  # the kernels the traffic counters were taken on

    def traffic(*ks_):
        t = [load_traffic(k, w.name) for k in ks_]
        return None if (not plain or any(x is None for x in t)) else sum(t)

    peak = None if args.no_peak else measured_peak(dev)

    def roof(kernel, fl, ms, tr):
        a = fl / ms / 1e9
        r = {"bound": "mfma", "kernel": kernel, "achieved": round(a, 2), "peak": MI355X_PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(a / MI355X_PEAK_BF16_TFLOPS, 4), "traffic": tr,
             "flops_per_launch": fl, "ms_per_launch": round(ms, 4)}
        if peak:
            r["frac_of_measured_peak"] = round(a / peak["tflops"], 4)
        return r

    # the dominant kernel is the backward pair (its two launches together carry the backward's work,
    # each product counted once); the forward, the spec kernel, gets its own entry
    roof_bwd = roof("bwd_dk+bwd_dq" if not js else "js_bwd", bwd_fl if not teacher else step_flops(w, P)[1],
                    kern["js_bwd"]["ms"] if js else kern["bwd_dk"]["ms"] + kern["bwd_dq"]["ms"],
                    traffic("bwd_dk", "bwd_dq"))
    roof_fwd = roof("js_fwd" if js else "fwd", fwd_fl, fwd_ms, traffic("fwd"))
    value = (fwd_fl + bwd_fl) / step_ms / 1e9
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded N(0,1) bf16 inputs of the workload's shape)",
        "config": {"workload": w.name + (f"-hks{hk_s}" if hk_s != H else "") + (
                       f"-packed{len(seg and lens)}seg" if seg else "") + ("-js" if js else "") + ("-teacher" if teacher else ""),
                   "B": B, "H": H,
                   "N_Q": w.Nq, "N_K": w.Nk, "d_t": w.d_t, "d_s": w.d_s, "causal": w.causal, "teacher_grads": teacher,
                   "student_key_heads": hk_s, "divergence": args.divergence},
        "fwd_ms": fwd_ms, "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(fwd_fl / fwd_ms / 1e9, 2), "bwd_tflops": round(bwd_fl / bwd_ms / 1e9, 2),
        "fwd_frac_of_bf16_peak": round(fwd_fl / fwd_ms / 1e9 / MI355X_PEAK_BF16_TFLOPS, 4),
        "bwd_frac_of_bf16_peak": round(bwd_fl / bwd_ms / 1e9 / MI355X_PEAK_BF16_TFLOPS, 4),
        "extra_hbm_bytes": 12 * B * H * w.Nq + (4 * B * H * w.Nq if js else 0) + 4 * ws_floats,
        "workspace_bytes": 4 * ws_floats,
        "library_alloc_bytes": int(max(first_call_alloc, steady_alloc)),
        "materialised_bytes_avoided": 2 * 4 * P,
        "kernels": kern, "wall_s_timed": round(wall, 3),
        "roofline": roof_bwd,
        "roofline_fwd": roof_fwd,
    }
    if peak:
        out["measured_peak"] = peak
    plain_line = plain and args.workload == 3
    if not args.no_autograd:
        out["autograd"] = autograd_step(w, qt, kt, qs, ks, g, step_ms, seg=seg, direction=args.divergence)
    del qt, kt, qs, ks, g, kl, lt, ls, dq, dk, dqt, dkt
    torch.cuda.empty_cache()
    if plain_line and not args.no_configs:
        # the same step on every synthetic workload; this line's own numbers stand for workload 3
        cfg = {}
        for wid in sorted(wl.WORKLOADS):
            wi = wl.WORKLOADS[wid]
            if wid == args.workload:
                ms = {k: kern[k]["ms"] for k in ("fwd", "bwd_dk", "bwd_dq")}
                cfg[wi.name] = config_entry(wi, ms, step_ms, out["library_alloc_bytes"], peak, ws_floats)
                continue
            print(f"bench: timing {wi.name}", file=sys.stderr, flush=True)
            big = wi.pairs_per_head() * wi.B * wi.H > 1e10
            ms, sms, la, wsf = time_step(wi, dev, steps=min(args.steps, 5) if big else args.steps,
                                         warmup=min(args.warmup, 2))
            cfg[wi.name] = config_entry(wi, ms, sms, la, peak, wsf)
        out["configs"] = cfg
    if args.power and not seg and not js and not teacher:
        print("bench: sampling power", file=sys.stderr, flush=True)
        out["power"] = power_profile(w, dev)
    if not args.no_cpu_baseline and not seg and not js:  # the CPU sample is of the dense KL workload's rows
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

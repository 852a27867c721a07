"""Python binding of libstreamkl.so (the C ABI in include/streamkl.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  torch supplies device memory and the current HIP stream.  When the
library is missing, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libstreamkl.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADER = os.path.join(INCLUDE, "streamkl.h")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_SCRATCH = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_FLOATS = 16 << 20  # STREAMKL_NOALLOC_SCRATCH_FLOATS
FP32, BF16 = 0, 1


class StreamKLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_I64x3 = ctypes.c_int64 * 3


class Problem(ctypes.Structure):
    """Mirror of streamkl_problem_t."""

    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("Nq", ctypes.c_int64), ("Nk", ctypes.c_int64),
                ("d_t", ctypes.c_int32), ("d_s", ctypes.c_int32),
                ("scale_t", ctypes.c_float), ("scale_s", ctypes.c_float),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("stride_qt", _I64x3), ("stride_kt", _I64x3), ("stride_qs", _I64x3), ("stride_ks", _I64x3),
                ("Hk_t", ctypes.c_int64), ("Hk_s", ctypes.c_int64),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("max_seqlen_q", ctypes.c_int64), ("max_seqlen_k", ctypes.c_int64),
                ("workspace", ctypes.c_void_p), ("workspace_floats", ctypes.c_int64)]

    @property
    def packed(self) -> bool:
        return bool(self.cu_seqlens_q)

    def stat_shape(self):
        """Shape of kl, lse_t, lse_s and g: [B, H, Nq], or [H, Nq] for a packed batch."""
        return (self.H, self.Nq) if self.packed else (self.B, self.H, self.Nq)

    def dq_shape(self, d: int):
        return (self.H, self.Nq, d) if self.packed else (self.B, self.H, self.Nq, d)

    def dk_shape(self, hk: int, d: int):
        return (hk, self.Nk, d) if self.packed else (self.B, hk, self.Nk, d)


_lib = None
_vp = ctypes.c_void_p
_P = ctypes.POINTER(Problem)


def lib() -> ctypes.CDLL:
    """Load libstreamkl.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_kl_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.streamkl_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.streamkl_bwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.streamkl_bwd_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.streamkl_bwd_dq.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.streamkl_bwd_dk.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.streamkl_js_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.streamkl_js_bwd.argtypes = [_P] + [_vp] * 14
        for f in ("streamkl_fwd", "streamkl_bwd", "streamkl_bwd_dq", "streamkl_bwd_dk", "streamkl_js_fwd",
                  "streamkl_js_bwd", "streamkl_bwd_noalloc", "streamkl_version"):
            getattr(L, f).restype = ctypes.c_int
        L.streamkl_workspace_floats.argtypes = [_P]
        L.streamkl_workspace_floats.restype = ctypes.c_int64
        L.streamkl_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp, ctypes.POINTER(ctypes.c_double), _vp]
        L.streamkl_probe_mfma.restype = ctypes.c_int
        L.streamkl_status_string.argtypes = [ctypes.c_int]
        L.streamkl_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def declared_symbols() -> list:
    """Entry points declared in the library's headers (include/*.h)."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            txt = open(os.path.join(INCLUDE, f)).read()
            names |= set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(streamkl_\w+)\s*\(", txt, re.M))
    return sorted(names)


def status_string(status: int) -> str:
    return lib().streamkl_status_string(status).decode()


def version() -> int:
    return lib().streamkl_version()


def _check(status: int, what: str):
    if status != OK:
        raise StreamKLError(status, f"{what}: {status_string(status)}")


def attach_workspace(p: Problem, device, stream=None):
    """Give p the workspace the library asks for (grouped key heads with few key heads: the key-owner
    work of each group is then split over several workgroups; small causal forwards: the long query
    blocks' key tiles are split over two workgroups).  Returns the tensor (or None), which
    must stay alive until the launches that use it are enqueued; torch's allocator keeps it from
    being reused before they run on its stream."""
    import torch
    n = lib().streamkl_workspace_floats(ctypes.byref(p))
    if n <= 0:
        return None
    ws = torch.empty(n, dtype=torch.float32, device=device)
    if stream is not None:
        ws.record_stream(stream)
    p.workspace, p.workspace_floats = ws.data_ptr(), n
    return ws


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_problem(qt, kt, qs, ks, causal: bool, scale_t: Optional[float] = None,
                 scale_s: Optional[float] = None, cu_seqlens_q=None, cu_seqlens_k=None,
                 max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                 validate: bool = True) -> Problem:
    """Describe q [B, H, Nq, d] and k [B, Hk, Nk, d] tensors (d unit-stride) as a streamkl_problem_t.

    Each side's key-head count Hk (k.shape[1]) must divide H: query head h reads key head
    h // (H // Hk) of that side (grouped-query attention; Hk == H is one key head per query head).

    Packed variable-length batch: pass cu_seqlens_q and cu_seqlens_k (int32 device tensors of
    length B + 1, the segments' row offsets) and q [Nq, H, d], k [Nk, Hk, d] holding every
    segment's rows one after another.  The offsets are read back (a synchronisation) and checked:
    non-negative, non-decreasing, within the packed rows, keys for every segment with queries (as
    many as its queries when causal), and no segment longer than max_seqlen_q / max_seqlen_k, which
    default to the longest segment; a ValueError is raised before anything is launched.
    validate=False skips the read-back (both max_seqlen must then be given); the kernels clamp
    every offset into the packed axis, so unchecked offsets cannot reach outside the buffers."""
    import torch
    packed = cu_seqlens_q is not None or cu_seqlens_k is not None
    if packed:
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise ValueError("a packed batch needs both cu_seqlens_q and cu_seqlens_k")
        for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
            if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous() or c.device != qt.device:
                raise ValueError(f"{name} must be a contiguous int32 vector on the inputs' device")
        if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 >= 1 entries")
        for name, t in (("q_t", qt), ("k_t", kt), ("q_s", qs), ("k_s", ks)):
            if t.dim() != 3:
                raise ValueError(f"{name} of a packed batch must be [N, heads, d], got {tuple(t.shape)}")
        # the packed axis is the n axis of a one-entry batch
        qt, kt, qs, ks = (t.permute(1, 0, 2).unsqueeze(0) for t in (qt, kt, qs, ks))
    for name, t in (("q_t", qt), ("k_t", kt), ("q_s", qs), ("k_s", ks)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got {tuple(t.shape)}")
        if t.stride(-1) != 1 and t.shape[-1] > 1:
            raise ValueError(f"{name}: the d axis must be contiguous")
        if t.dtype != qt.dtype:
            raise ValueError("all four inputs must share one dtype")
    B, H, Nq, d_t = qt.shape
    Hk_t, Nk = kt.shape[1], kt.shape[2]
    Hk_s, d_s = ks.shape[1], qs.shape[3]
    if (tuple(kt.shape) != (B, Hk_t, Nk, d_t) or tuple(qs.shape) != (B, H, Nq, d_s)
            or tuple(ks.shape) != (B, Hk_s, Nk, d_s)):
        raise ValueError(f"shape mismatch: {tuple(qt.shape)} {tuple(kt.shape)} {tuple(qs.shape)} {tuple(ks.shape)}")
    for name, hk in (("k_t", Hk_t), ("k_s", Hk_s)):
        if H > 0 and (hk < 1 or H % hk != 0):
            raise ValueError(f"{name} has {hk} heads, which does not divide the {H} query heads")
    dt = {torch.bfloat16: BF16, torch.float32: FP32}.get(qt.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {qt.dtype}")
    p = Problem()
    p.B, p.H, p.Nq, p.Nk, p.d_t, p.d_s = B, H, Nq, Nk, d_t, d_s
    p.Hk_t, p.Hk_s = Hk_t, Hk_s
    p.scale_t = 1.0 / math.sqrt(d_t) if scale_t is None else scale_t
    p.scale_s = 1.0 / math.sqrt(d_s) if scale_s is None else scale_s
    p.causal = int(bool(causal))
    p.dtype = dt
    for f, t in (("stride_qt", qt), ("stride_kt", kt), ("stride_qs", qs), ("stride_ks", ks)):
        getattr(p, f)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    if packed:
        p.B = cu_seqlens_q.numel() - 1
        p.cu_seqlens_q, p.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
        if validate:
            # one read-back of both offset vectors (a synchronisation); the kernels themselves clamp
            # every offset into the packed axis, so unchecked offsets cannot reach outside the buffers
            lq, lk = _segment_lengths(cu_seqlens_q, Nq, "cu_seqlens_q"), _segment_lengths(cu_seqlens_k, Nk, "cu_seqlens_k")
            for i, (nq, nk) in enumerate(zip(lq, lk)):
                if nq > 0 and (nk == 0 or (causal and nk < nq)):
                    raise ValueError(f"segment {i} has {nq} query rows and {nk} keys: "
                                     + ("causal needs at least as many keys as queries" if nk else "rows without keys"))
            for name, m, lens in (("max_seqlen_q", max_seqlen_q, lq), ("max_seqlen_k", max_seqlen_k, lk)):
                if m is not None and lens and max(lens) > int(m):
                    raise ValueError(f"{name} = {int(m)} is below the longest segment ({max(lens)})")
            p.max_seqlen_q = (max(lq) if lq else 0) if max_seqlen_q is None else int(max_seqlen_q)
            p.max_seqlen_k = (max(lk) if lk else 0) if max_seqlen_k is None else int(max_seqlen_k)
        else:
            if max_seqlen_q is None or max_seqlen_k is None:
                raise ValueError("validate=False needs max_seqlen_q and max_seqlen_k")
            p.max_seqlen_q, p.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    return p


def _segment_lengths(cu, n: int, name: str) -> list:
    """Segment lengths of a packed axis of n rows from its offsets (read back to the host): the offsets
    must start at 0 or above, never decrease and end at n or below."""
    c = [int(v) for v in cu.cpu().tolist()]
    if c and c[0] < 0:
        raise ValueError(f"{name}[0] = {c[0]} is negative")
    for i in range(len(c) - 1):
        if c[i + 1] < c[i]:
            raise ValueError(f"{name} decreases at entry {i + 1} ({c[i]} -> {c[i + 1]})")
    if c and c[-1] > n:
        raise ValueError(f"{name}[-1] = {c[-1]} is past the {n} packed rows")
    return [c[i + 1] - c[i] for i in range(len(c) - 1)]


_PACKED_DOC = """Packed variable-length batch: cu_seqlens_q, cu_seqlens_k (and optionally max_seqlen_q,
    max_seqlen_k, validate) as in make_problem; outputs then take the C ABI's packed layout: statistics
    [H, Nq], dQ [H, Nq, d], dK [Hk, Nk, d]."""


def fwd(qt, kt, qs, ks, *, causal: bool, scale_t=None, scale_s=None, out=None, stream=None, cu_seqlens_q=None,
        cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, validate=True, split=True
        ) -> Tuple["torch.Tensor", "torch.Tensor", "torch.Tensor"]:
    """Per-row KL(P_t || P_s), LSE_t, LSE_s as float32 [B, H, Nq] (streamkl_fwd).  A small causal
    problem gets the workspace that lets the library split its long query blocks' keys over two
    workgroups (results within float rounding of the unsplit forward); split=False passes none, so
    every query block is one workgroup, the arrangement a packed batch takes."""
    import torch
    p = make_problem(qt, kt, qs, ks, causal, scale_t, scale_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, validate)
    if out is None:
        out = tuple(torch.empty(p.stat_shape(), dtype=torch.float32, device=qt.device) for _ in range(3))
    kl, lse_t, lse_s = out
    ws = attach_workspace(p, qt.device, stream) if split else None  # noqa: F841 (alive through the call)
    _check(lib().streamkl_fwd(ctypes.byref(p), _ptr(qt), _ptr(kt), _ptr(qs), _ptr(ks), _ptr(kl), _ptr(lse_t),
                              _ptr(lse_s), _stream(stream)), "streamkl_fwd")
    return kl, lse_t, lse_s


def bwd(qt, kt, qs, ks, lse_t, lse_s, g, *, causal: bool, kl=None, teacher_grads: bool = False,
        student_grads: bool = True, scale_t=None, scale_s=None, out=None, stream=None, cu_seqlens_q=None,
        cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, validate=True):
    """Gradients of sum_i g_i KL_i (streamkl_bwd): (dq_s, dk_s, dq_t, dk_t), the pairs not asked for
    returned as None (student pair by default, teacher pair with teacher_grads=True)."""
    import torch
    p = make_problem(qt, kt, qs, ks, causal, scale_t, scale_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, validate)
    dev = qt.device
    if out is None:
        out = [None, None, None, None]
        if student_grads:
            out[0] = torch.empty(p.dq_shape(p.d_s), dtype=torch.float32, device=dev)
            out[1] = torch.empty(p.dk_shape(p.Hk_s, p.d_s), dtype=torch.float32, device=dev)
        if teacher_grads:
            out[2] = torch.empty(p.dq_shape(p.d_t), dtype=torch.float32, device=dev)
            out[3] = torch.empty(p.dk_shape(p.Hk_t, p.d_t), dtype=torch.float32, device=dev)
    out = list(out) + [None] * (4 - len(out))
    dq_s, dk_s = (out[0], out[1]) if student_grads else (None, None)
    dq_t, dk_t = (out[2], out[3]) if teacher_grads else (None, None)
    ws = attach_workspace(p, qt.device, stream)  # noqa: F841 (kept alive through the call)
    _check(lib().streamkl_bwd(ctypes.byref(p), _ptr(qt), _ptr(kt), _ptr(qs), _ptr(ks), _ptr(lse_t), _ptr(lse_s),
                              _ptr(kl), _ptr(g), _ptr(dq_s), _ptr(dk_s), _ptr(dq_t), _ptr(dk_t), _stream(stream)),
           "streamkl_bwd")
    return dq_s, dk_s, dq_t, dk_t


def bwd_noalloc(qt, kt, qs, ks, lse_t, lse_s, g, *, causal: bool, out, kl=None, scale_t=None, scale_s=None,
                stream=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, validate=True):
    """streamkl_bwd_noalloc: bwd's gradients into the caller's `out` = [dq_s, dk_s, dq_t, dk_t] (a pair
    None = not computed), with the grouped-key workspace taken from the library's static per-GPU
    scratch instead of an allocation.  Nothing here or in the library allocates device memory."""
    p = make_problem(qt, kt, qs, ks, causal, scale_t, scale_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, validate)
    out = list(out) + [None] * (4 - len(out))
    _check(lib().streamkl_bwd_noalloc(ctypes.byref(p), _ptr(qt), _ptr(kt), _ptr(qs), _ptr(ks), _ptr(lse_t),
                                      _ptr(lse_s), _ptr(kl), _ptr(g), *(_ptr(x) for x in out), _stream(stream)),
           "streamkl_bwd_noalloc")
    return tuple(out)


def bwd_dq(qt, kt, qs, ks, lse_t, lse_s, g, *, causal: bool, scale_t=None, scale_s=None, out=None, stream=None,
           cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, validate=True):
    """Student dQ only: the query-owner half of the backward (streamkl_bwd_dq)."""
    import torch
    p = make_problem(qt, kt, qs, ks, causal, scale_t, scale_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, validate)
    if out is None:
        out = torch.empty(p.dq_shape(p.d_s), dtype=torch.float32, device=qt.device)
    _check(lib().streamkl_bwd_dq(ctypes.byref(p), _ptr(qt), _ptr(kt), _ptr(qs), _ptr(ks), _ptr(lse_t), _ptr(lse_s),
                                 _ptr(g), _ptr(out), _stream(stream)), "streamkl_bwd_dq")
    return out


def bwd_dk(qt, kt, qs, ks, lse_t, lse_s, g, *, causal: bool, scale_t=None, scale_s=None, out=None, stream=None,
           cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, validate=True):
    """Student dK only: the key-owner half of the backward (streamkl_bwd_dk)."""
    import torch
    p = make_problem(qt, kt, qs, ks, causal, scale_t, scale_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, validate)
    if out is None:
        out = torch.empty(p.dk_shape(p.Hk_s, p.d_s), dtype=torch.float32, device=qt.device)
    ws = attach_workspace(p, qt.device, stream)  # noqa: F841 (kept alive through the call)
    _check(lib().streamkl_bwd_dk(ctypes.byref(p), _ptr(qt), _ptr(kt), _ptr(qs), _ptr(ks), _ptr(lse_t), _ptr(lse_s),
                                 _ptr(g), _ptr(out), _stream(stream)), "streamkl_bwd_dk")
    return out


def js_fwd(qt, kt, qs, ks, *, causal: bool, scale_t=None, scale_s=None, out=None, stream=None, cu_seqlens_q=None,
           cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, validate=True):
    """Per-row Jensen-Shannon divergence (streamkl_js_fwd): (js, lse_t, lse_s, js_t), float32 in the
    layout of fwd's outputs; js_t is the teacher half KL(P_t || M), which js_bwd needs."""
    import torch
    p = make_problem(qt, kt, qs, ks, causal, scale_t, scale_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, validate)
    if out is None:
        out = tuple(torch.empty(p.stat_shape(), dtype=torch.float32, device=qt.device) for _ in range(4))
    js, lse_t, lse_s, js_t = out
    _check(lib().streamkl_js_fwd(ctypes.byref(p), _ptr(qt), _ptr(kt), _ptr(qs), _ptr(ks), _ptr(js), _ptr(lse_t),
                                 _ptr(lse_s), _ptr(js_t), _stream(stream)), "streamkl_js_fwd")
    return js, lse_t, lse_s, js_t


def js_bwd(qt, kt, qs, ks, lse_t, lse_s, js, js_t, g, *, causal: bool, teacher_grads: bool = False,
           student_grads: bool = True, scale_t=None, scale_s=None, out=None, stream=None, cu_seqlens_q=None,
           cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, validate=True):
    """Gradients of sum_i g_i JS_i (streamkl_js_bwd): (dq_s, dk_s, dq_t, dk_t) as bwd returns them."""
    import torch
    p = make_problem(qt, kt, qs, ks, causal, scale_t, scale_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, validate)
    dev = qt.device
    if out is None:
        out = [None, None, None, None]
        if student_grads:
            out[0] = torch.empty(p.dq_shape(p.d_s), dtype=torch.float32, device=dev)
            out[1] = torch.empty(p.dk_shape(p.Hk_s, p.d_s), dtype=torch.float32, device=dev)
        if teacher_grads:
            out[2] = torch.empty(p.dq_shape(p.d_t), dtype=torch.float32, device=dev)
            out[3] = torch.empty(p.dk_shape(p.Hk_t, p.d_t), dtype=torch.float32, device=dev)
    out = list(out) + [None] * (4 - len(out))
    dq_s, dk_s = (out[0], out[1]) if student_grads else (None, None)
    dq_t, dk_t = (out[2], out[3]) if teacher_grads else (None, None)
    ws = attach_workspace(p, qt.device, stream)  # noqa: F841 (kept alive through the call)
    _check(lib().streamkl_js_bwd(ctypes.byref(p), _ptr(qt), _ptr(kt), _ptr(qs), _ptr(ks), _ptr(lse_t), _ptr(lse_s),
                                 _ptr(js), _ptr(js_t), _ptr(g), _ptr(dq_s), _ptr(dk_s), _ptr(dq_t), _ptr(dk_t),
                                 _stream(stream)), "streamkl_js_bwd")
    return dq_s, dk_s, dq_t, dk_t


for _f in (fwd, bwd, bwd_dq, bwd_dk, js_fwd, js_bwd):
    _f.__doc__ += "\n\n    " + _PACKED_DOC

"""The backward of small problems runs its query-owner kernels on a second stream beside the key-owner
kernels (streamkl_bwd).  Checked here: the same bits as with every kernel on the caller's stream
(streamkl_bwd_noalloc never uses the second stream), the ordering against work before and after the
call, and a HIP graph capture of the caller's stream, which must take the kernels of both streams.
The problems have 1100 rows (both streams long enough for the second stream, with a ragged last tile)
in grids of 15 workgroups per kernel (far below the device's compute units)."""
import numpy as np
import pytest
import torch

from attention_kl_amd import streamkl as S
from attention_kl_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _problem(seed, B=1, H=3, N=1100, d=128, causal=True):
    w = wl.custom(B, H, N, N, d, d, causal)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 41])))
    qt, kt, qs, ks = (torch.from_numpy(rng.standard_normal(s).astype(np.float32)).cuda().to(torch.bfloat16)
                      for s in ((B, H, N, d), (B, H, N, d), (B, H, N, d), (B, H, N, d)))
    g = torch.from_numpy(rng.uniform(-1.0, 2.0, (B, H, N)).astype(np.float32)).cuda()
    return w, (qt, kt, qs, ks), g


def _empty_grads(w):
    shp = [(w.B, w.H, w.Nq, w.d_s), (w.B, w.H, w.Nk, w.d_s), (w.B, w.H, w.Nq, w.d_t), (w.B, w.H, w.Nk, w.d_t)]
    return [torch.full(s, float("nan"), dtype=torch.float32, device="cuda") for s in shp]


def _same_bits(a, b):
    return all(torch.equal(x.view(torch.int32), y.view(torch.int32)) for x, y in zip(a, b))


@pytest.mark.parametrize("causal", [True, False])
def test_two_streams_give_the_one_stream_bits(causal):
    print(f"case two streams causal={causal}", flush=True)
    w, x, g = _problem(3 + causal, causal=causal)
    kl, lt, ls = S.fwd(*x, causal=causal)
    a = S.bwd(*x, lt, ls, g, kl=kl, causal=causal, teacher_grads=True, out=_empty_grads(w))
    b = S.bwd_noalloc(*x, lt, ls, g, kl=kl, causal=causal, out=_empty_grads(w))
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(t).all()) for t in a)
    assert _same_bits(a, b)


def test_two_streams_follow_the_callers_stream_order():
    """Inputs written just before the call and outputs read just after it, all on the caller's stream:
    the second stream waits for the writes, the caller's stream for its kernels."""
    print("case stream order", flush=True)
    w, x, g = _problem(5)
    kl, lt, ls = S.fwd(*x, causal=True)
    ref = S.bwd(*x, lt, ls, g, kl=kl, causal=True, teacher_grads=True)
    torch.cuda.synchronize()
    x2 = [t.clone() for t in x]
    for _ in range(3):
        for t in x2:  # overwrite the inputs with garbage, then restore them, both on the caller's stream
            t.fill_(7.0)
        for t, s in zip(x2, x):
            t.copy_(s)
        got = S.bwd(*x2, lt, ls, g, kl=kl, causal=True, teacher_grads=True, out=_empty_grads(w))
        sums = [t.double().sum() for t in got]  # read right after the call, on the caller's stream
        torch.cuda.synchronize()
        assert _same_bits(got, ref)
        assert all(float(s) == float(r.double().sum()) for s, r in zip(sums, ref))


def test_graph_capture_takes_both_streams():
    print("case graph capture", flush=True)
    w, x, g = _problem(6)
    kl, lt, ls = S.fwd(*x, causal=True)
    ref = S.bwd(*x, lt, ls, g, kl=kl, causal=True, teacher_grads=True)  # eager; also makes the second stream
    torch.cuda.synchronize()
    outs = _empty_grads(w)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            S.bwd(*x, lt, ls, g, kl=kl, causal=True, teacher_grads=True, out=outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs:  # eager work between replays, and outputs that only a replay can fill
            t.fill_(float("nan"))
        S.fwd(*x, causal=True, out=(kl, lt, ls))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same_bits(outs, ref), f"replay {r}"


def test_calls_from_two_threads_on_two_streams():
    """Two host threads, each on its own stream, calling the backward at once: they share the device's
    second stream and its events under the library's lock, and each gets the bits of a lone call."""
    import threading
    print("case two threads", flush=True)
    probs = [_problem(20 + k) for k in range(2)]
    refs, fwds = [], []
    for w, x, g in probs:
        kl, lt, ls = S.fwd(*x, causal=True)
        fwds.append((kl, lt, ls))
        refs.append(S.bwd(*x, lt, ls, g, kl=kl, causal=True, teacher_grads=True))
    torch.cuda.synchronize()
    results = [[None] * 6 for _ in probs]
    errors = []

    def worker(k):
        try:
            w, x, g = probs[k]
            kl, lt, ls = fwds[k]
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                for r in range(6):
                    results[k][r] = S.bwd(*x, lt, ls, g, kl=kl, causal=True, teacher_grads=True, out=_empty_grads(w))
            st.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        for r in range(6):
            assert _same_bits(results[k][r], refs[k]), f"thread {k} call {r}"

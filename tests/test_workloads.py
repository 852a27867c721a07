"""The seeded input generators: rounding, determinism, per-head regeneration, config shapes."""
import numpy as np
import torch

from attention_kl_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    mine = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    back = wl.bf16_bits_to_f32(mine)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_heads_regenerate_independently():
    w = wl.custom(2, 3, 40, 48, 64, 64, True, seed=7)
    full = wl.full_f32(w)
    for b in range(2):
        for h in range(3):
            one = wl.head_f32(w, b, h)
            for a, f in zip(one, full):
                np.testing.assert_array_equal(a, f[b, h])
    assert not np.array_equal(full[0][0, 0], full[0][0, 1])


def test_recipes():
    w = wl.WORKLOADS[2]
    qt, kt, qs, ks = wl.head_f32(wl.custom(1, 1, 64, 64, 128, 128, True, recipe="noise", sigma=0.1, seed=2), 0, 0)
    assert 0.05 < np.std(qs - qt) < 0.15  # student = teacher + 0.1 N(0,1), bf16-rounded
    bits = wl.f32_to_bf16_bits(qt)
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(bits), qt)  # already bf16 values
    pk = wl.Workload("p", 1, 1, 16, 1000, 8, 8, True, "fp32", "independent", peak_frac=0.01, peak_scale=4.0, seed=3)
    kt_p = wl.head_f32(pk, 0, 0)[1]
    kt_0 = wl.head_f32(wl.Workload("p", 1, 1, 16, 1000, 8, 8, True, "fp32", "independent", seed=3), 0, 0)[1]
    ratio = np.abs(kt_p).sum(1) / np.abs(kt_0).sum(1)
    assert np.sum(np.isclose(ratio, 4.0)) == 10 and np.sum(np.isclose(ratio, 1.0)) == 990
    assert w.B * w.H * w.Nq == 65536


def test_workload_flops():
    c3 = wl.WORKLOADS[3]
    assert c3.pairs_per_head() == 32768 * 32769 // 2
    assert abs(c3.fwd_flops() - 8.796e12) / 8.796e12 < 1e-3
    assert wl.WORKLOADS[4].pairs_per_head() == 8192 * 8192
    g = wl.head_g(c3, 0, 5)
    assert g.shape == (32768,) and g.min() >= 0.5 and g.max() <= 1.5


def _bench_module():
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    return bench


def test_bench_kernel_classes_follow_the_owner_argument():
    """Profiler rows are attributed by the OWN_Q template argument, in demangled and mangled names."""
    k = _bench_module()._kernel_class
    assert k("void skl::fwd_kernel<__bf16, 128, 128, true>(skl::FwdArgs)") == "fwd"
    assert k("void skl::bwd_kernel<__bf16, 128, 128, true, false, true, false>(skl::BwdArgs)") == "bwd_dq"
    assert k("void skl::bwd_kernel<__bf16, 128, 128, true, false, false, false>(skl::BwdArgs)") == "bwd_dk"
    assert k("void skl::bwd_kernel<__bf16, 128, 128, true, true, false, true>(skl::BwdArgs)") == "bwd_dk"
    assert k("_ZN3skl10bwd_kernelIDF16bLi128ELi128ELb1ELb0ELb1ELb0EEEvNS_7BwdArgsE") == "bwd_dq"
    assert k("_ZN3skl10bwd_kernelIDF16bLi128ELi128ELb1ELb0ELb0ELb1EEEvNS_7BwdArgsE") == "bwd_dk"
    assert k("void at::native::copy_kernel") == "copy" and k("other") is None


def test_pair_counts_match_a_brute_force_mask():
    """Allowed pairs (the unit of every flop count) against the mask counted element by element:
    bottom-right causal alignment with more keys than queries, equal lengths, and non-causal."""
    for nq, nk, causal in [(5, 5, True), (3, 7, True), (64, 100, True), (33, 33, False), (1, 9, True)]:
        w = wl.custom(1, 1, nq, nk, 64, 64, causal)
        i = np.arange(nq)[:, None]
        j = np.arange(nk)[None, :]
        allowed = (j <= i + nk - nq) if causal else np.ones((nq, nk), bool)
        assert w.pairs_per_head() == int(allowed.sum()), (nq, nk, causal)


def test_step_flops_count_each_product_once():
    """Forward 2 (d_t + d_s) and backward 2 (d_t + 3 d_s) per allowed pair; JS doubles the forward;
    teacher gradients add 4 d_t."""
    bench = _bench_module()
    w = wl.custom(2, 3, 40, 56, 128, 64, True)
    P = w.pairs_per_head() * 2 * 3
    f, b = bench.step_flops(w)
    assert f == 2.0 * P * (128 + 64) and b == 2.0 * P * (128 + 3 * 64)
    fj, _ = bench.step_flops(w, js=True)
    _, bt = bench.step_flops(w, teacher=True)
    assert fj == 2 * f and bt == b + 4.0 * P * 128


def test_counter_ingest_keeps_the_workload_launches(tmp_path):
    """FETCH_SIZE rows are summed per dispatch and averaged over each kernel's dispatches at its largest
    grid (the workload's own launches); the bench's small warm-up launches and other kernels drop out."""
    bench = _bench_module()
    fwd = "_ZN3skl10fwd_kernelIDF16bLi128ELi128ELb1ELb0ELb1EEEvNS_7FwdArgsE"
    dq = "_ZN3skl10bwd_kernelIDF16bLi128ELi128ELb1ELb0ELb1ELb0ELb0EEEvNS_7BwdArgsE"
    rows = [  # dispatch, kernel, grid, counter, value (two per-XCD rows for some dispatches)
        (1, fwd, 256, "FETCH_SIZE", 5.0), (2, fwd, 4096, "FETCH_SIZE", 100.0), (2, fwd, 4096, "FETCH_SIZE", 20.0),
        (3, fwd, 4096, "FETCH_SIZE", 140.0), (3, fwd, 4096, "WRITE_SIZE", 9.0), (4, dq, 512, "FETCH_SIZE", 1.0),
        (5, dq, 8192, "FETCH_SIZE", 70.0), (6, "void at::native::copy_kernel", 99, "FETCH_SIZE", 8.0),
        (7, "other_kernel", 4096, "FETCH_SIZE", 1e9)]
    p = tmp_path / "c.csv"
    with open(p, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
        for d, k, g, c, v in rows:
            f.write(f'{d},"{k}",{g},{c},{v}\n')
    m = bench._pmc_means(str(p), "FETCH_SIZE")
    assert m == {"fwd": 130.0, "bwd_dq": 70.0, "copy": 8.0}

"""GPU parity of the calibration path: stats-only pass (critical values) -> quantile inversion ->
least-squares fit of lambda * L = alpha * exp(beta * s), against the oracle's own calibration."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import host64

pytestmark = pytest.mark.gpu

L_VALUES = (1024, 2048, 4096)
S_VALUES = (0.3, 0.5, 0.7)
SAMPLE = [(0, 1), (1, 3), (2, 5), (3, 7)]   # (q head, q tile) of the calibration sample


def _stats(m, inp, L):
    nqt = L // 128
    crit = torch.full((1, 4, nqt, nqt), 123.0, dtype=torch.float32, device="cuda")
    m.blasst_prefill(inp.q, inp.k, inp.v, None, causal=True, block_q=128, block_k=128, lam=0.0, crit=crit,
                     stats_only=True)
    torch.cuda.synchronize()
    return crit.cpu().numpy()


def _lib():
    import long_context_online_amd as m
    m.lib()
    return m


def test_calibration_matches_oracle():
    m = _lib()
    gpu_pts, ref_pts = [], []
    for i, L in enumerate(L_VALUES):
        inp = synth.prefill_inputs(batch=1, hq=4, hkv=1, L=L, d=128, block_k=128, window=True,
                                   seed=synth.config_seed(4, 10 + i), device="cuda")
        crit = _stats(m, inp, L)
        q, k, v = host64(inp.q), host64(inp.k), host64(inp.v)
        gpu_sample, ref_sample = [], []
        for (h, t) in SAMPLE:
            ref = oracle.prefill_tile(q, k, v, 0, h, t, causal=True, block_q=128, block_k=128, num_splits=1,
                                      ln_lam=-math.inf)
            live = ref["mask"] != oracle.NOT_LIVE
            g = crit[0, h, t]
            assert np.array_equal(np.isnan(g), ~live)
            fin = np.isfinite(ref["crit"]) & live
            assert np.all(np.abs(g[fin] - ref["crit"][fin]) < 2e-3)
            gpu_sample.append(g[live])
            ref_sample.append(ref["crit"][live])
        gs, rs = np.concatenate(gpu_sample), np.concatenate(ref_sample)
        for s in S_VALUES:
            ln_g = m.blasst_calib_quantile(gs.astype(np.float32), s)
            ln_r = oracle.quantile_ln_lambda(rs, s)
            # the library's threshold splits the oracle's critical values at the target within one
            # value (plus values within rounding distance of it)
            near = np.count_nonzero(np.abs(rs - ln_g) < 2e-3)
            got = oracle.achieved_sparsity(rs, ln_g)
            assert abs(got - oracle.achieved_sparsity(rs, ln_r)) <= (1 + near) / rs.size + 1e-12
            gpu_pts.append((L, s, math.exp(ln_g)))
            ref_pts.append((L, s, math.exp(ln_r)))
    ga, gb, gr = m.blasst_calibrate(*(np.array([p[j] for p in gpu_pts]) for j in range(3)))
    ra, rb, rr = oracle.fit_alpha_beta(*(np.array([p[j] for p in ref_pts]) for j in range(3)))
    print(f"gpu fit alpha={ga:.5g} beta={gb:.5g} rmse={gr:.4g}; oracle fit alpha={ra:.5g} beta={rb:.5g} rmse={rr:.4g}")
    assert abs(math.log(ga) - math.log(ra)) < 0.05 and abs(gb - rb) < 0.1


# ------------------------------------------------------------------------------------------------
# the calibration sweep and the long prefill at their own sizes (32 q / 8 kv heads, d = 128)
# ------------------------------------------------------------------------------------------------

SWEEP_L = (4096, 8192, 16384, 32768, 65536, 131072)


def _sweep_inputs(L):
    """The benchmark's calibration-sweep inputs at length L (seed 1000 * 4 + index of L)."""
    return synth.prefill_inputs(batch=1, hq=32, hkv=8, L=L, d=128, block_k=128, window=True,
                                seed=synth.config_seed(4, SWEEP_L.index(L)), device="cuda")


def _stats_pass(m, inp):
    L = inp.q.shape[2]
    nqt = L // 128
    crit = torch.full((1, 32, nqt, nqt), 123.0, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    m.blasst_prefill(inp.q, inp.k, inp.v, None, causal=True, block_q=128, block_k=128, lam=0.0, crit=crit,
                     counters=cnt, stats_only=True)
    torch.cuda.synchronize()
    assert int(cnt[0]) == 32 * nqt * (nqt + 1) // 2 and int(cnt[1]) == 0
    return crit


def _oracle_crit(inp, h, t):
    """The oracle's critical values of tile (head h, query tile t), from host copies of that head and
    of its kv head."""
    q = host64(inp.q[:, h:h + 1])
    k = host64(inp.k[:, h // 4:h // 4 + 1])
    v = host64(inp.v[:, h // 4:h // 4 + 1])
    ref = oracle.prefill_tile(q, k, v, 0, 0, t, causal=True, block_q=128, block_k=128, num_splits=1,
                              ln_lam=-math.inf)
    return ref


def _sample(nqt):
    import bench
    return bench.stratified_tiles(torch, nqt, 32, bench.CALIB_TILES, 4242)


@pytest.mark.parametrize("L", SWEEP_L[1:])
def test_stats_pass_full_size(L):
    """The calibration pass at the sweep's sizes (L = 8K ... 128K, 32 q / 8 kv heads): the critical
    values of the benchmark's 8 calibration tiles and of 12 more seeded tiles (last, middle and first
    causal levels among them) against the oracle, and the library's quantile of the sample against the
    oracle's at s = 0.3, 0.5, 0.7 and 0.75."""
    m = _lib()
    inp = _sweep_inputs(L)
    crit = _stats_pass(m, inp)
    nqt = L // 128
    rng = np.random.default_rng(L)
    extra = [(0, nqt - 1), (31, nqt // 2), (17, 0)] + [(int(h), int(t)) for h, t in
                                                         zip(rng.integers(0, 32, 9), rng.integers(0, nqt, 9))]
    sample = _sample(nqt)
    worst = 0.0
    gpu_s, ref_s = [], []
    for i, (h, t) in enumerate(sample + extra):
        ref = _oracle_crit(inp, h, t)
        g = crit[0, h, t].cpu().numpy()
        live = ref["mask"] != oracle.NOT_LIVE
        assert np.array_equal(np.isnan(g), ~live), (h, t)
        assert np.array_equal(np.isinf(g[live]), np.isinf(ref["crit"][live])), (h, t)
        fin = live & np.isfinite(ref["crit"])
        err = float(np.max(np.abs(g[fin] - ref["crit"][fin]))) if fin.any() else 0.0
        assert err < 2e-3, (h, t, err)
        worst = max(worst, err)
        if i < len(sample):
            gpu_s.append(g[live])
            ref_s.append(ref["crit"][live])
    gs, rs = np.concatenate(gpu_s), np.concatenate(ref_s)
    for s in (0.3, 0.5, 0.7, 0.75):
        ln_g = m.blasst_calib_quantile(gs.astype(np.float32), s)
        ln_r = oracle.quantile_ln_lambda(rs, s)
        near = np.count_nonzero(np.abs(rs - ln_g) < 2e-3)
        got = oracle.achieved_sparsity(rs, ln_g)
        assert abs(got - oracle.achieved_sparsity(rs, ln_r)) <= (1 + near) / rs.size + 1e-12, (s, ln_g, ln_r)
    print(f"L={L}: {len(sample) + len(extra)} tiles, max crit error {worst:.3g}")


def test_calibration_fit_and_long_prefill_full_size():
    """The whole calibration of the sweep (L = 4K ... 128K, s = 0.3 / 0.5 / 0.7, the benchmark's
    8-tile sample per L): the GPU stats passes and the library's quantile and fit against the oracle's
    quantile and fit over the oracle's critical values of the same sample; then the L = 131072 prefill
    at the fitted lambda for s = 0.75 with sampled tiles against the oracle."""
    m = _lib()
    gpu_pts, ref_pts = [], []
    for L in SWEEP_L:
        inp = _sweep_inputs(L)
        crit = _stats_pass(m, inp)
        gpu_s, ref_s = [], []
        for h, t in _sample(L // 128):
            ref = _oracle_crit(inp, h, t)
            live = ref["mask"] != oracle.NOT_LIVE
            gpu_s.append(crit[0, h, t].cpu().numpy()[live])
            ref_s.append(ref["crit"][live])
        gs, rs = np.concatenate(gpu_s), np.concatenate(ref_s)
        for s in (0.3, 0.5, 0.7):
            gpu_pts.append((L, s, math.exp(m.blasst_calib_quantile(gs.astype(np.float32), s))))
            ref_pts.append((L, s, math.exp(oracle.quantile_ln_lambda(rs, s))))
        del inp, crit
        torch.cuda.empty_cache()
    ga, gb, gr = m.blasst_calibrate(*(np.array([p[j] for p in gpu_pts]) for j in range(3)))
    ra, rb, rr = oracle.fit_alpha_beta(*(np.array([p[j] for p in ref_pts]) for j in range(3)))
    print(f"gpu fit alpha={ga:.5g} beta={gb:.5g} rmse={gr:.4g}; oracle fit alpha={ra:.5g} beta={rb:.5g} rmse={rr:.4g}")
    assert abs(math.log(ga) - math.log(ra)) < 0.05 and abs(gb - rb) < 0.1
    from tests.test_gpu_prefill import check_full_size_prefill
    lam = m.blasst_lambda_for(ga, gb, 0.75, 131072)
    assert lam == pytest.approx(oracle.lambda_for(ga, gb, 0.75, 131072), rel=1e-12)
    sp, n, rep = check_full_size_prefill(m, _sweep_inputs(131072), lam, None, seed=75, count=10)
    print(f"L=131072 at the fitted lambda {lam:.6g}: sparsity {sp:.4f}; {n} tiles vs oracle: {rep}")


def test_long_prefill_131072_at_sample_calibrated_lambda():
    """The long prefill the benchmark times at L = 131072 (32 q / 8 kv heads, bf16 in/out) at the
    lambda calibrated for 75 % from its 8-tile sample: 26 tiles against the oracle (the last, a middle
    and the first causal level among them), every tile's mask against its critical values."""
    m = _lib()
    from tests.test_gpu_prefill import benchmark_lambda, check_full_size_prefill
    inp = _sweep_inputs(131072)
    lam = benchmark_lambda(m, inp, 0.75)
    sp, n, rep = check_full_size_prefill(m, inp, lam, 0.75, seed=131, count=20)
    print(f"lambda={lam:.6g} sparsity {sp:.4f}; {n} tiles vs oracle: {rep}")

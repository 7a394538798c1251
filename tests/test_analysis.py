"""Per-head sparsity summaries (host logic) and, on the oracle, the spread of per-head sparsity under
one threshold when heads differ in how peaked their attention is."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from long_context_online_amd import analysis


def test_head_sparsity_summary():
    h = np.array([[[10, 5], [10, 0], [4, 4], [0, 0]]], dtype=np.int64)
    sp = analysis.head_sparsity(h)
    assert sp.shape == (1, 4) and np.isnan(sp[0, 3])
    assert np.array_equal(sp[0, :3], [0.5, 0.0, 1.0])
    st = analysis.head_sparsity_stats(torch.tensor(h))
    assert st["heads"] == 3 and st["min"] == 0.0 and st["max"] == 1.0 and st["median"] == 0.5
    assert st["p25"] == 0.25 and st["p75"] == 0.75 and abs(st["overall"] - 9 / 24) < 1e-15
    assert abs(st["std"] - math.sqrt(1 / 6)) < 1e-12
    with pytest.raises(ValueError):
        analysis.head_sparsity(np.array([[3, 4]]))
    with pytest.raises(ValueError):
        analysis.head_sparsity_stats(np.zeros((2, 2), dtype=np.int64))


def test_oracle_per_head_sparsity_spreads_under_one_threshold():
    """Weakly peaked heads (strength 0.25-0.5) keep every block at lambda = 0.01; strongly peaked ones
    (>= 1) skip about half; heads on one kv head saturate at the same sparsity once every block
    without a boosted key is skipped."""
    strength = [0.25, 1.75, 0.5, 1.5, 0.75, 1.25, 1.0, 0.35]
    inp = synth.prefill_inputs(batch=1, hq=8, hkv=2, L=768, d=128, block_k=128, window=True, seed=31,
                               head_strength=strength)
    q, k, v = (t.double().numpy() for t in (inp.q, inp.k, inp.v))
    counts = np.zeros((1, 8, 2), dtype=np.int64)
    for h in range(8):
        for t in range(6):
            r = oracle.prefill_tile(q, k, v, 0, h, t, causal=True, block_q=128, block_k=128, num_splits=1,
                                    ln_lam=math.log(0.01))
            counts[0, h] += [(r["mask"] != oracle.NOT_LIVE).sum(), (r["mask"] == oracle.SKIPPED).sum()]
    sp = dict(zip(strength, analysis.head_sparsity(counts)[0]))
    assert sp[0.25] == sp[0.35] == sp[0.5] == 0.0
    assert all(sp[c] > 0.4 for c in (1.0, 1.25, 1.5, 1.75))
    assert 0.0 < sp[0.75] < sp[1.0]
    st = analysis.head_sparsity_stats(counts)
    assert st["std"] > 0.25

"""Pins for the backward oracle (fp64): central differences of the block-sequential forward oracle
with its decisions held fixed, the textbook dense-attention gradient at lambda = 0, and invariants
of the softmax Jacobian."""

import math

import numpy as np
import pytest

import oracle
from oracle import KEPT, SKIPPED, NOT_LIVE
from oracle import backward as bw


def _problem(rng, B=1, Hq=2, Hkv=1, Lq=10, Lk=12, D=4, Dv=3):
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, Lk, D))
    k[:, :, 0] *= 3.0
    v = rng.standard_normal((B, Hkv, Lk, Dv))
    do = rng.standard_normal((B, Hq, Lq, Dv))
    return q, k, v, do


def _forward_fixed(q, k, v, mask, causal, bq, bk, scale):
    """O of the numpy block-sequential oracle, every live block's decision forced to the mask's."""
    B, Hq, Lq, _ = q.shape
    O = np.zeros((B, Hq, Lq, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            for t in range(mask.shape[2]):
                force = {j: int(mask[b, h, t, j]) for j in range(mask.shape[3]) if mask[b, h, t, j] != NOT_LIVE}
                r = oracle.prefill_tile(q, k, v, b, h, t, causal=causal, block_q=bq, block_k=bk, num_splits=1,
                                        ln_lam=-math.inf, scale=scale, force=force)
                O[b, h, t * bq:(t + 1) * bq] = r["o"]
    return O


@pytest.mark.parametrize("causal,lam", [(True, 0.3), (True, 0.6), (False, 0.5)])
def test_gradients_match_central_differences_of_the_forward_oracle(causal, lam):
    rng = np.random.default_rng(1 + int(lam * 10))
    q, k, v, do = _problem(rng)
    bq = bk = 4
    scale = 0.7
    mask = oracle.prefill(q, k, v, causal=causal, block_q=bq, block_k=bk, lam=lam, scale=scale)["mask"]
    assert (mask == SKIPPED).any()
    g = bw.prefill_backward(q, k, v, do, mask, causal=causal, block_q=bq, block_k=bk, scale=scale)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = np.sum(do * _forward_fixed(q, k, v, mask, causal, bq, bk, scale))
            x[idx] = old - h
            fm = np.sum(do * _forward_fixed(q, k, v, mask, causal, bq, bk, scale))
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - g[name])) < 1e-7, name


def test_lambda_zero_is_the_textbook_attention_gradient():
    """All blocks kept: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)), dQ = scale dS K,
    dK = scale dS^T Q (per head, GQA heads summed), written out in numpy."""
    rng = np.random.default_rng(5)
    q, k, v, do = _problem(rng, B=2, Hq=4, Hkv=2, Lq=9, Lk=14, D=5, Dv=4)
    scale = 0.45
    mask = oracle.prefill(q, k, v, causal=True, block_q=3, block_k=5, lam=0.0, scale=scale)["mask"]
    assert not (mask == SKIPPED).any()
    g = bw.prefill_backward(q, k, v, do, mask, causal=True, block_q=3, block_k=5, scale=scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    Lq, Lk = 9, 14
    vis = np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq)
    for b in range(2):
        for hh in range(4):
            kv = hh // 2
            s = np.where(vis, scale * q[b, hh] @ k[b, kv].T, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, kv]
            dp = do[b, hh] @ v[b, kv].T
            ds = p * (dp - np.sum(do[b, hh] * o, axis=1, keepdims=True))
            dq[b, hh] = scale * ds @ k[b, kv]
            dk[b, kv] += scale * ds.T @ q[b, hh]
            dv[b, kv] += p.T @ do[b, hh]
    for name, want in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.max(np.abs(g[name] - want)) < 1e-12, name


def test_softmax_jacobian_invariants_and_skipped_blocks_get_nothing():
    """Each row's dS sums to zero over its kept keys, so dK sums to zero over the keys of each kv head;
    dV sums to the sum of dO over rows that see a kept key; a key block that no tile keeps has
    dK = dV = 0, and changing its keys or values leaves O unchanged."""
    rng = np.random.default_rng(9)
    q, k, v, do = _problem(rng, B=1, Hq=2, Hkv=1, Lq=8, Lk=16, D=4, Dv=3)
    bq = bk = 4
    scale = 0.8
    q = np.abs(q)
    k[:, :, 0] = 5.0            # a dominant first key every row sees ...
    k[:, :, 12:16] = 0.0        # ... and a flat last block every tile skips (logit 0, 12+ below the max)
    for causal in (True, False):
        mask = oracle.prefill(q, k, v, causal=causal, block_q=bq, block_k=bk, lam=0.5, scale=scale)["mask"]
        g = bw.prefill_backward(q, k, v, do, mask, causal=causal, block_q=bq, block_k=bk, scale=scale)
        assert np.max(np.abs(g["dk"].sum(axis=2))) < 1e-12
        keep = bw.kept_keys(mask, 8, 16, bq, bk, causal)
        has = keep.any(axis=-1)
        assert np.max(np.abs(g["dv"].sum(axis=2)[0, 0] - (do * has[..., None]).sum(axis=(1, 2))[0])) < 1e-12
        dead = [j for j in range(4) if not (mask[0, :, :, j] == KEPT).any()]
        assert 3 in dead, mask
        for j in dead:
            assert np.all(g["dk"][0, 0, j * bk:(j + 1) * bk] == 0) and np.all(g["dv"][0, 0, j * bk:(j + 1) * bk] == 0)
            k2, v2 = k.copy(), v.copy()
            k2[0, 0, j * bk:(j + 1) * bk] += 1.0
            v2[0, 0, j * bk:(j + 1) * bk] -= 2.0
            o2 = bw.prefill_backward(q, k2, v2, do, mask, causal=causal, block_q=bq, block_k=bk, scale=scale)["o"]
            assert np.max(np.abs(o2 - g["o"])) < 1e-14


def test_gqa_gradient_is_mha_with_repeated_kv_summed():
    rng = np.random.default_rng(13)
    q, k, v, do = _problem(rng, B=1, Hq=4, Hkv=2, Lq=12, Lk=12, D=4, Dv=3)
    mask = oracle.prefill(q, k, v, causal=True, block_q=4, block_k=4, lam=0.4, scale=0.6)["mask"]
    g = bw.prefill_backward(q, k, v, do, mask, causal=True, block_q=4, block_k=4, scale=0.6)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    m = bw.prefill_backward(q, kr, vr, do, mask, causal=True, block_q=4, block_k=4, scale=0.6)
    assert np.max(np.abs(g["dq"] - m["dq"])) < 1e-13
    assert np.max(np.abs(g["dk"] - m["dk"].reshape(1, 2, 2, 12, 4).sum(axis=2))) < 1e-13
    assert np.max(np.abs(g["dv"] - m["dv"].reshape(1, 2, 2, 12, 3).sum(axis=2))) < 1e-13


def test_dq_rows_is_the_full_backward_restricted_to_those_rows():
    rng = np.random.default_rng(17)
    q, k, v, do = _problem(rng, B=2, Hq=4, Hkv=2, Lq=20, Lk=24, D=4, Dv=3)
    mask = oracle.prefill(q, k, v, causal=True, block_q=4, block_k=8, lam=0.4, scale=0.6)["mask"]
    g = bw.prefill_backward(q, k, v, do, mask, causal=True, block_q=4, block_k=8, scale=0.6)
    rows = np.array([0, 3, 7, 19, 12])
    for b, h in ((0, 1), (1, 3)):
        got = bw.dq_rows(q, k, v, do, mask, b, h, rows, causal=True, block_q=4, block_k=8, scale=0.6)
        assert np.max(np.abs(got - g["dq"][b, h, rows])) < 1e-13

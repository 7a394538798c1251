"""Pins for the fp64 oracle: each check compares it with something other than itself."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax, logsumexp

import oracle
from oracle import KEPT, SKIPPED, NOT_LIVE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _num(x):
    if isinstance(x, str):
        return eval(x, {"__builtins__": {}}, {"exp": math.exp, "log": math.log, "inf": math.inf})
    return float(x)


# ---------------------------------------------------------------------------------------------
# hand examples (golden)
# ---------------------------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_examples(ex):
    q = np.array(ex["q"])
    keys = np.array(ex["keys"])
    vals = np.array(ex["values"])
    vis = np.ones((q.shape[0], keys.shape[0]), dtype=bool)
    ln_lam = _num(ex["ln_lambda"]) if ex["ln_lambda"] != "-inf" else -math.inf
    r = oracle.tile_sequential(q, keys, vals, vis, 1, ex["num_splits"], ln_lam, 1.0)
    assert r["mask"].tolist() == ex["mask"]
    for i, row in enumerate(ex["o"]):
        for c, expr in enumerate(row):
            assert abs(r["o"][i, c] - _num(expr)) < 1e-13
    for i, expr in enumerate(ex["lse"]):
        assert abs(r["lse"][i] - _num(expr)) < 1e-12
    assert abs(oracle.sparsity(r["mask"]) - _num(ex["sparsity"])) < 1e-15
    if "crit" in ex:
        for got, want in zip(r["crit"], ex["crit"]):
            want = _num(want) if want != "inf" else math.inf
            assert got == want


# ---------------------------------------------------------------------------------------------
# random problems
# ---------------------------------------------------------------------------------------------

def _random_prefill(rng, B=1, Hq=4, Hkv=2, Lq=37, Lk=45, D=8, Dv=6, peaky=True):
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, Lk, D))
    v = rng.standard_normal((B, Hkv, Lk, Dv))
    if peaky:
        # make some keys dominant so that skipping happens at moderate thresholds
        k[:, :, 0, :] *= 4.0
        idx = rng.choice(Lk, size=max(1, Lk // 8), replace=False)
        k[:, :, idx, :] *= 2.5
    return q, k, v


def _bruteforce_attention(q, k, v, causal, scale, keep=None):
    """softmax over the visible (and kept) pairs of the full logit matrix, per head."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, Lq, v.shape[3]))
    LSE = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            logits = np.einsum("id,kd->ik", q[b, h], k[b, g]) * scale
            allowed = np.ones((Lq, Lk), dtype=bool)
            if causal:
                for i in range(Lq):
                    for kk in range(Lk):
                        allowed[i, kk] = kk - (Lk - Lq) <= i
            if keep is not None:
                allowed &= keep[b, h]
            for i in range(Lq):
                if not allowed[i].any():
                    continue
                row = np.where(allowed[i], logits[i], -np.inf)
                O[b, h, i] = softmax(row) @ v[b, g]
                LSE[b, h, i] = logsumexp(row)
    return O, LSE


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(37, 45, 8, 16, 1), (64, 64, 16, 16, 3), (20, 50, 7, 9, 2), (45, 37, 8, 8, 1)])
def test_lambda_zero_is_dense_softmax(causal, shape):
    """lambda = 0 never skips, so the result is textbook attention (to 1e-9)."""
    Lq, Lk, bq, bk, S = shape
    rng = np.random.default_rng(Lq * 100 + Lk)
    q, k, v = _random_prefill(rng, Lq=Lq, Lk=Lk)
    scale = 0.37
    r = oracle.prefill(q, k, v, causal=causal, block_q=bq, block_k=bk, num_splits=S, lam=0.0, scale=scale)
    O, LSE = _bruteforce_attention(q, k, v, causal, scale)
    assert np.max(np.abs(r["o"] - O)) < 1e-9
    fin = np.isfinite(LSE)
    assert np.array_equal(fin, np.isfinite(r["lse"]))
    assert np.max(np.abs(r["lse"][fin] - LSE[fin])) < 1e-9
    assert not np.any(r["mask"] == SKIPPED)


def _keep_keys_from_mask(mask, Lq, Lk, bq, bk):
    """Expand a per-(tile, block) mask to a per-(row, key) keep matrix."""
    B, Hq, nqt, nkb = mask.shape
    keep = np.zeros((B, Hq, Lq, Lk), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for t in range(nqt):
                for j in range(nkb):
                    if mask[b, h, t, j] == KEPT:
                        keep[b, h, t * bq:(t + 1) * bq, j * bk:(j + 1) * bk] = True
    return keep


@pytest.mark.parametrize("seed", range(6))
def test_sequential_equals_softmax_over_kept_keys(seed):
    """The block-sequential rule equals exact softmax restricted to the kept blocks (1e-12), and its
    decisions equal the prefix-max closed form."""
    rng = np.random.default_rng(seed)
    Lq, Lk, bq, bk = 33, 41, 8, 5
    S = 1 + seed % 3
    q, k, v = _random_prefill(rng, Lq=Lq, Lk=Lk)
    scale = 0.45
    for ln_lam in [-12.0, -6.0, -3.0, -1.5, -0.5, 0.0]:
        r = oracle.prefill(q, k, v, causal=True, block_q=bq, block_k=bk, num_splits=S,
                           lam=math.exp(ln_lam), scale=scale)
        keep = _keep_keys_from_mask(r["mask"], Lq, Lk, bq, bk)
        O, LSE = _bruteforce_attention(q, k, v, True, scale, keep=keep)
        assert np.max(np.abs(r["o"] - O)) < 1e-12
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                for t in range(r["mask"].shape[2]):
                    rows = np.arange(t * bq, min((t + 1) * bq, Lq))
                    vis = np.arange(Lk)[None, :] <= rows[:, None] + (Lk - Lq)
                    m2, c2 = oracle.keep_mask_closed_form(q[b, h, rows], k[b, h // 2], vis, bk, S,
                                                          ln_lam, scale)
                    assert np.array_equal(m2, r["mask"][b, h, t])
                    live = m2 != NOT_LIVE
                    a, c = c2[live], r["crit"][b, h, t][live]
                    assert np.array_equal(np.isinf(a), np.isinf(c))
                    assert np.allclose(a[np.isfinite(a)], c[np.isfinite(c)], atol=1e-12, rtol=0)


def test_mask_is_crit_below_threshold_and_first_block_kept():
    """skip <=> crit < ln(lambda); the first block of every split is kept (crit = +inf)."""
    rng = np.random.default_rng(7)
    q, k, v = _random_prefill(rng, Lq=40, Lk=40)
    for S in (1, 2, 3):
        for lam in [1e-6, 1e-3, 0.05, 0.3, 1.0]:
            r = oracle.prefill(q, k, v, causal=True, block_q=8, block_k=4, num_splits=S, lam=lam, scale=0.5)
            live = r["mask"] != NOT_LIVE
            assert np.array_equal(r["mask"][live] == SKIPPED, r["crit"][live] < math.log(lam))
            # first block of each split: recompute split starts independently
            B, Hq, nqt, nkb = r["mask"].shape
            for b in range(B):
                for h in range(Hq):
                    for t in range(nqt):
                        J = int(np.count_nonzero(live[b, h, t]))
                        size = -(-J // S)
                        for start in range(0, J, size):
                            assert r["mask"][b, h, t, start] == KEPT
                            assert r["crit"][b, h, t, start] == math.inf


def test_sparsity_monotone_in_lambda():
    rng = np.random.default_rng(11)
    q, k, v = _random_prefill(rng, Lq=48, Lk=48)
    prev = -1.0
    for lam in [0.0, 1e-8, 1e-5, 1e-3, 0.01, 0.05, 0.1, 0.3, 0.6, 1.0]:
        r = oracle.prefill(q, k, v, causal=True, block_q=8, block_k=4, num_splits=2, lam=lam, scale=0.5)
        s = oracle.sparsity(r["mask"])
        assert s >= prev
        prev = s
    assert prev > 0.1


def test_splits_at_least_blocks_is_dense():
    rng = np.random.default_rng(3)
    q, k, v = _random_prefill(rng, Lq=24, Lk=24)
    r = oracle.prefill(q, k, v, causal=True, block_q=8, block_k=4, num_splits=6, lam=1.0, scale=0.5)
    assert not np.any(r["mask"] == SKIPPED)
    O, _ = _bruteforce_attention(q, k, v, True, 0.5)
    assert np.max(np.abs(r["o"] - O)) < 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(5)
    q, k, v = _random_prefill(rng, Hq=6, Hkv=2, Lq=30, Lk=30)
    kw = dict(causal=True, block_q=8, block_k=6, num_splits=1, lam=0.02, scale=0.5)
    r1 = oracle.prefill(q, k, v, **kw)
    r2 = oracle.prefill(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), **kw)
    assert np.array_equal(r1["mask"], r2["mask"])
    assert np.max(np.abs(r1["o"] - r2["o"])) == 0.0


def test_a_over_L_threshold():
    assert oracle.ln_threshold(a=2.0, L=512) == math.log(2.0 / 512)
    assert oracle.ln_threshold(a=0.0, L=512) == -math.inf
    assert oracle.ln_threshold(a=5000.0, L=512) == 0.0          # clamped to lambda = 1
    with pytest.raises(ValueError):
        oracle.ln_threshold(lam=1.5)


# ---------------------------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------------------------

def _random_paged(rng, B=3, Hq=8, Hkv=2, D=8, Dv=6, page=4, lens=(23, 16, 9), latent=False):
    n_pages = [-(-n // page) for n in lens]
    P = sum(n_pages) + 3
    perm = rng.permutation(P)
    kc = np.full((P, Hkv, page, D), np.nan)
    vc = None if latent else np.full((P, Hkv, Dv, page), np.nan)
    table = np.zeros((B, max(n_pages)), dtype=np.int64)
    Kc, Vc = [], []
    off = 0
    for b in range(B):
        Kb = rng.standard_normal((Hkv, lens[b], D))
        Kb[:, 0] *= 3.0
        Vb = rng.standard_normal((Hkv, lens[b], Dv))
        Kc.append(Kb)
        Vc.append(Vb)
        for p in range(n_pages[b]):
            pid = perm[off + p]
            table[b, p] = pid
            n = min(page, lens[b] - p * page)
            kc[pid, :, :n] = Kb[:, p * page:p * page + n]
            if not latent:
                vc[pid, :, :, :n] = np.transpose(Vb[:, p * page:p * page + n], (0, 2, 1))
        table[b, n_pages[b]:] = perm[-1]
        off += n_pages[b]
    q = rng.standard_normal((B, Hq, D))
    return q, kc, vc, table, np.array(lens), Kc, Vc


@pytest.mark.parametrize("S", [1, 2, 5])
def test_decode_equals_dense_on_contiguous_kv_at_lambda_zero(S):
    rng = np.random.default_rng(20 + S)
    q, kc, vc, table, lens, Kc, Vc = _random_paged(rng)
    r = oracle.decode(q, kc, vc, table, lens, page_size=4, block_k=8, num_splits=S, lam=0.0, scale=0.4)
    B, Hq, D = q.shape
    G = Hq // kc.shape[1]
    for b in range(B):
        for h in range(Hq):
            logits = 0.4 * Kc[b][h // G] @ q[b, h]
            w = softmax(logits)
            assert np.max(np.abs(r["o"][b, h] - w @ Vc[b][h // G])) < 1e-9
            assert abs(r["lse"][b, h] - logsumexp(logits)) < 1e-9


def test_decode_tile_is_noncausal_prefill_tile():
    """A decode tile equals a prefill tile whose rows are the tile's q heads, over the gathered keys."""
    rng = np.random.default_rng(31)
    q, kc, vc, table, lens, Kc, Vc = _random_paged(rng)
    lam = 0.08
    r = oracle.decode(q, kc, vc, table, lens, page_size=4, block_k=4, num_splits=2, lam=lam, scale=0.4)
    G = q.shape[1] // kc.shape[1]
    for b in range(q.shape[0]):
        for g in range(kc.shape[1]):
            rows = q[b, g * G:(g + 1) * G]
            t = oracle.tile_sequential(rows, Kc[b][g], Vc[b][g], np.ones((G, lens[b]), bool), 4, 2,
                                       math.log(lam), 0.4)
            assert np.array_equal(t["o"], r["o"][b, g * G:(g + 1) * G])
            n = t["mask"].shape[0]
            assert np.array_equal(t["mask"], r["mask"][b, g, 0, :n])


def test_decode_tile_rows_one_is_per_head():
    rng = np.random.default_rng(32)
    q, kc, vc, table, lens, Kc, Vc = _random_paged(rng)
    lam = 0.1
    r = oracle.decode(q, kc, vc, table, lens, page_size=4, block_k=4, num_splits=1, lam=lam,
                      tile_rows=1, scale=0.4)
    G = q.shape[1] // kc.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            t = oracle.tile_sequential(q[b, h:h + 1], Kc[b][h // G], Vc[b][h // G],
                                       np.ones((1, lens[b]), bool), 4, 1, math.log(lam), 0.4)
            assert np.max(np.abs(t["o"][0] - r["o"][b, h])) < 1e-13


def test_latent_decode_equals_gqa_with_copied_values():
    """Latent attention (V = first Dv channels of K, one shared head) equals ordinary decode with a
    separate V cache holding a copy of those channels."""
    rng = np.random.default_rng(40)
    q, kc, _, table, lens, Kc, _ = _random_paged(rng, Hq=6, Hkv=1, D=10, latent=True)
    Dv = 7
    vc = np.transpose(kc[..., :Dv], (0, 1, 3, 2)).copy()
    kw = dict(page_size=4, block_k=8, num_splits=2, lam=0.05, scale=0.3)
    r1 = oracle.decode(q, kc, None, table, lens, head_dim_v=Dv, **kw)
    r2 = oracle.decode(q, kc, vc, table, lens, **kw)
    assert np.array_equal(r1["mask"], r2["mask"])
    assert np.max(np.abs(r1["o"] - r2["o"])) == 0.0


@pytest.mark.parametrize("T,tile_rows,S", [(2, 3, 1), (4, 6, 2), (3, 2, 3)])
def test_multi_token_latent_decode_equals_gqa_with_copied_values(T, tile_rows, S):
    """Several query tokens per sequence on latent attention (one shared head, V = the first Dv
    channels of K) equal multi-token decode with a separate V cache holding a copy of those channels
    (masks and outputs, at a threshold that skips), and at lambda = 0 they equal causal softmax over
    those keys and values written out with scipy: token t of a sequence of length L sees keys
    0 ... L - T + t."""
    rng = np.random.default_rng(41 + T)
    lens = (23, 16, T + 1)
    _, kc, _, table, lens, Kc, _ = _random_paged(rng, Hq=6, Hkv=1, D=10, latent=True, lens=lens)
    q = _token_queries(rng, 3, T, 6, 10)
    # an attention sink at token 0 (the last channel, outside the V channels) so that blocks skip
    q[..., -1] = 1.0
    for b in range(3):
        kc[table[b, 0], 0, 0, -1] = 30.0
        Kc[b][0, 0, -1] = 30.0
    Dv = 7
    vc = np.transpose(kc[..., :Dv], (0, 1, 3, 2)).copy()
    kw = dict(page_size=4, block_k=4, num_splits=S, scale=0.3, tile_rows=tile_rows)
    for lam in (0.2, 0.0):
        r1 = oracle.decode(q, kc, None, table, lens, head_dim_v=Dv, lam=lam, **kw)
        r2 = oracle.decode(q, kc, vc, table, lens, lam=lam, **kw)
        assert np.array_equal(r1["mask"], r2["mask"])
        assert np.max(np.abs(r1["o"] - r2["o"])) == 0.0
        assert np.array_equal(r1["lse"], r2["lse"])
        if lam > 0:
            assert np.any(r1["mask"] == SKIPPED)
    for b in range(3):
        L = int(lens[b])
        K = Kc[b][0]
        for t in range(T):
            logits = 0.3 * (q[b, t] @ K.T)[:, :L - T + t + 1]
            want = softmax(logits, axis=1) @ K[:L - T + t + 1, :Dv]
            assert np.max(np.abs(r1["o"][b, t] - want)) < 1e-12
            assert np.max(np.abs(r1["lse"][b, t] - logsumexp(logits, axis=1))) < 1e-12


def test_decode_a_over_L_uses_each_sequence_length():
    rng = np.random.default_rng(41)
    q, kc, vc, table, lens, Kc, Vc = _random_paged(rng)
    a = 0.9
    r = oracle.decode(q, kc, vc, table, lens, page_size=4, block_k=4, num_splits=1, a=a, scale=0.4)
    for b in range(q.shape[0]):
        rb = oracle.decode(q[b:b + 1], kc, vc, table[b:b + 1], lens[b:b + 1], page_size=4, block_k=4,
                           num_splits=1, lam=min(1.0, a / lens[b]), scale=0.4)
        assert np.array_equal(rb["o"][0], r["o"][b])


def _token_queries(rng, B, T, Hq, D):
    return rng.standard_normal((B, T, Hq, D))


@pytest.mark.parametrize("T,S", [(1, 1), (3, 1), (4, 3), (7, 2)])
def test_multi_token_decode_dense_is_causal_softmax(T, S):
    """T query tokens per sequence at lambda = 0: token t of sequence b is softmax attention over keys
    0 .. seq_len - T + t (written out here with scipy), whatever the splits."""
    rng = np.random.default_rng(60 + T)
    _, kc, vc, table, lens, Kc, Vc = _random_paged(rng)
    B, Hq, Hkv = 3, 8, 2
    G = Hq // Hkv
    q = _token_queries(rng, B, T, Hq, 8)
    r = oracle.decode(q, kc, vc, table, lens, page_size=4, block_k=8, num_splits=S, lam=0.0, scale=0.4)
    assert r["o"].shape == (B, T, Hq, 6) and r["lse"].shape == (B, T, Hq)
    for b in range(B):
        for t in range(T):
            n = lens[b] - T + t + 1
            for h in range(Hq):
                logits = 0.4 * Kc[b][h // G][:n] @ q[b, t, h]
                assert np.max(np.abs(r["o"][b, t, h] - softmax(logits) @ Vc[b][h // G][:n])) < 1e-9
                assert abs(r["lse"][b, t, h] - logsumexp(logits)) < 1e-9


def test_multi_token_decode_one_token_is_single_token_decode():
    rng = np.random.default_rng(61)
    q, kc, vc, table, lens, _, _ = _random_paged(rng)
    kw = dict(page_size=4, block_k=4, num_splits=2, lam=0.1, scale=0.4)
    r1 = oracle.decode(q, kc, vc, table, lens, **kw)
    r4 = oracle.decode(q[:, None], kc, vc, table, lens, **kw)
    assert np.array_equal(r1["o"], r4["o"][:, 0]) and np.array_equal(r1["lse"], r4["lse"][:, 0])
    assert np.array_equal(r1["mask"], r4["mask"])


@pytest.mark.parametrize("T,S,lam", [(4, 1, 0.5), (5, 2, 0.7), (8, 1, 0.9)])
def test_multi_token_decode_single_head_tile_is_prefill_tile(T, S, lam):
    """With one q head per tile, a decode tile of T tokens is the prefill tile of Lq = T queries
    over the sequence's keys (block_q = T, bottom-right causal): the same decisions and outputs,
    reached through the paged gather on one side and contiguous tensors on the other."""
    rng = np.random.default_rng(62 + T)
    _, kc, vc, table, lens, Kc, Vc = _random_paged(rng, lens=(23, 16, 12))
    q = _token_queries(rng, 3, T, 8, 8)
    r = oracle.decode(q, kc, vc, table, lens, page_size=4, block_k=4, num_splits=S, lam=lam, tile_rows=1,
                      scale=0.4)
    G = 4
    skipped = 0
    for b in range(3):
        for h in range(8):
            p = oracle.prefill(q[b, :, h][None, None], Kc[b][h // G][None, None], Vc[b][h // G][None, None],
                               causal=True, block_q=T, block_k=4, num_splits=S, lam=lam, scale=0.4)
            n = p["mask"].shape[-1]
            assert np.array_equal(p["mask"][0, 0, 0], r["mask"][b, h // G, h % G, :n])
            assert np.max(np.abs(p["o"][0, 0] - r["o"][b, :, h])) < 1e-12
            assert np.max(np.abs(p["lse"][0, 0] - r["lse"][b, :, h])) < 1e-12
            skipped += int((p["mask"] == SKIPPED).sum())
    assert skipped > 0


def test_multi_token_decode_rows_without_keys():
    """A sequence shorter than T: its first T - seq_len tokens see no key (o = 0, lse = -inf), the
    rest are causal softmax over what they see."""
    rng = np.random.default_rng(63)
    _, kc, vc, table, lens, Kc, Vc = _random_paged(rng, lens=(23, 3, 9))
    T = 5
    q = _token_queries(rng, 3, T, 8, 8)
    r = oracle.decode(q, kc, vc, table, lens, page_size=4, block_k=8, num_splits=1, lam=0.3, scale=0.4)
    assert np.all(r["o"][1, :2] == 0.0) and np.all(r["lse"][1, :2] == -np.inf)
    for t in (2, 3, 4):
        n = 3 - T + t + 1
        for h in range(8):
            logits = 0.4 * Kc[1][h // 4][:n] @ q[1, t, h]
            assert np.max(np.abs(r["o"][1, t, h] - softmax(logits) @ Vc[1][h // 4][:n])) < 1e-12


def test_decode_empty_sequence():
    """A sequence of length 0 (a reading: it has no key, so nothing to attend to) gives o = 0,
    lse = -inf and no live block, for a fixed lambda, for a / L and at lambda = 0, and leaves the other
    sequences exactly as they are in a batch without it."""
    rng = np.random.default_rng(64)
    q, kc, vc, table, lens, Kc, Vc = _random_paged(rng, lens=(23, 5, 9))
    lens0 = lens.copy()
    lens0[1] = 0
    others = [0, 2]
    for kw in (dict(lam=0.3), dict(a=2.0), dict(lam=0.0)):
        r = oracle.decode(q, kc, vc, table, lens0, page_size=4, block_k=8, num_splits=2, scale=0.4, **kw)
        assert np.all(r["o"][1] == 0.0) and np.all(r["lse"][1] == -np.inf)
        assert np.all(r["mask"][1] == NOT_LIVE) and np.all(np.isnan(r["crit"][1]))
        r2 = oracle.decode(q[others], kc, vc, table[others], lens[others], page_size=4, block_k=8, num_splits=2,
                           scale=0.4, **kw)
        assert np.array_equal(r["o"][others], r2["o"]) and np.array_equal(r["lse"][others], r2["lse"])
        assert np.array_equal(r["mask"][others], r2["mask"])


# ---------------------------------------------------------------------------------------------
# the dense reference itself
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["causal", "random", "causal_offset", "full"])
def test_softmax_attention_equals_library_attention(kind):
    """oracle.softmax_attention against torch's scaled_dot_product_attention (fp64, CPU, boolean
    mask) for the output and scipy's logsumexp for the LSE, on masks built here independently:
    bottom-right causal, causal with more rows than keys (rows without any visible key), a seeded
    random mask with empty rows, and no mask.  A non-default scale catches a dropped or doubled
    scale; the random mask catches a dropped visibility test."""
    import torch
    rng = np.random.default_rng({"causal": 1, "random": 2, "causal_offset": 3, "full": 4}[kind])
    R, N, D, Dv = 23, 31, 12, 7
    if kind == "causal_offset":
        R, N = 40, 29          # rows 0..10 see no key under bottom-right alignment
    q = rng.standard_normal((R, D)) * 1.7
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, Dv))
    if kind in ("causal", "causal_offset"):
        vis = np.array([[c <= r + (N - R) for c in range(N)] for r in range(R)])
    elif kind == "random":
        vis = rng.random((R, N)) < 0.3
        vis[[2, 9]] = False
        vis[5] = False
        vis[5, 17] = True      # a row with exactly one visible key
    else:
        vis = np.ones((R, N), dtype=bool)
    scale = 0.29
    o, lse = oracle.softmax_attention(q, k, v, vis, scale)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    want = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=t(vis),
                                                            scale=scale)[0, 0].numpy()
    empty = ~vis.any(axis=1)
    assert (kind in ("random", "causal_offset")) == bool(empty.any())
    assert np.max(np.abs(o[~empty] - want[~empty])) < 1e-12
    assert np.all(o[empty] == 0.0) and np.all(lse[empty] == -np.inf)
    logits = scale * (q @ k.T)
    for r in np.nonzero(~empty)[0]:
        assert abs(lse[r] - logsumexp(logits[r][vis[r]])) < 1e-12
    if kind == "random":
        # a single visible key gets all the weight
        assert np.max(np.abs(o[5] - v[17])) < 1e-14 and abs(lse[5] - logits[5, 17]) < 1e-14

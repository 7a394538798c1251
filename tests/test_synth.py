"""The seeded generator: determinism, boosts, statistics and the paged layout."""

import math

import numpy as np
import torch

import synth


def test_prefill_is_deterministic():
    a = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=256, d=64, block_k=32, seed=5)
    b = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=256, d=64, block_k=32, seed=5)
    c = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=256, d=64, block_k=32, seed=6)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v)]:
        assert torch.equal(x, y)
    assert not torch.equal(a.q, c.q)


def test_prefill_boosts_and_logit_std():
    d, L, bk = 128, 2048, 128
    p = synth.prefill_inputs(batch=1, hq=2, hkv=1, L=L, d=d, dtype=torch.float32, block_k=bk,
                             window=False, seed=1)
    q, k = p.q[0].double(), p.k[0, 0].double()
    logits = p.scale * q @ k.T                          # [2, L, L]
    al = set(p.aligned[0][0])
    assert len(al) == round(0.1 * (L // bk)) and 0 not in al
    content = torch.ones(L, dtype=torch.bool)
    content[0] = False
    for j in al:
        content[j * bk:(j + 1) * bk] = False
    std = logits[:, :, content].std().item()
    assert 0.95 < std < 1.05
    # sink and aligned boosts are exact in the control channels
    assert torch.allclose(p.scale * q[..., d - 2] * k[0, d - 2], torch.full_like(q[..., 0], 10.0), atol=1e-5)
    j = min(al)
    assert abs(p.scale * k[j * bk, d - 1].item() - 6.0) < 1e-5


def test_window_boost_decays():
    d, L = 128, 4096
    p = synth.prefill_inputs(batch=1, hq=8, hkv=1, L=L, d=d, dtype=torch.float32, block_k=128,
                             window=True, seed=2)
    q, k = p.q[0, :, :, :d - 2].double(), p.k[0, 0, :, :d - 2].double()
    logits = p.scale * q @ k.T
    i = torch.arange(1024, L)
    for delta, tol in [(0, 0.3), (512, 0.3), (2048, 0.3)]:
        mean = logits[:, i, i - delta].mean().item()
        assert abs(mean - 3.0 * math.exp(-delta / 512.0)) < tol, (delta, mean)


def test_bf16_rne_helper_matches_torch_cast():
    x = np.random.default_rng(0).standard_normal(10000) * 100
    want = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).double().numpy()
    assert np.array_equal(synth.to_bf16_rne_numpy(x), want)


def test_paged_layout():
    B, ctx, page = 3, 200, 16
    d = synth.decode_inputs(batch=B, hq=8, hkv=2, ctx=ctx, d=64, page_size=page, block_k=64, seed=9,
                            seq_lens=[200, 37, 64])
    bt = d.block_table
    lens = d.seq_lens.tolist()
    used = []
    for b in range(B):
        npg = -(-lens[b] // page)
        used += bt[b, :npg].tolist()
        # slots after the last key are NaN; keys before it are finite
        last = bt[b, npg - 1].item()
        n_last = lens[b] - (npg - 1) * page
        assert torch.isfinite(d.k_cache[last, :, :n_last].float()).all()
        assert torch.isnan(d.k_cache[last, :, n_last:].float()).all()
        assert torch.isnan(d.v_cache_t[last, :, :, n_last:].float()).all()
        # unused table entries point at a NaN page
        for pid in bt[b, npg:].tolist():
            assert torch.isnan(d.k_cache[pid].float()).all()
    assert len(set(used)) == len(used)          # pages are not shared
    P = d.k_cache.shape[0]
    spare = sorted(set(range(P)) - set(used))
    assert len(spare) >= 1
    for pid in spare:
        assert torch.isnan(d.k_cache[pid].float()).all()
    # sink at token 0 of every sequence
    for b in range(B):
        first = bt[b, 0].item()
        assert abs(d.scale * d.k_cache[first, :, 0, 62].float() - 10.0).max() < 0.05


def test_latent_cache_has_no_v():
    d = synth.decode_inputs(batch=2, hq=16, hkv=1, ctx=64, d=72, dv=64, page_size=16, block_k=64,
                            seed=1, latent=True)
    assert d.v_cache_t is None and d.head_dim_v == 64 and d.k_cache.shape[1] == 1


def test_head_strength_scales_each_heads_boosts():
    """head_strength c_h: sink boost 10 c_h, aligned boost 6 c_h, window boost 3 c_h per q head, unit
    content-logit spread kept; None is the homogeneous draw, bit for bit."""
    d, L, bk = 128, 4096, 128
    base = synth.prefill_inputs(batch=1, hq=4, hkv=1, L=L, d=d, dtype=torch.float32, block_k=bk, seed=4)
    ones = synth.prefill_inputs(batch=1, hq=4, hkv=1, L=L, d=d, dtype=torch.float32, block_k=bk, seed=4,
                                head_strength=[1.0] * 4)
    assert torch.equal(base.q, ones.q) and torch.equal(base.k, ones.k) and torch.equal(base.v, ones.v)
    c = [0.5, 1.0, 1.5, 2.0]
    p = synth.prefill_inputs(batch=1, hq=4, hkv=1, L=L, d=d, dtype=torch.float32, block_k=bk, seed=4,
                             head_strength=c)
    assert torch.equal(p.k, base.k) and torch.equal(p.v, base.v)
    q, k = p.q[0].double(), p.k[0, 0].double()
    j = min(p.aligned[0][0])
    i = torch.arange(1024, L)
    for h, ch in enumerate(c):
        assert torch.allclose(p.scale * q[h, :, d - 2] * k[0, d - 2], torch.full((L,), 10.0 * ch, dtype=torch.float64),
                              atol=1e-5)
        assert abs(p.scale * q[h, 0, d - 1].item() * k[j * bk, d - 1].item() - 6.0 * ch) < 1e-5
        content = p.scale * q[h, :, :d - 2] @ k[:, :d - 2].T
        assert abs(content[i, i].mean().item() - 3.0 * ch) < 0.3, (h, content[i, i].mean().item())
        assert 0.9 < content[i, i - 2048].std().item() < 1.1
    try:
        synth.prefill_inputs(batch=1, hq=4, hkv=1, L=256, d=64, block_k=64, seed=4, head_strength=[1.0])
    except ValueError:
        pass
    else:
        raise AssertionError("a wrong-length head_strength must be rejected")


def test_decode_multi_token_queries_sit_at_the_last_positions():
    """num_q_tokens = T: q [B, T, Hq, D]; token t's content correlates with the key at its own
    position seq_len - T + t (window boost about 3 there, decaying away from it)."""
    T, L, d = 8, 2048, 128
    x = synth.decode_inputs(batch=2, hq=16, hkv=1, ctx=L, d=d, dtype=torch.float32, seed=12, num_q_tokens=T)
    assert x.q.shape == (2, T, 16, d)
    k = x.k_cache[x.block_table[0].long(), 0].reshape(-1, d)[:L, :d - 2].double()
    q = x.q[0, :, :, :d - 2].double()
    own = torch.stack([x.scale * q[t] @ k[L - T + t] for t in range(T)])     # [T, Hq]
    assert abs(own.mean().item() - 3.0) < 0.5
    far = torch.stack([x.scale * q[t] @ k[L - T + t - 1500] for t in range(T)])
    assert abs(far.mean().item()) < 1.0 and own.mean().item() - far.mean().item() > 2.0
    try:
        synth.decode_inputs(batch=1, hq=4, hkv=1, ctx=5, d=64, seed=1, num_q_tokens=6)
    except ValueError:
        pass
    else:
        raise AssertionError("more query tokens than keys must be rejected")

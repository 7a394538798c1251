"""GPU parity of blasst_prefill_paged (chunked prefill against a paged cache, through the C ABI) against
the fp64 oracle: per sequence, the oracle's prefill tiles over the sequence's keys gathered from the
pages, with the queries as the last Lq positions (bottom-right causal)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import Report, check_tile, host64

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_online_amd as m
    m.lib()
    return m


def _run(m, d, *, splits, lam=None, a=None, out_dtype=torch.float32, stats_only=False):
    q = d.q.permute(0, 2, 1, 3)          # [B, Hq, Lq, D] view of the [B, Lq, Hq, D] queries
    B, Hq, Lq, D = q.shape
    nqt = -(-Lq // 128)
    nkb = -(-(d.block_table.shape[1] * d.page_size) // 128)
    o = None if stats_only else torch.full((B, Hq, Lq, d.head_dim_v), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device="cuda")
    mask = torch.full((B, Hq, nqt, nkb), 7, dtype=torch.uint8, device="cuda")
    crit = torch.full((B, Hq, nqt, nkb), 12345.0, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    m.blasst_prefill_paged(q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, num_splits=splits, lam=lam, a=a,
                           lse=None if stats_only else lse, skip_mask=mask, crit=crit, counters=cnt,
                           stats_only=stats_only)
    torch.cuda.synchronize()
    return o, lse, mask, crit, cnt


def _gather(d, b):
    """The sequence's keys and values as contiguous fp64 [1, Hkv, L, D] arrays, and L."""
    L = int(d.seq_lens[b])
    npg = -(-L // d.page_size)
    ids = d.block_table[b, :npg].long()
    kc = host64(d.k_cache[ids])
    vc = host64(d.v_cache_t[ids])
    bt = np.arange(npg)[None, :]
    Hkv = kc.shape[1]
    K, V = [], []
    for g in range(Hkv):
        k_, v_ = oracle.gather_pages(kc, vc, bt, 0, g, L, d.page_size, d.head_dim_v)
        K.append(k_)
        V.append(v_)
    return np.ascontiguousarray(np.stack(K)[None]), np.ascontiguousarray(np.stack(V)[None]), L


def _compare(d, res, *, splits, lam=None, a=None, out_bf16=False, tiles=None):
    o, lse, mask, crit, cnt = res
    q = d.q.permute(0, 2, 1, 3)
    B, Hq, Lq, _ = q.shape
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    rep = Report()
    nqt = mh.shape[2]
    for b in range(B):
        K, V, L = _gather(d, b)
        qb = host64(q[b:b + 1])
        ln_lam = oracle.ln_threshold(lam=lam) if lam is not None else oracle.ln_threshold(a=a, L=L)
        kw = dict(causal=True, block_q=128, block_k=128, num_splits=splits, ln_lam=ln_lam)
        for h in range(Hq):
            for t in range(nqt):
                if tiles is not None and (b, h, t) not in tiles:
                    continue
                ref = oracle.prefill_tile(qb, K, V, 0, h, t, **kw)
                n = ref["mask"].shape[0]
                assert np.all(mh[b, h, t, n:] == 2), "blocks past the sequence must be not live"
                r0, r1 = t * 128, min((t + 1) * 128, Lq)
                check_tile(rep, ref, mh[b, h, t], ch[b, h, t], ln_lam,
                           lambda f: oracle.prefill_tile(qb, K, V, 0, h, t, force=f, **kw),
                           None if o is None else host64(o[b, h, r0:r1]),
                           None if o is None else lse[b, h, r0:r1].cpu().double().numpy(), out_bf16=out_bf16)
    if tiles is None:
        assert int(cnt[0]) == int((mh != 2).sum()) and int(cnt[1]) == int((mh == 1).sum())
    return rep


@pytest.mark.parametrize("a", [0.0, 4.0, 30.0])
@pytest.mark.parametrize("splits", [1, 3])
def test_paged_prefill_ragged_contexts(a, splits):
    """A 300-token chunk of four sequences with contexts 1000, 300 (the chunk is the whole
    sequence), 777 and 2048 tokens, 8 q / 2 kv heads, lambda = a / seq_len per sequence."""
    m = _lib()
    T = 300
    d = synth.decode_inputs(batch=4, hq=8, hkv=2, ctx=None, d=128, seq_lens=[1000, 300, 777, 2048], seed=101,
                            device="cuda", num_q_tokens=T)
    res = _run(m, d, splits=splits, a=a)
    rep = _compare(d, res, splits=splits, a=a)
    print(f"a={a} S={splits}: {rep}")
    if a == 0.0:
        assert rep.skipped == 0


def test_paged_prefill_bf16_out_odd_group_and_short_sequences():
    """bf16 output, a group of 3 q heads per kv head (one head per workgroup), and sequences shorter
    than the chunk: rows that see no key get o = 0 and lse = -inf."""
    m = _lib()
    T = 200
    d = synth.decode_inputs(batch=3, hq=6, hkv=2, ctx=None, d=128, seq_lens=[400, 250, 200], seed=102,
                            device="cuda", num_q_tokens=T)
    d.seq_lens[2] = 150    # rows 0 ... 49 of sequence 2 see no key
    res = _run(m, d, splits=1, lam=0.01, out_dtype=torch.bfloat16)
    o, lse = res[0], res[1]
    assert torch.all(o[2, :, :50] == 0) and torch.all(lse[2, :, :50] == float("-inf"))
    rep = _compare(d, res, splits=1, lam=0.01, out_bf16=True)
    print(rep)


def test_paged_matches_contiguous_prefill():
    """One sequence whose pages are permuted in the pool, against the contiguous prefill kernel run on
    the same keys and values laid out contiguously: the same scores, so the same skip mask and
    critical values bit for bit; outputs and LSE to fp32 rounding (the paged kernel orders keys
    differently inside its P.V products)."""
    m = _lib()
    T, L = 384, 1500
    d = synth.decode_inputs(batch=1, hq=8, hkv=2, ctx=L, d=128, seed=103, device="cuda", num_q_tokens=T)
    res = _run(m, d, splits=2, lam=0.02)
    K, V, _ = _gather(d, 0)
    k = torch.tensor(K, dtype=torch.float32).to(torch.bfloat16).cuda()
    v = torch.tensor(V, dtype=torch.float32).to(torch.bfloat16).cuda()
    q = d.q.permute(0, 2, 1, 3)
    o = torch.empty(1, 8, T, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(1, 8, T, dtype=torch.float32, device="cuda")
    mask = torch.empty_like(res[2])
    crit = torch.empty_like(res[3])
    m.blasst_prefill(q, k, v, o, causal=True, block_q=128, block_k=128, num_splits=2, lam=0.02, lse=lse,
                     skip_mask=mask, crit=crit)
    torch.cuda.synchronize()
    nkb = -(-L // 128)
    assert torch.equal(mask[..., :nkb], res[2][..., :nkb])
    torch.testing.assert_close(res[3][..., :nkb], crit[..., :nkb], rtol=0, atol=0, equal_nan=True)
    torch.testing.assert_close(res[0], o, rtol=2e-5, atol=2e-6)
    torch.testing.assert_close(res[1], lse, rtol=0, atol=2e-5)


def test_stats_only_matches_full_pass():
    m = _lib()
    d = synth.decode_inputs(batch=2, hq=8, hkv=2, ctx=None, d=128, seq_lens=[900, 1300], seed=104, device="cuda",
                            num_q_tokens=256)
    full = _run(m, d, splits=1, a=8.0)
    st = _run(m, d, splits=1, a=8.0, stats_only=True)
    assert torch.equal(full[2], st[2]) and torch.equal(full[4], st[4])
    assert torch.allclose(full[3], st[3], rtol=0, atol=0, equal_nan=True)


def test_chunk_of_32k_contexts_sampled_tiles():
    """The chunked-prefill benchmark shape: 4 sequences whose 32768-token contexts end with a
    2048-token chunk, 32 q / 8 kv heads; sampled tiles against the oracle."""
    m = _lib()
    T, L = 2048, 32768
    d = synth.decode_inputs(batch=4, hq=32, hkv=8, ctx=L, d=128, seed=synth.config_seed(6), device="cuda",
                            num_q_tokens=T)
    res = _run(m, d, splits=1, a=float(L) * 0.02)
    tiles = {(0, 0, 15), (1, 13, 0), (3, 31, 7), (2, 7, 11)}
    rep = _compare(d, res, splits=1, a=float(L) * 0.02, tiles=tiles)
    mh = res[2].cpu().numpy()
    print(f"sparsity {(mh == 1).sum() / (mh != 2).sum():.3f}; {rep}")


@pytest.mark.parametrize("splits", [1, 2])
def test_paged_prefill_one_to_three_blocks(splits):
    """Contexts of 100, 128, 129, 256 and 257 keys (one, one, two, two and three 128-key blocks, the
    last page partly filled or full) with a 64-token chunk: the first blocks' page ids, which the
    kernel stages before its block loop, and sequences that end inside or at the end of a page."""
    m = _lib()
    d = synth.decode_inputs(batch=5, hq=8, hkv=2, ctx=None, d=128, seq_lens=[100, 128, 129, 256, 257], seed=105,
                            device="cuda", num_q_tokens=64)
    res = _run(m, d, splits=splits, lam=0.02)
    rep = _compare(d, res, splits=splits, lam=0.02)
    print(f"S={splits}: {rep}")

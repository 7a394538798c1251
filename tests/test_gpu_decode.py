"""GPU parity of blasst_decode (paged split-KV, through the C ABI) against the fp64 oracle."""

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


def _run(m, d, *, splits, lam=None, a=None, tile_rows=0, out_dtype=torch.float32, stats_only=False):
    B, Hq = d.q.shape[0], d.q.shape[-2]       # q [B, Hq, D] or [B, T, Hq, D]
    Hkv = d.k_cache.shape[1]
    G = Hq // Hkv
    tr = G if tile_rows == 0 else tile_rows
    dev = d.q.device
    max_pages = d.block_table.shape[1]
    nkb = -(-(max_pages * d.page_size) // 64)
    rows = tuple(d.q.shape[:-1])
    o = None if stats_only else torch.full(rows + (d.head_dim_v,), float("nan"), dtype=out_dtype, device=dev)
    lse = torch.full(rows, float("nan"), dtype=torch.float32, device=dev)
    mask = torch.full((B, Hkv, G // tr, nkb), 7, dtype=torch.uint8, device=dev)
    crit = torch.full((B, Hkv, G // tr, nkb), 12345.0, dtype=torch.float32, device=dev)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    kw = dict(page_size=d.page_size, block_k=64, num_splits=splits, lam=lam, a=a, tile_rows=tile_rows,
              head_dim_v=d.head_dim_v, lse=None if stats_only else lse, skip_mask=mask, crit=crit,
              counters=cnt, stats_only=stats_only)
    nbytes = m.blasst_decode_workspace_size(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, **kw)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    m.blasst_decode(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, workspace=ws, **kw)
    torch.cuda.synchronize()
    return o, lse, mask, crit, cnt


def _tile_inputs(d, b):
    """Host fp64 copies of what one sequence's tiles read: its query, its pages (renumbered 0..n-1)."""
    L = int(d.seq_lens[b])
    npg = -(-L // d.page_size)
    ids = d.block_table[b, :npg].long()
    kc = host64(d.k_cache[ids])
    vc = host64(d.v_cache_t[ids]) if d.v_cache_t is not None else None
    bt = np.arange(npg, dtype=np.int64)[None, :]
    return host64(d.q[b:b + 1]), kc, vc, bt, np.array([L])


def _compare(d, res, *, splits, lam=None, a=None, tiles=None, tile_rows=0, out_bf16=False):
    o, lse, mask, crit, cnt = res
    sl = d.seq_lens.cpu().numpy()
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    oh = host64(o) if o is not None else None
    lh = lse.cpu().double().numpy()
    B, Hq = d.q.shape[0], d.q.shape[-2]
    Hkv = d.k_cache.shape[1]
    G = Hq // Hkv
    tr = G if tile_rows == 0 else tile_rows
    multi = d.q.dim() == 4
    rep = Report()
    if tiles is None:
        tiles = [(b, g, rt) for b in range(B) for g in range(Hkv) for rt in range(G // tr)]
    cache = {}
    for (b, g, rt) in tiles:
        if b not in cache:
            cache = {b: _tile_inputs(d, b)}
        qh, kc, vc, bt, sl1 = cache[b]
        ln_lam = oracle.ln_threshold(lam=lam) if lam is not None else oracle.ln_threshold(a=a, L=int(sl[b]))
        kw = dict(page_size=d.page_size, block_k=64, num_splits=splits, ln_lam=ln_lam, tile_rows=tr,
                  head_dim_v=d.head_dim_v)
        ref = oracle.decode_tile(qh, kc, vc, bt, sl1, 0, g, rt, **kw)
        h0 = g * G + rt * tr
        nb = ref["mask"].shape[0]
        assert np.all(mh[b, g, rt, nb:] == 2)
        check_tile(rep, ref, mh[b, g, rt], ch[b, g, rt], ln_lam,
                   lambda f: oracle.decode_tile(qh, kc, vc, bt, sl1, 0, g, rt, force=f, **kw),
                   None if oh is None else (oh[b, :, h0:h0 + tr].reshape(-1, oh.shape[-1]) if multi
                                            else oh[b, h0:h0 + tr]),
                   None if oh is None else (lh[b, :, h0:h0 + tr].reshape(-1) if multi else lh[b, h0:h0 + tr]),
                   out_bf16=out_bf16)
    return rep


@pytest.mark.parametrize("splits", [1, 3, 16, 24])
@pytest.mark.parametrize("a", [0.0, 2.0, 20.0])
def test_gqa_paged_ragged(splits, a):
    """32 q / 8 kv heads, d = 128, ragged sequence lengths (including a one-page and a one-token
    sequence), 16-token pages in a permuted pool with NaN spare pages.  24 splits: the combine merges
    two chunks of splits, and splits past a sequence's blocks hold empty partials."""
    m = _lib()
    lens = [1000, 64, 17, 2048, 1, 333]
    d = synth.decode_inputs(batch=len(lens), hq=32, hkv=8, ctx=None, d=128, seq_lens=lens, seed=3,
                            device="cuda")
    res = _run(m, d, splits=splits, a=a)
    rep = _compare(d, res, splits=splits, a=a)
    print(f"S={splits} a={a}: {rep}")
    o, _, mask, _, cnt = res
    mh = mask.cpu().numpy()
    assert int(cnt[0]) == int((mh != 2).sum()) and int(cnt[1]) == int((mh == 1).sum())
    if a == 0.0:
        assert rep.skipped == 0


@pytest.mark.parametrize("tile_rows", [1, 2, 4])
def test_tile_rows_and_bf16_out(tile_rows):
    m = _lib()
    d = synth.decode_inputs(batch=3, hq=16, hkv=4, ctx=900, d=128, seed=4, device="cuda")
    res = _run(m, d, splits=4, lam=0.003, tile_rows=tile_rows, out_dtype=torch.bfloat16)
    rep = _compare(d, res, splits=4, lam=0.003, tile_rows=tile_rows, out_bf16=True)
    print(rep)


def test_mha_and_mqa():
    m = _lib()
    for hq, hkv in [(8, 8), (8, 1)]:
        d = synth.decode_inputs(batch=2, hq=hq, hkv=hkv, ctx=700, d=128, seed=5, device="cuda")
        res = _run(m, d, splits=2, lam=0.01)
        print(_compare(d, res, splits=2, lam=0.01))


def test_stats_only_matches_full_pass():
    m = _lib()
    d = synth.decode_inputs(batch=4, hq=32, hkv=8, ctx=2000, d=128, seed=6, device="cuda")
    full = _run(m, d, splits=4, lam=0.005)
    st = _run(m, d, splits=4, lam=0.005, stats_only=True)
    assert torch.equal(full[2], st[2]) and torch.equal(full[4], st[4])
    assert torch.allclose(full[3], st[3], rtol=0, atol=0, equal_nan=True)


@pytest.mark.parametrize("ctx", [32768])
def test_gqa_decode_full_size_sampled(ctx):
    """Batch 32, 32 q / 8 kv heads, d = 128, 16-token pages, 64-token blocks, 16 splits (the
    benchmark's launch configuration); sampled tiles against the oracle, all masks consistent with
    the critical values."""
    m = _lib()
    d = synth.decode_inputs(batch=32, hq=32, hkv=8, ctx=ctx, d=128, seed=synth.config_seed(3), device="cuda")
    a = 0.02 * ctx
    res = _run(m, d, splits=16, a=a)
    o, lse, mask, crit, cnt = res
    ln_lam = math.log(min(1.0, a / ctx))
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    live = mh != 2
    decided = np.where(live, np.where(ch < ln_lam, 1, 0), 2)
    band = live & (np.abs(ch - ln_lam) < 1e-3)
    assert np.array_equal(decided[~band], mh[~band])
    assert torch.isfinite(o).all()
    tiles = [(0, 0, 0), (5, 3, 0), (17, 7, 0), (31, 4, 0)]
    rep = _compare(d, res, splits=16, a=a, tiles=tiles)
    print(f"sparsity {float((mh == 1).sum()) / live.sum():.3f}; {rep}")


@pytest.mark.parametrize("tile_rows", [128, 64])
@pytest.mark.parametrize("splits", [1, 4, 12])
@pytest.mark.parametrize("a", [0.0, 2.0, 20.0])
def test_latent_mla_ragged(tile_rows, splits, a):
    """Latent attention: 128 q heads on one 576-channel latent head, V = first 512 channels, ragged
    sequence lengths, NaN-poisoned spare pages and tail slots."""
    m = _lib()
    lens = [1000, 64, 17]
    d = synth.decode_inputs(batch=3, hq=128, hkv=1, ctx=None, d=576, dv=512, seq_lens=lens, seed=8,
                            device="cuda", latent=True)
    res = _run(m, d, splits=splits, a=a, tile_rows=tile_rows)
    rep = _compare(d, res, splits=splits, a=a, tile_rows=tile_rows)
    print(f"tile_rows={tile_rows} S={splits} a={a}: {rep}")
    if a == 0.0:
        assert rep.skipped == 0


@pytest.mark.parametrize("splits", [8, 16])
def test_latent_mla_full_size_sampled(splits):
    """Batch 64, 128 q heads on one latent head (576 / 512), context 32768, 16-token pages, 64-token
    blocks, 128-head tiles, 8 splits (the benchmarked launch) and 16: sampled sequences against the
    oracle."""
    m = _lib()
    d = synth.decode_inputs(batch=64, hq=128, hkv=1, ctx=32768, d=576, dv=512, seed=synth.config_seed(5),
                            device="cuda", latent=True)
    a = 0.02 * 32768
    res = _run(m, d, splits=splits, a=a, tile_rows=128, out_dtype=torch.bfloat16)
    o, lse, mask, crit, cnt = res
    ln_lam = math.log(min(1.0, a / 32768))
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    live = mh != 2
    decided = np.where(live, np.where(ch < ln_lam, 1, 0), 2)
    band = live & (np.abs(ch - ln_lam) < 1e-3)
    assert np.array_equal(decided[~band], mh[~band])
    assert torch.isfinite(o.float()).all()
    rep = _compare(d, res, splits=splits, a=a, tiles=[(0, 0, 0), (37, 0, 0), (63, 0, 0)], tile_rows=128,
                   out_bf16=True)
    print(f"sparsity {float((mh == 1).sum()) / live.sum():.3f}; {rep}")


@pytest.mark.parametrize("splits", [1, 4])
def test_latent_mla_late_large_logit_redo(splits):
    """A key far above everything before it in its split (scaled logit +60 against a first-block
    maximum near +10): the 128-head latent kernel must raise its reference max and redo the split
    (its accumulation reference is fixed by the first kept block); the result still matches the
    oracle."""
    m = _lib()
    lens = [1000, 300]
    d = synth.decode_inputs(batch=2, hq=128, hkv=1, ctx=None, d=576, dv=512, seq_lens=lens, seed=11,
                            device="cuda", latent=True)
    scale = 1.0 / math.sqrt(576)
    for b, key in ((0, 700), (1, 290)):
        pid = int(d.block_table[b, key // d.page_size])
        # channel 574 is the sink channel: q = 1 there, so this key's logit is 60 after scaling
        d.k_cache[pid, 0, key % d.page_size, 574] = 60.0 / scale
    res = _run(m, d, splits=splits, a=0.0, tile_rows=128)
    rep = _compare(d, res, splits=splits, a=0.0, tile_rows=128)
    print(f"S={splits}: {rep}")
    assert rep.skipped == 0


@pytest.mark.parametrize("T,tile_rows,splits", [(2, 0, 1), (4, 4, 3), (8, 2, 16), (16, 1, 5), (3, 4, 1)])
@pytest.mark.parametrize("a", [0.0, 4.0])
def test_multi_token_decode(T, tile_rows, splits, a):
    """T query tokens per sequence (the last T positions; token t sees keys <= seq_len - T + t) against
    the paged cache: 16 q / 4 kv heads, ragged lengths including sequences no longer than T and a
    one-token one, every (T, tile_rows) that fills up to the 16 query columns of a tile."""
    m = _lib()
    lens = [700, 64, 2 * T + 1, 1500, T, 130]
    d = synth.decode_inputs(batch=len(lens), hq=16, hkv=4, ctx=None, d=128, seq_lens=lens, seed=50 + T,
                            device="cuda", num_q_tokens=T)
    res = _run(m, d, splits=splits, a=a, tile_rows=tile_rows)
    rep = _compare(d, res, splits=splits, a=a, tile_rows=tile_rows)
    print(f"T={T} tile_rows={tile_rows} S={splits} a={a}: {rep}")
    if a == 0.0:
        assert rep.skipped == 0


def test_multi_token_decode_full_size_sampled():
    """The multi-token benchmark launch: batch 32, 32 q / 8 kv heads, d = 128, context 32768, the last
    4 positions of each sequence as queries, tiles of 4 tokens x 4 heads, 8 splits; sampled tiles
    against the oracle, all masks consistent with the critical values."""
    m = _lib()
    ctx, T = 32768, 4
    d = synth.decode_inputs(batch=32, hq=32, hkv=8, ctx=ctx, d=128, seed=synth.config_seed(3, 2), device="cuda",
                            num_q_tokens=T)
    a = 0.05 * ctx
    res = _run(m, d, splits=8, a=a, tile_rows=4)
    o, lse, mask, crit, cnt = res
    ln_lam = math.log(min(1.0, a / ctx))
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    live = mh != 2
    decided = np.where(live, np.where(ch < ln_lam, 1, 0), 2)
    band = live & (np.abs(ch - ln_lam) < 1e-3)
    assert np.array_equal(decided[~band], mh[~band])
    assert torch.isfinite(o).all()
    rep = _compare(d, res, splits=8, a=a, tile_rows=4, tiles=[(0, 0, 0), (13, 5, 0), (31, 7, 0)])
    print(f"sparsity {float((mh == 1).sum()) / live.sum():.3f}; {rep}")


def test_multi_token_decode_short_sequence_rows_without_keys():
    """seq_lens below T: the first T - seq_len tokens see no key and get o = 0, lse = -inf; the others
    match the oracle (the cache holds more keys than seq_lens admits, and they must stay unread)."""
    m = _lib()
    T = 6
    d = synth.decode_inputs(batch=3, hq=8, hkv=2, ctx=None, d=128, seq_lens=[40, 200, 6], seed=71,
                            device="cuda", num_q_tokens=T)
    d.seq_lens[0] = 4    # tokens 0, 1 of sequence 0 see nothing
    d.seq_lens[2] = 1    # only the last token of sequence 2 sees a key
    res = _run(m, d, splits=2, lam=0.05, tile_rows=2)
    o, lse = res[0].cpu(), res[1].cpu()
    assert torch.all(o[0, :2] == 0) and torch.all(lse[0, :2] == float("-inf"))
    assert torch.all(o[2, :5] == 0) and torch.all(lse[2, :5] == float("-inf"))
    rep = _compare(d, res, splits=2, lam=0.05, tile_rows=2)
    print(rep)


def test_multi_token_one_token_equals_single_token_layout():
    """T = 1 through the [B, 1, Hq, D] layout gives the bits of the [B, Hq, D] call."""
    m = _lib()
    d = synth.decode_inputs(batch=4, hq=32, hkv=8, ctx=3000, d=128, seed=72, device="cuda")
    r1 = _run(m, d, splits=4, lam=0.01)
    d.q = d.q[:, None].contiguous()
    r4 = _run(m, d, splits=4, lam=0.01)
    assert torch.equal(r1[0], r4[0][:, 0]) and torch.equal(r1[1], r4[1][:, 0]) and torch.equal(r1[2], r4[2])

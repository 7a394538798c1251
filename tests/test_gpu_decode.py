"""GPU parity of blasst_decode (paged split-KV, through the C ABI) against the fp64 oracle."""

import ctypes
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


def _tile_inputs(d, b, g):
    """Host fp64 copies of what the tiles of sequence b and kv head g read: the queries of the q heads
    that share kv head g, and that head's slice of the sequence's pages (renumbered 0..n-1), as a
    problem with one sequence and one kv head."""
    L = int(d.seq_lens[b])
    npg = -(-L // d.page_size)
    ids = d.block_table[b, :npg].long()
    Hq, Hkv = d.q.shape[-2], d.k_cache.shape[1]
    G = Hq // Hkv
    kc = host64(d.k_cache[ids, g:g + 1])
    vc = host64(d.v_cache_t[ids, g:g + 1]) if d.v_cache_t is not None else None
    bt = np.arange(npg, dtype=np.int64)[None, :]
    return host64(d.q[b:b + 1, ..., g * G:(g + 1) * G, :]), kc, vc, bt, np.array([L])


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
        if (b, g) not in cache:
            cache = {(b, g): _tile_inputs(d, b, g)}
        qh, kc, vc, bt, sl1 = cache[(b, g)]
        if lam is not None:
            ln_lam = oracle.ln_threshold(lam=lam)
        else:  # an empty sequence has no block to decide on
            ln_lam = -math.inf if int(sl[b]) == 0 else oracle.ln_threshold(a=a, L=int(sl[b]))
        kw = dict(page_size=d.page_size, block_k=64, num_splits=splits, ln_lam=ln_lam, tile_rows=tr,
                  head_dim_v=d.head_dim_v)
        ref = oracle.decode_tile(qh, kc, vc, bt, sl1, 0, 0, rt, **kw)
        h0 = g * G + rt * tr
        nb = ref["mask"].shape[0]
        assert np.all(mh[b, g, rt, nb:] == 2)
        check_tile(rep, ref, mh[b, g, rt], ch[b, g, rt], ln_lam,
                   lambda f: oracle.decode_tile(qh, kc, vc, bt, sl1, 0, 0, rt, force=f, **kw),
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


@pytest.mark.parametrize("latent", [False, True])
@pytest.mark.parametrize("splits,a", [(1, 2.0), (3, 2.0), (3, 0.0)])
def test_decode_empty_sequence(latent, splits, a):
    """A sequence of length 0 between others (its table row points at valid pages, none is read): o = 0,
    lse = -inf, no live block; the other sequences as the oracle gives them."""
    m = _lib()
    if latent:
        d = synth.decode_inputs(batch=3, hq=128, hkv=1, ctx=None, d=576, dv=512, seq_lens=[300, 1, 70], seed=14,
                                device="cuda", latent=True)
    else:
        d = synth.decode_inputs(batch=3, hq=32, hkv=8, ctx=None, d=128, seq_lens=[300, 1, 70], seed=14,
                                device="cuda")
    d.seq_lens[1] = 0
    tr = 128 if latent else 0
    res = _run(m, d, splits=splits, a=a, tile_rows=tr)
    o, lse, mask, _, _ = res
    assert torch.all(o[1] == 0).item() and torch.all(lse[1] == -math.inf).item()
    assert torch.all(mask[1] == 2).item()
    rep = _compare(d, res, splits=splits, a=a, tile_rows=tr)
    print(f"latent={latent} S={splits} a={a}: {rep}")


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


def _calibrated_lambda(m, d, *, splits, target, tile_rows=0):
    """lambda at a target sparsity the way the benchmark sets it: one stats-only pass over every tile
    of the batch (critical values only), then the library's quantile of all of them."""
    if target == 0.0:
        return 0.0
    crit = _run(m, d, splits=splits, lam=0.0, tile_rows=tile_rows, stats_only=True)[3].cpu().numpy()
    return math.exp(m.blasst_calib_quantile(crit, target))


def _seeded_tiles(B, Hkv, n_rt, count, seed, must=()):
    """`count` distinct (sequence, kv head, row tile) picks from a seeded generator, plus `must`,
    sorted so that the tiles of one (sequence, kv head) are compared together."""
    rng = np.random.default_rng(seed)
    every = [(b, g, rt) for b in range(B) for g in range(Hkv) for rt in range(n_rt)]
    pick = {every[i] for i in rng.choice(len(every), size=min(count, len(every)), replace=False)}
    return sorted(pick | set(must))


def _check_whole_mask(res, ln_lam, target):
    """Every tile of the launch: the mask is its critical values compared with ln(lambda) (outside
    the margin band), the counters are the mask's counts, and the sparsity is the calibrated one."""
    o, lse, mask, crit, cnt = res
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    live = mh != 2
    decided = np.where(live, np.where(ch < ln_lam, 1, 0), 2)
    band = live & (np.abs(ch - ln_lam) < 1e-3)
    assert np.array_equal(decided[~band], mh[~band])
    assert int(cnt[0]) == int(live.sum()) and int(cnt[1]) == int((mh == 1).sum())
    assert torch.isfinite(o.float()).all()
    sp = float((mh == 1).sum()) / live.sum()
    if target == 0.0:
        assert sp == 0.0
    else:
        assert abs(sp - target) < 0.02, f"sparsity {sp} at target {target}"
    return sp


@pytest.mark.parametrize("target", [0.73, 0.0])
@pytest.mark.parametrize("ctx", [32768, 131072])
def test_gqa_decode_full_size_at_benchmark_threshold(ctx, target):
    """The benchmarked decode launches: batch 32, 32 q / 8 kv heads, d = 128, context 32768 and
    131072, 16-token pages, 64-token blocks, 16 splits, bf16 output, lambda calibrated for 73 %
    sparsity exactly as the benchmark does it (and lambda = 0).  26 seeded tiles (all 16 splits of
    each) against the oracle, and every tile's mask against its critical values."""
    m = _lib()
    seed = synth.config_seed(3) if ctx == 32768 else synth.config_seed(3, 1)
    d = synth.decode_inputs(batch=32, hq=32, hkv=8, ctx=ctx, d=128, seed=seed, device="cuda")
    lam = _calibrated_lambda(m, d, splits=16, target=target)
    res = _run(m, d, splits=16, lam=lam, out_dtype=torch.bfloat16)
    ln_lam = oracle.ln_threshold(lam=lam)
    sp = _check_whole_mask(res, ln_lam, target)
    tiles = _seeded_tiles(32, 8, 1, 24, seed, must=[(0, 0, 0), (31, 7, 0)])
    rep = _compare(d, res, splits=16, lam=lam, tiles=tiles, out_bf16=True)
    print(f"ctx={ctx} lambda={lam:.6g} sparsity {sp:.4f}; {rep}")
    assert rep.live == len(tiles) * (ctx // 64)


def test_gqa_decode_no_decision_mode_equals_lambda_zero():
    """Threshold mode NONE (the decode kernel without any decision logic) gives the bits of
    lambda = 0 (which the oracle checks here too), keeps every block whatever `a` holds (here 5,
    which as a / L would skip), and is refused with decision diagnostics."""
    m = _lib()
    from long_context_online_amd import blasst as bl
    d = synth.decode_inputs(batch=4, hq=32, hkv=8, ctx=None, d=128, seq_lens=[3000, 64, 1, 777], seed=12,
                            device="cuda")
    ref = _run(m, d, splits=4, lam=0.0)
    print(_compare(d, ref, splits=4, lam=0.0))
    o = torch.full((4, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((4, 32), float("nan"), dtype=torch.float32, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    kw = dict(page_size=16, block_k=64, num_splits=4, lse=lse, counters=cnt, no_decision=True)
    ws = torch.empty(m.blasst_decode_workspace_size(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, **kw),
                     dtype=torch.uint8, device="cuda")
    p = bl.decode_params(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, workspace=ws, **kw)
    p.thr.a = 5.0       # not read in mode NONE
    assert m.lib().blasst_decode(ctypes.byref(p), bl._stream(None)) == 0
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])
    assert int(cnt[1]) == 0 and int(cnt[0]) == int(ref[4][0]) > 0
    mask = torch.empty_like(ref[2])
    with pytest.raises(m.BlasstError):
        m.blasst_decode(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, page_size=16, block_k=64,
                        num_splits=1, no_decision=True, skip_mask=mask)


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


@pytest.mark.parametrize("tile_rows", [128, 64])
@pytest.mark.parametrize("splits,a", [(1, 8.0), (2, 0.0)])
def test_latent_mla_long_splits(tile_rows, splits, a):
    """Latent decode with splits of more than 128 blocks (one sequence of 20000 tokens, 313 blocks,
    another of 9000): the 128-head kernel reads its page ids a 64-block window at a time, so these
    splits run through several window refills; every row against the oracle."""
    m = _lib()
    d = synth.decode_inputs(batch=2, hq=128, hkv=1, ctx=None, d=576, dv=512, seq_lens=[20000, 9000], seed=13,
                            device="cuda", latent=True)
    res = _run(m, d, splits=splits, a=a, tile_rows=tile_rows)
    rep = _compare(d, res, splits=splits, a=a, tile_rows=tile_rows)
    print(f"tile_rows={tile_rows} S={splits} a={a}: {rep}")
    if a == 0.0:
        assert rep.skipped == 0
    else:
        assert rep.skipped > 0


def _mla_full_size():
    return synth.decode_inputs(batch=64, hq=128, hkv=1, ctx=32768, d=576, dv=512, seed=synth.config_seed(5),
                               device="cuda", latent=True)


@pytest.mark.parametrize("splits,target", [(8, 0.73), (8, 0.5), (4, 0.73)])
def test_latent_mla_full_size_at_benchmark_threshold(splits, target):
    """The benchmarked latent decode: batch 64, 128 q heads on one latent head (576 / 512), context
    32768, 16-token pages, 64-token blocks, 128-head tiles, bf16 output, lambda calibrated for the
    target as the benchmark does (8 splits at 73 % and 50 %; 4 splits from its split sweep).  24
    seeded sequences against the oracle, every tile's mask against its critical values."""
    m = _lib()
    d = _mla_full_size()
    lam = _calibrated_lambda(m, d, splits=splits, target=target, tile_rows=128)
    res = _run(m, d, splits=splits, lam=lam, tile_rows=128, out_dtype=torch.bfloat16)
    sp = _check_whole_mask(res, oracle.ln_threshold(lam=lam), target)
    tiles = _seeded_tiles(64, 1, 1, 22, synth.config_seed(5), must=[(0, 0, 0), (63, 0, 0)])
    rep = _compare(d, res, splits=splits, lam=lam, tiles=tiles, tile_rows=128, out_bf16=True)
    print(f"S={splits} lambda={lam:.6g} sparsity {sp:.4f}; {rep}")


def test_latent_mla_full_size_redo_with_splits():
    """The 128-head latent kernel's redo path at full size and in the benchmark's launch (8 splits):
    in four sequences a key inside a split, past that split's first block, gets a scaled logit of +60
    (against a first-block maximum near +10), so those splits raise their reference max and start
    over; at lambda = 0 every sequence still matches the oracle and nothing is skipped."""
    m = _lib()
    d = _mla_full_size()
    scale = 1.0 / math.sqrt(576)
    planted = {3: 4096 + 700, 17: 2 * 4096 + 64 * 9 + 5, 40: 7 * 4096 + 4095, 63: 5 * 4096 + 2000}
    for b, key in planted.items():
        pid = int(d.block_table[b, key // d.page_size])
        d.k_cache[pid, 0, key % d.page_size, 574] = 60.0 / scale   # the sink channel: q = 1 there
    res = _run(m, d, splits=8, lam=0.0, tile_rows=128, out_dtype=torch.float32)
    _check_whole_mask(res, -math.inf, 0.0)
    tiles = sorted({(b, 0, 0) for b in planted} | {(0, 0, 0), (30, 0, 0)})
    rep = _compare(d, res, splits=8, lam=0.0, tiles=tiles, tile_rows=128)
    print(rep)
    assert rep.skipped == 0


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


@pytest.mark.parametrize("T", [2, 4])
def test_multi_token_decode_full_size_at_benchmark_threshold(T):
    """The benchmarked multi-token launches: batch 32, 32 q / 8 kv heads, d = 128, context 32768, the
    last T positions of each sequence as queries, tiles of T tokens x 4 heads, 8 splits, bf16 output,
    lambda calibrated for 73 % as the benchmark does; 24 seeded tiles against the oracle, every
    tile's mask against its critical values."""
    m = _lib()
    ctx = 32768
    d = synth.decode_inputs(batch=32, hq=32, hkv=8, ctx=ctx, d=128, seed=synth.config_seed(3, 2), device="cuda",
                            num_q_tokens=T)
    lam = _calibrated_lambda(m, d, splits=8, target=0.73, tile_rows=4)
    res = _run(m, d, splits=8, lam=lam, tile_rows=4, out_dtype=torch.bfloat16)
    sp = _check_whole_mask(res, oracle.ln_threshold(lam=lam), 0.73)
    tiles = _seeded_tiles(32, 8, 1, 22, synth.config_seed(3, 2) + T, must=[(0, 0, 0), (31, 7, 0)])
    rep = _compare(d, res, splits=8, lam=lam, tile_rows=4, tiles=tiles, out_bf16=True)
    print(f"T={T} lambda={lam:.6g} sparsity {sp:.4f}; {rep}")


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


@pytest.mark.parametrize("T,splits", [(2, 1), (2, 3), (4, 1), (4, 5)])
@pytest.mark.parametrize("a", [0.0, 4.0])
@pytest.mark.parametrize("rows", [64, 128])
def test_multi_token_latent_decode(T, splits, a, rows):
    """T query tokens per sequence on the latent cache (128 heads on one 576-channel latent head, V =
    the first 512 channels): tiles of 64 or 128 rows = T tokens x rows / T heads (the 64-row and the
    128-row kernels), each token seeing keys up to seq_len - T + t; ragged lengths including
    sequences no longer than T, NaN-poisoned spare pages."""
    m = _lib()
    lens = [700, 64, T + 1, 333, T]
    d = synth.decode_inputs(batch=len(lens), hq=128, hkv=1, ctx=None, d=576, dv=512, seq_lens=lens, seed=90 + T,
                            device="cuda", latent=True, num_q_tokens=T)
    tr = rows // T
    res = _run(m, d, splits=splits, a=a, tile_rows=tr)
    rep = _compare(d, res, splits=splits, a=a, tile_rows=tr)
    print(f"T={T} S={splits} a={a}: {rep}")
    if a == 0.0:
        assert rep.skipped == 0


@pytest.mark.parametrize("T,rows", [(2, 128), (4, 128), (2, 64)])
def test_multi_token_latent_decode_full_size_at_benchmark_threshold(T, rows):
    """The benchmarked multi-token latent launch: batch 64, 128 heads on one latent head, context
    32768, the last T positions of each sequence as queries, 128-row tiles (T tokens x 128 / T heads;
    the benchmark's choice) or 64-row tiles, 8 splits, bf16 output, lambda calibrated for 73 % as the
    benchmark does; 20 seeded tiles against the oracle, every tile's mask against its critical
    values."""
    m = _lib()
    d = synth.decode_inputs(batch=64, hq=128, hkv=1, ctx=32768, d=576, dv=512, seed=synth.config_seed(5, T),
                            device="cuda", latent=True, num_q_tokens=T)
    tr = rows // T
    lam = _calibrated_lambda(m, d, splits=8, target=0.73, tile_rows=tr)
    res = _run(m, d, splits=8, lam=lam, tile_rows=tr, out_dtype=torch.bfloat16)
    sp = _check_whole_mask(res, oracle.ln_threshold(lam=lam), 0.73)
    tiles = _seeded_tiles(64, 1, 128 // tr, 18, synth.config_seed(5, T), must=[(0, 0, 0), (63, 0, 128 // tr - 1)])
    rep = _compare(d, res, splits=8, lam=lam, tile_rows=tr, tiles=tiles, out_bf16=True)
    print(f"T={T} lambda={lam:.6g} sparsity {sp:.4f}; {rep}")

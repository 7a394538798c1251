"""GPU parity of blasst_prefill (through the C ABI) against the fp64 oracle."""

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


def _run(m, q, k, v, *, causal, bq, bk, splits, lam=None, a=None, out_dtype=torch.float32, stats_only=False):
    B, Hq, Lq, D = q.shape
    Lk, Dv = k.shape[2], v.shape[3]
    nqt, nkb = -(-Lq // bq), -(-Lk // bk)
    dev = q.device
    o = None if stats_only else torch.full((B, Hq, Lq, Dv), float("nan"), dtype=out_dtype, device=dev)
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=dev)
    mask = torch.full((B, Hq, nqt, nkb), 7, dtype=torch.uint8, device=dev)
    crit = torch.full((B, Hq, nqt, nkb), 12345.0, dtype=torch.float32, device=dev)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    hcnt = torch.zeros(B, Hq, 2, dtype=torch.int64, device=dev)
    m.blasst_prefill(q, k, v, o, causal=causal, block_q=bq, block_k=bk, num_splits=splits, lam=lam, a=a,
                     lse=None if stats_only else lse, skip_mask=mask, crit=crit, counters=cnt,
                     head_counters=hcnt, stats_only=stats_only)
    torch.cuda.synchronize()
    _check_counters(mask, cnt, hcnt)
    return o, lse, mask, crit, cnt, hcnt


def _check_counters(mask, cnt, hcnt):
    """The global and per-head counters are exactly the mask's counts (bit-exact integer work)."""
    mh = mask.cpu().numpy()
    h = hcnt.cpu().numpy()
    assert np.array_equal(h[..., 0], (mh != 2).sum(axis=(2, 3))), "per-head live counts differ from the mask"
    assert np.array_equal(h[..., 1], (mh == 1).sum(axis=(2, 3))), "per-head skip counts differ from the mask"
    assert int(cnt[0]) == int(h[..., 0].sum()) and int(cnt[1]) == int(h[..., 1].sum())


def _compare_all(q, k, v, res, *, causal, bq, bk, splits, ln_lam, tiles=None, out_bf16=False):
    o, lse, mask, crit, cnt, _ = res
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    B, Hq, Lq, _ = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    nqt = mh.shape[2]
    rep = Report()
    full = tiles is None
    if full:
        tiles = [(b, h, t) for b in range(B) for h in range(Hq) for t in range(nqt)]
        qh, kh, vh = host64(q), host64(k), host64(v)
    cache = {}
    for (b, h, t) in tiles:
        r0, r1 = t * bq, min((t + 1) * bq, Lq)
        if full:
            qt_, kt_, vt_, bb, hh, tt = qh, kh, vh, b, h, t
        else:
            # host copies of this head's queries and of its kv head only (kept while consecutive tiles
            # share them)
            if (b, h) not in cache:
                kv = cache.get("kv") if cache.get("kv_id") == (b, h // G) else \
                    (host64(k[b:b + 1, h // G:h // G + 1]), host64(v[b:b + 1, h // G:h // G + 1]))
                cache = {(b, h): host64(q[b:b + 1, h:h + 1]), "kv": kv, "kv_id": (b, h // G)}
            qt_ = cache[(b, h)]
            kt_, vt_ = cache["kv"]
            bb, hh, tt = 0, 0, t
        kw = dict(causal=causal, block_q=bq, block_k=bk, num_splits=splits, ln_lam=ln_lam)
        ref = oracle.prefill_tile(qt_, kt_, vt_, bb, hh, tt, **kw)
        gpu_o = None if o is None else host64(o[b, h, r0:r1])
        gpu_l = None if o is None else lse[b, h, r0:r1].cpu().double().numpy()
        check_tile(rep, ref, mh[b, h, t], ch[b, h, t], ln_lam,
                   lambda f: oracle.prefill_tile(qt_, kt_, vt_, bb, hh, tt, force=f, **kw),
                   gpu_o, gpu_l, out_bf16=out_bf16)
    # counters agree with the mask
    live = int((mh != 2).sum())
    assert int(cnt[0]) == live and int(cnt[1]) == int((mh == 1).sum())
    return rep


@pytest.mark.parametrize("a", [0.0, 0.5, 2.0, 8.0])
def test_tiny_mha_fp32(a):
    """fp32 MHA prefill, batch 1, 2 heads, L = 512, d = 64, causal, 64 x 64 blocks, lambda = a / L."""
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=2, hkv=2, L=512, d=64, dtype=torch.float32, block_k=64,
                               window=False, seed=synth.config_seed(1), device="cuda")
    res = _run(m, inp.q, inp.k, inp.v, causal=True, bq=64, bk=64, splits=1, a=a)
    ln_lam = oracle.ln_threshold(a=a, L=512)
    rep = _compare_all(inp.q, inp.k, inp.v, res, causal=True, bq=64, bk=64, splits=1, ln_lam=ln_lam)
    print(f"a={a}: {rep}")
    assert rep.max_err < 1e-4
    if a == 0.0:
        assert rep.skipped == 0


@pytest.mark.parametrize("a", [0.0, 1.0, 4.0, 16.0])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gqa_bf16_ragged(a, out_dtype):
    """bf16 GQA prefill with a ragged last tile (L = 600, 128 x 128 blocks), two sequences."""
    m = _lib()
    L = 600
    inp = synth.prefill_inputs(batch=2, hq=4, hkv=2, L=L, d=128, block_k=128, window=True, seed=77,
                               device="cuda")
    res = _run(m, inp.q, inp.k, inp.v, causal=True, bq=128, bk=128, splits=1, a=a, out_dtype=out_dtype)
    rep = _compare_all(inp.q, inp.k, inp.v, res, causal=True, bq=128, bk=128, splits=1,
                       ln_lam=oracle.ln_threshold(a=a, L=L), out_bf16=out_dtype == torch.bfloat16)
    print(f"a={a} {out_dtype}: {rep}")


@pytest.mark.parametrize("D,blk", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_shapes_splits_and_offsets(D, blk, causal):
    """Lq != Lk (bottom-right causal), num_splits = 3, every head-dim / block-size kernel."""
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=1, L=700, d=D, block_k=blk, window=True, seed=5,
                               device="cuda", Lq=250)
    lam = 0.004
    res = _run(m, inp.q, inp.k, inp.v, causal=causal, bq=blk, bk=blk, splits=3, lam=lam)
    rep = _compare_all(inp.q, inp.k, inp.v, res, causal=causal, bq=blk, bk=blk, splits=3,
                       ln_lam=math.log(lam))
    print(rep)


@pytest.mark.parametrize("D,blk", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv,lam", [(3, 3, 0.004), (6, 2, 0.004), (3, 3, 0.0)])
def test_odd_groups_query_tile_pairs(D, blk, causal, hq, hkv, lam):
    """GQA groups of odd size (MHA among them) put two query tiles of one head in a workgroup: every
    head-dim / block-size kernel, Lq != Lk with an odd number of query tiles (the last pair's second
    tile is empty), 3 splits, outputs, masks, critical values and counters against the oracle; the
    stats-only pass gives the same masks and critical values."""
    m = _lib()
    inp = synth.prefill_inputs(batch=2, hq=hq, hkv=hkv, L=700, d=D, block_k=blk, window=True, seed=6,
                               device="cuda", Lq=300)
    res = _run(m, inp.q, inp.k, inp.v, causal=causal, bq=blk, bk=blk, splits=3, lam=lam)
    assert res[2].shape[2] % 2 == 1
    rep = _compare_all(inp.q, inp.k, inp.v, res, causal=causal, bq=blk, bk=blk, splits=3,
                       ln_lam=math.log(lam) if lam > 0 else -math.inf)
    st = _run(m, inp.q, inp.k, inp.v, causal=causal, bq=blk, bk=blk, splits=3, lam=lam, stats_only=True)
    assert torch.equal(st[2], res[2])
    assert np.array_equal(st[3].cpu().numpy(), res[3].cpu().numpy(), equal_nan=True)   # NaN: not live
    print(rep)


def test_strided_layout_matches_contiguous():
    """q/k/v/o given as [B, L, H, D] storage viewed as [B, H, L, D] (token-major) give the same result."""
    m = _lib()
    inp = synth.prefill_inputs(batch=2, hq=8, hkv=2, L=384, d=128, block_k=128, seed=9, device="cuda")
    kw = dict(causal=True, bq=128, bk=128, splits=1, lam=0.01)
    ref = _run(m, inp.q, inp.k, inp.v, **kw)
    qs = inp.q.transpose(1, 2).contiguous().transpose(1, 2)
    ks = inp.k.transpose(1, 2).contiguous().transpose(1, 2)
    vs = inp.v.transpose(1, 2).contiguous().transpose(1, 2)
    got = _run(m, qs, ks, vs, **kw)
    assert torch.equal(ref[2], got[2])
    assert torch.equal(ref[0], got[0])


def test_stats_only_matches_full_pass():
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=8, hkv=2, L=1024, d=128, block_k=128, seed=10, device="cuda")
    kw = dict(causal=True, bq=128, bk=128, splits=1, lam=0.003)
    full = _run(m, inp.q, inp.k, inp.v, **kw)
    st = _run(m, inp.q, inp.k, inp.v, stats_only=True, **kw)
    assert torch.equal(full[2], st[2])
    assert torch.allclose(full[3], st[3], rtol=0, atol=0, equal_nan=True)
    assert torch.equal(full[4], st[4])
    assert torch.equal(full[5], st[5])


def benchmark_lambda(m, inp, target):
    """lambda for a target sparsity, set the way the benchmark sets it: a stats-only pass (critical
    values of every tile), the benchmark's seeded 8-tile (1024-row) calibration sample, and the
    library's quantile of that sample's critical values."""
    import bench
    if target == 0.0:
        return 0.0
    B, Hq, L, _ = inp.q.shape
    nqt = -(-L // 128)
    crit = torch.empty(B, Hq, nqt, -(-inp.k.shape[2] // 128), dtype=torch.float32, device=inp.q.device)
    m.blasst_prefill(inp.q, inp.k, inp.v, None, causal=True, block_q=128, block_k=128, lam=0.0, crit=crit,
                     stats_only=True)
    torch.cuda.synchronize()
    sample = torch.stack([crit[0, h, t] for h, t in bench.stratified_tiles(torch, nqt, Hq, bench.CALIB_TILES, 4242)])
    return math.exp(m.blasst_calib_quantile(sample.cpu().numpy(), target))


def seeded_prefill_tiles(Hq, nqt, count, seed):
    """Tiles of the last, a middle and the first causal level of a few heads, plus `count` seeded
    picks over all (head, query tile)."""
    rng = np.random.default_rng(seed)
    must = {(0, nqt - 1), (Hq - 1, nqt - 1), (Hq // 2, nqt // 2), (Hq // 3, nqt // 2 - 1), (1, 0), (Hq - 2, 1)}
    picks = {(int(h), int(t)) for h, t in zip(rng.integers(0, Hq, count), rng.integers(0, nqt, count))}
    return sorted((0, h, t) for h, t in must | picks)


def check_full_size_prefill(m, inp, lam, target, *, seed, count=20):
    """Runs the benchmark's prefill launch (bf16 out) at lambda and checks it: the sampled tiles against
    the oracle (mask, critical values, O, LSE), every tile's mask against its critical values, the
    counters against the mask, and the achieved sparsity against the calibration target."""
    B, Hq, L, _ = inp.q.shape
    res = _run(m, inp.q, inp.k, inp.v, causal=True, bq=128, bk=128, splits=1, lam=lam, out_dtype=torch.bfloat16)
    o, lse, mask, crit, cnt, _ = res
    ln_lam = oracle.ln_threshold(lam=lam)
    mh, ch = mask.cpu().numpy(), crit.cpu().numpy()
    live = mh != 2
    nqt = L // 128
    assert live.sum() == B * Hq * nqt * (nqt + 1) // 2
    decided = np.where(live, np.where(ch < ln_lam, 1, 0), 2)
    band = live & (np.abs(ch - ln_lam) < 1e-3)
    assert np.array_equal(decided[~band], mh[~band])
    sp = float((mh == 1).sum()) / live.sum()
    if target == 0.0:
        assert sp == 0.0
    elif target is not None:
        assert abs(sp - target) < 0.05, f"sparsity {sp} at target {target}"
    tiles = seeded_prefill_tiles(Hq, nqt, count, seed)
    rep = _compare_all(inp.q, inp.k, inp.v, res, causal=True, bq=128, bk=128, splits=1, ln_lam=ln_lam, tiles=tiles,
                       out_bf16=True)
    return sp, len(tiles), rep


@pytest.mark.parametrize("target", [0.75, 0.5, 0.0])
def test_llama8b_gqa_32k_at_benchmark_thresholds(target):
    """The benchmarked prefill launch (32 q / 8 kv heads, d = 128, L = 32768, causal, 128 x 128 blocks,
    bf16 in/out, on the benchmark's own seeded inputs) at lambda calibrated for 75 % and 50 % sparsity
    exactly as the benchmark does it, and at lambda = 0: 26 tiles against the oracle, every tile's
    mask against its critical values."""
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=32, hkv=8, L=32768, d=128, block_k=128, window=True,
                               seed=synth.config_seed(2), device="cuda")
    lam = benchmark_lambda(m, inp, target)
    sp, n, rep = check_full_size_prefill(m, inp, lam, target, seed=int(target * 100) + 7)
    print(f"lambda={lam:.6g} sparsity {sp:.4f} over all tiles; {n} tiles vs oracle: {rep}")


def test_no_decision_mode_equals_lambda_zero():
    """Threshold mode NONE (the variant without any decision logic, for measuring what the decisions
    cost) gives the same bits as lambda = 0 and the oracle's dense attention."""
    import long_context_online_amd as m
    m.lib()
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=640, d=128, block_k=128, window=True, seed=77,
                               device="cuda")
    outs = []
    for kw in ({"lam": 0.0}, {"no_decision": True}):
        o = torch.empty(1, 4, 640, 128, dtype=torch.float32, device="cuda")
        lse = torch.empty(1, 4, 640, dtype=torch.float32, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        m.blasst_prefill(inp.q, inp.k, inp.v, o, causal=True, block_q=128, block_k=128, lse=lse, counters=cnt, **kw)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu(), cnt.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert int(outs[1][2][1]) == 0 and int(outs[1][2][0]) == int(outs[0][2][0])
    q, k, v = host64(inp.q), host64(inp.k), host64(inp.v)
    from oracle.blasst_oracle import causal_visible
    ref = oracle.softmax_attention(q[0, 1], k[0, 0], v[0, 0], causal_visible(np.arange(640), 640, 640, 640),
                                  1 / math.sqrt(128))
    assert np.max(np.abs(outs[1][0][0, 1].double().numpy() - ref[0])) < 1e-2


@pytest.mark.parametrize("dtype,blk", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_heterogeneous_heads_per_head_sparsity(dtype, blk):
    """Heads of very different peakedness (head strengths 0.25 ... 1.75) under ONE threshold: every
    tile matches the oracle, the per-head counters match the oracle's per-head counts outside the
    decision band, and the per-head sparsities spread out, more peaked heads skipping more."""
    m = _lib()
    L, hq = 768, 8
    strength = [0.25, 1.75, 0.5, 1.5, 0.75, 1.25, 1.0, 0.35]
    inp = synth.prefill_inputs(batch=1, hq=hq, hkv=2, L=L, d=128 if dtype == torch.bfloat16 else 64,
                               dtype=dtype, block_k=blk, window=True, seed=31, device="cuda",
                               head_strength=strength)
    lam = 0.01
    res = _run(m, inp.q, inp.k, inp.v, causal=True, bq=blk, bk=blk, splits=1, lam=lam)
    rep = _compare_all(inp.q, inp.k, inp.v, res, causal=True, bq=blk, bk=blk, splits=1, ln_lam=math.log(lam))
    h = res[5].cpu().numpy()[0]
    sp = h[:, 1] / h[:, 0]
    print(f"{rep}; per-head sparsity by strength: " +
          ", ".join(f"{c}:{s:.3f}" for c, s in sorted(zip(strength, sp))))
    order = np.argsort(strength)
    assert sp[order[-1]] > sp[order[0]] + 0.2


@pytest.mark.parametrize("splits", [1, 2])
def test_more_queries_than_keys(splits):
    """Lq = 500 queries over Lk = 300 keys, bottom-right causal: the first 200 rows see no key (O = 0,
    LSE = -inf), the rest match the oracle; the tile that straddles the boundary votes with rows
    that see nothing."""
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=500, d=128, block_k=128, window=True, seed=61,
                               device="cuda")
    k = inp.k[:, :, :300].contiguous()
    v = inp.v[:, :, :300].contiguous()
    res = _run(m, inp.q, k, v, causal=True, bq=128, bk=128, splits=splits, lam=0.01)
    o, lse = res[0], res[1]
    assert torch.all(o[:, :, :200] == 0) and torch.all(lse[:, :, :200] == float("-inf"))
    rep = _compare_all(inp.q, k, v, res, causal=True, bq=128, bk=128, splits=splits, ln_lam=math.log(0.01))
    print(rep)


@pytest.mark.parametrize("lam", [0.0, 0.01])
def test_late_large_logit_raises_the_reference_with_probabilities_pending(lam):
    """A key of block 3 gets a scaled logit of about +40 for every query that sees it (first-block
    maxima are near +10), so the accumulation reference of those rows jumps at block 3 while block 2's
    probabilities are still waiting for their P.V product: the kernel must rescale O, the row sums and
    those pending probabilities alike.  Every tile against the oracle, fp32 and bf16 output."""
    m = _lib()
    L = 640
    for out_dtype in (torch.float32, torch.bfloat16):
        inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=L, d=128, block_k=128, window=True, seed=91,
                                   device="cuda")
        scale = 1.0 / math.sqrt(128)
        inp.k[0, :, 3 * 128 + 17, 126] = 40.0 / scale   # channel D - 2 carries the sink: q = 1 there
        res = _run(m, inp.q, inp.k, inp.v, causal=True, bq=128, bk=128, splits=1, lam=lam, out_dtype=out_dtype)
        rep = _compare_all(inp.q, inp.k, inp.v, res, causal=True, bq=128, bk=128, splits=1,
                           ln_lam=oracle.ln_threshold(lam=lam), out_bf16=out_dtype == torch.bfloat16)
        print(f"lambda={lam} {out_dtype}: {rep}")


@pytest.mark.parametrize("D,blk", [(128, 128), (64, 64)])
def test_v_staging_every_block_gives_the_same_bits(D, blk):
    """Staging V for every live block (the pages' policy) instead of only for kept blocks changes
    which bytes are loaded, not what is computed: outputs, LSE, masks and counters are bit-identical
    at a threshold that skips, and the oracle agrees."""
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=900, d=D, block_k=blk, window=True, seed=95, device="cuda")
    outs = []
    for vs in (m.blasst.V_KEPT, m.blasst.V_ALL):
        o = torch.full((1, 4, 900, D), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.empty(1, 4, 900, dtype=torch.float32, device="cuda")
        mask = torch.empty(1, 4, -(-900 // blk), -(-900 // blk), dtype=torch.uint8, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        m.blasst_prefill(inp.q, inp.k, inp.v, o, causal=True, block_q=blk, block_k=blk, lam=0.01, lse=lse,
                         skip_mask=mask, counters=cnt, v_staging=vs)
        torch.cuda.synchronize()
        outs.append((o, lse, mask, cnt))
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x, y)
    assert int(outs[0][3][1]) > 0
    res = _run(m, inp.q, inp.k, inp.v, causal=True, bq=blk, bk=blk, splits=1, lam=0.01)
    assert torch.equal(res[0], outs[0][0])
    print(_compare_all(inp.q, inp.k, inp.v, res, causal=True, bq=blk, bk=blk, splits=1, ln_lam=math.log(0.01)))

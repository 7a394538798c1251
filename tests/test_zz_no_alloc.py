"""blasst_decode_no_alloc (decode for callers that cannot allocate: its split partials live in the
library's per-GPU scratch array) against blasst_decode with a caller workspace, through the C ABI:
the same bits, on calls in a row whose later inputs are smaller than the first."""

import ctypes

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _decode_both(m, d, *, splits, tile_rows=0, out_dtype=torch.bfloat16, **thr):
    from long_context_online_amd import blasst as bl
    rows = tuple(d.q.shape[:-1])
    Hkv = d.k_cache.shape[1]
    G = d.q.shape[-2] // Hkv
    tr = G if tile_rows == 0 else tile_rows
    nkb = -(-(d.block_table.shape[1] * d.page_size) // 64)
    out = []
    for no_alloc in (False, True):
        o = torch.full(rows + (d.head_dim_v,), float("nan"), dtype=out_dtype, device="cuda")
        lse = torch.full(rows, float("nan"), dtype=torch.float32, device="cuda")
        mask = torch.full((d.q.shape[0], Hkv, G // tr, nkb), 7, dtype=torch.uint8, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        kw = dict(page_size=d.page_size, block_k=64, num_splits=splits, tile_rows=tile_rows,
                  head_dim_v=d.head_dim_v, lse=lse, skip_mask=mask, counters=cnt, **thr)
        if no_alloc:
            p = bl.decode_params(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, **kw)
            st = m.lib().blasst_decode_no_alloc(ctypes.byref(p), bl._stream(None))
            assert st == 0, m.lib().blasst_last_error()
        else:
            n = m.blasst_decode_workspace_size(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, **kw)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
            m.blasst_decode(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, o, workspace=ws, **kw)
        torch.cuda.synchronize()
        out.append((o, lse, mask, cnt))
    (o0, l0, m0, c0), (o1, l1, m1, c1) = out
    assert torch.isfinite(o0.float()).all()
    assert torch.equal(o0, o1) and torch.equal(l0, l1) and torch.equal(m0, m1) and torch.equal(c0, c1)
    return int(c0[1]) / int(c0[0])


def test_no_alloc_decode_equals_workspace_decode():
    import long_context_online_amd as m
    m.lib()
    # 1: the larger call (GQA, batch 8, 16 splits)
    d = synth.decode_inputs(batch=8, hq=32, hkv=8, ctx=5000, d=128, seed=81, device="cuda")
    sp1 = _decode_both(m, d, splits=16, lam=0.01)
    # 2: smaller, ragged, another split count and threshold mode, fp32 output
    d = synth.decode_inputs(batch=3, hq=16, hkv=4, ctx=None, d=128, seq_lens=[700, 33, 1], seed=82, device="cuda")
    sp2 = _decode_both(m, d, splits=4, a=2.0, out_dtype=torch.float32)
    # 3: smaller again, multi-token tiles
    d = synth.decode_inputs(batch=2, hq=16, hkv=4, ctx=300, d=128, seed=83, device="cuda", num_q_tokens=3)
    sp3 = _decode_both(m, d, splits=3, lam=0.02, tile_rows=4)
    # 4: latent (MLA-shaped) decode through the same scratch
    d = synth.decode_inputs(batch=2, hq=128, hkv=1, ctx=None, d=576, dv=512, seq_lens=[1500, 90], seed=84,
                            device="cuda", latent=True)
    sp4 = _decode_both(m, d, splits=4, lam=0.05, tile_rows=128)
    print(f"sparsity of the four calls: {sp1:.3f} {sp2:.3f} {sp3:.3f} {sp4:.3f}")

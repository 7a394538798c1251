"""GPU parity of blasst_prefill_backward (through the C ABI) against the fp64 backward oracle.

The forward runs on the GPU first (fp32 output, fp32 LSE, skip mask); the backward takes those, and
the oracle differentiates softmax attention over the kept keys with the same mask.  Tolerance: the
gradients go through bf16 operands (P and dS, a relative rounding of at most 2^-8 each, summed over
many terms with fp32 accumulation), so elementwise |GPU - oracle| <= 1e-2 * max(1, max|oracle|) of
each tensor is the bar (plus half a bf16 ulp of the value for bf16 gradients); errors are printed.
With the forward's output in bf16, D = rowsum(dO * O) carries O's rounding, and the bar adds the bound
that error propagates to (derived in test_bf16_forward_output_within_the_propagated_bound)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import backward as bw
from oracle import KEPT, SKIPPED
from tests.gpu_util import host64

pytestmark = pytest.mark.gpu

REL = 1e-2


def _lib():
    import long_context_online_amd as m
    m.lib()
    return m


def _forward(m, inp, *, causal, lam, o_dtype=torch.float32):
    q, k, v = inp.q, inp.k, inp.v
    B, Hq, Lq, D = q.shape
    Lk = k.shape[2]
    nqt, nkb = -(-Lq // 128), -(-Lk // 128)
    o = torch.empty(B, Hq, Lq, D, dtype=o_dtype, device="cuda")
    lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device="cuda")
    mask = torch.empty(B, Hq, nqt, nkb, dtype=torch.uint8, device="cuda")
    m.blasst_prefill(q, k, v, o, causal=causal, block_q=128, block_k=128, lam=lam, lse=lse, skip_mask=mask)
    return o, lse, mask


def _backward(m, inp, o, lse, dout, mask, *, causal, grad_dtype=torch.float32):
    q, k, v = inp.q, inp.k, inp.v
    dq = torch.full(q.shape, float("nan"), dtype=grad_dtype, device="cuda")
    dk = torch.full(k.shape, float("nan"), dtype=grad_dtype, device="cuda")
    dv = torch.full(v.shape, float("nan"), dtype=grad_dtype, device="cuda")
    kw = dict(causal=causal, skip_mask=mask)
    n = m.blasst_prefill_backward_workspace_size(q, k, v, o, dout, lse, dq, dk, dv, **kw)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    m.blasst_prefill_backward(q, k, v, o, dout, lse, dq, dk, dv, workspace=ws, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(got, want, name, grad_bf16=False):
    g = host64(got)
    assert np.all(np.isfinite(g)), f"{name}: non-finite gradient"
    err = np.abs(g - want)
    scale = max(1.0, float(np.max(np.abs(want))))
    tol = REL * scale + (np.abs(want) * 2.0 ** -8 if grad_bf16 else 0.0)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{name}: max err {err.max():.3g} (scale {scale:.3g}) at {bad[:5].tolist()}"
    return float(err.max()) / scale


def _dout(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)


@pytest.mark.parametrize("lam", [0.0, 0.02, 0.3])
@pytest.mark.parametrize("hq,hkv,causal", [(4, 2, True), (3, 1, True), (2, 2, True), (3, 1, False), (2, 2, False)])
def test_backward_matches_oracle_ragged(lam, hq, hkv, causal):
    """GQA / MQA with an odd group / MHA, L = 600 (a ragged last tile and block, an odd number of query
    tiles: odd groups pair two query tiles of one head and leave the last pair's second tile empty),
    two sequences, the forward's mask at thresholds from dense to very sparse."""
    m = _lib()
    L = 600
    inp = synth.prefill_inputs(batch=2, hq=hq, hkv=hkv, L=L, d=128, block_k=128, window=True, seed=80 + hq,
                               device="cuda")
    o, lse, mask = _forward(m, inp, causal=causal, lam=lam)
    dout = _dout(o.shape, 5)
    dq, dk, dv = _backward(m, inp, o, lse, dout, mask, causal=causal)
    mh = mask.cpu().numpy()
    ref = bw.prefill_backward(host64(inp.q), host64(inp.k), host64(inp.v), host64(dout), mh, causal=causal,
                              block_q=128, block_k=128)
    errs = [_check(dq, ref["dq"], "dq"), _check(dk, ref["dk"], "dk"), _check(dv, ref["dv"], "dv")]
    skipped = int((mh == SKIPPED).sum())
    print(f"lam={lam} hq={hq} hkv={hkv} causal={causal}: skipped {skipped} rel errs dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    if lam == 0.3:
        assert skipped > 0


@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
def test_backward_noncausal_lq_ne_lk_and_bf16_gradients(grad_dtype):
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=700, d=128, block_k=128, window=True, seed=91,
                               device="cuda", Lq=300)
    for causal in (False, True):
        o, lse, mask = _forward(m, inp, causal=causal, lam=0.05)
        dout = _dout(o.shape, 6)
        dq, dk, dv = _backward(m, inp, o, lse, dout, mask, causal=causal, grad_dtype=grad_dtype)
        ref = bw.prefill_backward(host64(inp.q), host64(inp.k), host64(inp.v), host64(dout), mask.cpu().numpy(),
                                  causal=causal, block_q=128, block_k=128)
        bf = grad_dtype == torch.bfloat16
        errs = [_check(dq, ref["dq"], "dq", bf), _check(dk, ref["dk"], "dk", bf), _check(dv, ref["dv"], "dv", bf)]
        print(f"causal={causal} {grad_dtype}: rel errs {errs}")


def test_bf16_forward_output_within_the_propagated_bound():
    """O stored in bf16 (the usual training setup) enters only D_i = sum_d dO_id O_id.  Rounding O
    to bf16 moves D_i by at most dD_i = 2^-8 sum_d |dO_id| |O_id|, which moves dS_ik = scale P_ik
    (dP_ik - D_i) by scale P_ik dD_i, hence dQ_id by at most scale dD_i max_k |K_kd| (P sums to 1
    over a row) and dK_kd by at most scale sum_i P_ik dD_i |q_id|; dV does not depend on D.  The bar
    is the fp32-output bar plus these bounds, computed from the oracle's O and P."""
    m = _lib()
    L = 600
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=L, d=128, block_k=128, window=True, seed=93, device="cuda")
    o, lse, mask = _forward(m, inp, causal=True, lam=0.02, o_dtype=torch.bfloat16)
    dout = _dout(o.shape, 9)
    dq, dk, dv = _backward(m, inp, o, lse, dout, mask, causal=True)
    mh = mask.cpu().numpy()
    q, k, v, do = host64(inp.q), host64(inp.k), host64(inp.v), host64(dout)
    ref = bw.prefill_backward(q, k, v, do, mh, causal=True, block_q=128, block_k=128)
    scale = 1 / math.sqrt(128)
    keep = bw.kept_keys(mh, L, L, 128, 128, True)
    dD = 2.0 ** -8 * np.sum(np.abs(do) * np.abs(ref["o"]), axis=-1)                    # [1, Hq, L]
    G = 2
    tq = np.zeros_like(q)
    tk = np.zeros_like(k)
    for h in range(4):
        g = h // G
        s = scale * q[0, h] @ k[0, g].T
        P = np.where(keep[0, h], np.exp(s - np.where(np.isfinite(ref["lse"][0, h]), ref["lse"][0, h], 0)[:, None]), 0)
        tq[0, h] = scale * dD[0, h][:, None] * np.max(np.abs(k[0, g]), axis=0)[None, :]
        tk[0, g] += scale * (P * dD[0, h][:, None]).T @ np.abs(q[0, h])
    for got, want, extra, name in ((dq, ref["dq"], tq, "dq"), (dk, ref["dk"], tk, "dk"), (dv, ref["dv"], 0.0, "dv")):
        g64 = host64(got)
        err = np.abs(g64 - want)
        tol = REL * max(1.0, float(np.max(np.abs(want)))) + extra
        assert np.all(err <= tol), f"{name}: {float((err - tol).max())} over the bound"
        print(f"{name}: max err {err.max():.3g}, max bound {np.max(tol):.3g}")


def test_null_mask_is_the_all_kept_mask():
    """skip_mask = NULL (dense backward) gives the bits of the backward with a lambda = 0 mask."""
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=512, d=128, block_k=128, seed=92, device="cuda")
    o, lse, mask = _forward(m, inp, causal=True, lam=0.0)
    dout = _dout(o.shape, 7)
    r1 = _backward(m, inp, o, lse, dout, mask, causal=True)
    r2 = _backward(m, inp, o, lse, dout, None, causal=True)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_llama8b_gqa_32k_backward_sampled_and_invariants():
    """The benchmark's prefill shape (32 q / 8 kv heads, d = 128, L = 32768, causal) at a sparse
    threshold: sampled dQ rows against the oracle row by row; the softmax-Jacobian invariants (dK sums
    to zero over each kv head's keys, dV sums to the sum of dO over the rows of the group); keys in
    blocks that no tile of the group kept have exactly zero dK and dV.

    A row of dQ sums up to 32768 terms dS_ik K_k whose dS goes through bf16, so its bar is the
    rounding bound of that sum, 1e-3 + 2^-8 * sum_k |dS_ik| |K_kd| (dS from the closed form in fp64),
    rather than a fraction of the row's own (small) magnitude."""
    m = _lib()
    L = 32768
    inp = synth.prefill_inputs(batch=1, hq=32, hkv=8, L=L, d=128, block_k=128, window=True,
                               seed=synth.config_seed(2), device="cuda")
    o, lse, mask = _forward(m, inp, causal=True, lam=0.02)
    dout = _dout(o.shape, 8)
    dq, dk, dv = _backward(m, inp, o, lse, dout, mask, causal=True)
    mh = mask.cpu().numpy()
    assert np.all(np.isfinite(dq.cpu().numpy())) and np.all(np.isfinite(dk.cpu().numpy()))
    # sampled dQ rows
    for h, rows in ((0, [0, 1, 127, 128, 4000]), (13, [32767, 20000, 17]), (31, [9999, 30000])):
        g = h // 4
        rows = np.array(rows)
        qh = host64(inp.q[:, h:h + 1])
        kh, vh = host64(inp.k[:, g:g + 1]), host64(inp.v[:, g:g + 1])
        dh = host64(dout[:, h:h + 1])
        want = bw.dq_rows(qh, kh, vh, dh, mh[:, h:h + 1], 0, 0, rows, causal=True, block_q=128, block_k=128)
        got = dq[0, h, rows].double().cpu().numpy()
        sc = 1 / math.sqrt(128)
        K, V = kh[0, 0], vh[0, 0]
        keep = bw.kept_keys(mh[:, h:h + 1], L, L, 128, 128, True)[0, 0, rows]
        s = np.where(keep, sc * qh[0, 0, rows] @ K.T, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        p /= p.sum(axis=1, keepdims=True)
        dp = dh[0, 0, rows] @ V.T
        ds = sc * p * (dp - np.sum(dh[0, 0, rows] * (p @ V), axis=1, keepdims=True))
        bound = 1e-3 + 2.0 ** -8 * (np.abs(ds) @ np.abs(K))
        err = np.abs(got - want)
        print(f"head {h} rows {rows.tolist()}: dq err {err.max():.3g}, bound there {bound.flat[err.argmax()]:.3g}")
        assert np.all(err <= bound)
    dk64 = dk.double()
    dv64 = dv.double()
    colsum = dk64.sum(dim=2).abs().max().item()
    assert colsum <= 1e-3 * dk64.abs().sum(dim=2).max().item(), colsum
    rows_with_keys = torch.isfinite(lse) & (lse > float("-inf"))
    want_dv = (dout.double() * rows_with_keys[..., None]).view(1, 8, 4, L, 128).sum(dim=(2, 3))
    err = (dv64.sum(dim=2) - want_dv).abs().max().item()
    assert err <= 1e-3 * want_dv.abs().max().item() + 1e-2, err
    kept_any = (mh == KEPT).reshape(1, 8, 4, 256, 256).any(axis=(2, 3))      # [1, Hkv, nkb]
    dead = np.argwhere(~kept_any[0])
    print(f"sparsity {(mh == SKIPPED).sum() / (mh != 2).sum():.3f}; key blocks no tile kept: {len(dead)}")
    for g, j in dead[:20]:
        assert torch.all(dk[0, g, j * 128:(j + 1) * 128] == 0) and torch.all(dv[0, g, j * 128:(j + 1) * 128] == 0)


def test_backward_more_queries_than_keys():
    """Lq = 500 over Lk = 300 (bottom-right causal): rows without keys get no gradient and add nothing."""
    m = _lib()
    inp = synth.prefill_inputs(batch=1, hq=4, hkv=2, L=500, d=128, block_k=128, window=True, seed=62,
                               device="cuda")

    class Cut:
        q = inp.q
        k = inp.k[:, :, :300].contiguous()
        v = inp.v[:, :, :300].contiguous()

    o, lse, mask = _forward(m, Cut, causal=True, lam=0.02)
    dout = _dout(o.shape, 10)
    dq, dk, dv = _backward(m, Cut, o, lse, dout, mask, causal=True)
    assert torch.all(dq[:, :, :200] == 0)
    ref = bw.prefill_backward(host64(Cut.q), host64(Cut.k), host64(Cut.v), host64(dout), mask.cpu().numpy(),
                              causal=True, block_q=128, block_k=128)
    errs = [_check(dq, ref["dq"], "dq"), _check(dk, ref["dk"], "dk"), _check(dv, ref["dv"], "dv")]
    print(f"rel errs {errs}")

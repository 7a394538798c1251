"""Helpers shared by the GPU parity tests: run the oracle on tiles and compare with the GPU."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle import KEPT, SKIPPED, NOT_LIVE

BAND = 1e-3          # |crit - ln(lambda)| below this: either decision is a correct result
O_TOL = 1e-2         # max abs error of outputs (fp32 output)
CRIT_TOL = 2e-3      # critical values: GPU fp32 vs oracle fp64


def bf16_half_ulp(x):
    """Half a bfloat16 ulp of |x| (elementwise), for bf16-output comparisons."""
    ax = np.maximum(np.abs(x), 1e-30)
    e = np.floor(np.log2(ax))
    return 2.0 ** (e - 8)


def host64(t):
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()


class Report:
    def __init__(self):
        self.in_band = 0
        self.flips = 0
        self.live = 0
        self.skipped = 0
        self.max_err = 0.0
        self.max_lse_err = 0.0
        self.max_crit_err = 0.0

    def __repr__(self):
        return (f"live={self.live} skipped={self.skipped} in_band={self.in_band} flips={self.flips} "
                f"max_err={self.max_err:.3g} max_lse_err={self.max_lse_err:.3g} max_crit_err={self.max_crit_err:.3g}")


def check_tile(rep: Report, ref: dict, gpu_mask, gpu_crit, ln_lam, rerun, gpu_o, gpu_lse=None,
               out_bf16=False):
    """Compares one tile.  ref: oracle result; rerun(force) re-runs the oracle with forced
    decisions.  Masks must agree outside the margin band; O is compared against the oracle
    following the GPU's in-band choices."""
    m_ref = ref["mask"]
    n = m_ref.shape[0]
    gm = np.asarray(gpu_mask[:n])
    live = m_ref != NOT_LIVE
    assert np.array_equal(gm == NOT_LIVE, ~live), "live blocks differ"
    c = ref["crit"]
    band = live & np.isfinite(c) & (np.abs(c - ln_lam) < BAND) if math.isfinite(ln_lam) else np.zeros(n, bool)
    out = live & ~band
    bad = np.nonzero(out & (gm != m_ref))[0]
    assert bad.size == 0, f"mask differs outside the band at blocks {bad[:10]} (crit {c[bad[:10]]}, ln_lam {ln_lam})"
    rep.live += int(live.sum())
    rep.skipped += int((gm == SKIPPED).sum())
    rep.in_band += int(band.sum())
    flips = np.nonzero(band & (gm != m_ref))[0]
    rep.flips += int(flips.size)
    if gpu_crit is not None:
        gc = np.asarray(gpu_crit[:n], dtype=np.float64)
        fin = live & np.isfinite(c)
        assert np.array_equal(np.isinf(gc[live]), np.isinf(c[live])), "infinite crit values differ"
        assert np.all(np.isnan(gc[~live])), "crit of blocks that are not live must be NaN"
        if fin.any():
            err = float(np.max(np.abs(gc[fin] - c[fin])))
            rep.max_crit_err = max(rep.max_crit_err, err)
            assert err < CRIT_TOL, f"crit error {err}"
    ref_o = ref
    if flips.size:
        ref_o = rerun({int(j): int(gm[j]) for j in flips})
    if gpu_o is not None:
        o = np.asarray(gpu_o, dtype=np.float64)
        err_arr = np.abs(o - ref_o["o"])
        tol = O_TOL + (bf16_half_ulp(ref_o["o"]) if out_bf16 else 0.0)
        assert np.all(np.isfinite(o)), "non-finite output"
        assert np.all(err_arr <= tol), f"output error {err_arr.max()}"
        rep.max_err = max(rep.max_err, float(err_arr.max()))
    if gpu_lse is not None:
        gl = np.asarray(gpu_lse, dtype=np.float64)
        rl = ref_o["lse"]
        assert np.array_equal(np.isinf(gl), np.isinf(rl))
        fin = np.isfinite(rl)
        if fin.any():
            e = float(np.max(np.abs(gl[fin] - rl[fin])))
            rep.max_lse_err = max(rep.max_lse_err, e)
            assert e < 1e-2, f"lse error {e}"

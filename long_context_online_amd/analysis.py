"""Host-side summaries of the kernels' diagnostic outputs (no GPU work here).

Per-head sparsity: the pages observe that the fraction of skipped blocks varies strongly from head
to head and layer to layer, and that one threshold adapts to it without a per-head top-k or head
pruning (BLASST: Dynamic Blocked Attention Sparsity via Softmax Thresholding, "Sparsity
distribution").  The prefill kernels count, per q head, the live blocks and the skipped ones
(`head_counters`); this module turns those counts into the statistics of that analysis."""

from __future__ import annotations

import numpy as np


def head_sparsity(head_counters) -> np.ndarray:
    """Per-head sparsity (skipped / live blocks) from head_counters [..., 2] (live, skipped); heads
    with no live block get NaN.  Accepts a torch tensor or an array; returns float64 of shape [...]."""
    h = head_counters.cpu().numpy() if hasattr(head_counters, "cpu") else np.asarray(head_counters)
    if h.shape[-1] != 2:
        raise ValueError("head_counters needs a last dimension of 2 (live, skipped)")
    live = h[..., 0].astype(np.float64)
    skipped = h[..., 1].astype(np.float64)
    if np.any(skipped > live) or np.any(skipped < 0):
        raise ValueError("skipped counts must lie in [0, live]")
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(live > 0, skipped / np.where(live > 0, live, 1.0), np.nan)


def head_sparsity_stats(head_counters) -> dict:
    """Distribution of per-head sparsity over all (batch, head) entries: min, quartiles, max, mean,
    standard deviation, the overall (block-weighted) sparsity and the per-head values."""
    h = head_counters.cpu().numpy() if hasattr(head_counters, "cpu") else np.asarray(head_counters)
    sp = head_sparsity(h).reshape(-1)
    sp = sp[np.isfinite(sp)]
    if sp.size == 0:
        raise ValueError("no head has a live block")
    q = np.quantile(sp, [0.0, 0.25, 0.5, 0.75, 1.0])
    live = float(h[..., 0].sum())
    return {"heads": int(sp.size), "min": float(q[0]), "p25": float(q[1]), "median": float(q[2]),
            "p75": float(q[3]), "max": float(q[4]), "mean": float(sp.mean()), "std": float(sp.std()),
            "overall": float(h[..., 1].sum()) / live, "per_head": [float(x) for x in sp]}

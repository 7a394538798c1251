"""Gradients of the BLASST prefill with the forward's skip decisions held fixed (fp64, CPU;
test infrastructure only).

What it computes: sparsity-aware training runs the BLASST forward and lets the skipped blocks
receive no gradient in the backward pass ([xllm] 训练流程, 稀疏感知训练).  The decisions are a
branch, not a differentiable function of the inputs, so the backward differentiates the function the
forward actually evaluated: for each query row, softmax attention over the keys that the row sees
AND whose block its tile kept,

    O_i = sum_{k in K_i} softmax_k(scale * q_i . k_k) v_k,     K_i = {visible keys of kept blocks},

with the mask from the forward fixed.  A row with no key in K_i has O_i = 0 and gets no gradient.
The gradients are taken by torch autograd in float64 on the CPU from that closed form (no blocking,
no online softmax), so they are the exact derivative up to fp64 rounding.

Reading (where the pages are silent): the mask is the forward's skip mask at tile-block granularity
(KEPT blocks contribute, SKIPPED and NOT_LIVE do not), the same tiles and blocks as the forward.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from .blasst_oracle import KEPT, causal_visible


def kept_keys(mask, Lq: int, Lk: int, block_q: int, block_k: int, causal: bool) -> np.ndarray:
    """[B, Hq, Lq, Lk] bool: key k counts for row i iff the row sees it and the tile-block of (i, k)
    is KEPT in the forward mask [B, Hq, n_qtiles, n_kblocks]."""
    mask = np.asarray(mask)
    kept = mask == KEPT
    rows_tile = np.arange(Lq) // block_q
    keys_block = np.arange(Lk) // block_k
    keep = kept[:, :, rows_tile][:, :, :, keys_block]
    if causal:
        keep = keep & causal_visible(np.arange(Lq), Lk, Lq, Lk)[None, None]
    return keep


def attention_on_kept(q, k, v, keep, scale):
    """Differentiable O [B, Hq, Lq, Dv] (torch fp64): softmax attention of each row over its kept keys;
    kv head of q head h is h // (Hq / Hkv).  Rows with no kept key give 0."""
    G = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    s = scale * (q @ kk.transpose(-1, -2))
    s = s.masked_fill(~keep, -math.inf)
    has = keep.any(dim=-1, keepdim=True)
    s = torch.where(has, s, torch.zeros_like(s))        # rows with no key: finite, zeroed below
    p = torch.softmax(s, dim=-1) * keep
    return p @ vv, torch.where(has[..., 0], torch.logsumexp(s, dim=-1), torch.full_like(s[..., 0], -math.inf))


def prefill_backward(q, k, v, do, mask, *, causal: bool, block_q: int, block_k: int, scale=None):
    """dQ [B, Hq, Lq, D], dK [B, Hkv, Lk, D], dV [B, Hkv, Lk, Dv] of sum(dO * O) for the sparse prefill
    with the given forward mask (numpy fp64), plus O and LSE of that forward."""
    q = torch.as_tensor(np.asarray(q, dtype=np.float64)).clone().requires_grad_(True)
    k = torch.as_tensor(np.asarray(k, dtype=np.float64)).clone().requires_grad_(True)
    v = torch.as_tensor(np.asarray(v, dtype=np.float64)).clone().requires_grad_(True)
    do = torch.as_tensor(np.asarray(do, dtype=np.float64))
    B, Hq, Lq, D = q.shape
    Lk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    keep = torch.as_tensor(kept_keys(mask, Lq, Lk, block_q, block_k, causal))
    o, lse = attention_on_kept(q, k, v, keep, scale)
    dq, dk, dv = torch.autograd.grad(o, (q, k, v), grad_outputs=do)
    return {"dq": dq.numpy(), "dk": dk.numpy(), "dv": dv.numpy(), "o": o.detach().numpy(),
            "lse": lse.detach().numpy()}


def dq_rows(q, k, v, do, mask, b: int, h: int, rows, *, causal: bool, block_q: int, block_k: int, scale=None):
    """dQ of the given query rows of (sequence b, q head h) only, by the same closed form and autograd
    (each row's output depends on its own query only, so its dQ needs no other row): cheap at any L.
    Returns [len(rows), D]."""
    rows = np.asarray(rows)
    q = np.asarray(q)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = np.asarray(k).shape[1], np.asarray(k).shape[2]
    g = h // (Hq // Hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask = np.asarray(mask)
    kept = mask[b, h][rows // block_q][:, np.arange(Lk) // block_k] == KEPT          # [R, Lk]
    if causal:
        kept = kept & causal_visible(rows, Lk, Lq, Lk)
    qr = torch.as_tensor(np.asarray(q[b, h, rows], dtype=np.float64))[None, None].clone().requires_grad_(True)
    kk = torch.as_tensor(np.asarray(np.asarray(k)[b, g], dtype=np.float64))[None, None]
    vv = torch.as_tensor(np.asarray(np.asarray(v)[b, g], dtype=np.float64))[None, None]
    dd = torch.as_tensor(np.asarray(np.asarray(do)[b, h, rows], dtype=np.float64))[None, None]
    o, _ = attention_on_kept(qr, kk, vv, torch.as_tensor(kept)[None, None], scale)
    (dq,) = torch.autograd.grad(o, (qr,), grad_outputs=dd)
    return dq[0, 0].numpy()

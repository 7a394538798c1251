"""Seeded synthetic Q/K/V with the score structure of long-context attention.

Score structure (the workload description this stands in for; the pages measure on real models
that are not available here):
  * content channels: logits of standard deviation 1;
  * an attention sink at token 0: +10 logit for every query;
  * a seeded 10 % of key blocks "aligned" with the queries of a kv head: +6 logit;
  * optionally a local window: an expected +3 logit for keys close to the query, decaying as
    3 * exp(-distance / 512).

Construction (exact in the channels it uses, so the boosts are exact up to the I/O rounding):
  * the last two channels of the q/k head dim are control channels: channel D-2 carries the sink
    (q = 1, k = 10 / scale at token 0, 0 elsewhere), channel D-1 the aligned blocks (q = 1,
    k = 6 / scale on the aligned keys, 0 elsewhere); scale = 1 / sqrt(D);
  * the other D-2 content channels: keys N(0, 1); queries N(0, 1) times sqrt(D / (D-2)) so that
    scale * q.k has unit variance;
  * the window: keys follow an AR(1) stream z_t = rho z_{t-1} + sqrt(1 - rho^2) e_t per channel
    with rho = exp(-1/512), and a query at position i is gamma z_i + sqrt(1 - gamma^2) eta with
    gamma = 3 / sqrt(D-2), giving E[scale q_i.k_t] = 3 rho^|i-t| while keeping unit marginals.
    A decode query sits one AR step past the last key.

All draws come from a torch.Generator on the requested device, seeded explicitly, in a fixed
order; the values are cast to the I/O dtype with round-to-nearest-even (torch's cast).  Large
inputs are generated on the GPU; the same seed on another device gives other (equally valid)
numbers, so a check always reads the inputs back from the tensors it was given.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SINK_BOOST = 10.0
ALIGNED_BOOST = 6.0
ALIGNED_FRACTION = 0.10
WINDOW_BOOST = 3.0
WINDOW_LEN = 512.0


def to_bf16_rne_numpy(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to the nearest bfloat16 (ties to even), returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _ar1(gen, lead, T, C, device, rho=math.exp(-1.0 / WINDOW_LEN), chunk=256):
    """AR(1) stream [*lead, T, C] (float32) with unit stationary variance, via a chunked scan."""
    a = math.sqrt(1.0 - rho * rho)
    z_prev = torch.randn(*lead, 1, C, generator=gen, device=device)       # stationary start
    eps = torch.randn(*lead, T, C, generator=gen, device=device)
    out = torch.empty_like(eps)
    t = torch.arange(chunk, device=device, dtype=torch.float64)
    pw = (rho ** (t + 1)).float().view(-1, 1)        # rho^(i+1)
    pi = (rho ** t).float().view(-1, 1)              # rho^i
    ipw = (rho ** (-t)).float().view(-1, 1)          # rho^-u
    for c0 in range(0, T, chunk):
        n = min(chunk, T - c0)
        e = eps[..., c0:c0 + n, :]
        acc = torch.cumsum(e * ipw[:n], dim=-2) * (a * pi[:n])
        z = acc + pw[:n] * z_prev
        out[..., c0:c0 + n, :] = z
        z_prev = z[..., n - 1:n, :]
    return out, z_prev


def _aligned_blocks(gen, n_blocks: int, device):
    """round(10 %) of the key blocks 1..n-1, drawn without replacement."""
    n_al = int(round(ALIGNED_FRACTION * n_blocks))
    if n_blocks <= 1 or n_al == 0:
        return torch.zeros(0, dtype=torch.long, device=device)
    perm = torch.randperm(n_blocks - 1, generator=gen, device=device)[:n_al] + 1
    return torch.sort(perm).values


@dataclass
class PrefillInputs:
    q: torch.Tensor      # [B, Hq, L, D]
    k: torch.Tensor      # [B, Hkv, L, D]
    v: torch.Tensor      # [B, Hkv, L, Dv]
    scale: float
    aligned: list = field(default_factory=list)   # per (b, kv head): aligned block indices


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, Dqk], or [B, T, Hq, Dqk] with T query tokens per sequence
    k_cache: torch.Tensor      # [P, Hkv, page, Dqk]
    v_cache_t: torch.Tensor | None   # [P, Hkv, Dv, page] (None: V = K[..., :Dv], latent attention)
    block_table: torch.Tensor  # [B, max_pages] int32
    seq_lens: torch.Tensor     # [B] int32
    page_size: int
    scale: float
    head_dim_v: int
    aligned: list = field(default_factory=list)


def prefill_inputs(*, batch, hq, hkv, L, d, dv=None, dtype=torch.bfloat16, block_k=128,
                   window=True, seed=0, device="cpu", Lq=None, head_strength=None):
    """Q/K/V for a causal prefill (Lq = L unless given; queries are the last Lq positions).

    head_strength: optional per-q-head factors c_h for heterogeneous heads: head h's query weights
    the sink and aligned channels by c_h (boosts c_h * 10 and c_h * 6) and its window correlation is
    c_h * gamma (boost about c_h * 3), so small c_h gives flat, hard-to-skip attention and large c_h
    peaked attention.  None gives every head factor 1 (the homogeneous inputs)."""
    dv = d if dv is None else dv
    Lq = L if Lq is None else Lq
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    G = hq // hkv
    dc = d - 2
    scale = 1.0 / math.sqrt(d)
    qscale = math.sqrt(d / dc)
    gamma = WINDOW_BOOST / math.sqrt(dc)
    n_blocks = -(-L // block_k)
    gen = _gen(seed, device)
    q = torch.empty(batch, hq, Lq, d, dtype=dtype, device=device)
    k = torch.empty(batch, hkv, L, d, dtype=dtype, device=device)
    v = torch.empty(batch, hkv, L, dv, dtype=dtype, device=device)
    aligned = []
    for b in range(batch):
        if window:
            z, _ = _ar1(gen, (hkv,), L, dc, device)                       # [Hkv, L, dc]
        else:
            z = torch.randn(hkv, L, dc, generator=gen, device=device)
        kf = torch.zeros(hkv, L, d, device=device)
        kf[..., :dc] = z
        kf[:, 0, d - 2] = SINK_BOOST / scale
        al_b = []
        for g in range(hkv):
            al = _aligned_blocks(gen, n_blocks, device)
            al_b.append(al.cpu().tolist())
            for j in al.cpu().tolist():
                kf[g, j * block_k:min((j + 1) * block_k, L), d - 1] = ALIGNED_BOOST / scale
        aligned.append(al_b)
        k[b] = kf.to(dtype)
        del kf
        eta = torch.randn(hq, Lq, dc, generator=gen, device=device)
        if head_strength is None:
            cs = torch.ones(hq, 1, 1, device=device)
        else:
            if len(head_strength) != hq:
                raise ValueError("head_strength needs one factor per q head")
            cs = torch.tensor([float(c) for c in head_strength], device=device).view(hq, 1, 1)
        if window:
            zq = z[:, L - Lq:, :].repeat_interleave(G, dim=0)             # head h uses kv head h // G
            if head_strength is None:
                qc = gamma * zq + math.sqrt(1.0 - gamma * gamma) * eta
            else:
                gh = torch.clamp(gamma * cs, max=0.95)
                qc = gh * zq + torch.sqrt(1.0 - gh * gh) * eta
            del zq
        else:
            qc = eta
        qf = cs.expand(hq, Lq, 1).repeat(1, 1, d)
        qf[..., :dc] = qc * qscale
        q[b] = qf.to(dtype)
        del qf, qc, eta, z
        v[b] = torch.randn(hkv, L, dv, generator=gen, device=device).to(dtype)
    return PrefillInputs(q=q, k=k, v=v, scale=scale, aligned=aligned)


def decode_inputs(*, batch, hq, hkv, ctx, d, dv=None, dtype=torch.bfloat16, page_size=16,
                  block_k=64, window=True, seed=0, device="cpu", latent=False, seq_lens=None,
                  num_q_tokens=None):
    """One query token per sequence over a paged KV cache with randomly permuted pages.

    ctx: the context length of every sequence, unless seq_lens (a list) gives one per sequence.
    num_q_tokens=T: q is [B, T, Hq, D] instead, T query tokens at the last T positions of each
    sequence (their keys are in the cache); token t correlates with the key at its own position
    seq_len - T + t, as a prefill query does.
    latent=True: one shared latent head; V is the first dv channels of K (no V cache).
    Pages beyond a sequence's length, the slots after its last key and 1/16 extra spare pages
    are filled with NaN, so a wrong gather poisons the result.  Unused block-table entries point
    at a spare (NaN) page.
    """
    dv = d if dv is None else dv
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    G = hq // hkv
    dc = d - 2
    scale = 1.0 / math.sqrt(d)
    qscale = math.sqrt(d / dc)
    gamma = WINDOW_BOOST / math.sqrt(dc)
    lens = [int(ctx)] * batch if seq_lens is None else [int(x) for x in seq_lens]
    if len(lens) != batch or min(lens) < 1:
        raise ValueError("need one positive length per sequence")
    pages_per_seq = [-(-n // page_size) for n in lens]
    max_pages = max(pages_per_seq)
    live = sum(pages_per_seq)
    spare = max(1, live // 16)
    P = live + spare
    gen = _gen(seed, device)
    perm = torch.randperm(P, generator=gen, device=device).to(torch.int32)
    # equal lengths: one AR(1) scan for the whole batch (far fewer small kernels than one per sequence)
    batched = window and len(set(lens)) == 1
    if batched:
        z_all, z_last_all = _ar1(gen, (batch, hkv), lens[0], dc, device)
    block_table = torch.empty(batch, max_pages, dtype=torch.int32, device=device)
    spare_ids = perm[live:]
    k_cache = torch.full((P, hkv, page_size, d), float("nan"), dtype=dtype, device=device)
    v_cache_t = None if latent else torch.full((P, hkv, dv, page_size), float("nan"), dtype=dtype, device=device)
    T = num_q_tokens
    if T is not None and (T < 1 or T > min(lens)):
        raise ValueError("num_q_tokens must lie in [1, shortest sequence]")
    q = torch.empty((batch, hq, d) if T is None else (batch, T, hq, d), dtype=dtype, device=device)
    aligned = []
    off = 0
    for b in range(batch):
        n, npg = lens[b], pages_per_seq[b]
        ids = perm[off:off + npg]
        off += npg
        block_table[b, :npg] = ids
        if npg < max_pages:
            block_table[b, npg:] = spare_ids[0]
        n_blocks = -(-n // block_k)
        if batched:
            z, z_last = z_all[b], z_last_all[b]
        elif window:
            z, z_last = _ar1(gen, (hkv,), n, dc, device)                 # [Hkv, n, dc]
        else:
            z = torch.randn(hkv, n, dc, generator=gen, device=device)
            z_last = None
        kf = torch.full((hkv, npg * page_size, d), float("nan"), device=device)
        kf[:, :n, :dc] = z
        kf[:, :n, d - 2:] = 0.0
        kf[:, 0, d - 2] = SINK_BOOST / scale
        al_b = []
        for g in range(hkv):
            al = _aligned_blocks(gen, n_blocks, device)
            al_b.append(al.cpu().tolist())
            for j in al.cpu().tolist():
                kf[g, j * block_k:min((j + 1) * block_k, n), d - 1] = ALIGNED_BOOST / scale
        aligned.append(al_b)
        kpages = kf.to(dtype).view(hkv, npg, page_size, d).permute(1, 0, 2, 3)
        k_cache[ids.long()] = kpages
        del kf, kpages
        if T is not None:
            eta = torch.randn(T, hq, dc, generator=gen, device=device)
            if window:
                zt = z[:, n - T:n, :].permute(1, 0, 2).repeat_interleave(G, dim=1)   # [T, Hq, dc]
                qc = gamma * zt + math.sqrt(1.0 - gamma * gamma) * eta
            else:
                qc = eta
            qf = torch.ones(T, hq, d, device=device)
            qf[..., :dc] = qc * qscale
            q[b] = qf.to(dtype)
            del qf, qc, eta
        else:
            eta = torch.randn(hq, dc, generator=gen, device=device)
            if window:
                rho = math.exp(-1.0 / WINDOW_LEN)
                e_next = torch.randn(hkv, dc, generator=gen, device=device)
                z_q = rho * z_last[:, 0, :] + math.sqrt(1.0 - rho * rho) * e_next   # position n
                qc = gamma * z_q.repeat_interleave(G, dim=0) + math.sqrt(1.0 - gamma * gamma) * eta
            else:
                qc = eta
            qf = torch.ones(hq, d, device=device)
            qf[:, :dc] = qc * qscale
            q[b] = qf.to(dtype)
            del qf, qc, eta
        del z
        if not latent:
            vf = torch.full((hkv, npg * page_size, dv), float("nan"), device=device)
            vf[:, :n] = torch.randn(hkv, n, dv, generator=gen, device=device)
            vpages = vf.to(dtype).view(hkv, npg, page_size, dv).permute(1, 0, 3, 2)   # [npg, Hkv, Dv, page]
            v_cache_t[ids.long()] = vpages
            del vf, vpages
    seq = torch.tensor(lens, dtype=torch.int32, device=device)
    return DecodeInputs(q=q, k_cache=k_cache, v_cache_t=v_cache_t, block_table=block_table,
                        seq_lens=seq, page_size=page_size, scale=scale,
                        head_dim_v=dv, aligned=aligned)

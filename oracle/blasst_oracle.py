"""Block-sequential BLASST attention in fp64 (oracle; test infrastructure only).

What it computes (the pages' method, restated):
  * Tiled online-softmax attention: along each query row the KV blocks are visited left to
    right, keeping a running max m, a running sum l and an unnormalised output o
    ([xllm] 解决方案概述 and 整体框架图; [nerve] online-softmax paragraph).
  * For block j, the block-local row max m~ is computed; m^(j) is the running max after
    processing block j, i.e. max(m^(j-1), m~) ([xllm] 核心公式, definitions under the skip
    condition).  The block is skipped when exp(m~ - m^(j)) < lambda, i.e.
    m~ - m^(j) < ln(lambda), strictly ([xllm] 核心公式; [gist-de] 2. Methodik / Kernidee;
    [gist-ja] 2.1).
  * A skipped block contributes nothing: its exp, its V load and its P.V product are all
    elided ([gist-de] Kernidee, the three saved operations; [gist-ja] 2.1; [fugu] abstract).
  * The decision is taken for the whole query tile: one vote per warp in the pages
    ([xllm] 模型组件).  Reading taken here: the block is skipped only if EVERY row of the
    tile satisfies the condition, each row with its own running max.
  * lambda = a / L with L the context length ([xllm] 核心公式, threshold calibration;
    [gist-de] Kalibrierung).

Readings where the pages are silent (each listed in the design notes of the repository):
  * num_splits: the live blocks of a tile are cut into num_splits contiguous chunks of
    ceil(J/num_splits) blocks; each chunk starts with m = -inf, l = 0, o = 0 and is finished
    as O_s = o/l, lse_s = m + ln l; chunks are merged with a log-sum-exp combine.
  * Causal visibility is bottom-right aligned: key k is visible to query row i iff
    k <= i + (Lk - Lq).
  * Arithmetic with -inf: a row with no visible key in the block has m~ = -inf and its
    difference m~ - m is -inf (it votes "skip"); lambda must lie in [0, 1] (ln 0 = -inf means
    dense).
  * Critical value of a tile-block: c = max over rows of (m~_i - m_i^(j-1)), the difference
    against the running max BEFORE the block, with (finite) - (-inf) = +inf.  For lambda <= 1
    "c < ln(lambda)" is the same decision as the pages' rule with the post-update max.

Everything is plain numpy in float64; inputs are upcast from their I/O dtype by the caller.
"""

from __future__ import annotations

import math

import numpy as np

KEPT = 0
SKIPPED = 1
NOT_LIVE = 2

NEG_INF = -np.inf


def ln_threshold(lam: float | None = None, a: float | None = None, L: int | None = None) -> float:
    """ln(lambda) for a threshold given as lambda, or as a and L with lambda = a / L.

    [xllm] 核心公式 (threshold calibration lambda = a/L).  lambda = a/L is clamped to 1 (a
    reading: the rule is only defined for lambda <= 1 here).  lambda = 0 gives -inf (dense).
    """
    if lam is None:
        if a is None or L is None:
            raise ValueError("give lambda, or a and L")
        if a < 0 or L <= 0:
            raise ValueError("a must be >= 0 and L > 0")
        lam = min(1.0, a / L)
    if not (0.0 <= lam <= 1.0):
        raise ValueError("lambda must lie in [0, 1]")
    return NEG_INF if lam == 0.0 else math.log(lam)


def softmax_attention(q, k, v, visible, scale):
    """Textbook softmax(scale * q k^T) v over the visible (row, key) pairs, fp64.

    [xllm] 核心公式, standard attention softmax(QK^T / sqrt(d_k)) V.  Rows with no visible key
    get O = 0 and lse = -inf.  Returns (O [R, Dv], lse [R]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    s = np.where(visible, s, NEG_INF)
    R = s.shape[0]
    o = np.zeros((R, v.shape[1]))
    lse = np.full(R, NEG_INF)
    for i in range(R):
        if not visible[i].any():
            continue
        mx = s[i].max()
        p = np.exp(s[i] - mx)
        den = p.sum()
        o[i] = (p @ v) / den
        lse[i] = mx + math.log(den)
    return o, lse


def _block_ranges(n_keys: int, block_k: int):
    return [(j * block_k, min((j + 1) * block_k, n_keys)) for j in range((n_keys + block_k - 1) // block_k)]


def _split_chunks(live_blocks, num_splits: int):
    """Contiguous chunks of ceil(J / num_splits) live blocks; empty chunks dropped (a reading)."""
    J = len(live_blocks)
    if J == 0:
        return []
    size = -(-J // num_splits)
    return [live_blocks[s:s + size] for s in range(0, J, size)]


def _diff(a, b):
    """a - b elementwise with the conventions (finite) - (-inf) = +inf, (-inf) - x = -inf."""
    out = np.empty_like(a)
    for i in range(a.shape[0]):
        if a[i] == NEG_INF:
            out[i] = NEG_INF
        elif b[i] == NEG_INF:
            out[i] = np.inf
        else:
            out[i] = a[i] - b[i]
    return out


def tile_sequential(q_rows, keys, values, visible, block_k, num_splits, ln_lam, scale, force=None):
    """BLASST forward for one query tile, block by block, left to right (the step-by-step rule).

    q_rows [R, Dqk], keys [N, Dqk], values [N, Dv], visible [R, N] bool.
    force: optional {block index: KEPT or SKIPPED} overriding the rule for those blocks.  It exists
    for blocks whose critical value lies within rounding distance of ln(lambda), where either
    decision is a correct result (a reading); the caller decides which blocks qualify.
    Returns a dict:
      o [R, Dv], lse [R]   combined output over the splits
      mask [nb] int8       KEPT / SKIPPED / NOT_LIVE per key block
      crit [nb] float      critical value per live block (nan when not live)
      split_of [nb] int    split index per live block (-1 when not live)
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if not (np.isfinite(q_rows).all() and np.isfinite(keys).all() and np.isfinite(values).all()):
        raise ValueError("oracle inputs must be finite")
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    if ln_lam > 0.0:
        raise ValueError("ln(lambda) must be <= 0")
    R, Dv = q_rows.shape[0], values.shape[1]
    ranges = _block_ranges(keys.shape[0], block_k)
    nb = len(ranges)
    mask = np.full(nb, NOT_LIVE, dtype=np.int8)
    crit = np.full(nb, np.nan)
    split_of = np.full(nb, -1, dtype=np.int64)
    live = [j for j, (k0, k1) in enumerate(ranges) if visible[:, k0:k1].any()]

    split_o, split_lse = [], []
    for s_idx, chunk in enumerate(_split_chunks(live, num_splits)):
        m = np.full(R, NEG_INF)
        l = np.zeros(R)
        o = np.zeros((R, Dv))
        for pos, j in enumerate(chunk):
            k0, k1 = ranges[j]
            sc = scale * (q_rows @ keys[k0:k1].T)
            sc = np.where(visible[:, k0:k1], sc, NEG_INF)
            m_blk = sc.max(axis=1)                      # block-local row max m~
            m_after = np.maximum(m, m_blk)              # running max after block j
            c_rule = _diff(m_blk, m_after)              # m~ - m^(j), the pages' quantity
            skip = bool(np.all(c_rule < ln_lam))        # every row of the tile must agree
            crit[j] = np.max(_diff(m_blk, m))           # against the max before the block
            split_of[j] = s_idx
            if pos == 0 and skip:
                raise AssertionError("first block of a split was skipped")
            if force is not None and j in force:
                skip = force[j] == SKIPPED
                if skip:
                    m_after = m                             # a skipped block adds nothing
            if skip:
                mask[j] = SKIPPED
                # nothing is added: no exp, no V, no P.V; the running max cannot rise
                # (m~ < m^(j) on every row since ln(lambda) <= 0).
                continue
            mask[j] = KEPT
            has = m_after > NEG_INF
            alpha = np.where(has, np.exp(np.where(has, m - np.where(has, m_after, 0.0), 0.0)), 1.0)
            p = np.where(has[:, None], np.exp(sc - np.where(has, m_after, 0.0)[:, None]), 0.0)
            l = alpha * l + p.sum(axis=1)
            o = alpha[:, None] * o + p @ values[k0:k1]
            m = m_after
        o_s = np.where(l[:, None] > 0, o / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse_s = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
        split_o.append(o_s)
        split_lse.append(lse_s)
    o, lse = combine_splits(split_o, split_lse, R, Dv)
    return {"o": o, "lse": lse, "mask": mask, "crit": crit, "split_of": split_of}


def combine_splits(split_o, split_lse, R, Dv):
    """Log-sum-exp merge of per-split normalised outputs (a reading; not on the pages).

    LSE = log sum_s exp(lse_s); O = sum_s exp(lse_s - LSE) O_s.  Rows where every split has
    lse = -inf get O = 0, LSE = -inf.
    """
    o = np.zeros((R, Dv))
    lse = np.full(R, NEG_INF)
    if not split_o:
        return o, lse
    L = np.stack(split_lse)            # [S, R]
    O = np.stack(split_o)              # [S, R, Dv]
    for i in range(R):
        col = L[:, i]
        if np.all(col == NEG_INF):
            continue
        mx = col.max()
        w = np.exp(col - mx)
        tot = w.sum()
        lse[i] = mx + math.log(tot)
        o[i] = (w[:, None] * O[:, i, :]).sum(axis=0) / tot
    return o, lse


def keep_mask_closed_form(q_rows, keys, visible, block_k, num_splits, ln_lam, scale):
    """Decisions without running the accumulation: block j of a split is skipped iff it is not the
    split's first block and max over rows of (m~_ij - max_{j' < j in the split} m~_ij') < ln(lambda).

    Derived from the rule for lambda <= 1 (a skipped block never raises the running max), so the
    running max is the prefix max of the block maxima.  Returns (mask [nb], crit [nb]).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    ranges = _block_ranges(keys.shape[0], block_k)
    nb = len(ranges)
    mask = np.full(nb, NOT_LIVE, dtype=np.int8)
    crit = np.full(nb, np.nan)
    s_all = np.where(visible, scale * (q_rows @ keys.T), NEG_INF)
    bmax = np.stack([s_all[:, k0:k1].max(axis=1) for (k0, k1) in ranges], axis=1)  # [R, nb]
    live = [j for j, (k0, k1) in enumerate(ranges) if visible[:, k0:k1].any()]
    for chunk in _split_chunks(live, num_splits):
        prefix = np.full(q_rows.shape[0], NEG_INF)
        for pos, j in enumerate(chunk):
            c = np.max(_diff(bmax[:, j], prefix)) if pos > 0 else np.inf
            crit[j] = c
            mask[j] = SKIPPED if c < ln_lam else KEPT
            prefix = np.maximum(prefix, bmax[:, j])
    return mask, crit


def sparsity(mask) -> float:
    """Fraction of skipped tile-blocks among live tile-blocks (a reading: block-count ratio)."""
    mask = np.asarray(mask)
    live = np.count_nonzero(mask != NOT_LIVE)
    return float(np.count_nonzero(mask == SKIPPED)) / live if live else 0.0


# ----------------------------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------------------------

def causal_visible(rows, n_keys, Lq, Lk):
    """Bottom-right aligned causal visibility for the given query row indices (a reading)."""
    rows = np.asarray(rows)
    return np.arange(n_keys)[None, :] <= (rows[:, None] + (Lk - Lq))


def prefill_tile(q, k, v, b, hq, qt, *, causal, block_q, block_k, num_splits, ln_lam, scale=None,
                 force=None):
    """One prefill query tile: rows [qt*block_q, ...) of q head hq in batch b.

    q [B, Hq, Lq, Dqk], k [B, Hkv, Lk, Dqk], v [B, Hkv, Lk, Dv] (any array-likes, upcast to
    fp64).  The kv head is hq // (Hq / Hkv) (GQA/MQA mapping; [xllm] 核心思想 item 4 lists
    MHA, GQA, MQA, MLA).
    """
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // (Hq // Hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    r0, r1 = qt * block_q, min((qt + 1) * block_q, Lq)
    rows = np.arange(r0, r1)
    if causal:
        vis = causal_visible(rows, Lk, Lq, Lk)
    else:
        vis = np.ones((r1 - r0, Lk), dtype=bool)
    return tile_sequential(np.asarray(q[b, hq, r0:r1], dtype=np.float64),
                           np.asarray(k[b, g], dtype=np.float64),
                           np.asarray(v[b, g], dtype=np.float64),
                           vis, block_k, num_splits, ln_lam, scale, force=force)


def prefill(q, k, v, *, causal, block_q, block_k, num_splits=1, lam=None, a=None, scale=None):
    """Whole prefill: O [B, Hq, Lq, Dv], LSE [B, Hq, Lq], mask/crit [B, Hq, n_qtiles, n_kblocks]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Lq, _ = q.shape
    Lk, Dv = k.shape[2], v.shape[3]
    ln_lam = ln_threshold(lam=lam, a=a, L=Lk)
    nqt = -(-Lq // block_q)
    nkb = -(-Lk // block_k)
    O = np.zeros((B, Hq, Lq, Dv))
    LSE = np.full((B, Hq, Lq), NEG_INF)
    mask = np.full((B, Hq, nqt, nkb), NOT_LIVE, dtype=np.int8)
    crit = np.full((B, Hq, nqt, nkb), np.nan)
    for b in range(B):
        for hq in range(Hq):
            for qt in range(nqt):
                r = prefill_tile(q, k, v, b, hq, qt, causal=causal, block_q=block_q, block_k=block_k,
                                 num_splits=num_splits, ln_lam=ln_lam, scale=scale)
                r0, r1 = qt * block_q, min((qt + 1) * block_q, Lq)
                O[b, hq, r0:r1] = r["o"]
                LSE[b, hq, r0:r1] = r["lse"]
                mask[b, hq, qt] = r["mask"]
                crit[b, hq, qt] = r["crit"]
    return {"o": O, "lse": LSE, "mask": mask, "crit": crit}


# ----------------------------------------------------------------------------------------------
# decode over a paged KV cache
# ----------------------------------------------------------------------------------------------

def gather_pages(k_cache, v_cache_t, block_table, b, g, seq_len, page_size, head_dim_v):
    """Contiguous K [seq_len, Dqk] and V [seq_len, Dv] of sequence b, kv head g.

    k_cache [P, Hkv, page, Dqk].  v_cache_t [P, Hkv, Dv, page] holds V transposed inside each
    page; None means V is the first Dv channels of K (latent attention, MLA).
    """
    n_pages = -(-seq_len // page_size)
    if n_pages == 0:  # an empty sequence (a reading: no keys, so nothing to attend to)
        dv = head_dim_v if head_dim_v is not None else (v_cache_t.shape[2] if v_cache_t is not None else k_cache.shape[-1])
        return np.zeros((0, k_cache.shape[-1])), np.zeros((0, dv))
    ks, vs = [], []
    for p in range(n_pages):
        pid = int(block_table[b][p])
        ks.append(np.asarray(k_cache[pid, g], dtype=np.float64))
        if v_cache_t is not None:
            vs.append(np.asarray(v_cache_t[pid, g], dtype=np.float64).T)
    K = np.concatenate(ks, axis=0)[:seq_len]
    V = np.concatenate(vs, axis=0)[:seq_len] if v_cache_t is not None else K[:, :head_dim_v].copy()
    return K, V


def _decode_queries(q):
    """q [B, Hq, Dqk] (one query token per sequence) or [B, T, Hq, Dqk] (T query tokens, the last T
    positions of each sequence) as fp64 [B, T, Hq, Dqk], and whether it had the token axis."""
    q = np.asarray(q, dtype=np.float64)
    if q.ndim == 3:
        return q[:, None], False
    if q.ndim != 4:
        raise ValueError("q must be [B, Hq, D] or [B, T, Hq, D]")
    return q, True


def decode_tile(q, k_cache, v_cache_t, block_table, seq_lens, b, g, rt, *, page_size, block_k,
                num_splits, ln_lam, tile_rows, head_dim_v, scale=None, force=None):
    """One decode tile: the tile_rows q heads [g*G + rt*tile_rows, ...) of sequence b that share
    kv head g (G = Hq/Hkv), for each of the sequence's T query tokens.

    q [B, Hq, Dqk] has one query token per sequence, which sees every key < seq_len.  q
    [B, T, Hq, Dqk] has T query tokens, the last T positions of the sequence (the tokens a decode
    step verifies, or a chunk of a prefill continued against the paged cache: the pages' method
    serves both phases, xllm-io review, 核心思想 item 2); token t sees keys
    k <= seq_len - T + t (bottom-right causal, as in prefill).  The tile's rows are token-major:
    row t * tile_rows + i is token t of head g*G + rt*tile_rows + i, and every row votes.
    """
    q4, _ = _decode_queries(q)
    B, T, Hq, D = q4.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    L = int(seq_lens[b])
    K, V = gather_pages(k_cache, v_cache_t, block_table, b, g, L, page_size, head_dim_v)
    h0 = g * G + rt * tile_rows
    rows = q4[b, :, h0:h0 + tile_rows].reshape(T * tile_rows, D)
    tok = np.repeat(np.arange(T), tile_rows)
    vis = np.arange(L)[None, :] <= (L - T + tok)[:, None]
    return tile_sequential(rows, K, V, vis, block_k, num_splits, ln_lam, scale, force=force)


def decode(q, k_cache, v_cache_t, block_table, seq_lens, *, page_size, block_k, num_splits,
           lam=None, a=None, tile_rows=None, head_dim_v=None, scale=None):
    """Whole paged decode.  q [B, Hq, Dqk], or [B, T, Hq, Dqk] for T query tokens per sequence
    (see decode_tile).  With a given, lambda_b = min(1, a / seq_lens[b]).

    Returns O [B, Hq, Dv] and LSE [B, Hq] ([B, T, Hq, Dv] and [B, T, Hq] with the token axis),
    mask/crit [B, Hkv, Hq/Hkv/tile_rows, n_kblocks(max)].
    """
    q4, tokens = _decode_queries(q)
    B, T, Hq, D = q4.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    tile_rows = G if tile_rows is None else tile_rows
    if G % tile_rows:
        raise ValueError("tile_rows must divide Hq/Hkv")
    if head_dim_v is None:
        head_dim_v = v_cache_t.shape[2] if v_cache_t is not None else D
    n_rt = G // tile_rows
    nkb = -(-int(max(seq_lens)) // block_k)
    O = np.zeros((B, T, Hq, head_dim_v))
    LSE = np.full((B, T, Hq), NEG_INF)
    mask = np.full((B, Hkv, n_rt, nkb), NOT_LIVE, dtype=np.int8)
    crit = np.full((B, Hkv, n_rt, nkb), np.nan)
    for b in range(B):
        if lam is None and int(seq_lens[b]) == 0:
            ln_lam = NEG_INF  # a / L is undefined for an empty sequence, which has no block to decide on
        else:
            ln_lam = ln_threshold(lam=lam, a=a, L=int(seq_lens[b])) if lam is None else ln_threshold(lam=lam)
        for g in range(Hkv):
            for rt in range(n_rt):
                r = decode_tile(q4, k_cache, v_cache_t, block_table, seq_lens, b, g, rt,
                                page_size=page_size, block_k=block_k, num_splits=num_splits,
                                ln_lam=ln_lam, tile_rows=tile_rows, head_dim_v=head_dim_v, scale=scale)
                h0 = g * G + rt * tile_rows
                O[b, :, h0:h0 + tile_rows] = r["o"].reshape(T, tile_rows, head_dim_v)
                LSE[b, :, h0:h0 + tile_rows] = r["lse"].reshape(T, tile_rows)
                n = r["mask"].shape[0]
                mask[b, g, rt, :n] = r["mask"]
                crit[b, g, rt, :n] = r["crit"]
    if not tokens:
        O, LSE = O[:, 0], LSE[:, 0]
    return {"o": O, "lse": LSE, "mask": mask, "crit": crit}

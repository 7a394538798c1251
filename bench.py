"""Benchmark of the BLASST hot path on one MI355X.

One step = one sparse prefill of the Llama-3.1-8B-shaped GQA problem (batch 1, 32 q / 8 kv heads,
d = 128, L = 32768, bf16 in, fp32 accumulation, causal, 128 x 128 blocks) at the threshold
calibrated for 75 % sparsity, followed by one sparse paged decode (batch 32, 32 q / 8 kv heads,
d = 128, context 32768, 16-token pages, 64-token blocks, 16 splits) at the threshold calibrated for
73 % sparsity.  Inputs are seeded synthetic tensors resident in HBM before timing starts.

Printed (one JSON line): prefill dense-equivalent TFLOP/s as `value`, decode HBM GB/s (bytes the
kernel actually has to read and write), the speedups over the same kernels at lambda = 0, roofline
fractions, and the fp64 oracle's throughput on the host cores as a baseline.  Untimed extras in the
same line (skipped with --quick): prefill at 50 % sparsity, decode at context 131072, the latent
(MLA-shaped) decode at 50 % and 73 % sparsity, and the calibration sweep (lambda * L = alpha *
exp(beta * s) fitted over L = 4K..128K and s = 0.3/0.5/0.7, achieved-vs-target sparsity, and the
prefill at L = 131072, s = 0.75).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill dense-equiv TFLOPS & decode HBM GB/s; speedup vs λ=0 at ~70% sparsity"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0

# prefill workload
P_B, P_HQ, P_HKV, P_L, P_D, P_BLK = 1, 32, 8, 32768, 128, 128
P_TARGET = 0.75
C_B, C_L, C_T = 4, 32768, 2048      # chunked prefill: sequences, context length, chunk length
# decode workload
D_B, D_HQ, D_HKV, D_CTX, D_D, D_PAGE, D_BLK, D_SPLITS = 32, 32, 8, 32768, 128, 16, 64, 16
D_TARGET = 0.73
# multi-token decode: 8 splits (with 16, the per-split first blocks that every tile keeps cap the
# sparsity of tiles with T x 4 voting rows at 67-70 % even at lambda = 1)
MT_SPLITS = 8
CALIB_TILES = 8  # prefill calibration sample: 8 query tiles of 128 rows (1024 rows)
# latent (MLA-shaped) decode
M_B, M_HQ, M_D, M_DV, M_CTX, M_TARGETS = 64, 128, 576, 512, 32768, (0.5, 0.73)
# 8 splits: 512 workgroups of 64 blocks; with 16 the per-split first blocks (always kept) cap the
# sparsity at 65 % even at lambda = 1, and the partials to merge double (see mla_decode.splits_sweep)
M_SPLITS = 8
CHUNKED_KERNEL = "prefill_bf16_kernel<128, 128, 2, false, false, true, true, false>"
DEC_KERNEL = {False: "decode_gqa_kernel<false, true>", True: "decode_mla_kernel<false, false>"}
MLA_WORKLOAD = ("latent decode, DeepSeek-shaped: batch 64, 128 q heads on one latent head, 576-dim scores, "
                "V = first 512 channels, context 32768, 16-token pages, 64-token blocks, 8 splits, 128-head "
                "tiles, bf16")
# calibration sweep
C_L_VALUES = (4096, 8192, 16384, 32768, 65536, 131072)
C_S_VALUES = (0.3, 0.5, 0.7)
C_FINAL_L, C_FINAL_S = 131072, 0.75


def profile_record(kernel):
    """The committed rocprofv3 record of `kernel` (profiles/traffic.json), or None when the kernel's
    sources have changed since it was taken."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[kernel]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    return rec if h.hexdigest() == rec["source_sha256"] else None


def profiled_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by what the counter reads for a plain device copy of known size), or None
    when the kernel's sources have changed since those counters were taken."""
    rec = profile_record(kernel)
    return rec["traffic_bytes"] if rec else None


def profiled_counters(kernel):
    """MFMA work and busy fraction and LDS bank conflicts of `kernel` per launch, from the committed
    rocprofv3 SQ counter pass (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops, SQ_VALU_MFMA_BUSY_CYCLES over
    4 SIMDs x SQ_BUSY_CU_CYCLES, SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE), or None."""
    rec = profile_record(kernel)
    return rec.get("sq") if rec else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "mla", "backward", "chunked"], default="all",
                    help="restrict the timed step (for profiling runs; backward: the prefill's backward with "
                         "the forward's skip mask at the calibrated lambda; chunked: the chunked prefill against "
                         "the paged cache)")
    ap.add_argument("--quick", action="store_true",
                    help="only the timed step (no 128K decode, latent decode or calibration sweep)")
    ap.add_argument("--profile-only", action="store_true",
                    help="profiling run: calibration pass, warm-up and timed steps only (no dense or diagnostic "
                         "launches, so each kernel's profiler average is the timed average), plus a plain "
                         "256 MiB device copy per step whose byte counters scale the profiler's traffic counters")
    return ap.parse_args()


# ------------------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the prefill workload (run before the GPU is
# touched, so worker processes can be forked safely)
# ------------------------------------------------------------------------------------------------

_CPU_INPUT = None  # (q, k, v) fp64 arrays, inherited by the forked workers


def _oracle_worker(args):
    from threadpoolctl import threadpool_limits
    import oracle
    qt, ln_lam = args
    q, k, v = _CPU_INPUT
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.prefill_tile(q, k, v, 0, 0, qt, causal=True, block_q=P_BLK, block_k=P_BLK, num_splits=1,
                            ln_lam=ln_lam)
        return time.perf_counter() - t0


def cpu_baseline(seconds: float):
    import multiprocessing as mp

    import numpy as np
    import torch

    import synth
    import oracle
    global _CPU_INPUT
    # every core this process may run on, up to 16: the host's CPU share of one GPU on the box
    avail = len(os.sched_getaffinity(0))
    cores = min(16, avail)
    # one kv head's keys at the full length, one q head of it; tiles at the causal end (256 blocks)
    inp = synth.prefill_inputs(batch=1, hq=1, hkv=1, L=P_L, d=P_D, block_k=P_BLK, window=True,
                               seed=2000, device="cpu")
    q = inp.q.float().double().numpy()
    k = inp.k.float().double().numpy()
    v = inp.v.float().double().numpy()
    # the benchmark's operating point on these inputs: ln(lambda) for 75 % sparsity from the critical
    # values of an 8-tile sample, the same recipe as the GPU calibration, in the oracle's arithmetic
    nqt = P_L // P_BLK
    crit = []
    for i in range(CALIB_TILES):
        qt = int((i + 0.5) * nqt / CALIB_TILES)
        rows = np.arange(qt * P_BLK, (qt + 1) * P_BLK)
        vis = oracle.blasst_oracle.causal_visible(rows, P_L, P_L, P_L)
        _, c = oracle.keep_mask_closed_form(q[0, 0, rows], k[0, 0], vis, P_BLK, 1, -math.inf, 1.0 / math.sqrt(P_D))
        crit.append(c[~np.isnan(c)])
    ln_lam = oracle.quantile_ln_lambda(np.concatenate(crit), P_TARGET)
    _CPU_INPUT = (q, k, v)
    # size the sample: time one tile, then run enough tiles for about `seconds` of wall time
    t_one = _oracle_worker((255, ln_lam))
    n_tiles = max(cores, int(seconds * cores / max(t_one, 1e-3)))
    n_tiles = min(n_tiles, 4096)
    qts = [255 - (i % 64) for i in range(n_tiles)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_worker, [(qt, ln_lam) for qt in qts], chunksize=1)
    wall = time.perf_counter() - t0
    # dense-equivalent flops of the sampled tiles: 4 * d * visible (row, key) pairs
    flops = 0.0
    for qt in qts:
        r0 = qt * P_BLK
        pairs = sum(r + 1 for r in range(r0, r0 + P_BLK))
        flops += 4.0 * P_D * pairs
    model = open("/proc/cpuinfo").read().split("model name")[1].split("\n")[0].strip(" :\t") \
        if os.path.exists("/proc/cpuinfo") else "unknown"
    return {
        "value": flops / wall / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": cores, "kind": "oracle",
        "sample": f"{n_tiles} prefill query tiles of 128 rows x up to 32768 keys (q tiles 192-255 of one "
                  f"head), lambda={math.exp(ln_lam):.5g} calibrated for {P_TARGET:.0%} sparsity on an 8-tile "
                  f"sample as on the GPU; fp64 numpy, one BLAS thread per worker on {cores} of the {avail} cores "
                  f"this process may use (16 = the host CPU share of one GPU); {wall:.1f} s; CPU {model}",
    }


# ------------------------------------------------------------------------------------------------
# GPU side
# ------------------------------------------------------------------------------------------------

def stratified_tiles(torch, nqt, n_heads, count, seed):
    """Seeded calibration sample: random heads, query tiles spread evenly over the sequence."""
    g = torch.Generator().manual_seed(seed)
    heads = torch.randint(0, n_heads, (count,), generator=g).tolist()
    tiles = [int((i + 0.5) * nqt / count) for i in range(count)]
    return list(zip(heads, tiles))


class Prefill:
    def __init__(self, m, torch, synth, L=P_L, seed=None, head_strength=None):
        self.m = m
        self.torch = torch
        dev = "cuda"
        self.L = L
        seed = synth.config_seed(2) if seed is None else seed
        self.inp = synth.prefill_inputs(batch=P_B, hq=P_HQ, hkv=P_HKV, L=L, d=P_D, block_k=P_BLK,
                                        window=True, seed=seed, device=dev, head_strength=head_strength)
        self.nqt = L // P_BLK
        self.nkb = L // P_BLK
        self.o = torch.empty(P_B, P_HQ, L, P_D, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(P_B, P_HQ, L, dtype=torch.float32, device=dev)
        self.live = P_B * P_HQ * self.nqt * (self.nqt + 1) // 2
        self.dense_flops = 4.0 * P_B * P_HQ * P_D * L * (L + 1) / 2
        # every input read once and every output written once (bf16 q, k, v, o; fp32 lse)
        self.min_bytes = 2 * P_B * L * P_D * (2 * P_HQ + 2 * P_HKV) + 4 * P_B * P_HQ * L

    def run(self, lam, **diag):
        self.m.blasst_prefill(self.inp.q, self.inp.k, self.inp.v, self.o, causal=True, block_q=P_BLK,
                              block_k=P_BLK, lam=lam, lse=self.lse, **diag)

    def run_no_decision(self):
        self.m.blasst_prefill(self.inp.q, self.inp.k, self.inp.v, self.o, causal=True, block_q=P_BLK,
                              block_k=P_BLK, no_decision=True, lse=self.lse)

    def decision_overhead(self, steps):
        """The same dense work with and without the decision logic: lambda = 0 (votes taken, every
        block kept) against threshold mode NONE (the kernel variant without votes)."""
        t0 = timed(self.torch, lambda: self.run(0.0), steps)
        t1 = timed(self.torch, self.run_no_decision, steps)
        t0 = min(t0, timed(self.torch, lambda: self.run(0.0), steps))
        t1 = min(t1, timed(self.torch, self.run_no_decision, steps))
        return {"lambda0_ms": round(t0, 4), "no_decision_ms": round(t1, 4),
                "no_decision_over_lambda0_throughput": round(t1 / t0, 4)}

    def v_staging_ablation(self, lam, steps):
        """What not loading the V blocks of skipped blocks is worth: the same threshold with V staged
        for every live block (the pages' policy) against V staged for kept blocks only."""
        kept = timed(self.torch, lambda: self.run(lam), steps)
        every = timed(self.torch, lambda: self.run(lam, v_staging=1), steps)
        kept = min(kept, timed(self.torch, lambda: self.run(lam), steps))
        every = min(every, timed(self.torch, lambda: self.run(lam, v_staging=1), steps))
        dense = timed(self.torch, lambda: self.run(0.0), steps)
        return {"v_kept_only_ms": round(kept, 4), "v_every_block_ms": round(every, 4),
                "speedup_from_skipping_v_loads": round(every / kept, 3),
                "speedup_vs_dense_with_v_every_block": round(dense / every, 3), "lambda": lam}

    def head_stats(self, lam):
        """Distribution over q heads of the sparsity one threshold gives each head (per-head counters)."""
        from long_context_online_amd import analysis
        h = self.torch.zeros(P_B, P_HQ, 2, dtype=self.torch.int64, device="cuda")
        self.run(lam, head_counters=h)
        self.torch.cuda.synchronize()
        st = analysis.head_sparsity_stats(h)
        return {k: (round(v, 4) if isinstance(v, float) else
                    [round(x, 3) for x in v] if isinstance(v, list) else v) for k, v in st.items()}

    def stats(self):
        """Stats pass (QK^T, block maxima and decisions only): critical values of every tile."""
        torch = self.torch
        crit = torch.empty(P_B, P_HQ, self.nqt, self.nkb, dtype=torch.float32, device="cuda")
        self.m.blasst_prefill(self.inp.q, self.inp.k, self.inp.v, None, causal=True, block_q=P_BLK,
                              block_k=P_BLK, lam=0.0, crit=crit, stats_only=True)
        torch.cuda.synchronize()
        return crit

    def calibrate(self, target, crit=None):
        """ln(lambda) at the target sparsity from the critical values of an 8-tile (1024-row) sample."""
        crit = self.stats() if crit is None else crit
        sample = self.torch.stack([crit[0, h, t] for h, t in stratified_tiles(self.torch, self.nqt, P_HQ,
                                                                               CALIB_TILES, 4242)])
        return math.exp(self.m.blasst_calib_quantile(sample.cpu().numpy(), target))

    def measure(self, lam, steps):
        torch = self.torch
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.run(lam, counters=cnt)
        torch.cuda.synchronize()
        live, skipped = int(cnt[0]), int(cnt[1])
        sparse_ms = timed(torch, lambda: self.run(lam), steps)
        dense_ms = timed(torch, lambda: self.run(0.0), steps)
        return {"ms": round(sparse_ms, 4), "dense_ms": round(dense_ms, 4),
                "speedup_vs_dense": round(dense_ms / sparse_ms, 3),
                "dense_equiv_tflops": round(self.dense_flops / (sparse_ms * 1e-3) / 1e12, 2),
                "dense_tflops": round(self.dense_flops / (dense_ms * 1e-3) / 1e12, 2),
                "lambda": lam, "sparsity": round(skipped / live, 4)}

    def deviation_from_dense(self, lam):
        """max |O(lambda) - O(0)| over every output element (both bf16, as the benchmark writes them)."""
        self.run(0.0)
        dense = self.o.float().clone()
        self.run(lam)
        dev = (self.o.float() - dense).abs()
        r = {"max_abs_dev_from_dense": round(float(dev.max()), 5),
             "mean_abs_dev_from_dense": round(float(dev.mean()), 6)}
        del dense, dev
        return r


class Decode:
    def __init__(self, m, torch, synth, ctx=D_CTX, latent=False, seed=None, num_q_tokens=None, tile_rows=None,
                 splits=None):
        self.m = m
        self.torch = torch
        self.latent = latent
        self.splits = splits if splits is not None else (M_SPLITS if latent else D_SPLITS)
        self.ctx = ctx
        self.T = 1 if num_q_tokens is None else num_q_tokens
        dev = "cuda"
        if latent:
            self.B, self.Hq, self.Hkv, self.D, self.Dv, self.tile_rows = M_B, M_HQ, 1, M_D, M_DV, M_HQ
        else:
            self.B, self.Hq, self.Hkv, self.D, self.Dv, self.tile_rows = D_B, D_HQ, D_HKV, D_D, D_D, 0
        seed = (synth.config_seed(5) if latent else synth.config_seed(3)) if seed is None else seed
        self.d = synth.decode_inputs(batch=self.B, hq=self.Hq, hkv=self.Hkv, ctx=ctx, d=self.D, dv=self.Dv,
                                     page_size=D_PAGE, block_k=D_BLK, window=True, seed=seed, device=dev,
                                     latent=latent, num_q_tokens=num_q_tokens)
        if tile_rows is not None:
            self.tile_rows = tile_rows
        rows = tuple(self.d.q.shape[:-1])
        self.o = torch.empty(rows + (self.Dv,), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(rows, dtype=torch.float32, device=dev)
        self.nkb = -(-(self.d.block_table.shape[1] * D_PAGE) // D_BLK)
        n = m.blasst_decode_workspace_size(self.d.q, self.d.k_cache, self.d.v_cache_t, self.d.block_table,
                                           self.d.seq_lens, self.o, **self._kw(0.0))
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def _kw(self, lam):
        return dict(page_size=D_PAGE, block_k=D_BLK, num_splits=self.splits, lam=lam, lse=self.lse,
                    tile_rows=self.tile_rows, head_dim_v=self.Dv)

    def run(self, lam, **diag):
        d = self.d
        self.m.blasst_decode(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, self.o, workspace=self.ws,
                             **self._kw(lam), **diag)

    def run_no_decision(self):
        d = self.d
        kw = self._kw(0.0)
        del kw["lam"]
        self.m.blasst_decode(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, self.o, workspace=self.ws,
                             no_decision=True, **kw)

    def decision_overhead(self, steps):
        """The same dense work with and without the decision logic: lambda = 0 (every block voted on
        and kept) against threshold mode NONE (the kernel variant without votes)."""
        t0 = timed(self.torch, lambda: self.run(0.0), steps)
        t1 = timed(self.torch, self.run_no_decision, steps)
        t0 = min(t0, timed(self.torch, lambda: self.run(0.0), steps))
        t1 = min(t1, timed(self.torch, self.run_no_decision, steps))
        return {"lambda0_ms": round(t0, 4), "no_decision_ms": round(t1, 4),
                "no_decision_over_lambda0_throughput": round(t1 / t0, 4)}

    def deviation_from_dense(self, lam):
        """max |O(lambda) - O(0)| over every output element (both bf16, as the benchmark writes them):
        what skipping costs in output terms at this operating point."""
        self.run(0.0)
        dense = self.o.float().clone()
        self.run(lam)
        dev = (self.o.float() - dense).abs()
        r = {"max_abs_dev_from_dense": round(float(dev.max()), 5),
             "mean_abs_dev_from_dense": round(float(dev.mean()), 6)}
        del dense, dev
        return r

    def mask_shape(self):
        G = self.Hq // self.Hkv
        return (self.B, self.Hkv, G // self.tile_rows if self.tile_rows else 1, self.nkb)

    def calibrate(self, target):
        """ln(lambda) at the target sparsity from the critical values of every tile of the batch
        (32 x 8 tiles of 4 rows, or 64 tiles of 128 rows: the ~1000-row sample)."""
        torch = self.torch
        crit = torch.empty(*self.mask_shape(), dtype=torch.float32, device="cuda")
        self.run(0.0, crit=crit, stats_only=True)
        torch.cuda.synchronize()
        return math.exp(self.m.blasst_calib_quantile(crit.cpu().numpy(), target))

    def bytes_moved(self, mask):
        """HBM bytes the kernel has to move: all K of every sequence, V of kept blocks (none extra
        for latent attention, where V is part of K), q, the page table, the per-split partials
        (written and read back) and the output."""
        kept = int((mask == 0).sum())
        k_bytes = self.B * self.Hkv * self.ctx * self.D * 2
        v_bytes = 0 if self.latent else kept * D_BLK * self.Dv * 2     # every block is full here
        rows = self.B * self.T * self.Hq          # query rows (tokens x heads)
        q_bytes = rows * self.D * 2
        table = self.d.block_table.numel() * 4
        parts = rows * self.splits * (self.Dv + 1) * 4 * 2
        out = rows * self.Dv * 2 + rows * 4
        dense_v = 0 if self.latent else self.B * self.Hkv * self.ctx * self.Dv * 2
        return (k_bytes + v_bytes + q_bytes + table + parts + out,
                k_bytes + dense_v + q_bytes + table + parts + out)

    def measure(self, lam, steps, ms=None):
        torch = self.torch
        mask = torch.empty(*self.mask_shape(), dtype=torch.uint8, device="cuda")
        self.run(lam, skip_mask=mask)
        torch.cuda.synchronize()
        mh = mask.cpu().numpy()
        kept, live = int((mh == 0).sum()), int((mh != 2).sum())
        moved, dense_bytes = self.bytes_moved(mh)
        sparse_ms = timed(torch, lambda: self.run(lam), steps) if ms is None else ms
        dense_ms = timed(torch, lambda: self.run(0.0), steps)
        r = {"ms": round(sparse_ms, 4), "dense_ms": round(dense_ms, 4),
             "speedup_vs_dense": round(dense_ms / sparse_ms, 3),
             "hbm_gbps": round(moved / (sparse_ms * 1e-3) / 1e9, 1),
             "dense_hbm_gbps": round(dense_bytes / (dense_ms * 1e-3) / 1e9, 1),
             "bytes_moved": moved, "lambda": lam, "a": lam * self.ctx, "sparsity": round(1.0 - kept / live, 4)}
        if self.latent:
            blocks = live
            flops = blocks * D_BLK * self.Hq * (self.D * 2) + kept * D_BLK * self.Hq * (self.Dv * 2)
            r["mfma_tflops"] = round(flops / (sparse_ms * 1e-3) / 1e12, 2)
        return r


class PagedPrefill:
    """Chunked prefill against the paged cache: C_B sequences whose C_L-token contexts end with a
    C_T-token chunk (the queries), 32 q / 8 kv heads, d 128, 16-token pages in a permuted pool."""

    def __init__(self, m, torch, synth, seed=None):
        self.m, self.torch = m, torch
        seed = synth.config_seed(6) if seed is None else seed
        self.d = synth.decode_inputs(batch=C_B, hq=P_HQ, hkv=P_HKV, ctx=C_L, d=P_D, page_size=D_PAGE,
                                     block_k=P_BLK, window=True, seed=seed, device="cuda", num_q_tokens=C_T)
        self.q = self.d.q.permute(0, 2, 1, 3)
        self.o = torch.empty(C_B, P_HQ, C_T, P_D, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(C_B, P_HQ, C_T, dtype=torch.float32, device="cuda")
        self.nqt = C_T // P_BLK
        self.nkb = -(-(self.d.block_table.shape[1] * D_PAGE) // P_BLK)
        pairs = C_T * (C_L - C_T) + C_T * (C_T + 1) // 2
        self.dense_flops = 4.0 * C_B * P_HQ * P_D * pairs

    def run(self, lam, **diag):
        d = self.d
        self.m.blasst_prefill_paged(self.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, self.o, lam=lam,
                                    lse=self.lse, **diag)

    def calibrate(self, target):
        torch = self.torch
        crit = torch.empty(C_B, P_HQ, self.nqt, self.nkb, dtype=torch.float32, device="cuda")
        d = self.d
        self.m.blasst_prefill_paged(self.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, None, lam=0.0,
                                    crit=crit, stats_only=True)
        torch.cuda.synchronize()
        g = torch.Generator().manual_seed(4343)
        picks = [(int(torch.randint(0, C_B, (1,), generator=g)), int(torch.randint(0, P_HQ, (1,), generator=g)),
                  int((i + 0.5) * self.nqt / CALIB_TILES)) for i in range(CALIB_TILES)]
        sample = torch.stack([crit[b, h, t] for b, h, t in picks])
        return math.exp(self.m.blasst_calib_quantile(sample.cpu().numpy(), target))

    def measure(self, lam, steps):
        torch = self.torch
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.run(lam, counters=cnt)
        torch.cuda.synchronize()
        live, skipped = int(cnt[0]), int(cnt[1])
        sparse_ms = timed(torch, lambda: self.run(lam), steps)
        dense_ms = timed(torch, lambda: self.run(0.0), steps)
        return {"ms": round(sparse_ms, 4), "dense_ms": round(dense_ms, 4),
                "speedup_vs_dense": round(dense_ms / sparse_ms, 3),
                "dense_equiv_tflops": round(self.dense_flops / (sparse_ms * 1e-3) / 1e12, 2),
                "dense_tflops": round(self.dense_flops / (dense_ms * 1e-3) / 1e12, 2),
                "lambda": lam, "sparsity": round(skipped / live, 4),
                "workload": f"chunked prefill against the paged cache: {C_B} sequences, {C_L}-token contexts "
                            f"ending with a {C_T}-token chunk, 32 q / 8 kv heads, d 128, 16-token pages"}


class Backward:
    """The backward of the bench prefill (sparsity-aware training): gradients with the forward's
    skip mask at the given lambda, bf16 gradients, the forward's output in bf16.  Dense-equivalent
    FLOPs follow the usual count for attention backward, five products of the forward's size (QK^T
    recomputed, dP, dV, dQ, dK); the kernels issue seven (the dQ kernel recomputes QK^T and dP), on
    the kept tile-blocks only."""

    def __init__(self, m, torch, pre, lam):
        self.m, self.torch, self.pre, self.lam = m, torch, pre, lam
        inp = pre.inp
        B, Hq, L, D = inp.q.shape
        self.mask = torch.empty(B, Hq, pre.nqt, pre.nkb, dtype=torch.uint8, device="cuda")
        pre.run(lam, skip_mask=self.mask)
        g = torch.Generator(device="cuda").manual_seed(4321)
        self.dout = torch.randn(pre.o.shape, generator=g, device="cuda").to(torch.bfloat16)
        self.grads = (torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v))
        self.args = (inp.q, inp.k, inp.v, pre.o, self.dout, pre.lse) + self.grads
        n = m.blasst_prefill_backward_workspace_size(*self.args, causal=True)
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def run(self, sparse=True):
        self.m.blasst_prefill_backward(*self.args, causal=True, skip_mask=self.mask if sparse else None,
                                       workspace=self.ws)

    def measure(self, steps, ms=None):
        torch = self.torch
        self.run()
        self.run(False)
        sparse_ms = timed(torch, self.run, steps) if ms is None else ms
        dense_ms = timed(torch, lambda: self.run(False), steps)
        mh = self.mask.cpu().numpy()
        live, kept = int((mh != 2).sum()), int((mh == 0).sum())
        dense_flops = 2.5 * self.pre.dense_flops
        issued = 7 * 2.0 * P_BLK * P_BLK * P_D * kept
        return {"ms": round(sparse_ms, 4), "dense_ms": round(dense_ms, 4),
                "speedup_vs_dense": round(dense_ms / sparse_ms, 3), "sparsity": round(1 - kept / live, 4),
                "lambda": self.lam, "dense_equiv_tflops": round(dense_flops / (sparse_ms * 1e-3) / 1e12, 2),
                "dense_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
                "issued_tflops": round(issued / (sparse_ms * 1e-3) / 1e12, 2),
                "workload": "the bench prefill's backward: dQ, dK, dV (bf16) from bf16 O and dO, forward skip mask"}


SWEEP_TARGETS = (0.4, 0.5, 0.6, 0.7, 0.8, 0.9)


def sparsity_sweep(obj, steps):
    """Speedup over lambda = 0 at calibrated target sparsities 40 ... 90 % (the layout of the pages'
    speedup-versus-sparsity table); lambda is capped at 1, so high targets may not be reachable and
    the achieved sparsity is what the line reports."""
    out = []
    for t in SWEEP_TARGETS:
        lam = obj.calibrate(t)
        r = obj.measure(lam, steps)
        out.append({"target": t, "sparsity": r["sparsity"], "speedup_vs_dense": r["speedup_vs_dense"],
                    "ms": r["ms"], "dense_ms": r["dense_ms"], "lambda": lam})
    return out


def head_heterogeneity(m, torch, synth, pre, lam_p, steps):
    """Per-head sparsity under one threshold: the bench workload (heads alike) and the same shape
    with heads of different peakedness (head strengths spread geometrically over 0.25 ... 2, in a
    seeded order), each with lambda calibrated for 75% overall sparsity."""
    out = {"homogeneous": pre.head_stats(lam_p)}
    g = torch.Generator().manual_seed(synth.config_seed(2, 7))
    perm = torch.randperm(P_HQ, generator=g).tolist()
    strength = [0.25 * 8.0 ** (perm[h] / (P_HQ - 1)) for h in range(P_HQ)]
    het = Prefill(m, torch, synth, seed=synth.config_seed(2, 7), head_strength=strength)
    lam = het.calibrate(P_TARGET)
    r = het.measure(lam, steps)
    r["head_strength"] = [round(c, 3) for c in strength]
    r["per_head"] = het.head_stats(lam)
    out["heterogeneous"] = r
    del het
    torch.cuda.empty_cache()
    return out


def timed(torch, fn, steps):
    """Average time of fn over `steps` calls (HIP events on torch's current stream, which is the
    stream the library launches on)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def calibration_sweep(m, torch, synth, steps):
    """Calibration: stats pass per L, 8-tile sample, quantile inversion per target s, least-squares
    fit of lambda * L = alpha * exp(beta * s), achieved-vs-target sparsity of the fitted thresholds on
    every tile, and the long prefill at L = 131072, s = 0.75."""
    import numpy as np
    pts, crits = [], {}
    final = None
    for i, L in enumerate(C_L_VALUES):
        p = Prefill(m, torch, synth, L=L, seed=synth.config_seed(4, i))
        crit = p.stats()
        for s in C_S_VALUES:
            pts.append((L, s, p.calibrate(s, crit=crit)))
        c = crit.cpu().numpy().ravel()
        crits[L] = c[~np.isnan(c)]
        if L == C_FINAL_L:
            final = p
        else:
            del p
        del crit
        torch.cuda.empty_cache()
    L_arr, s_arr, lam_arr = (np.array([x[k] for x in pts], dtype=np.float64) for k in range(3))
    alpha, beta, rmse = m.blasst_calibrate(L_arr, s_arr, lam_arr)
    table = []
    errs = []
    for L in C_L_VALUES:
        row = {"L": L}
        for s in C_S_VALUES:
            lam = m.blasst_lambda_for(alpha, beta, s, L)
            ach = float(np.mean(crits[L] < math.log(lam)))
            row[f"s{s}"] = round(ach, 4)
            errs.append(abs(ach - s))
        table.append(row)
    lam_final = m.blasst_lambda_for(alpha, beta, C_FINAL_S, C_FINAL_L)
    fin = final.measure(lam_final, max(2, steps // 3))
    fin["target_sparsity"] = C_FINAL_S
    fin["threshold"] = "fitted model alpha * exp(beta * s) / L"
    lam_direct = final.calibrate(C_FINAL_S)
    fin_direct = final.measure(lam_direct, max(2, steps // 3))
    fin_direct["target_sparsity"] = C_FINAL_S
    fin_direct["threshold"] = "quantile of the 8-tile sample at L = 131072"
    return {"alpha": alpha, "beta": beta, "fit_rmse_ln_lambdaL": round(rmse, 4),
            "points": [{"L": int(L), "s": s, "lambda": lam} for (L, s, lam) in pts],
            "achieved_sparsity_with_fit": table, "mean_abs_sparsity_error": round(float(np.mean(errs)), 4),
            "max_abs_sparsity_error": round(float(np.max(errs)), 4),
            "prefill_131072_s075": fin,
            "prefill_131072_s075_sample_calibrated": fin_direct,
            "workload": "GQA 32 q / 8 kv heads, d 128, bf16, causal, 128x128 blocks; L in 4K..128K; "
                        "s in {0.3, 0.5, 0.7}; 8-tile (1024-row) sample per L"}


def percentiles(xs):
    """p10 / p50 / p90 of per-launch times (ms) from the timed steps (nearest rank)."""
    ys = sorted(xs)
    pick = lambda q: ys[min(len(ys) - 1, max(0, int(math.ceil(q * len(ys))) - 1))]
    return [round(pick(0.1), 4), round(pick(0.5), 4), round(pick(0.9), 4)]


def stream_ceilings(torch, x):
    """Read-only streaming ceilings from this package's own probe kernels (libblasst_ceiling.so:
    16-byte non-temporal loads, nothing written but one word per thread) over the 4 GiB buffer x:
    a contiguous sweep, and 4 KB pages in a seeded random order (the access pattern of a paged KV
    cache of 16-token pages of a 128-dim bf16 head).  Best over a few grid sizes."""
    import ctypes
    path = os.path.join(ROOT, "long_context_online_amd", "libblasst_ceiling.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m long_context_online_amd.build`")
    lib = ctypes.CDLL(path)
    lib.blasst_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_void_p]
    lib.blasst_ceiling_stream_pages.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int, ctypes.c_void_p]
    nbytes = x.numel() * x.element_size()
    page = lib.blasst_ceiling_page_bytes()
    n_pages = nbytes // page
    gen = torch.Generator().manual_seed(11)
    table = torch.randperm(n_pages, generator=gen).to(torch.int32).to("cuda")
    grids = (1024, 2048, 4096)
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run(fn):
        rc = fn()
        if rc != 0:
            raise RuntimeError(f"streaming ceiling kernel failed: {rc}")

    res = {}
    for name, nb, call in (
            ("read_contiguous_4gib_gbps", nbytes,
             lambda g: lib.blasst_ceiling_stream_read(x.data_ptr(), nbytes, out.data_ptr(), g, stream)),
            ("read_4kb_pages_random_4gib_gbps", n_pages * page,
             lambda g: lib.blasst_ceiling_stream_pages(x.data_ptr(), table.data_ptr(), n_pages, out.data_ptr(), g,
                                                       stream))):
        best = 0.0
        for g in grids:
            run(lambda: call(g))
            ms = timed(torch, lambda: run(lambda: call(g)), 10)
            best = max(best, nb / (ms * 1e-3) / 1e9)
        res[name] = round(best, 1)
    del table, out
    return res


def practical_ceilings(torch):
    """Measured ceilings on this GPU, as context for the roofline fractions: a bf16 GEMM through the
    vendor BLAS (torch.matmul, 8192^3), a plain device-to-device copy of 4 GiB, library reductions
    over it, and this package's read-only streaming probes (contiguous and random 4 KB pages)."""
    out = {}
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    ms = timed(torch, lambda: torch.matmul(a, b), 10)
    out["bf16_gemm_8192_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    del a, b
    x = torch.empty(2 * 1024 ** 3, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    y.copy_(x)
    ms = timed(torch, lambda: y.copy_(x), 5)
    out["copy_4gib_gbps_read_plus_write"] = round(2 * x.numel() * 2 / (ms * 1e-3) / 1e9, 1)
    del y
    # library reductions over the same 4 GiB (output a few bytes); the best of two
    best = 0.0
    for fn in (lambda: torch.amax(x), lambda: torch.sum(x, dtype=torch.float32)):
        fn()
        ms = timed(torch, fn, 5)
        best = max(best, x.numel() * 2 / (ms * 1e-3) / 1e9)
    out["reduction_4gib_gbps"] = round(best, 1)
    out.update(stream_ceilings(torch, x))
    del x
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the multi-GPU path (context sharding "
                                   "of decode with an all-gather of per-split partials) is not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    cpu = None if (args.no_cpu_baseline or args.profile_only) else cpu_baseline(args.cpu_seconds)

    import torch

    import long_context_online_amd as m
    import synth

    m.lib()
    torch.cuda.init()
    pre = Prefill(m, torch, synth) if args.only in ("all", "prefill") else None
    if args.only == "mla":  # the latent decode as the timed step (profiling runs)
        dec = Decode(m, torch, synth, ctx=M_CTX, latent=True)
    else:
        dec = Decode(m, torch, synth) if args.only in ("all", "decode") else None
    bwd = None
    if args.only == "backward":  # the prefill's backward as the timed step
        base = Prefill(m, torch, synth)
        bwd = Backward(m, torch, base, base.calibrate(P_TARGET))
    chk = PagedPrefill(m, torch, synth) if args.only == "chunked" else None  # chunked prefill as the timed step
    torch.cuda.synchronize()

    lam_p = pre.calibrate(P_TARGET) if pre else None
    lam_d = (dec.calibrate(M_TARGETS[-1] if dec.latent else D_TARGET)) if dec else None
    lam_c = chk.calibrate(P_TARGET) if chk else None

    def step():
        if pre:
            pre.run(lam_p)
        if chk:
            chk.run(lam_c)
        if dec:
            dec.run(lam_d)
        if bwd:
            bwd.run()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_only:
        ref_src = torch.empty(128 * 1024 * 1024, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        ref_dst = torch.empty_like(ref_src)
    # timed region: exactly `steps` steps, with per-kernel events inside
    ev = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        if pre:
            pre.run(lam_p)
        if chk:
            chk.run(lam_c)
        e[1].record()
        if dec:
            dec.run(lam_d)
        if bwd:
            bwd.run()
        e[2].record()
        ev.append(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pre_all = [e[0].elapsed_time(e[1]) for e in ev]
    dec_all = [e[1].elapsed_time(e[2]) for e in ev]
    pre_ms = sum(pre_all) / args.steps
    dec_ms = sum(dec_all) / args.steps
    if args.profile_only:
        for _ in range(args.steps):
            ref_dst.copy_(ref_src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_only": True, "steps": args.steps, "warmup": args.warmup,
                          "prefill_ms": round(pre_ms, 4) if pre else None,
                          "chunked_prefill_ms": round(pre_ms, 4) if chk else None, "chunked_lambda": lam_c,
                          "decode_ms": round(dec_ms, 4) if dec else None,
                          "backward_ms": round(dec_ms, 4) if bwd else None,
                          "prefill_lambda": lam_p, "decode_lambda": lam_d,
                          "reference_copy_bytes": 2 * ref_src.numel() * ref_src.element_size()}))
        return

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": round(wall_ms, 4), "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    config = {"workload": "", "parallelism": "none (1 GPU)"}
    if pre:
        r = pre.measure(lam_p, max(3, args.steps // 2))
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        pre.run(lam_p, counters=cnt)
        torch.cuda.synchronize()
        live, skipped = int(cnt[0]), int(cnt[1])
        kept = live - skipped
        alg_flops = (live + kept) * 2.0 * P_BLK * P_BLK * P_D
        tflops = pre.dense_flops / (pre_ms * 1e-3) / 1e12
        achieved = alg_flops / (pre_ms * 1e-3) / 1e12
        result.update({"value": round(tflops, 2), "unit": "TFLOP/s (dense-equivalent)"})
        r.update({"ms": round(pre_ms, 4), "speedup_vs_dense": round(r["dense_ms"] / pre_ms, 3),
                  "dense_equiv_tflops": round(tflops, 2), "target_sparsity": P_TARGET,
                  "live_tile_blocks": live, "frac_of_bf16_peak_dense_equiv": round(tflops / PEAK_BF16_TFLOPS, 4)})
        r["timed_step_ms_p10_p50_p90"] = percentiles(pre_all)
        result["prefill"] = r
        result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                              "traffic": profiled_traffic("prefill_bf16_kernel<128, 128, 2, false, false, true, false, false>"),
                              "traffic_unit": "HBM bytes per launch",
                              "counters": profiled_counters("prefill_bf16_kernel<128, 128, 2, false, false, true, false, false>"),
                              "min_bytes": pre.min_bytes,
                              "kernel": "prefill_bf16_kernel<128, 128, 2, bf16 out>",
                              "algorithmic": "QK^T on every live 128x128 tile-block + PV on kept ones, "
                                             "4.19 MFLOP each",
                              "time_source": "mean launch time from HIP events on the launch stream over the "
                                             "timed steps (the profiler's kernel average is in profiles/)"}
        config["workload"] = ("GQA prefill, Llama-3.1-8B-shaped: batch 1, 32 q / 8 kv heads, d 128, L 32768, causal, "
                              "128x128 blocks, bf16 in/out, lambda calibrated for 75% sparsity")
        config.update({"batch": P_B, "seq_len": P_L, "q_heads": P_HQ, "kv_heads": P_HKV, "head_dim": P_D})
        if not args.quick:
            r.update(pre.deviation_from_dense(lam_p))
            lam50 = pre.calibrate(0.5)
            result["prefill_s050"] = pre.measure(lam50, max(3, args.steps // 2))
            result["prefill_s050"]["target_sparsity"] = 0.5
            result["prefill_decision_overhead"] = pre.decision_overhead(max(3, args.steps // 2))
            # the headline step against both dense references: the same kernel at lambda = 0 (speedup_vs_dense)
            # and the variant without any decision logic
            r["speedup_vs_no_decision_dense"] = round(
                result["prefill_decision_overhead"]["no_decision_ms"] / r["ms"], 3)
            result["prefill_v_staging"] = pre.v_staging_ablation(lam_p, max(3, args.steps // 2))
            result["prefill_heads"] = head_heterogeneity(m, torch, synth, pre, lam_p, max(3, args.steps // 2))
            bw = Backward(m, torch, pre, lam_p)
            result["prefill_backward"] = bw.measure(max(3, args.steps // 2))
            del bw
            result["prefill_speedup_vs_sparsity"] = sparsity_sweep(pre, max(3, args.steps // 2))
    if dec:
        r = dec.measure(lam_d, args.steps, ms=dec_ms)
        r.update({"target_sparsity": M_TARGETS[-1] if dec.latent else D_TARGET,
                  "frac_of_hbm_peak": round(r["hbm_gbps"] / PEAK_HBM_GBPS, 4),
                  "workload": (MLA_WORKLOAD if dec.latent else
                               "paged GQA decode: batch 32, 32 q / 8 kv heads, d 128, context 32768, 16-token "
                               "pages, 64-token blocks, 16 splits, bf16")})
        r["timed_step_ms_p10_p50_p90"] = percentiles(dec_all)
        result["decode"] = r
        if not args.quick:
            r.update(dec.deviation_from_dense(lam_d))
        if not args.quick and not dec.latent:
            result["decode_decision_overhead"] = dec.decision_overhead(args.steps)
            result["decode_speedup_vs_sparsity"] = sparsity_sweep(dec, args.steps)
        result["roofline_decode"] = {"bound": "hbm", "achieved": r["hbm_gbps"], "peak": PEAK_HBM_GBPS,
                                     "unit": "GB/s", "frac": round(r["hbm_gbps"] / PEAK_HBM_GBPS, 4),
                                     "traffic": profiled_traffic(DEC_KERNEL[dec.latent]),
                                     "traffic_unit": f"HBM bytes per launch of {DEC_KERNEL[dec.latent]}",
                                     "counters": profiled_counters(DEC_KERNEL[dec.latent]),
                                     "kernel": f"{DEC_KERNEL[dec.latent]} + decode_combine_kernel",
                                     "time_source": "mean time of the split and combine launches from HIP events "
                                                    "on the launch stream over the timed steps"}
        if not pre:
            result.update({"value": r["hbm_gbps"], "unit": "GB/s"})
            config["workload"] = r["workload"]
    if bwd:
        r = bwd.measure(args.steps, ms=dec_ms)
        r["timed_step_ms_p10_p50_p90"] = percentiles(dec_all)
        result["prefill_backward"] = r
        result.update({"value": r["dense_equiv_tflops"], "unit": "TFLOP/s (dense-equivalent, backward)"})
        config["workload"] = r["workload"]
    del pre, dec, bwd
    torch.cuda.empty_cache()
    if not args.quick and args.only == "all":
        d128 = Decode(m, torch, synth, ctx=131072, seed=synth.config_seed(3, 1))
        lam = d128.calibrate(D_TARGET)
        r = d128.measure(lam, args.steps)
        r.update({"target_sparsity": D_TARGET, "frac_of_hbm_peak": round(r["hbm_gbps"] / PEAK_HBM_GBPS, 4)})
        r.update(d128.deviation_from_dense(lam))
        result["decode_131072"] = r
        del d128
        torch.cuda.empty_cache()
        cp = PagedPrefill(m, torch, synth)
        lam = cp.calibrate(P_TARGET)
        r = cp.measure(lam, args.steps)
        r["target_sparsity"] = P_TARGET
        r["profiled_traffic_bytes_per_launch"] = profiled_traffic(CHUNKED_KERNEL)
        r["profiled_counters"] = profiled_counters(CHUNKED_KERNEL)
        result["chunked_prefill"] = r
        del cp
        torch.cuda.empty_cache()
        result["decode_multi_token"] = {}
        for T in (2, 4):
            for sp in (MT_SPLITS, D_SPLITS):
                mt = Decode(m, torch, synth, seed=synth.config_seed(3, 2), num_q_tokens=T, tile_rows=D_HQ // D_HKV,
                            splits=sp)
                lam = mt.calibrate(D_TARGET)
                r = mt.measure(lam, args.steps)
                r.update({"target_sparsity": D_TARGET, "frac_of_hbm_peak": round(r["hbm_gbps"] / PEAK_HBM_GBPS, 4),
                          "splits": sp,
                          "workload": f"the decode workload with {T} query tokens per sequence (the last {T} "
                                      f"positions), tiles of {T} tokens x 4 heads, {sp} splits"})
                result["decode_multi_token"][f"T{T}" if sp == MT_SPLITS else f"T{T}_splits{sp}"] = r
                del mt
                torch.cuda.empty_cache()
        mla = Decode(m, torch, synth, ctx=M_CTX, latent=True)
        result["mla_decode"] = {"workload": MLA_WORKLOAD}
        for tgt in M_TARGETS:
            lam = mla.calibrate(tgt)
            r = mla.measure(lam, args.steps)
            r.update({"target_sparsity": tgt, "frac_of_hbm_peak": round(r["hbm_gbps"] / PEAK_HBM_GBPS, 4),
                      "profiled_traffic_bytes_per_launch": profiled_traffic(DEC_KERNEL[True])})
            r.update(mla.deviation_from_dense(lam))
            result["mla_decode"][f"s{tgt}"] = r
        del mla
        torch.cuda.empty_cache()
        result["mla_decode"]["splits_sweep"] = []
        for sp in (4, 8, 16):
            mla = Decode(m, torch, synth, ctx=M_CTX, latent=True, splits=sp)
            lam = mla.calibrate(M_TARGETS[-1])
            r = mla.measure(lam, args.steps)
            result["mla_decode"]["splits_sweep"].append(
                {"splits": sp, "target": M_TARGETS[-1], "sparsity": r["sparsity"], "ms": r["ms"],
                 "dense_ms": r["dense_ms"], "speedup_vs_dense": r["speedup_vs_dense"], "hbm_gbps": r["hbm_gbps"],
                 "lambda": r["lambda"]})
            del mla
            torch.cuda.empty_cache()
        result["mla_decode"]["multi_token"] = {}
        for T in (2, 4):
            mt = Decode(m, torch, synth, ctx=M_CTX, latent=True, seed=synth.config_seed(5, T), num_q_tokens=T,
                        tile_rows=M_HQ // T, splits=M_SPLITS)
            lam = mt.calibrate(M_TARGETS[-1])
            r = mt.measure(lam, args.steps)
            r.update({"target_sparsity": M_TARGETS[-1], "frac_of_hbm_peak": round(r["hbm_gbps"] / PEAK_HBM_GBPS, 4),
                      "splits": M_SPLITS,
                      "workload": f"the latent decode workload with {T} query tokens per sequence (the last {T} "
                                  f"positions), tiles of {T} tokens x {M_HQ // T} heads, {M_SPLITS} splits"})
            result["mla_decode"]["multi_token"][f"T{T}"] = r
            del mt
            torch.cuda.empty_cache()
        result["calibration"] = calibration_sweep(m, torch, synth, args.steps)
        result["ceilings"] = practical_ceilings(torch)
        # the paged GQA decode against the read rate of its own access pattern (random 4 KB pages)
        paged = result["ceilings"]["read_4kb_pages_random_4gib_gbps"]
        for key in ("decode", "decode_131072"):
            if key in result and paged > 0:
                result[key]["frac_of_paged_read_ceiling"] = round(result[key]["hbm_gbps"] / paged, 4)
    result["config"] = config
    result["context"] = {"pages_prefill_speedup": "1.62x at 74.7% sparsity (B200/H200, pages' abstract)",
                         "pages_decode_speedup": "1.48x at 73.2% sparsity"}
    result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()

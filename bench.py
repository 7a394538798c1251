"""Benchmark of the BLASST hot path on one MI355X.

One step = one sparse prefill of the Llama-3.1-8B-shaped GQA problem (batch 1, 32 q / 8 kv heads,
d = 128, L = 32768, bf16 in, fp32 accumulation, causal, 128 x 128 blocks) at the threshold
calibrated for 75 % sparsity, followed by one sparse paged decode (batch 32, 32 q / 8 kv heads,
d = 128, context 32768, 16-token pages, 64-token blocks, 16 splits) at the threshold calibrated for
73 % sparsity.  Inputs are seeded synthetic tensors resident in HBM before timing starts.

Printed (one JSON line): prefill dense-equivalent TFLOP/s as `value`, decode HBM GB/s (bytes the
kernel actually has to read and write), the speedups over the same kernels at lambda = 0, roofline
fractions, and the fp64 oracle's throughput on the host cores as a baseline.
"""

from __future__ import annotations

import argparse
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
# decode workload
D_B, D_HQ, D_HKV, D_CTX, D_D, D_PAGE, D_BLK, D_SPLITS = 32, 32, 8, 32768, 128, 16, 64, 16
D_TARGET = 0.73
CALIB_TILES = 8  # prefill calibration sample: 8 query tiles of 128 rows (1024 rows)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--only", choices=["all", "prefill", "decode"], default="all",
                    help="restrict the timed step (for profiling runs)")
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
    global _CPU_INPUT
    cores = min(16, len(os.sched_getaffinity(0)))
    # one kv head's keys at the full length, one q head of it; tiles at the causal end (256 blocks)
    inp = synth.prefill_inputs(batch=1, hq=1, hkv=1, L=P_L, d=P_D, block_k=P_BLK, window=True,
                               seed=2000, device="cpu")
    q = inp.q.float().double().numpy()
    k = inp.k.float().double().numpy()
    v = inp.v.float().double().numpy()
    ln_lam = math.log(0.02)
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
                  f"head, lambda=0.02), fp64 numpy, one BLAS thread per worker; {wall:.1f} s; CPU {model}",
    }


# ------------------------------------------------------------------------------------------------
# GPU side
# ------------------------------------------------------------------------------------------------

class Prefill:
    def __init__(self, m, torch, synth):
        self.m = m
        self.torch = torch
        dev = "cuda"
        self.inp = synth.prefill_inputs(batch=P_B, hq=P_HQ, hkv=P_HKV, L=P_L, d=P_D, block_k=P_BLK,
                                        window=True, seed=synth.config_seed(2), device=dev)
        self.nqt = P_L // P_BLK
        self.nkb = P_L // P_BLK
        self.o = torch.empty(P_B, P_HQ, P_L, P_D, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(P_B, P_HQ, P_L, dtype=torch.float32, device=dev)
        self.live = P_B * P_HQ * self.nqt * (self.nqt + 1) // 2
        self.dense_flops = 4.0 * P_B * P_HQ * P_D * P_L * (P_L + 1) / 2

    def run(self, lam, **diag):
        self.m.blasst_prefill(self.inp.q, self.inp.k, self.inp.v, self.o, causal=True, block_q=P_BLK,
                              block_k=P_BLK, lam=lam, lse=self.lse, **diag)

    def calibrate(self, target):
        """Stats pass (QK^T, block maxima and decisions only) -> critical values of a sample of
        8 query tiles (1024 rows) -> ln(lambda) at the target sparsity."""
        torch = self.torch
        crit = torch.empty(P_B, P_HQ, self.nqt, self.nkb, dtype=torch.float32, device="cuda")
        self.m.blasst_prefill(self.inp.q, self.inp.k, self.inp.v, None, causal=True, block_q=P_BLK,
                              block_k=P_BLK, lam=0.0, crit=crit, stats_only=True)
        torch.cuda.synchronize()
        # seeded heads, query tiles spread evenly over the sequence (short and long rows alike)
        g = torch.Generator().manual_seed(4242)
        heads = torch.randint(0, P_HQ, (CALIB_TILES,), generator=g).tolist()
        tiles = [int((i + 0.5) * self.nqt / CALIB_TILES) for i in range(CALIB_TILES)]
        sample = torch.stack([crit[0, h, t] for h, t in zip(heads, tiles)]).cpu().numpy()
        ln_lam = self.m.blasst_calib_quantile(sample, target)
        return math.exp(ln_lam)


class Decode:
    def __init__(self, m, torch, synth):
        self.m = m
        self.torch = torch
        dev = "cuda"
        self.d = synth.decode_inputs(batch=D_B, hq=D_HQ, hkv=D_HKV, ctx=D_CTX, d=D_D, page_size=D_PAGE,
                                     block_k=D_BLK, window=True, seed=synth.config_seed(3), device=dev)
        self.o = torch.empty(D_B, D_HQ, D_D, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(D_B, D_HQ, dtype=torch.float32, device=dev)
        self.nkb = -(-(self.d.block_table.shape[1] * D_PAGE) // D_BLK)
        kw = self._kw(0.0)
        n = m.blasst_decode_workspace_size(self.d.q, self.d.k_cache, self.d.v_cache_t, self.d.block_table,
                                           self.d.seq_lens, self.o, **kw)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def _kw(self, lam):
        return dict(page_size=D_PAGE, block_k=D_BLK, num_splits=D_SPLITS, lam=lam, lse=self.lse)

    def run(self, lam, **diag):
        d = self.d
        self.m.blasst_decode(d.q, d.k_cache, d.v_cache_t, d.block_table, d.seq_lens, self.o, workspace=self.ws,
                             **self._kw(lam), **diag)

    def calibrate(self, target):
        torch = self.torch
        crit = torch.empty(D_B, D_HKV, 1, self.nkb, dtype=torch.float32, device="cuda")
        self.run(0.0, crit=crit, stats_only=True)
        torch.cuda.synchronize()
        return math.exp(self.m.blasst_calib_quantile(crit.cpu().numpy(), target))

    def bytes_moved(self, mask):
        """HBM bytes the kernel must move: all K of every sequence, V of kept blocks, q, the page
        table, the per-split partials (written and read back) and the output."""
        import numpy as np
        kept = int((mask == 0).sum())
        live = int((mask != 2).sum())
        k_bytes = D_B * D_HKV * D_CTX * D_D * 2
        v_bytes = kept * D_BLK * D_D * 2          # every block is full at this context length
        q_bytes = D_B * D_HQ * D_D * 2
        table = self.d.block_table.numel() * 4
        parts = D_B * D_HQ * D_SPLITS * (D_D + 1) * 4 * 2
        out = D_B * D_HQ * D_D * 2 + D_B * D_HQ * 4
        dense = k_bytes * 2 + q_bytes + table + parts + out
        return k_bytes + v_bytes + q_bytes + table + parts + out, dense, kept, live


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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the multi-GPU path (context sharding "
                                   "of decode with an all-gather of per-split partials) is not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    import numpy as np
    import torch

    import long_context_online_amd as m
    import synth

    m.lib()
    torch.cuda.init()
    pre = Prefill(m, torch, synth) if args.only in ("all", "prefill") else None
    dec = Decode(m, torch, synth) if args.only in ("all", "decode") else None
    torch.cuda.synchronize()

    lam_p = pre.calibrate(P_TARGET) if pre else None
    lam_d = dec.calibrate(D_TARGET) if dec else None

    def step():
        if pre:
            pre.run(lam_p)
        if dec:
            dec.run(lam_d)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, with per-kernel events inside
    ev = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        if pre:
            pre.run(lam_p)
        e[1].record()
        if dec:
            dec.run(lam_d)
        e[2].record()
        ev.append(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": round(wall_ms, 4), "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    config = {"workload": "", "parallelism": "none (1 GPU)"}
    if pre:
        mask = torch.empty(P_B, P_HQ, pre.nqt, pre.nkb, dtype=torch.uint8, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        pre.run(lam_p, skip_mask=mask, counters=cnt)
        torch.cuda.synchronize()
        live, skipped = int(cnt[0]), int(cnt[1])
        kept = live - skipped
        dense_ms = timed(torch, lambda: pre.run(0.0), max(3, args.steps // 2))
        alg_flops = (live + kept) * 2.0 * P_BLK * P_BLK * P_D
        tflops = pre.dense_flops / (pre_ms * 1e-3) / 1e12
        achieved = alg_flops / (pre_ms * 1e-3) / 1e12
        result.update({"value": round(tflops, 2), "unit": "TFLOP/s (dense-equivalent)"})
        result["prefill"] = {
            "ms": round(pre_ms, 4), "dense_ms": round(dense_ms, 4), "speedup_vs_dense": round(dense_ms / pre_ms, 3),
            "dense_equiv_tflops": round(tflops, 2), "dense_tflops": round(pre.dense_flops / (dense_ms * 1e-3) / 1e12, 2),
            "lambda": lam_p, "target_sparsity": P_TARGET, "sparsity": round(skipped / live, 4),
            "live_tile_blocks": live, "frac_of_bf16_peak_dense_equiv": round(tflops / PEAK_BF16_TFLOPS, 4),
        }
        result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                              "kernel": "prefill_bf16_kernel<128,128,4,bf16 out>",
                              "algorithmic": "QK^T on every live 128x128 tile-block + PV on kept ones, 4.19 MFLOP each"}
        config["workload"] = ("GQA prefill, Llama-3.1-8B-shaped: batch 1, 32 q / 8 kv heads, d 128, L 32768, causal, "
                              "128x128 blocks, bf16 in/out, lambda calibrated for 75% sparsity")
        config.update({"batch": P_B, "seq_len": P_L, "q_heads": P_HQ, "kv_heads": P_HKV, "head_dim": P_D})
    if dec:
        mask = torch.empty(D_B, D_HKV, 1, dec.nkb, dtype=torch.uint8, device="cuda")
        dec.run(lam_d, skip_mask=mask)
        torch.cuda.synchronize()
        mh = mask.cpu().numpy()
        moved, dense_bytes, kept, live = dec.bytes_moved(mh)
        dense_ms = timed(torch, lambda: dec.run(0.0), max(3, args.steps))
        gbps = moved / (dec_ms * 1e-3) / 1e9
        result["decode"] = {
            "ms": round(dec_ms, 4), "dense_ms": round(dense_ms, 4), "speedup_vs_dense": round(dense_ms / dec_ms, 3),
            "hbm_gbps": round(gbps, 1), "dense_hbm_gbps": round(dense_bytes / (dense_ms * 1e-3) / 1e9, 1),
            "bytes_moved": moved, "lambda": lam_d, "a": lam_d * D_CTX, "target_sparsity": D_TARGET,
            "sparsity": round(1.0 - kept / live, 4), "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "workload": "paged GQA decode: batch 32, 32 q / 8 kv heads, d 128, context 32768, 16-token pages, "
                        "64-token blocks, 16 splits, bf16",
        }
        result["roofline_decode"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None}
        if not pre:
            result.update({"value": round(gbps, 1), "unit": "GB/s"})
            config["workload"] = result["decode"]["workload"]
    result["config"] = config
    result["context"] = {"pages_prefill_speedup": "1.62x at 74.7% sparsity (B200/H200, pages' abstract)",
                         "pages_decode_speedup": "1.48x at 73.2% sparsity"}
    result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()

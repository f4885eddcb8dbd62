"""Benchmark of the MTP verify pass on one MI355X.

Headline: effective weight GB/s of the nvfp4 verify GEMM on the dense
FFN-up shape (K=4096 -> N=14336), M = 8 draft rows, and the M = 1/2/4/8
sweep with the M=8 / M=1 time ratio.  A step is one verify GEMM call over
one batch of activations.

Method:
* R rotating copies of the weights (R * 33 MB >= 1 GiB, four times the
  256 MiB Infinity Cache) so every step streams its weights from HBM;
* the R calls are captured once in a HIP graph (torch.cuda.CUDAGraph) and
  replayed, so host launch overhead does not leak into the timing;
* K timed steps bracketed by torch.cuda.synchronize(); HIP events recorded
  on the launch stream give the average duration per call;
* effective GB/s = algorithmic weight bytes (4-bit codes + E4M3 scales,
  9/16 byte per weight) / time;
* the CPU oracle (fp64, all host threads) runs the same workload once for
  the baseline.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--m", type=int, default=8, help="rows of the headline pass")
    ap.add_argument("--no-sweep", action="store_true", help="skip the M=1/2/4 sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for PMC scaling)")
    return ap.parse_args()


class GemmRunner:
    """R rotating weight copies of one nvfp4 matrix and a captured graph of
    one verify call per copy."""

    def __init__(self, bv, w, x, M, dev):
        self.bv = bv
        self.N, self.K, self.M = w["N"], w["K"], M
        self.bytes_per_call = W.weight_bytes(self.N, self.K)
        self.R = max(2, -(-ROTATE_BYTES // self.bytes_per_call))
        codes = torch.from_numpy(w["codes"]).to(dev)
        scales = torch.from_numpy(w["scales"]).to(dev)
        packed = bv.pack_weights(bv.FMT_NVFP4, codes, scales, self.N, self.K)
        del codes, scales
        self.packed = [packed] + [packed.clone() for _ in range(self.R - 1)]
        self.x = torch.from_numpy(np.ascontiguousarray(x[:M]).view(np.int16)).to(dev)
        self.y = torch.empty((M, self.N), dtype=torch.float32, device=dev)
        self.ws = bv.gemm_workspace(self.N, self.K, dev)
        self.graphs = {}

    def call(self, i):
        self.bv.verify_gemm(self.bv.FMT_NVFP4, self.x, self.packed[i % self.R], self.N, self.K,
                            1.0, y=self.y, ws=self.ws)

    def graph(self, n):
        """A graph of n consecutive calls over the rotating copies."""
        if n not in self.graphs:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for i in range(n):          # warm the launch path outside capture
                    self.call(i)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    self.call(i)
            self.graphs[n] = g
        return self.graphs[n]

    def run(self, steps):
        full, tail = divmod(steps, self.R)
        for _ in range(full):
            self.graph(self.R).replay()
        if tail:
            self.graph(tail).replay()

    def time(self, steps, warmup):
        for n in {self.R, steps % self.R} - {0}:
            self.graph(n)
        self.run(warmup)
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        self.run(steps)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = e0.elapsed_time(e1)
        return wall, ev_ms / steps


def cpu_baseline(cfg, M):
    import oracle
    w = cfg["w"]
    x = cfg["x"][:M]
    threads = max(1, min(16, os.cpu_count() or 1))
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.gemm(w, x, nthreads=threads)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": round(W.weight_bytes(w["N"], w["K"]) / t / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"whole workload (M={M}, K={w['K']}, N={w['N']}), fp64 serial sums with "
                      f"|x*w| bound, {threads} threads, median of 3 runs of {t:.2f}s"}


def copy_calibration(dev):
    """Plain device-to-device copies of a known size (for FETCH_SIZE and
    WRITE_SIZE scaling); returns the bytes moved per copy."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return n


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this verify-pass build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import bit_verify_gemm_amd as bv
    bv.lib()
    dev = torch.device("cuda:0")
    cfg = W.config1(M=8)
    M = args.m

    runner = GemmRunner(bv, cfg["w"], cfg["x"], M, dev)
    wall, per_call_ms = runner.time(args.steps, args.warmup)
    bytes_call = runner.bytes_per_call
    value = bytes_call * args.steps / wall / 1e9
    achieved = bytes_call / (per_call_ms * 1e-3) / 1e9

    sweep = {}
    if not args.no_sweep:
        for m in (1, 2, 4, 8):
            if m == M:
                sweep[str(m)] = {"us_per_call": round(per_call_ms * 1e3, 3),
                                 "gbs": round(achieved, 1)}
                continue
            r = GemmRunner(bv, cfg["w"], cfg["x"], m, dev)
            _, ms = r.time(args.steps, args.warmup)
            sweep[str(m)] = {"us_per_call": round(ms * 1e3, 3),
                             "gbs": round(bytes_call / (ms * 1e-3) / 1e9, 1)}
            del r
            torch.cuda.empty_cache()

    if args.copy_calibration:
        copy_calibration(dev)

    out = {
        "metric": "effective weight GB/s (% of HBM peak) for nvfp4 verify GEMM at M=1/2/4/8",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"nvfp4 verify GEMM, dense FFN-up K=4096 -> N=14336, M={M} "
                               f"bf16 rows, fp32 accumulate",
                   "M": M, "K": 4096, "N": 14336, "weight_bytes_per_call": bytes_call,
                   "rotating_weight_copies": runner.R, "graph_replay": True},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None},
    }
    if sweep:
        out["m_sweep"] = sweep
        if "1" in sweep and "8" in sweep:
            out["m8_over_m1_time"] = round(sweep["8"]["us_per_call"] / sweep["1"]["us_per_call"], 4)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, M)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

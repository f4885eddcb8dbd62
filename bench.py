"""Benchmark of the MTP verify pass on one MI355X.

Headline (one JSON line): effective weight GB/s of the nvfp4 verify GEMM on
the dense FFN-up shape (K=4096 -> N=14336) with M = 8 rows, plus the
M = 1/2/4/8 sweep and the M=8 / M=1 time ratio.  A step is one verify GEMM
call over one batch of activations (this workload's whole pass).

The same run also reports, as context next to the headline, the other
steps of the verify pass at their own workloads:
* the Q4_0 projections of one 27B-class decoder layer (M = 8), one by one
  and with Q|K|V and gate|up fused along N,
* the 5376 -> 262144 LM head (M = 8) and the greedy, rejection and sampled
  (full sampler pipeline, sparse top-k) accept steps on its logits,
* the routed MoE pass (8 tokens, 128 experts, top-8, 2048 -> 768 -> 2048),
  with its unique-expert bytes,
* multi-row verify attention: 8 rows over a 32768-key prefix (32 query heads
  on 8 KV heads of dim 128), with the KV bytes it reads.

Method:
* weights are packed once (mtp_pack_weights, outside the timed region);
* R rotating copies of the weights (R * bytes >= 1 GiB, four times the
  256 MiB Infinity Cache) so every call streams its weights from HBM;
* the headline runs exactly W untimed warm-up calls, then exactly K timed
  calls (--warmup, --steps) launched directly on one stream behind a
  GPU-side lead (a bounded spin kernel recorded before the first event, long
  enough for the host to enqueue all K); HIP events on that stream around
  the K calls give their GPU time, gaps between launches included.
  `value`, `ms_per_step` and `roofline.achieved` all come from that one
  clock; a sustained figure over at least 20 ms of back-to-back calls (HIP
  graph replays) is reported beside it, and the in-kernel average of the
  committed rocprofv3 trace of the same kernel;
* effective GB/s = algorithmic weight bytes (4-bit codes + block scales,
  9/16 byte per weight) / time;
* the CPU oracle (fp64) runs repeated whole passes of the same workload for
  a bounded sample as the baseline, on the host threads this process may
  use (the OMP_NUM_THREADS share where it is set, else every core of its
  affinity mask); os.cpu_count() is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 1 << 30
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_nvfp4_4096x14336_m8_pmc.md")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "gemm_nvfp4_4096x14336_m8_kernel_trace.md")
SUSTAIN_S = 0.020                 # the sustained figure's timed region, at least
ONLY = ("all", "headline", "sweep", "c0", "c2", "c3", "lmhead", "moe", "attn", "kv", "ceiling")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_verify_gemm_amd", "csrc", f)
                  for f in ("engine.h", "device.h", "gemm.hip")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400,
                    help="headline calls timed (exactly this many; 2400 take about 22 ms)")
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--m", type=int, default=8, help="rows of the headline pass")
    ap.add_argument("--no-sweep", action="store_true", help="skip the M=1/2/4 sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (Q4_0 layer, LM head + accept, MoE)")
    ap.add_argument("--only-headline", action="store_true",
                    help="time the headline GEMM only (for profiler runs; = --only headline)")
    ap.add_argument("--only", choices=ONLY, default="all",
                    help="the headline and one other workload (for profiler runs)")
    ap.add_argument("--sustain-ms", type=float, default=SUSTAIN_S * 1e3,
                    help="timed region of the sustained figure (0: skip it, for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for PMC scaling)")
    return ap.parse_args()


def dev_bits(a: np.ndarray, dev) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


class Graphed:
    """calls(0..R-1) captured once in a graph, replayed on demand."""

    def __init__(self, calls, R):
        self.R = R
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(R):             # warm the launch path outside capture
                calls(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            for i in range(R):
                calls(i)

    def ms_per_call(self, calls_wanted):
        """HIP-event time per call over about calls_wanted calls."""
        reps = max(1, -(-calls_wanted // self.R))
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            self.g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * self.R)


LEAD_FIXED_MS = 2.0        # GPU-side lead before the headline's timed calls ...
LEAD_PER_CALL_MS = 0.04    # ... plus this per call (about 4x the host's enqueue cost)


def sleep_cycles_per_ms() -> float:
    """Rate of torch.cuda._sleep (a bounded spin on the GPU clock), measured
    on its own: it paces nothing but the lead below."""
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    n = 2_000_000
    e0.record(stream)
    torch.cuda._sleep(n)
    e1.record(stream)
    torch.cuda.synchronize()
    return n / max(e0.elapsed_time(e1), 1e-3)


def time_exact(calls, R, steps, warmup):
    """Exactly `warmup` untimed calls, then exactly `steps` timed calls,
    launched directly on the current stream; call i uses rotating copy
    i mod R, and the warm-up takes the copies just before copy 0 so that the
    timed calls start on the least recently read ones.  The timed calls sit
    behind a GPU-side lead (a bounded spin kernel, before the first event) of
    LEAD_FIXED_MS + steps * LEAD_PER_CALL_MS, so the host has enqueued them
    all before the GPU reaches them and they run back to back: the two HIP
    events bracket the GPU time of exactly those calls.  (A freshly
    instantiated graph of the same calls runs 0.4-1.5 us per call slower on
    its first replay, and a graph cannot be warmed without extra calls.)
    Returns (seconds by HIP events, host seconds to enqueue the timed calls,
    lead in ms); the enqueue time must stay below the lead."""
    for i in range(warmup):
        calls((R - warmup % R + i) % R)
    cyc = sleep_cycles_per_ms()
    lead_ms = LEAD_FIXED_MS + steps * LEAD_PER_CALL_MS
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(lead_ms * cyc))
    e0.record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        calls(i % R)
    enqueue = time.perf_counter() - t0
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3, enqueue, lead_ms


def time_graph(calls, R, steps, warmup):
    """Capture calls(0..R-1) in one graph; replay it so that about `steps`
    calls are timed.  Returns (wall seconds, ms per call from HIP events,
    calls timed)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(R):                 # warm the launch path outside capture
            calls(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(R):
            calls(i)
    reps = max(1, -(-steps // R))
    for _ in range(max(1, -(-warmup // R))):
        g.replay()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / (reps * R), reps * R


class Gemm:
    """R rotating packed copies of one matrix; one verify call per copy."""

    def __init__(self, bv, fmt, codes, scales, N, K, x, dev, g=1.0):
        self.bv, self.fmt, self.N, self.K, self.g = bv, fmt, N, K, g
        self.bytes = W.weight_bytes(N, K)
        self.R = max(2, -(-ROTATE_BYTES // self.bytes))
        packed = bv.pack_weights(fmt, codes, scales, N, K)
        self.packed = [packed] + [packed.clone() for _ in range(self.R - 1)]
        self.x = x
        self.y = torch.empty((x.shape[0], N), dtype=torch.float32, device=dev)
        self.ws = bv.gemm_workspace(N, K, dev)

    def __call__(self, i):
        self.bv.verify_gemm(self.fmt, self.x, self.packed[i % self.R], self.N, self.K, self.g,
                            y=self.y, ws=self.ws)


def gemm_from_host(bv, w, x, M, dev):
    return Gemm(bv, w["format"], dev_bits(w["codes"], dev), dev_bits(w["scales"], dev), w["N"],
                w["K"], dev_bits(x[:M], dev), dev, float(w.get("g", 1.0)))


def host_threads():
    """The host threads this process may use: its OMP_NUM_THREADS share
    where one is set (the GPU hosts give each GPU a share of their cores),
    else every core of its affinity mask."""
    aff = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    n = int(omp) if omp.isdigit() and int(omp) > 0 else aff
    return max(1, min(n, aff)), aff


def cpu_baseline(cfg, M, budget_s=1.5):
    """The oracle as it stands, on repeated whole passes of the workload
    until about budget_s of wall time, on host_threads() threads."""
    import oracle
    w = cfg["w"]
    x = cfg["x"][:M]
    threads, aff = host_threads()
    oracle.gemm(w, x, nthreads=threads)                # load and warm
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm(w, x, nthreads=threads)
        reps += 1
        t = time.perf_counter() - t0
        if t >= budget_s:
            break
    return {"value": round(W.weight_bytes(w["N"], w["K"]) * reps / t / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{reps} whole passes of the workload (M={M}, K={w['K']}, N={w['N']}, "
                      f"fp64 sums with the |x*w| bound) in {t:.2f} s wall on {threads} threads "
                      f"(about {t * threads:.0f} CPU-seconds; the process may use {aff} cores, "
                      f"OMP_NUM_THREADS={os.environ.get('OMP_NUM_THREADS', 'unset')}, "
                      f"os.cpu_count()={os.cpu_count()})",
            "host_cpu_count": os.cpu_count(), "affinity_cores": aff}


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def trace_average_ns():
    """The headline kernel's average duration in the committed rocprofv3
    kernel trace, if it was taken on the current kernel sources; else None."""
    try:
        text = open(TRACE_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"headline_kernel_average_ns:\s*([0-9.]+)", text)
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != kernel_source_hash():
        return None
    return float(m.group(1))


def pmc_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != kernel_source_hash():
        return None
    return float(m.group(1))


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


def extra_q4_layer(bv, dev, steps, warmup):
    cfg = W.config2(M=8)
    out = {}
    total_bytes, total_us = 0, 0.0
    for name, p in cfg["proj"].items():
        gm = gemm_from_host(bv, p["w"], p["x"], 8, dev)
        _, ms, _ = time_graph(gm, gm.R, steps, warmup)
        out[name] = {"N": gm.N, "K": gm.K, "us": round(ms * 1e3, 3),
                     "gbs": round(gm.bytes / (ms * 1e-3) / 1e9, 1)}
        total_bytes += gm.bytes
        total_us += ms * 1e3
        del gm
        torch.cuda.empty_cache()
    out["layer"] = {"bytes": total_bytes, "us": round(total_us, 3),
                    "gbs": round(total_bytes / (total_us * 1e-6) / 1e9, 1)}
    # the same layer with the projections that share an input fused along N
    # (Q|K|V and gate|up), as a decoder runs them
    P = cfg["proj"]
    fused_us = out["o"]["us"] + out["down"]["us"]
    for fname, names in (("qkv_fused", ("q", "k", "v")), ("gate_up_fused", ("gate", "up"))):
        ws = [P[n]["w"] for n in names]
        fw = {"format": W.FMT_Q4_0, "K": ws[0]["K"], "N": sum(w["N"] for w in ws), "g": 1.0,
              "codes": np.concatenate([w["codes"] for w in ws]),
              "scales": np.concatenate([w["scales"] for w in ws])}
        gm = gemm_from_host(bv, fw, P[names[0]]["x"], 8, dev)
        _, ms, _ = time_graph(gm, gm.R, steps, warmup)
        out[fname] = {"N": gm.N, "K": gm.K, "us": round(ms * 1e3, 3),
                      "gbs": round(gm.bytes / (ms * 1e-3) / 1e9, 1)}
        fused_us += ms * 1e3
        del gm
        torch.cuda.empty_cache()
    out["layer_fused"] = {"bytes": total_bytes, "us": round(fused_us, 3),
                          "gbs": round(total_bytes / (fused_us * 1e-6) / 1e9, 1)}
    return out


def extra_c0_chain(bv, dev, steps, warmup):
    """The tiny verify pass end to end: x[4][2048] -> nvfp4 2048x2048 (bf16
    output) -> nvfp4 head 2048 -> 1024 -> greedy acceptance of 3 drafts, as
    one chain of launches per call, over rotating copies of both matrices."""
    c = W.config0()
    M, V = c["M"], c["V"]
    b1, b2 = W.weight_bytes(2048, 2048), W.weight_bytes(V, 2048)
    R = max(2, -(-ROTATE_BYTES // (b1 + b2)))
    p1 = bv.pack_weights(bv.FMT_NVFP4, dev_bits(c["w1"]["codes"], dev),
                         dev_bits(c["w1"]["scales"], dev), 2048, 2048)
    p2 = bv.pack_weights(bv.FMT_NVFP4, dev_bits(c["head"]["codes"], dev),
                         dev_bits(c["head"]["scales"], dev), V, 2048)
    w1s = [p1] + [p1.clone() for _ in range(R - 1)]
    w2s = [p2] + [p2.clone() for _ in range(R - 1)]
    x = dev_bits(c["x"], dev)
    yb = torch.empty((M, 2048), dtype=torch.int16, device=dev)
    z = torch.empty((M, V), dtype=torch.float32, device=dev)
    d = torch.from_numpy(c["drafts"]).to(dev)
    outs = (torch.empty(M, dtype=torch.int32, device=dev),
            torch.empty(2, dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int64, device=dev))
    ws = bv.accept_workspace(M, V, dev)

    def chain(i):
        bv.verify_gemm(bv.FMT_NVFP4, x, w1s[i % R], 2048, 2048, 1.0, y_bf16=yb, want_fp32=False)
        bv.verify_gemm(bv.FMT_NVFP4, yb, w2s[i % R], V, 2048, 1.0, y=z)
        bv.accept_greedy(z, d, 100, outs=outs, ws=ws)

    _, ms, n = time_graph(chain, R, max(R, steps // 4), max(R, warmup // 4))
    res = {"M": M, "K": 2048, "N": 2048, "V": V, "weight_bytes": b1 + b2,
           "us_per_pass": round(ms * 1e3, 3), "gbs": round((b1 + b2) / (ms * 1e-3) / 1e9, 1),
           "launches_per_pass": 4, "passes_timed": n}
    del w1s, w2s
    torch.cuda.empty_cache()
    return res


def extra_q4_layer_sweep(bv, dev, steps, warmup):
    """The 27B-class Q4_0 layer as a decoder runs it (Q|K|V and gate|up fused
    along N: four launches), one graph per row count M = 1, 2, 4, 8, over
    rotating copies of the whole layer."""
    cfg = W.config2(M=8)
    P = cfg["proj"]
    mats = []
    for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
        ws = [P[n]["w"] for n in names]
        fw = {"format": W.FMT_Q4_0, "K": ws[0]["K"], "N": sum(w["N"] for w in ws),
              "codes": np.concatenate([w["codes"] for w in ws]),
              "scales": np.concatenate([w["scales"] for w in ws])}
        mats.append((fw, P[names[0]]["x"]))
    layer_bytes = sum(W.weight_bytes(fw["N"], fw["K"]) for fw, _ in mats)
    R = max(2, -(-ROTATE_BYTES // layer_bytes))
    packed = []
    for fw, _ in mats:
        pk = bv.pack_weights(W.FMT_Q4_0, dev_bits(fw["codes"], dev), dev_bits(fw["scales"], dev),
                             fw["N"], fw["K"])
        packed.append([pk] + [pk.clone() for _ in range(R - 1)])
    wss = [bv.gemm_workspace(fw["N"], fw["K"], dev) for fw, _ in mats]
    out = {"bytes": layer_bytes, "launches": 4}
    for M in (1, 2, 4, 8):
        xs = [dev_bits(x[:M], dev) for _, x in mats]
        ys = [torch.empty((M, fw["N"]), dtype=torch.float32, device=dev) for fw, _ in mats]

        def layer(i, xs=xs, ys=ys):
            for j, (fw, _) in enumerate(mats):
                bv.verify_gemm(W.FMT_Q4_0, xs[j], packed[j][i % R], fw["N"], fw["K"], 1.0,
                               y=ys[j], ws=wss[j])

        _, ms, _ = time_graph(layer, R, max(4 * R, steps // 16), max(R, warmup // 16))
        out[str(M)] = {"us": round(ms * 1e3, 3),
                       "gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                       "plans": [{k: bv.gemm_plan_info(W.FMT_Q4_0, M, fw["N"], fw["K"])[k]
                                  for k in ("S", "J", "KG", "TW", "grid")} for fw, _ in mats]}
    out["m8_over_m1_time"] = round(out["8"]["us"] / out["1"]["us"], 4)
    del packed
    torch.cuda.empty_cache()
    return out


def extra_lm_head_and_accept(bv, dev, steps, warmup, gemm_only=False):
    c = W.config3_inputs(M=8)
    M, V = c["M"], c["V"]
    gm = gemm_from_host(bv, c["w"], c["x"], M, dev)
    _, ms, _ = time_graph(gm, gm.R, max(20, steps // 20), max(4, warmup // 20))
    out = {"lm_head": {"N": V, "K": c["K"], "us": round(ms * 1e3, 3),
                       "gbs": round(gm.bytes / (ms * 1e-3) / 1e9, 1)}}
    if gemm_only:
        return out
    gm(0)
    torch.cuda.synchronize()
    logits = gm.y
    # the planted drafts follow the row argmax of the logits (lowest index on
    # ties; these logits hold no NaN)
    am = np.argmax(logits.cpu().numpy(), axis=1).astype(np.int32)
    drafts = W.plant_drafts(am, c["L"], c["filler"], c["miss"], V)
    dd = torch.from_numpy(drafts).to(dev)
    q = torch.from_numpy(c["q"]).to(dev)
    u = torch.from_numpy(c["u"]).to(dev)
    outs = (torch.empty(M, dtype=torch.int32, device=dev),
            torch.empty(2, dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int64, device=dev))
    ws = bv.accept_workspace(M, V, dev)

    def greedy(i):
        bv.accept_greedy(logits, dd, 100, outs=outs, ws=ws)

    def rejection(i):
        bv.accept_rejection(logits, q, dd, u, c["temperature"], c["top_p"], 100, outs=outs,
                            ws=ws)

    # 16 back-to-back calls per graph (the same logits, which stay in the
    # caches as they would right after the LM head), so that the graph's own
    # launch cost is spread as it is for the GEMM timings
    # the full sampler pipeline on the sparse top-k path (penalties over a
    # 64-token window of a seeded history, top-k 64, top-p, min-p)
    sp = bv.Sampler(temperature=c["temperature"], top_p=c["top_p"], min_p=0.01, top_k=64,
                    repeat_penalty=1.1, penalty_last_n=64)
    hist = torch.from_numpy(np.random.default_rng(7).integers(0, V, (1, 64)).astype(np.int32)).to(dev)
    hlen = torch.full((1,), 64, dtype=torch.int32, device=dev)
    u1 = u.view(1, M)
    d1 = dd.view(1, M - 1)
    q1 = q.view(1, M - 1, V)
    sws = torch.zeros(bv.accept_sampled_workspace_bytes(1, M, V, 64, True), dtype=torch.uint8,
                      device=dev)
    souts = (torch.empty((1, M), dtype=torch.int32, device=dev),
             torch.empty((1, 2), dtype=torch.int32, device=dev),
             torch.empty(1, dtype=torch.int64, device=dev))

    def sampled(i):
        bv.accept_sampled(logits, d1, u1, sp, draft_probs=q1, history=hist, history_len=hlen,
                          outs=souts, ws=sws)

    # the same step on logits ~ N(0,1) (a nucleus of many thousand tokens,
    # unlike the head's own logits, whose nucleus is mostly one token)
    zs = torch.from_numpy(W.spread_logits(3, M, V)).to(dev)
    ams = np.argmax(W.spread_logits(3, M, V), axis=1).astype(np.int32)
    dds = torch.from_numpy(W.plant_drafts(ams, c["L"], c["filler"], c["miss"], V)).to(dev)

    def rejection_spread(i):
        bv.accept_rejection(zs, q, dds, u, c["temperature"], c["top_p"], 100, outs=outs, ws=ws)

    _, ms_g, _ = time_graph(greedy, 16, max(64, steps // 4), 32)
    _, ms_r, _ = time_graph(rejection, 16, max(64, steps // 4), 32)
    _, ms_rs, _ = time_graph(rejection_spread, 16, max(64, steps // 4), 32)
    _, ms_s, _ = time_graph(sampled, 16, max(64, steps // 4), 32)
    out["accept_greedy"] = {"M": M, "V": V, "us": round(ms_g * 1e3, 3), "planted_L": c["L"]}
    out["accept_rejection"] = {"M": M, "V": V, "us": round(ms_r * 1e3, 3),
                               "temperature": c["temperature"], "top_p": c["top_p"]}
    out["accept_rejection_spread_logits"] = {"M": M, "V": V, "us": round(ms_rs * 1e3, 3),
                                             "logits": "N(0,1)",
                                             "temperature": c["temperature"],
                                             "top_p": c["top_p"]}
    out["accept_sampled"] = {"B": 1, "M": M, "V": V, "us": round(ms_s * 1e3, 3),
                             "temperature": c["temperature"], "top_p": c["top_p"],
                             "top_k": 64, "min_p": 0.01, "repeat_penalty": 1.1,
                             "penalty_last_n": 64}
    del gm
    torch.cuda.empty_cache()
    return out


def extra_moe(bv, dev, steps, warmup):
    c = W.config4()
    T, E, F, H, topk = c["T"], c["E"], c["F"], c["H"], c["topk"]
    gu, dn = c["gate_up"], c["down"]
    per_expert = W.weight_bytes(2 * F, H) + W.weight_bytes(H, F)
    R = max(2, -(-ROTATE_BYTES // (per_expert * E)))
    gup = bv.pack_weights(gu["format"], dev_bits(gu["codes"], dev), dev_bits(gu["scales"], dev),
                          2 * F, H, count=E)
    dnp = bv.pack_weights(dn["format"], dev_bits(dn["codes"], dev), dev_bits(dn["scales"], dev),
                          H, F, count=E)
    gups = [gup] + [gup.clone() for _ in range(R - 1)]
    dnps = [dnp] + [dnp.clone() for _ in range(R - 1)]
    x = dev_bits(c["x"], dev)
    ids = torch.from_numpy(c["ids"]).to(dev)
    gw = torch.from_numpy(c["gw"]).to(dev)
    out_t = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(bv.moe_workspace_bytes(T, H, F, E, topk), dtype=torch.uint8, device=dev)

    def call(i):
        bv.verify_moe(gu["format"], x, ids, gw, gups[i % R], dnps[i % R], E, F, out=out_t, ws=ws)

    # the M = 1 baseline: the first token alone (its 8 experts)
    ws1 = torch.empty(bv.moe_workspace_bytes(1, H, F, E, topk), dtype=torch.uint8, device=dev)
    out1 = torch.empty((1, H), dtype=torch.float32, device=dev)

    def call1(i):
        bv.verify_moe(gu["format"], x[:1], ids[:1], gw[:1], gups[i % R], dnps[i % R], E, F,
                      out=out1, ws=ws1)

    _, ms, _ = time_graph(call, R, max(40, steps // 10), 10)
    _, ms1, _ = time_graph(call1, R, max(40, steps // 10), 10)
    uniq = len(np.unique(c["ids"]))
    ub = uniq * per_expert
    return {"T": T, "E": E, "topk": topk, "H": H, "F": F, "unique_experts": uniq,
            "unique_bytes": ub, "us": round(ms * 1e3, 3), "gbs": round(ub / (ms * 1e-3) / 1e9, 1),
            "m1_gemv_bytes": topk * per_expert, "m1_us": round(ms1 * 1e3, 3),
            "m1_gbs": round(topk * per_expert / (ms1 * 1e-3) / 1e9, 1),
            "t8_over_m1_time": round(ms / ms1, 4), "no_dedup_bytes": T * topk * per_expert}


def extra_verify_attention(bv, dev, steps, warmup):
    """Causal attention of 8 verify rows over a 32768-key prefix: 32 query
    heads on 8 KV heads of dim 128 (bf16), each KV head read once for all
    8 x 4 query rows; rotating copies of the cache (>= 1 GiB)."""
    M, Hq, Hkv, D, L = 8, 32, 8, 128, 32768 - 8
    rng = np.random.default_rng(31)
    q = dev_bits(W.to_bf16_bits(rng.standard_normal((M, Hq, D)).astype(np.float32)), dev)
    kv_bytes = 2 * Hkv * (L + M) * D * 2
    R = max(2, -(-ROTATE_BYTES // kv_bytes))
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    caches = []
    for _ in range(R):
        k = torch.randn((Hkv, L + M, D), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((Hkv, L + M, D), generator=g, device=dev).to(torch.bfloat16)
        caches.append((k.view(torch.int16), v.view(torch.int16)))
    out = torch.empty((M, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(bv.attention_workspace_bytes(M, Hq, Hkv, D, L), dtype=torch.uint8, device=dev)

    def call(i):
        k, v = caches[i % R]
        bv.verify_attention(q, k, v, L, out=out, ws=ws)

    _, ms, _ = time_graph(call, R, max(64, steps // 8), max(16, warmup // 8))
    res = {"M": M, "Hq": Hq, "Hkv": Hkv, "D": D, "keys": L + M, "kv_bytes": kv_bytes,
           "us": round(ms * 1e3, 3), "gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1)}
    res["frac_of_hbm_peak"] = round(res["gbs"] / PEAK_HBM_GBS, 4)
    del caches
    torch.cuda.empty_cache()
    return res


def extra_kv_rollback(bv, dev, steps, warmup):
    """Verify-step cache writes and the commit of a rotating-cache stack:
    52 sliding-window layers (a 1024-key window on a 1031-row ring), 16 KV
    heads of dim 128, 8 verify rows written past the wrap (every write
    destroys a live row, so every one is copied out).  append: one layer's
    write, as the forward issues it per layer; restore: one call over all 52
    layers with every draft rejected (7 of 8 rows given back per head)."""
    NL, Hkv, D, M, cap = 52, 16, 128, 8, 1031
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    kc = torch.randint(-32768, 32767, (NL, 1, Hkv, cap, D), generator=g, dtype=torch.int16,
                       device=dev)
    vc = torch.randint_like(kc, -32768, 32767)
    kn = torch.randint(-32768, 32767, (NL, 1, M, Hkv * D), generator=g, dtype=torch.int16,
                       device=dev)
    vn = torch.randint_like(kn, -32768, 32767)
    snap = bv.kv_snapshot(kc, M)
    base = torch.tensor([5000], dtype=torch.int64, device=dev)
    roll = torch.tensor([5001], dtype=torch.int64, device=dev)
    layer_snap = [(snap[0][i:i + 1], snap[1][i:i + 1]) for i in range(NL)]

    def append(i):
        bv.kv_append(kc[i:i + 1], vc[i:i + 1], kn[i:i + 1], vn[i:i + 1], base, True, layer_snap[i])

    def restore(i):
        bv.kv_restore(kc, vc, M, base, roll, True, snap)

    _, ms_a, _ = time_graph(append, NL, max(NL, steps // 4), max(NL, warmup // 4))
    _, ms_r, _ = time_graph(restore, 8, max(64, steps // 16), max(16, warmup // 16))
    row = D * 2
    a_bytes = 2 * Hkv * M * row * 4          # read new + old, write snapshot + cache, K and V
    r_bytes = NL * 2 * Hkv * (M - 1) * row * 2
    res = {"layers": NL, "Hkv": Hkv, "D": D, "M": M, "ring_rows": cap,
           "append_us_per_layer": round(ms_a * 1e3, 3), "append_bytes": a_bytes,
           "restore_us": round(ms_r * 1e3, 3), "restore_bytes": r_bytes,
           "restore_gbs": round(r_bytes / (ms_r * 1e-3) / 1e9, 1)}
    del kc, vc, kn, vn, snap, layer_snap
    torch.cuda.empty_cache()
    return res


def read_ceiling(bv, dev, steps, warmup):
    """The read rate one launch reaches on this GPU: a plain read of every
    byte (mtp_read_probe, the best of its launch shapes), timed like the
    verify GEMMs (graph replays over rotating copies) on buffers of the C1
    matrix's size, the LM head's size and 2 GiB."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for name, nb in (("33mb", W.weight_bytes(14336, 4096)), ("793mb", W.weight_bytes(262144, 5376)),
                     ("2gib", 2 << 30)):
        nb = (nb + 15) // 16 * 16
        R = max(1, -(-ROTATE_BYTES // nb))   # >= 1 GiB of copies (2 GiB: one)
        bufs = [torch.zeros(nb, dtype=torch.uint8, device=dev) for _ in range(R)]

        best = None
        for shape in range(bv.read_probe_shapes()):
            def call(i, shape=shape):
                bv.read_probe(bufs[i % R], sink, shape)

            _, ms, _ = time_graph(call, R, max(R, steps // 8), max(R, warmup // 8))
            if best is None or ms < best[0]:
                best = (ms, shape)
        ms, shape = best
        out[name] = {"bytes": nb, "copies": R, "best_shape": shape, "us": round(ms * 1e3, 3),
                     "gbs": round(nb / (ms * 1e-3) / 1e9, 1)}
        del bufs
        torch.cuda.empty_cache()
    return out


def depth_controller(bv, sweep):
    """The draft depth the controller picks on this run's measured cost of
    one verify pass per width (M = 1, 2, 4, 8; linear in between) plus a
    drafter costing a tenth of the M = 1 pass per draft token, for constant
    per-position acceptance rates."""
    ms = sorted(int(m) for m in sweep)
    us = [sweep[str(m)]["us_per_call"] for m in ms]
    verify = np.interp(np.arange(1, 9), ms, us)
    cost = verify + 0.1 * us[0] * np.arange(8)
    out = {"cost_us_per_step": [round(float(c), 3) for c in cost],
           "draft_us_per_token": round(0.1 * us[0], 3)}
    for a in (0.5, 0.7, 0.9):
        d, rate = bv.choose_draft_depth(np.full(7, a), cost)
        out[f"accept_{a}"] = {"depth": d, "tokens_per_us": round(float(rate[d]), 4),
                              "speedup_vs_plain": round(float(rate[d] / rate[0]), 3)}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (the verify pass here has no multi-GPU "
              "path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    only = "headline" if args.only_headline else args.only
    want = lambda name: only == name or (only == "all" and not args.no_extra)  # noqa: E731
    import bit_verify_gemm_amd as bv
    bv.lib()
    dev = torch.device("cuda:0")
    cfg = W.config1(M=8)
    M = args.m

    # headline: exactly --steps calls, one HIP-event clock
    head = gemm_from_host(bv, cfg["w"], cfg["x"], M, dev)
    t_ev, t_enq, lead_ms = time_exact(head, head.R, args.steps, args.warmup)
    bytes_call = head.bytes
    value = bytes_call * args.steps / t_ev / 1e9
    plan = bv.gemm_plan_info(bv.FMT_NVFP4, M, cfg["w"]["N"], cfg["w"]["K"])
    # beside it: at least 20 ms of back-to-back calls (whole replays of the
    # rotating copies)
    per = t_ev / args.steps
    sustained = None
    if args.sustain_ms > 0:
        g = Graphed(head, head.R)
        g.ms_per_call(head.R)
        n_sus = max(head.R, int(args.sustain_ms * 1e-3 / per) + 1)
        ms_sus = g.ms_per_call(n_sus)
        n_sus = -(-n_sus // head.R) * head.R
        sustained = {"calls": n_sus, "timed_ms": round(ms_sus * n_sus, 3),
                     "us_per_call": round(ms_sus * 1e3, 3),
                     "gbs": round(bytes_call / (ms_sus * 1e-3) / 1e9, 1)}
        del g

    # M sweep: the row counts take turns in 5 rounds and each reports its
    # median, so that clock drift between separate measurements does not
    # enter the ratios between them
    sweep = {}
    if only in ("all", "sweep") and not args.no_sweep:
        ms_of = {m: [] for m in (1, 2, 4, 8)}
        runners = {m: gemm_from_host(bv, cfg["w"], cfg["x"], m, dev) for m in ms_of}
        graphs = {m: Graphed(r, r.R) for m, r in runners.items()}
        for gm in graphs.values():
            gm.ms_per_call(gm.R)
        n_each = max(runners[1].R, int(SUSTAIN_S / per / 4) + 1)
        for _ in range(5):
            for m, gm in graphs.items():
                ms_of[m].append(gm.ms_per_call(n_each))
        for m, v in ms_of.items():
            ms = float(np.median(v))
            sweep[str(m)] = {"us_per_call": round(ms * 1e3, 3),
                             "gbs": round(bytes_call / (ms * 1e-3) / 1e9, 1),
                             "frac_of_hbm_peak": round(bytes_call / (ms * 1e-3) / 1e9
                                                       / PEAK_HBM_GBS, 4)}
        del graphs, runners
        torch.cuda.empty_cache()

    steps_x, warm_x = 2000, 2000      # call counts of the other workloads' timings
    extra = {}
    if want("c0"):
        extra["c0_tiny_chained_pass"] = extra_c0_chain(bv, dev, steps_x, warm_x)
    if want("c2"):
        extra["q4_0_layer_27b_m8"] = extra_q4_layer(bv, dev, steps_x, warm_x)
        extra["q4_0_layer_27b_fused_m_sweep"] = extra_q4_layer_sweep(bv, dev, steps_x, warm_x)
    if want("c3"):
        extra["lm_head_5376x262144_m8"] = extra_lm_head_and_accept(bv, dev, steps_x, warm_x)
    elif only == "lmhead":      # the LM-head GEMM alone (for counter runs)
        extra["lm_head_5376x262144_m8"] = extra_lm_head_and_accept(bv, dev, steps_x, warm_x,
                                                                   gemm_only=True)
    if want("moe"):
        extra["moe_8tok_128x_top8"] = extra_moe(bv, dev, steps_x, warm_x)
    if want("attn"):
        extra["verify_attention_32k"] = extra_verify_attention(bv, dev, steps_x, warm_x)
    if want("kv"):
        extra["kv_rollback_52x16x128"] = extra_kv_rollback(bv, dev, steps_x, warm_x)

    ceiling = None
    if want("ceiling"):
        ceiling = read_ceiling(bv, dev, steps_x, warm_x)
        ceiling["c1_frac_of_33mb_ceiling"] = round(value / ceiling["33mb"]["gbs"], 4)
        if sustained:
            ceiling["c1_sustained_frac_of_33mb_ceiling"] = round(sustained["gbs"]
                                                                 / ceiling["33mb"]["gbs"], 4)

    if args.copy_calibration:
        copy_calibration(dev)

    traffic = pmc_traffic()
    trace_ns = trace_average_ns()
    out = {
        "metric": "effective weight GB/s (% of HBM peak) for nvfp4 verify GEMM at M=1/2/4/8",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_ev / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"nvfp4 verify GEMM, dense FFN-up K=4096 -> N=14336, M={M} "
                               f"bf16 rows (staged exactly as fp16), fp32 accumulate",
                   "M": M, "K": 4096, "N": 14336, "weight_bytes_per_call": bytes_call,
                   "rotating_weight_copies": head.R, "graph_replay": True,
                   "timed_region_ms_hip_events": round(t_ev * 1e3, 4),
                   "launch": "direct, behind a GPU-side lead",
                   "lead_ms": round(lead_ms, 3), "enqueue_ms": round(t_enq * 1e3, 3),
                   "enqueue_within_lead": bool(t_enq * 1e3 < lead_ms),
                   "plan": {k: plan[k] for k in ("S", "J", "KG", "TW", "grid", "threads")}},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(value / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
    }
    if sustained:
        out["sustained"] = sustained
    if trace_ns:
        out["roofline"]["kernel_trace_avg_ns"] = trace_ns
        out["roofline"]["kernel_trace_achieved"] = round(bytes_call / trace_ns, 1)
    if sweep:
        out["m_sweep"] = sweep
        if "1" in sweep and "8" in sweep:
            out["m8_over_m1_time"] = round(sweep["8"]["us_per_call"] / sweep["1"]["us_per_call"], 4)
            out["depth_controller"] = depth_controller(bv, sweep)
    if extra:
        out["other_workloads"] = extra
    if ceiling:
        out["read_ceiling"] = ceiling
    if not args.no_cpu and only == "all":
        out["cpu_baseline"] = cpu_baseline(cfg, M)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the compensated 4-bit linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

Workload (the headline): Llama-7B-shaped decode projections 4096->4096,
4096->11008 and 11008->4096 at M = 1, 4, 16 and 32 tokens; 4-bit weights
with group-128 fp16 scale and zero-point, compensator rank 32 with the
sigmoid gate, fp16 activations N(0, 1) with 1% of input channels x20.
One step = the twelve compensated decode calls (3 shapes x 4 token counts)
through the phase-aware entry point, each on a different copy of its layer:
the copies rotate over more than 1 GiB so that the 256 MiB Infinity Cache
cannot serve the weights.  Steps are captured once in HIP graphs and
replayed.

Printed: one JSON line with the decode throughput in algorithmic GB/s
(value), the roofline of the dominant kernel, the CPU oracle timed on a
bounded sample, and extra context (per-call breakdown, compensator overhead
against the same kernel with rank 0, prefill TFLOP/s).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "decode GB/s & prefill TFLOP/s (% roofline), compensator overhead vs plain W4A16"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
ROTATION_BYTES = 1 << 30


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work of one call (bytes the method must move, flops it must do)
# ---------------------------------------------------------------------------


def call_bytes(N, K, G, r, M, act=2):
    b = N * K // 2 + 4 * N * (K // G) + act * (M * K + M * N)
    if r > 0:
        b += act * (r * K + N * r + K)
    return b


def call_flops(N, K, r, M):
    f = 2 * M * N * K
    if r > 0:
        f += 2 * M * r * (K + N) + 2 * M * K
    return f


# ---------------------------------------------------------------------------
# device set-up
# ---------------------------------------------------------------------------


def clone_layer(lay):
    from quantized_gemm_error_amd.spear import SpearLayer
    c = lambda t: None if t is None else t.clone()  # noqa: E731
    return SpearLayer(lay.N, lay.K, lay.group_size, c(lay.qweight), c(lay.scales), c(lay.zeros),
                      lay.rank, c(lay.A), c(lay.B), c(lay.w_gate), lay.b_gate)


def layer_bytes(lay):
    tot = 0
    for t in (lay.qweight, lay.scales, lay.zeros, lay.A, lay.B, lay.w_gate):
        if t is not None:
            tot += t.numel() * t.element_size()
    return tot


class DecodeWorkload:
    """Rotating copies of the three 7B projections plus their inputs."""

    def __init__(self, device, rank_override=None):
        import torch

        from quantized_gemm_error_amd import spear, synth
        w = synth.WORKLOADS["llama7b-decode"]
        self.tokens = list(w["tokens"])
        self.shapes = list(w["shapes"])
        self.G = w["group_size"]
        self.r = w["rank"] if rank_override is None else rank_override
        base = []
        for i, (K, N) in enumerate(self.shapes):
            hl = synth.make_layer(N, K, self.G, w["rank"], seed=w["seed"] + 10 * i)
            lay = spear.layer_to_device(hl, device)
            base.append(lay if self.r > 0 else lay.without_compensator())
        set_bytes = sum(layer_bytes(l) for l in base)
        self.n_sets = max(2, -(-ROTATION_BYTES // set_bytes))
        self.sets = [base] + [[clone_layer(l) for l in base] for _ in range(self.n_sets - 1)]
        self.rotation_bytes = set_bytes * self.n_sets
        maxM = max(self.tokens)
        self.x = {}
        for K in sorted({k for k, _ in self.shapes}):
            xb = synth.make_activations(maxM, K, seed=w["seed"] + K, outliers=True)
            xt = spear.act_to_device(xb, "f16", device)
            for M in self.tokens:
                self.x[(K, M)] = xt[:M].contiguous()
        self.y = {(N, M): torch.empty((M, N), dtype=torch.float16, device=device)
                  for _, N in self.shapes for M in self.tokens}
        self.ws = [spear.new_workspace(l, maxM) for l in base] if self.r > 0 else None
        # the calls of one step: (shape index, M)
        self.calls = [(si, M) for M in self.tokens for si in range(len(self.shapes))]
        self.step_bytes = sum(call_bytes(self.shapes[si][1], self.shapes[si][0], self.G, self.r, M)
                              for si, M in self.calls)
        self.step_flops = sum(call_flops(self.shapes[si][1], self.shapes[si][0], self.r, M)
                              for si, M in self.calls)
        self.counter = 0

    def issue(self, si, M, set_idx, stream=None):
        from quantized_gemm_error_amd import spear
        K, N = self.shapes[si]
        lay = self.sets[set_idx][si]
        ws = None if self.ws is None else self.ws[si]
        spear.spear_linear(lay, self.x[(K, M)], y=self.y[(N, M)], workspace=ws, main_stream=stream)


def capture_graphs(torch, fn_per_phase, n_phases, stream):
    graphs = []
    for ph in range(n_phases):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn_per_phase(ph)
        graphs.append(g)
    return graphs


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------


def timed_decode_steps(torch, wl, steps, warmup):
    """Replay captured steps; HIP events on the stream time each kernel class.

    A step is two graphs replayed back to back on one stream: the launches of
    the dominant kernel (one token block, M <= 16: nine calls) and the M = 32
    launches (three calls).  Events recorded on the same stream before, between
    and after the two replays give each class's device time per step.
    """
    stream = torch.cuda.Stream()
    n_calls = len(wl.calls)
    n_phases = wl.n_sets // int(np.gcd(wl.n_sets, n_calls))
    classes = {"one_block": [c for c in range(n_calls) if wl.calls[c][1] <= 16],
               "two_blocks": [c for c in range(n_calls) if wl.calls[c][1] > 16]}

    def issue_class(ph, cls):
        for c in classes[cls]:
            si, M = wl.calls[c]
            wl.issue(si, M, (ph * n_calls + c) % wl.n_sets, stream)

    with torch.cuda.stream(stream):
        for ph in range(n_phases):          # eager warm-up of every layer copy
            for cls in classes:
                issue_class(ph, cls)
    torch.cuda.synchronize()
    graphs = []
    for ph in range(n_phases):
        pair = []
        for cls in classes:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                issue_class(ph, cls)
            pair.append(g)
        graphs.append(pair)
    for i in range(warmup):
        for g in graphs[i % n_phases]:
            g.replay()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(steps):
            ga, gb = graphs[i % n_phases]
            e0, e1, e2 = evs[i]
            e0.record(stream)
            ga.replay()
            e1.record(stream)
            gb.replay()
            e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = evs[0][0].elapsed_time(evs[-1][2])
    cls_ms = {"one_block": sum(e[0].elapsed_time(e[1]) for e in evs),
              "two_blocks": sum(e[1].elapsed_time(e[2]) for e in evs)}
    return total_ms, wall, cls_ms, classes


def graph_call_time_ms(torch, issue_fn, n, reps=5):
    """Average device time per call of n back-to-back calls captured in one graph."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(n):
            issue_fn(i, stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            issue_fn(i, stream)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):   # replay() runs on the current stream
            s.record(stream)
            g.replay()
            e.record(stream)
        torch.cuda.synchronize()
        t = s.elapsed_time(e) / n
        best = t if best is None else min(best, t)
    return best


def decode_overhead(torch, wl_ec, wl_r0):
    out = {}
    for si, (K, N) in enumerate(wl_ec.shapes):
        for M in wl_ec.tokens:
            n = wl_ec.n_sets
            t_ec = graph_call_time_ms(torch, lambda i, s: wl_ec.issue(si, M, i % n, s), n)
            t_r0 = graph_call_time_ms(torch, lambda i, s: wl_r0.issue(si, M, i % n, s), n)
            b = call_bytes(N, K, wl_ec.G, wl_ec.r, M)
            out[f"{K}->{N} M={M}"] = {
                "us_ec": round(t_ec * 1e3, 3), "us_r0": round(t_r0 * 1e3, 3),
                "overhead_pct": round(100.0 * (t_ec / t_r0 - 1.0), 2),
                "GBps_ec": round(b / (t_ec * 1e-3) / 1e9, 1),
                "hbm_frac_ec": round(b / (t_ec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
    return out


def prefill_context(torch, device):
    """Llama-7B prefill, M = 2048, bf16: TFLOP/s with the aux stream, and rank 0."""
    from quantized_gemm_error_amd import spear, synth
    w = synth.WORKLOADS["llama7b-prefill"]
    M = w["tokens"][0]
    aux = torch.cuda.Stream()
    out = {}
    for i, (K, N) in enumerate(w["shapes"]):
        hl = synth.make_layer(N, K, w["group_size"], w["rank"], seed=w["seed"] + 10 * i, dtype="bf16")
        lay = spear.layer_to_device(hl, device)
        lay0 = lay.without_compensator()
        x = spear.act_to_device(synth.make_activations(M, K, seed=w["seed"], dtype="bf16",
                                                       outliers=True), "bf16", device)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        ws = spear.new_workspace(lay, M)

        def run_ec(_i, s):
            spear.spear_linear_prefill(lay, x, y=y, workspace=ws, main_stream=s, aux_stream=aux)

        def run_r0(_i, s):
            spear.spear_linear_prefill(lay0, x, y=y, main_stream=s)
        t_ec = graph_call_time_ms(torch, run_ec, 4)
        t_r0 = graph_call_time_ms(torch, run_r0, 4)
        f = call_flops(N, K, w["rank"], M)
        out[f"{K}->{N} M={M}"] = {
            "us_ec": round(t_ec * 1e3, 1), "us_r0": round(t_r0 * 1e3, 1),
            "TFLOPs_ec": round(f / (t_ec * 1e-3) / 1e12, 1),
            "mfma_frac_ec": round(f / (t_ec * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "overhead_pct": round(100.0 * (t_ec / t_r0 - 1.0), 2),
        }
        del lay, lay0, x, y, ws
    return out


def cpu_baseline(budget_s=12.0):
    """The float64 oracle on the same decode calls, until about budget_s of CPU work."""
    import oracle
    from quantized_gemm_error_amd import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        n_threads = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(limits=n_threads)
        blas = [i.get("num_threads") for i in threadpool_info()]
        cores = int(max(blas)) if blas else 1
    except Exception:  # pragma: no cover
        limiter, cores = None, 1
    w = synth.WORKLOADS["llama7b-decode"]
    layers = []
    for i, (K, N) in enumerate(w["shapes"]):
        hl = synth.make_layer(N, K, w["group_size"], w["rank"], seed=w["seed"] + 10 * i)
        layers.append((hl, oracle.pack_int4(hl.q)))
    xs = {K: synth.make_activations(max(w["tokens"]), K, seed=w["seed"] + K, outliers=True)
          for K in {k for k, _ in w["shapes"]}}
    done_bytes, calls = 0, 0
    t0 = time.perf_counter()
    while True:
        for M in w["tokens"]:
            for hl, words in layers:
                oracle.spear_linear_ref(xs[hl.K][:M], words, hl.scales, hl.zeros, hl.group_size, "f16",
                                        hl.A, hl.B, hl.w_gate, hl.b_gate)
                done_bytes += call_bytes(hl.N, hl.K, hl.group_size, hl.rank, M)
                calls += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{calls} compensated decode calls of the same workload (oracle float64 NumPy: "
                      f"int4 unpack, dequant, matmul), {dt:.1f} s; elementwise NumPy is single-threaded, "
                      f"BLAS uses {cores} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extra", action="store_true", help="skip overhead/prefill context")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_gemm_error_amd import spear
    spear.load_library()
    dev = "cuda:0"
    torch.cuda.set_device(0)

    log("building decode workload")
    wl = DecodeWorkload(dev)
    n_sets, rot_bytes = wl.n_sets, wl.rotation_bytes
    log(f"{n_sets} layer-set copies, rotation {rot_bytes / 2**30:.2f} GiB")
    total_ms, wall, cls_ms, classes = timed_decode_steps(torch, wl, args.steps, args.warmup)
    ms_per_step = total_ms / args.steps
    value = wl.step_bytes * args.steps / (total_ms * 1e-3) / 1e9
    log(f"decode: {ms_per_step * 1e3:.1f} us/step, {value:.1f} GB/s")

    # dominant kernel: decode_kernel, one token block (M <= 16), compensated, group-wise
    dom_calls = [wl.calls[c] for c in classes["one_block"]]
    dom_bytes = sum(call_bytes(wl.shapes[si][1], wl.shapes[si][0], wl.G, wl.r, M) for si, M in dom_calls)
    n_launch = len(dom_calls) * args.steps
    dom_ms = cls_ms["one_block"]
    achieved = dom_bytes * args.steps / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "decode_kernel<f16, one 16-token block, compensated, group-wise>",
                "avg_launch_us": round(dom_ms / n_launch * 1e3, 3), "launches_timed": n_launch,
                "bytes_per_launch_avg": int(dom_bytes / len(dom_calls))}
    two_calls = [wl.calls[c] for c in classes["two_blocks"]]
    two_bytes = sum(call_bytes(wl.shapes[si][1], wl.shapes[si][0], wl.G, wl.r, M) for si, M in two_calls)
    per_class = {"one_block_GBps": round(achieved, 1),
                 "two_blocks_GBps": round(two_bytes * args.steps / (cls_ms["two_blocks"] * 1e-3) / 1e9, 1),
                 "two_blocks_avg_launch_us": round(cls_ms["two_blocks"] / (len(two_calls) * args.steps) * 1e3, 3)}

    extra = {"decode_kernel_classes": per_class, "wall_s": round(wall, 3)}
    if not args.no_extra:
        log("overhead vs rank 0")
        wl0 = DecodeWorkload(dev, rank_override=0)
        extra["decode_overhead_vs_rank0"] = decode_overhead(torch, wl, wl0)
        del wl0
        torch.cuda.empty_cache()
        log("prefill context")
        del wl
        torch.cuda.empty_cache()
        extra["prefill_llama7b_bf16_M2048"] = prefill_context(torch, dev)
    cpu = None
    if not args.no_cpu:
        log("cpu oracle baseline")
        cpu = cpu_baseline()

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama7b-decode: 4096->4096, 4096->11008, 11008->4096 at M in "
                               "{1,4,16,32}; W4 g128 fp16 scale/zero; rank-32 compensator, sigmoid "
                               "gate; fp16 x N(0,1) with 1% channels x20",
                   "step": "12 compensated decode calls, graph-replayed",
                   "layer_copies": n_sets, "rotation_GiB": round(rot_bytes / 2**30, 3)},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

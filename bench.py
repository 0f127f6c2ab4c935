#!/usr/bin/env python3
"""Benchmark of the compensated 4-bit linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
    python bench.py --prefill-only      (the prefill calls alone, for profiling)

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
COPY_CAL_BYTES = 256 << 20


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Sticky error words of the workspaces each leg used (bit 0: a decode launch gave up
# waiting for its compensator producers).  Recorded in the JSON line; any bit set makes
# the run exit with status 3 after printing it.
WS_FLAGS: dict = {}


def record_flags(leg: str, workspaces) -> None:
    from quantized_gemm_error_amd import spear
    word = 0
    for ws in workspaces:
        if ws is not None:
            word |= spear.spear_workspace_flags(ws)
    WS_FLAGS[leg] = WS_FLAGS.get(leg, 0) | word
    if word:
        log(f"workspace flags {word:#x} after {leg}")


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
        # rank 0 gets a workspace too, so that it takes the same (split-K) launch shapes
        self.ws = [spear.new_workspace(l, maxM) for l in base]
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
    """Replay captured steps back to back; HIP events on the stream time the run.

    One graph holds a whole rotation of steps (each step's twelve calls, on
    the next copies of the layers); the timed region replays it, then
    per-step graphs for the remainder, exactly `steps` steps in all, with
    events only before the first and after the last launch, as a serving
    loop that captures its decode steps would run.  Two more passes of the same length replay only one kernel class
    each (the dominant one-token-block launches, M <= 16: nine calls a step;
    and the M = 32 launches: three) to give each class's device time per
    launch.
    """
    stream = torch.cuda.Stream()
    n_calls = len(wl.calls)
    n_phases = wl.n_sets // int(np.gcd(wl.n_sets, n_calls))
    classes = {"all": list(range(n_calls)),
               "one_block": [c for c in range(n_calls) if wl.calls[c][1] <= 16],
               "two_blocks": [c for c in range(n_calls) if wl.calls[c][1] > 16]}

    def issue_class(ph, cls):
        for c in classes[cls]:
            si, M = wl.calls[c]
            wl.issue(si, M, (ph * n_calls + c) % wl.n_sets, stream)

    with torch.cuda.stream(stream):
        for ph in range(n_phases):          # eager warm-up of every layer copy
            issue_class(ph, "all")
    torch.cuda.synchronize()
    # per class: one graph holding a whole rotation (n_phases steps), and one
    # graph per phase for a remainder of fewer steps
    full, per_phase = {}, {}
    for cls in classes:
        per_phase[cls] = []
        for ph in range(n_phases):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                issue_class(ph, cls)
            per_phase[cls].append(g)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for ph in range(n_phases):
                issue_class(ph, cls)
        full[cls] = g

    def run(cls, n):
        q, r = divmod(n, n_phases)
        with torch.cuda.stream(stream):    # replay() runs on the current stream
            for _ in range(q):
                full[cls].replay()
            for ph in range(r):
                per_phase[cls][ph].replay()

    run("all", warmup)
    torch.cuda.synchronize()
    out = {}
    for cls in classes:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        run(cls, steps)
        e1.record(stream)
        torch.cuda.synchronize()
        out[cls] = (e0.elapsed_time(e1), time.perf_counter() - t0)
    total_ms, wall = out["all"]
    cls_ms = {c: out[c][0] for c in ("one_block", "two_blocks")}
    return total_ms, wall, cls_ms, classes


def graph_times_ms(torch, variants, n, rounds=5, warm_ms=50.0):
    """Average device time per call of each variant: n back-to-back calls captured in one
    graph per variant.  The graphs are first replayed in turn until the GPU has been busy
    for warm_ms (so that every variant runs at the same, settled clock), then timed in
    alternation, `rounds` replays each; the best replay of each counts."""
    stream = torch.cuda.Stream()
    graphs = {}
    for name, issue_fn in variants.items():
        with torch.cuda.stream(stream):
            for i in range(n):
                issue_fn(i, stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                issue_fn(i, stream)
        graphs[name] = g

    def timed(g):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):   # replay() runs on the current stream
            s.record(stream)
            g.replay()
            e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e)

    busy = 0.0
    while busy < warm_ms:
        for g in graphs.values():
            busy += timed(g)
    best = {}
    names = list(graphs)
    for r in range(rounds):
        for k in range(len(names)):
            name = names[(r + k) % len(names)]
            t = timed(graphs[name]) / n
            best[name] = t if name not in best else min(best[name], t)
    return best


def graph_call_time_ms(torch, issue_fn, n, reps=5):
    """Average device time per call of n back-to-back calls captured in one graph."""
    return graph_times_ms(torch, {"v": issue_fn}, n, rounds=reps)["v"]


def decode_overhead(torch, wl_ec, wl_r0):
    """Per shape and M: the fused decode call with the compensator, the same kernel at rank 0,
    and the unfused form of the same call (the prefill path at decode M: the compensator
    kernel, U, the split-K GEMM and the kernel that adds U B^T, four launches), which is the
    pages' naive-insertion comparison."""
    from quantized_gemm_error_amd import spear
    out = {}
    for si, (K, N) in enumerate(wl_ec.shapes):
        for M in wl_ec.tokens:
            n = wl_ec.n_sets

            def unfused(i, s):
                spear.spear_linear_prefill(wl_ec.sets[i % n][si], wl_ec.x[(K, M)], y=wl_ec.y[(N, M)],
                                           workspace=wl_ec.ws[si], main_stream=s)
            t = graph_times_ms(torch, {"ec": lambda i, s: wl_ec.issue(si, M, i % n, s),
                                       "r0": lambda i, s: wl_r0.issue(si, M, i % n, s),
                                       "unfused": unfused}, n)
            t_ec, t_r0 = t["ec"], t["r0"]
            b = call_bytes(N, K, wl_ec.G, wl_ec.r, M)
            out[f"{K}->{N} M={M}"] = {
                "us_ec": round(t_ec * 1e3, 3), "us_r0": round(t_r0 * 1e3, 3),
                "us_unfused": round(t["unfused"] * 1e3, 3),
                "unfused_over_fused": round(t["unfused"] / t_ec, 3),
                "overhead_pct": round(100.0 * (t_ec / t_r0 - 1.0), 2),
                "GBps_ec": round(b / (t_ec * 1e-3) / 1e9, 1),
                "hbm_frac_ec": round(b / (t_ec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
    return out


def prefill_context(torch, device):
    """Llama-7B prefill, M = 2048, bf16: TFLOP/s of the serial schedule (compensator,
    then the GEMM with the compensator in its epilogue), of the concurrent schedule
    (compensator on an aux stream, merge after the join), and of rank 0 (same workspace)."""
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

        def run_serial(_i, s):
            spear.spear_linear_prefill(lay, x, y=y, workspace=ws, main_stream=s)

        def run_conc(_i, s):
            spear.spear_linear_prefill(lay, x, y=y, workspace=ws, main_stream=s, aux_stream=aux)

        def run_r0(_i, s):
            spear.spear_linear_prefill(lay0, x, y=y, workspace=ws, main_stream=s)
        t = graph_times_ms(torch, {"serial": run_serial, "conc": run_conc, "r0": run_r0}, 4)
        record_flags("prefill", [ws])
        t_s, t_c, t_r0 = t["serial"], t["conc"], t["r0"]
        f = call_flops(N, K, w["rank"], M)
        out[f"{K}->{N} M={M}"] = {
            "us_ec": round(t_s * 1e3, 1), "us_ec_concurrent": round(t_c * 1e3, 1),
            "us_r0": round(t_r0 * 1e3, 1),
            "TFLOPs_ec": round(f / (t_s * 1e-3) / 1e12, 1),
            "mfma_frac_ec": round(f / (t_s * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "overhead_pct": round(100.0 * (t_s / t_r0 - 1.0), 2),
            "overhead_pct_concurrent": round(100.0 * (t_c / t_r0 - 1.0), 2),
        }
        del lay, lay0, x, y, ws
    return out


def random_layer(torch, N, K, G, r, device, gen, act):
    """A 4-bit layer drawn directly on the device, for timing only (values do not change
    the work): random packed codes, fp16 scales in [0.001, 0.005), integer zero-points,
    A, B ~ N(0, 0.01), w_g ~ N(0, 0.05)."""
    from quantized_gemm_error_amd.spear import SpearLayer, qweight_rows
    ng = K // G
    qw = torch.randint(-2**31, 2**31 - 1, (qweight_rows(N), K // 8), dtype=torch.int32,
                       device=device, generator=gen)
    sc = (torch.rand((N, ng), device=device, generator=gen) * 0.004 + 0.001).to(torch.float16)
    zp = torch.randint(0, 16, (N, ng), device=device, generator=gen).to(torch.float16)
    lay = SpearLayer(N=N, K=K, group_size=G, qweight=qw, scales=sc, zeros=zp, rank=r)
    if r > 0:
        lay.A = (torch.randn((r, K), device=device, generator=gen) * 0.01).to(act)
        lay.B = (torch.randn((N, r), device=device, generator=gen) * 0.01).to(act)
        lay.w_gate = (torch.randn((K,), device=device, generator=gen) * 0.05).to(act)
    return lay


def llama70b_context(torch, device):
    """Llama-70B layer projections, per-channel 4-bit, rank 64, fp16, M in {1, 64, 256}
    through the phase-aware entry point; layer copies rotate over >= 1 GiB."""
    from quantized_gemm_error_amd import spear, synth
    w = synth.WORKLOADS["llama70b-layer"]
    gen = torch.Generator(device=device)
    gen.manual_seed(w["seed"])
    r = w["rank"]
    base = [random_layer(torch, N, K, K, r, device, gen, torch.float16) for K, N in w["shapes"]]
    set_bytes = sum(layer_bytes(l) for l in base)
    n_sets = max(2, -(-ROTATION_BYTES // set_bytes))
    sets = [base] + [[clone_layer(l) for l in base] for _ in range(n_sets - 1)]
    out = {}
    for si, (K, N) in enumerate(w["shapes"]):
        for M in w["tokens"]:
            x = torch.randn((M, K), device=device, generator=gen).to(torch.float16)
            y = torch.empty((M, N), dtype=torch.float16, device=device)
            ws = spear.new_workspace(base[si], M)
            t = graph_times_ms(torch, {
                "ec": lambda i, s: spear.spear_linear(sets[i % n_sets][si], x, y=y, workspace=ws,
                                                      main_stream=s),
                "r0": lambda i, s: spear.spear_linear(sets[i % n_sets][si].without_compensator(), x,
                                                      y=y, workspace=ws, main_stream=s)}, n_sets)
            record_flags("llama70b", [ws])
            t_ec, t_r0 = t["ec"], t["r0"]
            b, f = call_bytes(N, K, K, r, M), call_flops(N, K, r, M)
            gbs, tfs = b / (t_ec * 1e-3) / 1e9, f / (t_ec * 1e-3) / 1e12
            out[f"{K}->{N} M={M}"] = {
                "phase": spear.spear_linear_plan(base[si], M, ws.numel())["path"],
                "us_ec": round(t_ec * 1e3, 2), "us_r0": round(t_r0 * 1e3, 2),
                "overhead_pct": round(100.0 * (t_ec / t_r0 - 1.0), 2),
                "GBps_ec": round(gbs, 1), "hbm_frac_ec": round(gbs / HBM_PEAK_GBS, 4),
                "TFLOPs_ec": round(tfs, 1), "mfma_frac_ec": round(tfs / MFMA_F16_PEAK_TFLOPS, 4)}
            del ws, x, y
    del sets, base
    torch.cuda.empty_cache()
    return {"layer_copies": n_sets, "calls": out}


def rank_gate_context(torch, device):
    """The pages' per-rank gate (hidden 16, alpha 1) against the scalar gate and rank 0 on the
    7B shapes: decode at M = 1 and 16 (fp16) and prefill at M = 2048 (bf16); layer copies rotate
    over >= 1 GiB."""
    from quantized_gemm_error_amd import spear, synth
    w = synth.WORKLOADS["llama7b-decode"]
    gen = torch.Generator(device=device)
    gen.manual_seed(w["seed"] + 77)
    out = {}
    for K, N in w["shapes"]:
        for M, act in ((1, torch.float16), (16, torch.float16), (2048, torch.bfloat16)):
            base = random_layer(torch, N, K, w["group_size"], w["rank"], device, gen, act)
            n_sets = max(2, -(-ROTATION_BYTES // layer_bytes(base)))
            sets = [base] + [clone_layer(base) for _ in range(n_sets - 1)]
            rg = spear.rank_gate_to_device(synth.make_rank_gate(w["rank"], 16, seed=K + N,
                                                                 t_scale=0.01 * K ** 0.5), 1.0, device)
            x = torch.randn((M, K), device=device, generator=gen).to(act)
            y = torch.empty((M, N), dtype=act, device=device)
            ws = spear.new_workspace(base, M)

            def with_gate(l, gate):
                return spear.SpearLayer(l.N, l.K, l.group_size, l.qweight, l.scales, l.zeros, l.rank,
                                        l.A, l.B, l.w_gate, l.b_gate, gate)
            def variant(mk):
                return lambda i, s: spear.spear_linear(mk(sets[i % n_sets]), x, y=y, workspace=ws,
                                                       main_stream=s)
            t = graph_times_ms(torch, {"rank_gate": variant(lambda l: with_gate(l, rg)),
                                       "scalar_gate": variant(lambda l: l),
                                       "r0": variant(lambda l: l.without_compensator())}, n_sets)
            record_flags("rank_gate", [ws])
            out[f"{K}->{N} M={M}"] = {
                "us_rank_gate": round(t["rank_gate"] * 1e3, 2), "us_scalar_gate": round(t["scalar_gate"] * 1e3, 2),
                "us_r0": round(t["r0"] * 1e3, 2),
                "overhead_pct_rank_gate": round(100.0 * (t["rank_gate"] / t["r0"] - 1.0), 2),
                "overhead_pct_scalar_gate": round(100.0 * (t["scalar_gate"] / t["r0"] - 1.0), 2)}
            del sets, base, x, y, ws
            torch.cuda.empty_cache()
    return out


PROMPT = 8192  # prompt length for the serving leg's time-to-first-token figures
STREAM_REQUESTS = 12          # request stream: prompts 512..4096 tokens (multiples of 256),
STREAM_GAP_MS = 20.0          # 16..48 output tokens, exponential gaps between arrivals
STREAM_DENSITIES = (0, 4, 16, 32)
STREAM_STATIC = (512, 1024, 2048)
# inter-token targets: the pages quote 16 and 22 ms for whole models on their hardware; on
# this 96-linear stack the predicted steps cross 12 ms (1024-token chunks) and 20 ms (2048)
# between compensator densities 0 and 32, so those targets show the selector adapting
STREAM_SLOS_MS = (12.0, 16.0, 20.0)


def simulate_stream(requests, choose_chunk, run_step, max_batch=32):
    """Continuous batching over a request stream, on a virtual clock driven by measured steps.

    requests: (arrival_ms, prompt_tokens, output_tokens) per request, in arrival order.
    Requests are prefilled one at a time, first come first served, a chunk per step;
    every request past its prefill decodes one token per step, at most max_batch of them
    (a request starts its prefill only while fewer than max_batch are past it).
    choose_chunk(n_decoding) gives the step's chunk size; run_step(chunk_tokens,
    n_decoding) runs the step and returns its time in ms, which advances the clock.  A
    request's first token comes at the end of the step that holds its last prompt chunk
    (time to first token = that time minus its arrival); each later token comes one step
    after the previous one (inter-token latency = that step's time)."""
    pending = sorted(range(len(requests)), key=lambda i: requests[i][0])
    t, nxt = 0.0, 0
    fifo, running, last, left = [], [], {}, {}
    cur, cur_left = None, 0
    ttft, itl, steps, chunks_used = [], [], 0, {}
    done = 0
    while done < len(requests):
        while nxt < len(pending) and requests[pending[nxt]][0] <= t:
            fifo.append(pending[nxt])
            nxt += 1
        if cur is None and fifo and len(running) < max_batch:
            cur = fifo.pop(0)
            cur_left = requests[cur][1]
        n = len(running)
        c = min(choose_chunk(n), cur_left) if cur is not None else 0
        if c == 0 and n == 0:
            t = max(t, requests[pending[nxt]][0])   # idle until the next arrival
            continue
        t += run_step(c, n)
        steps += 1
        if c:
            chunks_used[c] = chunks_used.get(c, 0) + 1
        for r in list(running):
            itl.append(t - last[r])
            last[r] = t
            left[r] -= 1
            if left[r] == 0:
                running.remove(r)
                done += 1
        if cur is not None:
            cur_left -= c
            if cur_left == 0:
                ttft.append(t - requests[cur][0])
                if requests[cur][2] > 1:
                    running.append(cur)
                    last[cur], left[cur] = t, requests[cur][2] - 1
                else:
                    done += 1
                cur = None
    return {"ttft": ttft, "itl": itl, "steps": steps, "makespan_ms": t, "chunks": chunks_used}


def stream_summary(res, slos, requests):
    ttft, itl = np.asarray(res["ttft"]), np.asarray(res["itl"])
    out = {"ttft_ms_mean": round(float(ttft.mean()), 2), "ttft_ms_p90": round(float(np.percentile(ttft, 90)), 2),
           "itl_ms_p50": round(float(np.percentile(itl, 50)), 3), "itl_ms_p99": round(float(np.percentile(itl, 99)), 3),
           "itl_ms_max": round(float(itl.max()), 3),
           "steps": res["steps"], "makespan_ms": round(res["makespan_ms"], 1),
           "tokens_per_s": round(1e3 * sum(p + o for _, p, o in requests) / res["makespan_ms"], 1),
           "chunk_steps": {str(k): v for k, v in sorted(res["chunks"].items())}}
    for slo in slos:
        out[f"itl_over_{slo:g}ms_pct"] = round(100.0 * float((itl > slo).mean()), 2)
    return out


def serving_context(torch, device):
    """Chunked serving over a 32-block stack of the three 7B projections (random-init g128
    4-bit; every block carries a rank-32 compensator, and a density d switches on those of d
    seeded blocks).  A step is one prefill chunk of C tokens plus 32 decode tokens through
    every linear.  A latency table measured per (shape, compensated or not, C or decode)
    predicts the step time at every density; the chunk selector picks C for each budget.  At
    the configured density (4 blocks) every budget's chosen step is run and timed; at the
    other densities (0, 8, 16, 32) the step chosen for a 16 ms budget is.  Last, a seeded
    request stream runs under continuous batching with static chunk sizes and with the
    SLO-aware selector, and its measured time to first token and inter-token latency are
    reported per density (simulate_stream)."""
    from quantized_gemm_error_amd import spear, synth
    w = synth.WORKLOADS["llama7b-stack-serving"]
    gen = torch.Generator(device=device)
    gen.manual_seed(w["seed"])
    shapes, chunks, n_dec = list(w["shapes"]), list(w["chunks"]), w["decode_tokens"]
    nb = w["blocks"]
    stack = [[random_layer(torch, N, K, w["group_size"], w["rank"], device, gen, torch.float16)
              for K, N in shapes] for b in range(nb)]
    plain = [[l.without_compensator() for l in blk] for blk in stack]
    densities = (0, w["ec_blocks"], 8, 16, nb)
    ec_sets = {d: {int(b) for b in synth.ec_block_indices(nb, d, w["seed"])} if d else set()
               for d in densities}
    maxC = max(chunks) + n_dec
    xs = {K: torch.randn((maxC, K), device=device, generator=gen).to(torch.float16)
          for K in {k for k, _ in shapes}}
    ys = {N: torch.empty((maxC, N), dtype=torch.float16, device=device) for N in {n for _, n in shapes}}
    # one workspace for every linear: the calls are ordered on one stream
    nws = max(spear.spear_workspace_bytes(stack[0][si], maxC) for si in range(len(shapes)))
    wbuf = torch.zeros(nws + 256, dtype=torch.uint8, device=device)
    ws = wbuf[(-wbuf.data_ptr()) % 256:][:nws]

    def call(b, si, M, s, ec):
        K, N = shapes[si]
        lay = stack[b][si] if ec else plain[b][si]
        spear.spear_linear(lay, xs[K][:M], y=ys[N][:M], workspace=ws, main_stream=s)

    # latency table: each entry timed over all blocks in turn (cold weights)
    lut = {}
    for si in range(len(shapes)):
        for ec in (True, False):
            for M in chunks + [n_dec]:
                lut[(si, ec, M)] = graph_call_time_ms(
                    torch, lambda i, s: call(i % nb, si, M, s, ec), nb, reps=3)

    def predicted(C, ecs):
        return sum(lut[(si, b in ecs, C)] + lut[(si, b in ecs, n_dec)]
                   for b in range(nb) for si in range(len(shapes)))

    def measured(C, ecs, merged=False):
        def step(_i, s):
            for b in range(nb):
                for si in range(len(shapes)):
                    if merged:   # the chunk and the decode tokens as one batch of C + n_dec rows
                        call(b, si, C + n_dec, s, b in ecs)
                    else:
                        call(b, si, C, s, b in ecs)
                        call(b, si, n_dec, s, b in ecs)
        return graph_call_time_ms(torch, step, 1, reps=3)

    all_bytes = sum(layer_bytes(l) for blk in plain for l in blk)
    ec_bytes_per_block = sum(layer_bytes(stack[0][si]) - layer_bytes(plain[0][si]) for si in range(len(shapes)))
    out = {"densities": {}}
    for d in densities:
        ecs = ec_sets[d]
        pred = [predicted(C, ecs) for C in chunks]
        rec = {"ec_blocks": sorted(ecs),
               "predicted_step_ms": dict(zip(map(str, chunks), [round(p, 3) for p in pred])),
               "compensator_memory_pct": round(100.0 * d * ec_bytes_per_block / all_bytes, 3),
               "budgets": []}
        # a prompt of PROMPT tokens prefilled in chunks of C while 32 decode tokens run along:
        # time to first token = ceil(PROMPT / C) steps; inter-token latency of the decode
        # tokens meanwhile = one step (both predicted from the table)
        rec["prompt_tokens"] = PROMPT
        rec["ttft_itl_ms"] = {str(C): {"ttft": round(-(-PROMPT // C) * p, 3), "itl": round(p, 3)}
                              for C, p in zip(chunks, pred)}
        budgets = (1.0, 2.0, 4.0, 8.0, 16.0, w["budget_ms"]) if d == w["ec_blocks"] else (16.0,)
        for budget in budgets:
            C, violated = spear.spear_select_chunk(chunks, pred, budget)
            t = measured(C, ecs)
            rec["budgets"].append({"budget_ms": budget, "chunk": C, "violated": bool(violated),
                                   "predicted_ms": round(pred[chunks.index(C)], 3),
                                   "measured_ms": round(t, 3), "slo_met": bool(t <= budget)})
        if d == w["ec_blocks"]:
            # merged mixed batch: each linear runs once on the chunk's C rows plus the decode
            # tokens' rows (the prefill path), against the two separate calls
            rec["merged_vs_separate_ms"] = {str(C): {"separate": round(measured(C, ecs), 3),
                                                     "merged": round(measured(C, ecs, merged=True), 3)}
                                            for C in chunks}
        out["densities"][str(d)] = rec

    # A seeded request stream under continuous batching: each step one prefill chunk and
    # one decode token per running request, every step run from captured graphs and
    # timed.  Static chunk sizes against the SLO-aware selector (the largest chunk whose
    # predicted step time, from the table above, meets the inter-token target; the
    # largest chunk when nothing is decoding), at several compensator densities.
    rng = np.random.default_rng(w["seed"] + 1)
    n_req = STREAM_REQUESTS
    requests = [(float(a), int(p) * 256, int(o)) for a, p, o in
                zip(np.cumsum(rng.exponential(STREAM_GAP_MS, n_req)), rng.integers(2, 17, n_req),
                    rng.integers(16, 49, n_req))]
    sizes = sorted({256 * k for k in range(1, max(chunks) // 256 + 1)})
    stream = torch.cuda.Stream()
    stream_out = {"requests": n_req, "mean_gap_ms": STREAM_GAP_MS,
                  "prompt_tokens": [p for _, p, _ in requests], "output_tokens": [o for _, _, o in requests],
                  "slo_ms": list(STREAM_SLOS_MS), "densities": {}}
    for d in STREAM_DENSITIES:
        ecs = ec_sets[d] if d in ec_sets else {int(b) for b in synth.ec_block_indices(nb, d, w["seed"])}
        gp, gd = {}, {}
        for c in sizes:
            gp[c] = capture_graphs(torch, lambda _p: [call(b, si, c, stream, b in ecs) for b in range(nb)
                                                       for si in range(len(shapes))], 1, stream)[0]
        for n in range(1, n_dec + 1):
            gd[n] = capture_graphs(torch, lambda _p: [call(b, si, n, stream, b in ecs) for b in range(nb)
                                                       for si in range(len(shapes))], 1, stream)[0]
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def run_step(c, n):
            with torch.cuda.stream(stream):
                ev0.record(stream)
                if c:
                    gp[c].replay()
                if n:
                    gd[n].replay()
                ev1.record(stream)
            ev1.synchronize()
            return ev0.elapsed_time(ev1)

        for _ in range(3):                          # settle the clocks
            run_step(max(chunks), n_dec)
        pred_pre = {C: sum(lut[(si, b in ecs, C)] for b in range(nb) for si in range(len(shapes)))
                    for C in chunks}
        pred_dec = sum(lut[(si, b in ecs, n_dec)] for b in range(nb) for si in range(len(shapes)))
        rec = {"predicted_step_ms": {str(C): round(pred_pre[C] + pred_dec, 3) for C in chunks}}
        policies = {f"static_{C}": (lambda C: lambda n: C)(C) for C in STREAM_STATIC}

        def slo_policy(slo):
            def choose(n):
                if n == 0:
                    return max(chunks)
                C, _violated = spear.spear_select_chunk(chunks, [pred_pre[C] + pred_dec for C in chunks], slo)
                return C
            return choose
        for slo in STREAM_SLOS_MS:
            policies[f"slo_{slo:g}ms"] = slo_policy(slo)
        for name, choose in policies.items():
            rec[name] = stream_summary(simulate_stream(requests, choose, run_step, max_batch=n_dec),
                                       STREAM_SLOS_MS, requests)
        stream_out["densities"][str(d)] = rec
        del gp, gd
    out["request_stream"] = stream_out
    record_flags("serving", [ws])
    del stack, plain, xs, ys, ws, wbuf
    torch.cuda.empty_cache()
    return out


def serving_step(torch, device, steps=5):
    """One step of the serving stack, for profiling: every linear of the 32-block stack at a
    1024-token prefill chunk plus the 32 decode tokens, compensators on the configured 4
    blocks, captured in one graph and replayed `steps` times; prints the step time."""
    from quantized_gemm_error_amd import spear, synth
    w = synth.WORKLOADS["llama7b-stack-serving"]
    gen = torch.Generator(device=device)
    gen.manual_seed(w["seed"])
    shapes, n_dec, nb, C = list(w["shapes"]), w["decode_tokens"], w["blocks"], 1024
    ecs = {int(b) for b in synth.ec_block_indices(nb, w["ec_blocks"], w["seed"])}
    stack = [[random_layer(torch, N, K, w["group_size"], w["rank"], device, gen, torch.float16)
              for K, N in shapes] for b in range(nb)]
    stack = [[l if b in ecs else l.without_compensator() for l in blk] for b, blk in enumerate(stack)]
    xs = {K: torch.randn((C, K), device=device, generator=gen).to(torch.float16) for K, _ in shapes}
    ys = {N: torch.empty((C, N), dtype=torch.float16, device=device) for _, N in shapes}
    # one workspace for every linear (the calls are ordered on one stream), sized for the largest
    ws = spear.new_workspace(max((l for blk in stack for l in blk),
                                 key=lambda l: spear.spear_workspace_bytes(l, C)), C)

    def step(_i, s):
        for blk in stack:
            for si, (K, N) in enumerate(shapes):
                spear.spear_linear(blk[si], xs[K][:C], y=ys[N][:C], workspace=ws, main_stream=s)
                spear.spear_linear(blk[si], xs[K][:n_dec], y=ys[N][:n_dec], workspace=ws, main_stream=s)
    t = graph_times_ms(torch, {"step": step}, 1, rounds=steps, warm_ms=0.0)["step"]
    record_flags("serving", [ws])
    return {"chunk": C, "decode_tokens": n_dec, "ec_blocks": sorted(ecs), "step_ms": round(t, 3)}


def ceilings(torch, device):
    """Context only: a 1 GiB device-to-device copy, and hipBLASLt bf16 GEMMs at the prefill
    shapes (dense bf16 weights, torch.matmul)."""
    from quantized_gemm_error_amd import synth
    out = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["d2d_copy_GBps"] = round(5 * 2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    # a device copy of one layer's weight bytes (4-bit words plus g128 scales and zeros), on
    # copies rotating over >= 1 GiB as the decode bench does: the launch-to-launch floor of
    # streaming that many bytes once (read + write counted)
    lay_copy = {}
    for K, N in synth.LLAMA7B_SHAPES:
        nbytes = N * K // 2 + 4 * N * K // 128
        n = max(2, -(-ROTATION_BYTES // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=device) for _ in range(n)]
        dsts = [torch.empty(nbytes, dtype=torch.uint8, device=device) for _ in range(2)]
        t = graph_call_time_ms(torch, lambda i, st: dsts[i % 2].copy_(bufs[i]), n)
        lay_copy[f"{K}->{N}"] = {"bytes_read": nbytes, "us": round(t * 1e3, 3),
                                 "read_GBps": round(nbytes / (t * 1e-3) / 1e9, 1)}
        del bufs, dsts
    out["layer_sized_copy"] = lay_copy
    gemm = {}
    for K, N in synth.LLAMA7B_SHAPES:
        a = torch.randn((2048, K), device=device).to(torch.bfloat16)
        bt = torch.randn((N, K), device=device).to(torch.bfloat16).t().contiguous()  # [K][N]
        torch.matmul(a, bt)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            torch.matmul(a, bt)
        e1.record()
        torch.cuda.synchronize()
        gemm[f"{K}->{N} M=2048"] = round(10 * 2 * 2048 * K * N / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        del a, bt
    out["hipblaslt_bf16_dense_TFLOPs"] = gemm
    torch.cuda.empty_cache()
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


# ---------------------------------------------------------------------------
# rocprofv3 summaries (CPU only): kernel-trace statistics and HBM traffic
# ---------------------------------------------------------------------------

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_llama7b_traffic.json")
DOMINANT_SOURCES = ("quantized_gemm_error_amd/csrc/decode.hip",
                    "quantized_gemm_error_amd/csrc/decode_impl.inc",
                    "quantized_gemm_error_amd/csrc/decode_w8.hip",
                    "quantized_gemm_error_amd/csrc/decode_w4.hip",
                    "quantized_gemm_error_amd/csrc/device_common.h",
                    "quantized_gemm_error_amd/csrc/internal.h")
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_trace -o run -- "
             "python3 bench.py --steps 300 --warmup 10 --no-extra --no-cpu")
PMC_CMD = ("rocprofv3 --pmc {counter} -f csv -d gpurun_out/prof_{tag} -o run -- "
           "python3 bench.py --steps 10 --warmup 2 --no-extra --no-cpu --copy-calibration")


def dominant_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _decode_template_args(name):
    """(DT, MB, EC, PERCH, ...) of a decode_kernel or decode_split_kernel instantiation, else
    None."""
    for key in ("decode_kernel<", "decode_split_kernel<"):
        if key in name:
            inner = name[name.index(key) + len(key):].split(">")[0]
            return tuple(t.strip() for t in inner.split(","))
    return None


def _is_dominant(name):
    t = _decode_template_args(name)
    return t is not None and t[1] == "1" and t[2] == "true"


def _short(name):
    """A kernel's name without return type, namespaces and parameter list."""
    n = name.replace("(anonymous namespace)::", "").replace("void ", "").rsplit("(", 1)[0]
    return n.replace("spear::w4::", "w4::").replace("spear::w8::", "w8::").replace("spear::", "")


def measured_traffic():
    """HBM bytes per dominant launch from the committed counter summary, or None if the
    kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    if rec.get("kernel_sources_sha256") != dominant_sources_sha256():
        return None, "kernel sources changed since the counters were taken"
    return rec.get("traffic_bytes_per_launch"), None


def summarize_profiles(trace_dir, fetch_dir, write_dir, out_dir):
    import csv
    import statistics

    def rows(path):
        with open(path, newline="") as f:
            return list(csv.DictReader(f))

    os.makedirs(out_dir, exist_ok=True)
    # ---- kernel trace --------------------------------------------------------
    stats = rows(os.path.join(trace_dir, "run_kernel_stats.csv"))
    trace = rows(os.path.join(trace_dir, "run_kernel_trace.csv"))
    trace.sort(key=lambda r: int(r["Dispatch_Id"]))
    dom = [r for r in trace if _is_dominant(r["Kernel_Name"])]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in dom]
    # start-to-start spacing of back-to-back dominant dispatches (the graph's cadence)
    spacing = []
    for a, b in zip(trace, trace[1:]):
        if _is_dominant(a["Kernel_Name"]) and _is_dominant(b["Kernel_Name"]) and \
                int(b["Dispatch_Id"]) == int(a["Dispatch_Id"]) + 1:
            spacing.append((int(b["Start_Timestamp"]) - int(a["Start_Timestamp"])) / 1e3)
    bench_line = None
    log_path = trace_dir.rstrip("/") + ".log"
    if os.path.exists(log_path):
        for ln in open(log_path):
            if ln.startswith("{"):
                bench_line = json.loads(ln)
    # the pass that replays only the dominant launches: the longest run of
    # consecutive dominant dispatches; its span per launch is what HIP events
    # around that pass measure
    runs, cur = [], []
    for r in trace:
        if _is_dominant(r["Kernel_Name"]) and (not cur or int(r["Dispatch_Id"]) == int(cur[-1]["Dispatch_Id"]) + 1):
            cur.append(r)
        else:
            if cur:
                runs.append(cur)
            cur = [r] if _is_dominant(r["Kernel_Name"]) else []
    if cur:
        runs.append(cur)
    longest = max(runs, key=len)
    span_us = (int(longest[-1]["End_Timestamp"]) - int(longest[0]["Start_Timestamp"])) / 1e3 / len(longest)
    agree = ["", f"- dominant-only pass: {len(longest)} consecutive dispatches, span per launch "
                 f"{span_us:.3f} us, mean duration {statistics.mean((int(r['End_Timestamp']) - int(r['Start_Timestamp'])) / 1e3 for r in longest):.3f} us"]
    if bench_line is not None:
        b_us = bench_line["roofline"]["avg_launch_us"]
        agree += ["", f"bench.py's own figure in the same run (HIP events around that pass): {b_us:.3f} us "
                      f"per launch; trace span / bench = {span_us / b_us:.3f}."]
    lines = ["# decode_kernel, Llama-7B decode projections: rocprofv3 kernel trace", "",
             "Command (repository root, one MI355X):", "", "    " + TRACE_CMD, "",
             "Dominant kernel: the decode kernels with one 16-token block (M <= 16) and the "
             "compensator, all their instantiations (the three shapes and M select the "
             "row-block width, the staging mode and, for the 11008-wide K at M = 16, the "
             "split-K launch decode_split_kernel).", "",
             f"- dispatches: {len(dom)}",
             f"- mean kernel duration: {statistics.mean(dur):.3f} us (median {statistics.median(dur):.3f})",
             f"- mean start-to-start spacing of consecutive dispatches: "
             f"{statistics.mean(spacing):.3f} us over {len(spacing)} pairs" if spacing else "- no pairs",
             *agree,
             "", "rocprofv3 stamps a kernel's start when the previous one in the stream ends, so "
                 "for back-to-back launches its duration is the launch-to-launch time.",
             "", "Per kernel (rocprofv3 --stats):", "",
             "| kernel | calls | average us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{_short(r['Name'])[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {r['Percentage']} |")
    with open(os.path.join(out_dir, "decode_kernel_llama7b_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # ---- counters --------------------------------------------------------------
    def counter_pass(d):
        rs = rows(os.path.join(d, "run_counter_collection.csv"))
        rs.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [r for r in rs if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")][-3:]
        cal = statistics.mean(float(r["Counter_Value"]) for r in copies)  # KiB per 256 MiB copy
        scale = cal / (COPY_CAL_BYTES / 1024.0)
        per = {}
        for r in rs:
            if _is_dominant(r["Kernel_Name"]):
                per.setdefault((_short(r["Kernel_Name"]), r["Grid_Size"]), []).append(float(r["Counter_Value"]))
        allv = [v for vs in per.values() for v in vs]
        return scale, cal, per, statistics.mean(allv), len(allv)

    f_scale, f_cal, f_per, f_mean, f_n = counter_pass(fetch_dir)
    w_scale, w_cal, w_per, w_mean, w_n = counter_pass(write_dir)
    fetch_b = f_mean * 1024.0 / f_scale
    write_b = w_mean * 1024.0 / w_scale
    traffic = fetch_b + write_b
    lines = ["# decode_kernel, Llama-7B decode projections: HBM traffic from counters", "",
             "Commands (repository root, one MI355X, one counter per pass):", "",
             "    " + PMC_CMD.format(counter="FETCH_SIZE", tag="fetch"),
             "    " + PMC_CMD.format(counter="WRITE_SIZE", tag="write"), "",
             "Scale: the last three dispatches of each pass are device-to-device copies of "
             f"{COPY_CAL_BYTES >> 20} MiB (`__amd_rocclr_copyBuffer`).", "",
             f"- FETCH_SIZE per copy: {f_cal:.1f} KiB -> scale {f_scale:.5f}",
             f"- WRITE_SIZE per copy: {w_cal:.1f} KiB -> scale {w_scale:.5f}", "",
             f"Dominant kernel (M <= 16, compensated), mean over {f_n} / {w_n} dispatches:", "",
             f"- FETCH_SIZE {f_mean:.1f} KiB -> {fetch_b / 1e6:.3f} MB read",
             f"- WRITE_SIZE {w_mean:.1f} KiB -> {write_b / 1e6:.3f} MB written",
             f"- traffic per launch: {traffic / 1e6:.3f} MB", "",
             "| instantiation | grid (threads) | dispatches | FETCH KiB | WRITE KiB | scaled MB |",
             "|---|---:|---:|---:|---:|---:|"]
    for k in sorted(f_per):
        fv, wv = f_per[k], w_per.get(k, [0.0])
        fm, wm = statistics.mean(fv), statistics.mean(wv)
        lines.append(f"| `{k[0]}` | {k[1]} | {len(fv)} | {fm:.1f} | {wm:.1f} | "
                     f"{(fm / f_scale + wm / w_scale) * 1024 / 1e6:.3f} |")
    with open(os.path.join(out_dir, "decode_kernel_llama7b_hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    rec = {"kernel": "decode_kernel and decode_split_kernel, M <= 16, compensated (all instantiations)",
           "kernel_sources_sha256": dominant_sources_sha256(),
           "traffic_bytes_per_launch": int(round(traffic)),
           "fetch_bytes_per_launch": int(round(fetch_b)), "write_bytes_per_launch": int(round(write_b)),
           "fetch_scale": round(f_scale, 6), "write_scale": round(w_scale, 6),
           "dispatches": [f_n, w_n],
           "commands": [PMC_CMD.format(counter="FETCH_SIZE", tag="fetch"),
                        PMC_CMD.format(counter="WRITE_SIZE", tag="write")]}
    with open(TRAFFIC_FILE if out_dir == os.path.dirname(TRAFFIC_FILE)
              else os.path.join(out_dir, os.path.basename(TRAFFIC_FILE)), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


LAYER_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_{tag}_trace -o run -- python3 bench.py {mode}",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_{tag}_fetch -o run -- python3 bench.py {mode} --copy-calibration",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_{tag}_write -o run -- python3 bench.py {mode} --copy-calibration",
}
LAYER_MODES = {"llama70b_layer": "--llama70b-only", "serving_step_7b": "--serving-step"}


def summarize_layer_profiles(tag, title, trace_dir, fetch_dir, write_dir, out_dir):
    """Per (kernel, grid size): dispatches, mean duration (trace run) and mean HBM bytes read
    and written per dispatch (FETCH_SIZE and WRITE_SIZE runs, each scaled by what the same
    counter reads for a device-to-device copy of known size)."""
    import csv
    import statistics

    def rows(path):
        with open(path, newline="") as f:
            return list(csv.DictReader(f))

    trace = rows(os.path.join(trace_dir, "run_kernel_trace.csv"))
    dur = {}
    for r in trace:
        if r["Kernel_Name"].startswith("__amd_rocclr") or "at::" in r["Kernel_Name"]:
            continue   # copies and the set-up's torch kernels
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        key = (_short(r["Kernel_Name"]), grid)
        dur.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counter_pass(d):
        rs = rows(os.path.join(d, "run_counter_collection.csv"))
        rs.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [r for r in rs if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")][-3:]
        cal = statistics.mean(float(r["Counter_Value"]) for r in copies)
        scale = cal / (COPY_CAL_BYTES / 1024.0)
        per = {}
        for r in rs:
            if r["Kernel_Name"].startswith("__amd_rocclr"):
                continue
            per.setdefault((_short(r["Kernel_Name"]), int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return scale, cal, {k: statistics.mean(v) * 1024.0 / scale for k, v in per.items()}

    f_scale, f_cal, fetch = counter_pass(fetch_dir)
    w_scale, w_cal, write = counter_pass(write_dir)
    mode = LAYER_MODES.get(tag, "")
    lines = [f"# {title}: rocprofv3 trace and HBM traffic", "",
             "Commands (repository root, one MI355X; counters one per pass):", ""]
    lines += ["    " + LAYER_CMDS[k].format(tag=tag, mode=mode) for k in ("trace", "fetch", "write")]
    lines += ["", f"Byte scale: the last three dispatches of each counter pass copy {COPY_CAL_BYTES >> 20} "
                  f"MiB device to device; FETCH_SIZE reads {f_cal:.1f} KiB (scale {f_scale:.5f}), "
                  f"WRITE_SIZE {w_cal:.1f} KiB (scale {w_scale:.5f}) per copy.", "",
              "rocprofv3 stamps a kernel's start when the previous one in the stream ends, so "
              "back-to-back durations are launch to launch.", "",
              "| kernel | grid (threads) | dispatches | mean us | read MB | written MB | GB/s (read+written) |",
              "|---|---:|---:|---:|---:|---:|---:|"]
    for key in sorted(dur, key=lambda k: -statistics.mean(dur[k]) * len(dur[k])):
        d = statistics.mean(dur[key])
        fb, wb = fetch.get(key), write.get(key)
        rate = f"{(fb + wb) / (d * 1e-6) / 1e9:.0f}" if fb is not None and wb is not None and d > 0 else "-"
        lines.append(f"| `{key[0][:80]}` | {key[1]} | {len(dur[key])} | {d:.2f} | "
                     f"{'-' if fb is None else f'{fb / 1e6:.3f}'} | {'-' if wb is None else f'{wb / 1e6:.3f}'} | {rate} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{tag}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


PREFILL_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_prefill_trace -o run -- "
                     "python3 bench.py --prefill-only")
PREFILL_PMC = (("pmc1", "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
                        "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES GRBM_GUI_ACTIVE"),
               ("pmc2", "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS SQ_WAIT_ANY "
                        "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_LDS_DATA_FIFO_FULL SQ_VALU_MFMA_COEXEC_CYCLES "
                        "GRBM_GUI_ACTIVE"))
PREFILL_PMC_CMD = ("rocprofv3 --pmc {counters} -f csv -d gpurun_out/prof_prefill_{tag} -o run -- "
                   "python3 bench.py --prefill-only")


def summarize_prefill_profiles(trace_dir, pmc1_dir, pmc2_dir, out_dir):
    """profiles/prefill_kernels_llama7b_m2048.md from the prefill-only trace and counter passes."""
    import csv
    import re
    import statistics

    def rows(path):
        with open(path, newline="") as f:
            return list(csv.DictReader(f))

    def short(name):
        m = re.search(r"(prefill_\w+)(<[^>]*>)?", name)
        return (m.group(1) + (m.group(2) or "")) if m else name.split("(")[0][:60]

    trace = [r for r in rows(os.path.join(trace_dir, "run_kernel_trace.csv")) if "prefill_" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    # the calls run shape by shape (4096->4096, 4096->11008, 11008->4096); the 86-tile
    # grid of the GEMM marks the middle shape
    n_of = lambda r: int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
    mid = [i for i, r in enumerate(trace) if "gemm" in r["Kernel_Name"] and n_of(r) == 86]
    lo = mid[0]
    while lo > 0 and "gemm" not in trace[lo - 1]["Kernel_Name"]:
        lo -= 1
    parts = {"4096->4096": trace[:lo], "4096->11008": trace[lo:mid[-1] + 1], "11008->4096": trace[mid[-1] + 1:]}
    lines = ["# Prefill kernels, Llama-7B projections at M = 2048 (bf16): rocprofv3 trace and counters", "",
             "Commands (repository root, one MI355X):", "", "    " + PREFILL_TRACE_CMD]
    for tag, counters in PREFILL_PMC:
        lines.append("    " + PREFILL_PMC_CMD.format(counters=counters, tag=tag))
    lines += ["", "`bench.py --prefill-only` runs, per shape, the serial schedule (compensator, U, "
                  "then the GEMM with U B^T in its epilogue), the concurrent schedule and rank 0, "
                  "each as graph replays.  rocprofv3 stamps a kernel's start when the previous one "
                  "in the stream ends, so durations are launch to launch.", "",
              "Median duration per kernel and shape (us):", "",
              "| shape | kernel | dispatches | median us |", "|---|---|---:|---:|"]
    for shape, rs in parts.items():
        per = {}
        for r in rs:
            per.setdefault(short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for k, v in per.items():
            lines.append(f"| {shape} | `{k}` | {len(v)} | {statistics.median(v):.1f} |")

    def pmc(d):
        per = {}
        for r in rows(os.path.join(d, "run_counter_collection.csv")):
            if "prefill_" not in r["Kernel_Name"]:
                continue
            per.setdefault(short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        return {k: {c: statistics.mean(v) for c, v in cs.items()} for k, cs in per.items()}

    c1, c2 = pmc(pmc1_dir), pmc(pmc2_dir)
    lines += ["", "Counters per dispatch, mean over the dispatches of each kernel (all three shapes). "
                  "GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's busy cycles are an "
                  "eighth of it; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x "
                  "1024 SIMDs).", "",
              "| kernel | MFMA busy | VALU instr per MFMA | LDS bank-conflict cycles / LDS active | "
              "MFMA cycles with VALU co-issue | LDS wait / all wait |",
              "|---|---:|---:|---:|---:|---:|"]
    for k in sorted(c1):
        a, b = c1[k], c2.get(k, {})
        xcd = a["GRBM_GUI_ACTIVE"] / 8.0
        busy = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd * 1024) if xcd else 0.0
        vpm = a["SQ_INSTS_VALU"] / a["SQ_INSTS_MFMA"] if a.get("SQ_INSTS_MFMA") else float("nan")
        bank = a["SQ_LDS_BANK_CONFLICT"] / a["SQ_LDS_IDX_ACTIVE"] if a.get("SQ_LDS_IDX_ACTIVE") else 0.0
        co = (b.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / a["SQ_VALU_MFMA_BUSY_CYCLES"]
              if a.get("SQ_VALU_MFMA_BUSY_CYCLES") else 0.0)
        lw = b.get("SQ_WAIT_INST_LDS", 0.0) / b["SQ_WAIT_ANY"] if b.get("SQ_WAIT_ANY") else 0.0
        vpm_s = f"{vpm:.2f}" if vpm == vpm else "-"
        lines.append(f"| `{k}` | {100 * busy:.1f}% | {vpm_s} | {100 * bank:.1f}% | {100 * co:.1f}% | "
                     f"{100 * lw:.1f}% |")
    lines += ["", "Raw means per dispatch:", "", "| kernel | counter | value |", "|---|---|---:|"]
    for k in sorted(c1):
        for c, v in sorted({**c1[k], **c2.get(k, {})}.items()):
            lines.append(f"| `{k}` | {c} | {v:.4g} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "prefill_kernels_llama7b_m2048.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extra", action="store_true", help="skip overhead/prefill context")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 256 MiB device to device three times: the "
                         "reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from rocprofv3 CSV output (no GPU)")
    ap.add_argument("--summarize-prefill-profiles", nargs=3, metavar=("TRACE_DIR", "PMC1_DIR", "PMC2_DIR"),
                    help="write the prefill profile summary from rocprofv3 CSV output (no GPU)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the Llama-7B prefill calls (M = 2048, bf16) and print them: "
                         "the command that the prefill kernel profiles are taken with")
    ap.add_argument("--llama70b-only", action="store_true",
                    help="run only the Llama-70B layer leg and print it (profiling)")
    ap.add_argument("--serving-step", action="store_true",
                    help="replay one serving step (32 blocks x 3 linears, 1024-token chunk + 32 "
                         "decode tokens) a few times and print its time (profiling)")
    ap.add_argument("--summarize-layer-profiles", nargs=5,
                    metavar=("TAG", "TITLE", "TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/TAG.md: per kernel and grid, duration and copy-scaled "
                         "HBM bytes from rocprofv3 CSV output (no GPU)")
    ap.add_argument("--serving-only", action="store_true",
                    help="run only the serving-stack leg (latency table, chunk selector, request "
                         "stream) and print it")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, out_dir=os.path.join(ROOT, "profiles"))
        return
    if args.summarize_prefill_profiles:
        summarize_prefill_profiles(*args.summarize_prefill_profiles, out_dir=os.path.join(ROOT, "profiles"))
        return
    if args.summarize_layer_profiles:
        summarize_layer_profiles(*args.summarize_layer_profiles, out_dir=os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_gemm_error_amd import spear
    spear.load_library()
    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.prefill_only:
        print(json.dumps({"prefill_llama7b_bf16_M2048": prefill_context(torch, dev)}), flush=True)
        return
    if args.serving_only:
        print(json.dumps({"serving_stack_7b": serving_context(torch, dev)}), flush=True)
        return
    if args.llama70b_only or args.serving_step:
        out = ({"llama70b_layer_fp16": llama70b_context(torch, dev)} if args.llama70b_only
               else {"serving_step": serving_step(torch, dev)})
        if args.copy_calibration:   # the reference copies that scale the byte counters
            src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps(out), flush=True)
        return

    log("building decode workload")
    wl = DecodeWorkload(dev)
    n_sets, rot_bytes = wl.n_sets, wl.rotation_bytes
    log(f"{n_sets} layer-set copies, rotation {rot_bytes / 2**30:.2f} GiB")
    total_ms, wall, cls_ms, classes = timed_decode_steps(torch, wl, args.steps, args.warmup)
    record_flags("decode", wl.ws)
    ms_per_step = total_ms / args.steps
    value = wl.step_bytes * args.steps / (total_ms * 1e-3) / 1e9
    log(f"decode: {ms_per_step * 1e3:.1f} us/step, {value:.1f} GB/s")

    if args.copy_calibration:
        src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # dominant kernel: decode_kernel, one token block (M <= 16), compensated, group-wise
    dom_calls = [wl.calls[c] for c in classes["one_block"]]
    dom_bytes = sum(call_bytes(wl.shapes[si][1], wl.shapes[si][0], wl.G, wl.r, M) for si, M in dom_calls)
    n_launch = len(dom_calls) * args.steps
    dom_ms = cls_ms["one_block"]
    achieved = dom_bytes * args.steps / (dom_ms * 1e-3) / 1e9
    traffic, traffic_note = measured_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                "traffic_note": traffic_note,
                "kernel": "decode_kernel / decode_split_kernel<f16, one 16-token block, compensated, group-wise>",
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
        record_flags("decode_overhead", wl.ws + wl0.ws)
        del wl0
        torch.cuda.empty_cache()
        log("prefill context")
        del wl
        torch.cuda.empty_cache()
        extra["prefill_llama7b_bf16_M2048"] = prefill_context(torch, dev)
        log("llama-70B layer")
        extra["llama70b_layer_fp16"] = llama70b_context(torch, dev)
        log("per-rank gate")
        extra["rank_gate_7b"] = rank_gate_context(torch, dev)
        log("serving stack")
        extra["serving_stack_7b"] = serving_context(torch, dev)
        log("ceilings")
        extra["ceilings"] = ceilings(torch, dev)
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
        "roofline": roofline, "cpu_baseline": cpu, "workspace_flags": WS_FLAGS, "extra": extra,
    }
    print(json.dumps(line), flush=True)
    if any(WS_FLAGS.values()):
        log("a workspace error flag is set: the timings above ran a fallback path")
        sys.exit(3)


if __name__ == "__main__":
    main()

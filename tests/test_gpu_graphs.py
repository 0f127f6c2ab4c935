"""The layer's calls captured in HIP graphs (torch.cuda.graph) and replayed.

The pages run the prefill compensator beside the GEMM as a static graph, and decode
steps are replayed from graphs by serving loops.  Each test captures the calls once,
replays the graph many times with eager work and synchronisations between replays, and
checks every replay bit for bit against the eager result, which itself is checked
against the float64 oracle on sampled rows.  The workspace's flags and counters must be
back at zero at the end: the decode kernels reset them on every call, and a replay
that skipped the reset would show up as a wrong output or a non-zero counter.
"""

import numpy as np
import pytest

from quantized_gemm_error_amd import spear, synth

from gpu_helpers import assert_close, gpu_y_f64, note, oracle_y, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"
WS_HEADER_BYTES = 2048 + 128 * 128


def _header_zero(ws):
    return not bool(ws[:WS_HEADER_BYTES].any().item())


def _eager_noise(lay, x, ws):
    """Unrelated eager work between replays: another decode call and a torch op."""
    spear.spear_linear_decode(lay, x, workspace=ws)
    torch.randn(1 << 16, device=DEV).sum()


def _replay_and_check(graph, outs, refs, replays, noise, stream):
    for it in range(replays):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()   # the fills (current stream) before the replay (its own stream)
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, refs)):
            if not torch.equal(o.view(torch.int16), r.view(torch.int16)):
                raise AssertionError(f"replay {it}, call {j}: output differs from the eager call")
        noise()
        torch.cuda.synchronize()


def test_decode_step_graph_replayed():
    """The headline decode step (the three Llama-7B projections at 1, 4, 16 and 32 tokens,
    g128, rank 32), captured once and replayed 120 times."""
    w = synth.WORKLOADS["llama7b-decode"]
    layers, hls, wss, xs, xbs = [], [], [], {}, {}
    for i, (K, N) in enumerate(w["shapes"]):
        hl = synth.make_layer(N, K, w["group_size"], w["rank"], seed=w["seed"] + 10 * i)
        hls.append(hl)
        layers.append(spear.layer_to_device(hl, DEV))
        wss.append(spear.new_workspace(layers[-1], 32))
    for K in {k for k, _ in w["shapes"]}:
        xbs[K] = synth.make_activations(32, K, seed=w["seed"] + K, outliers=True)
        xs[K] = spear.act_to_device(xbs[K], "f16", DEV)
    calls = [(si, M) for M in w["tokens"] for si in range(len(w["shapes"]))]
    outs = [torch.empty((M, w["shapes"][si][1]), dtype=torch.float16, device=DEV) for si, M in calls]
    stream = torch.cuda.Stream()

    def step():
        for (si, M), y in zip(calls, outs):
            K = w["shapes"][si][0]
            spear.spear_linear(layers[si], xs[K][:M], y=y, workspace=wss[si],
                               main_stream=torch.cuda.current_stream())

    note("decode step eager")
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    for (si, M), r in zip(calls, refs):
        K, N = w["shapes"][si]
        rows = sample_rows(N, 64, seed=si + M)
        assert_close(gpu_y_f64(r, "f16")[:, rows], oracle_y(hls[si], xbs[K][:M], rows=rows),
                     f"eager {K}->{N} M={M}")
    note("decode step capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    note("decode step replays")
    _replay_and_check(g, outs, refs, 120,
                      lambda: _eager_noise(layers[0], xs[4096][:3], wss[0]), stream)
    for ws in wss:
        assert spear.spear_workspace_flags(ws) == 0
        assert _header_zero(ws)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_concurrent_prefill_graph_replayed(dtype):
    """The pages' prefill schedule (compensator on an aux stream beside the GEMM, joined
    before the merge) captured as one graph with its fork and join, replayed 100 times;
    Llama-7B 4096->4096 at 2048 tokens, and 4096->11008 at 300 tokens (K split)."""
    w = synth.WORKLOADS["llama7b-prefill"]
    cases = [(4096, 4096, 2048), (4096, 11008, 300)]
    layers, hls, xbs, xs, outs, wss = [], [], [], [], [], []
    for i, (K, N, M) in enumerate(cases):
        hl = synth.make_layer(N, K, w["group_size"], w["rank"], seed=w["seed"] + i, dtype=dtype)
        hls.append(hl)
        layers.append(spear.layer_to_device(hl, DEV))
        xbs.append(synth.make_activations(M, K, seed=w["seed"] + i, dtype=dtype, outliers=True))
        xs.append(spear.act_to_device(xbs[-1], dtype, DEV))
        act = torch.bfloat16 if dtype == "bf16" else torch.float16
        outs.append(torch.empty((M, N), dtype=act, device=DEV))
        wss.append(spear.new_workspace(layers[-1], M))
    stream, aux = torch.cuda.Stream(), torch.cuda.Stream()

    def run():
        for lay, x, y, ws in zip(layers, xs, outs, wss):
            spear.spear_linear_prefill(lay, x, y=y, workspace=ws,
                                       main_stream=torch.cuda.current_stream(), aux_stream=aux)

    note(f"concurrent prefill eager {dtype}")
    with torch.cuda.stream(stream):
        run()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    for (K, N, M), hl, xb, r in zip(cases, hls, xbs, refs):
        rows = sample_rows(N, 64, seed=N)
        toks = np.unique(np.r_[np.random.default_rng(M).choice(M, 32, replace=False), M - 1])
        assert_close(gpu_y_f64(r, dtype)[np.ix_(toks, rows)], oracle_y(hl, xb[toks], rows=rows),
                     f"eager {K}->{N} M={M}")
    note(f"concurrent prefill capture {dtype}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    torch.cuda.synchronize()
    note(f"concurrent prefill replays {dtype}")

    def noise():
        spear.spear_linear_prefill(layers[0], xs[0][:64], workspace=wss[0])
        torch.randn(1 << 16, device=DEV).sum()
    _replay_and_check(g, outs, refs, 100, noise, stream)


def test_decode_soak_graph_replayed():
    """About 5,000 decode calls on one workspace: 50 calls of mixed token counts (1..32)
    on two layers (one long enough in K that 16 or more tokens take the split-K launch)
    captured in one graph and replayed 100 times; stops at the first replay whose outputs
    differ from the eager calls."""
    specs = [(1024, 8192, 128, 32), (1536, 4096, 0, 24)]   # N, K, G, r
    layers, hls = [], []
    for i, (N, K, G, r) in enumerate(specs):
        hl = synth.make_layer(N, K, G, r, seed=900 + i, b_gate=0.2)
        hls.append(hl)
        layers.append(spear.layer_to_device(hl, DEV))
    nws = max(spear.spear_workspace_bytes(l, 32) for l in layers)
    buf = torch.zeros(nws + 256, dtype=torch.uint8, device=DEV)
    ws = buf[(-buf.data_ptr()) % 256:][:nws]
    xbs = [synth.make_activations(32, s[1], seed=950 + i, outliers=True) for i, s in enumerate(specs)]
    xs = [spear.act_to_device(xb, "f16", DEV) for xb in xbs]
    Ms = [1, 2, 3, 4, 5, 7, 8, 11, 13, 16, 17, 20, 24, 29, 31, 32]
    calls = [(i % 2, Ms[(7 * i) % len(Ms)]) for i in range(50)]
    outs = [torch.empty((M, specs[li][0]), dtype=torch.float16, device=DEV) for li, M in calls]
    paths = {spear.spear_linear_plan(layers[li], M, nws)["path"] for li, M in calls}
    assert paths == {"decode", "decode_split"}
    stream = torch.cuda.Stream()

    def run():
        for (li, M), y in zip(calls, outs):
            spear.spear_linear_decode(layers[li], xs[li][:M], y=y, workspace=ws,
                                      stream=torch.cuda.current_stream())

    note("soak eager")
    with torch.cuda.stream(stream):
        run()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    full = [oracle_y(hl, xb) for hl, xb in zip(hls, xbs)]
    for (li, M), r in zip(calls, refs):
        assert_close(gpu_y_f64(r, "f16"), full[li][:M], f"eager layer {li} M={M}")
    note("soak capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    torch.cuda.synchronize()
    note("soak replays (100 x 50 calls)")
    _replay_and_check(g, outs, refs, 100, lambda: None, stream)
    assert spear.spear_workspace_flags(ws) == 0
    assert _header_zero(ws)


def test_library_graph_of_layer_calls():
    """The library's own static graph (spear_graph_*): a prefill call whose compensator runs
    on the graph's aux branch, a decode call, a second prefill call sharing the decode call's
    workspace, and a 1031-token call that the dispatch splits (prefill for 1024 tokens, decode
    for the last 7), captured once and launched 100 times; every launch equals the eager calls
    (the same schedule: prefill with an aux stream) bit for bit."""
    specs = [(1024, 4096, 128, 32, 512), (2048, 1024, 0, 16, 4), (2048, 1024, 0, 16, 200)]
    hl1 = synth.make_layer(1024, 4096, 128, 32, seed=31, b_gate=0.1)
    hl2 = synth.make_layer(2048, 1024, 0, 16, seed=32, b_gate=-0.2)
    l1, l2 = spear.layer_to_device(hl1, DEV), spear.layer_to_device(hl2, DEV)
    ws1, ws2 = spear.new_workspace(l1, 1031), spear.new_workspace(l2, 200)
    xb1 = synth.make_activations(1031, 4096, seed=33, outliers=True)
    xb2 = synth.make_activations(200, 1024, seed=34, outliers=True)
    x1, x2 = spear.act_to_device(xb1, "f16", DEV), spear.act_to_device(xb2, "f16", DEV)
    assert spear.spear_linear_plan(l1, 1031, ws1.numel())["path"] == "prefill_decode_tail"
    calls = [(l1, x1[:512], ws1), (l2, x2[:4], ws2), (l2, x2, ws2), (l1, x1, ws1)]
    outs = [torch.empty((x.shape[0], lay.N), dtype=torch.float16, device=DEV) for lay, x, _ in calls]
    stream, aux = torch.cuda.Stream(), torch.cuda.Stream()
    note("library graph eager")
    with torch.cuda.stream(stream):
        for (lay, x, ws), y in zip(calls, outs):
            spear.spear_linear(lay, x, y=y, workspace=ws, main_stream=stream, aux_stream=aux)
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    for (hl, xb, M), r in zip([(hl1, xb1, 512), (hl2, xb2, 4), (hl2, xb2, 200), (hl1, xb1, 1031)],
                              refs):
        rows = sample_rows(hl.N, 64, seed=M)
        toks = np.unique(np.r_[np.random.default_rng(M).choice(M, min(M, 24), replace=False), M - 1])
        assert_close(gpu_y_f64(r, "f16")[np.ix_(toks, rows)], oracle_y(hl, xb[:M][toks], rows=rows),
                     f"eager M={M}")
    note("library graph build")
    g = spear.SpearGraph()
    for (lay, x, ws), y in zip(calls, outs):
        g.add(lay, x, y=y, workspace=ws)
    g.end()
    with pytest.raises(spear.SpearError):
        g.add(l2, x2[:4], y=outs[1], workspace=ws2)     # ended: nothing more can be added
    note("library graph launches")

    class _Replay:
        def replay(self):
            g.launch(torch.cuda.current_stream())
    _replay_and_check(_Replay(), outs, refs, 100,
                      lambda: _eager_noise(l2, x2[:3], ws2), stream)
    assert spear.spear_workspace_flags(ws2) == 0 and _header_zero(ws2)
    assert spear.spear_workspace_flags(ws1) == 0 and _header_zero(ws1)
    g.destroy()

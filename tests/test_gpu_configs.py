"""GPU parity at the serving stack's shapes: the Llama-7B projections with fp16
activations, g128 4-bit weights and a rank-32 compensator, at every prefill chunk the
chunk selector chooses from (256, 512, 1024, 2048 tokens) and at each chunk plus the 32
decode tokens of a merged mixed batch, through the phase-aware entry point in both
prefill schedules.  Sampled output rows and tokens against the float64 oracle.
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
W = synth.WORKLOADS["llama7b-stack-serving"]
MAX_M = max(W["chunks"]) + W["decode_tokens"]


@pytest.mark.parametrize("K,N", synth.LLAMA7B_SHAPES)
def test_serving_shapes_fp16_prefill(K, N):
    hl = synth.make_layer(N, K, W["group_size"], W["rank"], seed=W["seed"] + K + N, dtype="f16",
                          b_gate=0.1)
    lay = spear.layer_to_device(hl, DEV)
    xb = synth.make_activations(MAX_M, K, seed=W["seed"] + K, dtype="f16", outliers=True)
    x = spear.act_to_device(xb, "f16", DEV)
    ws = spear.new_workspace(lay, MAX_M)   # one workspace for every call, as the stack uses
    rows = sample_rows(N, 96, seed=K + N)
    aux = torch.cuda.Stream()
    for C in W["chunks"]:
        for M in (C, C + W["decode_tokens"]):
            # the last tokens too: past 1024 the dispatch gives the last 32 to the decode path
            toks = np.unique(np.r_[np.random.default_rng(M).choice(M, 40, replace=False), 0,
                                   M - 1 - np.arange(0, 32, 5)])
            path = spear.spear_linear_plan(lay, M, ws.numel())["path"]
            assert path == ("prefill_decode_tail" if M == C + W["decode_tokens"] and C >= 1024
                            else "prefill"), (M, path)
            ref = oracle_y(hl, xb[toks], rows=rows)
            for schedule in ("serial", "concurrent"):
                note(f"serving fp16 prefill K={K} N={N} M={M} {schedule}")
                y = spear.spear_linear(lay, x[:M], workspace=ws,
                                       aux_stream=aux if schedule == "concurrent" else None)
                torch.cuda.synchronize()
                assert_close(gpu_y_f64(y, "f16")[np.ix_(toks, rows)], ref,
                             f"{K}->{N} M={M} {schedule}")
    assert spear.spear_workspace_flags(ws) == 0

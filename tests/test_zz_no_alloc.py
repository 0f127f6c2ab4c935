"""The no-allocation decode entry point (spear_linear_decode_noalloc) against the
workspace entry point (spear_linear_decode), through the C ABI.

Two calls in a row on one GPU, the second with fewer tokens than the first, for each
case: the outputs must equal the workspace entry point's bit for bit (the same launch
runs on the same inputs) and match the float64 oracle within the elementwise tolerance.
The scratch array keeps the last call's contents, so the second call also checks that
the first left its counters at zero.
"""

import pytest

from quantized_gemm_error_amd import spear, synth

from gpu_helpers import assert_close, gpu_y_f64, note, oracle_y, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"

CASES = [
    # N, K, G, r, (M first, M second), dtype
    (4096, 11008, 128, 32, (32, 4), "f16"),   # Llama-7B down projection: split-K launch, then unsplit
    (4096, 4096, 128, 32, (16, 1), "f16"),    # 4096x4096: 8-wave, then 4-wave launch
    (8192, 28672, 28672, 64, (8, 2), "f16"),  # Llama-70B 28672->8192, per-channel, rank 64: split-K twice
    (640, 2048, 0, 24, (17, 5), "bf16"),      # bf16, two token blocks, then one
]


@pytest.mark.parametrize("N,K,G,r,Ms,dtype", CASES)
def test_noalloc_matches_workspace_entry_point(N, K, G, r, Ms, dtype):
    hl = synth.make_layer(N, K, G, r, seed=N + K, dtype=dtype, b_gate=0.2)
    lay = spear.layer_to_device(hl, DEV)
    rows = sample_rows(N, 128, seed=K)
    for M in Ms:
        note(f"noalloc N={N} K={K} r={r} M={M} {dtype} "
             f"{spear.spear_linear_plan(lay, M, spear.SPEAR_NOALLOC_SCRATCH_BYTES)['path']}")
        xb = synth.make_activations(M, K, seed=N + M, dtype=dtype, outliers=True)
        x = spear.act_to_device(xb, dtype, DEV)
        y_na = spear.spear_linear_decode_noalloc(lay, x)
        ws = spear.new_workspace(lay, M)
        y_ws = spear.spear_linear_decode(lay, x, workspace=ws)
        torch.cuda.synchronize()
        assert spear.spear_linear_plan(lay, M, spear.SPEAR_NOALLOC_SCRATCH_BYTES)["path"] == \
            spear.spear_linear_plan(lay, M, ws.numel())["path"]
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), f"M={M}"
        assert_close(gpu_y_f64(y_na, dtype)[:, rows], oracle_y(hl, xb, rows=rows), f"noalloc M={M}")


def test_noalloc_rejects_bad_arguments():
    hl = synth.make_layer(256, 512, 128, 8, seed=3)
    lay = spear.layer_to_device(hl, DEV)
    x = spear.act_to_device(synth.make_activations(129, 512, seed=3), "f16", DEV)
    with pytest.raises(spear.SpearError):
        spear.spear_linear_decode_noalloc(lay, x)          # 129 tokens: beyond decode
    y = spear.spear_linear_decode_noalloc(lay, x[:0])     # M = 0: a no-op
    assert y.shape == (0, 256)

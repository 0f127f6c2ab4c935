"""Seeded input generators: determinism, shapes and the workload recipes."""

import hashlib

import numpy as np

from quantized_gemm_error_amd import synth


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_layer_is_deterministic_per_seed():
    a = synth.make_layer(64, 256, 128, 8, seed=9)
    b = synth.make_layer(64, 256, 128, 8, seed=9)
    c = synth.make_layer(64, 256, 128, 8, seed=10)
    da = _digest(a.q, a.scales, a.zeros, a.A, a.B, a.w_gate)
    assert da == _digest(b.q, b.scales, b.zeros, b.A, b.B, b.w_gate)
    assert da != _digest(c.q, c.scales, c.zeros, c.A, c.B, c.w_gate)


def test_layer_shapes_and_ranges():
    lay = synth.make_layer(48, 512, 0, 16, seed=1)   # 0 = per-channel
    assert lay.group_size == 512
    assert lay.q.shape == (48, 512) and lay.q.dtype == np.uint8 and lay.q.max() <= 15
    assert lay.scales.shape == (48, 1) and lay.zeros.shape == (48, 1)
    assert lay.A.shape == (16, 512) and lay.B.shape == (48, 16) and lay.w_gate.shape == (512,)
    z = lay.zeros.view(np.float16).astype(np.float64)
    assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= 15
    s = lay.scales.view(np.float16).astype(np.float64)
    assert np.all(s > 0)


def test_activation_outliers():
    K = 4096
    idx = synth.outlier_channels(K, seed=2)
    assert len(idx) == 41 and len(set(idx.tolist())) == 41
    assert [len(synth.outlier_channels(k, 2)) for k in (8192, 11008, 28672)] == [82, 110, 287]
    x = synth.make_activations(64, K, seed=2, outliers=True).view(np.float16).astype(np.float64)
    mask = np.zeros(K, bool)
    mask[idx] = True
    assert 12 < np.std(x[:, mask]) < 28 and 0.8 < np.std(x[:, ~mask]) < 1.2


def test_bf16_activations_are_bf16():
    x = synth.make_activations(4, 64, seed=3, dtype="bf16")
    assert x.dtype == np.uint16
    assert not np.array_equal(x, synth.make_activations(4, 64, seed=3, dtype="f16"))


def test_workload_catalogue():
    w = synth.WORKLOADS
    assert w["llama7b-decode"]["tokens"] == (1, 4, 16, 32)
    assert w["llama7b-prefill"]["tokens"] == (2048,) and w["llama7b-prefill"]["dtype"] == "bf16"
    assert w["llama70b-layer"]["rank"] == 64
    idx = synth.ec_block_indices(32, 4, seed=5)
    assert len(idx) == 4 and len(set(idx.tolist())) == 4 and idx.max() < 32

"""Shared helpers of the GPU parity tests (not a test module)."""

from __future__ import annotations

import sys

import numpy as np

import oracle
from quantized_gemm_error_amd import spear, synth

TOL_REL = 1e-2  # |y - y_ref| <= 1e-2 * (1 + |y_ref|), elementwise


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_host_bits(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(__import__("torch").int16).numpy().view(np.uint16)


def gpu_y_f64(y, dtype: str) -> np.ndarray:
    return oracle.act_bits_to_f64(to_host_bits(y), dtype)


def assert_close(y_gpu64: np.ndarray, y_ref: np.ndarray, what: str = "") -> None:
    assert y_gpu64.shape == y_ref.shape, (y_gpu64.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu64)), f"{what}: non-finite output"
    err = np.abs(y_gpu64 - y_ref)
    bound = TOL_REL * (1.0 + np.abs(y_ref))
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert worst <= 1.0, f"{what}: max err/bound = {worst:.3f} (max abs err {float(err.max()):.3e})"


def oracle_y(hl: synth.SynthLayer, x_bits: np.ndarray, rows=None, with_ec=True) -> np.ndarray:
    """Oracle output [M][N] (or [M][len(rows)] for the selected output rows)."""
    sel = slice(None) if rows is None else np.asarray(rows)
    words = oracle.pack_int4(hl.q[sel])
    if with_ec and hl.rank > 0:
        return oracle.spear_linear_ref(x_bits, words, hl.scales[sel], hl.zeros[sel], hl.group_size,
                                       hl.dtype, hl.A, hl.B[sel], hl.w_gate, hl.b_gate)
    return oracle.spear_linear_ref(x_bits, words, hl.scales[sel], hl.zeros[sel], hl.group_size,
                                   hl.dtype)


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """n random rows plus the first and the last 16 (covers the ragged tail tile)."""
    rng = np.random.default_rng(seed)
    pick = rng.choice(N, size=min(n, N), replace=False)
    edge = np.r_[np.arange(min(16, N)), np.arange(max(0, N - 16), N)]
    return np.unique(np.r_[pick, edge])


def run(path: str, lay: spear.SpearLayer, x, ws=None, aux=None):
    if path == "decode":
        return spear.spear_linear_decode(lay, x, workspace=ws)
    if path == "prefill":
        return spear.spear_linear_prefill(lay, x, workspace=ws, aux_stream=aux)
    return spear.spear_linear(lay, x, workspace=ws, aux_stream=aux)

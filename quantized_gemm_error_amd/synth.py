"""Seeded synthetic inputs for the compensated 4-bit linear layer.

This module only draws numbers: Gaussian weights and activations, outlier
channels, element-format rounding and the round-to-nearest (RTN) 4-bit
quantizer that stands in for the quantization backend the layer sits on.  It
holds none of the compensated layer's own arithmetic (no dequantization, no
product, no gate, no packing), so the tests, the benchmark and the GPU path
can all draw the same inputs from it without sharing that arithmetic.

Shapes and distributions follow the workloads of the explanation pages of
"SPEAR: A System for Post-Quantization Error-Adaptive Recovery Enabling
Efficient Low-Bit LLM Serving" (gist.science, paper 2606.11244): Llama-shaped
projections at 7B and 70B scale (3.1 "Quality Recovery" names Llama-2-7B and
models from 1B to 70B; 3.2 "Serving Efficiency" uses 13B and 70B) with RTN
per-channel or group-wise 4-bit weights.  Real checkpoints are not used:
weights are N(0, 0.02), compensator factors N(0, 0.01), gate weights
N(0, 0.05), activations N(0, 1) with 1% of input channels scaled by 20 where
a workload asks for outliers.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# Element formats (rounding float32 draws to the storage formats)
# ---------------------------------------------------------------------------


def to_f16_bits(x) -> np.ndarray:
    """Round float32/64 values to binary16 (round-half-even) -> uint16 bits."""
    return np.asarray(x).astype(np.float16).view(np.uint16)


def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round-half-even) -> uint16 bits.

    Inputs here are finite draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def to_act_bits(x, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return to_f16_bits(x)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(f"unknown activation dtype {dtype!r}")


# ---------------------------------------------------------------------------
# RTN quantizer: the input producer (the pages name RTN, GPTQ, AWQ and
# OmniQuant as the 4-bit backends the compensators sit on)
# ---------------------------------------------------------------------------


def rtn_quantize(w, group_size: int, row_block: int = 1024):
    """Asymmetric round-to-nearest 4-bit quantization of w [N][K] (float32).

    Per row and group of ``group_size`` columns: s = fp16((max - min) / 15)
    (s = 1 for a constant group), z = clip(rint(-min / s), 0, 15) and
    q = clip(rint(w / s) + z, 0, 15), computed with the fp16-rounded s.
    Returns (q uint8 [N][K], scales fp16 bits [N][K/G], zeros fp16 bits).
    """
    w = np.asarray(w, dtype=np.float32)
    n_rows, k = w.shape
    if k % group_size != 0:
        raise ValueError("group_size must divide K")
    n_groups = k // group_size
    q = np.empty((n_rows, k), dtype=np.uint8)
    s_bits = np.empty((n_rows, n_groups), dtype=np.uint16)
    z_bits = np.empty((n_rows, n_groups), dtype=np.uint16)
    for r0 in range(0, n_rows, row_block):
        wb = w[r0:r0 + row_block].reshape(-1, n_groups, group_size)
        lo = wb.min(axis=2)
        hi = wb.max(axis=2)
        s = ((hi - lo) / np.float32(15.0)).astype(np.float16)
        s = np.where(s == 0, np.float16(1.0), s)
        s32 = s.astype(np.float32)
        z = np.clip(np.rint(-lo / s32), 0, 15).astype(np.float32)
        qb = np.clip(np.rint(wb / s32[:, :, None]) + z[:, :, None], 0, 15)
        q[r0:r0 + row_block] = qb.reshape(-1, k).astype(np.uint8)
        s_bits[r0:r0 + row_block] = s.view(np.uint16)
        z_bits[r0:r0 + row_block] = z.astype(np.float16).view(np.uint16)
    return q, s_bits, z_bits


# ---------------------------------------------------------------------------
# Layers and activations
# ---------------------------------------------------------------------------


@dataclass
class SynthLayer:
    """Host copy of one synthetic layer (all numpy, unpacked 4-bit codes)."""

    N: int
    K: int
    group_size: int
    rank: int
    dtype: str                 # activation dtype of A, B, w_gate: 'f16' or 'bf16'
    q: np.ndarray              # uint8 [N][K], codes 0..15
    scales: np.ndarray         # uint16 fp16 bits [N][K/G]
    zeros: np.ndarray          # uint16 fp16 bits [N][K/G]
    A: np.ndarray | None       # uint16 bits [r][K]
    B: np.ndarray | None       # uint16 bits [N][r]
    w_gate: np.ndarray | None  # uint16 bits [K]
    b_gate: float = 0.0
    w_fp32: np.ndarray | None = field(default=None, repr=False)  # pre-quantization draw


def make_layer(N: int, K: int, group_size: int, rank: int, seed: int, dtype: str = "f16",
               w_std: float = 0.02, ec_std: float = 0.01, wg_std: float = 0.05,
               b_gate: float = 0.0, keep_fp32: bool = False) -> SynthLayer:
    """Draw W ~ N(0, w_std), RTN-quantize it; draw A, B ~ N(0, ec_std), w_g ~ N(0, wg_std)."""
    G = K if group_size in (0, -1, None) else int(group_size)
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)
    q, s_bits, z_bits = rtn_quantize(w, G)
    A = B = wg = None
    if rank > 0:
        A = to_act_bits(rng.standard_normal((rank, K), dtype=np.float32) * np.float32(ec_std), dtype)
        B = to_act_bits(rng.standard_normal((N, rank), dtype=np.float32) * np.float32(ec_std), dtype)
        wg = to_act_bits(rng.standard_normal(K, dtype=np.float32) * np.float32(wg_std), dtype)
    return SynthLayer(N=N, K=K, group_size=G, rank=rank, dtype=dtype, q=q, scales=s_bits,
                      zeros=z_bits, A=A, B=B, w_gate=wg, b_gate=float(b_gate),
                      w_fp32=w if keep_fp32 else None)


def make_rank_gate(rank: int, hidden: int, seed: int, t_scale: float = 1.0):
    """The per-rank gate's MLP parameters, float32: W1 [hidden][rank] ~ N(0, 1/(rank t_scale^2)),
    b1 ~ N(0, 0.1), W2 [rank][hidden] ~ N(0, 1/hidden), b2 ~ N(0, 0.5).  t_scale is the
    typical size of a component of t = A x, so that the gate is not saturated."""
    rng = np.random.default_rng(seed + 31337)
    W1 = (rng.standard_normal((hidden, rank), dtype=np.float32) / np.float32(np.sqrt(rank) * t_scale))
    b1 = rng.standard_normal(hidden, dtype=np.float32) * np.float32(0.1)
    W2 = rng.standard_normal((rank, hidden), dtype=np.float32) / np.float32(np.sqrt(hidden))
    b2 = rng.standard_normal(rank, dtype=np.float32) * np.float32(0.5)
    return dict(W1=W1, b1=b1, W2=W2, b2=b2)


def outlier_channels(K: int, seed: int, frac: float = 0.01) -> np.ndarray:
    """round(frac*K) distinct input-channel indices, fixed by the seed."""
    n_out = int(round(frac * K))
    rng = np.random.default_rng(seed + 7919)
    return np.sort(rng.choice(K, n_out, replace=False))


def make_activations(M: int, K: int, seed: int, dtype: str = "f16", outliers: bool = False,
                     outlier_scale: float = 20.0, outlier_frac: float = 0.01) -> np.ndarray:
    """x ~ N(0, 1) [M][K] in the activation dtype (uint16 bits).

    With ``outliers`` the same round(1% K) input channels (fixed by the seed)
    are multiplied by ``outlier_scale`` for every token.
    """
    rng = np.random.default_rng(seed + 104729)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        x[:, outlier_channels(K, seed, outlier_frac)] *= np.float32(outlier_scale)
    return to_act_bits(x, dtype)


# ---------------------------------------------------------------------------
# Workloads (sizes from the pages' model scales; see module docstring)
# ---------------------------------------------------------------------------

LLAMA7B_SHAPES = ((4096, 4096), (4096, 11008), (11008, 4096))      # (K, N)
LLAMA70B_SHAPES = ((8192, 8192), (8192, 28672), (28672, 8192))     # (K, N)

WORKLOADS = {
    "small-512": dict(shapes=((512, 512),), group_size=0, rank=16, tokens=(1, 64),
                      dtype="f16", outliers=False, seed=1),
    "llama7b-decode": dict(shapes=LLAMA7B_SHAPES, group_size=128, rank=32, tokens=(1, 4, 16, 32),
                           dtype="f16", outliers=True, seed=2),
    "llama7b-prefill": dict(shapes=LLAMA7B_SHAPES, group_size=128, rank=32, tokens=(2048,),
                            dtype="bf16", outliers=True, seed=3),
    "llama70b-layer": dict(shapes=LLAMA70B_SHAPES, group_size=0, rank=64, tokens=(1, 64, 256),
                           dtype="f16", outliers=False, seed=4),
    "llama7b-stack-serving": dict(shapes=LLAMA7B_SHAPES, group_size=128, rank=32, blocks=32,
                                  ec_blocks=4, chunks=(256, 512, 1024, 2048), decode_tokens=32,
                                  budget_ms=50.0, dtype="f16", outliers=False, seed=5),
}


def ec_block_indices(blocks: int, ec_blocks: int, seed: int) -> np.ndarray:
    """Which blocks of a stack carry compensators, fixed by the seed."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(blocks, ec_blocks, replace=False))

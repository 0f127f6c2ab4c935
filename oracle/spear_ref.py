"""Float64 CPU restatement of the compensated 4-bit linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.

Source: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
Enabling Efficient Low-Bit LLM Serving", explanation pages on gist.science
(paper 2606.11244), English page, Technical Summary:

* 2.1 A "Input-Adaptive Error Compensators": an error compensator maps the
  input x to a low-rank space with A, scales it by an input-dependent gate and
  maps it back with B; the effective weight is W + alpha B diag(gamma(Ax)) A.
* 2.2 A "Phase-Aware Adaptive Kernel Fusion Dispatch": decode (M = 1) and
  prefill (M > 1) are two schedules of the same product.
* 2.2 C "SLO-Constrained EC-Aware Chunk Scheduling": the scheduler picks the
  largest prefill chunk whose latency, read from precomputed kernel-latency
  tables, meets the inter-token latency target.
* 1 "Problem Statement" and 3.1 "Quality Recovery": the weights are 4-bit
  (RTN per-channel among the quantizers named); the compensator repairs the
  quantization error, so W is the dequantized 4-bit weight.

Readings where the pages are silent (each is listed in the design notes):

* The weight is stored as unsigned 4-bit codes q in [0, 15] with an fp16 scale
  s and an fp16 zero-point z per output row and per group of G consecutive
  input columns; the dequantized weight is (q - z) * s.  G == K means one
  scale per output channel.
* Eight codes are packed per 32-bit word along K, lowest nibble first: code
  k = 8j + i of row n sits in bits 4i..4i+3 of word j of that row.
* The scalar gate g(x) = sigmoid(w_g . x + b_g) stands for the pages' gate,
  with alpha folded into B (alpha = 1).  ``rank_gate_linear_ref`` also gives
  the pages' own per-rank form, gamma(Ax) as a small bottleneck MLP.
* Intermediates are exact (float64); the GPU rounds only its output.

Everything is NumPy float64, written for reading, not for speed.
"""

from __future__ import annotations

import math

import numpy as np

ORACLE_IS_TEST_INFRASTRUCTURE = True

# ---------------------------------------------------------------------------
# Element formats
# ---------------------------------------------------------------------------


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) to float64, exactly."""
    u = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return u.view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64, exactly.

    A bfloat16 value is the upper half of a binary32 value, so widening the
    pattern by 16 zero bits gives the same number as a float32.
    """
    u = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32)
    return (u << np.uint32(16)).view(np.float32).astype(np.float64)


def act_bits_to_f64(bits, dtype: str) -> np.ndarray:
    """Activation-dtype bit patterns to float64; dtype is 'f16' or 'bf16'."""
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    raise ValueError(f"unknown activation dtype {dtype!r}")


# ---------------------------------------------------------------------------
# 4-bit packing (pages: 4-bit weights, Problem Statement; layout is a reading)
# ---------------------------------------------------------------------------


def unpack_int4(qweight) -> np.ndarray:
    """Packed words [N][K/8] (int32) -> codes [N][K] (uint8 in 0..15).

    Code k = 8j + i of a row is bits 4i..4i+3 of word j of that row.
    """
    words = np.ascontiguousarray(np.asarray(qweight, dtype=np.int32)).view(np.uint32)
    n_rows, n_words = words.shape
    q = np.empty((n_rows, 8 * n_words), dtype=np.uint8)
    for i in range(8):
        q[:, i::8] = (words >> np.uint32(4 * i)) & np.uint32(0xF)
    return q


def pack_int4(q) -> np.ndarray:
    """Codes [N][K] -> packed words [N][K/8] (int32); codes are masked to 4 bits.

    The inverse of ``unpack_int4`` on codes in 0..15.
    """
    q = np.asarray(q)
    n_rows, k = q.shape
    if k % 8 != 0:
        raise ValueError("K must be a multiple of 8 to pack 8 codes per word")
    codes = q.astype(np.uint32) & np.uint32(0xF)
    words = np.zeros((n_rows, k // 8), dtype=np.uint32)
    for i in range(8):
        words |= codes[:, i::8] << np.uint32(4 * i)
    return words.view(np.int32)


def tile_words(qweight) -> np.ndarray:
    """Row-major packed words [N][K/8] -> the GPU library's tiled order.

    A layout, not arithmetic: the pages fix 4-bit codes packed eight to a
    32-bit word and leave the order of the words in memory open.  The rows
    are padded with zero words to a multiple of 16 and taken in blocks of 16
    rows; inside a block, piece P (words 4P .. 4P + 3, codes 32P .. 32P + 31)
    of rows 0..15 comes first, then piece P + 1 of rows 0..15, and so on.
    The result is returned as int32 [ceil(N/16) 16][K/8], whose row index no
    longer names an output row.
    """
    words = np.ascontiguousarray(np.asarray(qweight, dtype=np.int32))
    n_rows, n_words = words.shape
    if n_words % 4 != 0:
        raise ValueError("K must be a multiple of 32 for the tiled order")
    n_pad = -(-n_rows // 16) * 16
    padded = np.zeros((n_pad, n_words), dtype=np.int32)
    padded[:n_rows] = words
    pieces = padded.reshape(n_pad // 16, 16, n_words // 4, 4)     # [block][row][piece][word]
    return np.ascontiguousarray(pieces.transpose(0, 2, 1, 3)).reshape(n_pad, n_words)


def untile_words(tiled, n_rows: int) -> np.ndarray:
    """The inverse of ``tile_words``: the first n_rows row-major rows."""
    t = np.ascontiguousarray(np.asarray(tiled, dtype=np.int32))
    n_pad, n_words = t.shape
    pieces = t.reshape(n_pad // 16, n_words // 4, 16, 4)          # [block][piece][row][word]
    return np.ascontiguousarray(pieces.transpose(0, 2, 1, 3)).reshape(n_pad, n_words)[:n_rows]


# ---------------------------------------------------------------------------
# Dequantization: W = dequant(W_q) (pages: the compensator repairs the error
# of the 4-bit weight; Problem Statement and 2.1 A)
# ---------------------------------------------------------------------------


def dequant(qweight, scales, zeros, group_size: int, rows=None) -> np.ndarray:
    """Dequantized weight W~[n, k] = (q[n, k] - z[n, k // G]) * s[n, k // G].

    ``scales`` and ``zeros`` are fp16 bit patterns [N][K/G]; the zero-point is
    an unscaled code value.  ``rows`` optionally selects output rows.
    """
    q = unpack_int4(qweight if rows is None else np.asarray(qweight)[rows])
    s = f16_bits_to_f64(scales if rows is None else np.asarray(scales)[rows])
    z = f16_bits_to_f64(zeros if rows is None else np.asarray(zeros)[rows])
    n_rows, k = q.shape
    if group_size <= 0 or k % group_size != 0:
        raise ValueError("group_size must divide K")
    n_groups = k // group_size
    if s.shape != (n_rows, n_groups) or z.shape != (n_rows, n_groups):
        raise ValueError("scales/zeros must be [N][K/G]")
    group_of_column = np.arange(k) // group_size
    return (q.astype(np.float64) - z[:, group_of_column]) * s[:, group_of_column]


# ---------------------------------------------------------------------------
# Gate (pages: a light input-dependent gate, 2.1 A; scalar form is a reading)
# ---------------------------------------------------------------------------


def sigmoid(z) -> np.ndarray:
    """Logistic function in float64, exact at +-inf (1 and 0) and at 0 (1/2).

    Uses 1/(1+e^-z) for z >= 0 and e^z/(1+e^z) for z < 0 so that no
    exponential overflows.
    """
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def gate(x64: np.ndarray, w_g64: np.ndarray, b_g: float) -> np.ndarray:
    """Per-token gate g[m] = sigmoid(w_g . x[m] + b_g), float64 [M]."""
    return sigmoid(x64 @ w_g64 + np.float64(b_g))


# ---------------------------------------------------------------------------
# The compensated linear layer
# ---------------------------------------------------------------------------


def spear_linear_ref(x, qweight, scales, zeros, group_size: int, dtype: str = "f16",
                     A=None, B=None, w_gate=None, b_gate: float = 0.0,
                     rows=None, row_chunk: int = 2048) -> np.ndarray:
    """y[m, n] = sum_k x[m,k] W~[n,k] + g[m] * sum_j B[n,j] (sum_k A[j,k] x[m,k]).

    The effective weight W~ + B diag(g) A of 2.1 A with the scalar gate
    g = sigmoid(w_g . x + b_g) and alpha = 1, computed directly in float64.

    x       activation bit patterns [M][K] (uint16, fp16 or bf16 per ``dtype``)
    qweight packed codes [N][K/8] (int32); scales, zeros fp16 bits [N][K/G]
    A, B    compensator bit patterns [r][K] and [N][r] in the activation dtype,
            or None for rank 0 (then the result is the plain 4-bit product)
    w_gate  gate weights [K] in the activation dtype; b_gate a Python float
    rows    optional output-row indices (returns [M][len(rows)])
    Returns float64 [M][N] (unrounded).
    """
    x64 = act_bits_to_f64(x, dtype)
    n_total = np.asarray(qweight).shape[0]
    row_ids = np.arange(n_total) if rows is None else np.asarray(rows)
    y = np.empty((x64.shape[0], row_ids.shape[0]), dtype=np.float64)
    for c0 in range(0, row_ids.shape[0], row_chunk):
        sel = row_ids[c0:c0 + row_chunk]
        w = dequant(qweight, scales, zeros, group_size, rows=sel)
        y[:, c0:c0 + sel.shape[0]] = x64 @ w.T
    rank = 0 if A is None else np.asarray(A).shape[0]
    if rank == 0:
        return y
    a64 = act_bits_to_f64(A, dtype)
    b64 = act_bits_to_f64(np.asarray(B)[row_ids], dtype)
    g = gate(x64, act_bits_to_f64(w_gate, dtype), b_gate)
    t = x64 @ a64.T                      # [M][r]   low-rank projection A x
    return y + g[:, None] * (t @ b64.T)  # [M][N]   + g * B (A x)


def rank_gate_linear_ref(x, qweight, scales, zeros, group_size: int, dtype: str,
                         A, B, W1, b1, W2, b2, alpha: float = 1.0) -> np.ndarray:
    """The pages' per-rank gate: y = W~ x + alpha * B diag(gamma(A x)) A x.

    gamma is read as a bottleneck MLP r -> h -> r with a ReLU hidden layer and
    a sigmoid output: gamma(t) = sigmoid(W2 relu(W1 t + b1) + b2), so each of
    the r rank components gets its own gate in (0, 1).  W1 [h][r], b1 [h],
    W2 [r][h], b2 [r] are float64 arrays; the other operands are as in
    ``spear_linear_ref``.  Returns float64 [M][N].
    """
    x64 = act_bits_to_f64(x, dtype)
    y = x64 @ dequant(qweight, scales, zeros, group_size).T
    t = x64 @ act_bits_to_f64(A, dtype).T                       # [M][r]
    hidden = np.maximum(t @ np.asarray(W1, np.float64).T + np.asarray(b1, np.float64), 0.0)
    gam = sigmoid(hidden @ np.asarray(W2, np.float64).T + np.asarray(b2, np.float64))
    return y + np.float64(alpha) * ((gam * t) @ act_bits_to_f64(B, dtype).T)


# ---------------------------------------------------------------------------
# Chunk selection (pages: 2.2 C, largest prefill chunk meeting the ITL target)
# ---------------------------------------------------------------------------


def select_chunk_ref(chunks, pred_ms, budget_ms: float):
    """Largest chunk whose predicted step latency fits the budget.

    ``chunks`` are candidate prefill chunk sizes and ``pred_ms`` the latency
    predicted for a step with that chunk (from measured kernel-latency
    tables).  Comparisons are in float32, the precision the library uses.
    Returns (chunk, violated): when no candidate fits, the smallest chunk and
    violated = True (a reading: the pages do not say what happens then).
    """
    chunks = [int(c) for c in chunks]
    if not chunks:
        raise ValueError("no candidate chunks")
    budget = np.float32(budget_ms)
    best = None
    for c, p in zip(chunks, pred_ms):
        if np.float32(p) <= budget and (best is None or c > best):
            best = c
    if best is None:
        return min(chunks), True
    return best, False


def _self_check() -> None:
    """Tiny sanity check used by the smoke entry point (not a pin)."""
    assert sigmoid(np.array([0.0]))[0] == 0.5
    assert math.isclose(float(sigmoid(np.array([2.0]))[0]), 1.0 / (1.0 + math.exp(-2.0)))

"""Pins of the float64 CPU oracle against things other than itself.

Each test checks the oracle against a fact fixed by the pages or by the
mathematics: a pure-Python brute force written independently (struct-decoded
fp16/bf16, bit-by-bit nibble extraction, tanh-form logistic), integer closed
forms, the gate's special values, rank-1 and full-rank closed forms, a
hand-derived worked example, and brute force for the chunk selector.
"""

import json
import math
import os
import struct

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from quantized_gemm_error_amd import synth

# ---------------------------------------------------------------------------
# Independent pure-Python brute force (no NumPy arithmetic)
# ---------------------------------------------------------------------------


def _half(bits):
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _act(bits, dtype):
    return _half(bits) if dtype == "f16" else _bf16(bits)


def _logistic(z):
    # tanh form: a different closed form from the oracle's exp form
    return 0.5 * (1.0 + math.tanh(z / 2.0)) if not math.isinf(z) else (1.0 if z > 0 else 0.0)


def brute_force(x, words, scales, zeros, G, dtype, A=None, B=None, wg=None, b_g=0.0):
    M, K = len(x), len(x[0])
    N = len(words)
    xv = [[_act(x[m][k], dtype) for k in range(K)] for m in range(M)]
    W = []
    for n in range(N):
        row = []
        for k in range(K):
            word = int(words[n][k // 8]) & 0xFFFFFFFF
            code = (word >> (4 * (k % 8))) & 0xF
            row.append((code - _half(zeros[n][k // G])) * _half(scales[n][k // G]))
        W.append(row)
    y = [[math.fsum(xv[m][k] * W[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    if A is None:
        return y
    r = len(A)
    Av = [[_act(A[j][k], dtype) for k in range(K)] for j in range(r)]
    Bv = [[_act(B[n][j], dtype) for j in range(r)] for n in range(N)]
    wv = [_act(wg[k], dtype) for k in range(K)]
    for m in range(M):
        zlog = math.fsum(wv[k] * xv[m][k] for k in range(K)) + b_g
        g = _logistic(zlog)
        t = [math.fsum(Av[j][k] * xv[m][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            y[m][n] += g * math.fsum(Bv[n][j] * t[j] for j in range(r))
    return y


def _random_case(rng, M, N, K, G, r, dtype):
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = synth.to_f16_bits(rng.uniform(0.001, 0.05, size=(N, K // G)))
    z = synth.to_f16_bits(rng.integers(0, 16, size=(N, K // G)).astype(np.float32))
    x = synth.to_act_bits(rng.standard_normal((M, K)).astype(np.float32), dtype)
    A = B = wg = None
    if r > 0:
        A = synth.to_act_bits(rng.standard_normal((r, K)).astype(np.float32) * 0.3, dtype)
        B = synth.to_act_bits(rng.standard_normal((N, r)).astype(np.float32) * 0.3, dtype)
        wg = synth.to_act_bits(rng.standard_normal(K).astype(np.float32) * 0.2, dtype)
    return q, s, z, x, A, B, wg


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------


def test_pack_hand_words():
    q = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [8, 9, 10, 11, 12, 13, 14, 15]], dtype=np.uint8)
    words = oracle.pack_int4(q)
    assert words.dtype == np.int32
    assert int(words[0, 0]) & 0xFFFFFFFF == 0x76543210
    assert int(words[1, 0]) & 0xFFFFFFFF == 0xFEDCBA98
    assert int(words[1, 0]) < 0  # the top nibble sets the sign bit of the int32


def test_pack_every_position_and_value():
    for i in range(8):
        for v in range(16):
            q = np.zeros((1, 8), dtype=np.uint8)
            q[0, i] = v
            assert int(oracle.pack_int4(q)[0, 0]) & 0xFFFFFFFF == v << (4 * i)
            back = oracle.unpack_int4(oracle.pack_int4(q))
            assert back.tolist() == q.tolist()


def test_pack_masks_high_bits():
    q = np.array([[0x1F, 0xF0, 0x3, 0, 0, 0, 0, 0xAB]], dtype=np.uint8)
    assert int(oracle.pack_int4(q)[0, 0]) & 0xFFFFFFFF == 0xB000030F


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 9), kw=st.integers(1, 6), seed=st.integers(0, 2**31 - 1))
def test_pack_unpack_roundtrip(n, kw, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(n, 8 * kw), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(q)), q)
    words = rng.integers(-2**31, 2**31, size=(n, kw), dtype=np.int64).astype(np.int32)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(words)), words)
    # bit-by-bit definition
    u = oracle.unpack_int4(words)
    for r in range(n):
        for j in range(kw):
            word = int(words[r, j]) & 0xFFFFFFFF
            for i in range(8):
                assert u[r, 8 * j + i] == (word >> (4 * i)) & 0xF


def _tiled_byte_address(n, k, K):
    # the tiled order as a wave-load address: 16-row block, 128-code tile of
    # 1 KB, 16-byte lane piece (quarter h of the tile, row n % 16), word, byte
    return ((n // 16) * 8 * K + (k // 128) * 1024 + (((k % 128) // 32) * 16 + n % 16) * 16
            + ((k % 32) // 8) * 4 + (k % 8) // 2)


@pytest.mark.parametrize("N,K", [(1, 32), (16, 128), (37, 160), (50, 416)])
def test_tile_words_byte_addresses(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    tiled = oracle.tile_words(oracle.pack_int4(q))
    n_pad = -(-N // 16) * 16
    assert tiled.shape == (n_pad, K // 8) and tiled.dtype == np.int32
    flat = tiled.view(np.uint8).ravel()
    assert flat.size == (n_pad // 16) * 8 * K
    seen = np.zeros(flat.size, dtype=bool)
    for n in range(N):
        for k in range(K):
            a = _tiled_byte_address(n, k, K)
            assert (int(flat[a]) >> (4 * (k % 2))) & 0xF == q[n, k], (n, k)
            seen[a] = True
    assert not flat[~seen].any()          # every other byte is row padding, zero
    assert np.array_equal(oracle.untile_words(tiled, N), oracle.pack_int4(q))


def test_tile_words_hand_cases():
    w = np.arange(1, 1 + 2 * 8, dtype=np.int32).reshape(2, 8)   # N = 2, K = 64: two pieces
    t = oracle.tile_words(w).ravel()
    assert t.size == 16 * 8
    assert t[:8].tolist() == [1, 2, 3, 4, 9, 10, 11, 12]         # piece 0 of rows 0, 1
    assert not t[8:64].any()                                      # piece 0 of padding rows
    assert t[64:72].tolist() == [5, 6, 7, 8, 13, 14, 15, 16]     # piece 1 of rows 0, 1
    assert not t[72:].any()
    w16 = np.arange(16 * 4, dtype=np.int32).reshape(16, 4)       # K = 32: one piece per row
    assert np.array_equal(oracle.tile_words(w16), w16)


@settings(max_examples=40, deadline=None)
@given(n=st.integers(1, 40), pieces=st.integers(1, 9), seed=st.integers(0, 2**31 - 1))
def test_tile_untile_roundtrip(n, pieces, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(-2**31, 2**31, size=(n, 4 * pieces), dtype=np.int64).astype(np.int32)
    t = oracle.tile_words(w)
    assert np.array_equal(oracle.untile_words(t, n), w)
    assert sorted(t.ravel().tolist()) == sorted(w.ravel().tolist() + [0] * (t.size - w.size))


def test_tile_words_rejects_partial_piece():
    with pytest.raises(ValueError):
        oracle.tile_words(np.zeros((2, 6), dtype=np.int32))


def test_pack_rejects_ragged_k():
    with pytest.raises(ValueError):
        oracle.pack_int4(np.zeros((2, 12), dtype=np.uint8))


# ---------------------------------------------------------------------------
# Element formats
# ---------------------------------------------------------------------------


def test_format_known_values():
    f16 = np.array([0x3C00, 0xC000, 0x3800, 0x7BFF, 0x0001, 0x8000], dtype=np.uint16)
    assert oracle.f16_bits_to_f64(f16).tolist() == [1.0, -2.0, 0.5, 65504.0, 2.0 ** -24, -0.0]
    bf = np.array([0x3F80, 0xC000, 0x3F00, 0x4080, 0x0001], dtype=np.uint16)
    assert oracle.bf16_bits_to_f64(bf).tolist() == [1.0, -2.0, 0.5, 4.0, 2.0 ** -133]


def test_bf16_rounding_of_generator():
    # 1 + 2^-8 is a tie between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1)
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -3.0], dtype=np.float32)
    bits = synth.to_bf16_bits(vals)
    assert oracle.bf16_bits_to_f64(bits).tolist() == [1.0, 1.0 + 2.0 ** -6, -3.0]


# ---------------------------------------------------------------------------
# Gate
# ---------------------------------------------------------------------------


def test_sigmoid_special_values():
    z = np.array([0.0, np.inf, -np.inf, 800.0, -800.0])
    s = oracle.sigmoid(z)
    assert s[0] == 0.5 and s[1] == 1.0 and s[2] == 0.0
    assert s[3] == 1.0 and s[4] == 0.0
    zz = np.linspace(-30, 30, 241)
    ref = np.array([_logistic(float(v)) for v in zz])
    assert np.max(np.abs(oracle.sigmoid(zz) - ref)) < 1e-15
    assert np.max(np.abs(oracle.sigmoid(-zz) - (1.0 - oracle.sigmoid(zz)))) < 1e-15


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K,G,r", [(1, 8, 16, 8, 0), (3, 5, 32, 8, 2), (2, 7, 24, 24, 4),
                                       (1, 32, 32, 32, 3), (3, 16, 32, 8, 1)])
def test_oracle_matches_brute_force(dtype, M, N, K, G, r):
    rng = np.random.default_rng(1000 * M + 100 * N + K + G + r)
    q, s, z, x, A, B, wg = _random_case(rng, M, N, K, G, r, dtype)
    b_g = float(rng.standard_normal())
    words = oracle.pack_int4(q)
    ref = oracle.spear_linear_ref(x, words, s, z, G, dtype, A, B, wg, b_g)
    bf = brute_force(x.tolist(), words.tolist(), s.tolist(), z.tolist(), G, dtype,
                     None if A is None else A.tolist(), None if B is None else B.tolist(),
                     None if wg is None else wg.tolist(), b_g)
    np.testing.assert_allclose(ref, np.array(bf), rtol=1e-12, atol=1e-12)


def test_integer_closed_form():
    """s = 1, integer zero-points and integer x: y is an exact integer product."""
    rng = np.random.default_rng(7)
    N, K, G, M = 12, 64, 16, 3
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zi = rng.integers(0, 16, size=(N, K // G))
    xi = rng.integers(-8, 9, size=(M, K))
    s = synth.to_f16_bits(np.ones((N, K // G), dtype=np.float32))
    z = synth.to_f16_bits(zi.astype(np.float32))
    x = synth.to_f16_bits(xi.astype(np.float32))
    w_int = q.astype(np.int64) - np.repeat(zi, G, axis=1)
    expect = xi.astype(np.int64) @ w_int.T
    got = oracle.spear_linear_ref(x, oracle.pack_int4(q), s, z, G)
    assert np.array_equal(got, expect.astype(np.float64))


def test_scale_is_per_group():
    """q - z = 1 everywhere and s = 2^g in group g: y = sum_g 2^g sum_{k in g} x_k."""
    N, K, G = 3, 32, 8
    q = np.full((N, K), 5, dtype=np.uint8)
    z = synth.to_f16_bits(np.full((N, K // G), 4.0, dtype=np.float32))
    s = synth.to_f16_bits(np.tile(2.0 ** np.arange(K // G), (N, 1)).astype(np.float32))
    xv = np.arange(K, dtype=np.float32) - 10
    y = oracle.spear_linear_ref(synth.to_f16_bits(xv[None, :]), oracle.pack_int4(q), s, z, G)
    expect = sum(2.0 ** g * xv[g * G:(g + 1) * G].sum() for g in range(K // G))
    assert y.shape == (1, N) and np.all(y == expect)


def _layer_case(seed, M=4, N=24, K=64, G=16, r=4, dtype="f16"):
    rng = np.random.default_rng(seed)
    q, s, z, x, A, B, wg = _random_case(rng, M, N, K, G, r, dtype)
    return oracle.pack_int4(q), s, z, x, A, B, wg, G


def test_gate_off_is_rank_zero_exactly():
    words, s, z, x, A, B, _, G = _layer_case(11)
    wg0 = np.zeros(A.shape[1], dtype=np.uint16)
    y_off = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B, wg0, -np.inf)
    y_r0 = oracle.spear_linear_ref(x, words, s, z, G, "f16")
    assert np.array_equal(y_off, y_r0)


def test_gate_on_and_half_closed_forms():
    words, s, z, x, A, B, _, G = _layer_case(12)
    wg0 = np.zeros(A.shape[1], dtype=np.uint16)
    x64, a64, b64 = (oracle.f16_bits_to_f64(v) for v in (x, A, B))
    y0 = oracle.spear_linear_ref(x, words, s, z, G, "f16")
    full = x64 @ (b64 @ a64).T          # B A x with the other association
    y1 = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B, wg0, np.inf)
    yh = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B, wg0, 0.0)
    np.testing.assert_allclose(y1 - y0, full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(yh - y0, 0.5 * full, rtol=1e-12, atol=1e-13)


def test_rank_one_closed_form():
    """A = e_j: the compensator adds g(x) * x_j * b for B = b (one column)."""
    words, s, z, x, _, _, _, G = _layer_case(13, r=0)
    K, j = 64, 17
    A = np.zeros((1, K), dtype=np.uint16)
    A[0, j] = 0x3C00  # 1.0
    rng = np.random.default_rng(5)
    bvals = rng.standard_normal(24).astype(np.float32)
    B = synth.to_f16_bits(bvals[:, None])
    wvals = rng.standard_normal(K).astype(np.float32) * 0.1
    wg = synth.to_f16_bits(wvals)
    b_g = 0.3
    y0 = oracle.spear_linear_ref(x, words, s, z, G, "f16")
    y = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B, wg, b_g)
    xs = [[_half(v) for v in row] for row in x.tolist()]
    wl = [_half(v) for v in wg.tolist()]
    bl = [_half(v) for v in B[:, 0].tolist()]
    for m in range(x.shape[0]):
        g = _logistic(math.fsum(a * b for a, b in zip(wl, xs[m])) + b_g)
        for n in range(24):
            assert math.isclose(y[m, n] - y0[m, n], g * xs[m][j] * bl[n], rel_tol=1e-9, abs_tol=1e-12)


def test_full_rank_absorption_recovers_fp16_product():
    """g = 1, A = I, B = fp16(W - W~): y equals the fp16-weight product up to B's rounding."""
    N = K = 64
    layer = synth.make_layer(N, K, 16, 0, seed=21, keep_fp32=True)
    W16 = layer.w_fp32.astype(np.float16).astype(np.float64)       # fp16 weight
    words = oracle.pack_int4(layer.q)
    Wq = oracle.dequant(words, layer.scales, layer.zeros, 16)
    D = W16 - Wq
    B = synth.to_f16_bits(D)
    A = synth.to_f16_bits(np.eye(K, dtype=np.float32))
    wg = np.zeros(K, dtype=np.uint16)
    x = synth.make_activations(3, K, seed=22)
    y = oracle.spear_linear_ref(x, words, layer.scales, layer.zeros, 16, "f16", A, B, wg, np.inf)
    x64 = oracle.f16_bits_to_f64(x)
    target = x64 @ W16.T
    bound = np.abs(x64) @ (np.abs(D) * 2.0 ** -11 + 2.0 ** -25).T + 1e-12
    assert np.all(np.abs(y - target) <= bound)
    # and the compensator really mattered
    assert np.max(np.abs(x64 @ Wq.T - target)) > 10 * np.max(bound)


def test_token_permutation():
    words, s, z, x, A, B, wg, G = _layer_case(14, M=6)
    perm = np.array([3, 0, 5, 1, 4, 2])
    y = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B, wg, 0.1)
    yp = oracle.spear_linear_ref(x[perm], words, s, z, G, "f16", A, B, wg, 0.1)
    np.testing.assert_allclose(yp, y[perm], rtol=1e-13, atol=1e-13)


def test_rows_subset_matches_full():
    words, s, z, x, A, B, wg, G = _layer_case(15)
    rows = np.array([0, 5, 23, 7])
    y = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B, wg, -0.2)
    ys = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B, wg, -0.2, rows=rows, row_chunk=3)
    np.testing.assert_allclose(ys, y[:, rows], rtol=1e-13, atol=1e-13)


def test_rtn_roundtrip_and_error_bound():
    """Requantizing W~ with its own (s, z) returns q; |W - W~| <= s/2 where not clipped."""
    layer = synth.make_layer(16, 256, 128, 0, seed=3, keep_fp32=True)
    words = oracle.pack_int4(layer.q)
    Wq = oracle.dequant(words, layer.scales, layer.zeros, 128)
    s = np.repeat(oracle.f16_bits_to_f64(layer.scales), 128, axis=1)
    z = np.repeat(oracle.f16_bits_to_f64(layer.zeros), 128, axis=1)
    assert np.array_equal(np.clip(np.rint(Wq / s) + z, 0, 15).astype(np.uint8), layer.q)
    interior = (layer.q > 0) & (layer.q < 15)
    err = np.abs(layer.w_fp32.astype(np.float64) - Wq)
    assert np.all(err[interior] <= s[interior] * (0.5 + 1e-3))


def test_hand_example(golden_dir):
    with open(os.path.join(golden_dir, "hand_example.json")) as f:
        ex = json.load(f)
    words = np.array([[int(h, 16)] for h in ex["packed_words_hex"]], dtype=np.uint32).view(np.int32)
    assert np.array_equal(oracle.pack_int4(np.array(ex["codes"], dtype=np.uint8)), words)
    s = np.array([[int(h, 16)] for h in ex["scales_f16_hex"]], dtype=np.uint16)
    z = np.array([[int(h, 16)] for h in ex["zeros_f16_hex"]], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.dequant(words, s, z, 8), np.array(ex["dequantized"]))
    for dtype, key in (("f16", "x_f16_hex"), ("bf16", "x_bf16_hex")):
        x = np.array([[int(h, 16) for h in ex[key]]], dtype=np.uint16)
        enc = synth.to_act_bits
        A = enc(np.array(ex["A"], dtype=np.float32), dtype)
        B = enc(np.array(ex["B"], dtype=np.float32), dtype)
        wg = enc(np.array(ex["w_gate"], dtype=np.float32), dtype)
        for case in ex["cases"]:
            b_g = float(case["b_gate"])
            y = oracle.spear_linear_ref(x, words, s, z, 8, dtype, A, B, wg, b_g)
            assert y[0].tolist() == case["y"], (dtype, case)


# ---------------------------------------------------------------------------
# The pages' per-rank gate (bottleneck MLP reading)
# ---------------------------------------------------------------------------


def test_rank_gate_reduces_to_scalar_gate():
    words, s, z, x, A, B, _, G = _layer_case(16)
    r, h = A.shape[0], 2
    beta = -0.7
    rng = np.random.default_rng(1)
    W1, b1 = rng.standard_normal((h, r)), rng.standard_normal(h)
    y_rank = oracle.rank_gate_linear_ref(x, words, s, z, G, "f16", A, B, W1, b1,
                                         np.zeros((r, h)), np.full(r, beta))
    y_scalar = oracle.spear_linear_ref(x, words, s, z, G, "f16", A, B,
                                       np.zeros(A.shape[1], dtype=np.uint16), beta)
    np.testing.assert_allclose(y_rank, y_scalar, rtol=1e-12, atol=1e-13)


def test_rank_gate_brute_force():
    rng = np.random.default_rng(2)
    M, N, K, G, r, h = 2, 5, 16, 8, 3, 2
    q, s, z, x, A, B, _ = _random_case(rng, M, N, K, G, r, "f16")
    W1, b1 = rng.standard_normal((h, r)), rng.standard_normal(h)
    W2, b2 = rng.standard_normal((r, h)), rng.standard_normal(r)
    alpha = 0.75
    words = oracle.pack_int4(q)
    y = oracle.rank_gate_linear_ref(x, words, s, z, G, "f16", A, B, W1, b1, W2, b2, alpha)
    base = brute_force(x.tolist(), words.tolist(), s.tolist(), z.tolist(), G, "f16")
    xs = [[_half(v) for v in row] for row in x.tolist()]
    for m in range(M):
        t = [math.fsum(_half(A[j, k]) * xs[m][k] for k in range(K)) for j in range(r)]
        hid = [max(0.0, math.fsum(W1[i, j] * t[j] for j in range(r)) + b1[i]) for i in range(h)]
        gam = [_logistic(math.fsum(W2[j, i] * hid[i] for i in range(h)) + b2[j]) for j in range(r)]
        for n in range(N):
            comp = math.fsum(_half(B[n, j]) * gam[j] * t[j] for j in range(r))
            assert math.isclose(y[m, n], base[m][n] + alpha * comp, rel_tol=1e-10, abs_tol=1e-12)


# ---------------------------------------------------------------------------
# Chunk selector
# ---------------------------------------------------------------------------


def test_select_chunk_brute_force_and_monotone():
    rng = np.random.default_rng(3)
    chunks = [256, 512, 1024, 2048]
    for _ in range(200):
        pred = np.sort(rng.uniform(0.5, 20.0, size=4)).astype(np.float32)
        if rng.random() < 0.3:
            pred = rng.uniform(0.5, 20.0, size=4).astype(np.float32)  # not monotone in C
        last = 0
        for budget in np.linspace(0.1, 25.0, 60).astype(np.float32):
            c, violated = oracle.select_chunk_ref(chunks, pred, float(budget))
            fits = [ch for ch, p in zip(chunks, pred) if p <= budget]
            if fits:
                assert (c, violated) == (max(fits), False)
                assert c >= last
                last = c
            else:
                assert (c, violated) == (256, True)


def test_select_chunk_edges():
    assert oracle.select_chunk_ref([256, 512], [1.0, 2.0], 2.0) == (512, False)
    assert oracle.select_chunk_ref([512, 256], [2.0, 1.0], 1.5) == (256, False)
    assert oracle.select_chunk_ref([512, 256], [2.0, 1.0], 0.5) == (256, True)
    with pytest.raises(ValueError):
        oracle.select_chunk_ref([], [], 1.0)

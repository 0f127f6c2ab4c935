"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/spear.h declares, and
reject invalid arguments on the host before anything is launched (these
calls make no HIP call).  Host-only logic (the chunk selector) is checked
against the oracle.
"""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from quantized_gemm_error_amd import spear

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "spear.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spear_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(spear.LIB_PATH):
        pytest.fail("libspear.so is not built: run python -m quantized_gemm_error_amd.build")
    return spear.load_library()


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert set(declared) == set(spear.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert spear.spear_status_string(0) == "ok"
    for st in (1, 2, 3, 4):
        assert spear.spear_status_string(st) not in ("ok", "unknown status")
    assert spear.spear_status_string(99) == "unknown status"
    assert spear.spear_version() >= 100


def test_select_chunk_matches_oracle(lib):
    rng = np.random.default_rng(0)
    chunks = [256, 512, 1024, 2048]
    for _ in range(300):
        pred = rng.uniform(0.5, 20.0, size=4).astype(np.float32)
        budget = float(np.float32(rng.uniform(0.1, 25.0)))
        assert spear.spear_select_chunk(chunks, pred.tolist(), budget) == \
            oracle.select_chunk_ref(chunks, pred, budget)
    assert spear.spear_select_chunk([7], [1.0], 1.0) == (7, False)
    assert spear.spear_select_chunk([7, 3], [math.inf, math.inf], 1e30) == (3, True)


def test_select_chunk_invalid(lib):
    with pytest.raises(spear.SpearError):
        spear.spear_select_chunk([], [], 1.0)
    with pytest.raises(spear.SpearError):
        spear.spear_select_chunk([0, 256], [1.0, 1.0], 5.0)


def test_decode_max_m_setting(lib):
    assert spear.spear_get_decode_max_m() == 32
    spear.spear_set_decode_max_m(16)
    assert spear.spear_get_decode_max_m() == 16
    spear.spear_set_decode_max_m(32)
    with pytest.raises(spear.SpearError):
        spear.spear_set_decode_max_m(0)
    with pytest.raises(spear.SpearError):
        spear.spear_set_decode_max_m(33)
    assert spear.spear_get_decode_max_m() == 32


def test_decode_split_min_m_setting(lib):
    assert spear.spear_get_decode_split_min_m() == 16
    assert spear.spear_get_decode_split_min_k() == 8192
    spear.spear_set_decode_split_min_k(1)
    assert spear.spear_get_decode_split_min_k() == 1
    spear.spear_set_decode_split_min_k(8192)
    with pytest.raises(spear.SpearError):
        spear.spear_set_decode_split_min_k(0)
    spear.spear_set_decode_split_min_m(33)  # never split
    assert spear.spear_get_decode_split_min_m() == 33
    spear.spear_set_decode_split_min_m(1)
    assert spear.spear_get_decode_split_min_m() == 1
    spear.spear_set_decode_split_min_m(16)
    with pytest.raises(spear.SpearError):
        spear.spear_set_decode_split_min_m(0)
    with pytest.raises(spear.SpearError):
        spear.spear_set_decode_split_min_m(34)
    assert spear.spear_get_decode_split_min_m() == 16


FAKE = 0x10000  # 64 KiB-aligned fake device address: validation never dereferences it


def _layer(**kw):
    c = spear.SpearLayerC(N=64, K=256, group_size=128, qweight=FAKE, scales=FAKE, zeros=FAKE,
                          rank=8, A=FAKE, B=FAKE, w_gate=FAKE, b_gate=0.0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _decode(lib, layer, dtype=0, x=FAKE * 2, y=FAKE * 3, M=1, ws=FAKE * 4, ws_bytes=1 << 20):
    return lib.spear_linear_decode(ctypes.byref(layer) if layer is not None else None, dtype, x, y,
                                   M, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(K=250), 1), (dict(K=136), 2), (dict(group_size=100), 1), (dict(group_size=64), 2),
    (dict(N=0), 1), (dict(qweight=None), 1), (dict(qweight=FAKE + 4), 1), (dict(rank=-1), 1),
    (dict(rank=129), 2), (dict(A=None), 1), (dict(w_gate=FAKE + 2), 1), (dict(b_gate=math.nan), 1),
])
def test_decode_rejects_bad_layer(lib, bad, code):
    assert _decode(lib, _layer(**bad)) == code
    assert lib.spear_last_error().decode() != ""


def _rank_gate(**kw):
    g = spear.SpearRankGateC(hidden=16, W1=FAKE, b1=FAKE, W2=FAKE, b2=FAKE, alpha=1.0)
    for k, v in kw.items():
        setattr(g, k, v)
    return g


@pytest.mark.parametrize("bad,code", [
    (dict(hidden=0), 1), (dict(hidden=65), 2), (dict(W1=None), 1), (dict(b2=None), 1),
    (dict(W2=FAKE + 2), 1), (dict(alpha=math.nan), 1), (dict(alpha=math.inf), 1),
])
def test_decode_rejects_bad_rank_gate(lib, bad, code):
    g = _rank_gate(**bad)
    lay = _layer(w_gate=None, b_gate=math.nan)   # ignored with a per-rank gate
    lay.rank_gate = ctypes.pointer(g)
    assert _decode(lib, lay) == code
    assert lib.spear_last_error().decode() != ""


def test_rank_gate_replaces_the_scalar_gate(lib):
    # with a per-rank gate, w_gate and b_gate are not needed; validation passes (M = 0: no-op)
    g = _rank_gate()
    lay = _layer(w_gate=None, b_gate=math.nan)
    lay.rank_gate = ctypes.pointer(g)
    assert _decode(lib, lay, M=0) == 0
    assert lib.spear_workspace_bytes(ctypes.byref(lay), 32) > 0
    # without one, a missing w_gate is an error
    assert _decode(lib, _layer(w_gate=None)) == 1


def test_rejects_bad_io_and_workspace(lib):
    lay = _layer()
    assert _decode(lib, None) == 1
    assert _decode(lib, lay, dtype=2) == 1
    assert _decode(lib, lay, x=None) == 1
    assert _decode(lib, lay, x=FAKE * 2 + 8) == 1          # x not 16-byte aligned
    assert _decode(lib, lay, y=FAKE * 2) == 1              # y aliases x
    assert _decode(lib, lay, M=33) == 1
    assert _decode(lib, lay, M=-1) == 1
    assert _decode(lib, lay, ws=None) == 3
    assert _decode(lib, lay, ws_bytes=16) == 3
    assert _decode(lib, lay, ws=FAKE * 4 + 16) == 3        # not 256-byte aligned
    assert _decode(lib, lay, M=0) == 0                     # no-op, nothing launched
    pre = lib.spear_linear_prefill
    assert pre(ctypes.byref(lay), 0, FAKE * 2, FAKE * 3, -5, FAKE * 4, 1 << 20, None, None) == 1
    assert pre(ctypes.byref(lay), 0, FAKE * 2, FAKE * 3, 0, FAKE * 4, 1 << 20, None, None) == 0
    assert pre(ctypes.byref(lay), 0, FAKE * 2, FAKE * 3, 2048, FAKE * 4, 64, None, None) == 3
    assert lib.spear_pack_int4(FAKE, FAKE, 4, 12, None) == 1
    assert lib.spear_pack_int4(None, FAKE, 4, 16, None) == 1
    assert lib.spear_pack_int4(FAKE, FAKE, 0, 16, None) == 0


def test_rank_zero_needs_no_compensator_pointers(lib):
    lay = _layer(rank=0, A=None, B=None, w_gate=None)
    assert lib.spear_workspace_bytes(ctypes.byref(lay), 1) >= 256
    # decode with r = 0 needs no workspace; validate only (M = 0 is a no-op)
    assert _decode(lib, lay, ws=None, ws_bytes=0, M=0) == 0


def test_workspace_bytes(lib):
    lay = _layer()
    small = lib.spear_workspace_bytes(ctypes.byref(lay), 1)
    big = lib.spear_workspace_bytes(ctypes.byref(lay), 2048)
    assert small >= 256 and big >= 2048 * 8 * 4
    assert lib.spear_workspace_bytes(ctypes.byref(_layer(K=250)), 1) == 0
    assert lib.spear_workspace_bytes(ctypes.byref(lay), -1) == 0

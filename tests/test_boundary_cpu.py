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
    assert spear.spear_get_decode_max_m() == 64
    spear.spear_set_decode_max_m(16)
    assert spear.spear_get_decode_max_m() == 16
    spear.spear_set_decode_max_m(128)
    assert spear.spear_get_decode_max_m() == 128
    spear.spear_set_decode_max_m(64)
    with pytest.raises(spear.SpearError):
        spear.spear_set_decode_max_m(0)
    with pytest.raises(spear.SpearError):
        spear.spear_set_decode_max_m(129)
    assert spear.spear_get_decode_max_m() == 64


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
    assert _decode(lib, lay, M=129) == 1
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
    assert lib.spear_pack_int4(FAKE, FAKE, 4, 16, None) == 1     # K % 32 != 0: no tiled order
    assert lib.spear_pack_int4(None, FAKE, 4, 32, None) == 1
    assert lib.spear_pack_int4(FAKE, FAKE + 4, 4, 32, None) == 1  # qweight not 16-byte aligned
    assert lib.spear_pack_int4(FAKE, FAKE, 0, 32, None) == 0
    assert lib.spear_tile_int4(FAKE, FAKE * 2, 4, 16, None) == 1
    assert lib.spear_tile_int4(None, FAKE, 4, 32, None) == 1
    assert lib.spear_tile_int4(FAKE + 4, FAKE * 2, 4, 32, None) == 1
    assert lib.spear_tile_int4(FAKE, FAKE + 32, 4, 32, None) == 1  # overlapping buffers
    assert lib.spear_tile_int4(FAKE, FAKE * 2, 0, 32, None) == 0


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


def _plan(layer, M, ws_bytes, phase="dispatch"):
    return spear.spear_linear_plan(layer, M, ws_bytes, phase)


@pytest.mark.parametrize("K", [4096, 8192, 16384, 28672])
@pytest.mark.parametrize("min_m", [1, 2, 4, 8, 9, 16, 33])
def test_decode_split_truth_table(lib, K, min_m):
    """Which token counts may take the split-K decode launch: M >= min_m at K >= min_k,
    and M >= max(2, ceil(min_m / 8)) at K >= 2 min_k; never with min_m = 33 and never
    without room for the partial tiles.  (A wanted split still needs its plan to fit,
    every workgroup resident at once; the cases that fit are checked below.)"""
    lay = _layer(N=8192, K=K, group_size=K, rank=64)
    old = spear.spear_get_decode_split_min_m(), spear.spear_get_decode_split_min_k()
    spear.spear_set_decode_split_min_m(min_m)
    spear.spear_set_decode_split_min_k(8192)
    try:
        big = lib.spear_workspace_bytes(ctypes.byref(lay), 32)
        for M in range(1, 33):
            want = min_m <= 32 and K >= 8192 and (
                M >= min_m or (K >= 16384 and M >= max(2, -(-min_m // 8))))
            p = _plan(lay, M, big)
            if not want:
                assert p["path"] == "decode", (M, p)
            if p["path"] == "decode_split":
                assert p["k_splits"] >= 2
                # with only the unsplit launch's workspace, the same call does not split
                assert _plan(lay, M, p["workspace_bytes"])["path"] == "decode"
    finally:
        spear.spear_set_decode_split_min_m(old[0])
        spear.spear_set_decode_split_min_k(old[1])


@pytest.mark.parametrize("K,N,G,r,M", [(28672, 8192, 28672, 64, m) for m in range(2, 9)] +
                         [(11008, 4096, 128, 32, 16), (11008, 4096, 128, 32, 32),
                          (20480, 384, 20480, 24, 2)])
def test_decode_split_taken_with_default_thresholds(lib, K, N, G, r, M):
    """The Llama-70B 28672->8192 layer (per-channel, rank 64) and the Llama-7B 11008->4096
    layer (g128, rank 32) take the split-K launch where it was measured to win."""
    assert spear.spear_get_decode_split_min_m() == 16
    assert spear.spear_get_decode_split_min_k() == 8192
    lay = _layer(N=N, K=K, group_size=G, rank=r)
    ws = lib.spear_workspace_bytes(ctypes.byref(lay), 32)
    assert _plan(lay, M, ws)["path"] == "decode_split"
    assert _plan(lay, 1, ws)["path"] == "decode"        # one token never splits by default


def test_plan_dispatch_and_errors(lib):
    lay = _layer(N=4096, K=4096, group_size=128, rank=32)
    ws = lib.spear_workspace_bytes(ctypes.byref(lay), 2048)
    assert _plan(lay, 0, ws)["path"] == "none"
    assert _plan(lay, 1, ws)["path"] == "decode"
    assert _plan(lay, 32, ws)["path"] == "decode"
    assert _plan(lay, 33, ws)["path"] == "decode_wide"
    assert _plan(lay, 64, ws)["path"] == "decode_wide"
    assert _plan(lay, 65, ws)["path"] == "prefill"
    assert _plan(lay, 2048, ws)["path"] == "prefill"
    assert _plan(lay, 2048, ws)["k_splits"] == 1
    assert _plan(lay, 64, ws, "prefill")["k_splits"] > 1   # 32 output tiles: K split
    assert _plan(lay, 16, ws, "prefill")["path"] == "prefill"
    assert _plan(lay, 33, ws, "decode")["path"] == "decode_wide"
    assert _plan(lay, 128, ws, "decode")["path"] == "decode_wide"
    with pytest.raises(spear.SpearError):
        _plan(lay, 129, ws, "decode")
    with pytest.raises(spear.SpearError):               # compensated: workspace required
        _plan(lay, 1, 0)
    with pytest.raises(spear.SpearError):
        _plan(lay, 2048, 1024)
    lay0 = _layer(N=4096, K=4096, group_size=128, rank=0, A=None, B=None, w_gate=None)
    assert _plan(lay0, 100, 0)["k_splits"] == 1        # rank 0 without a workspace: no split
    assert _plan(lay0, 100, 0)["workspace_bytes"] == 0


def test_prefill_plan_counts_the_split_gemm_producers(lib):
    """A K-split prefill GEMM with the scalar gate and K <= 16384 carries the compensator's
    producers in its launch (32-token blocks x at most 8 K-splits, padded to a multiple of 8
    workgroups ahead of the tiles); with K past 16384, the per-rank gate, an unsplit GEMM or
    rank 0 it has none."""
    def plan(M=100, **kw):
        lay = _layer(**kw)
        return _plan(lay, M, lib.spear_workspace_bytes(ctypes.byref(lay), M), "prefill")
    p = plan(N=512, K=2048, group_size=128, rank=32)
    assert p["k_splits"] > 1 and p["producers"] == 4 * 8            # 4 token blocks x 8 splits
    p0 = plan(N=512, K=2048, group_size=128, rank=0, A=None, B=None, w_gate=None)
    assert p0["producers"] == 0 and p["workgroups"] == p0["workgroups"] + 32
    assert plan(N=256, K=16640, group_size=128, rank=16)["producers"] == 0
    big = plan(M=2048, N=8192, K=4096, group_size=128, rank=32)
    assert big["k_splits"] == 1 and big["producers"] == 0


def test_dispatch_splits_off_a_short_decode_tail(lib):
    """spear_linear gives the last r = M mod 128 tokens to the decode path when 1 <= r <= 32,
    at least eight full 128-token tile rows precede them, r is within the decode threshold
    and the workspace holds the decode call's needs; the plan then describes the prefill
    launch for the first M - r tokens."""
    lay = _layer(N=4096, K=4096, group_size=128, rank=32)
    ws = lib.spear_workspace_bytes(ctypes.byref(lay), 2080)
    for M, tail in ((1056, 32), (1025, 1), (2080, 32), (2048 + 17, 17), (1024, 0), (1064, 0),
                    (288, 0), (544, 0), (1023, 0), (900, 0)):
        plan = _plan(lay, M, ws)
        assert plan["path"] == ("prefill_decode_tail" if tail else "prefill"), (M, plan)
        assert plan == dict(_plan(lay, M - tail, ws, "prefill"), path=plan["path"]), M
        assert _plan(lay, M, ws, "prefill")["path"] == "prefill"   # explicit prefill: never split
    old = spear.spear_get_decode_max_m()
    try:
        spear.spear_set_decode_max_m(16)                    # the tail must be a decode-sized M
        assert _plan(lay, 1056, ws)["path"] == "prefill"
        assert _plan(lay, 1040, ws)["path"] == "prefill_decode_tail"
    finally:
        spear.spear_set_decode_max_m(old)
    lay0 = _layer(N=4096, K=4096, group_size=128, rank=0, A=None, B=None, w_gate=None)
    assert _plan(lay0, 1056, 0)["path"] == "prefill_decode_tail"   # rank 0: no workspace needed


def test_workspace_holds_only_the_partials_a_call_can_split_into(lib):
    """Decode-sized workspaces carry no 32 MiB of GEMM partials: at M <= 32 the prefill
    split partials are at most ks * 32 * N * 4 bytes."""
    lay = _layer(N=4096, K=4096, group_size=128, rank=32)
    small = lib.spear_workspace_bytes(ctypes.byref(lay), 32)
    assert small <= 16 * 32 * 4096 * 4 + (2 << 20), small
    assert small < lib.spear_workspace_bytes(ctypes.byref(lay), 2048)
    for M in (1, 16, 32, 33, 64, 200, 640, 2048):
        need = lib.spear_workspace_bytes(ctypes.byref(lay), M)
        plan = _plan(lay, M, need)
        assert plan["workspace_bytes"] <= need


def test_decode_spin_limit_setting(lib):
    assert spear.spear_get_decode_spin_limit() == 1 << 20
    spear.spear_set_decode_spin_limit(0)
    assert spear.spear_get_decode_spin_limit() == 0
    spear.spear_set_decode_spin_limit(1 << 20)
    assert spear.spear_get_decode_spin_limit() == 1 << 20


def test_graph_calls_reject_null_handles(lib):
    assert lib.spear_graph_begin(None) == 1
    assert lib.spear_graph_add(None, ctypes.byref(_layer()), 0, FAKE * 2, FAKE * 3, 1, FAKE * 4,
                               1 << 20) == 1
    assert lib.spear_graph_end(None) == 1
    assert lib.spear_graph_launch(None, None) == 1
    assert lib.spear_graph_destroy(None) == 0


def test_decode_routes_long_k_to_wide_past_16_tokens(lib):
    """17..32 tokens take the wide launch where the column threshold wants the split-K launch,
    no split fits and the layer has at most 64 row tiles of 128; everywhere else below 33
    tokens the row-group kernels (split or not) serve the call."""
    def path(M, **kw):
        lay = _layer(**kw)
        return _plan(lay, M, lib.spear_workspace_bytes(ctypes.byref(lay), M), "decode")["path"]
    for r in (32, 0):
        for M in (17, 24, 32):
            assert path(M, N=4096, K=28672, group_size=128, rank=r) == "decode_wide"
            assert path(M, N=520, K=28672, group_size=128, rank=r) == "decode_wide"
            assert path(M, N=4096, K=11008, group_size=128, rank=r) == "decode_split"  # fits
            assert path(M, N=4096, K=4096, group_size=128, rank=r) == "decode"   # no split wanted
        assert path(32, N=4096, K=16384, group_size=128, rank=r) == "decode_wide"
        assert path(17, N=4096, K=16384, group_size=128, rank=r) == "decode_split"  # fits
        assert path(32, N=16384, K=16384, group_size=128, rank=r) == "decode"  # 128 tiles
        assert path(1, N=4096, K=28672, group_size=128, rank=r) == "decode"
    # long splits with group-wise scales: up to 32 scale groups a split (two staging rounds)
    assert path(16, N=4096, K=16384, group_size=128, rank=32) == "decode_split"
    assert path(4, N=4096, K=28672, group_size=128, rank=32) == "decode_split"
    # the rank-64 compensator's LDS leaves no split at 8192 x 8192 past 16 tokens; rank 0 splits
    assert path(17, N=8192, K=8192, group_size=8192, rank=64) == "decode_split"
    assert path(32, N=8192, K=8192, group_size=8192, rank=64) == "decode_wide"
    assert path(32, N=8192, K=8192, group_size=8192, rank=0) == "decode_split"
    # with the split switched off by its token threshold, nothing is routed
    assert lib.spear_set_decode_split_min_m(33) == 0
    try:
        assert path(32, N=4096, K=28672, group_size=128, rank=32) == "decode"
    finally:
        assert lib.spear_set_decode_split_min_m(16) == 0


@pytest.mark.parametrize("K,N,G,r", [(8192, 8192, 8192, 64), (8192, 28672, 8192, 64),
                                     (28672, 8192, 28672, 64), (4096, 4096, 128, 32),
                                     (11008, 4096, 128, 32), (512, 512, 512, 16), (640, 300, 128, 24)])
def test_wide_decode_plans(lib, K, N, G, r):
    """33..128 tokens plan the wide decode launch: tiles of 128 or 256 rows times K-splits
    (never an empty split) plus the compensator's producers, and a workspace that the call
    accepts; a compensated call needs one."""
    lay = _layer(N=N, K=K, group_size=G, rank=r)
    ws = lib.spear_workspace_bytes(ctypes.byref(lay), 128)
    for M in (33, 48, 64, 65, 100, 128):
        p = _plan(lay, M, ws, "decode")
        assert p["path"] == "decode_wide"
        nb = -(-K // 128)
        assert 1 <= p["k_splits"] <= nb
        nbs = -(-nb // p["k_splits"])
        assert -(-nb // nbs) == p["k_splits"]          # no empty split
        consumers = p["workgroups"] - p["producers"]
        assert consumers % p["k_splits"] == 0
        assert consumers // p["k_splits"] in (-(-N // 128), -(-N // 256))
        assert p["workspace_bytes"] <= ws
        assert _plan(lay, M, p["workspace_bytes"], "decode")["path"] == "decode_wide"
        with pytest.raises(spear.SpearError):       # compensated: the workspace is required
            _plan(lay, M, 0, "decode")

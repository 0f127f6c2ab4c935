"""The Python binding's argument checks, on CPU tensors (no library call, no GPU).

The C ABI receives bare pointers, so the binding must refuse, before it calls into
the library, every tensor whose shape, dtype, stride or device would make a kernel
read or write outside a buffer.  Each case here is rejected before the device check
(or by it), so nothing reaches libspear.
"""

import pytest

from quantized_gemm_error_amd import spear

torch = pytest.importorskip("torch")

N, K, G, R = 64, 256, 128, 8


def _layer(act=torch.float16, **kw):
    lay = spear.SpearLayer(
        N=N, K=K, group_size=G,
        qweight=torch.zeros((N, K // 8), dtype=torch.int32),
        scales=torch.zeros((N, K // G), dtype=torch.float16),
        zeros=torch.zeros((N, K // G), dtype=torch.float16),
        rank=R, A=torch.zeros((R, K), dtype=act), B=torch.zeros((N, R), dtype=act),
        w_gate=torch.zeros((K,), dtype=act), b_gate=0.0)
    for k, v in kw.items():
        setattr(lay, k, v)
    return lay


def _x(M=4, act=torch.float16):
    return torch.zeros((M, K), dtype=act)


CALLS = [spear.spear_linear_decode, spear.spear_linear_prefill, spear.spear_linear]


@pytest.mark.parametrize("fn", CALLS)
def test_valid_cpu_tensors_fail_only_on_the_device(fn):
    with pytest.raises(ValueError, match="GPU"):
        fn(_layer(), _x())


@pytest.mark.parametrize("fn", CALLS)
@pytest.mark.parametrize("x,exc", [
    (torch.zeros((4, K + 8), dtype=torch.float16), ValueError),      # wrong K
    (torch.zeros((K,), dtype=torch.float16), ValueError),            # 1-D
    (torch.zeros((2, 4, K), dtype=torch.float16), ValueError),       # 3-D
    (torch.zeros((K, 4), dtype=torch.float16).t(), ValueError),      # transposed view
    (torch.zeros((4, 2 * K), dtype=torch.float16)[:, ::2], ValueError),  # strided view
    (torch.zeros((4, K), dtype=torch.float32), TypeError),           # not fp16/bf16
])
def test_bad_activations(fn, x, exc):
    with pytest.raises(exc):
        fn(_layer(), x)


@pytest.mark.parametrize("fn", CALLS)
@pytest.mark.parametrize("y,exc", [
    (torch.zeros((4, N - 1), dtype=torch.float16), ValueError),      # too small
    (torch.zeros((3, N), dtype=torch.float16), ValueError),          # wrong M
    (torch.zeros((N, 4), dtype=torch.float16).t(), ValueError),      # not contiguous
    (torch.zeros((4, N), dtype=torch.bfloat16), TypeError),          # dtype differs from x
])
def test_bad_outputs(fn, y, exc):
    with pytest.raises(exc):
        fn(_layer(), _x(), y=y)


@pytest.mark.parametrize("fn", CALLS)
@pytest.mark.parametrize("field,value,exc", [
    ("A", torch.zeros((R, K), dtype=torch.bfloat16), TypeError),     # bf16 A with fp16 x
    ("B", torch.zeros((N, R), dtype=torch.bfloat16), TypeError),
    ("w_gate", torch.zeros((K,), dtype=torch.bfloat16), TypeError),
    ("A", torch.zeros((R, K - 8), dtype=torch.float16), ValueError),
    ("B", torch.zeros((R, N), dtype=torch.float16), ValueError),     # transposed shape
    ("A", torch.zeros((K, R), dtype=torch.float16).t(), ValueError),  # transposed view
    ("w_gate", None, ValueError),                                    # scalar gate without w_g
    ("qweight", torch.zeros((N, K // 8), dtype=torch.int64), TypeError),
    ("qweight", torch.zeros((N - 1, K // 8), dtype=torch.int32), ValueError),
    ("scales", torch.zeros((N, K // G), dtype=torch.float32), TypeError),
    ("zeros", torch.zeros((N, 1), dtype=torch.float16), ValueError),
])
def test_bad_layer_tensors(fn, field, value, exc):
    with pytest.raises(exc):
        fn(_layer(**{field: value}), _x())


def test_rank_zero_ignores_the_compensator_tensors():
    lay = _layer(rank=0, A=None, B=None, w_gate=None)
    with pytest.raises(ValueError, match="GPU"):
        spear.spear_linear_decode(lay, _x())


def test_rank_gate_shapes_checked():
    gate = spear.RankGate(hidden=16, W1=torch.zeros((16, R)), b1=torch.zeros(16),
                          W2=torch.zeros((R, 16)), b2=torch.zeros(R))
    with pytest.raises(ValueError, match="GPU"):   # valid: w_gate may be absent
        spear.spear_linear_decode(_layer(w_gate=None, rank_gate=gate), _x())
    bad = spear.RankGate(hidden=16, W1=torch.zeros((R, 16)), b1=torch.zeros(16),
                         W2=torch.zeros((R, 16)), b2=torch.zeros(R))
    with pytest.raises(ValueError, match="W1"):
        spear.spear_linear_decode(_layer(w_gate=None, rank_gate=bad), _x())
    bad64 = spear.RankGate(hidden=16, W1=torch.zeros((16, R), dtype=torch.float64),
                           b1=torch.zeros(16), W2=torch.zeros((R, 16)), b2=torch.zeros(R))
    with pytest.raises(TypeError):
        spear.spear_linear_decode(_layer(w_gate=None, rank_gate=bad64), _x())


def test_bf16_layer_needs_bf16_activations():
    lay = _layer(act=torch.bfloat16)
    with pytest.raises(TypeError):
        spear.spear_linear_decode(lay, _x(act=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        spear.spear_linear_decode(lay, _x(act=torch.bfloat16))


def test_workspace_must_be_contiguous():
    ws = torch.zeros(4096, dtype=torch.uint8)[::2]
    with pytest.raises(ValueError, match="workspace"):
        spear.spear_linear_decode(_layer(), _x(), workspace=ws)


@pytest.mark.parametrize("q,exc", [
    (torch.zeros((4, 16), dtype=torch.int32), TypeError),
    (torch.zeros((16,), dtype=torch.uint8), TypeError),
    (torch.zeros((16, 4), dtype=torch.uint8).t(), ValueError),
    (torch.zeros((4, 12), dtype=torch.uint8), ValueError),
])
def test_pack_rejects_bad_codes(q, exc):
    with pytest.raises(exc):
        spear.spear_pack_int4(q)


def test_pack_rejects_bad_output_and_cpu():
    q = torch.zeros((4, 32), dtype=torch.uint8)
    with pytest.raises(ValueError):
        spear.spear_pack_int4(q, qweight=torch.zeros((4, 4), dtype=torch.int32))  # unpadded
    with pytest.raises(ValueError, match="multiple of 32"):
        spear.spear_pack_int4(torch.zeros((4, 16), dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        spear.spear_pack_int4(q)


def test_tile_rejects_bad_words():
    with pytest.raises(TypeError):
        spear.spear_tile_int4(torch.zeros((4, 4), dtype=torch.int64))
    with pytest.raises(ValueError, match="multiple of 32"):
        spear.spear_tile_int4(torch.zeros((4, 2), dtype=torch.int32))
    with pytest.raises(ValueError):
        spear.spear_tile_int4(torch.zeros((4, 4), dtype=torch.int32),
                              qweight=torch.zeros((4, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        spear.spear_tile_int4(torch.zeros((4, 4), dtype=torch.int32))


def test_qweight_rows_padded_to_16():
    n = 50   # qweight holds qweight_rows(50) = 64 rows in the tiled order
    assert spear.qweight_rows(n) == 64 and spear.qweight_rows(64) == 64
    rows = dict(scales=torch.zeros((n, K // G), dtype=torch.float16),
                zeros=torch.zeros((n, K // G), dtype=torch.float16),
                B=torch.zeros((n, R), dtype=torch.float16))
    lay = _layer(N=n, qweight=torch.zeros((64, K // 8), dtype=torch.int32), **rows)
    with pytest.raises(ValueError, match="GPU"):      # valid shapes: fails only on the device
        spear.spear_linear_decode(lay, _x())
    lay = _layer(N=n, qweight=torch.zeros((n, K // 8), dtype=torch.int32), **rows)
    with pytest.raises(ValueError, match="qweight"):  # unpadded rows
        spear.spear_linear_decode(lay, _x())

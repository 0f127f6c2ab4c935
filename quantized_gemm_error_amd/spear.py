"""Thin ctypes binding of libspear (include/spear.h), same names as the C ABI.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libspear.so.  PyTorch supplies device memory and streams.  There is no
fallback: if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspear.so")

SPEAR_OK = 0
SPEAR_ERR_INVALID_ARGUMENT = 1
SPEAR_ERR_UNSUPPORTED = 2
SPEAR_ERR_WORKSPACE = 3
SPEAR_ERR_HIP = 4
SPEAR_F16 = 0
SPEAR_BF16 = 1
SPEAR_MAX_RANK = 128
SPEAR_MAX_DECODE_M = 128

# Every function the header declares, for the export check.
EXPORTED = (
    "spear_workspace_bytes", "spear_pack_int4", "spear_tile_int4", "spear_linear_decode", "spear_linear_prefill",
    "spear_linear", "spear_set_decode_max_m", "spear_get_decode_max_m",
    "spear_set_decode_split_min_m", "spear_get_decode_split_min_m",
    "spear_set_decode_split_min_k", "spear_get_decode_split_min_k", "spear_select_chunk",
    "spear_status_string", "spear_last_error", "spear_workspace_flags", "spear_version",
    "spear_linear_plan", "spear_set_decode_spin_limit", "spear_get_decode_spin_limit",
    "spear_linear_decode_noalloc", "spear_graph_begin", "spear_graph_add", "spear_graph_end",
    "spear_graph_launch", "spear_graph_destroy",
)
SPEAR_NOALLOC_SCRATCH_BYTES = 17 << 20

SPEAR_PATH_NONE = 0
SPEAR_PATH_DECODE = 1
SPEAR_PATH_DECODE_SPLIT = 2
SPEAR_PATH_PREFILL = 3
SPEAR_PATH_DECODE_WIDE = 4
PATH_NAMES = {0: "none", 1: "decode", 2: "decode_split", 3: "prefill", 4: "decode_wide",
              5: "prefill_decode_tail"}


class SpearError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"spear status {status}: {message}")
        self.status = status


class SpearRankGateC(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("W2", ctypes.c_void_p),
        ("b2", ctypes.c_void_p), ("alpha", ctypes.c_float),
    ]


class SpearLayerC(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("group_size", ctypes.c_int32),
        ("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
        ("rank", ctypes.c_int32),
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
        ("b_gate", ctypes.c_float),
        ("rank_gate", ctypes.POINTER(SpearRankGateC)),
    ]


class SpearPlanC(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32), ("workgroups", ctypes.c_int32),
        ("waves_per_workgroup", ctypes.c_int32), ("producers", ctypes.c_int32),
        ("k_splits", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspear.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m quantized_gemm_error_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    LP = ctypes.POINTER(SpearLayerC)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.spear_workspace_bytes.argtypes = [LP, i32]
    lib.spear_workspace_bytes.restype = sz
    lib.spear_pack_int4.argtypes = [P, P, i64, i64, P]
    lib.spear_pack_int4.restype = i32
    lib.spear_tile_int4.argtypes = [P, P, i64, i64, P]
    lib.spear_tile_int4.restype = i32
    lib.spear_linear_decode.argtypes = [LP, i32, P, P, i32, P, sz, P]
    lib.spear_linear_decode.restype = i32
    lib.spear_linear_decode_noalloc.argtypes = [LP, i32, P, P, i32, P]
    lib.spear_linear_decode_noalloc.restype = i32
    lib.spear_graph_begin.argtypes = [ctypes.POINTER(P)]
    lib.spear_graph_begin.restype = i32
    lib.spear_graph_add.argtypes = [P, LP, i32, P, P, i32, P, sz]
    lib.spear_graph_add.restype = i32
    lib.spear_graph_end.argtypes = [P]
    lib.spear_graph_end.restype = i32
    lib.spear_graph_launch.argtypes = [P, P]
    lib.spear_graph_launch.restype = i32
    lib.spear_graph_destroy.argtypes = [P]
    lib.spear_graph_destroy.restype = i32
    lib.spear_linear_prefill.argtypes = [LP, i32, P, P, i32, P, sz, P, P]
    lib.spear_linear_prefill.restype = i32
    lib.spear_linear.argtypes = [LP, i32, P, P, i32, P, sz, P, P]
    lib.spear_linear.restype = i32
    lib.spear_set_decode_max_m.argtypes = [i32]
    lib.spear_set_decode_max_m.restype = i32
    lib.spear_get_decode_max_m.argtypes = []
    lib.spear_get_decode_max_m.restype = i32
    lib.spear_set_decode_split_min_m.argtypes = [i32]
    lib.spear_set_decode_split_min_m.restype = i32
    lib.spear_get_decode_split_min_m.argtypes = []
    lib.spear_get_decode_split_min_m.restype = i32
    lib.spear_set_decode_split_min_k.argtypes = [i32]
    lib.spear_set_decode_split_min_k.restype = i32
    lib.spear_get_decode_split_min_k.argtypes = []
    lib.spear_get_decode_split_min_k.restype = i32
    lib.spear_select_chunk.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float), i32,
                                       ctypes.c_float, ctypes.POINTER(i32)]
    lib.spear_select_chunk.restype = i32
    lib.spear_status_string.argtypes = [i32]
    lib.spear_status_string.restype = ctypes.c_char_p
    lib.spear_last_error.argtypes = []
    lib.spear_last_error.restype = ctypes.c_char_p
    lib.spear_workspace_flags.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.spear_workspace_flags.restype = i32
    lib.spear_version.argtypes = []
    lib.spear_version.restype = i32
    lib.spear_linear_plan.argtypes = [LP, i32, sz, i32, ctypes.POINTER(SpearPlanC)]
    lib.spear_linear_plan.restype = i32
    lib.spear_set_decode_spin_limit.argtypes = [ctypes.c_uint32]
    lib.spear_set_decode_spin_limit.restype = i32
    lib.spear_get_decode_spin_limit.argtypes = []
    lib.spear_get_decode_spin_limit.restype = ctypes.c_uint32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != SPEAR_OK:
        lib = load_library()
        raise SpearError(status, f"{lib.spear_status_string(status).decode()}: "
                                 f"{lib.spear_last_error().decode()}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return SPEAR_F16
    if t.dtype == torch.bfloat16:
        return SPEAR_BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


@dataclass
class RankGate:
    """The per-rank gate gamma(t) = sigmoid(W2 relu(W1 t + b1) + b2) (see spear_rank_gate_t);
    W1 [hidden][r], b1 [hidden], W2 [r][hidden], b2 [r]: float32 device tensors."""

    hidden: int
    W1: object
    b1: object
    W2: object
    b2: object
    alpha: float = 1.0


@dataclass
class SpearLayer:
    """Device tensors of one compensated 4-bit layer (see spear_layer_t)."""

    N: int
    K: int
    group_size: int
    qweight: object             # int32 [qweight_rows(N)][K/8], tiled order
    scales: object              # float16 [N][K/G]
    zeros: object               # float16 [N][K/G]
    rank: int = 0
    A: object = None            # [r][K] activation dtype
    B: object = None            # [N][r]
    w_gate: object = None       # [K]
    b_gate: float = 0.0
    rank_gate: object = None    # RankGate, or None for the scalar gate

    def as_c(self) -> SpearLayerC:
        c = SpearLayerC(self.N, self.K, self.group_size, _ptr(self.qweight), _ptr(self.scales),
                        _ptr(self.zeros), self.rank, _ptr(self.A), _ptr(self.B),
                        _ptr(self.w_gate), float(self.b_gate), None)
        if self.rank_gate is not None:
            g = self.rank_gate
            c._rg = SpearRankGateC(int(g.hidden), _ptr(g.W1), _ptr(g.b1), _ptr(g.W2), _ptr(g.b2),
                                   float(g.alpha))  # kept alive with the struct
            c.rank_gate = ctypes.pointer(c._rg)
        return c

    def without_compensator(self) -> "SpearLayer":
        return SpearLayer(self.N, self.K, self.group_size, self.qweight, self.scales, self.zeros)


def spear_workspace_bytes(layer: SpearLayer, M: int) -> int:
    c = layer.as_c()
    return int(load_library().spear_workspace_bytes(ctypes.byref(c), int(M)))


def new_workspace(layer: SpearLayer, M: int, device="cuda"):
    """A zeroed, 256-byte aligned workspace for calls on `layer` with up to M tokens."""
    import torch
    n = spear_workspace_bytes(layer, M)
    if n == 0:
        raise SpearError(SPEAR_ERR_INVALID_ARGUMENT, "invalid layer or M for a workspace")
    buf = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + n]


def qweight_rows(N: int) -> int:
    """Rows of the packed weight tensor: N padded to a multiple of 16 (tiled order)."""
    return (int(N) + 15) // 16 * 16


def spear_pack_int4(q, qweight=None, stream=None):
    """uint8 codes [N][K] (device) -> int32 words [qweight_rows(N)][K/8] in the tiled order."""
    import torch
    _require(q.dim() == 2 and q.dtype == torch.uint8, "q must be a 2-D uint8 tensor [N][K]",
             TypeError)
    _require(q.is_contiguous(), "q must be contiguous")
    N, K = q.shape
    _require(K % 32 == 0, f"K={K} is not a multiple of 32")
    if qweight is None:
        qweight = torch.empty((qweight_rows(N), K // 8), dtype=torch.int32, device=q.device)
    _check_tensor(qweight, "qweight", (qweight_rows(N), K // 8), (torch.int32,))
    _require(q.device.type == "cuda" and qweight.device == q.device,
             f"q and qweight must be on one GPU (got {q.device} and {qweight.device})")
    _require(qweight.data_ptr() % 16 == 0, "qweight must be 16-byte aligned")
    _check(load_library().spear_pack_int4(_ptr(q), _ptr(qweight), N, K, _stream(stream)))
    return qweight


def spear_tile_int4(words, qweight=None, stream=None):
    """int32 words packed row after row [N][K/8] (device) -> the tiled order."""
    import torch
    _require(words.dim() == 2 and words.dtype == torch.int32,
             "words must be a 2-D int32 tensor [N][K/8]", TypeError)
    _require(words.is_contiguous(), "words must be contiguous")
    N, K = words.shape[0], 8 * words.shape[1]
    _require(K % 32 == 0, f"K={K} is not a multiple of 32")
    if qweight is None:
        qweight = torch.empty((qweight_rows(N), K // 8), dtype=torch.int32, device=words.device)
    _check_tensor(qweight, "qweight", (qweight_rows(N), K // 8), (torch.int32,))
    _require(words.device.type == "cuda" and qweight.device == words.device,
             f"words and qweight must be on one GPU (got {words.device} and {qweight.device})")
    _require(words.data_ptr() % 16 == 0 and qweight.data_ptr() % 16 == 0,
             "words and qweight must be 16-byte aligned")
    _check(load_library().spear_tile_int4(_ptr(words), _ptr(qweight), N, K, _stream(stream)))
    return qweight


def _require(cond, msg: str, exc=ValueError) -> None:
    if not cond:
        raise exc(msg)


def _check_tensor(t, name: str, shape, dtypes) -> None:
    """t is a contiguous tensor of exactly `shape` with a dtype in `dtypes`."""
    _require(t is not None, f"{name} is missing")
    _require(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    _require(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {dtypes}", TypeError)
    _require(t.is_contiguous(), f"{name} must be contiguous")


def _check_layer(layer: "SpearLayer", act) -> None:
    """Shapes, dtypes and contiguity of the layer's tensors, with activations of dtype act.

    The C ABI receives bare pointers and cannot check any of this; a wrong shape or
    stride would make the kernels read past the end of a buffer."""
    import torch
    N, K, G, r = layer.N, layer.K, layer.group_size, layer.rank
    _require(N >= 1 and K >= 1 and G >= 1 and K % G == 0 and K % 8 == 0,
             f"invalid layer geometry N={N} K={K} group_size={G}")
    bits16 = (torch.float16, torch.int16)   # fp16 values or their bit patterns
    _check_tensor(layer.qweight, "qweight", (qweight_rows(N), K // 8), (torch.int32,))
    _check_tensor(layer.scales, "scales", (N, K // G), bits16)
    _check_tensor(layer.zeros, "zeros", (N, K // G), bits16)
    if r > 0:
        _check_tensor(layer.A, "A", (r, K), (act,))
        _check_tensor(layer.B, "B", (N, r), (act,))
        if layer.rank_gate is None:
            _check_tensor(layer.w_gate, "w_gate", (K,), (act,))
        else:
            g = layer.rank_gate
            h = int(g.hidden)
            f32 = (torch.float32,)
            _check_tensor(g.W1, "rank_gate.W1", (h, r), f32)
            _check_tensor(g.b1, "rank_gate.b1", (h,), f32)
            _check_tensor(g.W2, "rank_gate.W2", (r, h), f32)
            _check_tensor(g.b2, "rank_gate.b2", (r,), f32)


def _layer_tensors(layer: "SpearLayer"):
    ts = [layer.qweight, layer.scales, layer.zeros]
    if layer.rank > 0:
        ts += [layer.A, layer.B, layer.w_gate]
        if layer.rank_gate is not None:
            g = layer.rank_gate
            ts += [g.W1, g.b1, g.W2, g.b2]
    return [t for t in ts if t is not None]


def _io(layer, x, y, workspace=None):
    """Check x, y, the workspace and the layer against each other; allocate y if None."""
    import torch
    _dtype_code(x)
    _require(x.dim() == 2, f"x must be 2-D [M][K], got {x.dim()}-D")
    _require(x.shape[1] == layer.K, f"x has {x.shape[1]} columns, the layer has K={layer.K}")
    _require(x.is_contiguous(), "x must be contiguous (row-major [M][K])")
    _check_layer(layer, x.dtype)
    M = x.shape[0]
    if y is not None:
        _check_tensor(y, "y", (M, layer.N), (x.dtype,))
    if workspace is not None:
        _require(workspace.is_contiguous(), "workspace must be contiguous")
    dev = x.device
    _require(dev.type == "cuda", f"x must be a GPU tensor, got {dev}")
    others = _layer_tensors(layer) + ([y] if y is not None else []) + \
        ([workspace] if workspace is not None else [])
    for t in others:
        _require(t.device == dev, f"every tensor must be on {dev}; found one on {t.device}")
    if y is None:
        y = torch.empty((M, layer.N), dtype=x.dtype, device=dev)
    else:
        xs, xe = x.data_ptr(), x.data_ptr() + x.numel() * x.element_size()
        ys, ye = y.data_ptr(), y.data_ptr() + y.numel() * y.element_size()
        _require(ye <= xs or xe <= ys or x.numel() == 0 or y.numel() == 0, "y must not overlap x")
    return M, y


def spear_linear_decode(layer: SpearLayer, x, y=None, workspace=None, stream=None):
    M, y = _io(layer, x, y, workspace)
    c = layer.as_c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().spear_linear_decode(ctypes.byref(c), _dtype_code(x), _ptr(x), _ptr(y), M,
                                              _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def spear_linear_decode_noalloc(layer: SpearLayer, x, y=None, stream=None):
    """spear_linear_decode on the library's own per-GPU scratch (no workspace, no allocation
    by the library; y is allocated here only when not given)."""
    M, y = _io(layer, x, y)
    c = layer.as_c()
    _check(load_library().spear_linear_decode_noalloc(ctypes.byref(c), _dtype_code(x), _ptr(x),
                                                      _ptr(y), M, _stream(stream)))
    return y


def spear_linear_prefill(layer: SpearLayer, x, y=None, workspace=None, main_stream=None,
                         aux_stream=None):
    M, y = _io(layer, x, y, workspace)
    c = layer.as_c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    aux = None if aux_stream is None else _stream(aux_stream)
    _check(load_library().spear_linear_prefill(ctypes.byref(c), _dtype_code(x), _ptr(x), _ptr(y), M,
                                               _ptr(workspace), ws_bytes, _stream(main_stream), aux))
    return y


def spear_linear(layer: SpearLayer, x, y=None, workspace=None, main_stream=None, aux_stream=None):
    M, y = _io(layer, x, y, workspace)
    c = layer.as_c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    aux = None if aux_stream is None else _stream(aux_stream)
    _check(load_library().spear_linear(ctypes.byref(c), _dtype_code(x), _ptr(x), _ptr(y), M,
                                       _ptr(workspace), ws_bytes, _stream(main_stream), aux))
    return y


class SpearGraph:
    """A static graph of layer calls held by the library (spear_graph_*): add calls with
    add(), then end(), then launch() as often as needed.  The tensors given to add() are
    kept referenced here, since the graph reads and writes them on every launch."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(load_library().spear_graph_begin(ctypes.byref(h)))
        self._h = h
        self._keep = []

    def add(self, layer: SpearLayer, x, y=None, workspace=None):
        M, y = _io(layer, x, y, workspace)
        c = layer.as_c()
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(load_library().spear_graph_add(self._h, ctypes.byref(c), _dtype_code(x), _ptr(x),
                                              _ptr(y), M, _ptr(workspace), ws_bytes))
        self._keep.append((layer, x, y, workspace))
        return y

    def end(self):
        _check(load_library().spear_graph_end(self._h))
        return self

    def launch(self, stream=None):
        _check(load_library().spear_graph_launch(self._h, _stream(stream)))

    def destroy(self):
        if self._h is not None:
            _check(load_library().spear_graph_destroy(self._h))
            self._h = None
            self._keep = []

    def __del__(self):
        try:
            self.destroy()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


def spear_set_decode_max_m(m: int) -> None:
    _check(load_library().spear_set_decode_max_m(int(m)))


def spear_get_decode_max_m() -> int:
    return int(load_library().spear_get_decode_max_m())


def spear_set_decode_split_min_m(m: int) -> None:
    _check(load_library().spear_set_decode_split_min_m(int(m)))


def spear_get_decode_split_min_m() -> int:
    return int(load_library().spear_get_decode_split_min_m())


def spear_set_decode_split_min_k(k: int) -> None:
    _check(load_library().spear_set_decode_split_min_k(int(k)))


def spear_get_decode_split_min_k() -> int:
    return int(load_library().spear_get_decode_split_min_k())


def spear_set_decode_spin_limit(polls: int) -> None:
    _check(load_library().spear_set_decode_spin_limit(int(polls)))


def spear_get_decode_spin_limit() -> int:
    return int(load_library().spear_get_decode_spin_limit())


def spear_select_chunk(chunks, pred_ms, budget_ms: float):
    """Largest chunk whose predicted latency fits the budget -> (chunk, violated)."""
    n = len(chunks)
    if n != len(pred_ms):
        raise ValueError("chunks and pred_ms differ in length")
    ca = (ctypes.c_int32 * max(n, 1))(*[int(c) for c in chunks])
    pa = (ctypes.c_float * max(n, 1))(*[float(p) for p in pred_ms])
    viol = ctypes.c_int32(0)
    lib = load_library()
    c = lib.spear_select_chunk(ca, pa, n, ctypes.c_float(budget_ms), ctypes.byref(viol))
    if c < 0:
        raise SpearError(SPEAR_ERR_INVALID_ARGUMENT, lib.spear_last_error().decode())
    return int(c), bool(viol.value)


def spear_status_string(status: int) -> str:
    return load_library().spear_status_string(int(status)).decode()


def spear_last_error() -> str:
    return load_library().spear_last_error().decode()


def spear_workspace_flags(workspace, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(load_library().spear_workspace_flags(_ptr(workspace), ctypes.byref(flags), _stream(stream)))
    return int(flags.value)


def spear_linear_plan(layer, M: int, workspace_bytes: int = 0, phase: str = "dispatch") -> dict:
    """The launch a call would take (nothing is launched): phase "dispatch" (spear_linear),
    "decode" or "prefill".  `layer` is a SpearLayer or a SpearLayerC."""
    c = layer if isinstance(layer, SpearLayerC) else layer.as_c()
    code = {"dispatch": 0, "decode": 1, "prefill": 2}[phase]
    out = SpearPlanC()
    _check(load_library().spear_linear_plan(ctypes.byref(c), int(M), int(workspace_bytes), code,
                                            ctypes.byref(out)))
    return {"path": PATH_NAMES.get(out.path, str(out.path)), "workgroups": out.workgroups,
            "waves_per_workgroup": out.waves_per_workgroup, "producers": out.producers,
            "k_splits": out.k_splits, "workspace_bytes": int(out.workspace_bytes)}


def spear_version() -> int:
    return int(load_library().spear_version())


def layer_to_device(host_layer, device="cuda", stream=None) -> SpearLayer:
    """Upload a synth.SynthLayer (unpacked codes) and pack it on the GPU."""
    import numpy as np
    import torch
    act = torch.float16 if host_layer.dtype == "f16" else torch.bfloat16

    def up(arr, dt):
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
        return t.view(dt)

    q = torch.from_numpy(np.ascontiguousarray(host_layer.q)).to(device)
    qweight = spear_pack_int4(q, stream=stream)
    lay = SpearLayer(N=host_layer.N, K=host_layer.K, group_size=host_layer.group_size,
                     qweight=qweight, scales=up(host_layer.scales, torch.float16),
                     zeros=up(host_layer.zeros, torch.float16), rank=host_layer.rank,
                     b_gate=host_layer.b_gate)
    if host_layer.rank > 0:
        lay.A = up(host_layer.A, act)
        lay.B = up(host_layer.B, act)
        lay.w_gate = up(host_layer.w_gate, act)
    return lay


def rank_gate_to_device(params, alpha: float = 1.0, device="cuda") -> RankGate:
    """float32 numpy W1, b1, W2, b2 (as from synth.make_rank_gate) -> a RankGate on the device."""
    import numpy as np
    import torch

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return RankGate(hidden=int(params["W1"].shape[0]), W1=up(params["W1"]), b1=up(params["b1"]),
                    W2=up(params["W2"]), b2=up(params["b2"]), alpha=float(alpha))


def act_to_device(bits, dtype: str, device="cuda"):
    """uint16 activation bit patterns (numpy) -> float16/bfloat16 device tensor."""
    import numpy as np
    import torch
    act = torch.float16 if dtype == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(act)


def inf_gate(sign: int) -> float:
    return math.copysign(math.inf, sign)

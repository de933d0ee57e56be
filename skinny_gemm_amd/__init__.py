"""Python binding of ``libqmoe.so`` (the C ABI in ``include/qmoe.h``).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  PyTorch provides device memory (tensors) and the stream.  When
the library is missing the import still succeeds, but the first call raises:
there is no CPU fallback.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmoe.so")

QTYPE = {"sym_int4": 0, "sym_int2": 1, "ternary": 2, "affine_int2": 3, "affine_int4": 4, "ternary_b3": 5}
DTYPE = {"bf16": 0, "f16": 1, "f32": 2}
PATH = {"auto": 0, "gemv": 1, "grouped": 2}
TOPK_WEIGHTS = {"renormalized": 0, "softmax_all": 1}
STATUS = {0: "OK", 1: "ERR_INVALID_ARGUMENT", 2: "ERR_UNSUPPORTED", 3: "ERR_WORKSPACE_TOO_SMALL",
          4: "ERR_DEVICE"}


class QmoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class QMatrixDesc(C.Structure):
    _fields_ = [("qtype", C.c_int32), ("block", C.c_int32), ("scale_dtype", C.c_int32),
                ("reserved", C.c_int32), ("rows", C.c_int64), ("cols", C.c_int64)]


class LayerDesc(C.Structure):
    _fields_ = [("num_experts", C.c_int32), ("hidden", C.c_int32), ("inter", C.c_int32),
                ("act_dtype", C.c_int32), ("fc1", QMatrixDesc), ("fc2", QMatrixDesc),
                ("activation", C.c_int32), ("reserved", C.c_int32)]


class ForwardOpts(C.Structure):
    _fields_ = [("path", C.c_int32), ("reserved", C.c_int32), ("h_out", C.c_void_p),
                ("ids_out", C.c_void_p), ("w_out", C.c_void_p), ("counts_out", C.c_void_p),
                ("events", C.POINTER(C.c_void_p)), ("num_events", C.c_int32), ("reserved2", C.c_int32),
                ("fc1_bias", C.c_void_p), ("fc2_bias", C.c_void_p), ("topk_weights", C.c_int32),
                ("reserved3", C.c_int32), ("workspace_limit", C.c_int64), ("swiglu_params", C.c_int32),
                ("swiglu_alpha", C.c_float), ("swiglu_beta", C.c_float), ("swiglu_limit", C.c_float)]


class Plan(C.Structure):
    _fields_ = [("path", C.c_int32), ("num_launches", C.c_int32), ("gemv_mmax", C.c_int32),
                ("gemv_fc1_waves", C.c_int32), ("gemv_fc2_waves", C.c_int32),
                ("max_active", C.c_int32), ("workspace_bytes", C.c_int64), ("kernels", C.c_char * 256),
                ("row_tile", C.c_int32), ("num_tiles", C.c_int32)]


_lib = None

# name -> (restype, argtypes)
_P, _I32, _SZ = C.c_void_p, C.c_int32, C.c_size_t
_SIGS = {
    "qmoe_abi_version": (C.c_int32, []),
    "qmoe_last_error": (C.c_char_p, []),
    "qmoe_prepacked_size": (C.c_int, [C.POINTER(LayerDesc), C.POINTER(_SZ)]),
    "qmoe_prepack": (C.c_int, [C.POINTER(LayerDesc)] + [_P] * 7 + [_SZ, _P]),
    "qmoe_prepack_scales": (C.c_int, [C.POINTER(LayerDesc)] + [_P] * 5 + [_SZ, _P]),
    "qmoe_workspace_size": (C.c_int, [C.POINTER(LayerDesc), _I32, _I32, C.POINTER(_SZ)]),
    "qmoe_forward": (C.c_int, [C.POINTER(LayerDesc), _P, _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "qmoe_forward_ex": (C.c_int, [C.POINTER(LayerDesc), _P, _P, _P, _I32, _I32, _P, _P, _SZ, _P,
                                  C.POINTER(ForwardOpts)]),
    "qmoe_forward_plan": (C.c_int, [C.POINTER(LayerDesc), _I32, _I32, C.POINTER(ForwardOpts),
                                    C.POINTER(Plan)]),
    "qmoe_route_workspace_size": (C.c_int, [_I32, _I32, _I32, C.POINTER(_SZ)]),
    "qmoe_route": (C.c_int, [_I32, _I32, _I32] + [_P] * 7 + [_SZ, _P]),
    "qmoe_unpack_codes": (C.c_int, [C.POINTER(LayerDesc), _P, _I32, _P, _P]),
    "qmoe_linear_prepacked_size": (C.c_int, [C.POINTER(QMatrixDesc), C.POINTER(_SZ)]),
    "qmoe_linear_prepack": (C.c_int, [C.POINTER(QMatrixDesc), _P, _P, _P, _P, _SZ, _P]),
    "qmoe_linear_workspace_size": (C.c_int, [C.POINTER(QMatrixDesc), _I32, C.POINTER(_SZ)]),
    "qmoe_linear": (C.c_int, [C.POINTER(QMatrixDesc), _P, _P, _I32, _I32, _P, _P, _SZ, _I32, _P]),
    "qmoe_linear_unpack_codes": (C.c_int, [C.POINTER(QMatrixDesc), _P, _P, _P]),
    "qmoe_read_probe": (C.c_int, [_P, _SZ, _P, _P]),
    "qmoe_forward_noalloc": (C.c_int, [C.POINTER(LayerDesc), _P, _P, _P, _I32, _I32, _P, _P]),
    "qmoe_channel_prepacked_size": (C.c_int, [C.POINTER(LayerDesc), C.POINTER(_SZ)]),
    "qmoe_channel_prepack": (C.c_int, [C.POINTER(LayerDesc)] + [_P] * 5 + [_SZ, _P]),
    "qmoe_channel_workspace_size": (C.c_int, [C.POINTER(LayerDesc), _I32, _I32, _I32, C.POINTER(_SZ)]),
    "qmoe_forward_channels": (C.c_int, [C.POINTER(LayerDesc), _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _SZ,
                                        _P]),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; "
                               f"g.build()'` (hipcc, gfx950). There is no fallback path.")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def last_error() -> str:
    return lib().qmoe_last_error().decode()


def _check(st: int):
    if st != 0:
        raise QmoeError(st, last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------ descriptors
def qmatrix_desc(fmt: str, block: int, scale_dtype: str, rows: int, cols: int) -> QMatrixDesc:
    return QMatrixDesc(QTYPE[fmt], block, DTYPE[scale_dtype], 0, rows, cols)


ACTIVATION = {"swiglu": 0, "relu": 1}


def layer_desc(E: int, H: int, I: int, act_dtype: str, fc1, fc2, activation: str = "swiglu") -> LayerDesc:
    """fc1/fc2 = (fmt, block, scale_dtype); FC1 has 2I rows (SwiGLU) or I (ReLU)."""
    rows1 = I if activation == "relu" else 2 * I
    return LayerDesc(E, H, I, DTYPE[act_dtype], qmatrix_desc(fc1[0], fc1[1], fc1[2], rows1, H),
                     qmatrix_desc(fc2[0], fc2[1], fc2[2], H, I), ACTIVATION[activation], 0)


# ------------------------------------------------------------------- MoE
def abi_version() -> int:
    return lib().qmoe_abi_version()


def prepacked_size(desc: LayerDesc) -> int:
    n = C.c_size_t()
    _check(lib().qmoe_prepacked_size(C.byref(desc), C.byref(n)))
    return n.value


def prepack(desc, fc1_codes, fc1_scales, fc1_biases, fc2_codes, fc2_scales, fc2_biases, dst,
            stream=None):
    _check(lib().qmoe_prepack(C.byref(desc), _ptr(fc1_codes), _ptr(fc1_scales), _ptr(fc1_biases),
                              _ptr(fc2_codes), _ptr(fc2_scales), _ptr(fc2_biases), _ptr(dst),
                              dst.numel() * dst.element_size(), _stream(stream)))


def prepack_scales(desc, fc1_scales, fc1_biases, fc2_scales, fc2_biases, packed, stream=None):
    """New scales (and affine biases) for an existing prepacked buffer; codes unchanged."""
    _check(lib().qmoe_prepack_scales(C.byref(desc), _ptr(fc1_scales), _ptr(fc1_biases), _ptr(fc2_scales),
                                     _ptr(fc2_biases), _ptr(packed), packed.numel() * packed.element_size(),
                                     _stream(stream)))


def workspace_size(desc, T: int, top_k: int) -> int:
    n = C.c_size_t()
    _check(lib().qmoe_workspace_size(C.byref(desc), T, top_k, C.byref(n)))
    return n.value


def forward(desc, packed, x, logits, T, top_k, y, ws, stream=None):
    _check(lib().qmoe_forward(C.byref(desc), _ptr(packed), _ptr(x), _ptr(logits), T, top_k, _ptr(y),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def forward_ex(desc, packed, x, logits, T, top_k, y, ws, stream=None, path="auto", h_out=None,
               ids_out=None, w_out=None, counts_out=None, events=None, fc1_bias=None, fc2_bias=None,
               topk_weights="renormalized", workspace_limit=0, swiglu=None):
    """``events``: optional list of raw hipEvent_t handles (ints), two per plan stage.
    ``fc1_bias`` [E][2I] / ``fc2_bias`` [E][H]: optional per-expert output biases
    in the activation dtype.  ``topk_weights``: "renormalized" (softmax over
    the selected logits) or "softmax_all" (selected entries of the softmax
    over all experts).  ``workspace_limit`` > 0 runs the tokens in row tiles
    whose workspace fits the limit (``forward_plan`` gives the tile sizes).
    ``swiglu`` = (alpha, beta, limit) selects the configurable SwiGLU
    (None: the plain silu(g) * u)."""
    ev = None
    if events:
        ev = (C.c_void_p * len(events))(*[C.c_void_p(int(e)) for e in events])
    opts = ForwardOpts(PATH[path], 0, _ptr(h_out), _ptr(ids_out), _ptr(w_out), _ptr(counts_out),
                       ev, len(events) if events else 0, 0, _ptr(fc1_bias), _ptr(fc2_bias),
                       TOPK_WEIGHTS[topk_weights], 0, int(workspace_limit), 1 if swiglu else 0,
                       *([float(v) for v in swiglu] if swiglu else [0.0, 0.0, 0.0]))
    _check(lib().qmoe_forward_ex(C.byref(desc), _ptr(packed), _ptr(x), _ptr(logits), T, top_k,
                                 _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
                                 C.byref(opts)))


def forward_noalloc(desc, packed, x, logits, T, top_k, y, stream=None):
    """qmoe_forward with the library's fixed device scratch as the workspace."""
    _check(lib().qmoe_forward_noalloc(C.byref(desc), _ptr(packed), _ptr(x), _ptr(logits), T, top_k, _ptr(y),
                                      _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def channel_prepacked_size(desc) -> int:
    n = C.c_size_t()
    _check(lib().qmoe_channel_prepacked_size(C.byref(desc), C.byref(n)))
    return n.value


def channel_prepack(desc, fc1_codes, fc1_scales, down_codes, down_scales, dst, stream=None):
    """Channel-packed buffer: FC1 rows as given, the down projection
    channel-major ([E][I][H*bits/8] codes, [E][I][H/block] scales)."""
    _check(lib().qmoe_channel_prepack(C.byref(desc), _ptr(fc1_codes), _ptr(fc1_scales), _ptr(down_codes),
                                      _ptr(down_scales), _ptr(dst), dst.numel() * dst.element_size(),
                                      _stream(stream)))


def channel_workspace_size(desc, T: int, top_k: int, Cn: int) -> int:
    n = C.c_size_t()
    _check(lib().qmoe_channel_workspace_size(C.byref(desc), T, top_k, Cn, C.byref(n)))
    return n.value


def forward_channels(desc, packed, x, logits, T, top_k, channels, Cn, y, ws, stream=None):
    """Gathered-channel forward: ``channels`` [T][top_k][Cn] int32 lists."""
    _check(lib().qmoe_forward_channels(C.byref(desc), _ptr(packed), _ptr(x), _ptr(logits), T, top_k,
                                       _ptr(channels), Cn, _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)))


def forward_plan(desc, T: int, top_k: int, path: str = "auto", topk_weights: str = "renormalized",
                 workspace_limit: int = 0) -> dict:
    opts = ForwardOpts(PATH[path], 0, None, None, None, None, None, 0, 0, None, None, TOPK_WEIGHTS[topk_weights], 0,
                       int(workspace_limit))
    p = Plan()
    _check(lib().qmoe_forward_plan(C.byref(desc), T, top_k, C.byref(opts), C.byref(p)))
    return {"path": p.path, "num_launches": p.num_launches, "gemv_mmax": p.gemv_mmax,
            "gemv_fc1_waves": p.gemv_fc1_waves, "gemv_fc2_waves": p.gemv_fc2_waves,
            "max_active": p.max_active, "workspace_bytes": p.workspace_bytes,
            "kernels": p.kernels.decode().split(",") if p.kernels else [],
            "row_tile": p.row_tile, "num_tiles": p.num_tiles}


def route_workspace_size(T: int, E: int, top_k: int) -> int:
    n = C.c_size_t()
    _check(lib().qmoe_route_workspace_size(T, E, top_k, C.byref(n)))
    return n.value


def route(T, E, top_k, logits, ids, w, counts, offsets, row_list, ws, stream=None):
    _check(lib().qmoe_route(T, E, top_k, _ptr(logits), _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets),
                            _ptr(row_list), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def unpack_codes(desc, packed, which: int, codes_out, stream=None):
    _check(lib().qmoe_unpack_codes(C.byref(desc), _ptr(packed), which, _ptr(codes_out), _stream(stream)))


# ----------------------------------------------------------------- dense
def linear_prepacked_size(desc: QMatrixDesc) -> int:
    n = C.c_size_t()
    _check(lib().qmoe_linear_prepacked_size(C.byref(desc), C.byref(n)))
    return n.value


def linear_prepack(desc, codes, scales, biases, dst, stream=None):
    _check(lib().qmoe_linear_prepack(C.byref(desc), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(dst),
                                     dst.numel() * dst.element_size(), _stream(stream)))


def linear_workspace_size(desc, M: int) -> int:
    n = C.c_size_t()
    _check(lib().qmoe_linear_workspace_size(C.byref(desc), M, C.byref(n)))
    return n.value


def linear(desc, packed, x, x_dtype: str, M: int, y, ws=None, path: str = "auto", stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().qmoe_linear(C.byref(desc), _ptr(packed), _ptr(x), DTYPE[x_dtype], M, _ptr(y), _ptr(ws),
                             nbytes, PATH[path], _stream(stream)))


def linear_unpack_codes(desc, packed, codes_out, stream=None):
    _check(lib().qmoe_linear_unpack_codes(C.byref(desc), _ptr(packed), _ptr(codes_out), _stream(stream)))


# ----------------------------------------------------------- diagnostics
def read_probe(src, sink, stream=None):
    """Stream every byte of the device tensor ``src`` (the HBM read-rate probe)."""
    _check(lib().qmoe_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))

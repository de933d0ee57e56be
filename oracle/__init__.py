"""CPU oracle of the low-bit quantized MoE expert FFN (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
double precision, scalar loops, see ``oracle.c``) and shares no code with the
HIP library.  Inputs are the canonical arrays of the ``synth`` package.

Functions follow the pages:

* ``unpack_codes``/``dequant``: block dequantization w = s*q (symmetric and
  ternary) or w = s*q + b (affine) -- onnxruntime PR 33005 (Current Scope:
  symmetric, no zero points, block 64) and MLX issue 3852 (affine groups,
  ternary as affine).
* ``route``: top-k routing and the per-expert row map -- onnxruntime PR 33005
  (Description: routing and expert-map kernels, rows expanded by expert).
* ``moe``: FC1, interleaved SwiGLU, FC2, top-k weighted combine --
  onnxruntime PR 33005 (Description).
* ``linear``: dense y = x W^T with W [N][K] -- MLX issue 3852 (repro).
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

FMT = {"sym_int4": 0, "sym_int2": 1, "ternary": 2, "affine_int2": 3, "affine_int4": 4, "ternary_b3": 5}
DT = {"bf16": 0, "f16": 1, "f32": 2}
BITS = {"sym_int4": 4, "sym_int2": 2, "ternary": 2, "affine_int2": 2, "affine_int4": 4}  # fixed-width formats

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        i64 = C.c_int64
        L.orc_half_to_double.restype = C.c_double
        L.orc_half_to_double.argtypes = [C.c_uint16, C.c_int]
        L.orc_double_to_half.restype = C.c_uint16
        L.orc_double_to_half.argtypes = [C.c_double, C.c_int]
        L.orc_halves_to_double.argtypes = [P, i64, C.c_int, P]
        L.orc_doubles_to_half.argtypes = [P, i64, C.c_int, P]
        L.orc_unpack_codes.restype = i64
        L.orc_unpack_codes.argtypes = [C.c_int, P, i64, i64, P]
        L.orc_unpack_codes_b.restype = i64
        L.orc_unpack_codes_b.argtypes = [C.c_int, C.c_int, P, i64, i64, P]
        L.orc_row_bytes.restype = i64
        L.orc_row_bytes.argtypes = [C.c_int, C.c_int, i64]
        L.orc_dequant.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, i64, i64, P]
        L.orc_route.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P, P, P]
        L.orc_silu.restype = C.c_double
        L.orc_silu.argtypes = [C.c_double]
        L.orc_swiglu.restype = C.c_double
        L.orc_swiglu.argtypes = [C.c_double] * 5
        L.orc_moe.restype = C.c_int
        L.orc_moe.argtypes = ([C.c_int] * 5 + [C.c_int] * 3 + [P] * 3 + [C.c_int] * 3 + [P] * 3
                              + [P, P, C.c_int, C.c_int] + [C.c_double] * 3 + [P, P, C.c_int] + [P] * 5)
        L.orc_moe_f32acc.restype = C.c_int
        L.orc_moe_f32acc.argtypes = ([C.c_int] * 5 + [C.c_int] * 3 + [P] * 3 + [C.c_int] * 3 + [P] * 3
                                     + [P, P, C.c_int, P, P])
        L.orc_moe_channels.restype = C.c_int
        L.orc_moe_channels.argtypes = ([C.c_int] * 5 + [C.c_int] * 3 + [P] * 2 + [C.c_int] * 3 + [P] * 2
                                       + [P, P, C.c_int, P, C.c_int] + [P] * 3)
        L.orc_linear.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, i64, i64, P, C.c_int, C.c_int,
                                 i64, i64, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- halves
def half_to_double(bits, dtype: str) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().orc_halves_to_double(_p(b), b.size, DT[dtype], _p(out))
    return out


def double_to_half(v, dtype: str) -> np.ndarray:
    a = _c(v, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_doubles_to_half(_p(a), a.size, DT[dtype], _p(out))
    return out


def silu(g: float) -> float:
    return lib().orc_silu(float(g))


PLAIN_SWIGLU = (1.0, 0.0, 0.0)


def swiglu(g: float, u: float, alpha: float = 1.0, beta: float = 0.0, limit: float = 0.0) -> float:
    """Configurable SwiGLU: clip (limit > 0), then g * sigmoid(alpha g) * (u + beta)."""
    return lib().orc_swiglu(float(g), float(u), float(alpha), float(beta), float(limit))


# ------------------------------------------------------------------ codec
def row_bytes(fmt: str, block: int, K: int) -> int:
    """Bytes of one packed row (base-3: ceil(block/5) bytes per block)."""
    return int(lib().orc_row_bytes(FMT[fmt], block, K))


def unpack_codes(fmt: str, packed, rows: int, K: int, block: int = 128):
    """Integer codes [rows][K] (int8) and the number of invalid fields (for
    base-3 rows, of weights in invalid bytes; the block matters only there)."""
    pk = _c(packed, np.uint8)
    assert pk.size == rows * row_bytes(fmt, block, K)
    out = np.empty((rows, K), dtype=np.int8)
    nbad = lib().orc_unpack_codes_b(FMT[fmt], block, _p(pk), rows, K, _p(out))
    return out, int(nbad)


def dequant(fmt: str, block: int, scale_dtype: str, codes, scales, biases, rows: int, K: int):
    """Dense float64 weights [rows][K]."""
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    out = np.empty((rows, K), dtype=np.float64)
    lib().orc_dequant(FMT[fmt], block, DT[scale_dtype], _p(c), _p(s), _p(b), rows, K, _p(out))
    return out


# ---------------------------------------------------------------- routing
def route(logits, top_k: int, renorm: bool = True):
    """Top-k ids, weights and the expert map.  ``renorm``: weights are the
    softmax over the selected logits; otherwise the softmax over all experts'
    logits, the selected probabilities kept unnormalised."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    S = T * top_k
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    rows = np.empty(max(S, 1), dtype=np.int32)
    lib().orc_route(T, E, top_k, int(bool(renorm)), _p(lg), _p(ids), _p(w), _p(counts), _p(offsets), _p(rows))
    return {"ids": ids, "w": w, "counts": counts, "offsets": offsets, "row_list": rows[:S]}


# -------------------------------------------------------------------- MoE
def moe(inp: dict, debug: bool = False, tokens=None, renorm: bool = True, threads: int = 1):
    """One MoE layer on the canonical inputs of ``synth.moe_inputs``.

    ``tokens`` selects a subset of token rows (each token's output depends
    only on its own activation and logits).  Optional ``fc1_expert_bias``
    [E][2I] and ``fc2_expert_bias`` [E][H] (16-bit patterns of the activation
    dtype) are per-expert output biases of FC1 and FC2.  Optional
    ``swiglu`` = (alpha, beta, limit) configures the SwiGLU (``swiglu``;
    default the plain silu(g) * u).  ``renorm`` selects
    the routing weights as in ``route``.  ``threads`` > 1 evaluates disjoint token
    subsets on that many host threads (the C library runs without the
    interpreter lock); a token's result does not depend on the others, so
    the outputs are identical to one thread.  Returns a dict with ``y64``
    (float64, unrounded), ``y`` (16-bit patterns of the activation dtype, or
    float32 values for f32 activations) and,
    with ``debug``, per-slot ``a``/``h``/``o`` in slot order t*k+j.
    """
    sp = inp["spec"]
    if threads > 1:
        idx = list(range(np.asarray(inp["x"]).shape[0])) if tokens is None else list(tokens)
        if len(idx) > 1:
            from concurrent.futures import ThreadPoolExecutor
            parts = [p for p in np.array_split(np.asarray(idx, dtype=np.int64), min(threads, len(idx))) if p.size]
            with ThreadPoolExecutor(len(parts)) as ex:
                outs = list(ex.map(lambda p: moe(inp, debug, p.tolist(), renorm, 1), parts))
            res = {"status": min(o["status"] for o in outs)}
            for key in ("y64", "y") + (("a", "h", "o") if debug else ()):
                res[key] = np.concatenate([o[key] for o in outs])
            return res
    adt = np.float32 if sp.act_dtype == "f32" else np.uint16   # f32 activations as values
    x = _c(inp["x"], adt)
    lg = _c(inp["logits"], np.float32)
    if tokens is not None:
        x = np.ascontiguousarray(x[tokens])
        lg = np.ascontiguousarray(lg[tokens])
    T = x.shape[0]
    H, I, k = sp.H, sp.I, sp.top_k
    y64 = np.empty((T, H), dtype=np.float64)
    y16 = np.empty((T, H), dtype=adt)
    a = h = o = None
    if debug:
        a = np.empty((T * k, I if sp.activation == "relu" else 2 * I), dtype=np.float64)
        h = np.empty((T * k, I), dtype=np.float64)
        o = np.empty((T * k, H), dtype=np.float64)
    arr = {n: _c(inp[n], np.uint8 if n.endswith("codes") else np.uint16)
           for n in ("fc1_codes", "fc1_scales", "fc1_biases", "fc2_codes", "fc2_scales", "fc2_biases")}
    eb = {n: _c(inp.get(n), adt) for n in ("fc1_expert_bias", "fc2_expert_bias")}
    rc = lib().orc_moe(
        sp.E, H, I, k, DT[sp.act_dtype],
        FMT[sp.fc1.fmt], sp.fc1.block, DT[sp.fc1.scale_dtype],
        _p(arr["fc1_codes"]), _p(arr["fc1_scales"]), _p(arr["fc1_biases"]),
        FMT[sp.fc2.fmt], sp.fc2.block, DT[sp.fc2.scale_dtype],
        _p(arr["fc2_codes"]), _p(arr["fc2_scales"]), _p(arr["fc2_biases"]),
        _p(eb["fc1_expert_bias"]), _p(eb["fc2_expert_bias"]), int(bool(renorm)), int(sp.activation == "relu"),
        *[float(v) for v in (inp.get("swiglu") or PLAIN_SWIGLU)],
        _p(x), _p(lg), T, _p(y64), _p(y16), _p(a), _p(h), _p(o))
    out = {"y64": y64, "y": y16, "status": rc}
    if debug:
        out.update(a=a, h=h, o=o)
    return out


def moe_f32acc(inp: dict, tokens=None):
    """The layer with every sum in single precision (``orc_moe_f32acc``):
    float dequantized weights, float dot products with k ascending, float
    silu, top-k weights and combine, one rounding to the activation dtype.
    SwiGLU, renormalised top-k weights, no expert biases.  Returns ``y32``
    (float32 sums) and ``y`` (rounded, as in ``moe``)."""
    sp = inp["spec"]
    assert sp.activation == "swiglu" and inp.get("fc1_expert_bias") is None
    adt = np.float32 if sp.act_dtype == "f32" else np.uint16
    x = _c(inp["x"], adt)
    lg = _c(inp["logits"], np.float32)
    if tokens is not None:
        x = np.ascontiguousarray(x[tokens])
        lg = np.ascontiguousarray(lg[tokens])
    T = x.shape[0]
    y32 = np.empty((T, sp.H), dtype=np.float32)
    y = np.empty((T, sp.H), dtype=adt)
    arr = {n: _c(inp[n], np.uint8 if n.endswith("codes") else np.uint16)
           for n in ("fc1_codes", "fc1_scales", "fc1_biases", "fc2_codes", "fc2_scales", "fc2_biases")}
    rc = lib().orc_moe_f32acc(
        sp.E, sp.H, sp.I, sp.top_k, DT[sp.act_dtype],
        FMT[sp.fc1.fmt], sp.fc1.block, DT[sp.fc1.scale_dtype],
        _p(arr["fc1_codes"]), _p(arr["fc1_scales"]), _p(arr["fc1_biases"]),
        FMT[sp.fc2.fmt], sp.fc2.block, DT[sp.fc2.scale_dtype],
        _p(arr["fc2_codes"]), _p(arr["fc2_scales"]), _p(arr["fc2_biases"]),
        _p(x), _p(lg), T, _p(y32), _p(y))
    return {"y32": y32, "y": y, "status": rc}


def moe_channels(inp: dict, channels, debug: bool = False):
    """Gathered channels (``orc_moe_channels``): ``channels`` [T][k][C] int32,
    entries < 0 unused; the down projection comes channel-major from
    ``inp["down_codes"]`` [E][I][H*bits/8] and ``inp["down_scales"]``
    [E][I][H/block] in the format ``inp["down_fmt"]`` = (fmt, block,
    scale_dtype).  SwiGLU layers with renormalised weights, no biases."""
    sp = inp["spec"]
    assert sp.activation == "swiglu" and sp.act_dtype in ("bf16", "f16", "f32")
    adt = np.float32 if sp.act_dtype == "f32" else np.uint16
    x = _c(inp["x"], adt)
    lg = _c(inp["logits"], np.float32)
    T = x.shape[0]
    ch = _c(channels, np.int32)
    assert ch.shape[:2] == (T, sp.top_k)
    Cn = ch.shape[2]
    dfmt, dblock, dsd = inp["down_fmt"]
    y64 = np.empty((T, sp.H), dtype=np.float64)
    y = np.empty((T, sp.H), dtype=adt)
    h = np.empty((T, sp.top_k, Cn), dtype=np.float64) if debug else None
    c1, s1 = _c(inp["fc1_codes"], np.uint8), _c(inp["fc1_scales"], np.uint16)
    cd, sd = _c(inp["down_codes"], np.uint8), _c(inp["down_scales"], np.uint16)
    rc = lib().orc_moe_channels(sp.E, sp.H, sp.I, sp.top_k, DT[sp.act_dtype],
                                FMT[sp.fc1.fmt], sp.fc1.block, DT[sp.fc1.scale_dtype], _p(c1), _p(s1),
                                FMT[dfmt], dblock, DT[dsd], _p(cd), _p(sd),
                                _p(x), _p(lg), T, _p(ch), Cn, _p(y64), _p(y), _p(h))
    out = {"y64": y64, "y": y, "status": rc}
    if debug:
        out["h"] = h
    return out


def linear(inp: dict, n0: int = 0, n1=None):
    """Dense y = x W^T for rows n in [n0, n1) of the canonical inputs of
    ``synth.linear_inputs``; returns y64 [M][n1-n0] and the rounded y."""
    sp = inp["spec"]
    N, K = inp["N"], sp.K
    n1 = N if n1 is None else n1
    x = _c(inp["x"], np.uint16)
    M = x.shape[0]
    c = _c(inp["codes"], np.uint8)
    s = _c(inp["scales"], np.uint16)
    b = _c(inp["biases"], np.uint16)
    y64 = np.empty((M, n1 - n0), dtype=np.float64)
    y16 = np.empty((M, n1 - n0), dtype=np.uint16)
    lib().orc_linear(FMT[sp.fmt.fmt], sp.fmt.block, DT[sp.fmt.scale_dtype], _p(c), _p(s), _p(b),
                     N, K, _p(x), DT[sp.act_dtype], M, n0, n1, _p(y64), _p(y16))
    return {"y64": y64, "y": y16}

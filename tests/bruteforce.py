"""Independent NumPy float64 brute force used to pin the oracle.

It shares nothing with ``oracle/``: fields are extracted with
``np.unpackbits``, 16-bit scales are decoded through NumPy's float16 and the
bfloat16-is-the-top-half-of-float32 definition, experts are selected with
``np.lexsort``, and the layer is computed as a *dense* mixture

    y_t = sum_e g[t, e] * W2_e (silu(gate_e(x_t)) * up_e(x_t)),

with g[t, e] = softmax of the top-k logits on the selected experts and 0
elsewhere, with no routing lists, offsets or per-slot bookkeeping.
"""

from __future__ import annotations

import numpy as np

OFFSET = {"sym_int4": 8, "sym_int2": 2, "ternary": 1, "affine_int2": 0, "affine_int4": 0}
BITS = {"sym_int4": 4, "sym_int2": 2, "ternary": 2, "affine_int2": 2, "affine_int4": 4}


def fields(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Stored fields u of packed rows [..., K*bits/8] -> [..., K] int64."""
    b = np.unpackbits(packed, axis=-1, bitorder="little").astype(np.int64)
    b = b.reshape(*packed.shape[:-1], K, bits)
    return (b << np.arange(bits, dtype=np.int64)).sum(-1)


def half_bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":  # f32 activations are carried as float32 values
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# base-3 digits of every byte value, least significant first, from numpy's
# base-3 string of the value (values of more than five digits stay invalid)
_B3 = np.array([[int(c) for c in np.base_repr(v, 3).zfill(5)[::-1][:5]] for v in range(243)], dtype=np.int64)


def b3_fields(packed: np.ndarray, block: int, K: int) -> np.ndarray:
    """Stored digits u of base-3 rows [..., K/block * ceil(block/5)] -> [..., K]."""
    per = (block + 4) // 5
    b = np.asarray(packed, dtype=np.int64).reshape(*packed.shape[:-1], K // block, per)
    assert (b < 243).all()
    d = _B3[b].reshape(*packed.shape[:-1], K // block, per * 5)[..., :block]
    return d.reshape(*packed.shape[:-1], K)


def dequant(fmt: str, block: int, sdtype: str, codes, scales, biases, K: int) -> np.ndarray:
    if fmt == "ternary_b3":
        q = b3_fields(np.asarray(codes, dtype=np.uint8), block, K) - 1
    else:
        q = fields(np.asarray(codes, dtype=np.uint8), BITS[fmt], K) - OFFSET[fmt]
    s = np.repeat(half_bits_to_f64(scales, sdtype), block, axis=-1)
    w = s * q
    if biases is not None:
        w = w + np.repeat(half_bits_to_f64(biases, sdtype), block, axis=-1)
    return w


def topk_gates(logits: np.ndarray, k: int, renorm: bool = True) -> np.ndarray:
    """Dense gate matrix g [T][E]: softmax over the selected logits, or
    (renorm False) the selected entries of the softmax over all logits."""
    T, E = logits.shape
    g = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        sel = order[:k]
        z = logits[t].astype(np.float64)
        p = np.exp(z - z.max())
        g[t, sel] = p[sel] / (p[sel].sum() if renorm else p.sum())
    return g


def moe_dense(inp: dict, renorm: bool = True) -> np.ndarray:
    sp = inp["spec"]
    E, H, I, k = sp.E, sp.H, sp.I, sp.top_k
    x = half_bits_to_f64(inp["x"], sp.act_dtype)
    g = topk_gates(np.asarray(inp["logits"]), k, renorm)
    y = np.zeros((x.shape[0], H), dtype=np.float64)
    for e in range(E):
        if not np.any(g[:, e]):
            continue
        W1 = dequant(sp.fc1.fmt, sp.fc1.block, sp.fc1.scale_dtype, inp["fc1_codes"][e],
                     inp["fc1_scales"][e], None if inp["fc1_biases"] is None else inp["fc1_biases"][e], H)
        W2 = dequant(sp.fc2.fmt, sp.fc2.block, sp.fc2.scale_dtype, inp["fc2_codes"][e],
                     inp["fc2_scales"][e], None if inp["fc2_biases"] is None else inp["fc2_biases"][e], I)
        a = x @ W1.T
        if inp.get("fc1_expert_bias") is not None:
            a = a + half_bits_to_f64(inp["fc1_expert_bias"][e], sp.act_dtype)[None, :]
        if getattr(sp, "activation", "swiglu") == "relu":
            h = np.maximum(a, 0.0)
        else:
            gate, up = a[:, 0::2], a[:, 1::2]
            alpha, beta, limit = inp.get("swiglu") or (1.0, 0.0, 0.0)
            if limit > 0:
                gate, up = np.minimum(gate, limit), np.clip(up, -limit, limit)
            h = gate * (1.0 / (1.0 + np.exp(-alpha * gate))) * (up + beta)
        o = h @ W2.T
        if inp.get("fc2_expert_bias") is not None:
            o = o + half_bits_to_f64(inp["fc2_expert_bias"][e], sp.act_dtype)[None, :]
        y += g[:, e:e + 1] * o
    return y


def linear_dense(inp: dict) -> np.ndarray:
    sp = inp["spec"]
    W = dequant(sp.fmt.fmt, sp.fmt.block, sp.fmt.scale_dtype, inp["codes"], inp["scales"],
                inp["biases"], sp.K)
    x = half_bits_to_f64(inp["x"], sp.act_dtype)
    return x @ W.T


def moe_channels_dense(inp: dict, channels) -> np.ndarray:
    """Gathered channels by dense masking: for each token, h over all channels
    of each selected expert, kept (with multiplicity) only where listed, then
    y_t = sum_j g_j * sum_c h_c D_e[c]."""
    sp = inp["spec"]
    E, H, I, k = sp.E, sp.H, sp.I, sp.top_k
    x = half_bits_to_f64(inp["x"], sp.act_dtype)
    logits = np.asarray(inp["logits"])
    dfmt, dblock, dsd = inp["down_fmt"]
    y = np.zeros((x.shape[0], H), dtype=np.float64)
    for t in range(x.shape[0]):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))[:k]
        z = logits[t].astype(np.float64)
        p = np.exp(z[order] - z[order].max())
        g = p / p.sum()
        for j, e in enumerate(order):
            W1 = dequant(sp.fc1.fmt, sp.fc1.block, sp.fc1.scale_dtype, inp["fc1_codes"][e], inp["fc1_scales"][e],
                         None, H)
            D = dequant(dfmt, dblock, dsd, inp["down_codes"][e], inp["down_scales"][e], None, H)
            a = W1 @ x[t]
            h = a[0::2] / (1.0 + np.exp(-a[0::2])) * a[1::2]
            mult = np.zeros(I)
            for c in np.asarray(channels)[t, j]:
                if c >= 0:
                    mult[c] += 1.0
            y[t] += g[j] * ((h * mult) @ D)
    return y

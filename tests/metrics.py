"""Parity metric for 16-bit (and f32) outputs against the oracle.

The workloads state a maximum relative error of 2e-3 with bf16 output and
fp32 accumulation.  Per element that bound is below one bf16 ulp (2^-8
relative), so a correct implementation that rounds once at the end could
still miss it on a single rounding straddle.  The reading used here:

* gate 1, per token row:  ||y - y_hat||_2 / ||y_hat||_2 <= 2e-3, where y_hat is
  the oracle's own rounded output (exact value rounded once to the dtype);
* gate 2, per element:     |y_i - y_hat_i| <= ulp(y_hat_i) + 2e-3 * rms(y64 row),
  which catches isolated wrong outputs that an L2 norm could hide;
* reported only: the fraction of bit-identical elements and the row error
  against the unrounded oracle value.
"""

from __future__ import annotations

import numpy as np

TOL = 2e-3


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":  # f32 outputs are carried as float32 values
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ulp(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.spacing(np.abs(np.asarray(bits, dtype=np.float32))).astype(np.float64)
    mag = np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)
    nxt = (mag.astype(np.uint32) + 1).astype(np.uint16)
    return np.abs(decode(nxt, dtype) - decode(mag, dtype))


def compare(y_bits: np.ndarray, ref_bits: np.ndarray, ref64: np.ndarray, dtype: str, tol: float = TOL):
    y = decode(y_bits, dtype)
    yh = decode(ref_bits, dtype)
    assert y.shape == yh.shape == ref64.shape, (y.shape, yh.shape, ref64.shape)
    y2 = y.reshape(-1, y.shape[-1])
    yh2 = yh.reshape(-1, yh.shape[-1])
    r64 = ref64.reshape(-1, ref64.shape[-1])
    finite = np.all(np.isfinite(y2))
    num = np.linalg.norm(y2 - yh2, axis=1)
    den = np.maximum(np.linalg.norm(yh2, axis=1), 1e-300)
    row_rel = num / den
    rms = np.sqrt(np.mean(r64 ** 2, axis=1, keepdims=True))
    elem_ok = np.abs(y2 - yh2) <= ulp(ref_bits, dtype).reshape(yh2.shape) + tol * rms
    rel64 = np.linalg.norm(y2 - r64, axis=1) / np.maximum(np.linalg.norm(r64, axis=1), 1e-300)
    res = {
        "finite": bool(finite),
        "max_row_rel": float(row_rel.max()) if row_rel.size else 0.0,
        "elem_ok": bool(elem_ok.all()),
        "n_elem_bad": int((~elem_ok).sum()),
        "frac_identical": float(np.mean(np.asarray(y_bits) == np.asarray(ref_bits))),
        "max_row_rel_vs_exact": float(rel64.max()) if rel64.size else 0.0,
    }
    res["ok"] = res["finite"] and res["max_row_rel"] <= tol and res["elem_ok"]
    return res

"""Counter-based SplitMix64 streams and the samplers built on them.

SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): the i-th output of a stream with
key ``g`` is ``mix64(g + (i + 1) * 0x9E3779B97F4A7C15)`` where ``mix64`` is the
variant-13 finaliser with shifts 30/27/31 and multipliers 0xBF58476D1CE4E5B9,
0x94D049BB133111EB.  Everything is vectorised NumPy uint64 arithmetic, which
wraps modulo 2**64 exactly as the definition requires.
"""

from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _fnv1a64(text: str) -> int:
    h = 0xCBF29CE484222325
    for b in text.encode("utf-8"):
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


class Key:
    """Stream key derived from (seed, workload name, tensor name)."""

    def __init__(self, seed: int, workload: str, tensor: str):
        base = np.array([(_fnv1a64(workload + "/" + tensor) ^ (seed * 0x9E3779B97F4A7C15))
                         & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
        self.value = np.uint64(_mix64(_mix64(base))[0])
        self.name = f"{workload}/{tensor}#{seed}"

    def sub(self, tag: str) -> "Key":
        k = Key.__new__(Key)
        base = np.array([int(self.value) ^ _fnv1a64(tag)], dtype=np.uint64)
        k.value = np.uint64(_mix64(base)[0])
        k.name = self.name + "." + tag
        return k


def raw_u64(key: Key, n: int, start: int = 0, chunk: int = 1 << 24) -> np.ndarray:
    """Outputs start .. start+n-1 of the stream ``key``."""
    out = np.empty(n, dtype=np.uint64)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        ctr = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
        with np.errstate(over="ignore"):
            out[c0:c1] = _mix64(key.value + ctr * _GOLDEN)
    return out


def uniform01(key: Key, n: int, open_low: bool = False) -> np.ndarray:
    """Float64 uniforms from the top 53 bits: [0, 1), or (0, 1] if open_low."""
    r = raw_u64(key, n) >> np.uint64(11)
    u = r.astype(np.float64)
    if open_low:
        u += 1.0
    return u * (1.0 / 9007199254740992.0)


def normals(key: Key, n: int) -> np.ndarray:
    """Standard normals by Box-Muller (cosine branch) in float64."""
    u1 = uniform01(key.sub("bm1"), n, open_low=True)
    u2 = uniform01(key.sub("bm2"), n)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (NumPy's nearest-even cast); uint16 bits."""
    return np.ascontiguousarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


def random_bytes(key: Key, nbytes: int) -> np.ndarray:
    n64 = (nbytes + 7) // 8
    return raw_u64(key, n64).view(np.uint8)[:nbytes].copy()


def codes_uniform(key: Key, nbytes: int) -> np.ndarray:
    """Packed codes whose every field is uniform over its 2**bits values.

    Uniform random bytes are exactly that for 2- and 4-bit fields.
    """
    return random_bytes(key, nbytes)


def ternary_digits(key: Key, nfields: int) -> np.ndarray:
    """Ternary stored digits u in {0, 1, 2} (q = u - 1) with the distribution
    of codes_ternary, one per weight, from the same random bits: the 2-bit
    and base-3 forms drawn with one key hold the same weights."""
    assert nfields % 4 == 0
    r = random_bytes(key, nfields // 4)
    lut = np.array([1, 1, 0, 2], dtype=np.uint8)
    out = np.empty(nfields, dtype=np.uint8)
    for f in range(4):
        out[f::4] = lut[(r >> (2 * f)) & 3]
    return out


def pack_base3(digits: np.ndarray, block: int) -> np.ndarray:
    """Rows of digits [..., K] in {0, 1, 2} -> base-3 storage [..., K/block *
    ceil(block/5)]: byte j of a block holds the block's digits 5j..5j+4 as
    sum d_i 3^i (least significant first); a block's last byte holds the
    block % 5 remaining digits."""
    d = np.asarray(digits, dtype=np.int64)
    K = d.shape[-1]
    assert K % block == 0
    per = (block + 4) // 5
    pad = per * 5 - block
    blocks = d.reshape(*d.shape[:-1], K // block, block)
    if pad:
        blocks = np.concatenate([blocks, np.zeros((*blocks.shape[:-1], pad), dtype=np.int64)], axis=-1)
    g = blocks.reshape(*blocks.shape[:-1], per, 5)
    v = (g * np.array([1, 3, 9, 27, 81], dtype=np.int64)).sum(-1)
    return v.astype(np.uint8).reshape(*d.shape[:-1], (K // block) * per)


def codes_ternary(key: Key, nfields: int) -> np.ndarray:
    """Packed 2-bit ternary fields with P(q=0)=1/2 and P(q=-1)=P(q=+1)=1/4.

    Two random bits r per weight pick the stored field value u: r in {0,1}
    gives u=1 (q=0), r=2 gives u=0 (q=-1), r=3 gives u=2 (q=+1).  Fields are
    packed four to a byte, LSB-first along K.
    """
    assert nfields % 4 == 0
    r = random_bytes(key, nfields // 4)
    lut = np.array([1, 1, 0, 2], dtype=np.uint8)
    out = np.zeros(nfields // 4, dtype=np.uint8)
    for f in range(4):
        out |= lut[(r >> (2 * f)) & 3] << (2 * f)
    return out

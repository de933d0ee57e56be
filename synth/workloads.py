"""The seeded synthetic workloads and their input recipes.

Five workloads, each named by what it is and its sizes:

``single_expert_int4``
    One expert FFN at M=1: x bf16 [1,512] ~N(0,1); gate/up W [2048,512] and
    down W [512,1024]; symmetric INT4 codes uniform in [-8,7]; block 64 along
    K; bf16 scales |N(0,0.02)|.
``switch_base_ternary``
    64 experts, hidden 768, intermediate 3072, top-1, batch-1 decode; ternary
    codes with P(0)=1/2; block 128; fp16 scales |N(0,0.02)|; logits N(0,1).
``dsv2lite_int4``
    64 experts, top-6, hidden 2048, intermediate 1408; symmetric INT4 block 64
    with bf16 scales; decode with T in {1,2,4,8}; logits N(0,1).
``mixed_int2_int4_prefill``
    128 experts, top-8, hidden 4096, intermediate 1536; FC1 symmetric INT2 and
    FC2 symmetric INT4, both block 64; 2048 tokens; logits N(0,1) plus a
    per-expert bias N(0,1) drawn once (skewed load).
``dense_affine2``
    Dense 2-bit affine matmul, K=5120 -> N in {17408, 248320}, group 128, codes
    uniform in {0..3}, fp16 scale |N(0,0.02)| and bias N(0,0.01), x fp16
    ~N(0,1), M in {1,2,3,4,5,8,10,16,32}.

The shapes of the MoE layers follow the model families the pages measure
(Switch-base, DeepSeek-V2-Lite, a GPT-OSS-20B-like mixed INT2/INT4 prefill)
and the dense shapes are the two of the MLX quantized_matmul M-sweep; no
trained weights exist here, so every code, scale and activation is drawn.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .rng import (Key, normals, f32_to_bf16_bits, f32_to_f16_bits, codes_uniform, codes_ternary, raw_u64,
                  ternary_digits, pack_base3)

# name -> (bits per stored field, has a per-block bias)
FORMATS = {
    "sym_int4": (4, False),
    "sym_int2": (2, False),
    "ternary": (2, False),
    "affine_int2": (2, True),
    "affine_int4": (4, True),
    "ternary_b3": (0, False),  # base-3: five weights per byte, ceil(block/5) bytes per block
}

DTYPES = ("bf16", "f16")


@dataclass(frozen=True)
class MatFmt:
    fmt: str
    block: int
    scale_dtype: str  # "bf16" | "f16"

    @property
    def bits(self) -> int:
        return FORMATS[self.fmt][0]

    @property
    def affine(self) -> bool:
        return FORMATS[self.fmt][1]

    def row_bytes(self, K: int) -> int:
        """Bytes of one packed row of K weights."""
        if self.fmt == "ternary_b3":
            return (K // self.block) * ((self.block + 4) // 5)
        return K * self.bits // 8


@dataclass(frozen=True)
class MoeSpec:
    name: str
    E: int
    H: int
    I: int
    top_k: int
    fc1: MatFmt
    fc2: MatFmt
    act_dtype: str = "bf16"
    tokens: tuple = (1,)
    logit_bias: bool = False
    scale_sigma: float = 0.02
    bias_sigma: float = 0.01
    activation: str = "swiglu"  # or "relu": FC1 is one [I][H] matrix, h = max(a, 0)

    @property
    def fc1_rows(self) -> int:
        return self.I if self.activation == "relu" else 2 * self.I


@dataclass(frozen=True)
class LinearSpec:
    name: str
    K: int
    Ns: tuple
    fmt: MatFmt
    act_dtype: str = "f16"
    Ms: tuple = (1,)
    scale_sigma: float = 0.02
    bias_sigma: float = 0.01


MOE_WORKLOADS = {
    "single_expert_int4": MoeSpec(
        "single_expert_int4", E=1, H=512, I=1024, top_k=1,
        fc1=MatFmt("sym_int4", 64, "bf16"), fc2=MatFmt("sym_int4", 64, "bf16"), tokens=(1,)),
    "switch_base_ternary": MoeSpec(
        "switch_base_ternary", E=64, H=768, I=3072, top_k=1,
        fc1=MatFmt("ternary", 128, "f16"), fc2=MatFmt("ternary", 128, "f16"), tokens=(1,)),
    "dsv2lite_int4": MoeSpec(
        "dsv2lite_int4", E=64, H=2048, I=1408, top_k=6,
        fc1=MatFmt("sym_int4", 64, "bf16"), fc2=MatFmt("sym_int4", 64, "bf16"), tokens=(1, 2, 4, 8)),
    "mixed_int2_int4_prefill": MoeSpec(
        "mixed_int2_int4_prefill", E=128, H=4096, I=1536, top_k=8,
        fc1=MatFmt("sym_int2", 64, "bf16"), fc2=MatFmt("sym_int4", 64, "bf16"), tokens=(2048,),
        logit_bias=True),
}

LINEAR_WORKLOADS = {
    "dense_affine2": LinearSpec(
        "dense_affine2", K=5120, Ns=(17408, 248320), fmt=MatFmt("affine_int2", 128, "f16"),
        act_dtype="f16", Ms=(1, 2, 3, 4, 5, 8, 10, 16, 32)),
}


def _to_bits(v64: np.ndarray, dtype: str) -> np.ndarray:
    v32 = v64.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(v32)
    if dtype == "f16":
        return f32_to_f16_bits(v32)
    if dtype == "f32":  # f32 activations are carried as float32 values
        return v32
    raise ValueError(dtype)


def canonical_matrix_bytes(fmt: MatFmt, N: int, K: int) -> int:
    """Bytes of one matrix in the canonical format: codes + scales (+ biases)."""
    nb = K // fmt.block
    per_row = fmt.row_bytes(K) + nb * 2 * (2 if fmt.affine else 1)
    return N * per_row


def _matrix(workload: str, tag: str, seed: int, fmt: MatFmt, E: int, N: int, K: int,
            scale_sigma: float, bias_sigma: float):
    assert K % fmt.block == 0 and (fmt.fmt == "ternary_b3" or (K * fmt.bits) % 8 == 0)
    kc = Key(seed, workload, tag + ".codes")
    nfields = E * N * K
    if fmt.fmt == "ternary":
        codes = codes_ternary(kc, nfields)
    elif fmt.fmt == "ternary_b3":
        codes = pack_base3(ternary_digits(kc, nfields).reshape(E * N, K), fmt.block)
    else:
        codes = codes_uniform(kc, nfields * fmt.bits // 8)
    codes = codes.reshape(E, N, fmt.row_bytes(K))
    nb = K // fmt.block
    s = np.abs(scale_sigma * normals(Key(seed, workload, tag + ".scales"), E * N * nb))
    scales = _to_bits(s, fmt.scale_dtype).reshape(E, N, nb)
    biases = None
    if fmt.affine:
        b = bias_sigma * normals(Key(seed, workload, tag + ".biases"), E * N * nb)
        biases = _to_bits(b, fmt.scale_dtype).reshape(E, N, nb)
    return codes, scales, biases


def moe_inputs(spec: MoeSpec, T: int, seed: int = 0, logits_mode: str = "iid",
               weight_copy: int = 0, weights: bool = True, expert_bias: float = 0.0) -> dict:
    """Inputs of one MoE layer call with T tokens.

    logits_mode: "iid" draws logits[t][e] ~ N(0,1) independently (plus the
    per-expert bias when the workload has one); "shared" draws one row and
    repeats it for every token, so every selected expert receives all T rows;
    "ties" rounds the iid draws to multiples of 0.5, so many logits of a row
    are equal and the selection depends on the tie rule.
    weight_copy selects an independent set of expert weights (distinct copies
    for cache-cold timing); activations and logits do not depend on it.
    expert_bias > 0 adds per-expert output biases of FC1 ([E][fc1 rows]) and FC2
    ([E][H]), N(0, expert_bias^2) in the activation dtype; otherwise both are
    None.
    """
    wl = spec.name
    out = {"spec": spec, "T": T, "seed": seed}
    if weights:
        wtag = "" if weight_copy == 0 else f"@copy{weight_copy}"
        out["fc1_codes"], out["fc1_scales"], out["fc1_biases"] = _matrix(
            wl, "fc1" + wtag, seed, spec.fc1, spec.E, spec.fc1_rows, spec.H, spec.scale_sigma, spec.bias_sigma)
        out["fc2_codes"], out["fc2_scales"], out["fc2_biases"] = _matrix(
            wl, "fc2" + wtag, seed, spec.fc2, spec.E, spec.H, spec.I, spec.scale_sigma, spec.bias_sigma)
    out["fc1_expert_bias"] = out["fc2_expert_bias"] = None
    if expert_bias > 0:
        wtag = "" if weight_copy == 0 else f"@copy{weight_copy}"
        b1 = expert_bias * normals(Key(seed, wl, "fc1_expert_bias" + wtag), spec.E * spec.fc1_rows)
        b2 = expert_bias * normals(Key(seed, wl, "fc2_expert_bias" + wtag), spec.E * spec.H)
        out["fc1_expert_bias"] = _to_bits(b1, spec.act_dtype).reshape(spec.E, spec.fc1_rows)
        out["fc2_expert_bias"] = _to_bits(b2, spec.act_dtype).reshape(spec.E, spec.H)
    x = normals(Key(seed, wl, f"x[T={T}]"), T * spec.H)
    out["x"] = _to_bits(x, spec.act_dtype).reshape(T, spec.H)
    if logits_mode == "iid":
        z = normals(Key(seed, wl, f"logits[T={T}]"), T * spec.E).reshape(T, spec.E)
    elif logits_mode == "shared":
        z = np.broadcast_to(normals(Key(seed, wl, "logits[shared]"), spec.E), (T, spec.E)).copy()
    elif logits_mode == "ties":
        z = np.round(2.0 * normals(Key(seed, wl, f"logits[T={T}]"), T * spec.E).reshape(T, spec.E)) / 2.0
    else:
        raise ValueError(logits_mode)
    if spec.logit_bias:
        z = z + normals(Key(seed, wl, "expert_bias"), spec.E)[None, :]
    out["logits"] = np.ascontiguousarray(z.astype(np.float32))
    return out


def linear_inputs(spec: LinearSpec, N: int, M: int, seed: int = 0, weight_copy: int = 0,
                  weights: bool = True) -> dict:
    """Inputs of one dense skinny-M quantized matmul y = x W^T, W [N][K]."""
    wl = f"{spec.name}[N={N}]"
    out = {"spec": spec, "N": N, "M": M, "seed": seed}
    if weights:
        wtag = "" if weight_copy == 0 else f"@copy{weight_copy}"
        c, s, b = _matrix(wl, "w" + wtag, seed, spec.fmt, 1, N, spec.K, spec.scale_sigma, spec.bias_sigma)
        out["codes"], out["scales"] = c[0], s[0]
        out["biases"] = None if b is None else b[0]
    x = normals(Key(seed, wl, f"x[M={M}]"), M * spec.K)
    out["x"] = _to_bits(x, spec.act_dtype).reshape(M, spec.K)
    return out


def custom_moe_spec(E: int, H: int, I: int, top_k: int, fc1: str = "sym_int4", fc2: Optional[str] = None,
                    block1: int = 64, block2: Optional[int] = None, scale_dtype: str = "bf16",
                    act_dtype: str = "bf16", logit_bias: bool = False, name: Optional[str] = None,
                    activation: str = "swiglu") -> MoeSpec:
    """A small MoE layer of the same recipe, for parity sweeps over shapes."""
    fc2 = fc2 or fc1
    block2 = block2 or block1
    nm = name or (f"custom_E{E}_H{H}_I{I}_k{top_k}_{fc1}{block1}_{fc2}{block2}_{scale_dtype}_{act_dtype}"
                  + ("" if activation == "swiglu" else f"_{activation}"))
    return MoeSpec(nm, E=E, H=H, I=I, top_k=top_k, fc1=MatFmt(fc1, block1, scale_dtype),
                   fc2=MatFmt(fc2, block2, scale_dtype), act_dtype=act_dtype, logit_bias=logit_bias,
                   activation=activation)


def custom_linear_spec(K: int, fmt: str = "affine_int2", block: int = 128, scale_dtype: str = "f16",
                       act_dtype: str = "f16", name: Optional[str] = None) -> LinearSpec:
    nm = name or f"custom_linear_K{K}_{fmt}{block}_{scale_dtype}_{act_dtype}"
    return LinearSpec(nm, K=K, Ns=(), fmt=MatFmt(fmt, block, scale_dtype), act_dtype=act_dtype)


def channel_inputs(spec: MoeSpec, inp: dict, budget: float, seed: int = 0, down: Optional[MatFmt] = None) -> dict:
    """Inputs of a gathered-channel call on top of ``moe_inputs``' arrays.

    The down projection stored channel-major: ``down_codes`` [E][I][H*bits/8]
    and ``down_scales`` [E][I][H/block] (row c is channel c's column of the
    down matrix, quantized along H), drawn with the same recipe in the format
    ``down`` (default: the layer's FC2 format).  ``channels`` [T][k][C] int32:
    per token, round(budget * k * I) distinct channel picks split at random
    over its k routed slots (so one slot may get many and another none), each
    slot's channels a random subset of [0, I) in random order, padded with -1
    to the longest list.
    """
    down = down or spec.fc2
    wl = spec.name
    c, sc, _ = _matrix(wl, "down_cm", seed, down, spec.E, spec.I, spec.H, spec.scale_sigma, spec.bias_sigma)
    out = {"down_codes": c, "down_scales": sc, "down_fmt": (down.fmt, down.block, down.scale_dtype)}
    T, k, I = inp["x"].shape[0], spec.top_k, spec.I
    n = int(round(budget * k * I))
    r = Key(seed, wl, f"channels[T={T},n={n}]")
    u = raw_u64(r, T * (k * I + 1)).reshape(T, k * I + 1)
    lists = []
    for t in range(T):
        # a random permutation of the (slot, channel) pairs, first n kept
        order = np.argsort(u[t, :k * I], kind="stable")[:n]
        slot, chan = order // I, order % I
        lists.append([chan[slot == j] for j in range(k)])
    C = max(1, max(len(l) for per in lists for l in per))
    ch = np.full((T, k, C), -1, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            ch[t, j, :len(lists[t][j])] = lists[t][j]
    out["channels"] = ch
    return out

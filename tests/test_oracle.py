"""Pins of the CPU oracle against facts fixed outside it (no GPU).

Each test ties one part of the oracle to something other than itself: bytes
hand-packed from the format definitions, library routines (NumPy float16
casts, lexsort, bincount, stable argsort, softmax), exact integer
arithmetic, identities between formats that the pages state, and an
independent dense float64 brute force on tiny shapes.
"""

import json
import os

import numpy as np
import pytest
import scipy.special

import synth
from synth.workloads import custom_moe_spec, custom_linear_spec
from tests import bruteforce as bf

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ 16-bit floats
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_half_decode_exhaustive(oracle_lib, dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_lib.half_to_double(bits, dtype)
    ref = bf.half_bits_to_f64(bits, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # encode(decode(b)) is the identity on every non-NaN pattern
    back = oracle_lib.double_to_half(got[~nan], dtype)
    assert np.array_equal(back, bits[~nan])


def test_f16_rounding_matches_numpy(oracle_lib):
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        (np.arange(-2048, 2048) + 0.5) * 2.0 ** -24,     # subnormal halfway points
        (np.arange(1024, 2048) + 0.5) * 2.0 ** -10,      # normal halfway points
        [65504.0, 65519.99, 65520.0, 1e6, -1e-9, 0.0, -0.0],
    ])
    got = oracle_lib.double_to_half(v, "f16")
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_is_nearest_even(oracle_lib):
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-38, 30, 20000),
        (np.arange(128, 256) + 0.5) * 2.0 ** -7,        # ties at exponent 0
        (np.arange(0, 128) + 0.5) * 2.0 ** -133,        # ties in the subnormal range
    ])
    got = oracle_lib.double_to_half(v, "bf16")
    g = oracle_lib.half_to_double(got, "bf16")
    # neighbours in bit space of |v|'s encoding
    mag = got & 0x7FFF
    lo = oracle_lib.half_to_double((mag - 1).astype(np.uint16), "bf16")
    hi = oracle_lib.half_to_double((mag + 1).astype(np.uint16), "bf16")
    a = np.abs(v)
    d = np.abs(np.abs(g) - a)
    ok_lo = (mag == 0) | (d <= np.abs(lo - a))
    ok_hi = d <= np.abs(hi - a)
    assert np.all(ok_lo & ok_hi)
    ties = (d == np.abs(lo - a)) | (d == np.abs(hi - a))
    assert np.all((mag[ties] & 1) == 0)
    # float32-representable values: bf16 is the RNE of the float32, which torch computes
    import torch
    f = rng.standard_normal(5000).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle_lib.double_to_half(f.astype(np.float64), "bf16"), ref)


# ------------------------------------------------------------------- codec
def test_codec_golden_bytes(oracle_lib):
    g = json.load(open(os.path.join(GOLD, "codec_bytes.json")))
    for case in g["cases"]:
        fmt = case["fmt"]
        bits = oracle_lib.BITS[fmt]
        K = 8 // bits
        codes, nbad = oracle_lib.unpack_codes(fmt, np.array([case["byte"]], np.uint8), 1, K)
        assert nbad == 0
        assert codes[0].tolist() == case["codes"], case
        if "values" in case:
            sd = "f16"
            s = oracle_lib.double_to_half(np.array([case["scale"]]), sd)
            b = oracle_lib.double_to_half(np.array([case["bias"]]), sd)
            # one block covering the byte (block >= K); pad to a block of 64
            nfield = 64
            row = np.full(nfield * bits // 8, case["byte"], dtype=np.uint8)
            W = oracle_lib.dequant(fmt, 64, sd, row, s, b, 1, nfield)
            assert W[0, :K].tolist() == case["values"]


@pytest.mark.parametrize("fmt", [f for f in synth.FORMATS if f != "ternary_b3"])  # base 3: its own pins below
def test_codec_all_bytes_vs_unpackbits(oracle_lib, fmt):
    bits = oracle_lib.BITS[fmt]
    packed = np.arange(256, dtype=np.uint8).reshape(256, 1)
    K = 8 // bits
    codes, nbad = oracle_lib.unpack_codes(fmt, packed, 256, K)
    u = bf.fields(packed, bits, K)
    if fmt == "ternary":
        assert nbad == int((u == 3).sum())
        ok = u != 3
        assert np.array_equal(codes[ok], (u - 1)[ok])
    else:
        assert nbad == 0
        assert np.array_equal(codes, u - bf.OFFSET[fmt])


def _rand_mat(fmt, N, K, block, sdtype, seed):
    spec = custom_linear_spec(K, fmt=fmt, block=block, scale_dtype=sdtype, act_dtype="bf16",
                              name=f"pin_{fmt}_{seed}")
    return synth.linear_inputs(spec, N, 1, seed=seed)


@pytest.mark.parametrize("sdtype", ["bf16", "f16"])
def test_dequant_cross_format_identities(oracle_lib, sdtype):
    """Symmetric b-bit == affine b-bit with bias -2^(b-1)*s; ternary == affine
    2-bit with bias -s (MLX issue 3852: ternary stored as affine has
    bias == -scale)."""
    N, K, B = 64, 256, 64
    for sym, aff, off in (("sym_int4", "affine_int4", 8), ("sym_int2", "affine_int2", 2),
                          ("ternary", "affine_int2", 1)):
        inp = _rand_mat(sym, N, K, B, sdtype, seed=3)
        s = oracle_lib.half_to_double(inp["scales"], sdtype)
        b = oracle_lib.double_to_half(-off * s, sdtype)          # exact: power-of-two multiple
        assert np.array_equal(oracle_lib.half_to_double(b, sdtype), -off * s)
        Ws = oracle_lib.dequant(sym, B, sdtype, inp["codes"], inp["scales"], None, N, K)
        Wa = oracle_lib.dequant(aff, B, sdtype, inp["codes"], inp["scales"], b, N, K)
        assert np.array_equal(Ws, Wa), sym


@pytest.mark.parametrize("fmt", list(synth.FORMATS))
def test_unit_scale_integer_matmul_is_exact(oracle_lib, fmt):
    """All-one scales and integer activations reproduce an int64 matmul exactly."""
    N, K, B, M = 64, 512, 64, 3
    inp = _rand_mat(fmt, N, K, B, "bf16", seed=5)
    inp["scales"][:] = 0x3F80                                    # bf16 1.0
    if inp["biases"] is not None:
        inp["biases"][:] = 0xC000                                # bf16 -2.0
    xi = np.random.default_rng(7).integers(-8, 9, size=(M, K))
    inp["x"] = oracle_lib.double_to_half(xi.astype(np.float64), "bf16").reshape(M, K)
    inp["M"] = M
    out = oracle_lib.linear(inp)
    if fmt == "ternary_b3":
        q = bf.b3_fields(inp["codes"], B, K) - 1
    else:
        q = bf.fields(inp["codes"], oracle_lib.BITS[fmt], K) - bf.OFFSET[fmt]
    if inp["biases"] is not None:
        q = q - 2
    ref = xi.astype(np.int64) @ q.T.astype(np.int64)
    assert np.array_equal(out["y64"], ref.astype(np.float64))


def test_moe_fc1_integer_exact(oracle_lib):
    spec = custom_moe_spec(E=2, H=128, I=64, top_k=1, fc1="sym_int4", name="pin_fc1_int")
    inp = synth.moe_inputs(spec, T=3, seed=1)
    inp["fc1_scales"][:] = 0x3F80
    xi = np.random.default_rng(3).integers(-8, 9, size=(3, 128))
    inp["x"] = oracle_lib.double_to_half(xi.astype(np.float64), "bf16").reshape(3, 128)
    out = oracle_lib.moe(inp, debug=True)
    r = oracle_lib.route(inp["logits"], 1)
    for t in range(3):
        e = r["ids"][t, 0]
        q = bf.fields(inp["fc1_codes"][e], 4, 128) - 8
        assert np.array_equal(out["a"][t], (q.astype(np.int64) @ xi[t]).astype(np.float64))


# ----------------------------------------------------------------- SwiGLU
def test_silu_pins(oracle_lib):
    assert oracle_lib.silu(0.0) == 0.0
    for g in np.linspace(-30, 30, 601):
        s1, s2 = oracle_lib.silu(g), oracle_lib.silu(-g)
        assert abs((s1 - s2) - g) <= 4 * np.spacing(max(abs(g), 1e-300)) + 1e-300
        ref = g * scipy.special.expit(g)
        assert abs(s1 - ref) <= 4 * np.spacing(abs(ref)) + 1e-300


def test_swiglu_zero_up_gives_zero(oracle_lib):
    spec = custom_moe_spec(E=1, H=64, I=64, top_k=1, name="pin_up0")
    inp = synth.moe_inputs(spec, T=2, seed=2)
    c = inp["fc1_codes"].copy()
    c[:, 1::2, :] = 0x88                                          # int4 code 0 in every up row
    inp["fc1_codes"] = c
    out = oracle_lib.moe(inp, debug=True)
    assert np.all(out["h"] == 0.0) and np.all(out["y64"] == 0.0)


# ---------------------------------------------------------------- routing
def _check_route(oracle_lib, logits, k):
    r = oracle_lib.route(logits, k)
    T, E = logits.shape
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        assert r["ids"][t].tolist() == order[:k].tolist()
        sel = logits[t, order[:k]].astype(np.float64)
        assert np.allclose(r["w"][t], scipy.special.softmax(sel), rtol=1e-13, atol=0)
        assert abs(r["w"][t].sum() - 1.0) <= k * 2.0 ** -52
        if k == 1:
            assert r["w"][t, 0] == 1.0
    flat = r["ids"].ravel()
    assert np.array_equal(r["counts"], np.bincount(flat, minlength=E))
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(r["row_list"], np.argsort(flat, kind="stable"))


@pytest.mark.parametrize("E,k", [(1, 1), (4, 2), (64, 6), (128, 8), (256, 8), (64, 1)])
def test_route_random(oracle_lib, E, k):
    lg = np.random.default_rng(E * 10 + k).standard_normal((33, E)).astype(np.float32)
    _check_route(oracle_lib, lg, k)


@pytest.mark.parametrize("E,k", [(8, 4), (64, 6), (256, 8)])
def test_route_ties(oracle_lib, E, k):
    rng = np.random.default_rng(11)
    lg = np.round(rng.standard_normal((40, E)) * 2).astype(np.float32) / 2   # many ties
    lg[0] = 0.0                                                              # all equal
    lg[1] = -1.0
    _check_route(oracle_lib, lg, k)
    r = oracle_lib.route(lg, k)
    assert r["ids"][0].tolist() == list(range(k))


@pytest.mark.parametrize("E,k", [(1, 1), (64, 1), (64, 6), (128, 8), (256, 8), (7, 7)])
def test_route_unnormalised(oracle_lib, E, k):
    # the selected entries of the softmax over all logits (scipy's), same ids
    # and expert map as the renormalised routing
    lg = np.random.default_rng(E + 7 * k).standard_normal((21, E)).astype(np.float32) * 2
    lg[3] = np.round(lg[3])                                      # ties
    r = oracle_lib.route(lg, k, renorm=False)
    n = oracle_lib.route(lg, k)
    for key in ("ids", "counts", "offsets", "row_list"):
        assert np.array_equal(r[key], n[key])
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(r["w"], np.take_along_axis(p, r["ids"], axis=1), rtol=1e-13, atol=0)
    if k == E:                                                   # nothing left out: both agree
        assert np.allclose(r["w"], n["w"], rtol=1e-14, atol=0)
    else:
        assert np.all(r["w"].sum(1) < 1.0)


# --------------------------------------------------- whole layer vs brute force
TINY = [
    dict(E=1, H=64, I=64, top_k=1, fc1="sym_int4"),
    dict(E=4, H=128, I=64, top_k=2, fc1="sym_int4"),
    dict(E=4, H=64, I=128, top_k=4, fc1="sym_int2", fc2="sym_int4"),
    dict(E=3, H=128, I=128, top_k=1, fc1="ternary", block1=128, scale_dtype="f16"),
    dict(E=4, H=128, I=64, top_k=2, fc1="affine_int2", fc2="affine_int4", block1=64, block2=64,
         scale_dtype="f16", act_dtype="f16"),
    dict(E=4, H=128, I=64, top_k=2, fc1="sym_int4", act_dtype="f32"),
]


@pytest.mark.parametrize("cfg", TINY, ids=lambda c: "-".join(str(v) for v in c.values()))
@pytest.mark.parametrize("T", [1, 2, 5])
def test_moe_vs_dense_bruteforce(oracle_lib, cfg, T):
    spec = custom_moe_spec(**cfg)
    inp = synth.moe_inputs(spec, T=T, seed=T)
    out = oracle_lib.moe(inp)
    ref = bf.moe_dense(inp)
    assert out["status"] == 0
    assert np.allclose(out["y64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    if spec.act_dtype == "f16":
        assert np.array_equal(out["y"], out["y64"].astype(np.float16).view(np.uint16))
    if spec.act_dtype == "f32":                                   # one RNE to f32, x read as f32
        assert out["y"].dtype == np.float32 and np.array_equal(out["y"], out["y64"].astype(np.float32))
        assert inp["x"].dtype == np.float32


@pytest.mark.parametrize("cfg", [TINY[1], TINY[2], TINY[4], TINY[5]],
                         ids=["int4-k2", "int2-int4-k4", "affine-f16", "int4-f32"])
@pytest.mark.parametrize("T", [1, 3])
def test_moe_expert_bias_vs_dense_bruteforce(oracle_lib, cfg, T):
    spec = custom_moe_spec(**cfg)
    inp = synth.moe_inputs(spec, T=T, seed=20 + T, expert_bias=0.1)
    out = oracle_lib.moe(inp)
    ref = bf.moe_dense(inp)
    assert np.allclose(out["y64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    plain = oracle_lib.moe(synth.moe_inputs(spec, T=T, seed=20 + T))["y64"]
    assert not np.allclose(out["y64"], plain)                     # the biases change the result


@pytest.mark.parametrize("cfg", [TINY[1], dict(E=6, H=64, I=128, top_k=3, fc1="sym_int2", fc2="sym_int4")],
                         ids=["int4-k2", "int2-int4-k3"])
def test_moe_unnormalised_weights_vs_dense_bruteforce(oracle_lib, cfg):
    spec = custom_moe_spec(**cfg)
    inp = synth.moe_inputs(spec, T=3, seed=31)
    out = oracle_lib.moe(inp, renorm=False)
    ref = bf.moe_dense(inp, renorm=False)
    assert np.allclose(out["y64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    assert not np.allclose(out["y64"], oracle_lib.moe(inp)["y64"])


RELU = [dict(E=4, H=128, I=128, top_k=2, fc1="sym_int4", activation="relu"),
        dict(E=3, H=128, I=256, top_k=1, fc1="ternary", block1=128, scale_dtype="f16", activation="relu")]


@pytest.mark.parametrize("cfg", RELU, ids=["int4-k2", "ternary-k1"])
@pytest.mark.parametrize("bias", [0.0, 0.1])
def test_moe_relu_ffn_vs_dense_bruteforce(oracle_lib, cfg, bias):
    spec = custom_moe_spec(**cfg)
    inp = synth.moe_inputs(spec, T=3, seed=41, expert_bias=bias)
    assert inp["fc1_codes"].shape[1] == spec.I                    # one [I][H] matrix
    out = oracle_lib.moe(inp, debug=True)
    ref = bf.moe_dense(inp)
    assert np.allclose(out["y64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(out["h"], np.maximum(out["a"], 0.0)) and np.any(out["h"] == 0.0)


def test_moe_relu_zero_weights_closed_form(oracle_lib):
    # all codes 0: a = b1, so h = max(b1, 0) and y = sum_j w_j * b2[e_j]
    spec = custom_moe_spec(E=5, H=64, I=64, top_k=2, activation="relu")
    inp = synth.moe_inputs(spec, T=3, seed=8, expert_bias=0.1)
    inp["fc1_codes"] = np.full_like(inp["fc1_codes"], 0x88)
    inp["fc2_codes"] = np.full_like(inp["fc2_codes"], 0x88)
    out = oracle_lib.moe(inp, debug=True)
    r = oracle_lib.route(inp["logits"], 2)
    b1 = bf.half_bits_to_f64(inp["fc1_expert_bias"], "bf16")
    b2 = bf.half_bits_to_f64(inp["fc2_expert_bias"], "bf16")
    assert np.array_equal(out["h"], np.maximum(b1[r["ids"].ravel()], 0.0))
    assert np.allclose(out["y64"], (r["w"][:, :, None] * b2[r["ids"]]).sum(axis=1), rtol=1e-14, atol=1e-16)


def test_moe_expert_bias_zero_weights_closed_form(oracle_lib):
    # all codes 0: FC1's output is its bias, so h = silu(b_gate) * b_up with the
    # gate in even rows, and y = sum_j w_j * b2[e_j]
    spec = custom_moe_spec(E=5, H=64, I=64, top_k=3)
    inp = synth.moe_inputs(spec, T=4, seed=3, expert_bias=0.1)
    inp["fc1_codes"] = np.full_like(inp["fc1_codes"], 0x88)
    inp["fc2_codes"] = np.full_like(inp["fc2_codes"], 0x88)
    out = oracle_lib.moe(inp, debug=True)
    r = oracle_lib.route(inp["logits"], 3)
    b1 = bf.half_bits_to_f64(inp["fc1_expert_bias"], "bf16")
    b2 = bf.half_bits_to_f64(inp["fc2_expert_bias"], "bf16")
    ids = r["ids"].ravel()
    assert np.array_equal(out["a"], b1[ids])
    g, u = b1[ids][:, 0::2], b1[ids][:, 1::2]
    assert np.allclose(out["h"], g / (1.0 + np.exp(-g)) * u, rtol=1e-14, atol=0)
    assert np.array_equal(out["o"], b2[ids])
    y = (r["w"][:, :, None] * b2[r["ids"]]).sum(axis=1)
    assert np.allclose(out["y64"], y, rtol=1e-14, atol=1e-16)


def test_moe_expert_permutation_invariance(oracle_lib):
    spec = custom_moe_spec(E=6, H=64, I=64, top_k=3)
    inp = synth.moe_inputs(spec, T=4, seed=9)
    base = oracle_lib.moe(inp)["y64"]
    perm = np.random.default_rng(0).permutation(6)
    p = dict(inp)
    for n in ("fc1_codes", "fc1_scales", "fc2_codes", "fc2_scales"):
        p[n] = inp[n][perm]
    p["logits"] = np.ascontiguousarray(inp["logits"][:, perm])
    assert np.array_equal(oracle_lib.moe(p)["y64"], base)
    tp = np.random.default_rng(1).permutation(4)
    q = dict(inp)
    q["x"] = np.ascontiguousarray(inp["x"][tp])
    q["logits"] = np.ascontiguousarray(inp["logits"][tp])
    assert np.array_equal(oracle_lib.moe(q)["y64"], base[tp])


def test_moe_token_subset_equals_full(oracle_lib):
    spec = custom_moe_spec(E=4, H=64, I=64, top_k=2)
    inp = synth.moe_inputs(spec, T=6, seed=4)
    full = oracle_lib.moe(inp)["y64"]
    sub = oracle_lib.moe(inp, tokens=[5, 1, 3])["y64"]
    assert np.array_equal(sub, full[[5, 1, 3]])


def test_ternary_invalid_field_reported(oracle_lib):
    spec = custom_moe_spec(E=1, H=128, I=128, top_k=1, fc1="ternary", block1=128, scale_dtype="f16")
    inp = synth.moe_inputs(spec, T=1, seed=0)
    assert oracle_lib.moe(inp)["status"] == 0
    inp["fc1_codes"] = inp["fc1_codes"].copy()
    inp["fc1_codes"][0, 5, 3] |= 0xC0
    assert oracle_lib.moe(inp)["status"] == -1


@pytest.mark.parametrize("fmt,block,sd,ad", [("affine_int2", 128, "f16", "f16"), ("sym_int4", 64, "bf16", "bf16"),
                                             ("ternary", 128, "f16", "bf16")])
def test_linear_vs_dense_bruteforce(oracle_lib, fmt, block, sd, ad):
    spec = custom_linear_spec(512, fmt=fmt, block=block, scale_dtype=sd, act_dtype=ad)
    inp = synth.linear_inputs(spec, 128, 5, seed=1)
    out = oracle_lib.linear(inp)
    ref = bf.linear_dense(inp)
    assert np.allclose(out["y64"], ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())
    sub = oracle_lib.linear(inp, 64, 96)
    assert np.array_equal(sub["y64"], out["y64"][:, 64:96])


# --------------------------------------------------------- page arithmetic
def test_page_byte_and_mac_counts():
    g = {c["what"]: c for c in json.load(open(os.path.join(GOLD, "page_arithmetic.json")))["cases"]}
    sp = synth.LINEAR_WORKLOADS["dense_affine2"]
    for N in sp.Ns:
        nbytes = synth.canonical_matrix_bytes(sp.fmt, N, sp.K)
        assert nbytes * 8 / (N * sp.K) == g["effective bits per weight of 2-bit affine, group 128, 16-bit scale and bias"]["value"]
    assert synth.canonical_matrix_bytes(sp.fmt, 17408, 5120) == 25067520
    mac = g["FMA per row of the 5120 -> 17408 matmul"]
    assert 5120 * 17408 == mac["exact"] and abs(mac["exact"] - mac["value_approx"]) / mac["value_approx"] < 0.01


# ------------------------------------------- fp32 vs fp64 accumulation
@pytest.mark.parametrize("name,T", [("single_expert_int4", 1), ("switch_base_ternary", 1), ("dsv2lite_int4", 2),
                                    ("mixed_int2_int4_prefill", 2)])
def test_fp32_accumulation_agrees_with_fp64(oracle_lib, name, T):
    """The layer evaluated with every sum in float (the fp32-accumulation
    reading) and in double: the same definitions in two precisions agree to
    within fp32 summation error, about sqrt(K) * 2^-24 relative for K-term
    sums of mixed signs (K <= 4096 here: below 4e-6; gate 2e-5), and their
    outputs rounded to the activation dtype differ only by rare one-ulp
    straddles, far inside the 2e-3 row tolerance."""
    from tests.metrics import compare
    spec = synth.MOE_WORKLOADS[name]
    inp = synth.moe_inputs(spec, T, 3)
    r64 = oracle_lib.moe(inp)
    r32 = oracle_lib.moe_f32acc(inp)
    assert r64["status"] == 0 and r32["status"] == 0
    y32 = r32["y32"].astype(np.float64)
    rel = np.linalg.norm(y32 - r64["y64"], axis=1) / np.linalg.norm(r64["y64"], axis=1)
    assert rel.max() < 2e-5, rel.max()
    res = compare(r32["y"], r64["y"], r64["y64"], spec.act_dtype)
    assert res["ok"] and res["frac_identical"] > 0.97, res


def test_threaded_evaluation_is_identical(oracle_lib):
    """Token subsets on several host threads give the one-thread result bit
    for bit (a token's output depends only on its own row)."""
    spec = custom_moe_spec(E=4, H=256, I=128, top_k=2, fc1="sym_int2", fc2="sym_int4")
    inp = synth.moe_inputs(spec, 37, 0)
    a = oracle_lib.moe(inp, debug=True)
    b = oracle_lib.moe(inp, debug=True, threads=5)
    for key in ("y64", "y", "a", "h", "o"):
        assert np.array_equal(a[key], b[key]), key
    sub = [3, 9, 30, 31]
    assert np.array_equal(oracle_lib.moe(inp, tokens=sub, threads=3)["y"], a["y"][sub])


# ------------------------------------------------------ configurable SwiGLU
SWIGLU_PARAMS = [(1.702, 1.0, 0.7), (0.5, -0.25, 0.0), (2.0, 0.5, 0.3)]


@pytest.mark.parametrize("params", SWIGLU_PARAMS, ids=["a1.702-b1-l0.7", "a0.5-bm0.25", "a2-b0.5-l0.3"])
def test_moe_configurable_swiglu_vs_dense_bruteforce(oracle_lib, params):
    """alpha, beta and limit against the independent float64 brute force; the
    inputs are scaled so that the limit clips a share of the gate and up values."""
    spec = custom_moe_spec(E=4, H=128, I=64, top_k=2, fc1="sym_int4")
    inp = synth.moe_inputs(spec, T=4, seed=41)
    inp["swiglu"] = params
    out = oracle_lib.moe(inp, debug=True)
    ref = bf.moe_dense(inp)
    assert np.allclose(out["y64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    assert not np.allclose(out["y64"], oracle_lib.moe(dict(inp, swiglu=None))["y64"])
    if params[2] > 0:
        a = out["a"]
        assert np.mean(np.abs(a) > params[2]) > 0.02, "the limit clips nothing"


def test_swiglu_closed_forms(oracle_lib):
    """The plain parameters reproduce silu(g) * u; u = -beta gives 0; a gate
    above the limit gives limit * sigmoid(alpha * limit) * (u + beta); a
    large alpha turns sigmoid into the step, h -> max(g, 0) * (u + beta)."""
    rng = np.random.default_rng(3)
    for g, u in rng.standard_normal((50, 2)) * 4:
        assert oracle_lib.swiglu(g, u) == oracle_lib.silu(g) * u
        assert oracle_lib.swiglu(g, -0.75, 1.3, 0.75, 0.0) == 0.0
        lim = 1.0
        if g > lim and abs(u) < lim:
            want = lim / (1.0 + np.exp(-1.702 * lim)) * (u + 1.0)
            assert abs(oracle_lib.swiglu(g, u, 1.702, 1.0, lim) - want) <= 1e-15 * abs(want) + 1e-300
        step = max(g, 0.0) * (u + 0.5)
        if abs(g) > 0.5:
            assert abs(oracle_lib.swiglu(g, u, 1e4, 0.5, 0.0) - step) <= 1e-12 * max(1.0, abs(step))
    # clipping of the up value on both sides
    assert oracle_lib.swiglu(2.0, 50.0, 1.0, 0.0, 3.0) == oracle_lib.swiglu(2.0, 3.0, 1.0, 0.0, 0.0)
    assert oracle_lib.swiglu(2.0, -50.0, 1.0, 0.0, 3.0) == oracle_lib.swiglu(2.0, -3.0, 1.0, 0.0, 0.0)


# --------------------------------------------------- gathered channels
def _transpose_fc2_to_down(inp):
    """Channel-major down projection equal to the FC2 matrix exactly: every
    FC2 scale of an expert set to that expert's first scale, the codes
    transposed and repacked along H (blocks of the FC2 block size)."""
    sp = inp["spec"]
    bits = bf.BITS[sp.fc2.fmt]
    q = bf.fields(np.asarray(inp["fc2_codes"], dtype=np.uint8), bits, sp.I)          # [E][H][I] fields
    s = np.repeat(np.asarray(inp["fc2_scales"])[:, :1, :1], sp.H, 1)
    s = np.repeat(s, sp.I // sp.fc2.block, 2)
    inp = dict(inp, fc2_scales=np.ascontiguousarray(s))
    qt = np.ascontiguousarray(np.transpose(q, (0, 2, 1)))                             # [E][I][H]
    per = 8 // bits
    packed = np.zeros(qt.shape[:2] + (sp.H // per,), dtype=np.uint8)
    for f in range(per):
        packed |= (qt[:, :, f::per] << (bits * f)).astype(np.uint8)
    ds = np.repeat(np.asarray(inp["fc2_scales"])[:, :1, :1], sp.I, 1)
    ds = np.repeat(ds, sp.H // sp.fc2.block, 2)
    inp["down_codes"], inp["down_scales"] = packed, np.ascontiguousarray(ds)
    inp["down_fmt"] = (sp.fc2.fmt, sp.fc2.block, sp.fc2.scale_dtype)
    return inp


@pytest.mark.parametrize("cfg", [dict(E=4, H=128, I=64, top_k=2, fc1="sym_int4"),
                                 dict(E=3, H=128, I=128, top_k=3, fc1="sym_int2", fc2="ternary", block2=128,
                                      scale_dtype="f16")], ids=["int4", "int2-ternary"])
def test_channels_all_selected_equal_the_full_layer(oracle_lib, cfg):
    """Every channel listed once, in order, with a down projection equal to
    FC2: the gathered layer is the full layer (same products, same order)."""
    spec = custom_moe_spec(**cfg)
    inp = _transpose_fc2_to_down(synth.moe_inputs(spec, T=3, seed=8))
    ch = np.broadcast_to(np.arange(spec.I, dtype=np.int32), (3, spec.top_k, spec.I)).copy()
    got = oracle_lib.moe_channels(inp, ch)
    ref = oracle_lib.moe(inp)
    assert np.array_equal(got["y64"], ref["y64"]) and np.array_equal(got["y"], ref["y"])


@pytest.mark.parametrize("budget", [0.05, 0.18, 0.6])
def test_channels_vs_dense_bruteforce(oracle_lib, budget):
    spec = custom_moe_spec(E=6, H=128, I=128, top_k=3, fc1="sym_int4")
    inp = synth.moe_inputs(spec, T=4, seed=9)
    inp.update(synth.channel_inputs(spec, inp, budget, seed=9))
    ch = inp["channels"]
    assert ch.shape[:2] == (4, 3) and (ch >= 0).sum() == 4 * round(budget * 3 * 128)
    got = oracle_lib.moe_channels(inp, ch)
    ref = bf.moe_channels_dense(inp, ch)
    assert np.allclose(got["y64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    # a repeated channel counts twice, an empty list gives zero
    ch2 = ch.copy()
    ch2[0, 0, :] = -1
    ch2[0, 0, 0] = ch2[0, 0, 1] = 5
    assert np.allclose(oracle_lib.moe_channels(inp, ch2)["y64"], bf.moe_channels_dense(inp, ch2),
                       rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    zero = oracle_lib.moe_channels(inp, np.full_like(ch, -1))
    assert np.all(zero["y64"] == 0.0)


# ------------------------------------------------------------ base-3 ternary
def test_base3_every_byte_value_decodes(oracle_lib):
    """All 243 valid bytes: with blocks of 5 weights (one byte per block), the
    codes are the byte's base-3 digits, least significant first, minus 1,
    against numpy's base-3 string of the value."""
    v = np.arange(243, dtype=np.uint8)
    codes, nbad = oracle_lib.unpack_codes("ternary_b3", v[None, :], 1, 5 * 243, block=5)
    assert nbad == 0
    want = np.array([[int(c) for c in np.base_repr(int(b), 3).zfill(5)[::-1]] for b in v]).reshape(-1) - 1
    assert np.array_equal(codes[0].astype(np.int64), want)


@pytest.mark.parametrize("block,limit_last", [(64, 81), (128, 27)])
def test_base3_invalid_bytes_are_flagged(oracle_lib, block, limit_last):
    """A full byte >= 243 and a block's last partial byte >= 3^(block mod 5)
    are invalid: each flags the weights it holds; the largest valid values
    are accepted."""
    per = (block + 4) // 5
    row = np.zeros((1, 2 * per), dtype=np.uint8)
    row[0, 0] = 242
    row[0, per - 1] = limit_last - 1
    assert oracle_lib.unpack_codes("ternary_b3", row, 1, 2 * block, block=block)[1] == 0
    bad = row.copy()
    bad[0, 3] = 243
    assert oracle_lib.unpack_codes("ternary_b3", bad, 1, 2 * block, block=block)[1] == 5
    bad = row.copy()
    bad[0, 2 * per - 1] = limit_last
    assert oracle_lib.unpack_codes("ternary_b3", bad, 1, 2 * block, block=block)[1] == block % 5
    spec = custom_moe_spec(E=1, H=block, I=block, top_k=1, fc1="ternary_b3", block1=block, fc2="ternary")
    inp = synth.moe_inputs(spec, T=1, seed=1)
    inp["fc1_codes"] = inp["fc1_codes"].copy()
    inp["fc1_codes"][0, 5, 0] = 255
    assert oracle_lib.moe(inp)["status"] == -1


@pytest.mark.parametrize("block", [64, 128])
def test_base3_equals_two_bit_ternary(oracle_lib, block):
    """The same digits stored in base 3 and as 2-bit ternary fields give the
    same matrix, the same layer output and the same gathered-channel output,
    bit for bit; the base-3 rows are 1.625 bits per weight."""
    spec2 = custom_moe_spec(E=4, H=640, I=128, top_k=2, fc1="ternary", fc2="ternary", block1=block)
    inp2 = synth.moe_inputs(spec2, T=3, seed=12)
    spec3 = custom_moe_spec(E=4, H=640, I=128, top_k=2, fc1="ternary_b3", fc2="ternary_b3", block1=block,
                            name="b3_of_" + spec2.name)
    inp3 = dict(inp2, spec=spec3)
    for m in ("fc1", "fc2"):
        rows, K = inp2[m + "_codes"].shape[1], (spec2.H if m == "fc1" else spec2.I)
        d = bf.fields(inp2[m + "_codes"], 2, K)
        inp3[m + "_codes"] = synth.pack_base3(d, block)
        assert inp3[m + "_codes"].shape[-1] * 8 / K == 1.625
        W2 = oracle_lib.dequant("ternary", block, "bf16", inp2[m + "_codes"][0], inp2[m + "_scales"][0], None,
                                rows, K)
        W3 = oracle_lib.dequant("ternary_b3", block, "bf16", inp3[m + "_codes"][0], inp3[m + "_scales"][0], None,
                                rows, K)
        assert np.array_equal(W2, W3)
    r2, r3 = oracle_lib.moe(inp2), oracle_lib.moe(inp3)
    assert r3["status"] == 0 and np.array_equal(r2["y64"], r3["y64"]) and np.array_equal(r2["y"], r3["y"])
    ch = synth.channel_inputs(spec2, inp2, 0.3, seed=12)
    d = bf.fields(ch["down_codes"], 2, spec2.H)
    c2 = dict(inp2, **ch)
    c3 = dict(inp3, **ch)
    c3.update(down_codes=synth.pack_base3(d, block), down_fmt=("ternary_b3", block, "bf16"))
    a, b = oracle_lib.moe_channels(c2, ch["channels"]), oracle_lib.moe_channels(c3, ch["channels"])
    assert b["status"] == 0 and np.array_equal(a["y64"], b["y64"])


def test_base3_moe_vs_dense_bruteforce(oracle_lib):
    """A base-3 layer against the independent float64 dense mixture (digits
    from numpy's base-3 strings)."""
    spec = custom_moe_spec(E=5, H=320, I=64, top_k=2, fc1="ternary_b3", fc2="ternary_b3", block1=64,
                           scale_dtype="f16")
    inp = synth.moe_inputs(spec, T=4, seed=13)
    out = oracle_lib.moe(inp)
    ref = bf.moe_dense(inp)
    assert out["status"] == 0
    assert np.max(np.abs(out["y64"] - ref)) <= 1e-12 * np.max(np.abs(ref))

"""GPU parity of the gathered-channel path (qmoe_forward_channels) against the
oracle's ``moe_channels``, within the row/element bounds of tests/metrics.py.

Inputs: ``synth.channel_inputs`` (per token, round(budget * k * I) distinct
(slot, channel) picks split at random over the k routed slots, padded with
-1) on top of the layer arrays of ``synth.moe_inputs``.
"""

import sys

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import custom_moe_spec
from tests.metrics import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import skinny_gemm_amd as q
    q.lib()
    yield


def _pack(spec, inp):
    import skinny_gemm_amd as q
    from skinny_gemm_amd.layer import to_device_bits
    dfmt, dblock, dsd = inp["down_fmt"]
    assert (dfmt, dblock, dsd) == (spec.fc2.fmt, spec.fc2.block, spec.fc2.scale_dtype)
    desc = q.layer_desc(spec.E, spec.H, spec.I, spec.act_dtype,
                        (spec.fc1.fmt, spec.fc1.block, spec.fc1.scale_dtype),
                        (spec.fc2.fmt, spec.fc2.block, spec.fc2.scale_dtype))
    packed = torch.empty(q.channel_prepacked_size(desc), dtype=torch.uint8, device="cuda")
    src = [to_device_bits(inp[k], None) for k in ("fc1_codes", "fc1_scales", "down_codes", "down_scales")]
    q.channel_prepack(desc, *src, packed)
    torch.cuda.synchronize()
    return desc, packed


def _run(desc, packed, spec, inp, channels):
    import skinny_gemm_amd as q
    from skinny_gemm_amd.layer import to_device_bits, bits_of
    T = inp["x"].shape[0]
    Cn = channels.shape[2]
    x = to_device_bits(inp["x"], spec.act_dtype)
    lg = torch.from_numpy(np.ascontiguousarray(inp["logits"], dtype=np.float32)).cuda()
    ch = torch.from_numpy(np.ascontiguousarray(channels, dtype=np.int32)).cuda()
    y = torch.empty((T, spec.H), dtype=x.dtype, device="cuda")
    ws = torch.empty(max(q.channel_workspace_size(desc, T, spec.top_k, Cn), 256), dtype=torch.uint8, device="cuda")
    q.forward_channels(desc, packed, x, lg, T, spec.top_k, ch, Cn, y, ws)
    torch.cuda.synchronize()
    return bits_of(y)


def run_case(spec, T, seed, budget, edit=None, repeat=False):
    log(f"[channels] {spec.name} T={T} seed={seed} budget={budget} edit={edit is not None}")
    inp = synth.moe_inputs(spec, T, seed)
    inp.update(synth.channel_inputs(spec, inp, budget, seed))
    channels = inp["channels"]
    if edit is not None:
        channels = edit(channels.copy(), spec)
    desc, packed = _pack(spec, inp)
    ybits = _run(desc, packed, spec, inp, channels)
    ref = oracle.moe_channels(inp, channels)
    assert ref["status"] == 0
    res = compare(ybits, ref["y"], ref["y64"], spec.act_dtype)
    log(f"       C={channels.shape[2]} y: max_row_rel={res['max_row_rel']:.3e} "
        f"identical={res['frac_identical']:.4f} vs_exact={res['max_row_rel_vs_exact']:.3e}")
    assert res["ok"], res
    if repeat:  # fixed summation order: identical bits on a second call
        assert np.array_equal(_run(desc, packed, spec, inp, channels), ybits)
    return res


@pytest.mark.parametrize("T,seed", [(1, 0), (1, 1), (4, 0), (8, 2)])
def test_channels_dsv2lite(T, seed):
    """The decode workload at an 18% channel budget."""
    run_case(synth.MOE_WORKLOADS["dsv2lite_int4"], T, seed, 0.18, repeat=(seed == 0))


@pytest.mark.parametrize("budget", [0.05, 0.5, 1.0])
def test_channels_budgets(budget):
    """From a few channels up to every channel of every routed expert (then the
    result is the full layer's)."""
    run_case(custom_moe_spec(8, 512, 256, 2), 3, 5, budget)


@pytest.mark.parametrize("fc1,fc2,block,sd,act", [
    ("sym_int2", "sym_int4", 64, "bf16", "bf16"),
    ("ternary", "ternary", 128, "f16", "f16"),
    ("sym_int4", "sym_int2", 128, "f16", "bf16"),
    ("sym_int2", "ternary", 64, "bf16", "f16"),
])
def test_channels_formats(fc1, fc2, block, sd, act):
    spec = custom_moe_spec(16, 768, 384, 4, fc1=fc1, fc2=fc2, block1=block, scale_dtype=sd, act_dtype=act)
    run_case(spec, 5, 3, 0.2)


def test_channels_wide_hidden():
    """H = 3072: three output chunks of 1024 per wave group, ragged C."""
    run_case(custom_moe_spec(8, 3072, 256, 3, fc1="sym_int2", fc2="sym_int4"), 2, 7, 0.3)


def test_channels_duplicates_and_padding():
    """A channel listed twice counts twice; -1 entries anywhere are skipped."""
    def edit(ch, spec):
        ch[:, 0, 1] = ch[:, 0, 0]           # duplicate
        ch[:, -1, 0] = -1                    # padding at the front of a list
        ch[0, :, :] = -1                     # a token with no channels at all
        return ch
    run_case(custom_moe_spec(8, 512, 256, 2), 4, 9, 0.25, edit=edit)


def test_channels_many_tokens():
    """Many tokens and groups: T = 48, k = 4."""
    run_case(custom_moe_spec(32, 512, 512, 4), 48, 11, 0.1)


def test_channels_empty_batch():
    import skinny_gemm_amd as q
    spec = custom_moe_spec(8, 512, 256, 2)
    inp = synth.moe_inputs(spec, 1, 0)
    inp.update(synth.channel_inputs(spec, inp, 0.2, 0))
    desc, packed = _pack(spec, inp)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    y = torch.empty((0, spec.H), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, spec.H), dtype=torch.bfloat16, device="cuda")
    q.forward_channels(desc, packed, x, x, 0, 2, x, 4, y, ws)  # T = 0: no device work
    torch.cuda.synchronize()


def test_channels_invalid_ternary_rejected():
    import skinny_gemm_amd as q
    from skinny_gemm_amd.layer import to_device_bits
    spec = custom_moe_spec(4, 256, 128, 1, fc1="ternary", fc2="ternary")
    inp = synth.moe_inputs(spec, 1, 0)
    inp.update(synth.channel_inputs(spec, inp, 0.2, 0))
    inp["down_codes"] = inp["down_codes"].copy()
    inp["down_codes"][1, 7, 3] = 0xFF  # four fields holding 3
    desc = q.layer_desc(spec.E, spec.H, spec.I, spec.act_dtype, ("ternary", 64, "bf16"), ("ternary", 64, "bf16"))
    packed = torch.empty(q.channel_prepacked_size(desc), dtype=torch.uint8, device="cuda")
    src = [to_device_bits(inp[k], None) for k in ("fc1_codes", "fc1_scales", "down_codes", "down_scales")]
    with pytest.raises(q.QmoeError, match="4 ternary fields"):
        q.channel_prepack(desc, *src, packed)


# ------------------------------------------------------------ base-3 rows
@pytest.mark.parametrize("H,block,sd,act,budget", [
    (640, 64, "bf16", "bf16", 0.2),
    (640, 128, "f16", "f16", 0.35),
    (768, 128, "f16", "bf16", 0.5),
    (2048, 64, "bf16", "bf16", 0.18),
    (2048, 128, "bf16", "f16", 0.1),
])
def test_channels_base3(H, block, sd, act, budget):
    """Both matrices in base-3 ternary (five weights per byte, block records
    with the scale inside) against the oracle."""
    spec = custom_moe_spec(16, H, 256, 4, fc1="ternary_b3", fc2="ternary_b3", block1=block, scale_dtype=sd,
                           act_dtype=act)
    run_case(spec, 5, 21, budget, repeat=True)


def test_channels_base3_dsv2lite_shape():
    """The decode layer's shape (E 64, k 6, H 2048, I 1408) in base 3 at the
    18% budget."""
    spec = custom_moe_spec(64, 2048, 1408, 6, fc1="ternary_b3", fc2="ternary_b3", block1=64)
    run_case(spec, 2, 22, 0.18)


def test_channels_base3_full_layer():
    """Every channel of every routed expert listed once (budget 1): the whole
    switch-shaped ternary layer from base-3 rows."""
    spec = custom_moe_spec(8, 768, 768, 1, fc1="ternary_b3", fc2="ternary_b3", block1=128, scale_dtype="f16")
    run_case(spec, 3, 23, 1.0)


def test_channels_base3_invalid_bytes_rejected():
    import skinny_gemm_amd as q
    from skinny_gemm_amd.layer import to_device_bits
    spec = custom_moe_spec(4, 640, 128, 1, fc1="ternary_b3", fc2="ternary_b3", block1=128)
    inp = synth.moe_inputs(spec, 1, 0)
    inp.update(synth.channel_inputs(spec, inp, 0.2, 0))
    inp["fc1_codes"] = inp["fc1_codes"].copy()
    inp["fc1_codes"][2, 9, 4] = 250          # a full byte >= 243
    inp["down_codes"] = inp["down_codes"].copy()
    inp["down_codes"][1, 3, 25] = 27         # a block's last byte (3 digits) >= 27
    desc = q.layer_desc(spec.E, spec.H, spec.I, spec.act_dtype, ("ternary_b3", 128, "bf16"),
                        ("ternary_b3", 128, "bf16"))
    packed = torch.empty(q.channel_prepacked_size(desc), dtype=torch.uint8, device="cuda")
    src = [to_device_bits(inp[k], None) for k in ("fc1_codes", "fc1_scales", "down_codes", "down_scales")]
    with pytest.raises(q.QmoeError, match="2 base-3 bytes"):
        q.channel_prepack(desc, *src, packed)


@pytest.mark.parametrize("fmt", ["sym_int4", "ternary_b3"])
def test_channels_many_experts_and_top16(fmt):
    """E = 128 (the routing wave then takes two logits per lane and the k
    rounds of arg-max instead of the per-lane rank count) and top-16 routing,
    for 16-bit and base-3 rows."""
    run_case(custom_moe_spec(128, 640, 128, 16, fc1=fmt, fc2=fmt, block1=128), 3, 31, 0.15)
    run_case(custom_moe_spec(256, 512, 128, 4, fc1=fmt, fc2=fmt, block1=128), 2, 32, 0.3)

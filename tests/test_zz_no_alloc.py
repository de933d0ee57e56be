"""The no-allocation forward entry point (qmoe_forward_noalloc) against
qmoe_forward with a caller workspace, through the C ABI: the same kernels on
the same inputs give the same bits, on two calls in a row of which the second
has fewer tokens (the fixed scratch keeps the first call's contents)."""

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import custom_moe_spec
from tests.metrics import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _pair(spec, T, seed):
    import skinny_gemm_amd as q
    from skinny_gemm_amd.layer import MoeLayer, to_device_bits, bits_of
    inp = synth.moe_inputs(spec, T, seed)
    layer = MoeLayer.from_spec(spec, inp)
    x = to_device_bits(inp["x"], spec.act_dtype)
    lg = torch.from_numpy(inp["logits"]).cuda()
    y_ref = torch.empty((T, spec.H), dtype=x.dtype, device="cuda")
    ws = layer.workspace(T, spec.top_k)
    q.forward(layer.desc, layer.packed, x, lg, T, spec.top_k, y_ref, ws)
    y = torch.full((T, spec.H), float("nan"), dtype=x.dtype, device="cuda")
    q.forward_noalloc(layer.desc, layer.packed, x, lg, T, spec.top_k, y)
    torch.cuda.synchronize()
    return inp, bits_of(y), bits_of(y_ref)


@pytest.mark.parametrize("spec,Ts", [
    (custom_moe_spec(E=8, H=256, I=128, top_k=2, fc1="sym_int2", fc2="sym_int4"), (40, 5)),   # grouped, then GEMV
    (synth.MOE_WORKLOADS["dsv2lite_int4"], (8, 3)),                                           # routing kernels, then small
    (custom_moe_spec(E=4, H=128, I=128, top_k=2, fc1="sym_int4", act_dtype="f32"), (20, 2)),  # f32: GEMV row tiles
], ids=["mixed-grouped-then-gemv", "dsv2lite-decode", "f32-row-tiles"])
def test_noalloc_matches_forward_on_two_calls(spec, Ts):
    for i, T in enumerate(Ts):
        inp, y, y_ref = _pair(spec, T, 200 + i)
        print(f"[noalloc] {spec.name} T={T}", flush=True)
        assert np.array_equal(y, y_ref), f"call {i} (T={T}) differs from qmoe_forward"
        ref = oracle.moe(inp)
        res = compare(y, ref["y"], ref["y64"], spec.act_dtype)
        assert res["ok"], res


def test_noalloc_rejects_a_call_beyond_the_scratch():
    import skinny_gemm_amd as q
    spec = synth.MOE_WORKLOADS["mixed_int2_int4_prefill"]
    d = q.layer_desc(spec.E, spec.H, spec.I, spec.act_dtype, (spec.fc1.fmt, spec.fc1.block, spec.fc1.scale_dtype),
                     (spec.fc2.fmt, spec.fc2.block, spec.fc2.scale_dtype))
    need = q.forward_plan(d, 2048, spec.top_k)["workspace_bytes"]
    assert need > q.NOALLOC_SCRATCH_BYTES
    fake = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QmoeError) as ei:
        q.forward_noalloc(d, fake, fake, fake, 2048, spec.top_k, fake)
    assert ei.value.status == 3 and "scratch" in str(ei.value)

"""Host-only checks of the C ABI (no GPU): the library loads, exports every
symbol the header declares, and rejects invalid calls before any launch."""

import ctypes as C
import os
import re

import pytest

import skinny_gemm_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(q.LIB_PATH), reason="libqmoe.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = q.lib()
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(q.exported_symbols())


def test_abi_version():
    assert q.abi_version() == 9


def _desc(**kw):
    d = dict(E=64, H=2048, I=1408, act="bf16", fc1=("sym_int4", 64, "bf16"), fc2=("sym_int4", 64, "bf16"))
    d.update(kw)
    return q.layer_desc(d["E"], d["H"], d["I"], d["act"], d["fc1"], d["fc2"])


def test_prepacked_size_matches_layout():
    d = _desc()
    n = q.prepacked_size(d)
    # header + per expert: codes + scales, each rounded to 256 bytes, then the
    # per-expert power-of-two pre-scales of the MFMA path (2 x E floats)
    fc1 = 2816 * 2048 // 2 + 2816 * 32 * 2
    fc2 = 2048 * 1408 // 2 + 2048 * 22 * 2
    r = lambda v: (v + 255) // 256 * 256
    assert n == (256 + 64 * (r(2816 * 1024) + r(2816 * 32 * 2)) + 64 * (r(2048 * 704) + r(2048 * 22 * 2))
                 + r(2 * 64 * 4))
    assert n >= 64 * (fc1 + fc2)


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), 1), (dict(E=257), 2),
    (dict(fc1=("sym_int4", 32, "bf16")), 2), (dict(fc1=("sym_int4", 96, "bf16")), 2),
    (dict(H=2000), 2), (dict(I=1400), 2),
    (dict(fc1=("sym_int4", 64, "f32")), 2),
])
def test_invalid_layer_rejected(kw, status):
    d = _desc(**kw)
    with pytest.raises(q.QmoeError) as ei:
        q.prepacked_size(d)
    assert ei.value.status == status, q.last_error()


def test_shape_mismatch_rejected():
    d = _desc()
    d.fc1.rows = 2048
    with pytest.raises(q.QmoeError) as ei:
        q.prepacked_size(d)
    assert ei.value.status == 1
    d = _desc()
    d.fc2.reserved = 1
    with pytest.raises(q.QmoeError):
        q.prepacked_size(d)


@pytest.mark.parametrize("T,k,status", [(-1, 1, 1), (1, 0, 1), (1, 65, 1), (4, 17, 2)])
def test_invalid_tokens_rejected(T, k, status):
    with pytest.raises(q.QmoeError) as ei:
        q.workspace_size(_desc(), T, k)
    assert ei.value.status == status


def test_forward_validation_before_launch():
    d = _desc()
    L = q.lib()
    fake = C.c_void_p(0x100000)  # never dereferenced: every case fails validation first
    ws_need = q.forward_plan(d, 4, 6)["workspace_bytes"]  # what this call's path needs
    # null pointers
    st = L.qmoe_forward(C.byref(d), None, fake, fake, 4, 6, fake, fake, ws_need, None)
    assert st == 1
    # misaligned workspace
    st = L.qmoe_forward(C.byref(d), fake, fake, fake, 4, 6, fake, C.c_void_p(0x100010), ws_need, None)
    assert st == 1
    # workspace too small
    st = L.qmoe_forward(C.byref(d), fake, fake, fake, 4, 6, fake, fake, ws_need - 1, None)
    assert st == 3
    # GEMV path forced beyond 16 rows
    opts = q.ForwardOpts(q.PATH["gemv"], 0, None, None, None, None, None, 0, 0)
    st = L.qmoe_forward_ex(C.byref(d), fake, fake, fake, 17, 6, fake, fake, 1 << 40, None, C.byref(opts))
    assert st == 2
    # T = 0 is a no-op even with null pointers
    assert L.qmoe_forward(C.byref(d), None, None, None, 0, 6, None, None, 0, None) == 0
    # unknown routing-weight mode, nonzero reserved field
    for bad in (dict(topk_weights=2), dict(topk_weights=-1), dict(reserved3=1)):
        opts = q.ForwardOpts(0, 0, None, None, None, None, None, 0, 0, None, None, 0, 0)
        for k, v in bad.items():
            setattr(opts, k, v)
        st = L.qmoe_forward_ex(C.byref(d), fake, fake, fake, 4, 6, fake, fake, ws_need, None, C.byref(opts))
        assert st == 1, bad


def test_prepack_validation():
    d = _desc(fc1=("affine_int2", 128, "f16"))
    L = q.lib()
    fake = C.c_void_p(0x100000)
    n = q.prepacked_size(d)
    # affine fc1 without biases
    assert L.qmoe_prepack(C.byref(d), fake, fake, None, fake, fake, None, fake, n, None) == 1
    # symmetric fc2 with biases
    assert L.qmoe_prepack(C.byref(d), fake, fake, fake, fake, fake, fake, fake, n, None) == 1
    # destination too small
    assert L.qmoe_prepack(C.byref(d), fake, fake, fake, fake, fake, None, fake, n - 1, None) == 3


def test_plan_gemv_decode():
    # up to 64 routed slots: FC1 routes the tokens itself
    p = q.forward_plan(_desc(), 1, 6)
    assert p["path"] == 1 and p["gemv_mmax"] == 1 and p["max_active"] == 6
    # one token, k > 1: FC2 over the six experts' concatenated K writes y
    assert p["kernels"] == ["route_fc1_swiglu", "gemv_fc2_combine"]
    assert p["num_launches"] == 2
    p1 = q.forward_plan(_desc(), 1, 1)
    assert p1["kernels"] == ["route_fc1_swiglu", "gemv_fc2"] and p1["num_launches"] == 2
    p2 = q.forward_plan(_desc(), 2, 6)
    assert p2["kernels"] == ["route_fc1_swiglu", "gemv_fc2", "combine"]
    # more slots: a routing kernel first
    p8 = q.forward_plan(_desc(), 8, 6)
    assert p8["gemv_mmax"] == 8 and p8["max_active"] == 48
    assert p8["kernels"] == ["route", "gemv_fc1_swiglu", "gemv_fc2", "combine"] and p8["num_launches"] == 4
    p16 = q.forward_plan(_desc(), 16, 1)
    assert p16["kernels"] == ["route_fc1_swiglu", "gemv_fc2"]
    p3 = q.forward_plan(_desc(), 3, 6)
    assert p3["gemv_mmax"] == 3
    p0 = q.forward_plan(_desc(), 0, 6)
    assert p0["num_launches"] == 0 and p0["kernels"] == []


def test_route_validation():
    L = q.lib()
    n = C.c_size_t()
    assert L.qmoe_route_workspace_size(8, 300, 2, C.byref(n)) == 2
    assert L.qmoe_route_workspace_size(8, 64, 65, C.byref(n)) == 1
    assert L.qmoe_route_workspace_size(8, 64, 6, C.byref(n)) == 0 and n.value > 0


def test_linear_validation():
    d = q.qmatrix_desc("affine_int2", 128, "f16", 17408, 5120)
    assert q.linear_prepacked_size(d) > 25067520
    L = q.lib()
    fake = C.c_void_p(0x100000)
    assert L.qmoe_linear(C.byref(d), fake, fake, 2, 4, fake, None, 0, 0, None) == 2   # f32 x
    assert L.qmoe_linear(C.byref(d), fake, fake, 1, 0, fake, None, 0, 0, None) == 0   # M = 0 no-op
    assert L.qmoe_linear(C.byref(d), None, fake, 1, 4, fake, None, 0, 0, None) == 1
    bad = q.qmatrix_desc("affine_int2", 128, "f16", 17400, 5120)
    with pytest.raises(q.QmoeError):
        q.linear_prepacked_size(bad)


def test_plan_grouped_prefill():
    d = q.layer_desc(128, 4096, 1536, "bf16", ("sym_int2", 64, "bf16"), ("sym_int4", 64, "bf16"))
    p = q.forward_plan(d, 2048, 8)
    assert p["path"] == 2
    assert p["kernels"] == ["route", "rowscale", "grouped_fc1_swiglu", "split_h", "grouped_fc2", "combine"]
    assert p["num_launches"] == 9  # top-k, count, expand, place, rowscale, FC1, split h, FC2, combine
    pg = q.forward_plan(_desc(), 4, 6, path="grouped")
    assert pg["path"] == 2 and pg["num_launches"] == 6
    assert q.workspace_size(d, 2048, 8) >= p["workspace_bytes"]


def test_plan_softmax_all_weights_stage():
    """The unnormalised routing weights come from the routing top-k itself:
    the same stages and launches as the renormalised default."""
    d = _desc()
    for T, k, path in [(1, 6, "auto"), (8, 6, "auto"), (1, 1, "auto"), (64, 6, "auto")]:
        base = q.forward_plan(d, T, k, path)
        p = q.forward_plan(d, T, k, path, topk_weights="softmax_all")
        assert p["kernels"] == base["kernels"] and p["num_launches"] == base["num_launches"], (T, k)


def _mixed_desc():
    return _desc(E=128, H=4096, I=1536, fc1=("sym_int2", 64, "bf16"), fc2=("sym_int4", 64, "bf16"))


@pytest.mark.parametrize("T,div", [(8193, 3), (8193, 40), (2048, 5), (37, 2)])
def test_plan_row_tiling_halves_until_the_tile_fits(T, div):
    d = _mixed_desc()
    full = q.forward_plan(d, T, 8)
    limit = full["workspace_bytes"] // div
    p = q.forward_plan(d, T, 8, workspace_limit=limit)
    R = T
    while True:                                      # the halving sequence, rounding up
        tiles = -(-T // R)
        last = T - (tiles - 1) * R
        need = max(q.forward_plan(d, n, 8)["workspace_bytes"] for n in {R, last})
        if need <= limit:
            break
        R = (R + 1) // 2
    assert (p["row_tile"], p["num_tiles"], p["workspace_bytes"]) == (R, tiles, need)
    assert p["workspace_bytes"] <= limit < full["workspace_bytes"]
    per = {n: q.forward_plan(d, n, 8)["num_launches"] for n in {R, last}}
    assert p["num_launches"] == (tiles - 1) * per[R] + per[last]


def test_plan_row_tiling_edges():
    d = _mixed_desc()
    big = q.forward_plan(d, 100, 8)
    p = q.forward_plan(d, 100, 8, workspace_limit=big["workspace_bytes"])       # fits: one tile
    assert (p["row_tile"], p["num_tiles"]) == (100, 1) and p["workspace_bytes"] == big["workspace_bytes"]
    with pytest.raises(q.QmoeError) as ei:                                       # not even one row
        q.forward_plan(d, 100, 8, workspace_limit=1)
    assert ei.value.status == 3
    with pytest.raises(q.QmoeError) as ei:
        q.forward_plan(d, 100, 8, workspace_limit=-1)
    assert ei.value.status == 1


def test_forward_row_tiling_validation_before_launch():
    d = _mixed_desc()
    L = q.lib()
    fake = C.c_void_p(0x100000)  # never dereferenced: every case fails validation first
    limit = q.forward_plan(d, 4096, 8)["workspace_bytes"] // 3
    tile_ws = q.forward_plan(d, 4096, 8, workspace_limit=limit)["workspace_bytes"]

    def call(ws_bytes, **kw):
        o = q.ForwardOpts(0, 0, None, None, None, None, None, 0, 0, None, None, 0, 0, limit)
        for k, v in kw.items():
            setattr(o, k, v)
        return L.qmoe_forward_ex(C.byref(d), fake, fake, fake, 4096, 8, fake, fake, ws_bytes, None, C.byref(o))
    assert call(tile_ws, counts_out=0x100000) == 2                               # counts need one tile
    assert call(tile_ws, num_events=2, events=C.cast(fake, C.POINTER(C.c_void_p))) == 2
    assert call(tile_ws - 1) == 3                                                # workspace of a tile
    o = q.ForwardOpts(0, 0, None, None, None, None, None, 0, 0, None, None, 0, 0, limit)
    assert L.qmoe_forward_ex(C.byref(d), None, fake, fake, 4096, 8, fake, fake, tile_ws, None, C.byref(o)) == 1


def test_prepack_scales_validation():
    L = q.lib()
    fake = C.c_void_p(0x100000)
    d = _desc()
    need = q.prepacked_size(d)
    assert L.qmoe_prepack_scales(C.byref(d), None, None, fake, None, fake, need, None) == 1       # null scales
    assert L.qmoe_prepack_scales(C.byref(d), fake, fake, fake, None, fake, need, None) == 1       # bias, symmetric
    assert L.qmoe_prepack_scales(C.byref(d), fake, None, fake, None, C.c_void_p(0x100010), need, None) == 1
    assert L.qmoe_prepack_scales(C.byref(d), fake, None, fake, None, fake, need - 1, None) == 3
    da = _desc(fc1=("affine_int2", 128, "f16"))
    assert L.qmoe_prepack_scales(C.byref(da), fake, None, fake, None, fake, q.prepacked_size(da), None) == 1


def test_plan_f32_activations():
    """f32 activations: on the GEMV path a split pass first and y from the
    combine (also for top-1); above 16 tokens the grouped path, whose FC1
    stages the fp32 rows itself after a row-maximum pass."""
    d = _desc(act="f32")
    assert q.forward_plan(d, 1, 6)["kernels"] == ["split_x", "route_fc1_swiglu", "gemv_fc2", "combine"]
    assert q.forward_plan(d, 8, 6)["kernels"] == ["split_x", "route", "gemv_fc1_swiglu", "gemv_fc2", "combine"]
    p1 = q.forward_plan(d, 1, 1)
    assert p1["kernels"] == ["split_x", "route_fc1_swiglu", "gemv_fc2", "combine"] and p1["num_launches"] == 4
    b = q.forward_plan(_desc(), 4, 6)["workspace_bytes"]
    assert q.forward_plan(d, 4, 6)["workspace_bytes"] == b + 2 * (4 * 2048 * 2)   # x hi + lo rows
    g4 = q.forward_plan(d, 4, 6, "grouped")
    assert g4["kernels"] == ["route", "rowscale", "grouped_fc1_swiglu", "split_h", "grouped_fc2", "combine"]
    p17 = q.forward_plan(d, 17, 6)          # the grouped path in one pass
    assert (p17["num_tiles"], p17["path"]) == (1, 2)
    L = q.lib()
    fake = C.c_void_p(0x100000)
    o = q.ForwardOpts(0, 0, None, None, None, None, None, 0, 0, fake, None, 0, 0, 0)   # expert bias
    assert L.qmoe_forward_ex(C.byref(d), fake, fake, fake, 4, 6, fake, fake, 1 << 30, None, C.byref(o)) == 2


def test_relu_layer_descriptor_and_plan():
    d = q.layer_desc(64, 768, 3072, "bf16", ("ternary", 128, "f16"), ("ternary", 128, "f16"), "relu")
    assert d.fc1.rows == 3072
    sw = q.layer_desc(64, 768, 3072, "bf16", ("ternary", 128, "f16"), ("ternary", 128, "f16"))
    assert q.prepacked_size(d) < q.prepacked_size(sw)              # FC1 half the rows
    assert q.forward_plan(d, 1, 1)["kernels"] == ["route_fc1_relu", "gemv_fc2"]
    assert q.forward_plan(d, 9, 2)["kernels"] == ["route", "gemv_fc1_relu", "gemv_fc2", "combine"]
    assert q.forward_plan(d, 64, 2)["kernels"] == ["route", "rowscale", "grouped_fc1_relu", "split_h", "grouped_fc2",
                                                   "combine"]
    bad = q.layer_desc(64, 768, 3072, "bf16", ("ternary", 128, "f16"), ("ternary", 128, "f16"), "relu")
    bad.fc1.rows = 2 * 3072                                         # SwiGLU-shaped FC1 with ReLU
    bad2 = q.layer_desc(64, 768, 3072, "bf16", ("ternary", 128, "f16"), ("ternary", 128, "f16"))
    bad2.activation = 7
    bad3 = q.layer_desc(64, 768, 3072, "bf16", ("ternary", 128, "f16"), ("ternary", 128, "f16"))
    bad3.reserved = 1
    for b in (bad, bad2, bad3):
        with pytest.raises(q.QmoeError) as ei:
            q.prepacked_size(b)
        assert ei.value.status == 1, q.last_error()


def test_row_tiling_reaches_the_gemv_path():
    """A layer the grouped kernels cannot take (an affine format with more
    than 80 blocks per row) runs above 16 rows in GEMV-path tiles of at most
    16 rows, with or without a workspace limit; a call pinned to the GEMV path
    does so only under a workspace limit."""
    aff = q.layer_desc(8, 6144, 256, "bf16", ("affine_int2", 64, "f16"), ("affine_int2", 64, "f16"))
    for lim in (0, 1 << 40):
        p = q.forward_plan(aff, 40, 2, workspace_limit=lim)
        assert (p["row_tile"], p["num_tiles"], p["path"]) == (10, 4, 1)
    pa = q.forward_plan(aff, 100, 2)
    assert pa["path"] == 1 and pa["row_tile"] <= 16 and pa["num_tiles"] * pa["row_tile"] >= 100
    with pytest.raises(q.QmoeError) as ei:
        q.forward_plan(aff, 100, 2, "grouped")
    assert ei.value.status == 2
    # a grouped-capable layer keeps one pass on the grouped path
    assert q.forward_plan(_desc(), 100, 6)["num_tiles"] == 1
    with pytest.raises(q.QmoeError) as ei:
        q.forward_plan(_desc(), 100, 6, path="gemv")
    assert ei.value.status == 2
    g = q.forward_plan(_desc(), 100, 6, path="gemv", workspace_limit=1 << 40)
    assert g["row_tile"] <= 16 and g["path"] == 1
    # a workspace limit alone never turns a supported grouped call into GEMV tiles
    big = q.forward_plan(_desc(), 100, 6)["workspace_bytes"]
    t = q.forward_plan(_desc(), 100, 6, workspace_limit=big // 2)
    assert t["num_tiles"] >= 2 and t["path"] == 2

def test_noalloc_rejects_beyond_scratch_before_any_launch():
    """qmoe_forward_noalloc checks the workspace against its fixed scratch on
    the host: the 2048-token mixed prefill needs more and is refused without
    touching the device (fake pointers)."""
    d = q.layer_desc(128, 4096, 1536, "bf16", ("sym_int2", 64, "bf16"), ("sym_int4", 64, "bf16"))
    L = q.lib()
    fake = C.c_void_p(0x100000)
    assert q.forward_plan(d, 2048, 8)["workspace_bytes"] > q.NOALLOC_SCRATCH_BYTES
    assert L.qmoe_forward_noalloc(C.byref(d), fake, fake, fake, 2048, 8, fake, None) == 3
    assert "scratch" in q.last_error()
    assert L.qmoe_forward_noalloc(C.byref(d), fake, fake, fake, -1, 8, fake, None) == 1
    assert L.qmoe_forward_noalloc(C.byref(d), fake, fake, fake, 0, 8, fake, None) == 0


def test_swiglu_parameters_validated_before_launch():
    d = _desc()
    L = q.lib()
    fake = C.c_void_p(0x100000)

    def opts(flag, a, b, lim):
        o = q.ForwardOpts()
        o.swiglu_params, o.swiglu_alpha, o.swiglu_beta, o.swiglu_limit = flag, a, b, lim
        return o
    for o in (opts(2, 1.0, 0.0, 0.0), opts(1, float("nan"), 0.0, 0.0), opts(1, 1.0, float("inf"), 0.0),
              opts(1, 1.0, 0.0, -1.0)):
        assert L.qmoe_forward_ex(C.byref(d), fake, fake, fake, 4, 6, fake, fake, 1 << 30, None, C.byref(o)) == 1
    relu = q.layer_desc(64, 768, 3072, "bf16", ("ternary", 128, "f16"), ("ternary", 128, "f16"), "relu")
    o = opts(1, 1.702, 1.0, 7.0)
    assert L.qmoe_forward_ex(C.byref(relu), fake, fake, fake, 4, 1, fake, fake, 1 << 30, None, C.byref(o)) == 1
    assert "SWIGLU" in q.last_error()


def test_channel_calls_validate_before_launch():
    """Gathered channels: unsupported layers and bad list lengths fail on the
    host; sizes follow the layout (FC1 rows and the channel-major down rows)."""
    ok = q.layer_desc(64, 2048, 1408, "bf16", ("sym_int4", 64, "bf16"), ("sym_int4", 64, "bf16"))
    n = q.channel_prepacked_size(ok)
    assert n >= 256 + 64 * 2816 * 1024 + 64 * 2816 * 32 * 2 + 64 * 1408 * 1024 + 64 * 1408 * 32 * 2
    ws = q.channel_workspace_size(ok, 4, 6, 300)
    groups = (6 * 300 + 15) // 16
    assert ws >= 4 * groups * 2048 * 4  # fp32 partial sums per token and group of 16 entries
    for bad in [q.layer_desc(8, 512, 256, "bf16", ("affine_int2", 64, "f16"), ("sym_int4", 64, "bf16")),
                q.layer_desc(8, 512, 256, "f32", ("sym_int4", 64, "bf16"), ("sym_int4", 64, "bf16")),
                q.layer_desc(8, 512, 256, "bf16", ("sym_int4", 64, "bf16"), ("sym_int4", 64, "bf16"), "relu"),
                q.layer_desc(8, 4160, 256, "bf16", ("sym_int4", 64, "bf16"), ("sym_int4", 64, "bf16"))]:
        with pytest.raises(q.QmoeError) as ei:
            q.channel_prepacked_size(bad)
        assert ei.value.status == 2  # unsupported
    for Cn in (0, 65537):
        with pytest.raises(q.QmoeError, match="list length"):
            q.channel_workspace_size(ok, 1, 6, Cn)
    st = q.lib().qmoe_forward_channels(C.byref(ok), None, None, None, 1, 6, None, 8, None, None, 0, None)
    assert st != 0 and "null" in q.last_error()


def test_base3_rows_only_on_the_channel_calls():
    """TERNARY_B3 layers: the MoE and dense calls refuse them, the channel
    calls take them when both matrices are base 3 and H <= 2048; the packed
    rows are block records (16 bytes per 64 weights, 28 per 128)."""
    b3 = q.layer_desc(8, 2048, 256, "bf16", ("ternary_b3", 128, "bf16"), ("ternary_b3", 64, "bf16"))
    for fn in (lambda: q.prepacked_size(b3), lambda: q.workspace_size(b3, 1, 2),
               lambda: q.linear_prepacked_size(q.qmatrix_desc("ternary_b3", 128, "f16", 64, 640))):
        with pytest.raises(q.QmoeError) as ei:
            fn()
        assert ei.value.status == 2
    n = q.channel_prepacked_size(b3)
    fc1 = 8 * 512 * 16 * 28          # 16 records of 28 B per FC1 row
    dn = 8 * 256 * 32 * 16           # 32 records of 16 B per down row
    assert fc1 + dn + 256 <= n <= fc1 + dn + 256 + 3 * 256
    mixed = q.layer_desc(8, 2048, 256, "bf16", ("ternary_b3", 128, "bf16"), ("ternary", 128, "bf16"))
    wide = q.layer_desc(8, 4096, 256, "bf16", ("ternary_b3", 128, "bf16"), ("ternary_b3", 128, "bf16"))
    for d in (mixed, wide):
        with pytest.raises(q.QmoeError) as ei:
            q.channel_prepacked_size(d)
        assert ei.value.status == 2

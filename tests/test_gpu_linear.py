"""GPU parity of the dense skinny-M quantized matmul (HIP kernels through the
C ABI) against the oracle."""

import os
import sys

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import custom_linear_spec
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


_cache = {}


def _layer(spec, N, seed):
    from skinny_gemm_amd.layer import QLinear
    key = (spec.name, N, seed)
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        w = synth.linear_inputs(spec, N, 1, seed)
        f = spec.fmt
        _cache[key] = (w, QLinear(f.fmt, f.block, f.scale_dtype, N, spec.K, w["codes"], w["scales"], w["biases"]))
    return _cache[key]


# host threads for the oracle (the GPU machine's CPU share is 16 cores)
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_rows_parallel(inp, N, chunk=8192):
    """oracle.linear over all N rows in chunks on ORACLE_THREADS host threads
    (the C call releases the GIL; each chunk is its own row range)."""
    from concurrent.futures import ThreadPoolExecutor
    spans = [(n0, min(N, n0 + chunk)) for n0 in range(0, N, chunk)]
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        parts = list(ex.map(lambda sp: oracle.linear(inp, sp[0], sp[1]), spans))
    return {"y": np.concatenate([p["y"] for p in parts], axis=1),
            "y64": np.concatenate([p["y64"] for p in parts], axis=1)}


def run_linear(spec, N, M, seed=0, rows=None, path="auto"):
    from skinny_gemm_amd.layer import to_device_bits, bits_of
    log(f"[linear] {spec.name} N={N} M={M} seed={seed} path={path}")
    w, lin = _layer(spec, N, seed)
    inp = synth.linear_inputs(spec, N, M, seed, weights=False)
    inp.update(codes=w["codes"], scales=w["scales"], biases=w["biases"])
    x = to_device_bits(inp["x"], spec.act_dtype)
    y = lin(x, spec.act_dtype, path=path)
    torch.cuda.synchronize()
    yb = bits_of(y)
    slices = rows or [(0, N)]
    worst = None
    for n0, n1 in slices:
        ref = oracle.linear(inp, n0, n1)
        res = compare(yb[:, n0:n1], ref["y"], ref["y64"], spec.act_dtype)
        assert res["ok"], (n0, n1, res)
        worst = res if worst is None or res["max_row_rel"] > worst["max_row_rel"] else worst
    log(f"       max_row_rel={worst['max_row_rel']:.3e} identical={worst['frac_identical']:.4f}")
    return worst


DENSE = synth.LINEAR_WORKLOADS["dense_affine2"]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 10, 16])
def test_dense_affine2_17408(M):
    run_linear(DENSE, 17408, M)


@pytest.mark.parametrize("M", [1, 3, 16])
def test_dense_affine2_248320_sampled_rows(M):
    N = 248320
    run_linear(DENSE, N, M, rows=[(0, 512), (123904, 124416), (N - 512, N)])


@pytest.mark.parametrize("fmt,block,sd,ad", [
    ("sym_int4", 64, "bf16", "bf16"), ("sym_int2", 64, "bf16", "f16"), ("ternary", 128, "f16", "bf16"),
    ("affine_int4", 128, "bf16", "f16"), ("affine_int2", 64, "bf16", "bf16")])
@pytest.mark.parametrize("M", [1, 7, 16])
def test_linear_sweep(fmt, block, sd, ad, M):
    spec = custom_linear_spec(1024, fmt=fmt, block=block, scale_dtype=sd, act_dtype=ad)
    run_linear(spec, 320, M, seed=M)


@pytest.mark.parametrize("fmt", ["sym_int4", "sym_int2", "ternary", "affine_int2", "affine_int4"])
@pytest.mark.parametrize("ad", ["bf16", "f16"])
def test_unit_scale_integer_inputs_bit_exact(fmt, ad):
    """All-one scales and small integer activations: every product and partial
    sum is an exact integer in fp32, so the GPU must equal the oracle bit for
    bit (all-one-scale codes reproduce a dense integer matmul)."""
    from skinny_gemm_amd.layer import QLinear, to_device_bits, bits_of
    K, N, M = 512, 128, 5
    spec = custom_linear_spec(K, fmt=fmt, block=64, scale_dtype="bf16", act_dtype=ad)
    inp = synth.linear_inputs(spec, N, M, seed=3)
    inp["scales"][:] = 0x3F80
    if inp["biases"] is not None:
        inp["biases"][:] = 0xC000
    xi = np.random.default_rng(1).integers(-8, 9, size=(M, K)).astype(np.float64)
    inp["x"] = oracle.double_to_half(xi, ad).reshape(M, K)
    lin = QLinear(fmt, 64, "bf16", N, K, inp["codes"], inp["scales"], inp["biases"])
    y = lin(to_device_bits(inp["x"], ad), ad)
    torch.cuda.synchronize()
    ref = oracle.linear(inp)
    assert np.array_equal(bits_of(y), ref["y"])


@pytest.mark.parametrize("N", [17408, 248320])
def test_dense_unpack_bit_exact(N):
    w, lin = _layer(DENSE, N, 0)
    got = lin.unpack().cpu().numpy()
    sl = slice(0, N) if N < 100000 else slice(N - 4096, N)
    ref, nbad = oracle.unpack_codes("affine_int2", w["codes"][sl], got[sl].shape[0], DENSE.K)
    assert nbad == 0 and np.array_equal(got[sl], ref)


@pytest.mark.parametrize("M", [17, 32, 64])
def test_dense_affine2_17408_mfma(M):
    run_linear(DENSE, 17408, M)


@pytest.mark.parametrize("M", [1, 4])
def test_dense_affine2_248320_all_rows(M):
    """The 248320-row matrix compared on every output row (the oracle in
    parallel row chunks)."""
    from skinny_gemm_amd.layer import to_device_bits, bits_of
    N = 248320
    log(f"[linear] all rows N={N} M={M} threads={ORACLE_THREADS}")
    w, lin = _layer(DENSE, N, 0)
    inp = synth.linear_inputs(DENSE, N, M, 0, weights=False)
    inp.update(codes=w["codes"], scales=w["scales"], biases=w["biases"])
    y = lin(to_device_bits(inp["x"], DENSE.act_dtype), DENSE.act_dtype)
    torch.cuda.synchronize()
    ref = oracle_rows_parallel(inp, N)
    res = compare(bits_of(y), ref["y"], ref["y64"], DENSE.act_dtype)
    log(f"       max_row_rel={res['max_row_rel']:.3e} identical={res['frac_identical']:.4f}")
    assert res["ok"], res


def test_dense_affine2_248320_m32_sampled_rows():
    N = 248320
    run_linear(DENSE, N, 32, rows=[(0, 512), (123904, 124416), (N - 512, N)])


@pytest.mark.parametrize("fmt,block,sd,ad", [
    ("sym_int4", 64, "bf16", "bf16"), ("sym_int2", 64, "bf16", "f16"), ("ternary", 128, "f16", "bf16"),
    ("affine_int4", 128, "bf16", "f16"), ("affine_int2", 64, "bf16", "bf16")])
@pytest.mark.parametrize("M", [1, 7, 40])
def test_linear_sweep_mfma(fmt, block, sd, ad, M):
    spec = custom_linear_spec(1024, fmt=fmt, block=block, scale_dtype=sd, act_dtype=ad)
    run_linear(spec, 320, M, seed=M + 50, path="grouped")

#!/usr/bin/env python3
"""Benchmark of the low-bit quantized MoE expert FFN on one MI355X.

A step is one MoE layer forward (route -> expand -> fused gate/up SwiGLU ->
down projection -> top-k combine) over one batch of synthetic tokens, through
the C ABI.  The default workload is the Switch-base-shaped ternary layer (64
experts, hidden 768, intermediate 3072, top-1, batch-1 decode).

Method (the MLX issue's repro times medians of 5 trials after warm calls):
  * the expert weights rotate over enough distinct prepacked copies (>= 1 GiB)
    that every step reads its experts from HBM, not from the 256 MB MALL;
    with top-1 routing the selected expert cycles through every expert of
    every copy before it repeats;
  * the K timed steps are captured once in a HIP graph (no host launch gaps)
    and replayed 5 times; ms_per_step is the median replay / K;
  * per-stage durations come from HIP events the library records around each
    stage on the launch stream, over K eager steps;
  * value = effective weight-read bandwidth: bytes of the experts each step
    touches (codes + scales) / time per step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
METRIC = "µs per MoE layer and effective weight-read HBM GB/s vs peak, tokens/expert M=1..32"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600,
                    help="timed steps; 600 x 1.9 MB of experts per step > 1 GiB per replay")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="switch_base_ternary")
    ap.add_argument("--tokens", type=int, default=0, help="tokens per step (default: the workload's first)")
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-extras", action="store_true", help="skip the M-sweep / other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration under rocprofv3)")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers
def expert_bytes(spec) -> int:
    import synth
    return (synth.canonical_matrix_bytes(spec.fc1, spec.fc1_rows, spec.H)
            + synth.canonical_matrix_bytes(spec.fc2, spec.H, spec.I))


def fc1_bytes(spec) -> int:
    import synth
    return synth.canonical_matrix_bytes(spec.fc1, spec.fc1_rows, spec.H)


def targeted_logits(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Swap each row's largest logit into column `targets[row]` (keeps the
    row's values, so each row is still a permutation of N(0,1) draws)."""
    lg = logits.copy()
    am = lg.argmax(1)
    r = np.arange(lg.shape[0])
    a, b = lg[r, am].copy(), lg[r, targets].copy()
    lg[r, targets], lg[r, am] = a, b
    return lg


def graph_time(run_steps, K, trials, check=None):
    """Capture run_steps() (K steps) in a HIP graph; median replay time / K (ms)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_steps()  # warm on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_steps()
    torch.cuda.synchronize()
    times = []
    for _ in range(trials):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / K)
        if check is not None:
            check()
    return statistics.median(times), times


# Sources that define the GEMV kernels and their launch shape: the counter
# figures in profiles/traffic.json stay valid while these are unchanged.
GEMV_SOURCES = ("abi.hip", "codec.hpp", "combine.hip", "gemv_impl.hpp", "qmoe_internal.h", "route_impl.hpp",
                "gemv_sym_int4.hip", "gemv_sym_int2.hip", "gemv_ternary.hip", "gemv_affine_int2.hip",
                "gemv_affine_int4.hip")


def src_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "skinny_gemm_amd", "csrc")
    for f in GEMV_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ MoE stepping
def make_layers(spec, rotate_bytes, seed=0):
    """Distinct prepacked weight copies totalling >= rotate_bytes."""
    import synth
    from skinny_gemm_amd.layer import MoeLayer
    layer_bytes = spec.E * expert_bytes(spec)
    L = max(1, math.ceil(rotate_bytes / layer_bytes))
    log(f"[bench] {spec.name}: {L} weight copies x {layer_bytes / 1e6:.1f} MB")
    t0 = time.time()
    layers, inp0 = [], None
    for c in range(L):
        inp = synth.moe_inputs(spec, 1, seed, weight_copy=c)
        if c == 0:
            inp0 = inp
        layers.append(MoeLayer.from_spec(spec, inp))
        del inp
    log(f"[bench] generated + prepacked in {time.time() - t0:.1f}s")
    return layers, inp0


class MoeBench:
    def __init__(self, spec, T, K, W, layers, inp0, seed=0, targeted=True):
        import torch
        import synth
        from skinny_gemm_amd.layer import to_device_bits
        self.spec, self.T, self.K, self.W = spec, T, K, W
        self.layers, self.inp0 = layers, inp0
        self.L = len(layers)
        n = K + W
        steps = synth.moe_inputs(spec, T * n, seed + 1, weights=False)
        lg = steps["logits"]
        if targeted and spec.top_k == 1:
            s = np.repeat(np.arange(n), T)
            t = np.tile(np.arange(T), n)
            tgt = ((s // self.L) * T + t) % spec.E
            lg = targeted_logits(lg, tgt)
        self.x_np = steps["x"].reshape(n, T, spec.H)
        self.lg_np = lg.reshape(n, T, spec.E)
        self.x = to_device_bits(steps["x"], spec.act_dtype).view(n, T, spec.H)
        self.lg = torch.from_numpy(np.ascontiguousarray(lg)).cuda().view(n, T, spec.E)
        self.y = torch.empty((T, spec.H), dtype=self.x.dtype, device="cuda")
        self.ws = self.layers[0].workspace(T, spec.top_k)
        self.kw = {}  # forward options of every step (the variants)

    def step(self, s, **kw):
        self.layers[s % self.L].forward(self.x[s], self.lg[s], self.spec.top_k, y=self.y, ws=self.ws,
                                        **self.kw, **kw)

    def run(self):
        for s in range(self.W, self.W + self.K):
            self.step(s)

    def time_graph(self, trials):
        import torch
        for s in range(self.W):
            self.step(s)
        torch.cuda.synchronize()
        self.step(self.W + self.K - 1)
        torch.cuda.synchronize()
        ref = self.y.clone()
        mismatch = []

        def check():
            if not torch.equal(self.y.view(torch.int16), ref.view(torch.int16)):
                mismatch.append(1)
        ms, all_ms = graph_time(self.run, self.K, trials, check)
        if mismatch:
            raise RuntimeError("graph replay output differs from the eager output")
        return ms, all_ms

    def touched(self):
        """Distinct experts routed per timed step (from the GPU's own counts)."""
        import torch
        from skinny_gemm_amd import forward_ex
        cnt = torch.empty((self.K, self.spec.E), dtype=torch.int32, device="cuda")
        for i, s in enumerate(range(self.W, self.W + self.K)):
            lay = self.layers[s % self.L]
            forward_ex(lay.desc, lay.packed, self.x[s], self.lg[s], self.T, self.spec.top_k, self.y, self.ws,
                       counts_out=cnt[i])
        torch.cuda.synchronize()
        return (cnt > 0).sum(1).cpu().numpy()

    def stage_names(self):
        """Stage list of the plan the forward call follows (one kernel each)."""
        from skinny_gemm_amd import forward_plan
        lay = self.layers[0]
        return forward_plan(lay.desc, self.T, self.spec.top_k)["kernels"]

    def stage_times(self, chunk=64):
        """Average duration (ms) of each plan stage over the K steps, from events
        recorded on the launch stream around every stage.  Each chunk of steps is
        queued behind a GPU sleep so the stages run back to back, as in the graph,
        instead of waiting on the host between launches."""
        import torch
        nst = len(self.stage_names())
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)] for _ in range(self.K)]
        for row in evs:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1 << 20)
        b.record()
        torch.cuda.synchronize()
        # Enough sleep to cover the host's enqueue of one chunk (~40 us per step).
        cycles = int((1 << 20) * max(1.0, chunk * 0.04 / max(a.elapsed_time(b), 1e-3)))
        steps = list(range(self.W, self.W + self.K))
        for c0 in range(0, self.K, chunk):
            torch.cuda._sleep(cycles)
            for i in range(c0, min(self.K, c0 + chunk)):
                self.step(steps[i], events=[e.cuda_event for e in evs[i]])
        torch.cuda.synchronize()
        out = np.zeros(nst)
        for row in evs:
            for j in range(nst):
                out[j] += row[2 * j].elapsed_time(row[2 * j + 1])
        return out / self.K


def bench_moe(spec, T, K, W, trials, layers, inp0, stages=True):
    b = MoeBench(spec, T, K, W, layers, inp0)
    ms, all_ms = b.time_graph(trials)
    touched = b.touched()
    wbytes = float(touched.mean()) * expert_bytes(spec)
    res = {"workload": spec.name, "T": T, "top_k": spec.top_k, "us_per_layer": ms * 1e3,
           "trials_us": [t * 1e3 for t in all_ms], "weight_copies": b.L,
           "experts_touched_per_step": float(touched.mean()),
           "weight_bytes_per_step": wbytes, "effective_GBps": wbytes / (ms * 1e-3) / 1e9}
    res["frac_of_hbm_peak"] = res["effective_GBps"] / HBM_PEAK_GBS
    if stages:
        st = b.stage_times()
        res["stage_us"] = dict(zip(b.stage_names(), (st * 1e3).tolist()))
        res["fc1_bytes_per_launch"] = float(touched.mean()) * fc1_bytes(spec)
    return res, b


# ---------------------------------------------------------------- dense
def bench_linear(spec, N, Ms, K_steps, trials, rotate_bytes, seed=0):
    import torch
    import synth
    from skinny_gemm_amd.layer import QLinear, to_device_bits
    wbytes = synth.canonical_matrix_bytes(spec.fmt, N, spec.K)
    L = max(1, math.ceil(rotate_bytes / wbytes))
    log(f"[bench] {spec.name} N={N}: {L} weight copies x {wbytes / 1e6:.1f} MB")
    lins = []
    for c in range(L):
        w = synth.linear_inputs(spec, N, 1, seed, weight_copy=c)
        f = spec.fmt
        lins.append(QLinear(f.fmt, f.block, f.scale_dtype, N, spec.K, w["codes"], w["scales"], w["biases"]))
        del w
    out = []
    for M in Ms:
        x = to_device_bits(synth.linear_inputs(spec, N, M, seed, weights=False)["x"], spec.act_dtype)
        y = torch.empty((M, N), dtype=x.dtype, device="cuda")
        ws = lins[0].workspace(M)

        def run():
            for i in range(K_steps):
                lins[i % L](x, spec.act_dtype, y=y, ws=ws)
        ms, _ = graph_time(run, K_steps, trials)
        out.append({"M": M, "us": ms * 1e3, "effective_GBps": wbytes / (ms * 1e-3) / 1e9})
        log(f"[bench]   M={M}: {ms * 1e3:.2f} us  {wbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
    t1 = out[0]["us"]
    for r in out:
        r["x_M1"] = r["us"] / t1
    return {"workload": f"{spec.name}[N={N}]", "weight_bytes": wbytes, "copies": L, "sweep": out}


# ----------------------------------------------------------- CPU baseline
def variant_times(b: "MoeBench", trials: int, inp_seed: int = 0) -> dict:
    """The same timed steps with per-expert FC1/FC2 output biases, then with
    unnormalised top-k weights (us per layer, graph replays)."""
    import synth
    from skinny_gemm_amd.layer import to_device_bits
    out = {}
    eb = synth.moe_inputs(b.spec, 1, inp_seed, weights=False, expert_bias=0.1)
    b1, b2 = to_device_bits(eb["fc1_expert_bias"]), to_device_bits(eb["fc2_expert_bias"])
    for lay in b.layers:
        lay.fc1_bias, lay.fc2_bias = b1, b2
    out["expert_bias_us"] = b.time_graph(trials)[0] * 1e3
    for lay in b.layers:
        lay.fc1_bias = lay.fc2_bias = None
    b.kw = {"topk_weights": "softmax_all"}
    out["softmax_all_weights_us"] = b.time_graph(trials)[0] * 1e3
    b.kw = {}
    return out


def runtime_scales_time(layer, inp, reps: int = 20) -> dict:
    """qmoe_prepack_scales on one prepacked layer, canonical scales resident."""
    import torch
    from skinny_gemm_amd import prepack_scales
    from skinny_gemm_amd.layer import to_device_bits
    dev = {k: to_device_bits(inp[k]) for k in ("fc1_scales", "fc1_biases", "fc2_scales", "fc2_biases")}
    args = (layer.desc, dev["fc1_scales"], dev["fc1_biases"], dev["fc2_scales"], dev["fc2_biases"], layer.packed)
    for _ in range(3):
        prepack_scales(*args)
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        prepack_scales(*args)
    e.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(e) * 1e3 / reps
    nbytes = sum(v.numel() * v.element_size() for v in dev.values() if v is not None)
    return {"us": us, "canonical_scale_bytes": nbytes, "read_GBps": nbytes / (us * 1e-6) / 1e9}


def tiled_prefill_time(layer, spec, T: int, div: int, reps: int = 3) -> dict:
    """One T-token prefill call untiled and row-tiled under 1/div of the
    untiled workspace (ms per call, event-timed)."""
    import torch
    import synth
    from skinny_gemm_amd import forward_plan
    from skinny_gemm_amd.layer import to_device_bits
    inp = synth.moe_inputs(spec, T, 5, weights=False)
    x = to_device_bits(inp["x"], spec.act_dtype)
    lg = torch.from_numpy(inp["logits"]).cuda()
    y = torch.empty((T, spec.H), dtype=x.dtype, device="cuda")
    full = forward_plan(layer.desc, T, spec.top_k)
    limit = full["workspace_bytes"] // div
    tiled = forward_plan(layer.desc, T, spec.top_k, workspace_limit=limit)
    res = {"T": T, "workspace_untiled": full["workspace_bytes"], "workspace_limit": limit,
           "workspace_tiled": tiled["workspace_bytes"], "row_tile": tiled["row_tile"], "tiles": tiled["num_tiles"]}
    for name, lim, nbytes in (("untiled_ms", 0, full["workspace_bytes"]), ("tiled_ms", limit, tiled["workspace_bytes"])):
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        layer.forward(x, lg, spec.top_k, y=y, ws=ws, workspace_limit=lim)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            layer.forward(x, lg, spec.top_k, y=y, ws=ws, workspace_limit=lim)
        e.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(e) / reps
        del ws
    return res


def cpu_baseline(b: "MoeBench", seconds: float):
    import oracle
    spec = b.spec
    inp = dict(b.inp0)
    n = 0
    t0 = time.perf_counter()
    elapsed = 0.0
    touched = 0
    while n < b.K + b.W and elapsed < seconds:
        inp["x"] = b.x_np[n]
        inp["logits"] = b.lg_np[n]
        r = oracle.route(inp["logits"], spec.top_k)
        touched += int((r["counts"] > 0).sum())
        oracle.moe(inp)
        n += 1
        elapsed = time.perf_counter() - t0
    per = elapsed / n
    gbs = touched / n * expert_bytes(spec) / per / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "us_per_layer": per * 1e6,
            "sample": f"{n} layer calls of {spec.name} (T={b.T}) on one host core, "
                      f"double-precision oracle, {elapsed:.1f}s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import skinny_gemm_amd
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    skinny_gemm_amd.lib()
    torch.cuda.set_device(0)
    spec = synth.MOE_WORKLOADS[args.workload]
    T = args.tokens or spec.tokens[0]

    layers, inp0 = make_layers(spec, args.rotate_bytes)
    head, b = bench_moe(spec, T, args.steps, args.warmup, args.trials, layers, inp0)
    log(f"[bench] {json.dumps(head)}")
    fc1_stage = next(n for n in head["stage_us"] if "fc1" in n)
    fc1_us = head["stage_us"][fc1_stage]
    achieved = head["fc1_bytes_per_launch"] / (fc1_us * 1e-6) / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        tr = json.load(open(tpath))
        ent = tr.get(f"{spec.name}:T{T}")
        if ent and ent.get("src_hash") == src_hash():
            traffic = ent.get("bytes_per_launch")
    line = {
        "metric": METRIC,
        "value": head["effective_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_layer"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 codes, scales, activations and logits)",
        "config": {"workload": spec.name, "tokens": T, "experts": spec.E, "top_k": spec.top_k,
                   "hidden": spec.H, "intermediate": spec.I, "weights": spec.fc1.fmt,
                   "block": spec.fc1.block, "us_per_layer": round(head["us_per_layer"], 3),
                   "frac_of_hbm_peak": head["frac_of_hbm_peak"], "weight_copies": head["weight_copies"]},
        "roofline": {"bound": "hbm", "kernel": fc1_stage, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "avg_launch_us": fc1_us,
                     "algorithmic_bytes_per_launch": head["fc1_bytes_per_launch"]},
        "stage_us": head["stage_us"],
    }
    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    variants = {}
    if not args.no_extras:
        variants[f"{spec.name}_T{T}"] = {"base_us": head["us_per_layer"], **variant_times(b, 3)}
        log(f"[bench] variants {json.dumps(variants)}")
    del b, layers
    torch.cuda.empty_cache()
    if not args.no_extras:
        # the same layer with the Switch Transformer's own ReLU FFN (FC1 one [I][H] matrix)
        import dataclasses
        rspec = dataclasses.replace(spec, activation="relu", name=spec.name + "_relu")
        layr, ir = make_layers(rspec, args.rotate_bytes)
        r, bb = bench_moe(rspec, T, args.steps, args.warmup, 3, layr, ir)
        variants[f"{rspec.name}_T{T}"] = {k: r[k] for k in ("us_per_layer", "effective_GBps", "stage_us")}
        log(f"[bench] variants {json.dumps(variants)}")
        del bb, layr
        torch.cuda.empty_cache()
        extras = {}
        d3 = synth.MOE_WORKLOADS["dsv2lite_int4"]
        extras["dsv2lite_int4"] = []
        lay3, i3 = make_layers(d3, args.rotate_bytes)
        for t in d3.tokens:
            r, bb = bench_moe(d3, t, 100, 10, 3, lay3, i3, stages=True)
            extras["dsv2lite_int4"].append({k: r[k] for k in ("T", "us_per_layer", "effective_GBps",
                                                              "frac_of_hbm_peak", "experts_touched_per_step",
                                                              "stage_us")})
            log(f"[bench] {json.dumps(extras['dsv2lite_int4'][-1])}")
            if t == 1:
                variants[f"{d3.name}_T1"] = {"base_us": r["us_per_layer"], **variant_times(bb, 3)}
                log(f"[bench] variants {json.dumps(variants)}")
            del bb
        variants[f"runtime_scales_{d3.name}"] = runtime_scales_time(lay3[0], i3)
        # f32 activations over the same prepacked weights (the packed buffer
        # does not depend on the activation dtype; only the descriptor does)
        import copy
        import dataclasses
        from skinny_gemm_amd import layer_desc
        d3f = dataclasses.replace(d3, act_dtype="f32", name=d3.name + "_f32")
        lay3f = []
        for lay in lay3:
            c = copy.copy(lay)
            c.act_dtype = "f32"
            c.desc = layer_desc(d3.E, d3.H, d3.I, "f32", (d3.fc1.fmt, d3.fc1.block, d3.fc1.scale_dtype),
                                (d3.fc2.fmt, d3.fc2.block, d3.fc2.scale_dtype))
            lay3f.append(c)
        for t in (1, 8):
            r, bb = bench_moe(d3f, t, 100, 10, 3, lay3f, i3, stages=False)
            base = next(x["us_per_layer"] for x in extras["dsv2lite_int4"] if x["T"] == t)
            variants[f"{d3.name}_T{t}_f32_activations"] = {"us": r["us_per_layer"], "bf16_us": base}
            del bb
        del lay3f
        log(f"[bench] variants {json.dumps(variants)}")
        del lay3
        torch.cuda.empty_cache()
        s1 = synth.MOE_WORKLOADS["single_expert_int4"]
        lay1, i1 = make_layers(s1, args.rotate_bytes)
        r, bb = bench_moe(s1, 1, len(lay1), 20, 3, lay1, i1)
        extras["single_expert_int4"] = {k: r[k] for k in ("us_per_layer", "effective_GBps", "stage_us")}
        log(f"[bench] {json.dumps(extras['single_expert_int4'])}")
        del bb, lay1
        torch.cuda.empty_cache()
        pf = synth.MOE_WORKLOADS["mixed_int2_int4_prefill"]
        layp, ip = make_layers(pf, 1.0)  # 880 MB per copy: already 3.4x the MALL
        r, bb = bench_moe(pf, 2048, 10, 2, 3, layp, ip)
        flops = 2.0 * 2048 * pf.top_k * (2 * pf.I * pf.H + pf.H * pf.I)
        r["tflops"] = flops / (r["us_per_layer"] * 1e-6) / 1e12
        extras["mixed_int2_int4_prefill"] = {k: r[k] for k in ("us_per_layer", "effective_GBps", "tflops",
                                                               "stage_us", "experts_touched_per_step")}
        log(f"[bench] {json.dumps(extras['mixed_int2_int4_prefill'])}")
        del bb
        torch.cuda.empty_cache()
        variants[f"{pf.name}_row_tiling"] = tiled_prefill_time(layp[0], pf, 8193, 3)
        log(f"[bench] variants {json.dumps(variants)}")
        del layp
        torch.cuda.empty_cache()
        dense = synth.LINEAR_WORKLOADS["dense_affine2"]
        extras["dense_affine2"] = [bench_linear(dense, N, [1, 2, 3, 4, 5, 8, 10, 16, 32], 50, 3, args.rotate_bytes)
                                   for N in dense.Ns]
        # The expert GEMV at M=1 with all 64 DeepSeek-V2-Lite-shaped experts
        # active (one row each): the gate/up matrices of the 64 experts read
        # as one [64 * 2816][2048] INT4 matrix by the same MFMA GEMV kernel
        # family (196 MB of weights per launch).
        from synth.workloads import custom_linear_spec
        d3 = synth.MOE_WORKLOADS["dsv2lite_int4"]
        allx = custom_linear_spec(d3.H, fmt=d3.fc1.fmt, block=d3.fc1.block, scale_dtype=d3.fc1.scale_dtype,
                                  act_dtype=d3.act_dtype)
        r = bench_linear(allx, d3.E * 2 * d3.I, [1, 2, 4, 8, 16], 20, 3, args.rotate_bytes)
        r["workload"] = f"dsv2lite_fc1_all{d3.E}_experts_as_dense[N={d3.E * 2 * d3.I},K={d3.H}]"
        extras["expert_gemv_all_experts_m1"] = r
        log(f"[bench] {json.dumps(r)}")
        extras["variants"] = variants
        line["extras"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

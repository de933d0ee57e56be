#!/usr/bin/env python3
"""Benchmark of the low-bit quantized MoE expert FFN on one MI355X.

A step is one MoE layer forward (route -> expand -> fused gate/up SwiGLU ->
down projection -> top-k combine) over one batch of synthetic tokens, through
the C ABI.  The headline workload is the largest single-GPU one: the mixed
INT2/INT4 prefill layer (128 experts, top-8, hidden 4096, intermediate 1536,
2048 tokens, skewed routing), 880.8 MB of expert weights and 618.5 GFLOP per
layer.

Method (the MLX issue's repro times medians of 5 trials after warm calls):
  * the expert weights rotate over distinct prepacked copies, and every graph
    replay touches at least --rotate-bytes (1 GiB) of distinct weights,
    whatever --steps says: the timed steps are max(--steps, the count that
    reaches that footprint), so the weights come from HBM, not from the
    256 MB MALL; with top-1 routing the selected expert cycles through every
    expert of every copy before it repeats;
  * the timed steps are captured once in a HIP graph (no host launch gaps)
    and replayed --trials times; ms_per_step is the median replay / steps;
  * per-stage durations come from the kernels' own dispatch timestamps (HIP
    events stamped by hipExtLaunchKernel), over the same steps run eagerly;
  * value = effective weight-read bandwidth: bytes of the experts each step
    touches (codes + scales) / time per step.  The roofline object reports
    the dominant kernel against its own bound (MFMA for the grouped prefill
    kernels, HBM for the decode GEMVs).
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
MFMA_F16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
METRIC = "µs per MoE layer and effective weight-read HBM GB/s vs peak, tokens/expert M=1..32"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps (raised until one replay touches --rotate-bytes of distinct weights)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixed_int2_int4_prefill")
    ap.add_argument("--tokens", type=int, default=0, help="tokens per step (default: the workload's first)")
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-extras", action="store_true", help="skip the decode, M-sweep and dense workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall seconds of the all-cores oracle sample (plus about 6 s on one core)")
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


def layer_flops(spec, T) -> dict:
    """Algorithmic flops of one layer call: 2 per multiply-add of FC1 and FC2
    over every routed slot."""
    S = T * spec.top_k
    return {"fc1": 2.0 * S * spec.fc1_rows * spec.H, "fc2": 2.0 * S * spec.H * spec.I}


def expected_touched(spec, T) -> float:
    """Expected distinct experts per step with i.i.d. logits (top-1 steps are
    targeted at distinct experts)."""
    if spec.top_k == 1:
        return float(min(T, spec.E))
    return spec.E * (1.0 - (1.0 - spec.top_k / spec.E) ** T)


def targeted_logits(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Swap each row's largest logit into column `targets[row]` (keeps the
    row's values, so each row is still a permutation of N(0,1) draws)."""
    lg = logits.copy()
    am = lg.argmax(1)
    r = np.arange(lg.shape[0])
    a, b = lg[r, am].copy(), lg[r, targets].copy()
    lg[r, targets], lg[r, am] = a, b
    return lg


def covering_logits(T: int, E: int, k: int, seed: int = 0) -> np.ndarray:
    """Logits whose top-k of token t are experts (t*k + j) mod E, j = 0..k-1,
    in that order (values 8 - j/2 above N(0,1) draws): T*k >= E slots cover
    every expert with one or two rows."""
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for t in range(T):
        for j in range(k):
            lg[t, (t * k + j) % E] = 8.0 - 0.5 * j
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
    for _ in range(2):  # untimed replays: clocks and caches settle before the trials
        g.replay()
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


def src_hash() -> str:
    """Hash of every kernel and host source of the library: stored counter
    figures (profiles/*.json) are used only while it matches."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "skinny_gemm_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "include", "qmoe.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def stored_profile(key: str):
    """Entry `key` of profiles/counters.json if it was taken with the current
    sources (else None)."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    ent = json.load(open(p)).get(key)
    if ent and ent.get("src_hash") == src_hash():
        return ent
    return None


# ------------------------------------------------------------ MoE stepping
def make_layers(spec, rotate_bytes, seed=0, min_copies=1):
    """Distinct prepacked weight copies totalling >= rotate_bytes."""
    import synth
    from skinny_gemm_amd.layer import MoeLayer
    layer_bytes = spec.E * expert_bytes(spec)
    L = max(min_copies, math.ceil(rotate_bytes / layer_bytes))
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
    """K timed steps (after W warm steps) of one workload over rotating
    weight copies; inputs come from a pool of distinct batches."""

    def __init__(self, spec, T, K, W, layers, inp0, seed=0, targeted=True, logits_mode="iid",
                 fixed_logits=None, pool_bytes=64 << 20):
        import torch
        import synth
        from skinny_gemm_amd.layer import to_device_bits
        self.spec, self.T, self.K, self.W = spec, T, K, W
        self.layers, self.inp0 = layers, inp0
        self.L = len(layers)
        n = K + W
        act_bytes = 4 if spec.act_dtype == "f32" else 2
        self.P = max(1, min(n, pool_bytes // max(1, T * spec.H * act_bytes)))  # distinct input batches
        steps = synth.moe_inputs(spec, T * self.P, seed + 1, logits_mode, weights=False)
        lg = steps["logits"]
        if fixed_logits is not None:
            lg = np.tile(fixed_logits, (self.P, 1))
        elif targeted and spec.top_k == 1 and logits_mode == "iid":
            s = np.repeat(np.arange(self.P), T)
            t = np.tile(np.arange(T), self.P)
            tgt = ((s // self.L) * T + t) % spec.E
            lg = targeted_logits(lg, tgt)
        self.x_np = steps["x"].reshape(self.P, T, spec.H)
        self.lg_np = lg.reshape(self.P, T, spec.E)
        self.x = to_device_bits(steps["x"], spec.act_dtype).view(self.P, T, spec.H)
        self.lg = torch.from_numpy(np.ascontiguousarray(lg)).cuda().view(self.P, T, spec.E)
        self.y = torch.empty((T, spec.H), dtype=self.x.dtype, device="cuda")
        self.ws = self.layers[0].workspace(T, spec.top_k)
        self.kw = {}  # forward options of every step (the variants)

    def step(self, s, **kw):
        self.layers[s % self.L].forward(self.x[s % self.P], self.lg[s % self.P], self.spec.top_k, y=self.y,
                                        ws=self.ws, **self.kw, **kw)

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
        """Distinct experts routed per timed step and distinct (copy, expert)
        pairs per replay (from the GPU's own counts)."""
        import torch
        from skinny_gemm_amd import forward_ex
        cnt = torch.empty((self.K, self.spec.E), dtype=torch.int32, device="cuda")
        for i, s in enumerate(range(self.W, self.W + self.K)):
            lay = self.layers[s % self.L]
            forward_ex(lay.desc, lay.packed, self.x[s % self.P], self.lg[s % self.P], self.T, self.spec.top_k,
                       self.y, self.ws, counts_out=cnt[i])
        torch.cuda.synchronize()
        c = (cnt > 0).cpu().numpy()
        per_step = c.sum(1)
        distinct = set()
        for i, s in enumerate(range(self.W, self.W + self.K)):
            for e in np.nonzero(c[i])[0]:
                distinct.add((s % self.L, int(e)))
        return per_step, len(distinct)

    def stage_names(self):
        """Stage list of the plan the forward call follows (one kernel each)."""
        from skinny_gemm_amd import forward_plan
        lay = self.layers[0]
        return forward_plan(lay.desc, self.T, self.spec.top_k)["kernels"]

    def stage_times(self, chunk=64):
        """Average duration (ms) of each plan stage over the K steps, from the
        dispatch timestamps of its kernels.  Each chunk of steps is queued
        behind a GPU sleep so the stages run back to back, as in the graph,
        instead of waiting on the host between launches; the same steps run
        once untimed right before the timed ones, so the clocks have left the
        sleep's idle state when the timed kernels start."""
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
        # Enough sleep to cover the host's enqueue of two chunks (~40 us per step).
        cycles = int((1 << 20) * max(1.0, 2 * chunk * 0.04 / max(a.elapsed_time(b), 1e-3)))
        steps = list(range(self.W, self.W + self.K))
        for c0 in range(0, self.K, chunk):
            torch.cuda._sleep(cycles)
            for i in range(c0, min(self.K, c0 + chunk)):
                self.step(steps[i])
            for i in range(c0, min(self.K, c0 + chunk)):
                self.step(steps[i], events=[e.cuda_event for e in evs[i]])
        torch.cuda.synchronize()
        out = np.zeros(nst)
        for row in evs:
            for j in range(nst):
                out[j] += row[2 * j].elapsed_time(row[2 * j + 1])
        return out / self.K


def timed_steps(spec, T, K, rotate_bytes, experts_per_step):
    """Steps per replay: at least K, and enough to touch rotate_bytes of
    distinct expert weights (experts per step x expert bytes)."""
    per_step = experts_per_step * expert_bytes(spec)
    return max(K, math.ceil(rotate_bytes / per_step))


def bench_moe(spec, T, K, W, trials, layers, inp0, stages=True, rotate_bytes=float(1 << 30),
              logits_mode="iid", fixed_logits=None, stage_steps=64):
    """Graph-replay timing of one workload; per-stage times over the first
    `stage_steps` steps run eagerly."""
    if fixed_logits is not None:
        eps = float(len(np.unique(np.argsort(-fixed_logits, 1, kind="stable")[:, :spec.top_k])))
    elif logits_mode == "shared":
        eps = float(spec.top_k)
    else:
        eps = expected_touched(spec, T)
    Ke = timed_steps(spec, T, K, rotate_bytes, eps)
    b = MoeBench(spec, T, Ke, W, layers, inp0, logits_mode=logits_mode, fixed_logits=fixed_logits)
    ms, all_ms = b.time_graph(trials)
    touched, distinct = b.touched()
    wbytes = float(touched.mean()) * expert_bytes(spec)
    res = {"workload": spec.name, "T": T, "top_k": spec.top_k, "us_per_layer": ms * 1e3,
           "trials_us": [t * 1e3 for t in all_ms], "steps": Ke, "weight_copies": b.L,
           "experts_touched_per_step": float(touched.mean()),
           "distinct_weight_bytes_per_replay": distinct * expert_bytes(spec),
           "weight_bytes_per_step": wbytes, "effective_GBps": wbytes / (ms * 1e-3) / 1e9}
    res["frac_of_hbm_peak"] = res["effective_GBps"] / HBM_PEAK_GBS
    if stages:
        K0, b.K = b.K, min(b.K, stage_steps)
        st = b.stage_times()
        b.K = K0
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
    K_steps = max(K_steps, L)  # every replay reads every copy
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
    return {"workload": f"{spec.name}[N={N}]", "weight_bytes": wbytes, "copies": L, "steps": K_steps,
            "sweep": out}


def read_ceiling(nbytes=1 << 30, reps=20) -> dict:
    """The library's streaming-read probe over a buffer 4x the MALL."""
    import torch
    from skinny_gemm_amd import read_probe
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        read_probe(src, sink)
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        read_probe(src, sink)
    e.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(e) * 1e3 / reps
    del src
    return {"bytes": nbytes, "us": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


# ------------------------------------------------------------- variants
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


# ----------------------------------------------------------- CPU baseline
def channel_decode_time(spec, T: int, budget: float, K: int = 32, trials: int = 5,
                        rotate_bytes: float = float(1 << 30), seed: int = 0) -> dict:
    """Gathered-channel calls (qmoe_forward_channels) at a per-token channel
    budget: graph-replay time per call over rotating channel-packed weight
    copies and distinct input batches, and the bytes of the listed FC1 rows
    and down rows (with their scales) each call reads."""
    import torch
    import synth
    import skinny_gemm_amd as q
    from skinny_gemm_amd.layer import to_device_bits
    desc = q.layer_desc(spec.E, spec.H, spec.I, spec.act_dtype, (spec.fc1.fmt, spec.fc1.block, spec.fc1.scale_dtype),
                        (spec.fc2.fmt, spec.fc2.block, spec.fc2.scale_dtype))
    size = q.channel_prepacked_size(desc)
    L = max(2, math.ceil(rotate_bytes / size))
    packs = []
    for c in range(L):
        inp = synth.moe_inputs(spec, 1, seed, weight_copy=c)
        inp.update(synth.channel_inputs(spec, inp, budget, seed))
        pk = torch.empty(size, dtype=torch.uint8, device="cuda")
        src = [to_device_bits(inp[k], None) for k in ("fc1_codes", "fc1_scales", "down_codes", "down_scales")]
        q.channel_prepack(desc, *src, pk)
        torch.cuda.synchronize()
        packs.append(pk)
        del src, inp
    P = K
    steps = synth.moe_inputs(spec, T * P, seed + 1, weights=False)
    ch = synth.channel_inputs(spec, steps, budget, seed + 1)["channels"]
    Cn = ch.shape[2]
    x = to_device_bits(steps["x"], spec.act_dtype).view(P, T, spec.H)
    lg = torch.from_numpy(np.ascontiguousarray(steps["logits"])).cuda().view(P, T, spec.E)
    chd = torch.from_numpy(ch).cuda().view(P, T, spec.top_k, Cn)
    y = torch.empty((T, spec.H), dtype=x.dtype, device="cuda")
    ws = torch.empty(q.channel_workspace_size(desc, T, spec.top_k, Cn), dtype=torch.uint8, device="cuda")

    def step(s):
        q.forward_channels(desc, packs[s % L], x[s % P], lg[s % P], T, spec.top_k, chd[s % P], Cn, y, ws)

    step(K - 1)
    torch.cuda.synchronize()
    ref = y.clone()
    bad = []

    def check():
        if not torch.equal(y.view(torch.int16), ref.view(torch.int16)):
            bad.append(1)
    ms, all_ms = graph_time(lambda: [step(s) for s in range(K)], K, trials, check)
    if bad:
        raise RuntimeError("graph replay output differs from the eager output")
    listed = float((ch >= 0).sum()) / P  # listed (slot, channel) entries per call
    # per listed entry: the gate and up rows of FC1 and one down row, [H] each
    nbytes = listed * (synth.canonical_matrix_bytes(spec.fc1, 2, spec.H)
                       + synth.canonical_matrix_bytes(spec.fc2, 1, spec.H))
    us = ms * 1e3
    out = {"T": T, "budget": budget, "channels_per_call": listed, "list_len": Cn, "us_per_call": us,
           "trials_us": [t * 1e3 for t in all_ms], "steps": K, "weight_copies": L,
           "listed_bytes_per_call": nbytes, "effective_GBps": nbytes / (us * 1e-6) / 1e9}
    del packs
    torch.cuda.empty_cache()
    return out


def base3_channel_times(rotate_bytes: float) -> list:
    import dataclasses
    import synth
    out = []
    sw = synth.MOE_WORKLOADS["switch_base_ternary"]
    d3 = synth.MOE_WORKLOADS["dsv2lite_int4"]
    d3t = dataclasses.replace(d3, name="dsv2lite_ternary", fc1=synth.MatFmt("ternary", 64, "bf16"),
                              fc2=synth.MatFmt("ternary", 64, "bf16"))
    for base, budget in ((sw, 1.0), (d3t, 0.18)):
        row = {"layer": base.name, "T": 1, "budget": budget}
        for fmt in ("ternary", "ternary_b3"):
            spec = dataclasses.replace(base, name=f"{base.name}_{fmt}",
                                       fc1=dataclasses.replace(base.fc1, fmt=fmt),
                                       fc2=dataclasses.replace(base.fc2, fmt=fmt))
            r = channel_decode_time(spec, 1, budget, rotate_bytes=rotate_bytes)
            row[fmt] = {k: r[k] for k in ("us_per_call", "listed_bytes_per_call", "effective_GBps", "list_len")}
        row["bytes_ratio"] = row["ternary_b3"]["listed_bytes_per_call"] / row["ternary"]["listed_bytes_per_call"]
        row["time_ratio"] = row["ternary_b3"]["us_per_call"] / row["ternary"]["us_per_call"]
        log(f"[bench] base-3 {json.dumps(row)}")
        out.append(row)
    return out


def cpu_baseline(b: "MoeBench", seconds: float):
    """The oracle (double precision, plain loops) on a bounded sample of the
    headline workload's tokens: first on one host core, then on all cores of
    this process's CPU share (at most 16) over disjoint token subsets.  The
    value is the all-cores rate scaled to a whole layer."""
    import oracle
    spec, T = b.spec, b.T
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    inp = dict(b.inp0)
    inp["x"], inp["logits"] = b.x_np[0], b.lg_np[0]
    r = oracle.route(inp["logits"], spec.top_k)
    wbytes = float((r["counts"] > 0).sum()) * expert_bytes(spec)
    # one core: single tokens until ~1/3 of the budget
    t0 = time.perf_counter()
    n1 = 0
    while n1 < T and time.perf_counter() - t0 < seconds / 3:
        oracle.moe(inp, tokens=[n1])
        n1 += 1
    per1 = (time.perf_counter() - t0) / n1
    # all cores: enough tokens for about `seconds` of wall time
    n = int(min(T, max(cores, round(cores * seconds / per1))))
    toks = list(range(n))
    t0 = time.perf_counter()
    oracle.moe(inp, tokens=toks, threads=cores)
    el = time.perf_counter() - t0
    layer_s = el * T / n
    return {"value": wbytes / layer_s / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_layer": layer_s * 1e6, "us_per_layer_one_core": per1 * T * 1e6,
            "sample": f"{n} of the {T} tokens of one {spec.name} layer call on {cores} host threads "
                      f"({el:.1f}s), and {n1} tokens on one thread; double-precision oracle, "
                      f"scaled to the whole layer ({wbytes / 1e6:.1f} MB of experts touched)"}


# ------------------------------------------------------------- extras
def decode_extras(args, variants) -> dict:
    import torch
    import synth
    import dataclasses
    import copy
    from skinny_gemm_amd.layer import MoeLayer  # noqa: F401
    from skinny_gemm_amd import layer_desc
    extras = {}
    rb = args.rotate_bytes
    # switch-base ternary decode, top-1
    sw = synth.MOE_WORKLOADS["switch_base_ternary"]
    lays, isw = make_layers(sw, rb)
    r, bb = bench_moe(sw, 1, 20, 20, 3, lays, isw, rotate_bytes=rb)
    extras["switch_base_ternary"] = {k: r[k] for k in ("us_per_layer", "trials_us", "steps", "effective_GBps",
                                                        "frac_of_hbm_peak", "distinct_weight_bytes_per_replay",
                                                        "stage_us")}
    log(f"[bench] {json.dumps(extras['switch_base_ternary'])}")
    variants[f"{sw.name}_T1"] = {"base_us": r["us_per_layer"], **variant_times(bb, 3)}
    del bb, lays
    torch.cuda.empty_cache()
    # the Switch Transformer's own ReLU FFN on the same shapes
    rsw = dataclasses.replace(sw, activation="relu", name=sw.name + "_relu")
    layr, ir = make_layers(rsw, rb)
    r, bb = bench_moe(rsw, 1, 20, 20, 3, layr, ir, rotate_bytes=rb)
    variants[f"{rsw.name}_T1"] = {k: r[k] for k in ("us_per_layer", "effective_GBps", "stage_us")}
    del bb, layr
    torch.cuda.empty_cache()
    # DeepSeek-V2-Lite-shaped decode, i.i.d. logits, T = 1, 2, 4, 8
    d3 = synth.MOE_WORKLOADS["dsv2lite_int4"]
    lay3, i3 = make_layers(d3, rb)
    extras["dsv2lite_int4"] = []
    for t in d3.tokens:
        r, bb = bench_moe(d3, t, 20, 10, 3, lay3, i3, rotate_bytes=rb)
        extras["dsv2lite_int4"].append({k: r[k] for k in ("T", "us_per_layer", "steps", "effective_GBps",
                                                          "frac_of_hbm_peak", "experts_touched_per_step",
                                                          "distinct_weight_bytes_per_replay", "stage_us")})
        log(f"[bench] {json.dumps(extras['dsv2lite_int4'][-1])}")
        if t == 1:
            variants[f"{d3.name}_T1"] = {"base_us": r["us_per_layer"], **variant_times(bb, 3)}
        del bb
    # gathered channels at an 18% budget against the full layer
    extras["dsv2lite_int4_channels"] = []
    for t in (1, 8):
        r = channel_decode_time(d3, t, 0.18, rotate_bytes=rb)
        r["full_layer_us"] = next(x["us_per_layer"] for x in extras["dsv2lite_int4"] if x["T"] == t)
        extras["dsv2lite_int4_channels"].append(r)
        log(f"[bench] channels {json.dumps(r)}")
    # base-3 ternary rows against 2-bit ternary rows on the gathered-channel
    # path: the switch-base layer whole (every channel of the routed expert)
    # and the DeepSeek-V2-Lite shape in ternary at the 18% budget
    extras["ternary_base3_channels"] = base3_channel_times(rb)
    # shared logits: every selected expert receives M = T rows (the M-sweep)
    extras["dsv2lite_int4_shared_M_sweep"] = []
    for t in (1, 2, 3, 4, 5, 8, 10, 16, 32):
        r, bb = bench_moe(d3, t, 20, 5, 3, lay3, i3, stages=False, rotate_bytes=rb, logits_mode="shared")
        extras["dsv2lite_int4_shared_M_sweep"].append({"M": t, "us_per_layer": r["us_per_layer"],
                                                       "steps": r["steps"],
                                                       "experts_touched_per_step": r["experts_touched_per_step"]})
        del bb
    t1 = extras["dsv2lite_int4_shared_M_sweep"][0]["us_per_layer"]
    for e in extras["dsv2lite_int4_shared_M_sweep"]:
        e["x_M1"] = e["us_per_layer"] / t1
    log(f"[bench] shared M-sweep {json.dumps(extras['dsv2lite_int4_shared_M_sweep'])}")
    # the fused gate/up GEMV with all 64 experts active, one or two rows each
    Tc = math.ceil(d3.E / d3.top_k)
    cov = covering_logits(Tc, d3.E, d3.top_k)
    r, bb = bench_moe(d3, Tc, 20, 5, 3, lay3, i3, rotate_bytes=rb, fixed_logits=cov)
    fc1_stage = next(n for n in r["stage_us"] if "fc1" in n)
    fc1_all = d3.E * fc1_bytes(d3)
    extras["dsv2lite_fc1_all_experts"] = {
        "T": Tc, "experts_touched_per_step": r["experts_touched_per_step"], "us_per_layer": r["us_per_layer"],
        "stage_us": r["stage_us"], "fc1_kernel": fc1_stage, "fc1_bytes_per_launch": fc1_all,
        "fc1_GBps": fc1_all / (r["stage_us"][fc1_stage] * 1e-6) / 1e9,
        "fc1_frac_of_hbm_peak": fc1_all / (r["stage_us"][fc1_stage] * 1e-6) / 1e9 / HBM_PEAK_GBS}
    log(f"[bench] {json.dumps(extras['dsv2lite_fc1_all_experts'])}")
    del bb
    variants[f"runtime_scales_{d3.name}"] = runtime_scales_time(lay3[0], i3)
    # f32 activations over the same prepacked weights (the packed buffer does
    # not depend on the activation dtype; only the descriptor does)
    d3f = dataclasses.replace(d3, act_dtype="f32", name=d3.name + "_f32")
    lay3f = []
    for lay in lay3:
        c = copy.copy(lay)
        c.act_dtype = "f32"
        c.desc = layer_desc(d3.E, d3.H, d3.I, "f32", (d3.fc1.fmt, d3.fc1.block, d3.fc1.scale_dtype),
                            (d3.fc2.fmt, d3.fc2.block, d3.fc2.scale_dtype))
        lay3f.append(c)
    for t in (1, 8):
        r, bb = bench_moe(d3f, t, 20, 10, 3, lay3f, i3, stages=False, rotate_bytes=rb)
        base = next(x["us_per_layer"] for x in extras["dsv2lite_int4"] if x["T"] == t)
        variants[f"{d3.name}_T{t}_f32_activations"] = {"us": r["us_per_layer"], "bf16_us": base}
        del bb
    del lay3f, lay3
    torch.cuda.empty_cache()
    s1 = synth.MOE_WORKLOADS["single_expert_int4"]
    lay1, i1 = make_layers(s1, rb)
    r, bb = bench_moe(s1, 1, len(lay1), 20, 3, lay1, i1, rotate_bytes=rb)
    extras["single_expert_int4"] = {k: r[k] for k in ("us_per_layer", "steps", "effective_GBps", "stage_us")}
    log(f"[bench] {json.dumps(extras['single_expert_int4'])}")
    del bb, lay1
    torch.cuda.empty_cache()
    return extras


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

    layers, inp0 = make_layers(spec, args.rotate_bytes, min_copies=2)
    head, b = bench_moe(spec, T, args.steps, args.warmup, args.trials, layers, inp0, rotate_bytes=args.rotate_bytes)
    log(f"[bench] {json.dumps(head)}")
    st = head["stage_us"]
    grouped = any(n.startswith("grouped") for n in st)
    if grouped:
        # MFMA-bound kernels: algorithmic flops per launch over their duration
        fl = layer_flops(spec, T)
        kern = {}
        for n, f in (("fc1", fl["fc1"]), ("fc2", fl["fc2"])):
            name = next(s for s in st if s.startswith("grouped_" + n))
            tf = f / (st[name] * 1e-6) / 1e12
            kern[name] = {"avg_launch_us": st[name], "flops_per_launch": f, "achieved_TFLOPs": tf,
                          "frac": tf / MFMA_F16_PEAK_TFLOPS}
        dom = max(kern, key=lambda k: kern[k]["avg_launch_us"])
        prof = stored_profile(f"{spec.name}:T{T}:{dom}")
        roof = {"bound": "mfma", "kernel": dom, "achieved": kern[dom]["achieved_TFLOPs"],
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": kern[dom]["frac"],
                "traffic": prof.get("hbm_bytes_per_launch") if prof else None,
                "traffic_source": "rocprofv3 FETCH_SIZE/WRITE_SIZE, stored in profiles/counters.json "
                                  "for the current sources" if prof else None,
                "avg_launch_us": kern[dom]["avg_launch_us"],
                "trace_avg_us": prof.get("trace_avg_us") if prof else None,
                "trace_median_us": prof.get("trace_median_us") if prof else None,
                "algorithmic_flops_per_launch": kern[dom]["flops_per_launch"],
                "dtype_peak": "f16 dense MFMA 2.5 PFLOP/s", "kernels": kern,
                "layer_TFLOPs": (fl["fc1"] + fl["fc2"]) / (head["us_per_layer"] * 1e-6) / 1e12}
        if prof and (prof.get("trace_median_us") or prof.get("trace_avg_us")):
            # against the trace's median dispatch (its average also counts the
            # first dispatches after idle periods, which run at lower clocks)
            roof["trace_agreement"] = kern[dom]["avg_launch_us"] / (prof.get("trace_median_us") or prof["trace_avg_us"])
    else:
        fc1_stage = next(n for n in st if "fc1" in n)
        achieved = head["fc1_bytes_per_launch"] / (st[fc1_stage] * 1e-6) / 1e9
        prof = stored_profile(f"{spec.name}:T{T}:{fc1_stage}")
        roof = {"bound": "hbm", "kernel": fc1_stage, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": prof.get("hbm_bytes_per_launch") if prof else None,
                "avg_launch_us": st[fc1_stage], "algorithmic_bytes_per_launch": head["fc1_bytes_per_launch"]}
    line = {
        "metric": METRIC,
        "value": head["effective_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["us_per_layer"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.act_dtype,
        "data": "synthetic (seeded SplitMix64 codes, scales, activations and logits)",
        "config": {"workload": spec.name, "tokens": T, "experts": spec.E, "top_k": spec.top_k,
                   "hidden": spec.H, "intermediate": spec.I,
                   "weights": f"fc1 {spec.fc1.fmt} block {spec.fc1.block}, fc2 {spec.fc2.fmt} block {spec.fc2.block}",
                   "us_per_layer": round(head["us_per_layer"], 3), "trials_us": head["trials_us"],
                   "frac_of_hbm_peak": head["frac_of_hbm_peak"], "weight_copies": head["weight_copies"],
                   "steps_asked": args.steps,
                   "distinct_weight_bytes_per_replay": head["distinct_weight_bytes_per_replay"]},
        "roofline": roof,
        "stage_us": st,
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
        log(f"[bench] cpu {json.dumps(line['cpu_baseline'])}")
    del b
    variants = {}
    if not args.no_extras:
        if spec.name == "mixed_int2_int4_prefill":
            variants[f"{spec.name}_row_tiling"] = tiled_prefill_time(layers[0], spec, 8193, 3)
            log(f"[bench] variants {json.dumps(variants)}")
    del layers
    torch.cuda.empty_cache()
    if not args.no_extras:
        extras = decode_extras(args, variants)
        dense = synth.LINEAR_WORKLOADS["dense_affine2"]
        extras["dense_affine2"] = [bench_linear(dense, N, list(dense.Ms), 20, 3, args.rotate_bytes)
                                   for N in dense.Ns]
        extras["read_ceiling"] = read_ceiling()
        log(f"[bench] read ceiling {json.dumps(extras['read_ceiling'])}")
        extras["variants"] = variants
        line["extras"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the NVFP4 skinny GEMM on one MI355X: achieved HBM GB/s and % of the 8 TB/s peak.

Headline workload: the full weight pass of decode at M = 1 (one token), the whole model read once
per token: 64 dense 5120-hidden decoder layers (q/k/v N=7168, o_proj N=5120, gate/up N=34816 at
K=5120; down K=17408 N=5120) and the NVFP4 lm_head (K=5120, N=151936), 257 GEMMs over 12.33 GB
of packed weights (weights seed 9, drawn on the device one tensor at a time and packed untimed;
x seed 10, bf16 with 4 outlier channels x20). One step = one pass through the whole hot path
(stream packed codes and scales, decode, multiply-accumulate, scale, store fp32 Y) for all 257
GEMMs, captured as one HIP graph; `warmup` replays, then exactly `steps` replays bracketed by
torch.cuda.synchronize() on the host clock. 12.33 GB is 48x the 256 MB Infinity Cache, so every
pass streams its weights from HBM. value = compulsory bytes of the pass / time per pass.

Beside it
  * the same pass at M = 16 (one request verifying 16 tokens), HIP events around the replays;
  * per GEMM (one launch at a time, HIP graphs of back-to-back launches rotating over cold
    weight copies > 512 MB, HIP events on the stream the graphs run on, median of five timed
    blocks): the M = 1 layer (seeds 1-6) -- its slowest GEMM, the one whose 64 launches take the
    largest share of the pass (gate/up), gives the roofline object -- and, under "also", the
    verify shapes at M = 16 (gate/up, down; seed 7) and M = 128 (all four; seed 8), with their
    fractions of the binding roof (HBM or bf16 MFMA);
  * the GPU output of the M = 1 layer checked against the oracle, and the oracle itself timed on
    the host cores on that layer (cpu_baseline; a bounded sample of the pass: one of its 64
    layers).
  * "invariant": the same per-GEMM workloads in the batch-invariant mode (NVFP4_PATH_INVARIANT:
    row m of Y is the same bits for any M).
  * "lm_head_argmax": the lm_head at M = 1, 16, 128, writing the logits (nvfp4_gemm) and folding
    them into the greedy token per row (nvfp4_gemm_argmax).
  * "fused_neighbours": q/k/v with the RMSNorm folded in and gate/up with RMSNorm and
    SiLU(gate)*up folded in, at M = 1, 16 and 128, beside the plain GEMMs.
  * "moe_grouped": the grouped (mixture-of-experts) GEMM, 128 experts with 8 routed per token,
    at decode (1 token) and verification (16 tokens), per call over rotating routings.
  * "tp8_shard": one GPU's share of the layer under 8-way tensor parallelism (q/k/v, gate/up
    split N; o_proj, down split K) at M = 1, 16, 128.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for NVFP4 skinny GEMM at M=1/16/128"
EQUIV_MODEL_GB = 17.9     # the page's checkpoint size, for the tokens/s-equivalent figure
CALIBRATION_BYTES = 256 << 20
COLD_BYTES = 512 << 20      # rotated weight bytes per timed GEMM: twice the Infinity Cache
LAUNCHES_PER_GRAPH = 32
TIMED_BLOCKS = 5            # per-call figures: median of this many timed blocks of replays


def timed_replays(graph, replays: int, stream) -> float:
    """Median over TIMED_BLOCKS blocks of the milliseconds per replay of `graph`, each block
    `replays` replays bracketed by HIP events on `stream` (a single block can catch a slow
    stretch: the first timing of a process runs slow, and blocks scatter by a few percent)."""
    import torch
    times = []
    for _ in range(TIMED_BLOCKS):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / replays)
    return sorted(times)[len(times) // 2]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def load_traffic(label: str):
    """HBM bytes per launch of the GEMM `label` from the committed rocprofv3 PMC summary
    (profiles/traffic.json), if it was taken on the current kernel sources; otherwise None."""
    from skinny_gemm_nvfp4_amd.profile_summary import source_hash
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(label)
    if not entry or entry.get("source_hash") != source_hash():
        return None
    return entry.get("bytes_per_launch")


class Layer:
    """Packed weights (C cold copies), activations and outputs of a list of GEMMs on the GPU."""

    def __init__(self, gemms, copies, dev, tag, launches):
        import torch
        import skinny_gemm_nvfp4_amd as nv
        self.tag = tag
        self.path = nv.PATH_AUTO   # nvfp4_gemm; PATH_INVARIANT times the batch-invariant mode
        self.launches = launches   # labels of the GEMM dispatches, in launch order
        self.capturing = False
        self.names = [g.name for g in gemms]
        self.shapes = [g.shape for g in gemms]
        self.X = [g.X.to(dev) for g in gemms]
        self.Y = [torch.empty((m, n), dtype=torch.float32, device=dev) for m, n, _ in self.shapes]
        self.packed = []
        for g in gemms:
            W = g.W.to(dev)
            p = nv.pack(W)
            del W
            self.packed.append([p] + [self._clone(p) for _ in range(copies - 1)])
        torch.cuda.synchronize()
        self.copies = copies

    @staticmethod
    def _clone(p):
        import skinny_gemm_nvfp4_amd as nv
        return nv.Packed(p.Wq.clone(), p.Ws.clone(), p.g.clone(), p.N)

    def run(self, c: int, i: int) -> None:
        import skinny_gemm_nvfp4_amd as nv
        nv.gemm(self.X[i], *self.packed[i][c], out=self.Y[i], path=self.path)
        if not self.capturing:
            self.launches.append(self.label(i))

    def label(self, i: int) -> str:
        import skinny_gemm_nvfp4_amd as nv
        M, N, K = self.shapes[i]
        mode = "invariant." if self.path == nv.PATH_INVARIANT else ""
        return f"{mode}{self.tag}.{self.names[i]} M={M} N={N} K={K}"

    def replayed(self) -> None:
        """Record the dispatches of one graph replay of `step`."""
        self.launches.extend(self.label(i) for i in range(len(self.names)))

    def step(self, c: int) -> None:
        for i in range(len(self.names)):
            self.run(c, i)

    def cold_copies(self, i: int) -> int:
        """Copies of GEMM i's weights that together exceed twice the 256 MB Infinity Cache, so a
        rotation over them streams from HBM; clones more copies when needed."""
        from skinny_gemm_nvfp4_amd import roofline as rl
        M, N, K = self.shapes[i]
        need = max(self.copies, -(-COLD_BYTES // rl.weight_bytes(K, N)))
        while len(self.packed[i]) < need:
            self.packed[i].append(self._clone(self.packed[i][0]))
        return need

    def kernel_times_us(self, launches: int):
        """Average duration of one launch of every GEMM on its own.

        Per GEMM, a HIP graph of LAUNCHES_PER_GRAPH back-to-back launches (rotating over cold
        weight copies) is replayed until about `launches` launches ran; HIP events on the stream
        the graphs run on bracket the replays. The figure is the kernel plus its share of the
        dispatch gap, which is what a launch costs in a stream of GEMMs."""
        import torch
        stream = torch.cuda.current_stream()
        out = []
        for i in range(len(self.names)):
            copies = self.cold_copies(i)
            self.run(0, i)                     # eager first launch: one-time set-up
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            self.capturing = True
            with torch.cuda.graph(graph):
                for j in range(LAUNCHES_PER_GRAPH):
                    self.run(j % copies, i)
            self.capturing = False
            replays = max(1, -(-launches // LAUNCHES_PER_GRAPH))
            graph.replay()                     # warm
            torch.cuda.synchronize()
            ms = timed_replays(graph, replays, stream)
            out.append(1e3 * ms / LAUNCHES_PER_GRAPH)
            self.launches.extend([self.label(i)] *
                                 ((TIMED_BLOCKS * replays + 1) * LAUNCHES_PER_GRAPH))
            del graph
        return out


def gemm_report(shape, us):
    from skinny_gemm_nvfp4_amd import roofline as rl
    M, N, K = shape
    gbs = rl.compulsory_bytes(M, N, K) / (us * 1e-6) / 1e9
    roof_s = max(rl.hbm_time_s(M, N, K), rl.mfma_time_s(M, N, K))
    return {"M": M, "N": N, "K": K, "us": round(us, 3), "GB_s": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / rl.HBM_PEAK_GBS, 2),
            "binding_roof": rl.binding_roof(M, N, K),
            "pct_binding_roof": round(100 * roof_s / (us * 1e-6), 2)}


def cpu_baseline(workload, seconds: float):
    """The oracle as it stands, timed on the host cores on the same layer (weights quantised by
    the oracle itself, untimed). Also returns the oracle outputs for the parity check."""
    import oracle
    from skinny_gemm_nvfp4_amd import inputs, roofline as rl
    packed = [oracle.quantize(g.W.numpy()) for g in workload.gemms]
    xbits = [inputs.bf16_bits(g.X) for g in workload.gemms]
    bytes_per_pass = sum(rl.compulsory_bytes(*g.shape) for g in workload.gemms)
    refs = None
    t0 = time.perf_counter()
    passes = 0
    while True:
        out = [oracle.gemm(x, *p) for x, p in zip(xbits, packed)]
        passes += 1
        refs = refs or out
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    rec = {"value": round(bytes_per_pass * passes / dt / 1e9, 4), "unit": "GB/s",
           "cores": cores, "kind": "oracle",
           "sample": f"one of the pass's 64 dense layers (4 GEMMs at M=1, seeds 1-6), "
                     f"{passes} pass(es) in {dt:.1f} s, double accumulation, OpenMP over "
                     "output columns; scaled to bytes of that layer per second",
           "cpu": cpu_model(), "nproc": os.cpu_count(),
           "affinity_cpus": len(os.sched_getaffinity(0))}
    # The same oracle on one core: one pass of the layer.
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    for x, p in zip(xbits, packed):
        oracle.gemm(x, *p)
    d1 = time.perf_counter() - t1
    oracle.set_num_threads(cores)
    rec["single_core"] = {"value": round(bytes_per_pass / d1 / 1e9, 4), "unit": "GB/s",
                          "cores": 1, "sample": f"one pass of the layer in {d1:.1f} s"}
    return rec, refs


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, family/model/stepping, and the
    number of sockets (physical ids)."""
    info, sockets = {}, set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "physical id":
                    sockets.add(val)
                elif key in ("model name", "cpu family", "model", "stepping") and key not in info:
                    info[key] = val
    except OSError:
        return "unknown"
    return (f"{info.get('model name', 'unknown')} (family {info.get('cpu family', '?')}, model "
            f"{info.get('model', '?')}, stepping {info.get('stepping', '?')}, "
            f"{max(1, len(sockets))} socket(s))")


class FullPass:
    """The whole synthetic weight pass: 64 dense layers (q/k/v, o_proj, gate/up, down) and the
    NVFP4 lm_head, 257 GEMMs over 12.33 GB of packed weights (seed 9, drawn on the device one
    tensor at a time and packed; x seed 10). One HIP graph per M holds the 257 launches in pass
    order; 12.33 GB is 48x the Infinity Cache, so every replay streams its weights from HBM."""

    def __init__(self, dev):
        import torch
        import skinny_gemm_nvfp4_amd as nv
        from skinny_gemm_nvfp4_amd import inputs, roofline as rl
        self.dev = dev
        self.shapes = inputs.full_pass_shapes()
        gen = torch.Generator(device=dev).manual_seed(9)
        self.packed = []
        for _, K, N in self.shapes:
            W = inputs.weights_on_device(gen, K, N, dev)
            self.packed.append(nv.pack(W))
            del W
        torch.cuda.synchronize()
        self.weight_bytes = sum(rl.weight_bytes(K, N) for _, K, N in self.shapes)

    def bytes_per_pass(self, M: int) -> int:
        from skinny_gemm_nvfp4_amd import roofline as rl
        return sum(rl.compulsory_bytes(M, N, K) for _, K, N in self.shapes)

    def labels(self, M: int):
        return [f"full_pass_m{M}.{name.split('.')[-1]} M={M} N={N} K={K}"
                for name, K, N in self.shapes]

    def graph(self, M: int):
        """Capture the pass at M rows; returns (graph, outputs). The replay's outputs are checked
        against an eager pass."""
        import torch
        import skinny_gemm_nvfp4_amd as nv
        from skinny_gemm_nvfp4_amd import inputs
        xs = {K: x.to(self.dev) for K, x in inputs.full_pass_activations(M).items()}
        ys = {N: torch.empty((M, N), dtype=torch.float32, device=self.dev)
              for N in {N for _, _, N in self.shapes}}

        def one_pass():
            for (_, K, N), p in zip(self.shapes, self.packed):
                nv.gemm(xs[K], *p, out=ys[N])

        one_pass()                                     # eager: one-time set-up
        torch.cuda.synchronize()
        eager = {N: y.clone() for N, y in ys.items()}
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_pass()
        for y in ys.values():
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for N, y in ys.items():
            if not torch.equal(y, eager[N]):
                raise RuntimeError(f"full pass M={M}: graph replay differs from the eager pass")
        graph.keep = (xs, ys)
        return graph

    def event_ms(self, graph, reps: int) -> float:
        """Milliseconds per replay, HIP events on the stream the graph runs on."""
        import torch
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def report(self, M: int, ms: float, timing: str):
        from skinny_gemm_nvfp4_amd import roofline as rl
        total = self.bytes_per_pass(M)
        gbs = total / (ms * 1e-3) / 1e9
        return {"M": M, "ms_per_pass": round(ms, 4), "bytes_per_pass": total,
                "GB_s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / rl.HBM_PEAK_GBS, 2),
                "passes_per_s": round(1e3 / ms, 1),
                "equiv_tok_s_17_9GB": round(gbs / EQUIV_MODEL_GB, 1), "timing": timing}


def graph_time_us(call, copies: int, launches: int, label: str, log_list) -> float:
    """Average duration of one call(c): a HIP graph of LAUNCHES_PER_GRAPH back-to-back calls
    rotating over `copies` cold weight copies, replayed in blocks of about `launches` calls, HIP
    events on the stream the graph runs on around each block, the median block (as
    Layer.kernel_times_us)."""
    import torch
    stream = torch.cuda.current_stream()
    call(0)                                    # eager first call: one-time set-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(LAUNCHES_PER_GRAPH):
            call(j % copies)
    replays = max(1, -(-launches // LAUNCHES_PER_GRAPH))
    graph.replay()                             # warm
    torch.cuda.synchronize()
    ms = timed_replays(graph, replays, stream)
    log_list.extend([label] * (1 + (TIMED_BLOCKS * replays + 1) * LAUNCHES_PER_GRAPH))
    del graph
    return 1e3 * ms / LAUNCHES_PER_GRAPH


def lm_head_argmax(dev, launches, steps: int):
    """The lm_head (K = 5120, N = 151936; weights seed 9 drawn on the device and packed, x seed
    10) at M = 1, 16 and 128: nvfp4_gemm writing the fp32 logits, and nvfp4_gemm_argmax folding
    them into the greedy token per row (index and value; logits never written). Both timed per
    call over cold weight copies; the greedy tokens are checked against the argmax of the
    logits of the same call."""
    import numpy as np
    import torch
    import skinny_gemm_nvfp4_amd as nv
    from skinny_gemm_nvfp4_amd import inputs, roofline as rl
    K, N = inputs.LM_HEAD_SHAPE
    gen = torch.Generator(device=dev).manual_seed(9)
    W = inputs.weights_on_device(gen, K, N, dev)
    p0 = nv.pack(W)
    del W
    copies = max(2, -(-COLD_BYTES // rl.weight_bytes(K, N)))
    packs = [p0] + [Layer._clone(p0) for _ in range(copies - 1)]
    xgen = inputs.generator(10)
    out = {"K": K, "N": N, "cold_copies": copies,
           "timing": "HIP events around graph replays of 32 calls rotating over cold copies"}
    for M in (1, 16, 128):
        X = inputs.activations(xgen, M, K).to(dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        idx = torch.empty(M, dtype=torch.int32, device=dev)
        val = torch.empty(M, dtype=torch.float32, device=dev)
        ws = nv.argmax_workspace(M, dev)

        def call_gemm(c):
            nv.gemm(X, *packs[c], out=Y)

        def call_argmax(c):
            p = packs[c]
            nv.gemm_argmax(X, p.Wq, p.Ws, p.g, p.N, out=(idx, val), workspace=ws)

        call_gemm(0)
        call_argmax(0)
        torch.cuda.synchronize()
        want = np.argmax(Y.cpu().numpy(), axis=1)
        if not np.array_equal(idx.cpu().numpy(), want):
            raise RuntimeError(f"lm_head M={M}: greedy tokens differ from the logits' argmax")
        launches.extend([f"lm_head.gemm M={M} N={N} K={K}",
                         f"lm_head.argmax M={M} N={N} K={K}"])
        gus = graph_time_us(call_gemm, copies, max(64, steps), f"lm_head.gemm M={M} N={N} K={K}",
                            launches)
        aus = graph_time_us(call_argmax, copies, max(64, steps),
                            f"lm_head.argmax M={M} N={N} K={K}", launches)
        # compulsory bytes of the greedy-token call: weights, X and the M (index, value) pairs
        abytes = rl.weight_bytes(K, N) + 2 * M * K + 8 * M
        agbs = abytes / (aus * 1e-6) / 1e9
        roof_s = max(abytes / (rl.HBM_PEAK_GBS * 1e9), rl.mfma_time_s(M, N, K))
        out[f"m{M}"] = {"gemm": gemm_report((M, N, K), gus),
                        "argmax": {"us": round(aus, 3), "bytes": abytes, "GB_s": round(agbs, 1),
                                   "pct_hbm_peak": round(100 * agbs / rl.HBM_PEAK_GBS, 2),
                                   "binding_roof": rl.binding_roof(M, N, K),
                                   "pct_binding_roof": round(100 * roof_s / (aus * 1e-6), 2)},
                        "logit_bytes_not_written": 4 * M * N}
        del X, Y, idx, val, ws
    del packs
    torch.cuda.empty_cache()
    return out


def moe_grouped(dev, launches, steps: int):
    """The grouped (mixture-of-experts) GEMM on the expert shapes of the workload (128 experts,
    8 routed per token; gate/up K = 2048, N = 1536 and down K = 768, N = 2048): decode (1 token,
    8 rows) and verification (16 tokens, 128 rows). Weights (seed 11, drawn on the device) in 4
    copies; 32 synthetic routings (seed 12) rotate with the copies, so consecutive calls read
    different experts and the weights stream from HBM. Bytes of a call: the routed experts'
    packed weights (each read once), X, Y and the offsets."""
    import torch
    import skinny_gemm_nvfp4_amd as nv
    from skinny_gemm_nvfp4_amd import inputs, roofline as rl
    E, topk = inputs.MOE_EXPERTS, inputs.MOE_TOPK
    copies, nrout = 4, LAUNCHES_PER_GRAPH
    wgen = torch.Generator(device=dev).manual_seed(11)
    rgen = inputs.generator(12)
    out = {"experts": E, "topk": topk, "cold_copies": copies, "routings": nrout,
           "timing": "HIP events around graph replays of 32 calls (routing r, copy r % 4)"}
    for shape, (K, N) in inputs.MOE_SHAPES.items():
        Ws_fp32 = [inputs.weights_on_device(wgen, K, N, dev) for _ in range(E)]
        packed = [nv.pack_experts(Ws_fp32)]
        del Ws_fp32
        packed += [tuple(t.clone() for t in packed[0]) for _ in range(copies - 1)]
        torch.cuda.synchronize()
        for tokens in (1, 16):
            rows = tokens * topk
            cases = []
            for _ in range(nrout):
                tok, offs = inputs.moe_routing(rgen, tokens, E, topk)
                x = inputs.activations(rgen, tokens, K)
                used = int((offs[1:] > offs[:-1]).sum())
                cases.append((x[tok].to(dev), offs.to(dev), used))
            Y = torch.empty((rows, N), dtype=torch.float32, device=dev)

            def call(c, cases=cases, Y=Y, N=N):
                X, offs, _ = cases[call.i % nrout]
                call.i += 1
                nv.gemm_grouped(X, offs, *packed[c], N, out=Y)
            call.i = 0
            label = f"moe.{shape} tokens={tokens} T={rows} N={N} K={K}"
            us = graph_time_us(lambda c: call(c), copies, max(64, steps), label, launches)
            nbytes = (sum(u for _, _, u in cases) / nrout) * rl.weight_bytes(K, N) + \
                2 * rows * K + 4 * rows * N + 4 * (E + 1)
            gbs = nbytes / (us * 1e-6) / 1e9
            out[f"{shape}_tokens{tokens}"] = {
                "T": rows, "N": N, "K": K, "us": round(us, 3),
                "experts_read_avg": round(sum(u for _, _, u in cases) / nrout, 2),
                "bytes_avg": round(nbytes), "GB_s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / rl.HBM_PEAK_GBS, 2)}
        del packed
        torch.cuda.empty_cache()
    return out


def fused_neighbours(dev, launches, steps: int):
    """The layer's q/k/v projection with the input RMSNorm folded in, and its gate/up projection
    with the post-attention RMSNorm and SiLU(gate) * up folded in (weight columns interleaved),
    at M = 1, 16 and 128 (weights seed 13 drawn on the device, x and gamma seed 14), next to the
    plain GEMM of the same shape. Bytes of a fused call: weights, X, gamma and its output (fp32 Y
    for q/k/v, bf16 H for gate/up)."""
    import torch
    import skinny_gemm_nvfp4_amd as nv
    from skinny_gemm_nvfp4_amd import inputs, roofline as rl
    K = inputs.HIDDEN
    wgen = torch.Generator(device=dev).manual_seed(13)
    xgen = inputs.generator(14)
    gamma = inputs.norm_weight(xgen, K).to(dev)
    out = {"eps": inputs.RMSNORM_EPS,
           "timing": "HIP events around graph replays of 32 calls rotating over cold copies"}
    for name, silu in (("qkv", False), ("gate_up", True)):
        N = inputs.LAYER_SHAPES[name][1]
        W = inputs.weights_on_device(wgen, K, N, dev)
        if silu:
            W = nv.interleave_gate_up(W)
        p0 = nv.pack(W)
        del W
        copies = max(2, -(-COLD_BYTES // rl.weight_bytes(K, N)))
        packs = [p0] + [Layer._clone(p0) for _ in range(copies - 1)]
        for M in (1, 16, 128):
            X = inputs.activations(xgen, M, K, outliers=4).to(dev)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            O = torch.empty((M, N // 2) if silu else (M, N),
                            dtype=torch.bfloat16 if silu else torch.float32, device=dev)

            def plain(c, X=X, Y=Y, packs=packs):
                nv.gemm(X, *packs[c], out=Y)

            ws = nv.fused_workspace(nv.FUSE_RMSNORM | (nv.FUSE_SILU_MUL if silu else 0), M, N,
                                    K, dev)

            def fused(c, X=X, O=O, packs=packs, N=N, silu=silu, ws=ws):
                p = packs[c]
                nv.gemm_fused(X, p.Wq, p.Ws, p.g, N, gamma=gamma, eps=inputs.RMSNORM_EPS,
                              silu_mul=silu, out=O, workspace=ws)

            lab = f"fused.{name} M={M} N={N} K={K}"
            pus = graph_time_us(plain, copies, max(64, steps), f"{lab} plain", launches)
            fus = graph_time_us(fused, copies, max(64, steps), lab, launches)
            fbytes = rl.weight_bytes(K, N) + 2 * M * K + 2 * K + (2 * M * N // 2 if silu
                                                                    else 4 * M * N)
            gbs = fbytes / (fus * 1e-6) / 1e9
            out[f"{name}_m{M}"] = {
                "fused": "rmsnorm + gemm + silu*up" if silu else "rmsnorm + gemm",
                "M": M, "N": N, "K": K, "fused_us": round(fus, 3), "plain_gemm_us": round(pus, 3),
                "fused_bytes": fbytes, "fused_GB_s": round(gbs, 1),
                "fused_pct_hbm_peak": round(100 * gbs / rl.HBM_PEAK_GBS, 2),
                # the round trips a separate SiLU * up kernel (fp32 gate/up) would add, and a
                # separate RMSNorm kernel's bf16 xhat where the call normalises X in LDS
                "bytes_not_moved": (8 * M * N if silu else 0) +
                                   (4 * M * K if ws is None else 0),
                "workspace_bytes": 0 if ws is None else ws.numel()}
        del packs
        torch.cuda.empty_cache()
    return out


def tp8_shard(dev, launches, steps: int):
    """One GPU's share of the dense layer under 8-way tensor parallelism (q/k/v and gate/up split
    N, o_proj and down split K) at M = 1, 16 and 128, per GEMM, as the other legs (the
    collective of the row-parallel halves is not part of a one-GPU run)."""
    import torch
    import skinny_gemm_nvfp4_amd as nv
    from skinny_gemm_nvfp4_amd import inputs, roofline as rl
    wgen = torch.Generator(device=dev).manual_seed(15)
    xgen = inputs.generator(16)
    out = {"tp": inputs.TP,
           "timing": "HIP events around graph replays of 32 calls rotating over cold copies"}
    for name, (K, N) in inputs.TP8_SHARD_SHAPES.items():
        p0 = nv.pack(inputs.weights_on_device(wgen, K, N, dev))
        copies = max(2, -(-COLD_BYTES // rl.weight_bytes(K, N)))
        packs = [p0] + [Layer._clone(p0) for _ in range(copies - 1)]
        for M in (1, 16, 128):
            X = inputs.activations(xgen, M, K).to(dev)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)

            def call(c, X=X, Y=Y, packs=packs):
                nv.gemm(X, *packs[c], out=Y)

            lab = f"tp8.{name} M={M} N={N} K={K}"
            us = graph_time_us(call, copies, max(64, steps), lab, launches)
            out[f"{name}_m{M}"] = gemm_report((M, N, K), us)
        del packs
        torch.cuda.empty_cache()
    return out


def main() -> int:
    global TIMED_BLOCKS
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cold-copies", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="skip the M=16 / M=128 shapes")
    ap.add_argument("--no-full-pass", action="store_true",
                    help="skip the M=16 weight pass (the M=1 pass is the headline)")
    ap.add_argument("--full-pass-reps", type=int, default=20)
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the 8-way tensor-parallel shard shapes")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the RMSNorm / SiLU(gate)*up fused-neighbour timing")
    ap.add_argument("--no-moe", action="store_true",
                    help="skip the grouped (mixture-of-experts) GEMM timing")
    ap.add_argument("--no-lm-head", action="store_true",
                    help="skip the lm_head GEMM vs greedy-token (argmax) timing at M=1/16/128")
    ap.add_argument("--no-invariant", action="store_true",
                    help="skip timing the batch-invariant mode (NVFP4_PATH_INVARIANT)")
    ap.add_argument("--launch-log", default=None,
                    help="write the label of every GEMM dispatch, in order, to this file (for "
                         "matching a rocprofv3 kernel trace to the GEMMs)")
    ap.add_argument("--timed-blocks", type=int, default=TIMED_BLOCKS,
                    help="timed blocks per per-call figure (the median is reported); counter "
                         "passes under a profiler use 1 to keep the dispatch count down")
    args = ap.parse_args()
    TIMED_BLOCKS = max(1, args.timed_blocks)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the GEMM would "
              "shard by output columns with no exchange); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import skinny_gemm_nvfp4_amd as nv
    from skinny_gemm_nvfp4_amd import inputs, roofline as rl
    from skinny_gemm_nvfp4_amd import profile_summary as ps

    nv.load_library()
    dev = torch.device("cuda:0")
    C = max(1, args.cold_copies)
    launches = []

    # One plain device-to-device copy of known size: under rocprofv3 --pmc it calibrates
    # FETCH_SIZE and WRITE_SIZE against bytes actually moved.
    log(f"calibration copy of {CALIBRATION_BYTES} bytes")
    src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # Headline: the full weight pass at M = 1 (one step = one pass, 257 GEMMs in one graph).
    log("generating and packing the full weight pass (64 layers + lm_head, seed 9)")
    fpass = FullPass(dev)
    g1 = fpass.graph(1)
    bytes_per_step = fpass.bytes_per_pass(1)
    labels1 = fpass.labels(1)
    log(f"timing {args.steps} replays of the M=1 pass after {args.warmup} warmup")
    for _ in range(args.warmup):
        g1.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g1.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launches.extend(labels1 * (2 + args.warmup + args.steps))
    ms_per_step = 1e3 * (t1 - t0) / args.steps
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    fp = {"gemms": len(fpass.shapes), "weight_bytes": fpass.weight_bytes,
          "m1": fpass.report(1, ms_per_step, "host clock around the timed replays")}
    del g1
    if not args.no_full_pass:
        reps = max(1, args.full_pass_reps)
        log(f"timing {reps} replays of the M=16 pass (HIP events)")
        g16 = fpass.graph(16)
        g16.replay()
        ms16 = fpass.event_ms(g16, reps)
        launches.extend(fpass.labels(16) * (3 + reps))
        fp["m16"] = fpass.report(16, ms16, "HIP events around the replays")
        del g16
    del fpass
    torch.cuda.empty_cache()

    # The layer's GEMMs one at a time (per-kernel figures, roofline of the pass's dominant
    # kernel) and the parity check against the oracle, on the M = 1 layer of seeds 1-6.
    log("generating and packing the M=1 dense layer (seeds 1-6)")
    wl = inputs.dense_layer_m1()
    layer = Layer(wl.gemms, C, dev, "dense_layer_m1", launches)
    layer.step(0)
    torch.cuda.synchronize()
    eager_Y = [y.clone() for y in layer.Y]

    log("per-kernel event timing")
    kus = layer.kernel_times_us(max(64, args.steps * 4))
    per_gemm = {n: gemm_report(s, us) for n, s, us in zip(layer.names, layer.shapes, kus)}
    # The pass's dominant kernel: the GEMM whose 64 launches take the largest share of the pass.
    dom = max(range(len(layer.names)), key=lambda i: kus[i])
    dom_bytes = rl.compulsory_bytes(*layer.shapes[dom])
    achieved = dom_bytes / (kus[dom] * 1e-6) / 1e9
    traffic = load_traffic(layer.label(dom))
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": rl.HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / rl.HBM_PEAK_GBS, 4),
            "traffic": traffic, "kernel": f"nvfp4 GEMM {layer.names[dom]} M=1 "
            f"K={layer.shapes[dom][2]} N={layer.shapes[dom][1]}",
            "share_of_pass": round(64 * kus[dom] * 1e-3 / ms_per_step, 3),
            "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(kus[dom], 3),
            "timing": "HIP events on the launch stream around graphs of back-to-back launches "
                      "over cold weight copies"}

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        cpu, refs = cpu_baseline(wl, args.cpu_seconds)
        worst = 0.0
        import oracle
        for (Yref, A), y in zip(refs, eager_Y):
            err = np.abs(y.cpu().numpy().astype(np.float64) - Yref)
            worst = max(worst, float((err / oracle.tolerance(A)).max()))
        parity = {"workload": "dense_layer_m1 (seeds 1-6)",
                  "worst_err_over_bound": float(f"{worst:.3g}"), "pass": worst <= 1.0}
        if worst > 1.0:
            raise RuntimeError(f"GPU output outside tolerance (worst ratio {worst})")

    also = {}
    invariant = {}
    if not args.no_invariant:
        # The batch-invariant mode (row m of Y the same bits for any M) on the same layer.
        log("timing the batch-invariant mode on dense_layer_m1")
        layer.path = nv.PATH_INVARIANT
        ius = layer.kernel_times_us(max(64, args.steps // 2))
        invariant["dense_layer_m1"] = {n: gemm_report(s, t)
                                       for n, s, t in zip(layer.names, layer.shapes, ius)}
        layer.path = nv.PATH_AUTO
    if not args.no_also:
        for wname, make in (("verify_m16", inputs.verify_m16),
                            ("batched_verify_m128", inputs.batched_verify_m128)):
            log(f"timing {wname}")
            w = make()
            lay = Layer(w.gemms, C, dev, wname, launches)
            us = lay.kernel_times_us(max(64, args.steps))
            also[wname] = {n: gemm_report(s, t) for n, s, t in zip(lay.names, lay.shapes, us)}
            if not args.no_invariant:
                lay.path = nv.PATH_INVARIANT
                ius = lay.kernel_times_us(max(64, args.steps // 2))
                invariant[wname] = {n: gemm_report(s, t)
                                    for n, s, t in zip(lay.names, lay.shapes, ius)}
            del lay
            torch.cuda.empty_cache()

    lmh = None
    if not args.no_lm_head:
        log("timing the lm_head: logits vs greedy token per row (nvfp4_gemm_argmax)")
        lmh = lm_head_argmax(dev, launches, args.steps)

    fused = None
    if not args.no_fused:
        log("timing the fused layer neighbours (RMSNorm prologue, SiLU(gate)*up epilogue)")
        fused = fused_neighbours(dev, launches, args.steps)

    moe = None
    if not args.no_moe:
        log("timing the grouped (mixture-of-experts) GEMM: decode and verify routings")
        moe = moe_grouped(dev, launches, args.steps)

    shard = None
    if not args.no_shard:
        log("timing one GPU's share of the layer under 8-way tensor parallelism")
        shard = tp8_shard(dev, launches, args.steps)

    m128 = {n: r["pct_binding_roof"] for n, r in also.get("batched_verify_m128", {}).items()}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full_weight_pass_m1", "M": 1, "layers": 64,
                   "gemms": len(labels1),
                   "shapes": "per layer q/k/v K=5120 N=7168, o_proj K=5120 N=5120, gate/up "
                             "K=5120 N=34816, down K=17408 N=5120; lm_head K=5120 N=151936",
                   "seeds": "weights 9, x 10", "bytes_per_step": bytes_per_step,
                   "weights": "nvfp4 (e2m1 codes, e4m3 scale per 16 along K, fp32 tensor scale)",
                   "accumulate": "f32", "x": "bf16", "y": "f32",
                   "timing": "one HIP graph of the 257 GEMMs per step, host clock"},
        "pct_hbm_peak": round(100 * value / rl.HBM_PEAK_GBS, 2),
        "equiv_tok_s_17_9GB": round(value / EQUIV_MODEL_GB, 1),
        "beside": {"full_pass_m16_pct_hbm_peak": fp.get("m16", {}).get("pct_hbm_peak"),
                   "batched_verify_m128_pct_binding_roof": m128 or None},
        "full_pass": fp,
        "per_gemm_m1": per_gemm,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "also": also,
        "invariant": invariant or None,
        "lm_head_argmax": lmh,
        "moe_grouped": moe,
        "fused_neighbours": fused,
        "tp8_shard": shard,
        "source_hash": ps.source_hash(),
    }
    if args.launch_log:
        with open(args.launch_log, "w") as f:
            f.write("\n".join(launches) + "\n")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

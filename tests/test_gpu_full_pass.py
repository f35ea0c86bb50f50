"""The full synthetic weight pass (64 dense layers of the 5120-hidden family + the NVFP4 lm_head,
12.33 GB of packed weights) run as the benchmark runs it: weights drawn on the device (seed 9,
one tensor at a time, in pass order) and packed by the GPU, x from seed 10, the 257 GEMMs of a
pass captured in one HIP graph at M = 1 and M = 16 and replayed.

Sampled against the oracle (the whole pass would take the oracle minutes to quantise): layer 0's
four GEMMs, layer 63's q/k/v and down projections and the lm_head. For each, the fp32 weight the
device drew is copied to the host; the oracle quantises it itself (the GPU's packed bytes must
equal the oracle's bit for bit) and computes the GEMM from its own bytes: every column at M = 1,
a seeded column sample plus both ends of N at M = 16.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import check_close, from_library_layout, say

pytestmark = pytest.mark.gpu

SAMPLED = {"layer0.qkv", "layer0.o_proj", "layer0.gate_up", "layer0.down", "layer63.qkv",
           "layer63.down", "lm_head"}


def _columns(N, seed, sample=2048):
    if N <= sample:
        return None
    mid = torch.randperm(N, generator=inputs.generator(seed))[:sample].numpy()
    return np.unique(np.r_[mid, np.arange(16), np.arange(N - 16, N)]).astype(np.int32)


def test_full_pass_sampled(device):
    shapes = inputs.full_pass_shapes()
    gen = torch.Generator(device=device).manual_seed(9)
    packed, host_W = [], {}
    say("full pass: drawing and packing 257 weights on the device")
    for name, K, N in shapes:
        W = inputs.weights_on_device(gen, K, N, device)
        packed.append(nv.pack(W))
        if name in SAMPLED:
            host_W[name] = W.cpu()
        del W
    torch.cuda.synchronize()
    refs = {}
    for i, (name, K, N) in enumerate(shapes):
        if name not in SAMPLED:
            continue
        say(f"full pass: oracle quantises {name} K={K} N={N}")
        Wq_o, Ws_o, g_o = oracle.quantize(host_W.pop(name).numpy())
        wq, ws, pad_zero = from_library_layout(packed[i].Wq.cpu().numpy(),
                                               packed[i].Ws.cpu().numpy(), N, K)
        assert pad_zero and np.array_equal(wq, Wq_o) and np.array_equal(ws, Ws_o), name
        assert float(packed[i].g.cpu()[0]) == float(g_o), name
        refs[i] = (Wq_o, Ws_o, g_o)
    for M in (1, 16):
        xs = {K: x.to(device) for K, x in inputs.full_pass_activations(M).items()}
        # one output per sampled GEMM, one shared scratch output per N for the others
        ys = {i: torch.empty((M, N), dtype=torch.float32, device=device)
              for i, (_, _, N) in enumerate(shapes) if i in refs}
        scratch = {N: torch.empty((M, N), dtype=torch.float32, device=device)
                   for _, _, N in shapes}

        def one_pass():
            for i, (_, K, N) in enumerate(shapes):
                nv.gemm(xs[K], *packed[i], out=ys.get(i, scratch[N]))

        one_pass()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_pass()
        for y in ys.values():
            y.fill_(float("nan"))
        say(f"full pass M={M}: graph replay")
        graph.replay()
        graph.replay()
        torch.cuda.synchronize()
        for i, (Wq_o, Ws_o, g_o) in refs.items():
            name, K, N = shapes[i]
            cols = None if M == 1 else _columns(N, seed=N + K)
            say(f"full pass M={M}: oracle {name}")
            Yref, A = oracle.gemm(inputs.bf16_bits(xs[K].cpu()), Wq_o, Ws_o, g_o, cols=cols)
            Y = ys[i].cpu().numpy().astype(np.float64)
            worst = check_close(Y if cols is None else Y[:, cols], Yref, A, f"M={M} {name}")
            say(f"  worst error / bound = {worst:.3g}")
        del graph, xs, ys, scratch
    del packed
    torch.cuda.empty_cache()

"""The GEMM captured in a HIP graph (as the benchmark times it) must reproduce the eager result
on every replay, with unrelated eager work and synchronisations between the replays."""
import pytest
import torch

import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(device):
    gen = inputs.generator(21)
    # (128, 1024, 4096) is narrow enough for the batch kernel to cut K across workgroups, so its
    # replays use the split-K workspace the eager warm-up allocated.
    shapes = [(1, 7168, 5120), (16, 1024, 17408), (128, 512, 5120), (3, 200, 1040),
              (128, 1024, 4096)]
    Xs, packs, Ys = [], [], []
    for M, N, K in shapes:
        W = inputs.weights(gen, K, N).to(device)
        packs.append(nv.pack(W))
        Xs.append(inputs.activations(gen, M, K).to(device))
        Ys.append(torch.empty((M, N), dtype=torch.float32, device=device))

    def step():
        for X, p, Y in zip(Xs, packs, Ys):
            nv.gemm(X, *p, out=Y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [y.clone() for y in Ys]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for y in Ys:
            y.fill_(float("nan"))                       # eager work between replays
        junk = torch.randn(1 << 20, device=device).sum()
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(Ys, eager)):
            assert torch.equal(y, e), f"replay {rep}: GEMM {i} differs from eager"
        del junk

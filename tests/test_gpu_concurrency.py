"""Concurrent and captured calls (include/nvfp4.h: the library owns no device memory, calls are
re-entrant, and a call's bits do not depend on the stream, on other calls in flight or on graph
capture).

Several requests verify their drafted tokens together, each group on its own stream ("SparkInfer"
README, speculative decoding sections), so two host threads drive two streams at once here: 128-row
GEMMs of narrow weights (the shapes that once split K through a shared buffer), a long-K one, and a
64-row fused RMSNorm + SiLU * up call with each thread's own workspace. Every result must equal the
bits of the same call run alone, and the oracle's bound. A call captured into a graph before that
shape ever ran eagerly must give the eager bits too.
"""
import threading

import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import FINITE_SCALES, check_close, random_case, say, to_device_packed

pytestmark = pytest.mark.gpu

SHAPES = [(128, 1024, 5120), (128, 520, 17408), (96, 1500, 2048)]
REPEATS = 6


def _cases(device, seed):
    out = []
    for i, (M, N, K) in enumerate(SHAPES):
        X, Wq, Ws, g = random_case(seed + i, M, N, K, FINITE_SCALES)
        out.append((X, Wq, Ws, g, to_device_packed(Wq, Ws, g, device)))
    return out


def test_two_streams_two_threads(device):
    cases = _cases(device, 9100)
    K, N, M = 1024, 1040, 64
    gen = inputs.generator(9150)
    W = nv.interleave_gate_up(inputs.weights(gen, K, N))
    fp = nv.pack(W.to(device))
    gamma = inputs.norm_weight(gen, K).to(device)
    Xf = inputs.activations(gen, M, K).to(device)
    fuse = nv.FUSE_RMSNORM | nv.FUSE_SILU_MUL

    def gemms(stream):
        Xd = [c[0].to(device) for c in cases]
        return [nv.gemm(X, c[4].Wq, c[4].Ws, c[4].g, c[4].N, stream=stream)
                for X, c in zip(Xd, cases)]

    def fused(stream, ws):
        return nv.gemm_fused(Xf, fp.Wq, fp.Ws, fp.g, N, gamma=gamma, eps=inputs.RMSNORM_EPS,
                             silu_mul=True, workspace=ws, stream=stream)

    say("concurrency: reference calls, one at a time")
    alone = [Y.cpu() for Y in gemms(torch.cuda.current_stream())]
    ws0 = nv.fused_workspace(fuse, M, N, K, device)
    alone_h = fused(torch.cuda.current_stream(), ws0).cpu()
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(device=device) for _ in range(2)]
    wss = [nv.fused_workspace(fuse, M, N, K, device) for _ in range(2)]
    results = [[] for _ in range(2)]
    errors = []
    start = threading.Barrier(2)

    def worker(t):
        try:
            s = streams[t]
            with torch.cuda.stream(s):
                start.wait()
                for _ in range(REPEATS):
                    results[t].append((gemms(s), fused(s, wss[t])))
            s.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    say(f"concurrency: 2 threads x {REPEATS} rounds on 2 streams")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        assert len(results[t]) == REPEATS
        for r, (Ys, H) in enumerate(results[t]):
            for c, (Y, Ya) in enumerate(zip(Ys, alone)):
                assert torch.equal(Y.cpu(), Ya), f"thread {t} round {r} shape {SHAPES[c]} differs"
            assert torch.equal(H.cpu(), alone_h), f"thread {t} round {r} fused call differs"
    for (X, Wq, Ws, g, _), Ya, (M_, N_, K_) in zip(cases, alone, SHAPES):
        Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
        check_close(Ya.numpy().astype(np.float64), Yref, A, f"concurrency M={M_} N={N_} K={K_}")


def test_first_call_under_capture(device):
    """Shapes this process has not run before, captured first and replayed, then run eagerly."""
    cases = _cases(device, 9200)
    # Shapes distinct from every other test's, so no plan for them exists yet.
    extra = [(112, 1328, 3072), (48, 700, 9216)]
    for i, (M, N, K) in enumerate(extra):
        X, Wq, Ws, g = random_case(9250 + i, M, N, K, FINITE_SCALES)
        cases.append((X, Wq, Ws, g, to_device_packed(Wq, Ws, g, device)))
    Xd = [c[0].to(device) for c in cases]
    Ys = [torch.full((c[0].shape[0], c[4].N), float("nan"), device=device) for c in cases]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("capture: first calls inside a graph")
    with torch.cuda.graph(graph):
        for X, c, Y in zip(Xd, cases, Ys):
            nv.gemm(X, c[4].Wq, c[4].Ws, c[4].g, c[4].N, out=Y)
    for rep in range(2):
        for Y in Ys:
            Y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"capture: replay {rep}")
        for X, c, Y in zip(Xd, cases, Ys):
            eager = nv.gemm(X, c[4].Wq, c[4].Ws, c[4].g, c[4].N)
            torch.cuda.synchronize()
            assert torch.equal(Y, eager), f"replay {rep}: captured M={X.shape[0]} N={c[4].N} differs"

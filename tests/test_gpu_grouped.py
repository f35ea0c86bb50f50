"""Grouped (mixture-of-experts) GEMM (nvfp4_gemm_grouped through the C ABI) against
oracle.grouped_gemm ("SparkInfer" README, section "Layout & scoring": fused MoE FFN and expert
dispatch).

Bars: |Y - Y_ref| <= 2e-3 * sum|x*w| + 1e-6 per output; bit equality for exact-sum inputs; the
same bits for every rows_per_item. Experts no row is routed to hold NaN scale bytes (0xFF), so a
read of the wrong expert shows up as NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import FINITE_SCALES, check_close, say, to_library_layout

pytestmark = pytest.mark.gpu


def _experts_to_device(Wq_plain, Ws_plain, g, N, K, device):
    """Plain-layout expert bytes [E][N][K/2], [E][N][K/16] -> back-to-back library layout."""
    E = Wq_plain.shape[0]
    wq = np.stack([to_library_layout(Wq_plain[e], Ws_plain[e], K)[0] for e in range(E)])
    ws = np.stack([to_library_layout(Wq_plain[e], Ws_plain[e], K)[1] for e in range(E)])
    return (torch.from_numpy(wq).to(device), torch.from_numpy(ws).to(device),
            torch.from_numpy(np.asarray(g, dtype=np.float32)).to(device))


def _random_experts(gen, E, N, K, used, scales=FINITE_SCALES):
    """Random packed bytes for the used experts; 0xFF (NaN scales) for the others."""
    Wq = np.full((E, N, K // 2), 0xFF, dtype=np.uint8)
    Ws = np.full((E, N, K // 16), 0xFF, dtype=np.uint8)
    for e in used:
        q, s = inputs.random_packed(gen, N, K, scales)
        Wq[e], Ws[e] = q.numpy(), s.numpy()
    g = np.array([0.003 * (1 + e % 7) for e in range(E)], dtype=np.float32)
    return Wq, Ws, g


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _run(X, offsets, dev_w, N, device, rpi=0):
    Wq, Ws, g = dev_w
    Y = nv.gemm_grouped(X.to(device), torch.from_numpy(np.asarray(offsets)).to(device), Wq, Ws,
                        g, N, rows_per_item=rpi)
    torch.cuda.synchronize()
    return Y.cpu().numpy().astype(np.float64)


COUNTS = [[3], [1, 0, 2, 0, 1], [0, 0, 5], [2, 1, 0, 4, 0, 0, 9, 1], [1] * 16,
          [0, 7, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 13]]


@pytest.mark.parametrize("counts", COUNTS)
def test_random_experts_against_oracle(device, counts):
    E = len(counts)
    offsets = _offsets(counts)
    T = int(offsets[-1])
    used = [e for e in range(E) if counts[e] > 0]
    for N, K in [(1, 16), (17, 272), (200, 1024), (65, 5120)]:
        gen = inputs.generator(T * 31 + N + K + E)
        Wq, Ws, g = _random_experts(gen, E, N, K, used)
        X = inputs.activations(gen, T, K)
        Yref, A = oracle.grouped_gemm(inputs.bf16_bits(X), offsets, Wq, Ws, g)
        dev_w = _experts_to_device(Wq, Ws, g, N, K, device)
        first = None
        for rpi in (0, 1, 2, 4):
            say(f"grouped counts={counts} N={N} K={K} rows_per_item={rpi}")
            Y = _run(X, offsets, dev_w, N, device, rpi)
            check_close(Y, Yref, A, f"grouped E={E} N={N} K={K} rpi={rpi}")
            if first is None:
                first = Y
            assert np.array_equal(Y, first), f"rows_per_item {rpi} changed the bits"


def test_exact_integer_sums(device):
    """Scales in {0.5, 1, 2}, g = 1, integer X: Y equals the oracle bit for bit."""
    counts = [2, 0, 3, 1, 0, 6]
    offsets = _offsets(counts)
    T, N, K = int(offsets[-1]), 67, 1040
    gen = inputs.generator(606)
    Wq, Ws, _ = _random_experts(gen, len(counts), N, K, [0, 2, 3, 5], [0x30, 0x38, 0x40])
    g = np.ones(len(counts), dtype=np.float32)
    X = inputs.integer_activations(gen, T, K)
    Yref, _ = oracle.grouped_gemm(inputs.bf16_bits(X), offsets, Wq, Ws, g)
    dev_w = _experts_to_device(Wq, Ws, g, N, K, device)
    for rpi in (1, 2, 4):
        say(f"grouped exact rows_per_item={rpi}")
        assert np.array_equal(_run(X, offsets, dev_w, N, device, rpi), Yref)


def test_offsets_are_clamped(device):
    """Offsets are clamped to [0, T] and made non-decreasing (running maximum): an expert whose
    end precedes its start has no rows, and the next expert starts where the running maximum
    stands."""
    T, N, K = 6, 40, 512
    gen = inputs.generator(707)
    Wq, Ws, g = _random_experts(gen, 3, N, K, [0, 1, 2])
    X = inputs.activations(gen, T, K)
    dev_w = _experts_to_device(Wq, Ws, g, N, K, device)
    for raw, clamped in [([-3, 2, 2, 100], [0, 2, 2, 6]), ([0, 4, 1, 6], None)]:
        say(f"grouped offsets {raw}")
        Y = _run(X, np.array(raw, dtype=np.int32), dev_w, N, device)
        if clamped is not None:
            Yref, A = oracle.grouped_gemm(inputs.bf16_bits(X), clamped, Wq, Ws, g)
            check_close(Y, Yref, A, f"clamped {raw}")
        else:
            # running maximum [0, 4, 4, 6]: expert 0 rows 0..3, expert 1 none, expert 2 rows 4, 5
            Yref, A = oracle.grouped_gemm(inputs.bf16_bits(X), [0, 4, 4, 6], Wq, Ws, g)
            check_close(Y, Yref, A, f"running maximum {raw}")


@pytest.mark.parametrize("tokens", [1, 16])
@pytest.mark.parametrize("shape", ["gate_up", "down"])
def test_moe_workload(device, tokens, shape):
    """128 experts, 8 routed per token (synthetic router), the expert shapes of the workload;
    weights of the routed experts from the quantisation recipe (packed by the GPU, and by the
    oracle from the same fp32 tensor), NaN bytes in every other expert."""
    K, N = inputs.MOE_SHAPES[shape]
    E = inputs.MOE_EXPERTS
    gen = inputs.generator(800 + tokens)
    token_of_row, offsets = inputs.moe_routing(gen, tokens, E, inputs.MOE_TOPK)
    used = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    Wq_dev = torch.full((E,) + nv.codes_shape(N, K), 0xFF, dtype=torch.uint8, device=device)
    Ws_dev = torch.full((E,) + nv.scales_shape(N, K), 0xFF, dtype=torch.uint8, device=device)
    g_dev = torch.full((E,), float("nan"), dtype=torch.float32, device=device)
    Wq_o = np.zeros((E, N, K // 2), dtype=np.uint8)
    Ws_o = np.zeros((E, N, K // 16), dtype=np.uint8)
    g_o = np.zeros(E, dtype=np.float32)
    for e in used:
        W = inputs.weights(gen, K, N)
        nv.pack(W.to(device), out=(Wq_dev[e], Ws_dev[e], g_dev[e:e + 1]))
        Wq_o[e], Ws_o[e], g_o[e] = oracle.quantize(W.numpy())
    x = inputs.activations(gen, tokens, K)
    X = x[token_of_row]
    say(f"moe {shape} tokens={tokens} rows={X.shape[0]} experts used={len(used)}")
    Y = nv.gemm_grouped(X.to(device), offsets.to(device), Wq_dev, Ws_dev, g_dev, N)
    torch.cuda.synchronize()
    Yref, A = oracle.grouped_gemm(inputs.bf16_bits(X), offsets.numpy(), Wq_o, Ws_o, g_o)
    check_close(Y.cpu().numpy().astype(np.float64), Yref, A, f"moe {shape} tokens={tokens}")


def test_graph_replays_match_eager(device):
    """The grouped GEMM in a HIP graph: same bits on every replay, with new routings written into
    the offsets between replays (the kernel reads them on the device)."""
    E, N, K, T = 32, 512, 2048, 24
    gen = inputs.generator(909)
    Wq, Ws, g = _random_experts(gen, E, N, K, range(E))
    dev_w = _experts_to_device(Wq, Ws, g, N, K, device)
    X = inputs.activations(gen, T, K).to(device)
    routings = [np.sort(torch.randint(0, E, (T,), generator=gen).numpy()) for _ in range(3)]
    offs = [_offsets(np.bincount(r, minlength=E)) for r in routings]
    offsets = torch.from_numpy(offs[0]).to(device)
    Y = torch.empty((T, N), dtype=torch.float32, device=device)
    eager = []
    for o in offs:
        offsets.copy_(torch.from_numpy(o))
        nv.gemm_grouped(X, offsets, *dev_w, N, out=Y)
        torch.cuda.synchronize()
        eager.append(Y.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.gemm_grouped(X, offsets, *dev_w, N, out=Y)
    for rep in range(6):
        offsets.copy_(torch.from_numpy(offs[rep % 3]))
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"grouped graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager[rep % 3]), f"replay {rep} differs"


def test_no_rows_and_most_experts(device):
    """T = 0 launches nothing and leaves Y as it was; E = 2048 (the most the kernel takes) with a
    handful of rows on scattered experts, the others empty."""
    N, K = 24, 256
    E = 2048
    gen = inputs.generator(1212)
    used = [3, 700, 701, 2047]
    Wq, Ws, g = _random_experts(gen, E, N, K, used)
    dev_w = _experts_to_device(Wq, Ws, g, N, K, device)
    Y = torch.full((0, N), 7.0, dtype=torch.float32, device=device)
    say("grouped T=0")
    nv.gemm_grouped(torch.empty((0, K), dtype=torch.bfloat16, device=device),
                    torch.zeros(E + 1, dtype=torch.int32, device=device), *dev_w, N, out=Y)
    torch.cuda.synchronize()
    counts = np.zeros(E, dtype=np.int64)
    counts[used] = [2, 1, 3, 1]
    offsets = _offsets(counts)
    X = inputs.activations(gen, int(offsets[-1]), K)
    say("grouped E=2048")
    Y = _run(X, offsets, dev_w, N, device)
    Yref, A = oracle.grouped_gemm(inputs.bf16_bits(X), offsets, Wq, Ws, g)
    check_close(Y, Yref, A, "E=2048")

"""Greedy-token GEMM (nvfp4_gemm_argmax through the C ABI): the lm_head's argmax per row without
writing the logits ("SparkInfer" README: greedy decode and verification; "Qwen3.8-27B-NVFP4-
RTX5090" model card: the lm_head is a full-vocabulary GEMM read on every token).

Bars:
  * against the GEMM it fuses: for every path and split, (index, value) equal the first column of
    each row's maximum of nvfp4_gemm_path's Y with the same path and split, and that maximum, bit
    for bit (the fold is an exact maximum, not an approximation);
  * against the oracle: exact-sum inputs (every partial sum exact in fp32) give exact logits, so
    the index must equal oracle.argmax_rows, ties to the first column included; for real-valued
    inputs the chosen column's oracle logit is within the two tolerances of the oracle's maximum,
    the value within tolerance of that logit, and the index is the oracle's wherever the oracle's
    best and second-best logits are further apart than their tolerances.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import FINITE_SCALES, random_case, say, to_device_packed

pytestmark = pytest.mark.gpu

# (path, split, M): every kernel family and its argmax writer, ragged M across row blocks/slabs.
CASES = [(nv.PATH_DOT, 16, 1), (nv.PATH_DOT, 4, 3), (nv.PATH_DOT, 8, 8),
         (nv.PATH_MFMA, 4, 5), (nv.PATH_MFMA, 8, 16), (nv.PATH_MFMA, 8, 33),
         (nv.PATH_BATCH, 0, 40), (nv.PATH_BATCH, 32, 128), (nv.PATH_BATCH, 64, 130),
         (nv.PATH_BATCH, 16, 64), (nv.PATH_BATCH, 128, 129), (nv.PATH_BATCH, 128, 100),
         (nv.PATH_INVARIANT, 0, 1), (nv.PATH_INVARIANT, 0, 17),
         (nv.PATH_AUTO, 0, 1), (nv.PATH_AUTO, 0, 16), (nv.PATH_AUTO, 0, 128)]


def _first_max(Y):
    """First column of each row's maximum of a GPU Y, -0 taken as +0 (numpy's argmax)."""
    return np.argmax(Y, axis=1)


def _run(X, packed, device, path, split):
    Y = nv.gemm(X.to(device), packed.Wq, packed.Ws, packed.g, packed.N, path=path, split=split)
    idx, val = nv.gemm_argmax(X.to(device), packed.Wq, packed.Ws, packed.g, packed.N, path=path,
                              split=split)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()


def _check_fused_equals_unfused(Y, idx, val, label):
    want = _first_max(Y)
    assert np.array_equal(idx, want), f"{label}: index differs from the GEMM's argmax"
    best = Y[np.arange(len(Y)), want] + np.float32(0.0)     # -0 -> +0
    assert np.array_equal(val.view(np.uint32), best.astype(np.float32).view(np.uint32)), \
        f"{label}: value differs from the GEMM's maximum"


def _check_against_oracle(idx, val, Yref, A, label):
    tol = oracle.tolerance(A)
    rows = np.arange(len(Yref))
    ref = oracle.argmax_rows(Yref)
    gap_ok = Yref[rows, idx] >= Yref[rows, ref] - (tol[rows, idx] + tol[rows, ref])
    assert gap_ok.all(), f"{label}: chosen column is not a maximum within tolerance"
    assert (np.abs(val.astype(np.float64) - Yref[rows, idx]) <= tol[rows, idx]).all(), \
        f"{label}: value outside tolerance"
    # Where the oracle's winner is clear of every other column, the index is unique.
    order = np.argsort(-Yref, axis=1, kind="stable")
    second = order[:, 1] if Yref.shape[1] > 1 else order[:, 0]
    clear = Yref[rows, ref] - Yref[rows, second] > tol[rows, ref] + tol[rows, second]
    if Yref.shape[1] > 1:
        assert np.array_equal(idx[clear], ref[clear]), f"{label}: clear winner missed"


@pytest.mark.parametrize("path,split,M", CASES)
def test_argmax_matches_gemm_and_oracle(device, path, split, M):
    for N, K in [(1003, 1024), (4099, 272), (65, 5120)]:
        X, Wq, Ws, g = random_case(11 * M + N + K, M, N, K, FINITE_SCALES)
        label = f"argmax path={path} split={split} M={M} N={N} K={K}"
        say(label)
        packed = to_device_packed(Wq, Ws, g, device)
        Y, idx, val = _run(X, packed, device, path, split)
        _check_fused_equals_unfused(Y, idx, val, label)
        Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
        _check_against_oracle(idx, val, Yref, A, label)


@pytest.mark.parametrize("path,split,M", [c for c in CASES if c[0] != nv.PATH_INVARIANT])
def test_exact_sums_and_ties_match_oracle_exactly(device, path, split, M):
    """Scales in {0.5, 1, 2}, g = 1, integer X: exact logits. Columns copied from earlier columns
    (across workgroups and within a group) tie exactly; the first must win, as in the oracle."""
    N, K = 2053, 1024
    gen = inputs.generator(500 + M)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=[0x30, 0x38, 0x40])
    X = inputs.integer_activations(gen, M, K)
    for dst, src in [(2052, 7), (1500, 3), (9, 8), (1027, 1026), (600, 2)]:
        Wq[dst] = Wq[src]
        Ws[dst] = Ws[src]
    Yref, _ = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), 1.0)
    label = f"exact argmax path={path} split={split} M={M}"
    say(label)
    packed = to_device_packed(Wq, Ws, 1.0, device)
    Y, idx, val = _run(X, packed, device, path, split)
    assert np.array_equal(Y.astype(np.float64), Yref), f"{label}: GEMM not exact"
    assert np.array_equal(idx, oracle.argmax_rows(Yref)), f"{label}: index differs from oracle"
    assert np.array_equal(val.astype(np.float64), Yref.max(axis=1) + 0.0), label


def test_constructed_ties_at_the_maximum(device):
    """Every row's maximum is reached by several columns (one per workgroup region); the first."""
    N, K, M = 4096, 512, 4
    Wq = np.full((N, K // 2), 0x11, dtype=np.uint8)          # 0.5 everywhere
    Ws = np.full((N, K // 16), 0x38, dtype=np.uint8)          # scale 1
    winners = [3000, 77, 3999, 1024]
    for n in winners:
        Wq[n] = 0x77                                          # 6.0 everywhere
    X = torch.ones(M, K, dtype=torch.bfloat16)
    packed = to_device_packed(torch.from_numpy(Wq), torch.from_numpy(Ws), 1.0, device)
    for path, split in [(nv.PATH_DOT, 16), (nv.PATH_MFMA, 8), (nv.PATH_BATCH, 0),
                        (nv.PATH_BATCH, 32)]:
        say(f"constructed ties path={path}")
        _, idx, val = _run(X, packed, device, path, split)
        assert idx.tolist() == [77] * M, (path, idx)
        assert val.tolist() == [6.0 * K] * M


def test_all_negative_and_zero_rows(device):
    """Rows of X that make every logit negative pick the value nearest zero; a zero row makes all
    logits zero (+0 or -0) and picks column 0."""
    N, K = 300, 256
    gen = inputs.generator(91)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=[0x38])
    Wq = np.asarray(Wq) | 0x88                                # every code negative (or -0)
    X = torch.zeros(3, K, dtype=torch.bfloat16)
    X[0] = 1.0
    X[1] = 0.5
    Yref, _ = oracle.gemm(inputs.bf16_bits(X), Wq, np.asarray(Ws), 1.0)
    packed = to_device_packed(torch.from_numpy(Wq), Ws, 1.0, device)
    for path, split in [(nv.PATH_DOT, 16), (nv.PATH_MFMA, 4), (nv.PATH_BATCH, 0)]:
        say(f"negative rows path={path}")
        Y, idx, val = _run(X, packed, device, path, split)
        assert np.array_equal(idx, oracle.argmax_rows(Yref)), (path, idx)
        assert idx[2] == 0 and val[2] == 0.0 and not np.signbit(val[2])


def test_invariant_argmax_is_the_same_for_any_m(device):
    """In the batch-invariant mode a row's greedy token and logit do not depend on M."""
    N, K = 2000, 1024
    X, Wq, Ws, g = random_case(4242, 130, N, K, FINITE_SCALES)
    packed = to_device_packed(Wq, Ws, g, device)
    _, idx_all, val_all = _run(X, packed, device, nv.PATH_INVARIANT, 0)
    for m0, m1 in [(0, 1), (5, 6), (0, 16), (120, 130), (3, 67)]:
        say(f"invariant argmax rows {m0}:{m1}")
        _, idx, val = _run(X[m0:m1], packed, device, nv.PATH_INVARIANT, 0)
        assert np.array_equal(idx, idx_all[m0:m1])
        assert np.array_equal(val.view(np.uint32), val_all[m0:m1].view(np.uint32))


@pytest.fixture(scope="module")
def lm_head(device):
    """The lm_head of the dense layer family, K = 5120, N = 151936, from the workload recipe
    (seed 9): GPU-packed weights and the oracle's own packing of the same fp32 tensor."""
    K, N = inputs.LM_HEAD_SHAPE
    gen = inputs.generator(9)
    W = inputs.weights(gen, K, N)
    say("lm_head: packing on the GPU and in the oracle")
    p = nv.pack(W.to(device))
    torch.cuda.synchronize()
    Wq_o, Ws_o, g_o = oracle.quantize(W.numpy())
    return p, (Wq_o, Ws_o, g_o), gen


@pytest.mark.parametrize("M", [1, 3, 16, 128])
def test_lm_head_shape(device, lm_head, M):
    """nvfp4_gemm_argmax's automatic path at the lm_head shape (M = 3: the dot-product kernel
    with two workgroups per compute unit; M = 16: the 16-row kernel's chunks of unequal tiles);
    the oracle on every column of every row."""
    p, (Wq_o, Ws_o, g_o), gen = lm_head
    X = inputs.activations(gen, M, inputs.LM_HEAD_SHAPE[0])
    say(f"lm_head argmax M={M}")
    Y, idx, val = _run(X, p, device, nv.PATH_AUTO, 0)
    _check_fused_equals_unfused(Y, idx, val, f"lm_head M={M}")
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq_o, Ws_o, g_o)
    _check_against_oracle(idx, val, Yref, A, f"lm_head M={M}")


def test_graph_replays_match_eager(device):
    """gemm_argmax captured in a HIP graph reproduces the eager result on every replay."""
    gen = inputs.generator(31)
    shapes = [(1, 151936 // 8, 5120), (16, 4096, 1024), (128, 2048, 1024)]
    runs = []
    for M, N, K in shapes:
        W = inputs.weights(gen, K, N).to(device)
        p = nv.pack(W)
        X = inputs.activations(gen, M, K).to(device)
        idx = torch.empty(M, dtype=torch.int32, device=device)
        val = torch.empty(M, dtype=torch.float32, device=device)
        ws = nv.argmax_workspace(M, device)
        runs.append((X, p, idx, val, ws))

    def step():
        for X, p, idx, val, ws in runs:
            nv.gemm_argmax(X, p.Wq, p.Ws, p.g, p.N, out=(idx, val), workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [(i.clone(), v.clone()) for _, _, i, v, _ in runs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for _, _, i, v, ws in runs:
            i.fill_(-7)
            v.fill_(float("nan"))
            ws.fill_(0xAB)                                   # stale workspace between replays
        torch.cuda.synchronize()
        say(f"argmax graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for n, ((_, _, i, v, _), (ei, ev)) in enumerate(zip(runs, eager)):
            assert torch.equal(i, ei) and torch.equal(v, ev), f"replay {rep}: call {n} differs"


@pytest.mark.parametrize("N", [1, 2, 5])
@pytest.mark.parametrize("M", [1, 16, 128])
def test_tiny_and_ragged_vocabularies(device, N, M):
    """One, two and five columns (fewer than a 4-column group): the fold still picks the first
    maximum of the GEMM's own output."""
    K = 64
    X, Wq, Ws, g = random_case(9000 + 10 * N + M, M, N, K, FINITE_SCALES)
    say(f"tiny argmax M={M} N={N}")
    packed = to_device_packed(Wq, Ws, g, device)
    Y, idx, val = _run(X, packed, device, nv.PATH_AUTO, 0)
    _check_fused_equals_unfused(Y, idx, val, f"tiny M={M} N={N}")
    assert idx.min() >= 0 and idx.max() < N

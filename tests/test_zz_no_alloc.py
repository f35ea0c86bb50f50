"""nvfp4_gemm_argmax_noalloc (keys in the library's static device array) against
nvfp4_gemm_argmax (keys in a caller workspace), through the C ABI.

Two calls in a row, the second with fewer rows and a narrower weight, so it runs on an array that
still holds the first call's keys; each must give the same index and value bits as the
workspace entry point (the same kernels and plan). Plus the limit: one row more than the array
holds is refused on the host.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import FINITE_SCALES, random_case, say, to_device_packed

pytestmark = pytest.mark.gpu

# (M, N, K): the largest row count the array holds on a 256-CU device, then smaller calls
# (16-row kernel, dot-product kernel) on narrower weights.
CALLS = [(128, 30011, 1024), (16, 7001, 2048), (3, 5003, 512)]


def _noalloc(X, p, N, device):
    M, K = X.shape
    index = torch.full((M,), -7, dtype=torch.int32, device=device)
    value = torch.full((M,), float("nan"), dtype=torch.float32, device=device)
    st = nv.nvfp4_gemm_argmax_noalloc(M, N, K, X.data_ptr(), p.Wq.data_ptr(), p.Ws.data_ptr(),
                                      p.g.data_ptr(), index.data_ptr(), value.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == nv.SUCCESS, nv.status_string(st)
    return index, value


def _with_workspace(X, p, N, device):
    M, K = X.shape
    index = torch.full((M,), -9, dtype=torch.int32, device=device)
    value = torch.full((M,), float("nan"), dtype=torch.float32, device=device)
    ws = torch.empty(nv.nvfp4_argmax_workspace_bytes(M), dtype=torch.uint8, device=device)
    st = nv.nvfp4_gemm_argmax(M, N, K, X.data_ptr(), p.Wq.data_ptr(), p.Ws.data_ptr(),
                              p.g.data_ptr(), index.data_ptr(), value.data_ptr(), ws.data_ptr(),
                              ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == nv.SUCCESS, nv.status_string(st)
    return index, value


def test_noalloc_matches_workspace_entry_point(device):
    for rep in range(2):
        for i, (M, N, K) in enumerate(CALLS):
            label = f"noalloc argmax rep={rep} call={i} M={M} N={N} K={K}"
            say(label)
            X, Wq, Ws, g = random_case(9300 + i, M, N, K, FINITE_SCALES)
            p = to_device_packed(Wq, Ws, g, device)
            Xd = X.to(device)
            i0, v0 = _noalloc(Xd, p, N, device)
            torch.cuda.synchronize()
            i1, v1 = _with_workspace(Xd, p, N, device)
            torch.cuda.synchronize()
            assert torch.equal(i0.cpu(), i1.cpu()), f"{label}: index differs"
            assert np.array_equal(v0.cpu().numpy().view(np.uint32),
                                  v1.cpu().numpy().view(np.uint32)), f"{label}: value differs"
            if rep == 0 and i > 0:
                # The oracle's greedy token where the top two logits are apart by more than the
                # GEMM's tolerance.
                Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
                idx_ref = oracle.argmax_rows(Yref)
                tol = oracle.tolerance(A)
                top2 = np.sort(Yref, axis=1)[:, -2:]
                clear = (top2[:, 1] - top2[:, 0]) > 2 * tol.max(axis=1)
                assert clear.any(), f"{label}: no row with a clear winner"
                got = i0.cpu().numpy()
                assert np.array_equal(got[clear], idx_ref[clear]), f"{label}: vs oracle"


def test_noalloc_rejects_rows_beyond_the_array(device):
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    limit = (4 << 20) // (8 * 16 * cus)
    M, N, K = limit + 1, 64, 256
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=device)
    Wq = torch.zeros(nv.nvfp4_codes_bytes(N, K), dtype=torch.uint8, device=device)
    Ws = torch.zeros(nv.nvfp4_scales_bytes(N, K), dtype=torch.uint8, device=device)
    g = torch.ones(1, dtype=torch.float32, device=device)
    index = torch.empty((M,), dtype=torch.int32, device=device)
    value = torch.empty((M,), dtype=torch.float32, device=device)
    st = nv.nvfp4_gemm_argmax_noalloc(M, N, K, X.data_ptr(), Wq.data_ptr(), Ws.data_ptr(),
                                      g.data_ptr(), index.data_ptr(), value.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == nv.ERROR_SCRATCH_LIMIT

"""The C ABI without a GPU: libnvfp4.so loads, exports every function include/nvfp4.h declares,
and rejects bad arguments on the host before any HIP call (so these run in a CPU container).

No call here reaches a kernel: every argument set is invalid by construction, and the ABI
validates before touching the runtime.
"""
import ctypes
import os
import re
import subprocess

import pytest

import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

# Plausible-looking device addresses; never dereferenced because validation fails first.
A16 = 0x7F0000000000
A16B = 0x7F0000100000
A16C = 0x7F0000200000
A16D = 0x7F0000300000
A16E = 0x7F0000400000
A16F = 0x7F0000600000   # workspace


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB):
        build.build()
    return binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) >= {"nvfp4_pack", "nvfp4_gemm", "nvfp4_gemm_path", "nvfp4_status_string",
                          "nvfp4_abi_version", "nvfp4_codes_bytes", "nvfp4_scales_bytes",
                          "nvfp4_gemm_argmax", "nvfp4_gemm_argmax_path",
                          "nvfp4_argmax_workspace_bytes"}
    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    for name in names:
        assert name in exported, f"{name} declared in nvfp4.h but not exported"
        assert hasattr(lib, name)


def test_abi_version_and_strings(lib):
    assert nv.abi_version() == 7
    for st in (nv.SUCCESS, nv.ERROR_INVALID_VALUE, nv.ERROR_MISALIGNED, nv.ERROR_LAUNCH,
               nv.ERROR_SCRATCH_LIMIT):
        assert nv.status_string(st)
    assert nv.status_string(99) == "unknown status"


@pytest.mark.parametrize("M,N,K", [(0, 16, 256), (-1, 16, 256), (1, 0, 256), (1, -5, 256),
                                   (1, 16, 0), (1, 16, 8), (1, 16, 17), (1, 16, 264 + 1),
                                   (1, 16, -16), (1, 16, 2 ** 22 + 16)])
def test_gemm_rejects_bad_sizes(lib, M, N, K):
    st = nv.nvfp4_gemm(M, N, K, A16, A16B, A16C, A16D, A16E, None)
    assert st == nv.ERROR_INVALID_VALUE


def test_gemm_rejects_null_pointers(lib):
    args = [A16, A16B, A16C, A16D, A16E]
    for i in range(5):
        bad = list(args)
        bad[i] = None
        assert nv.nvfp4_gemm(1, 16, 256, *bad, None) == nv.ERROR_INVALID_VALUE


def test_gemm_rejects_misaligned_pointers(lib):
    # X, Wq, Wscale need 16 bytes; gscale and Y need 4.
    for i, off in [(0, 8), (1, 4), (2, 1), (3, 2), (4, 2)]:
        bad = [A16, A16B, A16C, A16D, A16E]
        bad[i] += off
        assert nv.nvfp4_gemm(1, 16, 256, *bad, None) == nv.ERROR_MISALIGNED, i


def test_gemm_path_rejects_bad_options(lib):
    ptrs = [A16, A16B, A16C, A16D, A16E]
    assert nv.nvfp4_gemm_path(6, 0, 1, 16, 256, *ptrs, None) == nv.ERROR_INVALID_VALUE
    assert nv.nvfp4_gemm_path(-1, 0, 1, 16, 256, *ptrs, None) == nv.ERROR_INVALID_VALUE
    for split in (1, 2, 3, 32, -1):
        assert nv.nvfp4_gemm_path(0, split, 1, 16, 256, *ptrs, None) == nv.ERROR_INVALID_VALUE
    # the dot-product kernel covers M <= 8 only
    assert nv.nvfp4_gemm_path(nv.PATH_DOT, 0, 9, 16, 256, *ptrs, None) == nv.ERROR_INVALID_VALUE
    # the matrix-core kernel runs 4 or 8 waves per workgroup
    assert nv.nvfp4_gemm_path(nv.PATH_MFMA, 16, 16, 16, 256, *ptrs, None) == \
        nv.ERROR_INVALID_VALUE
    # the slab kernel's split is the rows of a row group: 16, 32, 64 or 128 (0: chosen)
    for split in (1, 2, 4, 8, 12, 256):
        assert nv.nvfp4_gemm_path(nv.PATH_BATCH, split, 128, 16, 256, *ptrs, None) == \
            nv.ERROR_INVALID_VALUE
    # path 4 (K cut across workgroups through a library workspace) no longer exists
    for split in (0, 2, 4, 8):
        assert nv.nvfp4_gemm_path(4, split, 128, 16, 256, *ptrs, None) == \
            nv.ERROR_INVALID_VALUE
    # the batch-invariant mode has no split to choose
    for split in (1, 2, 4, 8):
        assert nv.nvfp4_gemm_path(nv.PATH_INVARIANT, split, 16, 16, 256, *ptrs, None) == \
            nv.ERROR_INVALID_VALUE
    # the wave counts of the other kernels are 4, 8 or 16
    for split in (1, 2, 12):
        assert nv.nvfp4_gemm_path(nv.PATH_MFMA, split, 16, 16, 256, *ptrs, None) == \
            nv.ERROR_INVALID_VALUE
        if split != 12:   # 12 wavefronts is a dot-product kernel size
            assert nv.nvfp4_gemm_path(nv.PATH_DOT, split, 1, 16, 256, *ptrs, None) == \
                nv.ERROR_INVALID_VALUE
    assert nv.nvfp4_gemm_path(nv.PATH_BATCH, 12, 128, 16, 256, *ptrs, None) == \
        nv.ERROR_INVALID_VALUE


def test_gemm_rejects_overflowing_sizes(lib):
    # M * K * 2 bytes of X exceeds the documented 2^62-byte limit.
    big = 2 ** 31 - 1
    st = nv.nvfp4_gemm(big, big, 2 ** 31 - 16, A16, A16B, A16C, A16D, A16E, None)
    assert st == nv.ERROR_INVALID_VALUE


def test_pack_rejects_bad_arguments(lib):
    ok = [A16, A16B, A16C, A16D]
    assert nv.nvfp4_pack(8, 16, *ok, None) == nv.ERROR_INVALID_VALUE
    assert nv.nvfp4_pack(24, 16, *ok, None) == nv.ERROR_INVALID_VALUE
    assert nv.nvfp4_pack(256, 0, *ok, None) == nv.ERROR_INVALID_VALUE
    for i in range(4):
        bad = list(ok)
        bad[i] = None
        assert nv.nvfp4_pack(256, 16, *bad, None) == nv.ERROR_INVALID_VALUE
    for i, off in [(0, 4), (1, 8), (2, 2), (3, 2)]:
        bad = list(ok)
        bad[i] += off
        assert nv.nvfp4_pack(256, 16, *bad, None) == nv.ERROR_MISALIGNED


def test_tensor_helpers_require_device_tensors(lib):
    import torch
    with pytest.raises(ValueError):
        nv.gemm(torch.zeros(1, 32, dtype=torch.bfloat16), torch.zeros(1, 1, 4, 16, dtype=torch.uint8),
                torch.zeros(1, 1, 4, 2, dtype=torch.uint8), torch.ones(1), 4)
    with pytest.raises(ValueError):
        nv.pack(torch.zeros(32, 4))


def test_packed_sizes(lib):
    """Bytes of the packed arrays: 64 resp. 8 per (4-column group, 32-k chunk), padded up."""
    for N, K in [(1, 16), (4, 32), (5, 48), (7168, 5120), (5120, 17408), (151936, 5120)]:
        groups, chunks = -(-N // 4), -(-K // 32)
        assert nv.nvfp4_codes_bytes(N, K) == 64 * groups * chunks
        assert nv.nvfp4_scales_bytes(N, K) == 8 * groups * chunks
        assert nv.codes_shape(N, K) == (groups, chunks, 4, 16)
        assert nv.scales_shape(N, K) == (groups, chunks, 4, 2)
    assert nv.nvfp4_codes_bytes(0, 32) == 0 and nv.nvfp4_scales_bytes(4, 0) == 0


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(build, "LIB", str(tmp_path / "absent.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(ImportError):
        binding.load_library()


# ---- nvfp4_gemm_argmax: the same validation, plus the outputs and the workspace ----

A8F = 0x7F0000500000   # index
A8G = 0x7F0000600000   # value
A8H = 0x7F0000700000   # workspace
BIG_WS = 1 << 40       # larger than any workspace the library asks for


def _argmax(M, N, K, ptrs=None, ws_bytes=BIG_WS, path=None, split=0):
    p = ptrs or [A16, A16B, A16C, A16D, A8F, A8G, A8H]
    if path is None:
        return nv.nvfp4_gemm_argmax(M, N, K, *p, ws_bytes, None)
    return nv.nvfp4_gemm_argmax_path(path, split, M, N, K, *p, ws_bytes, None)


@pytest.mark.parametrize("M,N,K", [(0, 16, 256), (1, 0, 256), (1, 16, 8), (1, 16, 17),
                                   (1, 16, 2 ** 22 + 16)])
def test_argmax_rejects_bad_sizes(lib, M, N, K):
    assert _argmax(M, N, K) == nv.ERROR_INVALID_VALUE


def test_argmax_rejects_null_and_misaligned(lib):
    good = [A16, A16B, A16C, A16D, A8F, A8G, A8H]
    for i in range(len(good)):
        bad = list(good)
        bad[i] = 0
        assert _argmax(1, 16, 256, bad) == nv.ERROR_INVALID_VALUE, i
    # X, Wq, Wscale need 16 bytes; gscale, index, value 4; the workspace 8
    for i, off in [(0, 8), (1, 8), (2, 4), (3, 2), (4, 2), (5, 2), (6, 4)]:
        bad = list(good)
        bad[i] += off
        assert _argmax(1, 16, 256, bad) == nv.ERROR_MISALIGNED, i


def test_argmax_rejects_small_workspace_and_bad_paths(lib):
    need = nv.nvfp4_argmax_workspace_bytes(3)
    assert need >= 3 * 8 * 16 and need % (3 * 8) == 0
    assert nv.nvfp4_argmax_workspace_bytes(0) == 0
    assert nv.nvfp4_argmax_workspace_bytes(6) == 2 * need
    assert _argmax(3, 16, 256, ws_bytes=need - 1) == nv.ERROR_INVALID_VALUE
    assert _argmax(1, 16, 256, path=6) == nv.ERROR_INVALID_VALUE
    assert _argmax(9, 16, 256, path=nv.PATH_DOT) == nv.ERROR_INVALID_VALUE
    assert _argmax(16, 16, 256, path=nv.PATH_INVARIANT, split=2) == nv.ERROR_INVALID_VALUE


def test_argmax_noalloc_host_checks(lib):
    """nvfp4_gemm_argmax_noalloc: the same size, pointer and alignment rules as the workspace
    entry point, and more rows than its 4 MiB key array holds (128 on 256 compute units, the
    count the library assumes without a device) return NVFP4_ERROR_SCRATCH_LIMIT, all before
    any HIP call."""
    good = [A16, A16B, A16C, A16D, A8F, A8G]

    def call(M, N, K, p=None):
        return nv.nvfp4_gemm_argmax_noalloc(M, N, K, *(p or good), None)

    assert call(0, 16, 256) == nv.ERROR_INVALID_VALUE
    assert call(1, 16, 24) == nv.ERROR_INVALID_VALUE
    for i in range(len(good)):
        bad = list(good)
        bad[i] = 0
        assert call(1, 16, 256, bad) == nv.ERROR_INVALID_VALUE, i
    for i, off in [(0, 8), (1, 8), (2, 4), (3, 2), (4, 2), (5, 2)]:
        bad = list(good)
        bad[i] += off
        assert call(1, 16, 256, bad) == nv.ERROR_MISALIGNED, i
    assert call(129, 16, 256) == nv.ERROR_SCRATCH_LIMIT
    assert call(4096, 16, 256) == nv.ERROR_SCRATCH_LIMIT
    assert "static scratch" in nv.status_string(nv.ERROR_SCRATCH_LIMIT)


# ---- nvfp4_gemm_grouped: sizes, experts, pointers, alignment, rows per item ----

def _grouped(T, E, N, K, ptrs=None, rpi=0):
    p = ptrs or [A16, A8F, A16B, A16C, A16D, A16E]
    return nv.nvfp4_gemm_grouped(T, E, N, K, *p, rpi, None)


@pytest.mark.parametrize("T,E,N,K", [(-1, 4, 16, 256), (1, 0, 16, 256), (1, 2049, 16, 256),
                                     (1, 4, 0, 256), (1, 4, 16, 8), (1, 4, 16, 24),
                                     (1, 4, 16, 2 ** 22 + 16), (2 ** 31 - 1, 4, 2 ** 12, 16)])
def test_grouped_rejects_bad_sizes(lib, T, E, N, K):
    assert _grouped(T, E, N, K) == nv.ERROR_INVALID_VALUE


def test_grouped_rejects_null_misaligned_and_rows_per_item(lib):
    good = [A16, A8F, A16B, A16C, A16D, A16E]
    for i in range(len(good)):
        bad = list(good)
        bad[i] = 0
        assert _grouped(4, 8, 16, 256, bad) == nv.ERROR_INVALID_VALUE, i
    # X, Wq, Wscale need 16 bytes; offsets, gscale, Y 4
    for i, off in [(0, 8), (1, 2), (2, 4), (3, 8), (4, 2), (5, 2)]:
        bad = list(good)
        bad[i] += off
        assert _grouped(4, 8, 16, 256, bad) == nv.ERROR_MISALIGNED, i
    for rpi in (-1, 3, 8):
        assert _grouped(4, 8, 16, 256, rpi=rpi) == nv.ERROR_INVALID_VALUE


def test_grouped_with_no_rows_does_nothing(lib):
    # T = 0 is valid and launches nothing (so it needs no GPU)
    assert _grouped(0, 8, 16, 256) == nv.SUCCESS


# ---- nvfp4_gemm_fused: fuse flags, sizes, eps, pointers, alignment ----

def _fused(fuse, M, N, K, ptrs=None, eps=1e-6, ws=0, ws_bytes=0):
    p = ptrs or [A16, A16B, A16C, A16D, A16E, A8F]     # X, gamma, Wq, Wscale, gscale, out
    return nv.nvfp4_gemm_fused(fuse, M, N, K, p[0], p[1], eps, p[2], p[3], p[4], p[5], ws,
                               ws_bytes, None)


def test_fused_rejects_bad_arguments(lib):
    for fuse in (0, 4, -1):
        assert _fused(fuse, 1, 16, 256) == nv.ERROR_INVALID_VALUE
    assert _fused(nv.FUSE_SILU_MUL, 1, 20, 256) == nv.ERROR_INVALID_VALUE      # N % 8
    assert _fused(nv.FUSE_RMSNORM, 1, 16, 24) == nv.ERROR_INVALID_VALUE        # K % 16
    assert _fused(nv.FUSE_RMSNORM, 0, 16, 256) == nv.ERROR_INVALID_VALUE
    for eps in (-1e-6, float("nan"), float("inf")):
        assert _fused(nv.FUSE_RMSNORM, 1, 16, 256, eps=eps) == nv.ERROR_INVALID_VALUE
    good = [A16, A16B, A16C, A16D, A16E, A8F]
    for i in range(6):
        bad = list(good)
        bad[i] = 0
        st = _fused(nv.FUSE_RMSNORM, 1, 16, 256, bad)
        assert st == nv.ERROR_INVALID_VALUE, i
    # gamma is only needed for RMSNorm; then it needs 16 bytes
    bad = list(good)
    bad[1] += 8
    assert _fused(nv.FUSE_RMSNORM, 1, 16, 256, bad) == nv.ERROR_MISALIGNED
    # out: fp32 Y needs 4 bytes, bf16 H 2
    bad = list(good)
    bad[5] += 2
    assert _fused(nv.FUSE_RMSNORM, 1, 16, 256, bad) == nv.ERROR_MISALIGNED
    bad[5] = good[5] + 1
    assert _fused(nv.FUSE_SILU_MUL, 1, 16, 256, bad) == nv.ERROR_MISALIGNED


def test_fused_workspace_rules(lib):
    """The fused call's workspace: none needed where one kernel does everything (up to 4 rows
    with X in LDS, or no RMSNorm); otherwise the normalised X, M * K * 2 bytes rounded up to
    256; a call with less, or a null or misaligned workspace, is rejected before any HIP call."""
    assert nv.nvfp4_fused_workspace_bytes(nv.FUSE_SILU_MUL, 128, 16, 256) == 0
    assert nv.nvfp4_fused_workspace_bytes(nv.FUSE_RMSNORM, 1, 16, 256) == 0
    assert nv.nvfp4_fused_workspace_bytes(nv.FUSE_RMSNORM, 5, 16, 256) == 2560
    assert nv.nvfp4_fused_workspace_bytes(nv.FUSE_RMSNORM, 5, 16, 272) == 2816   # 2720 -> 2816
    need = nv.nvfp4_fused_workspace_bytes(nv.FUSE_RMSNORM | nv.FUSE_SILU_MUL, 128, 16, 5120)
    assert need == 128 * 5120 * 2
    assert nv.nvfp4_fused_workspace_bytes(0, 128, 16, 5120) == 0
    assert nv.nvfp4_fused_workspace_bytes(nv.FUSE_RMSNORM, 0, 16, 5120) == 0
    assert _fused(nv.FUSE_RMSNORM, 128, 16, 5120) == nv.ERROR_INVALID_VALUE            # none
    assert _fused(nv.FUSE_RMSNORM, 128, 16, 5120, ws=A16F, ws_bytes=need - 1) == \
        nv.ERROR_INVALID_VALUE                                                          # short
    assert _fused(nv.FUSE_RMSNORM, 128, 16, 5120, ws=0, ws_bytes=need) == \
        nv.ERROR_INVALID_VALUE                                                          # null
    assert _fused(nv.FUSE_RMSNORM, 128, 16, 5120, ws=A16F + 8, ws_bytes=need) == \
        nv.ERROR_MISALIGNED


# ---- plan choice with no GPU: every configuration is either rejected or reaches the launch ----

def _device_visible() -> bool:
    """False when the HIP runtime reports no device: then no call can start a kernel, so the
    library may be handed plausible-looking addresses that pass every host check."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return True
    n = ctypes.c_int(0)
    return hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0


SWEEP_M = (1, 2, 3, 4, 5, 8, 9, 16, 17, 33, 48, 49, 64, 65, 127, 128, 129, 257, 1000)
SWEEP_N = (16, 48, 80, 1040, 4352, 5120, 7168, 34816, 151936, 262144)
SWEEP_K = (16, 272, 640, 2176, 5120, 17408, 65536)
SPLITS = (0, 4, 8, 12, 16, 32, 64, 128)


def test_plans_cover_every_shape_without_a_device(lib):
    """Every planner runs on the host: for each shape, path and split the call either rejects the
    configuration (NVFP4_ERROR_INVALID_VALUE) or chooses a plan and reaches the first HIP call,
    which fails without a device (NVFP4_ERROR_LAUNCH). The automatic path, the batch and
    batch-invariant paths and the matrix-core path accept every shape here; the dot path every
    M <= 8. Planners assume 256 compute units when no device answers."""
    if _device_visible():
        pytest.skip("a GPU is visible: this sweep passes addresses that must never reach a kernel")
    inv, launch = nv.ERROR_INVALID_VALUE, nv.ERROR_LAUNCH
    ptrs = [A16, A16B, A16C, A16D, A16E]
    for M in SWEEP_M:
        for N in SWEEP_N:
            for K in SWEEP_K:
                for path in range(6):
                    for split in SPLITS:
                        st = nv.nvfp4_gemm_path(path, split, M, N, K, *ptrs, None)
                        assert st in (inv, launch), (M, N, K, path, split, st)
                accepts = [nv.PATH_AUTO, nv.PATH_MFMA, nv.PATH_BATCH, nv.PATH_INVARIANT]
                if M <= 8:
                    accepts.append(nv.PATH_DOT)
                for path in accepts:
                    st = nv.nvfp4_gemm_path(path, 0, M, N, K, *ptrs, None)
                    assert st == launch, (M, N, K, path, st)
                st = _argmax(M, N, K)
                assert st == launch, (M, N, K, st)
                for path in range(6):
                    assert _argmax(M, N, K, path=path) in (inv, launch), (M, N, K, path)
                st = nv.nvfp4_gemm_argmax_noalloc(M, N, K, A16, A16B, A16C, A16D, A8F, A8G, None)
                assert st == (launch if M <= 128 else nv.ERROR_SCRATCH_LIMIT), (M, N, K, st)
                for fuse in (nv.FUSE_RMSNORM, nv.FUSE_SILU_MUL,
                             nv.FUSE_RMSNORM | nv.FUSE_SILU_MUL):
                    need = nv.nvfp4_fused_workspace_bytes(fuse, M, N, K)
                    st = _fused(fuse, M, N, K, ws=A16F if need else 0, ws_bytes=need)
                    assert st == launch, (M, N, K, fuse, st)


def test_grouped_plans_without_a_device(lib):
    """The grouped call's plan for any token count, expert count and rows per item: accepted
    configurations reach the first HIP call (NVFP4_ERROR_LAUNCH without a device)."""
    if _device_visible():
        pytest.skip("a GPU is visible: this sweep passes addresses that must never reach a kernel")
    for T in (1, 2, 8, 15, 16, 17, 128, 1000):
        for E in (1, 8, 64, 128, 2048):
            for N, K in ((16, 16), (1536, 2048), (2048, 768), (5120, 17408)):
                for rpi in (0, 1, 2, 4):
                    st = _grouped(T, E, N, K, rpi=rpi)
                    assert st == nv.ERROR_LAUNCH, (T, E, N, K, rpi, st)

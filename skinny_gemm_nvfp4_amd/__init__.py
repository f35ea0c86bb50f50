"""MI355X-native NVFP4 skinny GEMM: Y[M,N] = X[M,K] . dequant(W)[K,N] for M = 1 .. 128.

The computation is the weight stream of LLM decode and speculative verification with NVFP4
weights (E2M1 codes, an E4M3 scale per 16 weights along K, an fp32 tensor scale), bf16 activations
and fp32 accumulation. The kernels are hand-written HIP for gfx950 in ``csrc/``, behind the C ABI of
``include/nvfp4.h`` (``libnvfp4.so``); ``binding`` marshals torch tensors into it.

The library is loaded on first use; nothing here runs on the CPU in its place.
"""
from .binding import (  # noqa: F401
    ERROR_INVALID_VALUE, ERROR_LAUNCH, ERROR_MISALIGNED, ERROR_SCRATCH_LIMIT, FUSE_RMSNORM, FUSE_SILU_MUL, PATH_AUTO,
    PATH_BATCH, PATH_DOT, PATH_INVARIANT, PATH_MFMA, SUCCESS,
    NVFP4Error, Packed, abi_version, argmax_workspace, codes_shape, fused_workspace, gemm,
    gemm_argmax, gemm_fused,
    gemm_grouped, interleave_gate_up, library_path, load_library, nvfp4_argmax_workspace_bytes, nvfp4_codes_bytes,
    nvfp4_fused_workspace_bytes, nvfp4_gemm, nvfp4_gemm_argmax, nvfp4_gemm_argmax_noalloc, nvfp4_gemm_argmax_path,
    nvfp4_gemm_fused, nvfp4_gemm_grouped,
    nvfp4_gemm_path,
    nvfp4_pack, nvfp4_scales_bytes, pack, pack_experts, scales_shape, status_string)

// api.cpp -- the extern "C" boundary of libnvfp4.so (declared in include/nvfp4.h).
//
// Every argument is checked on the host before the first HIP call, so an error return has no side
// effects and needs no GPU. Then the call enqueues its kernels on the caller's stream and returns
// without synchronising.
#include "nvfp4.h"

#include <stdint.h>

#include <algorithm>

#include "launch.h"

namespace {

constexpr unsigned long long kMaxBytes = 1ULL << 62;

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Sizes allowed by the ABI: 1 <= M, N; 16 <= K <= 2^22; K % 16 == 0; every array below 2^62
// bytes.
bool sizes_ok(long long M, long long N, long long K)
{
    if (M < 1 || N < 1 || K < 16 || K > nvfp4::kMaxK || (K % 16) != 0)
        return false;
    const unsigned long long m = (unsigned long long)M, n = (unsigned long long)N,
                             k = (unsigned long long)K;
    return m * k * 2ULL < kMaxBytes && n * k * 4ULL < kMaxBytes && m * n * 4ULL < kMaxBytes;
}

// Values `split` may take for any path (each path accepts a subset, checked when it is chosen).
bool split_ok(int split)
{
    switch (split) {
    case 0: case 4: case 8: case 12: case 16: case 32: case 64: case 128: return true;
    default: return false;
    }
}

nvfp4_status_t from_hip(hipError_t e)
{
    return e == hipSuccess ? NVFP4_SUCCESS : NVFP4_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

nvfp4_status_t nvfp4_pack(int K, int N, const float *W, uint8_t *Wq, uint8_t *Wscale,
                          float *gscale, void *stream)
{
    if (!sizes_ok(1, N, K))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!W || !Wq || !Wscale || !gscale)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(gscale, 4))
        return NVFP4_ERROR_MISALIGNED;
    return from_hip(nvfp4::launch_pack(K, N, W, Wq, Wscale, gscale,
                                       static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_gemm_path(int path, int split, int M, int N, int K, const uint16_t *X,
                               const uint8_t *Wq, const uint8_t *Wscale, const float *gscale,
                               float *Y, void *stream)
{
    if (!sizes_ok(M, N, K))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!X || !Wq || !Wscale || !gscale || !Y)
        return NVFP4_ERROR_INVALID_VALUE;
    if (path < NVFP4_PATH_AUTO || path > NVFP4_PATH_INVARIANT)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!split_ok(split))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(gscale, 4) ||
        !aligned(Y, 4))
        return NVFP4_ERROR_MISALIGNED;
    int p = path, s = split;
    if (!nvfp4::choose_config(M, N, K, &p, &s))
        return NVFP4_ERROR_INVALID_VALUE;
    nvfp4::GemmArgs a;
    a.X = X;
    a.Wq = Wq;
    a.Ws = Wscale;
    a.gscale = gscale;
    a.Y = Y;
    a.M = M;
    a.N = N;
    a.K = K;
    return from_hip(nvfp4::launch_gemm(p, s, a, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_gemm(int M, int N, int K, const uint16_t *X, const uint8_t *Wq,
                          const uint8_t *Wscale, const float *gscale, float *Y, void *stream)
{
    return nvfp4_gemm_path(NVFP4_PATH_AUTO, 0, M, N, K, X, Wq, Wscale, gscale, Y, stream);
}

uint64_t nvfp4_argmax_workspace_bytes(int M)
{
    if (M < 1)
        return 0;
    return (uint64_t)M * (uint64_t)nvfp4::kArgmaxSlotsPerCu *
           (uint64_t)nvfp4::device_compute_units() * 8u;
}

nvfp4_status_t nvfp4_gemm_argmax_path(int path, int split, int M, int N, int K,
                                      const uint16_t *X, const uint8_t *Wq,
                                      const uint8_t *Wscale, const float *gscale, int32_t *index,
                                      float *value, void *workspace, uint64_t workspace_bytes,
                                      void *stream)
{
    if (!sizes_ok(M, N, K))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!X || !Wq || !Wscale || !gscale || !index || !value || !workspace)
        return NVFP4_ERROR_INVALID_VALUE;
    if (path < NVFP4_PATH_AUTO || path > NVFP4_PATH_INVARIANT)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!split_ok(split))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(gscale, 4) ||
        !aligned(index, 4) || !aligned(value, 4) || !aligned(workspace, 8))
        return NVFP4_ERROR_MISALIGNED;
    if (workspace_bytes < nvfp4_argmax_workspace_bytes(M))
        return NVFP4_ERROR_INVALID_VALUE;
    int p = path, s = split;
    if (!nvfp4::choose_config(M, N, K, &p, &s))
        return NVFP4_ERROR_INVALID_VALUE;
    nvfp4::GemmArgs a;
    a.X = X;
    a.Wq = Wq;
    a.Ws = Wscale;
    a.gscale = gscale;
    a.Y = nullptr;
    a.M = M;
    a.N = N;
    a.K = K;
    a.keys = static_cast<unsigned long long *>(workspace);
    a.key_slots = 0;
    return from_hip(nvfp4::launch_gemm_argmax(p, s, a, index, value,
                                              static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_gemm_argmax(int M, int N, int K, const uint16_t *X, const uint8_t *Wq,
                                 const uint8_t *Wscale, const float *gscale, int32_t *index,
                                 float *value, void *workspace, uint64_t workspace_bytes,
                                 void *stream)
{
    return nvfp4_gemm_argmax_path(NVFP4_PATH_AUTO, 0, M, N, K, X, Wq, Wscale, gscale, index, value,
                                  workspace, workspace_bytes, stream);
}

nvfp4_status_t nvfp4_gemm_argmax_noalloc(int M, int N, int K, const uint16_t *X,
                                         const uint8_t *Wq, const uint8_t *Wscale,
                                         const float *gscale, int32_t *index, float *value,
                                         void *stream)
{
    if (!sizes_ok(M, N, K))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!X || !Wq || !Wscale || !gscale || !index || !value)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(gscale, 4) ||
        !aligned(index, 4) || !aligned(value, 4))
        return NVFP4_ERROR_MISALIGNED;
    if (M > nvfp4::argmax_scratch_rows())
        return NVFP4_ERROR_SCRATCH_LIMIT;
    int p = NVFP4_PATH_AUTO, s = 0;
    if (!nvfp4::choose_config(M, N, K, &p, &s))
        return NVFP4_ERROR_INVALID_VALUE;
    unsigned long long *keys = nullptr;
    if (nvfp4::argmax_scratch(&keys) != hipSuccess)
        return NVFP4_ERROR_LAUNCH;
    nvfp4::GemmArgs a;
    a.X = X;
    a.Wq = Wq;
    a.Ws = Wscale;
    a.gscale = gscale;
    a.Y = nullptr;
    a.M = M;
    a.N = N;
    a.K = K;
    a.keys = keys;
    a.key_slots = 0;
    return from_hip(nvfp4::launch_gemm_argmax(p, s, a, index, value,
                                              static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_gemm_grouped(int T, int E, int N, int K, const uint16_t *X,
                                  const int32_t *offsets, const uint8_t *Wq,
                                  const uint8_t *Wscale, const float *gscale, float *Y,
                                  int rows_per_item, void *stream)
{
    if (T < 0 || E < 1 || E > nvfp4::kGroupedMaxExperts)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!sizes_ok(std::max(T, 1), N, K))
        return NVFP4_ERROR_INVALID_VALUE;
    if (rows_per_item != 0 && rows_per_item != 1 && rows_per_item != 2 && rows_per_item != 4)
        return NVFP4_ERROR_INVALID_VALUE;
    // Every expert's weights, and the work items (row chunks x column groups), in range.
    const unsigned long long per = nvfp4::codes_bytes(N, K);
    if ((unsigned long long)E * per >= kMaxBytes ||
        (unsigned long long)T * (unsigned long long)nvfp4::num_groups(N) >= (1ULL << 40))
        return NVFP4_ERROR_INVALID_VALUE;
    if (T == 0)
        return NVFP4_SUCCESS;   // no rows: nothing to read or write (X and Y may be empty/null)
    if (!X || !offsets || !Wq || !Wscale || !gscale || !Y)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(offsets, 4) ||
        !aligned(gscale, 4) || !aligned(Y, 4))
        return NVFP4_ERROR_MISALIGNED;
    nvfp4::GroupedArgs a;
    a.X = X;
    a.offsets = offsets;
    a.Wq = Wq;
    a.Ws = Wscale;
    a.gscale = gscale;
    a.Y = Y;
    a.T = T;
    a.E = E;
    a.N = N;
    a.K = K;
    const int mr = nvfp4::grouped_rows_per_item(T, E, rows_per_item);
    return from_hip(nvfp4::launch_grouped(a, mr, static_cast<hipStream_t>(stream)));
}

uint64_t nvfp4_fused_workspace_bytes(int fuse, int M, int N, int K)
{
    if (fuse < 1 || fuse > (NVFP4_FUSE_RMSNORM | NVFP4_FUSE_SILU_MUL) || !sizes_ok(M, N, K))
        return 0;
    return nvfp4::fused_workspace_bytes((fuse & NVFP4_FUSE_RMSNORM) != 0,
                                        (fuse & NVFP4_FUSE_SILU_MUL) != 0, M, N, K);
}

nvfp4_status_t nvfp4_gemm_fused(int fuse, int M, int N, int K, const uint16_t *X,
                                const uint16_t *gamma, float eps, const uint8_t *Wq,
                                const uint8_t *Wscale, const float *gscale, void *out,
                                void *workspace, uint64_t workspace_bytes, void *stream)
{
    if (fuse < 1 || fuse > (NVFP4_FUSE_RMSNORM | NVFP4_FUSE_SILU_MUL))
        return NVFP4_ERROR_INVALID_VALUE;
    const bool norm = (fuse & NVFP4_FUSE_RMSNORM) != 0;
    const bool silu = (fuse & NVFP4_FUSE_SILU_MUL) != 0;
    if (!sizes_ok(M, N, K) || (silu && N % 8 != 0))
        return NVFP4_ERROR_INVALID_VALUE;
    if (norm && !(eps >= 0.0f && eps <= 3.0e38f))   // also rejects NaN
        return NVFP4_ERROR_INVALID_VALUE;
    if (!X || !Wq || !Wscale || !gscale || !out || (norm && !gamma))
        return NVFP4_ERROR_INVALID_VALUE;
    const uint64_t need = nvfp4_fused_workspace_bytes(fuse, M, N, K);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(gscale, 4) ||
        (norm && !aligned(gamma, 16)) || !aligned(out, silu ? 2 : 4) ||
        (need > 0 && !aligned(workspace, 16)))
        return NVFP4_ERROR_MISALIGNED;
    nvfp4::GemmArgs a;
    a.X = X;
    a.Wq = Wq;
    a.Ws = Wscale;
    a.gscale = gscale;
    a.Y = silu ? nullptr : static_cast<float *>(out);
    a.H = silu ? static_cast<uint16_t *>(out) : nullptr;
    a.gamma = norm ? gamma : nullptr;
    a.eps = eps;
    a.M = M;
    a.N = N;
    a.K = K;
    a.workspace = need > 0 ? workspace : nullptr;
    a.workspace_bytes = need > 0 ? (size_t)workspace_bytes : 0;
    return from_hip(nvfp4::launch_gemm_fused(a, static_cast<hipStream_t>(stream)));
}

const char *nvfp4_status_string(nvfp4_status_t status)
{
    switch (status) {
    case NVFP4_SUCCESS: return "success";
    case NVFP4_ERROR_INVALID_VALUE: return "invalid value (size, null pointer or path)";
    case NVFP4_ERROR_MISALIGNED: return "misaligned pointer";
    case NVFP4_ERROR_LAUNCH: return "kernel launch failed";
    case NVFP4_ERROR_SCRATCH_LIMIT:
        return "more rows than the static scratch of nvfp4_gemm_argmax_noalloc holds";
    default: break;
    }
    return "unknown status";
}

int nvfp4_abi_version(void)
{
    return NVFP4_ABI_VERSION;
}

uint64_t nvfp4_codes_bytes(int N, int K)
{
    if (N < 1 || K < 1)
        return 0;
    return nvfp4::codes_bytes(N, K);
}

uint64_t nvfp4_scales_bytes(int N, int K)
{
    if (N < 1 || K < 1)
        return 0;
    return nvfp4::scales_bytes(N, K);
}

}  // extern "C"

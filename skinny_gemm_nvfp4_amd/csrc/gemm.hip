// gemm.hip -- kernel selection and launch for the NVFP4 skinny GEMM Y[M,N] = X[M,K] . dequant(W)[K,N].
//
// Three kernel families (headers in this directory):
//   * gemv_stream.h (NVFP4_PATH_STREAM): persistent dot-product kernel, one workgroup per compute
//     unit with an equal share of the columns, X staged in LDS. Decode (M = 1) and the smallest M.
//   * gemv.h (NVFP4_PATH_DOT): tiled dot-product kernel, one workgroup per 4 C columns. Used
//     when X does not fit in LDS for the persistent kernel.
//   * verify_stream.h (NVFP4_PATH_MFMA_STREAM): persistent bf16 matrix-core kernel, one workgroup
//     per compute unit and 16-row block of X (speculative verification), K % 128 == 0.
//   * mfma.h (NVFP4_PATH_MFMA): tiled bf16 matrix-core kernel for the other K.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <set>
#include <utility>

#include "gemv.h"
#include "gemv_stream.h"
#include "launch.h"
#include "mfma.h"
#include "verify_stream.h"

namespace nvfp4 {

namespace {

typedef void (*KernelFn)(GemmArgs);
typedef void (*StreamFn)(GemmArgs, StreamLayout);

constexpr int kStreamDepth = 4;             // units in flight per wavefront
constexpr int kMaxLds = 160 * 1024;         // LDS per workgroup on gfx950
constexpr int kDefaultLds = 64 * 1024;      // above this a kernel must opt in

// ---- tiled dot-product kernels: [MR - 1][split index], C columns per quad ----
#define NVFP4_DOT_SPLITS(R, C, NARROW)                                                     \
    {                                                                                      \
        &gemv_kernel<R, C, 1, NARROW>, &gemv_kernel<R, C, 2, NARROW>,                      \
            &gemv_kernel<R, C, 4, NARROW>, &gemv_kernel<R, C, 8, NARROW>                   \
    }
#define NVFP4_DOT_TABLE(NARROW)                                                            \
    {                                                                                      \
        NVFP4_DOT_SPLITS(1, 4, NARROW), NVFP4_DOT_SPLITS(2, 2, NARROW),                    \
            NVFP4_DOT_SPLITS(3, 2, NARROW), NVFP4_DOT_SPLITS(4, 2, NARROW),                \
            NVFP4_DOT_SPLITS(5, 1, NARROW), NVFP4_DOT_SPLITS(6, 1, NARROW),                \
            NVFP4_DOT_SPLITS(7, 1, NARROW), NVFP4_DOT_SPLITS(8, 1, NARROW)                 \
    }
const KernelFn kDotWide[8][4] = NVFP4_DOT_TABLE(false);
const KernelFn kDotNarrow[8][4] = NVFP4_DOT_TABLE(true);
const int kDotColumns[8] = {4, 2, 2, 2, 1, 1, 1, 1};  // C of each MR

// ---- persistent dot-product kernels: [variant][MR - 1][wave index] ----
// variant 0: K % 512 == 0 (FAST); 1: K % 64 == 0; 2: any other K % 16 == 0 (NARROW).
#define NVFP4_STREAM_WAVES(R, FAST, NARROW)                                                \
    {                                                                                      \
        &gemv_stream_kernel<R, 4, kStreamDepth, FAST, NARROW>,                             \
            &gemv_stream_kernel<R, 8, kStreamDepth, FAST, NARROW>,                         \
            &gemv_stream_kernel<R, 16, kStreamDepth, FAST, NARROW>                         \
    }
#define NVFP4_STREAM_TABLE(FAST, NARROW)                                                   \
    {                                                                                      \
        NVFP4_STREAM_WAVES(1, FAST, NARROW), NVFP4_STREAM_WAVES(2, FAST, NARROW),          \
            NVFP4_STREAM_WAVES(3, FAST, NARROW), NVFP4_STREAM_WAVES(4, FAST, NARROW),      \
            NVFP4_STREAM_WAVES(5, FAST, NARROW), NVFP4_STREAM_WAVES(6, FAST, NARROW),      \
            NVFP4_STREAM_WAVES(7, FAST, NARROW), NVFP4_STREAM_WAVES(8, FAST, NARROW)       \
    }
const StreamFn kStream[3][8][3] = {NVFP4_STREAM_TABLE(true, false),
                                   NVFP4_STREAM_TABLE(false, false),
                                   NVFP4_STREAM_TABLE(false, true)};

// ---- MFMA kernels: [MT - 1][split index], NT column tiles ----
#define NVFP4_MFMA_SPLITS(T, NT, NARROW)                                                   \
    {                                                                                      \
        &mfma_kernel<T, NT, 1, NARROW>, &mfma_kernel<T, NT, 2, NARROW>,                    \
            &mfma_kernel<T, NT, 4, NARROW>, &mfma_kernel<T, NT, 8, NARROW>                 \
    }
#define NVFP4_MFMA_TABLE(NARROW)                                                           \
    {                                                                                      \
        NVFP4_MFMA_SPLITS(1, 2, NARROW), NVFP4_MFMA_SPLITS(2, 2, NARROW),                  \
            NVFP4_MFMA_SPLITS(3, 1, NARROW), NVFP4_MFMA_SPLITS(4, 1, NARROW),              \
            NVFP4_MFMA_SPLITS(5, 1, NARROW), NVFP4_MFMA_SPLITS(6, 1, NARROW),              \
            NVFP4_MFMA_SPLITS(7, 1, NARROW), NVFP4_MFMA_SPLITS(8, 1, NARROW)               \
    }
const KernelFn kMfmaWide[8][4] = NVFP4_MFMA_TABLE(false);
const KernelFn kMfmaNarrow[8][4] = NVFP4_MFMA_TABLE(true);
const int kMfmaColumnTiles[8] = {2, 2, 1, 1, 1, 1, 1, 1};  // NT of each MT

// ---- persistent matrix-core kernels: [TC index][wave index] ----
// TC column tiles of 16 are processed together; the smallest TC >= the workgroup's tile count is
// used, so that X is read once per workgroup.
const int kVerifyTiles[6] = {1, 2, 3, 4, 6, 9};
#define NVFP4_VERIFY_WAVES(TC) {&verify_stream_kernel<TC, 4>, &verify_stream_kernel<TC, 8>}
const KernelFn kVerify[6][2] = {NVFP4_VERIFY_WAVES(1), NVFP4_VERIFY_WAVES(2),
                                NVFP4_VERIFY_WAVES(3), NVFP4_VERIFY_WAVES(4),
                                NVFP4_VERIFY_WAVES(6), NVFP4_VERIFY_WAVES(9)};

int split_index(int split)
{
    switch (split) {
    case 1: return 0;
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
    default: return -1;
    }
}

int wave_index(int waves)
{
    switch (waves) {
    case 4: return 0;
    case 8: return 1;
    case 16: return 2;
    default: return -1;
    }
}

// Compute units of the current device, read once per device.
int compute_units()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 256;
    if (dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0)
            return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Lets `fn` use up to `bytes` of LDS (above the 64 KB default), once per kernel and device.
hipError_t allow_lds(const void *fn, int bytes)
{
    if (bytes <= kDefaultLds)
        return hipSuccess;
    static std::mutex mu;
    static std::set<std::pair<int, const void *>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({dev, fn}))
        return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e == hipSuccess)
        done.insert({dev, fn});
    return e;
}

// Workgroups, column-tile chunk and LDS bytes of the persistent matrix-core kernel; false if the
// shape needs the tiled kernel (K % 128 != 0, or a workgroup's code bytes reach 2^31).
struct VerifyPlan {
    int grid, tc_index, lds;
};

bool verify_plan(int N, int K, int waves, VerifyPlan *P)
{
    if (K % kVerifyWindow != 0)
        return false;
    const int G = std::max(1, std::min(compute_units(), (N + 15) / 16));
    const int cmax = (N + G - 1) / G;
    if ((long long)cmax * (K / 2) >= (1LL << 31))
        return false;
    const int tiles = (cmax + 15) / 16;
    int ti = 5;
    for (int i = 0; i < 6; i++)
        if (kVerifyTiles[i] >= tiles) {
            ti = i;
            break;
        }
    P->grid = G;
    P->tc_index = ti;
    P->lds = verify_lds_bytes(kVerifyTiles[ti], waves);
    return P->lds <= kMaxLds;
}

// Workgroups and LDS layout of the persistent kernel; false if X does not fit in LDS.
bool stream_plan(int M, int N, int K, int MR, int W, int *grid, StreamLayout *L)
{
    const int G = std::max(1, std::min(compute_units(), (N + 3) / 4));
    L->nwin = (K + kStreamWindow - 1) / kStreamWindow;
    L->row_bytes = L->nwin * (kStreamWindow / 32) * kStreamSlot;
    const long long x_bytes = (long long)M * L->row_bytes;
    const int cmax = (N + G - 1) / G;
    L->ngroups = (cmax + 3) / 4;
    // A group of nwin consecutive units touches every wavefront whose run starts inside it.
    L->slots = 1;
    const int sizes[2] = {N / G, cmax};
    for (int i = 0; i < 2; i++) {
        const long long units = (long long)((sizes[i] + 3) / 4) * L->nwin;
        if (units == 0)
            continue;
        for (long long first = 0; first < units; first += L->nwin) {
            const int n = stream_owner(first + L->nwin - 1, W, units) -
                          stream_owner(first, W, units) + 1;
            L->slots = std::max(L->slots, n);
        }
    }
    const long long part_bytes = (long long)L->ngroups * L->slots * MR * 4 * 4;
    if (x_bytes + part_bytes > kMaxLds)
        return false;
    if ((long long)cmax * (K / 2) >= (1LL << 31))  // a workgroup's byte range must fit a buffer
        return false;
    L->x_bytes = (int)x_bytes;
    L->part_bytes = (int)part_bytes;
    *grid = G;
    return true;
}

}  // namespace

bool choose_config(int M, int N, int K, int *path, int *split)
{
    if (*path == kPathAuto)
        *path = (M <= 4) ? kPathStream : kPathMfmaStream;
    if (*path == kPathMfmaStream) {
        VerifyPlan P;
        if (*split == 0) {
            // Wide chunks keep more bytes in flight per wave; narrow ones need more waves.
            if (!verify_plan(N, K, 8, &P))
                P.tc_index = -1;
            *split = (P.tc_index >= 4) ? 4 : 8;
        }
        if (*split != 4 && *split != 8)
            return false;
        if (verify_plan(N, K, *split, &P))
            return true;
        *path = kPathMfma;  // K % 128 != 0: tiled kernel
        *split = 0;
    }
    if (*path == kPathStream) {
        if (M > kDotMaxM)
            return false;
        if (*split == 0)
            *split = 16;
        StreamLayout L;
        int grid;
        if (wave_index(*split) < 0)
            return false;
        if (stream_plan(M, N, K, M, *split, &grid, &L))
            return true;
        *path = kPathDot;  // X does not fit in LDS: tiled kernel
        *split = 0;
    }
    if (*path == kPathDot && M > kDotMaxM)
        return false;
    if (*path != kPathDot && *path != kPathMfma)
        return false;
    if (*split == 0) {
        // Enough waves to keep every compute unit streaming: aim for >= 2048 waves (8 per CU),
        // with at least two K windows per wave.
        const bool dot = *path == kPathDot;
        const int mt = M >= 128 ? 8 : (M + 15) / 16;
        const int cols = dot ? 4 * kDotColumns[M - 1] : 16 * kMfmaColumnTiles[mt - 1];
        const long long tiles = (N + cols - 1) / cols;
        const int window = dot ? kGemvWindow : kMfmaWindow;
        const int steps = (K + window - 1) / window;
        int w = 1;
        while (w < 8 && tiles * w < 2048 && steps >= 2 * w)
            w *= 2;
        *split = w;
    }
    return split_index(*split) >= 0;
}

hipError_t launch_gemm(int path, int split, const GemmArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();  // start from a clean error state
    if (path == kPathMfmaStream) {
        VerifyPlan P;
        if (!verify_plan(a.N, a.K, split, &P))
            return hipErrorInvalidValue;
        const KernelFn fn = kVerify[P.tc_index][split == 4 ? 0 : 1];
        const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), P.lds);
        if (e != hipSuccess)
            return e;
        const unsigned mblocks = (unsigned)((a.M + 15) / 16);
        hipLaunchKernelGGL(fn, dim3((unsigned)P.grid, mblocks), dim3(kWave * split), P.lds,
                           stream, a);
        return hipGetLastError();
    }
    if (path == kPathStream) {
        StreamLayout L;
        int grid = 0;
        if (!stream_plan(a.M, a.N, a.K, a.M, split, &grid, &L))
            return hipErrorInvalidValue;
        const int variant = (a.K % kStreamWindow == 0) ? 0 : (a.K % 64 == 0 ? 1 : 2);
        const int wi = wave_index(split);
        const StreamFn fn = kStream[variant][a.M - 1][wi];
        const int lds = L.x_bytes + L.part_bytes;
        const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), lds);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(fn, dim3(grid), dim3(kWave * split), lds, stream, a, L);
        return hipGetLastError();
    }
    const bool narrow = (a.K % 64) != 0;
    const int si = split_index(split);
    const dim3 block(kWave * split);
    KernelFn fn;
    dim3 grid;
    if (path == kPathDot) {
        const int cols = 4 * kDotColumns[a.M - 1];
        fn = (narrow ? kDotNarrow : kDotWide)[a.M - 1][si];
        grid = dim3((unsigned)((a.N + cols - 1) / cols), 1, 1);
    } else {
        const int mt = a.M >= 128 ? 8 : (a.M + 15) / 16;
        const int cols = 16 * kMfmaColumnTiles[mt - 1];
        const unsigned mchunks = (unsigned)((a.M + 16 * mt - 1) / (16 * mt));
        fn = (narrow ? kMfmaNarrow : kMfmaWide)[mt - 1][si];
        grid = dim3((unsigned)((a.N + cols - 1) / cols), mchunks, 1);
    }
    hipLaunchKernelGGL(fn, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4

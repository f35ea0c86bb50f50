// gemm.hip -- kernel selection and launch for the NVFP4 skinny GEMM Y[M,N] = X[M,K] . dequant(W)[K,N].
//
// Two persistent kernel families (headers in this directory), one workgroup per compute unit
// with an equal share of the 4-column groups:
//   * gemv_stream.h (NVFP4_PATH_DOT): dot products against X staged in LDS. Decode (M = 1) and
//     the smallest M.
//   * mfma_stream.h (NVFP4_PATH_MFMA): bf16 matrix cores on 16-row blocks of X (speculative
//     verification of one request), and every shape whose X does not fit in LDS.
//   * mfma_batch.h (NVFP4_PATH_BATCH): bf16 matrix cores, each weight decoded once for up to 128
//     rows of X (verification of several requests together).
#include <algorithm>
#include <atomic>
#include <mutex>
#include <set>
#include <utility>

#include "gemv_stream.h"
#include "launch.h"
#include "mfma_batch.h"
#include "mfma_stream.h"

namespace nvfp4 {

namespace {

typedef void (*KernelFn)(GemmArgs);
typedef void (*StreamFn)(GemmArgs, StreamLayout);

constexpr int kStreamDepth = 4;             // units in flight per wavefront
constexpr int kMaxLds = 160 * 1024;         // LDS per workgroup on gfx950
constexpr int kDefaultLds = 64 * 1024;      // above this a kernel must opt in

// ---- dot-product kernels: [FAST][MR - 1][wave index] ----
#define NVFP4_STREAM_WAVES(R, FAST)                                                        \
    {                                                                                      \
        &gemv_stream_kernel<R, 4, kStreamDepth, FAST>,                                     \
            &gemv_stream_kernel<R, 8, kStreamDepth, FAST>,                                 \
            &gemv_stream_kernel<R, 16, kStreamDepth, FAST>                                 \
    }
#define NVFP4_STREAM_TABLE(FAST)                                                           \
    {                                                                                      \
        NVFP4_STREAM_WAVES(1, FAST), NVFP4_STREAM_WAVES(2, FAST),                          \
            NVFP4_STREAM_WAVES(3, FAST), NVFP4_STREAM_WAVES(4, FAST),                      \
            NVFP4_STREAM_WAVES(5, FAST), NVFP4_STREAM_WAVES(6, FAST),                      \
            NVFP4_STREAM_WAVES(7, FAST), NVFP4_STREAM_WAVES(8, FAST)                       \
    }
const StreamFn kStream[2][8][3] = {NVFP4_STREAM_TABLE(false), NVFP4_STREAM_TABLE(true)};

// ---- matrix-core kernels: [FAST][TC index][wave index] ----
// TC column tiles of 16 are processed together; the smallest TC >= the workgroup's tile count is
// used, so that X is read once per workgroup.
const int kMfmaTiles[6] = {1, 2, 3, 4, 6, 9};
#define NVFP4_MFMA_WAVES(TC, FAST)                                                         \
    {                                                                                      \
        &mfma_stream_kernel<TC, 4, FAST>, &mfma_stream_kernel<TC, 8, FAST>                 \
    }
#define NVFP4_MFMA_TABLE(FAST)                                                             \
    {                                                                                      \
        NVFP4_MFMA_WAVES(1, FAST), NVFP4_MFMA_WAVES(2, FAST), NVFP4_MFMA_WAVES(3, FAST),   \
            NVFP4_MFMA_WAVES(4, FAST), NVFP4_MFMA_WAVES(6, FAST), NVFP4_MFMA_WAVES(9, FAST) \
    }
const KernelFn kMfma[2][6][2] = {NVFP4_MFMA_TABLE(false), NVFP4_MFMA_TABLE(true)};

// ---- batch kernels: 4 tile lanes (one wavefront per SIMD), TCW = 1..3 tiles each per pass,
// loads 2 windows ahead ----
constexpr int kBatchRing = 3;
const KernelFn kBatch[3] = {&mfma_batch_kernel<1, 4, kBatchRing>,
                            &mfma_batch_kernel<2, 4, kBatchRing>,
                            &mfma_batch_kernel<3, 4, kBatchRing>};
const int kBatchLds[3] = {mfma_batch_lds_bytes(1, 4, kBatchRing),
                          mfma_batch_lds_bytes(2, 4, kBatchRing),
                          mfma_batch_lds_bytes(3, 4, kBatchRing)};
constexpr int kBatchWaves = 4;

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

// Workgroups over the 4-column groups: one per compute unit, at most one per group.
int group_grid(int N)
{
    return std::max(1, std::min(compute_units(), num_groups(N)));
}

// A workgroup's code bytes must stay below 2^31 (buffer offsets are 32-bit).
bool bytes_fit(int N, int K, int grid)
{
    const long long gmax = (num_groups(N) + grid - 1) / grid;
    return gmax * (long long)num_chunks(K) * kChunkCodeBytes < (1LL << 31);
}

// Workgroups and LDS layout of the dot-product kernel; false if X does not fit in LDS.
bool stream_plan(int M, int N, int K, int MR, int W, int *grid, StreamLayout *L)
{
    const int G = group_grid(N);
    L->nwin = (K + kStreamWindow - 1) / kStreamWindow;
    L->row_bytes = L->nwin * (kStreamWindow / 32) * kStreamSlot;
    const long long x_bytes = (long long)M * L->row_bytes;
    const int NG = num_groups(N);
    L->ngroups = (NG + G - 1) / G;
    // A group of nwin consecutive units touches every wavefront whose run starts inside it.
    L->slots = 1;
    const int sizes[2] = {NG / G, L->ngroups};
    for (int i = 0; i < 2; i++) {
        const long long units = (long long)sizes[i] * L->nwin;
        if (units == 0)
            continue;
        for (long long first = 0; first < units; first += L->nwin) {
            const int n = stream_owner(first + L->nwin - 1, W, units) -
                          stream_owner(first, W, units) + 1;
            L->slots = std::max(L->slots, n);
        }
    }
    const long long part_bytes = (long long)L->ngroups * L->slots * MR * 4 * 4;
    if (x_bytes + part_bytes > kMaxLds || !bytes_fit(N, K, G))
        return false;
    L->x_bytes = (int)x_bytes;
    L->part_bytes = (int)part_bytes;
    *grid = G;
    return true;
}

// Workgroups, column-tile chunk and LDS bytes of the matrix-core kernel.
struct MfmaPlan {
    int grid, tc_index, lds;
};

bool mfma_plan(int N, int K, int waves, MfmaPlan *P)
{
    const int G = group_grid(N);
    if (!bytes_fit(N, K, G))
        return false;
    const int gmax = (num_groups(N) + G - 1) / G;
    const int tiles = (gmax + 3) / 4;
    int ti = 5;
    for (int i = 0; i < 6; i++)
        if (kMfmaTiles[i] >= tiles) {
            ti = i;
            break;
        }
    P->grid = G;
    P->tc_index = ti;
    P->lds = mfma_stream_lds_bytes(kMfmaTiles[ti], waves);
    return P->lds <= kMaxLds;
}

// Wavefronts of the matrix-core kernel when the caller leaves it open: wide chunks keep more
// bytes in flight per wavefront, narrow ones need more wavefronts.
int mfma_default_waves(int N, int K)
{
    MfmaPlan P;
    if (!mfma_plan(N, K, 8, &P))
        return 4;
    return kMfmaTiles[P.tc_index] >= 6 ? 4 : 8;
}

// Batch kernel for this shape, its LDS bytes and grid; false if a workgroup's bytes overflow.
// Only on request (NVFP4_PATH_BATCH): its loads still run about one window ahead, so
// nvfp4_gemm keeps the 16-row kernel for every M.
bool batch_plan(int N, int K, KernelFn *fn, int *lds, int *grid)
{
    const int G = group_grid(N);
    if (!bytes_fit(N, K, G))
        return false;
    const int gmax = (num_groups(N) + G - 1) / G;
    const int tiles = (gmax + 3) / 4;
    const int i = std::min(3, (tiles + kBatchWaves - 1) / kBatchWaves) - 1;
    *fn = kBatch[i];
    *lds = kBatchLds[i];
    *grid = G;
    return *lds <= kMaxLds;
}

}  // namespace

bool choose_config(int M, int N, int K, int *path, int *split)
{
    if (*path == kPathAuto)
        *path = (M <= 4) ? kPathDot : kPathMfma;
    if (*path == kPathBatch) {
        if (*split != 0 && *split != kBatchWaves)
            return false;
        *split = kBatchWaves;
        KernelFn fn;
        int lds, grid;
        return batch_plan(N, K, &fn, &lds, &grid);
    }
    if (*path == kPathDot) {
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
        *path = kPathMfma;  // X does not fit in LDS
        *split = 0;
    }
    if (*path != kPathMfma)
        return false;
    if (*split == 0)
        *split = mfma_default_waves(N, K);
    if (*split != 4 && *split != 8)
        return false;
    MfmaPlan P;
    return mfma_plan(N, K, *split, &P);
}

hipError_t launch_gemm(int path, int split, const GemmArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();  // start from a clean error state
    if (path == kPathDot) {
        StreamLayout L;
        int grid = 0;
        if (!stream_plan(a.M, a.N, a.K, a.M, split, &grid, &L))
            return hipErrorInvalidValue;
        const int fast = (a.K % kStreamWindow == 0) ? 1 : 0;
        const StreamFn fn = kStream[fast][a.M - 1][wave_index(split)];
        const int lds = L.x_bytes + L.part_bytes;
        const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), lds);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(fn, dim3(grid), dim3(kWave * split), lds, stream, a, L);
        return hipGetLastError();
    }
    if (path == kPathBatch) {
        KernelFn fn;
        int lds, grid;
        if (!batch_plan(a.N, a.K, &fn, &lds, &grid))
            return hipErrorInvalidValue;
        const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), lds);
        if (e != hipSuccess)
            return e;
        const unsigned slabs = (unsigned)((a.M + 16 * kBatchMaxBlocks - 1) / (16 * kBatchMaxBlocks));
        hipLaunchKernelGGL(fn, dim3((unsigned)grid, slabs), dim3(kWave * kBatchWaves), lds,
                           stream, a);
        return hipGetLastError();
    }
    if (path != kPathMfma)
        return hipErrorInvalidValue;
    MfmaPlan P;
    if (!mfma_plan(a.N, a.K, split, &P))
        return hipErrorInvalidValue;
    const int fast = (a.K % kMfmaWindow == 0) ? 1 : 0;
    const KernelFn fn = kMfma[fast][P.tc_index][split == 4 ? 0 : 1];
    const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), P.lds);
    if (e != hipSuccess)
        return e;
    const unsigned mblocks = (unsigned)((a.M + 15) / 16);
    hipLaunchKernelGGL(fn, dim3((unsigned)P.grid, mblocks), dim3(kWave * split), P.lds, stream,
                       a);
    return hipGetLastError();
}

}  // namespace nvfp4

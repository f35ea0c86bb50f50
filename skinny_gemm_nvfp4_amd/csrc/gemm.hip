// gemm.hip -- kernel selection and launch for the NVFP4 skinny GEMM Y[M,N] = X[M,K] . dequant(W)[K,N].
//
// Two persistent kernel families (headers in this directory), one workgroup per compute unit
// with an equal share of the 4-column groups:
//   * gemv_stream.h (NVFP4_PATH_DOT): dot products against X staged in LDS. Decode (M = 1) and
//     the smallest M.
//   * mfma_stream.h (NVFP4_PATH_MFMA): bf16 matrix cores on 16-row blocks of X (speculative
//     verification of one request), and every shape whose X does not fit in LDS.
//   * mfma_slab.h (NVFP4_PATH_BATCH): bf16 matrix cores, each weight decoded once per workgroup
//     for slabs of up to 128 rows of X (verification of several requests together).
// None of them needs memory beyond the caller's arrays: every partial sum stays in a workgroup.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <set>
#include <utility>

#include "gemv_stream.h"
#include "launch.h"
#include "mfma_slab.h"
#include "mfma_stream.h"
#include "neighbours.h"

namespace nvfp4 {

namespace {

typedef void (*KernelFn)(GemmArgs);
typedef void (*StreamFn)(GemmArgs, StreamLayout);

// Units in flight per wavefront of the dot-product kernel: three for one row of X, two for more.
// Measured on the layer shapes with cold weights: a deeper ring only adds to the requests queued
// ahead of the first bytes every wavefront waits for (one row: 3 vs 4 saves 0.3-0.45 us on qkv and
// o_proj and is even on gate_up and down; four rows: 2 vs 4 saves 1-1.8 us).
constexpr int stream_depth(int rows) { return rows == 1 ? 3 : 2; }

// Wavefronts per workgroup of the dot-product kernel when the caller leaves it open: 12 for up to
// four rows, 16 for two to four rows of an lm_head-sized weight (more than 1024 units per compute
// unit) and for more rows. Measured with cold weights (medians of five interleaved runs), 12
// against 16 at M = 1: gate_up 18.8 vs 19.5 us, down 11.2 vs 12.0, lm_head 72.4 vs 73.0, q/k/v
// 6.7 vs 7.0, o_proj 6.2 vs 6.5 (8: within 0.1 us on the last two, slower on the others); at
// M = 2 and 4: q/k/v 7.8 vs 8.0 and 10.5 vs 10.7, o_proj 6.9 vs 7.2 and 9.0 vs 9.4, gate_up and
// down even, lm_head (two workgroups per CU) 75.8 vs 75.3 and 108.1 vs 105.1. 4 is slower
// everywhere. Four units in flight instead of three gained nothing at 12 wavefronts.
int dot_default_waves(int rows, int N, int K);
constexpr int kMaxLds = 160 * 1024;         // LDS per workgroup on gfx950
constexpr int kDefaultLds = 64 * 1024;      // above this a kernel must opt in

// ---- dot-product kernels: [FAST][MR - 1][wave index: 4, 8, 16, 12] ----
#define NVFP4_STREAM_WAVES(R, FAST)                                                        \
    {                                                                                      \
        &gemv_stream_kernel<R, 4, stream_depth(R), FAST>,                                  \
            &gemv_stream_kernel<R, 8, stream_depth(R), FAST>,                              \
            &gemv_stream_kernel<R, 16, stream_depth(R), FAST>,                             \
            &gemv_stream_kernel<R, 12, stream_depth(R), FAST>                              \
    }
#define NVFP4_STREAM_TABLE(FAST)                                                           \
    {                                                                                      \
        NVFP4_STREAM_WAVES(1, FAST), NVFP4_STREAM_WAVES(2, FAST),                          \
            NVFP4_STREAM_WAVES(3, FAST), NVFP4_STREAM_WAVES(4, FAST),                      \
            NVFP4_STREAM_WAVES(5, FAST), NVFP4_STREAM_WAVES(6, FAST),                      \
            NVFP4_STREAM_WAVES(7, FAST), NVFP4_STREAM_WAVES(8, FAST)                       \
    }
const StreamFn kStream[2][8][4] = {NVFP4_STREAM_TABLE(false), NVFP4_STREAM_TABLE(true)};

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

// ---- slab kernels: [MODE][RB index: 1, 2, 4, 8 row blocks][HT - 1][NR] ----
constexpr int kSlabMaxHT = 4;   // at most 2 * 4 + 1 = 9 tiles per pass
#define NVFP4_SLAB_NR(RB, HT, MODE)                                                         \
    {                                                                                       \
        &mfma_slab_kernel<RB, HT, 0, MODE>, &mfma_slab_kernel<RB, HT, 1, MODE>              \
    }
#define NVFP4_SLAB_HT(RB, MODE)                                                             \
    {                                                                                       \
        NVFP4_SLAB_NR(RB, 1, MODE), NVFP4_SLAB_NR(RB, 2, MODE), NVFP4_SLAB_NR(RB, 3, MODE),  \
            NVFP4_SLAB_NR(RB, 4, MODE)                                                      \
    }
#define NVFP4_SLAB_RB(MODE)                                                                 \
    {                                                                                       \
        NVFP4_SLAB_HT(1, MODE), NVFP4_SLAB_HT(2, MODE), NVFP4_SLAB_HT(4, MODE),             \
            NVFP4_SLAB_HT(8, MODE)                                                          \
    }
typedef void (*SlabFn)(GemmArgs, SlabLayout);
const SlabFn kSlab[3][4][kSlabMaxHT][2] = {NVFP4_SLAB_RB(kSlabStore), NVFP4_SLAB_RB(kSlabArgmax),
                                           NVFP4_SLAB_RB(kSlabSilu)};
#define NVFP4_SLAB_LDS_HT(RB, HT)                                                           \
    {                                                                                       \
        SlabShape<RB, HT, 0>::LDS, SlabShape<RB, HT, 1>::LDS                                \
    }
#define NVFP4_SLAB_LDS_RB(RB)                                                               \
    {                                                                                       \
        NVFP4_SLAB_LDS_HT(RB, 1), NVFP4_SLAB_LDS_HT(RB, 2), NVFP4_SLAB_LDS_HT(RB, 3),       \
            NVFP4_SLAB_LDS_HT(RB, 4)                                                        \
    }
constexpr int kSlabLds[4][kSlabMaxHT][2] = {NVFP4_SLAB_LDS_RB(1), NVFP4_SLAB_LDS_RB(2),
                                            NVFP4_SLAB_LDS_RB(4), NVFP4_SLAB_LDS_RB(8)};

int wave_index(int waves)
{
    switch (waves) {
    case 4: return 0;
    case 8: return 1;
    case 16: return 2;
    case 12: return 3;
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
    // The dynamic limit is what the kernel's static arrays leave of the compute unit's LDS.
    hipFuncAttributes attr;
    e = hipFuncGetAttributes(&attr, fn);
    if (e != hipSuccess)
        return e;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxLds - (int)attr.sharedSizeBytes);
    if (e == hipSuccess)
        done.insert({dev, fn});
    return e;
}

// Workgroups over the 4-column groups: one per compute unit, at most one per group (per pair of
// groups when `pair`: the SiLU(gate) * up epilogue needs the gate and up groups of a pair in the
// same workgroup).
int group_grid(int N, bool pair = false)
{
    return std::max(1, std::min(compute_units(), num_groups(N) / (pair ? 2 : 1)));
}

// A workgroup's code bytes must stay below 2^31 (buffer offsets are 32-bit).
bool bytes_fit(int N, int K, int grid, bool pair = false)
{
    const int u = pair ? 2 : 1;
    const long long gmax = u * ((num_groups(N) / u + grid - 1) / grid);
    return gmax * (long long)num_chunks(K) * kChunkCodeBytes < (1LL << 31);
}

// Units (512-k windows of a 4-column group) a compute unit streams with one workgroup per CU.
long long stream_units_per_cu(int N, int K)
{
    const long long G = group_grid(N);
    return (num_groups(N) + G - 1) / G * ((K + kStreamWindow - 1) / kStreamWindow);
}

// Workgroups per compute unit of the dot-product kernel: two for one row when a compute unit has
// more than 128 units to stream, two for two to four rows above 1024 units (the lm_head), else
// one. Measured (medians of five interleaved runs), two against one: at M = 1 with 12 wavefronts
// gate_up 18.1 vs 18.8 us, down 10.9 vs 11.2, lm_head 71.9 vs 72.3, while q/k/v and o_proj
// (50-70 units) are slower with two (7.1 vs 6.7, 6.9 vs 6.1); at M = 2 and 4 with 16 wavefronts
// lm_head 75.3 vs 76.8 and 105.1 vs 110.5, while gate_up is even and down (whose X fills more
// than half the LDS) slower (17.0 vs 13.6 at M = 2).
constexpr int kStreamTwoWgUnits = 128;
constexpr int kStreamLargeUnits = 1024;

// One row of a small weight (at most 128 units per compute unit: q/k/v, o_proj) runs three
// workgroups of four wavefronts per compute unit instead: measured q/k/v 6.2 against 6.7 us,
// o_proj 5.6 against 6.1 (the dispatcher balances the smaller workgroups across compute units).
int stream_wg_per_cu(int M, int N, int K, bool pair)
{
    if (pair || M > 4)
        return 1;
    const long long units = stream_units_per_cu(N, K);
    if (M == 1 && units <= kStreamTwoWgUnits)
        return 3;
    return units > (M == 1 ? kStreamTwoWgUnits : kStreamLargeUnits) ? 2 : 1;
}

// Workgroups and LDS layout of the dot-product kernel; false if X does not fit in LDS.
// (norm: the kernel normalises X itself, once per workgroup: one workgroup per CU.)
bool stream_plan(int M, int N, int K, int MR, int W, int *grid, StreamLayout *L, bool pair = false,
                 bool norm = false)
{
    const int G = std::max(1, std::min(compute_units() * stream_wg_per_cu(M, N, K, pair || norm),
                                       num_groups(N) / (pair ? 2 : 1)));
    const int u = pair ? 2 : 1;   // groups are dealt in units of u
    L->nwin = (K + kStreamWindow - 1) / kStreamWindow;
    L->row_bytes = L->nwin * (kStreamWindow / 32) * kStreamSlot;
    const long long x_bytes = (long long)M * L->row_bytes;
    const int NU = num_groups(N) / u;
    L->gunit = u;
    L->ngroups = u * ((NU + G - 1) / G);
    // A group of nwin consecutive units touches every wavefront whose run starts inside it.
    L->slots = 1;
    const int sizes[2] = {u * (NU / G), L->ngroups};
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
    // (1 KB of the LDS is left for the kernel's static arrays: the RMSNorm row sums.)
    if (x_bytes + part_bytes > kMaxLds - 1024 || !bytes_fit(N, K, G, pair))
        return false;
    L->x_bytes = (int)x_bytes;
    L->part_bytes = (int)part_bytes;
    L->gq = NU / G;
    L->gr = NU % G;
    L->rnwin = 1.0f / (float)L->nwin;
    *grid = G;
    return true;
}

int dot_default_waves(int rows, int N, int K)
{
    if (rows == 1)
        return stream_units_per_cu(N, K) <= kStreamTwoWgUnits ? 4 : 12;
    if (rows > 4 || stream_units_per_cu(N, K) > kStreamLargeUnits)
        return 16;
    return 12;
}

// Workgroups, column-tile chunk and LDS bytes of the matrix-core kernel.
struct MfmaPlan {
    int grid, tc_index, lds;
};

bool mfma_plan(int N, int K, int waves, MfmaPlan *P, bool pair = false)
{
    const int G = group_grid(N, pair);
    if (!bytes_fit(N, K, G, pair))
        return false;
    const int u = pair ? 2 : 1;
    const int gmax = u * ((num_groups(N) / u + G - 1) / G);
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

// Slab kernel plan for a slab of `rows` <= 128 rows: row groups of RG = 16 RB rows, tile sets
// (S = compute units / row groups, a multiple of 8), tiles per pass (TW = 2 HT + NR, at most 9) and
// passes.
struct SlabPlan {
    int rbi, rb;    // row blocks of a row group: index into 1, 2, 4, 8, and the count
    int rg;         // rows per row group: 16 * (the plan's row blocks), before trimming to the slab
    int P, S;       // row groups, tile sets
    int ht, nr;     // tiles per pass: 2 ht + nr
    int passes;
    int lds;
    int gunit;
};

int rb_index(int rb) { return rb <= 1 ? 0 : rb <= 2 ? 1 : rb <= 4 ? 2 : 3; }

// Row blocks the kernel takes for a group of `rows` rows: the next power of two of rows / 16.
int rb_for_rows(int rows)
{
    const int blocks = (rows + 15) / 16;
    return blocks <= 1 ? 1 : blocks <= 2 ? 2 : blocks <= 4 ? 4 : 8;
}

// Tiles per pass and passes for T tiles per set: at most 9 tiles per pass, the passes equal.
void slab_passes(int T, int *ht, int *nr, int *passes)
{
    const int maxtw = 2 * kSlabMaxHT + 1;
    *passes = std::max(1, (T + maxtw - 1) / maxtw);
    const int tw = std::max(2, (T + *passes - 1) / *passes);
    *ht = tw / 2;
    *nr = tw % 2;
}

// The plan for `rows` rows with row groups of rg rows (rg = 16, 32, 64 or 128; 0: best).
bool slab_plan(int rows, int N, int K, bool pair, int rg_req, SlabPlan *P)
{
    if (rows < 1 || rows > 16 * 8)
        return false;
    const int cus = compute_units();
    const int unit = pair ? 2 : 1;
    const int units = num_groups(N) / unit;
    if (units < 1)
        return false;
    // Automatic choice: 128-row groups when every compute unit has at least 4 tiles with them,
    // else 64-row groups (measured on the layer shapes at M = 128: q/k/v 28.4 us with 64-row
    // groups against 31.5 with 128 and 31.6 with 32; o_proj 25.9 / 31.3 / 28.6; down (K = 17408)
    // 73.7 / 90.8 / 82.6; gate/up, 8.5 tiles per compute unit, 73 with 128 against 88 with 64).
    int rg_auto = 128;
    if (rg_req == 0) {
        const int S1 = std::max(1, std::min(cus - cus % 8, units));
        const int tiles1 = (unit * ((units + S1 - 1) / S1) + 3) / 4;
        rg_auto = (tiles1 >= 4 || rows <= 64) ? 128 : 64;
    }
    auto try_rg = [&](int rg) {
        const int Pg = (rows + rg - 1) / rg;
        if (Pg > cus)
            return false;
        int S = cus / Pg;
        if (S >= 8)
            S -= S % 8;
        S = std::max(1, std::min(S, units));
        const int gmax = unit * ((units + S - 1) / S);
        if (!bytes_fit(N, K, S, pair))
            return false;
        const int T = (gmax + 3) / 4;
        int ht, nr, passes;
        slab_passes(T, &ht, &nr, &passes);
        const int rb = rb_for_rows(std::min(rows, rg));
        const int lds = kSlabLds[rb_index(rb)][ht - 1][nr];
        if (lds > kMaxLds)
            return false;
        P->rg = rg;
        P->rb = rb;
        P->rbi = rb_index(rb);
        P->P = Pg;
        P->S = S;
        P->ht = ht;
        P->nr = nr;
        P->passes = passes;
        P->lds = lds;
        P->gunit = unit;
        return true;
    };
    if (rg_req != 0)
        return try_rg(rg_req);
    if (try_rg(rg_auto))
        return true;
    for (int rg = 128; rg >= 16; rg /= 2)   // any plan that fits
        if (try_rg(rg))
            return true;
    return false;
}

// Tiles of 16 columns per workgroup when every compute unit takes an equal share of the groups.
int tiles_per_workgroup(int N)
{
    const int G = group_grid(N);
    return ((num_groups(N) + G - 1) / G + 3) / 4;
}

}  // namespace

hipError_t allow_dynamic_lds(const void *fn, int bytes)
{
    return allow_lds(fn, bytes);
}

bool choose_config(int M, int N, int K, int *path, int *split)
{
    // Automatic choice (measured on the layer shapes): the dot-product kernel for the smallest M;
    // the 16-row matrix-core kernel up to M = 16 and, up to M = 48, for narrow shapes (a few
    // tiles per compute unit) of moderate K, whose weights it reads once per row block; above
    // that the slab kernel, which decodes each weight once per workgroup for up to 128 rows.
    if (*path == kPathAuto) {
        const bool narrow = tiles_per_workgroup(N) < 6 && K <= 8192;
        *path = (M <= 4) ? kPathDot : (M <= 16 || (M <= 48 && narrow)) ? kPathMfma : kPathBatch;
    }
    if (*path == kPathBatch) {
        if (*split != 0 && *split != 16 && *split != 32 && *split != 64 && *split != 128)
            return false;
        SlabPlan P;
        return slab_plan(std::min(M, 128), N, K, false, *split, &P);
    }
    if (*path == kPathInvariant) {
        SlabPlan P;
        return *split == 0 && slab_plan(std::min(M, 128), N, K, false, 0, &P);
    }
    if (*path == kPathDot) {
        if (M > kDotMaxM)
            return false;
        if (*split == 0)
            *split = dot_default_waves(M, N, K);
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

namespace {

// Turns the keys of `rows` rows (row stride `slots`) into index and value.
hipError_t launch_finalize(const argkey_t *keys, int slots, int rows, int32_t *index,
                           float *value, hipStream_t stream)
{
    hipLaunchKernelGGL(argmax_finalize_kernel, dim3((unsigned)rows), dim3(256), 0, stream, keys,
                       slots, index, value);
    return hipGetLastError();
}

// launch_gemm, and in argmax mode (index != nullptr, a.keys the workspace of M *
// kArgmaxSlotsPerCu * compute units keys) the same kernels folding Y into keys, then the
// finalize kernel.
hipError_t launch_impl(int path, int split, const GemmArgs &a0, int32_t *index, float *value,
                       hipStream_t stream)
{
    const bool argmax = index != nullptr;
    const int cap = kArgmaxSlotsPerCu * compute_units();   // key row stride of the workspace
    GemmArgs a = a0;
    (void)hipGetLastError();  // start from a clean error state
    if (path == kPathDot) {
        StreamLayout L;
        int grid = 0;
        if (!stream_plan(a.M, a.N, a.K, a.M, split, &grid, &L, a.H != nullptr,
                         a.gamma != nullptr))
            return hipErrorInvalidValue;
        const int fast = (a.K % kStreamWindow == 0) ? 1 : 0;
        const StreamFn fn = kStream[fast][a.M - 1][wave_index(split)];
        const int lds = L.x_bytes + L.part_bytes;
        const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), lds);
        if (e != hipSuccess)
            return e;
        if (argmax)
            a.key_slots = grid;   // one key per workgroup
        if (a.key_slots > cap)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(fn, dim3(grid), dim3(kWave * split), lds, stream, a, L);
        const hipError_t le = hipGetLastError();
        if (le != hipSuccess || !argmax)
            return le;
        return launch_finalize(a.keys, a.key_slots, a.M, index, value, stream);
    }
    if (path == kPathBatch || path == kPathInvariant) {
        // Slabs of 128 rows, one launch each (the last one may be smaller).
        // Batch-invariant mode: the slab kernel for every M. Output (m, n) is the same bits under
        // every slab plan (row groups, tile sets, tiles per pass): its sum runs over the 128-k
        // windows in order within each of the four k-step lanes, then (((k3 + k2) + k1) + k0),
        // whatever workgroup, pass or row block it falls in; an MFMA row's arithmetic does not
        // depend on the other rows. So each slab takes the plan that suits its own rows.
        const bool pair = a.H != nullptr;
        const int mode = argmax ? kSlabArgmax : pair ? kSlabSilu : kSlabStore;
        constexpr int kSlabRows = 128;
        for (int m0 = 0; m0 < a.M; m0 += kSlabRows) {
            const int rows = std::min(kSlabRows, a.M - m0);
            SlabPlan P;
            if (!slab_plan(rows, a.N, a.K, pair, path == kPathInvariant ? 0 : split, &P))
                return hipErrorInvalidValue;
            const SlabFn fn = kSlab[mode][P.rbi][P.ht - 1][P.nr];
            const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), P.lds);
            if (e != hipSuccess)
                return e;
            GemmArgs b = a;
            b.X = a.X + (size_t)m0 * (size_t)a.K;
            b.Y = a.Y != nullptr ? a.Y + (size_t)m0 * (size_t)a.N : nullptr;
            b.H = a.H != nullptr ? a.H + (size_t)m0 * (size_t)(a.N / 2) : nullptr;
            b.M = rows;
            SlabLayout L;
            L.sets = P.S;
            L.rgroups = P.P;
            L.gunit = P.gunit;
            L.xcd = (P.S % 8 == 0 && P.P > 1) ? 1 : 0;
            L.passes = P.passes;
            L.key_slots = P.S;   // one key per row and tile set
            L.vec = pair ? (reinterpret_cast<uintptr_t>(b.H) % 8 == 0 ? 1 : 0)
                         : (b.Y != nullptr && reinterpret_cast<uintptr_t>(b.Y) % 16 == 0 &&
                            a.N % 4 == 0)
                               ? 1
                               : 0;
            argkey_t *slab_keys = argmax ? a.keys + (size_t)m0 * (size_t)cap : nullptr;
            b.keys = slab_keys;
            if (argmax && L.key_slots > cap)
                return hipErrorInvalidValue;
            hipLaunchKernelGGL(fn, dim3((unsigned)(P.S * P.P)), dim3(kWave * kSlabWaves), P.lds,
                               stream, b, L);
            hipError_t le = hipGetLastError();
            if (le != hipSuccess)
                return le;
            if (argmax) {
                le = launch_finalize(slab_keys, L.key_slots, rows, index + m0, value + m0, stream);
                if (le != hipSuccess)
                    return le;
            }
        }
        return hipSuccess;
    }
    if (path != kPathMfma)
        return hipErrorInvalidValue;
    MfmaPlan P;
    if (!mfma_plan(a.N, a.K, split, &P, a.H != nullptr))
        return hipErrorInvalidValue;
    const int fast = (a.K % kMfmaWindow == 0) ? 1 : 0;
    const KernelFn fn = kMfma[fast][P.tc_index][split == 4 ? 0 : 1];
    const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), P.lds);
    if (e != hipSuccess)
        return e;
    const unsigned mblocks = (unsigned)((a.M + 15) / 16);
    if (argmax)
        a.key_slots = P.grid * (split / 4);   // one key per four wavefronts
    if (a.key_slots > cap)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned)P.grid, mblocks), dim3(kWave * split), P.lds, stream,
                       a);
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess || !argmax)
        return le;
    return launch_finalize(a.keys, a.key_slots, a.M, index, value, stream);
}

}  // namespace

hipError_t launch_gemm(int path, int split, const GemmArgs &a, hipStream_t stream)
{
    GemmArgs b = a;
    b.keys = nullptr;
    b.key_slots = 0;
    return launch_impl(path, split, b, nullptr, nullptr, stream);
}

hipError_t launch_gemm_argmax(int path, int split, const GemmArgs &a, int32_t *index,
                              float *value, hipStream_t stream)
{
    if (a.keys == nullptr || index == nullptr || value == nullptr)
        return hipErrorInvalidValue;
    return launch_impl(path, split, a, index, value, stream);
}

int device_compute_units() { return compute_units(); }

// Keys of nvfp4_gemm_argmax_noalloc: a fixed 4 MiB array in device memory, one copy per GPU the
// library runs on, held until the process ends. Every call on a GPU uses the same array (calls
// that overlap in time on one GPU race on it). Host code never passes `scratch` itself to a
// kernel: on the host the name is only a handle, and its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) argkey_t scratch[kScratchKeys];

int argmax_scratch_rows()
{
    return (int)(kScratchKeys / ((size_t)kArgmaxSlotsPerCu * (size_t)compute_units()));
}

hipError_t argmax_scratch(argkey_t **keys)
{
    static std::atomic<argkey_t *> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    argkey_t *p = cache[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void *q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (q == nullptr)
            return hipErrorInvalidSymbol;
        p = static_cast<argkey_t *>(q);
        cache[dev].store(p, std::memory_order_release);
    }
    *keys = p;
    return hipSuccess;
}

namespace {

// Whether nvfp4_gemm_fused runs everything inside the dot-product kernel (up to 4 rows, X in LDS).
// (One row takes 12 wavefronts in one workgroup per CU here, whatever the weight's size: the
// RMSNorm prologue runs once per workgroup.)
bool fused_in_dot(int M, int N, int K, bool pair, int *waves, StreamLayout *L, int *grid)
{
    *waves = M == 1 ? 12 : dot_default_waves(M, N, K);
    return M <= 4 && stream_plan(M, N, K, M, *waves, grid, L, pair, true);
}

}  // namespace

size_t fused_workspace_bytes(bool norm, bool pair, int M, int N, int K)
{
    StreamLayout L;
    int grid, waves;
    if (!norm || fused_in_dot(M, N, K, pair, &waves, &L, &grid))
        return 0;
    return ((size_t)M * (size_t)K * 2 + 255) & ~(size_t)255;
}

hipError_t launch_gemm_fused(const GemmArgs &a, hipStream_t stream)
{
    const bool pair = a.H != nullptr;
    // Up to 4 rows the dot-product kernel does it all: X is staged in LDS anyway, so RMSNorm
    // costs two barriers and a pass over LDS, and the SiLU(gate) * up epilogue runs on the
    // column sums. Above, the RMSNorm is a row-wise kernel of its own writing the normalised X
    // to the caller's workspace (normalising X inside the matrix-core kernels repeats the work in
    // every workgroup: at 128 rows as much VALU work per window as decoding the weights); the
    // SiLU(gate) * up epilogue is inside the 16-row kernel (M <= 16) and the slab kernel.
    StreamLayout L;
    int grid, dw;
    const bool dot = fused_in_dot(a.M, a.N, a.K, pair, &dw, &L, &grid);
    const size_t xbytes = fused_workspace_bytes(a.gamma != nullptr, pair, a.M, a.N, a.K);
    if (xbytes > a.workspace_bytes || (xbytes > 0 && a.workspace == nullptr))
        return hipErrorInvalidValue;
    (void)hipGetLastError();
    GemmArgs b = a;
    b.keys = nullptr;
    b.key_slots = 0;
    if (xbytes > 0) {
        uint16_t *Xn = reinterpret_cast<uint16_t *>(a.workspace);
        hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3((unsigned)a.M), dim3(256), 0, stream, a.X,
                           a.gamma, a.eps, a.K, Xn);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        b.X = Xn;
        b.gamma = nullptr;
    }
    if (dot)
        return launch_impl(kPathDot, dw, b, nullptr, nullptr, stream);
    if (a.M <= 16) {
        MfmaPlan P;
        int split = 8;
        if (!mfma_plan(a.N, a.K, 8, &P, pair) || kMfmaTiles[P.tc_index] >= 6)
            split = 4;
        if (!mfma_plan(a.N, a.K, split, &P, pair))
            return hipErrorInvalidValue;
        return launch_impl(kPathMfma, split, b, nullptr, nullptr, stream);
    }
    return launch_impl(kPathBatch, 0, b, nullptr, nullptr, stream);
}

}  // namespace nvfp4

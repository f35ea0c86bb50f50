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
#include <map>
#include <mutex>
#include <set>
#include <utility>

#include "gemv_stream.h"
#include "launch.h"
#include "mfma_batch.h"
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

// ---- batch kernels: [TCW - 1][MB index: 1, 2, 4, 8 row blocks][KS index: 1, 2, 4] ----
// (second index of kBatchAll: 0 stores Y, 1 folds it into argmax keys)
#define NVFP4_BATCH_KS(TCW, MB, A)                                                         \
    {                                                                                      \
        &mfma_batch_kernel<TCW, MB, 1, 0, A>, &mfma_batch_kernel<TCW, MB, 2, 0, A>,        \
            &mfma_batch_kernel<TCW, MB, 4, 0, A>                                           \
    }
#define NVFP4_BATCH_MB(TCW, A)                                                             \
    {                                                                                      \
        NVFP4_BATCH_KS(TCW, 1, A), NVFP4_BATCH_KS(TCW, 2, A), NVFP4_BATCH_KS(TCW, 4, A),   \
            NVFP4_BATCH_KS(TCW, 8, A)                                                      \
    }
const KernelFn kBatchAll[2][3][4][3] = {
    {NVFP4_BATCH_MB(1, false), NVFP4_BATCH_MB(2, false), NVFP4_BATCH_MB(3, false)},
    {NVFP4_BATCH_MB(1, true), NVFP4_BATCH_MB(2, true), NVFP4_BATCH_MB(3, true)}};

template <int TCW, int MB, int KS>
constexpr int batch_lds()
{
    return BatchShape<TCW, MB, KS>::LDS;
}
#define NVFP4_BATCH_LDS_KS(TCW, MB)                                                        \
    {                                                                                      \
        batch_lds<TCW, MB, 1>(), batch_lds<TCW, MB, 2>(), batch_lds<TCW, MB, 4>()          \
    }
#define NVFP4_BATCH_LDS_MB(TCW)                                                            \
    {                                                                                      \
        NVFP4_BATCH_LDS_KS(TCW, 1), NVFP4_BATCH_LDS_KS(TCW, 2), NVFP4_BATCH_LDS_KS(TCW, 4), \
            NVFP4_BATCH_LDS_KS(TCW, 8)                                                     \
    }
constexpr int kBatchLds[3][4][3] = {NVFP4_BATCH_LDS_MB(1), NVFP4_BATCH_LDS_MB(2),
                                    NVFP4_BATCH_LDS_MB(3)};

// ---- batch kernels with remainder tiles (KS = 1): [(TCW, NR) index][MB index] ----
constexpr int kBatchNrCombos = 3;
constexpr int kBatchNrTcw[kBatchNrCombos] = {1, 1, 2};
constexpr int kBatchNrNr[kBatchNrCombos] = {1, 2, 1};
#define NVFP4_BATCH_NR_MB(TCW, NR, A)                                                      \
    {                                                                                      \
        &mfma_batch_kernel<TCW, 1, 1, NR, A>, &mfma_batch_kernel<TCW, 2, 1, NR, A>,        \
            &mfma_batch_kernel<TCW, 4, 1, NR, A>, &mfma_batch_kernel<TCW, 8, 1, NR, A>     \
    }
const KernelFn kBatchNrAll[2][kBatchNrCombos][4] = {
    {NVFP4_BATCH_NR_MB(1, 1, false), NVFP4_BATCH_NR_MB(1, 2, false),
     NVFP4_BATCH_NR_MB(2, 1, false)},
    {NVFP4_BATCH_NR_MB(1, 1, true), NVFP4_BATCH_NR_MB(1, 2, true),
     NVFP4_BATCH_NR_MB(2, 1, true)}};
#define NVFP4_BATCH_NR_LDS(TCW, NR)                                                        \
    {                                                                                      \
        BatchShape<TCW, 1, 1, NR>::LDS, BatchShape<TCW, 2, 1, NR>::LDS,                    \
            BatchShape<TCW, 4, 1, NR>::LDS, BatchShape<TCW, 8, 1, NR>::LDS                 \
    }
constexpr int kBatchNrLds[kBatchNrCombos][4] = {NVFP4_BATCH_NR_LDS(1, 1), NVFP4_BATCH_NR_LDS(1, 2),
                                                NVFP4_BATCH_NR_LDS(2, 1)};

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

int stream_wg_per_cu(int M, int N, int K, bool pair)
{
    if (pair || M > 4)
        return 1;
    const long long units = stream_units_per_cu(N, K);
    return units > (M == 1 ? kStreamTwoWgUnits : kStreamLargeUnits) ? 2 : 1;
}

// Workgroups and LDS layout of the dot-product kernel; false if X does not fit in LDS.
bool stream_plan(int M, int N, int K, int MR, int W, int *grid, StreamLayout *L, bool pair = false)
{
    const int G = std::max(1, std::min(compute_units() * stream_wg_per_cu(M, N, K, pair),
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
        return 12;
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

// Batch kernel for one slab of `rows` <= 128 rows: row blocks MB (1, 2, 4 or 8), tiles per
// consumer TCW and step split KS (ks_req unless 0), from a cycle estimate per compute unit. A
// window costs the slowest of: the busiest consumer's MFMAs (16 cycles each) or decode (about 80
// VALU cycles per tile and step); the X bytes from L2 (64 bytes per cycle); the LDS traffic (128
// bytes per cycle); the weight bytes at the compute unit's share of HBM (13 bytes per cycle); and
// the load latency spread over the windows in flight (about 4000 cycles / 4). Every pass also
// pays one latency to fill the pipeline.
constexpr double kLoadLatency = 4000.0;

struct BatchPlan {
    int tcw, mbi, ksi, mb, grid, lds;
    int nr;       // remainder tiles per pass (KS = 1 only), 0 for none
    int nri;      // index into kBatchNr when nr > 0
    int nslice;   // K slices across workgroups (split K), 1 for none
};

// Cycle estimate of one pass window (see batch_plan) for `units` tile-steps per consumer.
double batch_window_cost(int units, int MB, int KS, int pt)
{
    // X arrives from L2 about 1400 cycles after it is requested, XRING - 1 windows ahead.
    const int xring = MB >= 8 ? 2 : MB >= 4 ? 3 : 4;
    const double x_lat = 1400.0 / (xring - 1);
    const double mfma = 16.0 * units * MB;
    const double valu = 80.0 * units;
    const double x_l2 = 16.0 * MB * kBatchRowBytes / 64.0;
    const double lds = (16.0 * MB * kBatchRowBytes * (1 + kBatchConsumers / KS) +
                        2.0 * pt * (kBatchTileBytes + kWave * 4)) /
                       128.0;
    const double hbm = pt * (kBatchTileBytes + kWave * 4) / 13.0;
    const double lat = kLoadLatency / (kBatchWRing - 1);
    // (plus a tenth of the consumer's own work, which breaks ties toward spreading it)
    return std::max(std::max(std::max(mfma, valu), std::max(x_l2, lds)),
                    std::max(std::max(hbm, lat), x_lat)) +
           0.1 * std::max(mfma, valu);
}

bool batch_plan(int rows, int N, int K, int ks_req, int s_req, BatchPlan *P)
{
    // The Y descriptor covers rows * N floats with 32-bit offsets.
    if ((long long)rows * N * 4 >= (1LL << 31))
        return false;
    const int nwin = (K + kBatchWindow - 1) / kBatchWindow;
    const int mbi = rows <= 16 ? 0 : rows <= 32 ? 1 : rows <= 64 ? 2 : 3;
    const int MB = 1 << mbi;
    const int cus = compute_units();
    double best = 0.0;
    bool found = false;
    for (int si = 0; si < 4; si++) {
        const int S = 1 << si;   // K slices
        if ((s_req != 0 && S != s_req) || S > nwin)
            continue;
        const int G = std::max(1, std::min(num_groups(N), cus / S));
        if (!bytes_fit(N, K, G))
            continue;
        const int T = ((num_groups(N) + G - 1) / G + 3) / 4;
        const int nw = (nwin + S - 1) / S;   // windows of the longest slice
        // Split K adds the S partial slices' round trip and a second launch.
        const double reduce =
            S > 1 ? (S + 1.0) * rows * N * 4.0 / 2400.0 + kLoadLatency : 0.0;
        auto consider = [&](double cost, int tcw, int ksi, int nr, int nri) {
            cost += reduce;
            if (!found || cost < best - 1e-9) {
                best = cost;
                found = true;
                P->tcw = tcw;
                P->ksi = ksi;
                P->nr = nr;
                P->nri = nri;
                P->nslice = S;
                P->grid = G;
            }
        };
        for (int ksi = 0; ksi < 3; ksi++) {
            const int KS = 1 << ksi;
            if (ks_req != 0 && KS != ks_req)
                continue;
            const int TS = kBatchConsumers / KS;
            const int NSTEP = 4 / KS;
            for (int tcw = 1; tcw <= 3; tcw++) {
                if (kBatchLds[tcw - 1][mbi][ksi] > kMaxLds)
                    continue;
                const int PT = TS * tcw;
                double cost = 0.0;
                for (int t0 = 0; t0 < T; t0 += PT) {
                    const int pt = std::min(PT, T - t0);   // tiles of this pass
                    const int live = std::min(tcw, (pt + TS - 1) / TS);
                    cost += nw * batch_window_cost(live * NSTEP, MB, KS, pt) + kLoadLatency;
                }
                consider(cost, tcw, ksi, 0, 0);
            }
        }
        // Remainder variants (KS = 1): passes of 4 TCW + NR tiles, every consumer 4 TCW + NR
        // steps.
        if (ks_req == 0 || ks_req == 1) {
            for (int ci = 0; ci < kBatchNrCombos; ci++) {
                const int tcw = kBatchNrTcw[ci], nr = kBatchNrNr[ci];
                if (kBatchNrLds[ci][mbi] > kMaxLds)
                    continue;
                const int PT = kBatchConsumers * tcw + nr;
                double cost = 0.0;
                for (int t0 = 0; t0 < T; t0 += PT)
                    cost += nw * batch_window_cost(4 * tcw + nr, MB, 1, std::min(PT, T - t0)) +
                            kLoadLatency;
                consider(cost, tcw, 0, nr, ci);
            }
        }
    }
    if (!found)
        return false;
    P->mbi = mbi;
    P->mb = MB;
    P->lds = P->nr > 0 ? kBatchNrLds[P->nri][mbi] : kBatchLds[P->tcw - 1][mbi][P->ksi];
    return true;
}

// Library workspaces: one per device and kind (kind 0: the split-K partial sums; kind 1: the
// normalised X and the gate/up output of a fused call at M > 16), grown (never shrunk or freed:
// a captured graph may still hold an older one) on first need. Returns null when it would have
// to grow while the stream is being captured, or when the allocation fails.
float *batch_workspace(size_t bytes, hipStream_t stream, int kind = 0)
{
    static std::mutex mu;
    static std::map<std::pair<int, int>, std::pair<void *, size_t>> ws;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    auto &e = ws[{dev, kind}];
    if (e.first != nullptr && e.second >= bytes)
        return static_cast<float *>(e.first);
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return nullptr;
    }
    void *p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    e = {p, bytes};
    return static_cast<float *>(p);
}

// Batch-invariant mode: one plan per (N, K), the plan of a full 128-row slab (K slices included),
// used for every slab whatever its rows. Only the row-block count MB follows the rows, and a row's
// arithmetic does not depend on it: each row block has its own accumulators, the weight fragment
// it multiplies is the same, and the steps, the step split, the remainder partials and the K
// slices are added in the same order. So row m of Y is the same bits for any M. The workspace of
// a split plan is sized for a full slab on every call, so one call outside stream capture covers
// every later M.
bool invariant_plan(int N, int K, BatchPlan *P)
{
    return batch_plan(16 * kBatchMaxBlocks, N, K, 0, 0, P);
}

// The invariant plan adapted to a slab of `rows` rows: the row-block count and LDS bytes only.
void plan_for_rows(BatchPlan *P, int rows)
{
    P->mbi = rows <= 16 ? 0 : rows <= 32 ? 1 : rows <= 64 ? 2 : 3;
    P->mb = 1 << P->mbi;
    P->lds = P->nr > 0 ? kBatchNrLds[P->nri][P->mbi] : kBatchLds[P->tcw - 1][P->mbi][P->ksi];
}

// Tiles of 16 columns per workgroup when every compute unit takes an equal share of the groups.
int tiles_per_workgroup(int N)
{
    const int G = group_grid(N);
    return ((num_groups(N) + G - 1) / G + 3) / 4;
}

}  // namespace

bool choose_config(int M, int N, int K, int *path, int *split)
{
    // Automatic choice (measured on the layer shapes): the dot-product kernel for the smallest M;
    // the 16-row matrix-core kernel up to M = 16 and, up to M = 48, for narrow shapes (a few
    // tiles per compute unit) of moderate K, whose weights it reads once per row block; above
    // that the batch kernel, which decodes each weight once per 128 rows (and cuts K across
    // workgroups for narrow shapes).
    if (*path == kPathAuto) {
        const bool narrow = tiles_per_workgroup(N) < 6 && K <= 8192;
        *path = (M <= 4) ? kPathDot : (M <= 16 || (M <= 48 && narrow)) ? kPathMfma : kPathBatch;
    }
    if (*path == kPathBatch) {
        if (*split != 0 && *split != 1 && *split != 2 && *split != 4)
            return false;
        BatchPlan P;
        if (!batch_plan(std::min(M, 16 * kBatchMaxBlocks), N, K, *split, 0, &P))
            return false;
        *split = 1 << P.ksi;
        return true;
    }
    if (*path == kPathInvariant) {
        BatchPlan P;
        return *split == 0 && invariant_plan(N, K, &P);
    }
    if (*path == kPathBatchSplit) {
        if (*split != 2 && *split != 4 && *split != 8)
            return false;
        BatchPlan P;
        return batch_plan(std::min(M, 16 * kBatchMaxBlocks), N, K, 0, *split, &P);
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
        if (!stream_plan(a.M, a.N, a.K, a.M, split, &grid, &L, a.H != nullptr))
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
    if (path == kPathBatch || path == kPathBatchSplit || path == kPathInvariant) {
        const int ks_req = path == kPathBatch ? split : 0;
        const int s_req = path == kPathBatch ? 0 : split;
        BatchPlan fixed = {};
        if (path == kPathInvariant && !invariant_plan(a.N, a.K, &fixed))
            return hipErrorInvalidValue;
        // Slabs of 128 rows, one launch each (the last one may be smaller).
        constexpr int kSlab = 16 * kBatchMaxBlocks;
        for (int m0 = 0; m0 < a.M; m0 += kSlab) {
            const int rows = std::min(kSlab, a.M - m0);
            BatchPlan P = fixed;
            if (path == kPathInvariant)
                plan_for_rows(&P, rows);
            else if (!batch_plan(rows, a.N, a.K, ks_req, s_req, &P))
                return hipErrorInvalidValue;
            GemmArgs b = a;
            b.X = a.X + (size_t)m0 * (size_t)a.K;
            b.Y = a.Y != nullptr ? a.Y + (size_t)m0 * (size_t)a.N : nullptr;
            b.M = rows;
            float *ws = nullptr;
            const size_t stride = batch_slice_stride(rows, a.N);
            if (P.nslice > 1 && path == kPathInvariant) {
                // The slices are part of the invariant arithmetic: no unsplit fallback.
                ws = batch_workspace(
                    (size_t)P.nslice * batch_slice_stride(kSlab, a.N) * sizeof(float), stream);
                if (ws == nullptr)
                    return hipErrorStreamCaptureUnsupported;
            } else if (P.nslice > 1) {
                ws = batch_workspace((size_t)P.nslice * stride * sizeof(float), stream);
                if (ws == nullptr && !batch_plan(rows, a.N, a.K, ks_req, 1, &P))
                    return hipErrorInvalidValue;   // no workspace: run unsplit
            }
            // Argmax mode: the kernel folds Y into keys itself unless K is split, in which case
            // the partials go to the workspace as usual and the reduce kernel folds the sums.
            const int fold = (argmax && P.nslice == 1) ? 1 : 0;
            const KernelFn fn = P.nr > 0 ? kBatchNrAll[fold][P.nri][P.mbi]
                                         : kBatchAll[fold][P.tcw - 1][P.mbi][P.ksi];
            const hipError_t e = allow_lds(reinterpret_cast<const void *>(fn), P.lds);
            if (e != hipSuccess)
                return e;
            GemmArgs kb = b;
            kb.keys = nullptr;
            if (P.nslice > 1)
                kb.Y = ws;   // unscaled partial sums, slice by slice
            argkey_t *slab_keys = argmax ? a.keys + (size_t)m0 * (size_t)cap : nullptr;
            if (fold) {
                kb.keys = slab_keys;
                kb.key_slots = kBatchConsumers * P.grid;   // one key per consumer wavefront
                if (kb.key_slots > cap)
                    return hipErrorInvalidValue;
            }
            hipLaunchKernelGGL(fn, dim3((unsigned)P.grid, (unsigned)P.nslice),
                               dim3(kWave * kBatchWaves), P.lds, stream, kb);
            hipError_t le = hipGetLastError();
            if (le != hipSuccess)
                return le;
            int slots = kb.key_slots;
            if (P.nslice > 1 && argmax) {
                slots = std::min(cap, std::max(1, std::min((a.N + 255) / 256, 256)));
                hipLaunchKernelGGL(batch_reduce_argmax_kernel, dim3((unsigned)slots, (unsigned)rows),
                                   dim3(256), 0, stream, ws, P.nslice, a.N, (long long)stride,
                                   a.gscale, slab_keys, slots);
                le = hipGetLastError();
                if (le != hipSuccess)
                    return le;
            } else if (P.nslice > 1) {
                const long long count = (long long)rows * a.N;
                const unsigned blocks = (unsigned)((count + 4 * 256 - 1) / (4 * 256));
                hipLaunchKernelGGL(batch_reduce_kernel, dim3(blocks), dim3(256), 0, stream, ws,
                                   P.nslice, count, (long long)stride, a.gscale, b.Y);
                le = hipGetLastError();
                if (le != hipSuccess)
                    return le;
            }
            if (argmax) {
                le = launch_finalize(slab_keys, slots, rows, index + m0, value + m0, stream);
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

hipError_t launch_gemm_fused(const GemmArgs &a, hipStream_t stream)
{
    const bool pair = a.H != nullptr;
    // Up to 4 rows the dot-product kernel does it all: X is staged in LDS anyway, so RMSNorm
    // costs two barriers and a pass over LDS, and the SiLU(gate) * up epilogue runs on the
    // column sums. Above, the RMSNorm is a row-wise kernel of its own (normalising each X window
    // inside the 16-row kernel cost more than the launch); the SiLU(gate) * up epilogue stays in
    // the 16-row kernel (M <= 16) or follows the batch kernel as an elementwise kernel (M > 16,
    // the batch kernel reading each weight once per 128 rows).
    StreamLayout L;
    int grid;
    const int dw = dot_default_waves(a.M, a.N, a.K);
    const bool dot = a.M <= 4 && stream_plan(a.M, a.N, a.K, a.M, dw, &grid, &L, pair);
    const bool split_silu = pair && a.M > 16;
    const size_t xbytes = (!dot && a.gamma) ? ((size_t)a.M * a.K * 2 + 255) & ~(size_t)255 : 0;
    const size_t ybytes = split_silu ? (size_t)a.M * a.N * 4 : 0;
    uint8_t *ws = nullptr;
    if (xbytes + ybytes > 0) {
        ws = reinterpret_cast<uint8_t *>(batch_workspace(xbytes + ybytes, stream, 1));
        if (ws == nullptr)
            return hipErrorStreamCaptureUnsupported;   // (or out of memory)
    }
    (void)hipGetLastError();
    GemmArgs b = a;
    b.keys = nullptr;
    b.key_slots = 0;
    if (xbytes > 0) {
        uint16_t *Xn = reinterpret_cast<uint16_t *>(ws);
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
    if (split_silu) {
        b.H = nullptr;
        b.Y = reinterpret_cast<float *>(ws + xbytes);
    }
    int path = kPathAuto, split = 0;
    if (!choose_config(a.M, a.N, a.K, &path, &split))
        return hipErrorInvalidValue;
    hipError_t e = launch_impl(path, split, b, nullptr, nullptr, stream);
    if (e != hipSuccess || !split_silu)
        return e;
    const long long count = (long long)a.M * (a.N / 2);
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                       stream, b.Y, count, a.N, a.H);
    return hipGetLastError();
}

}  // namespace nvfp4

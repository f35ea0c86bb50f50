// grouped.hip -- launch of the grouped (mixture-of-experts) NVFP4 GEMM (grouped.h).
#include <algorithm>

#include "grouped.h"
#include "launch.h"

namespace nvfp4 {

namespace {

typedef void (*GroupedFn)(GroupedArgs, int);

// [LDSX][FAST][MR index: 1, 2, 4 rows per item]. Without LDSX the wavefronts per workgroup and
// the windows in flight per wavefront shrink as the rows grow (each window's X rows sit in
// registers); with X staged in LDS every row count keeps 16 wavefronts and 3 windows in flight.
#define NVFP4_GROUPED(L, F)                                                                \
    {                                                                                      \
        &grouped_gemv_kernel<1, 16, 3, F, L>, &grouped_gemv_kernel<2, 8, 3, F, L>,         \
            &grouped_gemv_kernel<4, 8, 2, F, L>                                            \
    }
#define NVFP4_GROUPED_LDSX(F)                                                              \
    {                                                                                      \
        &grouped_gemv_kernel<1, 16, 3, F, true>, &grouped_gemv_kernel<2, 16, 3, F, true>,  \
            &grouped_gemv_kernel<4, 16, 3, F, true>                                        \
    }
const GroupedFn kGrouped[2][2][3] = {{NVFP4_GROUPED(false, false), NVFP4_GROUPED(false, true)},
                                     {NVFP4_GROUPED_LDSX(false), NVFP4_GROUPED_LDSX(true)}};
const int kGroupedWaves[2][3] = {{16, 8, 8}, {16, 16, 16}};

// One row per item and at most 16 rows in all (decode: a token's routed experts): 8 wavefronts
// with 4 windows in flight each. A wavefront then has about one item and streams it in one round
// trip instead of two (measured: 3-8% faster on the decode calls, slower on 128 rows). [LDSX][FAST]
const GroupedFn kGroupedFew[2][2] = {
    {&grouped_gemv_kernel<1, 8, 4, false, false>, &grouped_gemv_kernel<1, 8, 4, true, false>},
    {&grouped_gemv_kernel<1, 8, 4, false, true>, &grouped_gemv_kernel<1, 8, 4, true, true>}};
constexpr int kGroupedFewRows = 16;

// Dynamic LDS for the staged X rows, next to the 24 KB of the expert tables (the kernel opts in
// above the 64 KB default).
constexpr int kGroupedXLds = 128 * 1024;

}  // namespace

int grouped_rows_per_item(int T, int E, int requested)
{
    if (requested != 0)
        return requested;
    // Decode routes each token to a few experts, one row each; verification puts a few rows on
    // the popular ones, and a chunk of two rows reads an expert's weights once for both
    // (measured at 16 tokens, 128 experts, top-8: gate/up 46.4 -> 37.2 us, down 33.5 -> 29.7
    // against one row per chunk; four rows per chunk 44.8 and 35.9).
    return 2 * T <= E ? 1 : T <= 2 * E ? 2 : 4;
}

hipError_t launch_grouped(const GroupedArgs &a, int rows_per_item, hipStream_t stream)
{
    const int mi = rows_per_item == 1 ? 0 : rows_per_item == 2 ? 1 : rows_per_item == 4 ? 2 : -1;
    if (mi < 0 || a.E < 1 || a.E > kGroupedMaxExperts)
        return hipErrorInvalidValue;
    if (a.T == 0)
        return hipSuccess;   // no rows: nothing to compute, no HIP call
    (void)hipGetLastError();  // start from a clean error state
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    const int fast = (a.K % kGroupedWindow == 0) ? 1 : 0;
    // Rows a workgroup stages: its items span at most ceil(items / G) + 1 consecutive items, so at
    // most ceil(chunks / G) + 2 row chunks, and chunks <= ceil(T / MR) + E (offsets are made
    // non-decreasing, so the experts' rows add up to at most T).
    const int MR = rows_per_item;
    const long long chunks = ((long long)a.T + MR - 1) / MR + a.E;
    const long long need = (long long)MR * ((chunks + cus - 1) / cus + 2);
    const int nwin = (a.K + kGroupedWindow - 1) / kGroupedWindow;
    const int row_bytes = nwin * (kGroupedWindow / kChunkK) * kGroupedSlot;
    const int ldsx = need * (row_bytes + 4) <= kGroupedXLds ? 1 : 0;
    const int xrows = ldsx ? (int)need : 0;
    const bool few = MR == 1 && a.T <= kGroupedFewRows;
    const GroupedFn fn = few ? kGroupedFew[ldsx][fast] : kGrouped[ldsx][fast][mi];
    const int waves = few ? 8 : kGroupedWaves[ldsx][mi];
    const int lds = xrows * (row_bytes + 4);
    const hipError_t le = allow_dynamic_lds(reinterpret_cast<const void *>(fn), lds);
    if (le != hipSuccess)
        return le;
    hipLaunchKernelGGL(fn, dim3((unsigned)cus), dim3(kWave * waves), (size_t)lds, stream, a,
                       xrows);
    return hipGetLastError();
}

}  // namespace nvfp4

// grouped.hip -- launch of the grouped (mixture-of-experts) NVFP4 GEMM (grouped.h).
#include <algorithm>

#include "grouped.h"
#include "launch.h"

namespace nvfp4 {

namespace {

typedef void (*GroupedFn)(GroupedArgs);

// [FAST][MR index: 1, 2, 4 rows per item]. Wavefronts per workgroup and windows in flight per
// wavefront shrink as the rows (and the x registers of a window) grow.
const GroupedFn kGrouped[2][3] = {
    {&grouped_gemv_kernel<1, 16, 3, false>, &grouped_gemv_kernel<2, 8, 3, false>,
     &grouped_gemv_kernel<4, 8, 2, false>},
    {&grouped_gemv_kernel<1, 16, 3, true>, &grouped_gemv_kernel<2, 8, 3, true>,
     &grouped_gemv_kernel<4, 8, 2, true>}};
const int kGroupedWaves[3] = {16, 8, 8};

}  // namespace

int grouped_rows_per_item(int T, int E, int requested)
{
    if (requested != 0)
        return requested;
    // Decode routes each token to a few experts, one row each; verification puts a few rows on
    // the popular ones.
    return T <= E ? 1 : T <= 2 * E ? 2 : 4;
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
    hipLaunchKernelGGL(kGrouped[fast][mi], dim3((unsigned)cus), dim3(kWave * kGroupedWaves[mi]), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4

// neighbours.h -- the RMSNorm before the GEMM as a kernel of its own, for the fused entry point
// (nvfp4_gemm_fused) above 4 rows (up to 4 the dot-product kernel normalises X in LDS itself;
// SiLU(gate) * up is always inside the GEMM kernels' epilogues) ("SparkInfer" README, section
// "Layout & scoring": RMSNorm and fused FFN kernels).
#pragma once

#include "device.h"

namespace nvfp4 {

// One workgroup of 256 threads per row m: Xn[m][k] = bf16((x * r) * gamma[k]) with
// r = 1 / sqrt(mean_k x^2 + eps). The sum of squares: thread t adds the 8-value pieces t,
// t + 256, ... in order (fma), then a fixed butterfly over the wavefront, then the four wavefronts
// in order, so its relative error stays below (K / 64 + 32) 2^-24, as in the dot-product kernel's
// prologue. The first 4 * 256 pieces of the row (K <= 8192: all of it) and their gamma pieces
// are loaded once, together, and kept in registers for the normalisation; longer rows read the
// rest again.
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const uint16_t *X, const uint16_t *gamma,
                                                           float eps, int K, uint16_t *Xn)
{
    constexpr int B = 4;   // pieces per thread kept in registers
    __shared__ float wsum[4];
    const size_t row = (size_t)blockIdx.x * (size_t)K;
    const int npieces = K / 8;
    auto sumsq = [](const u32x4_t &v, float t) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float lo = __uint_as_float(v[j] << 16);
            const float hi = __uint_as_float(v[j] & 0xFFFF0000u);
            t = __builtin_fmaf(lo, lo, t);
            t = __builtin_fmaf(hi, hi, t);
        }
        return t;
    };
    auto norm = [](const u32x4_t &v, const u32x4_t &gm, float r) {
        u32x4_t o;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float x0 = __uint_as_float(v[j] << 16) * r;
            const float x1 = __uint_as_float(v[j] & 0xFFFF0000u) * r;
            bf16x2_t y;
            y[0] = (__bf16)(x0 * __uint_as_float(gm[j] << 16));
            y[1] = (__bf16)(x1 * __uint_as_float(gm[j] & 0xFFFF0000u));
            o[j] = __builtin_bit_cast(uint32_t, y);
        }
        return o;
    };
    u32x4_t v[B], gm[B];
#pragma unroll
    for (int i = 0; i < B; i++) {
        const int p = threadIdx.x + 256 * i;
        v[i] = p < npieces ? *reinterpret_cast<const u32x4_t *>(X + row + 8 * p)
                           : u32x4_t{0u, 0u, 0u, 0u};
        gm[i] = p < npieces ? *reinterpret_cast<const u32x4_t *>(gamma + 8 * p)
                            : u32x4_t{0u, 0u, 0u, 0u};
    }
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < B; i++)
        t = sumsq(v[i], t);
    for (int p = threadIdx.x + 256 * B; p < npieces; p += 256)
        t = sumsq(*reinterpret_cast<const u32x4_t *>(X + row + 8 * p), t);
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1)
        t += __shfl_xor(t, d);
    if ((threadIdx.x & (kWave - 1)) == 0)
        wsum[threadIdx.x / kWave] = t;
    __syncthreads();
    const float s = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    const float r = 1.0f / __builtin_sqrtf(s / (float)K + eps);
#pragma unroll
    for (int i = 0; i < B; i++) {
        const int p = threadIdx.x + 256 * i;
        if (p < npieces)
            *reinterpret_cast<u32x4_t *>(Xn + row + 8 * p) = norm(v[i], gm[i], r);
    }
    for (int p = threadIdx.x + 256 * B; p < npieces; p += 256)
        *reinterpret_cast<u32x4_t *>(Xn + row + 8 * p) =
            norm(*reinterpret_cast<const u32x4_t *>(X + row + 8 * p),
                 *reinterpret_cast<const u32x4_t *>(gamma + 8 * p), r);
}

}  // namespace nvfp4

// neighbours.h -- the RMSNorm before the GEMM as a kernel of its own, for the fused entry point
// (nvfp4_gemm_fused) above 4 rows (up to 4 the dot-product kernel normalises X in LDS itself;
// SiLU(gate) * up is always inside the GEMM kernels' epilogues) ("SparkInfer" README, section
// "Layout & scoring": RMSNorm and fused FFN kernels).
#pragma once

#include "device.h"

namespace nvfp4 {

// One workgroup of 256 threads per row m: Xn[m][k] = bf16((x * r) * gamma[k]) with
// r = 1 / sqrt(mean_k x^2 + eps). The sum of squares: thread t adds the 8-value pieces t,
// t + 256, ... in order (fma; four loads in flight), then a fixed butterfly over the wavefront,
// then the four wavefronts in order, so its relative error stays below (K / 64 + 32) 2^-24, as in
// the dot-product kernel's prologue.
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const uint16_t *X, const uint16_t *gamma,
                                                           float eps, int K, uint16_t *Xn)
{
    constexpr int B = 4;   // pieces in flight per thread
    __shared__ float wsum[4];
    const size_t row = (size_t)blockIdx.x * (size_t)K;
    const int npieces = K / 8;
    float t = 0.0f;
    for (int p0 = threadIdx.x; p0 < npieces; p0 += B * 256) {
        u32x4_t v[B];
#pragma unroll
        for (int i = 0; i < B; i++) {
            const int p = p0 + 256 * i;
            v[i] = p < npieces ? *reinterpret_cast<const u32x4_t *>(X + row + 8 * p)
                               : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < B; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float lo = __uint_as_float(v[i][j] << 16);
                const float hi = __uint_as_float(v[i][j] & 0xFFFF0000u);
                t = __builtin_fmaf(lo, lo, t);
                t = __builtin_fmaf(hi, hi, t);
            }
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1)
        t += __shfl_xor(t, d);
    if ((threadIdx.x & (kWave - 1)) == 0)
        wsum[threadIdx.x / kWave] = t;
    __syncthreads();
    const float s = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    const float r = 1.0f / __builtin_sqrtf(s / (float)K + eps);
    for (int p0 = threadIdx.x; p0 < npieces; p0 += B * 256) {
        u32x4_t v[B], gm[B];
#pragma unroll
        for (int i = 0; i < B; i++) {
            const int p = p0 + 256 * i;
            if (p < npieces) {
                v[i] = *reinterpret_cast<const u32x4_t *>(X + row + 8 * p);
                gm[i] = *reinterpret_cast<const u32x4_t *>(gamma + 8 * p);
            }
        }
#pragma unroll
        for (int i = 0; i < B; i++) {
            const int p = p0 + 256 * i;
            if (p >= npieces)
                break;
            u32x4_t o;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x0 = __uint_as_float(v[i][j] << 16) * r;
                const float x1 = __uint_as_float(v[i][j] & 0xFFFF0000u) * r;
                bf16x2_t y;
                y[0] = (__bf16)(x0 * __uint_as_float(gm[i][j] << 16));
                y[1] = (__bf16)(x1 * __uint_as_float(gm[i][j] & 0xFFFF0000u));
                o[j] = __builtin_bit_cast(uint32_t, y);
            }
            *reinterpret_cast<u32x4_t *>(Xn + row + 8 * p) = o;
        }
    }
}

}  // namespace nvfp4

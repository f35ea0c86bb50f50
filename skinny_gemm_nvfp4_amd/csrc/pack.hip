// pack.hip -- NVFP4 quantisation (set-up step, not on the timed path) for gfx950.
//
// The page's checkpoint is quantised offline with NVIDIA ModelOpt to "NVFP4 W4A4, group size 16"
// ("Qwen3.8-27B-NVFP4-RTX5090" model card, table "Recipe (NVIDIA ModelOpt)"); the recipe used here
// is the workloads' own: g = amax / (6*448), per block s = E4M3(block_amax / (6 g)), codes =
// E2M1(w / (s g)). Every step is one fp32 IEEE operation, round-to-nearest-even, in that order;
// roundings to E4M3 / E2M1 are nearest with ties to the even code and saturate at 448 / 6.
//
// Three kernels on one stream:
//   1. pack_amax_kernel  : max |w| as an unsigned atomicMax on the fp32 bit pattern (for
//                          non-negative floats the bit order is the numeric order) into *gscale,
//                          which pack_clear_kernel zeroed first.
//   2. pack_scale_kernel : *gscale = amax / 2688 (one thread; correctly rounded division).
//   3. pack_quant_kernel : one thread per (block b, column n) of the padded layout (columns up
//                          to a multiple of 4, blocks up to a multiple of 2); consecutive lanes
//                          take consecutive n, so the 16 reads of a block are coalesced across
//                          the wavefront. Padding positions are written as zero bytes.
#include "device.h"
#include "launch.h"

namespace nvfp4 {

// Nearest E4M3 byte to t >= 0, ties to even, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float t)
{
    if (!(t < 448.0f))
        return 0x7Eu;
    if (t < 0.015625f) {
        // Below 2^-6 the E4M3 grid is the subnormal step 2^-9; t * 512 is exact and rintf rounds
        // half to even. The result 0..8 is also the byte (8 encodes 2^-6).
        return (uint32_t)rintf(t * 512.0f);
    }
    // Normal range: keep 3 mantissa bits of the fp32 pattern with round-half-even on the bits.
    const uint32_t u = __float_as_uint(t);
    const uint32_t rounded = u + 0x7FFFFu + ((u >> 20) & 1u);
    const uint32_t expo = (rounded >> 23) - 120u;  // fp32 bias 127 -> E4M3 bias 7
    const uint32_t mant = (rounded >> 20) & 7u;
    return (expo << 3) | mant;
}

// Nearest E2M1 code to q, ties to even, saturating at 6; the sign bit follows q (so -0.1 -> 8).
// The thresholds are the midpoints between neighbouring magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; at a
// midpoint the even code wins, hence '>' where the lower neighbour is even and '>=' otherwise.
__device__ __forceinline__ uint32_t f32_to_e2m1_rne_sat(float q)
{
    const float a = fabsf(q);
    const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                         (uint32_t)(a > 5.0f);
    return ((__float_as_uint(q) >> 31) << 3) | mag;
}

__global__ void pack_clear_kernel(uint32_t *slot)
{
    *slot = 0u;
}

__global__ __launch_bounds__(256) void pack_amax_kernel(const float4 *W, size_t count4,
                                                        uint32_t *slot)
{
    uint32_t best = 0u;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count4; i += stride) {
        const float4 v = W[i];
        best = max(best, __float_as_uint(v.x) & 0x7FFFFFFFu);
        best = max(best, __float_as_uint(v.y) & 0x7FFFFFFFu);
        best = max(best, __float_as_uint(v.z) & 0x7FFFFFFFu);
        best = max(best, __float_as_uint(v.w) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        best = max(best, (uint32_t)__shfl_xor((int)best, off));
    if ((threadIdx.x & (kWave - 1)) == 0)
        atomicMax(slot, best);
}

__global__ void pack_scale_kernel(float *gscale)
{
    const float amax = __uint_as_float(*reinterpret_cast<uint32_t *>(gscale));
    *gscale = amax / 2688.0f;  // 6 * 448
}

__global__ __launch_bounds__(256) void pack_quant_kernel(int K, int N, const float *W,
                                                         uint8_t *Wq, uint8_t *Ws,
                                                         const float *gscale)
{
    const int CH = num_chunks(K);
    const int NP = kGroupCols * num_groups(N);
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)(2 * CH) * (size_t)NP)
        return;
    const int n = (int)(idx % (size_t)NP);
    const int b = (int)(idx / (size_t)NP);
    uint8_t *codes_out = Wq + code_offset(n, b / 2, CH) + 8 * (b & 1);
    uint8_t *scale_out = Ws + scale_offset(n, b / 2, CH) + (b & 1);
    const float g = *gscale;

    // Padding (n >= N or k >= K), or an all-zero or underflowing tensor: every byte 0.
    if (n >= N || 16 * b >= K || g == 0.0f) {
        *reinterpret_cast<uint2 *>(codes_out) = make_uint2(0u, 0u);
        *scale_out = 0;
        return;
    }
    float w[16];
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        w[i] = W[(16 * (size_t)b + i) * (size_t)N + n];
        const float a = fabsf(w[i]);
        if (a > bmax)
            bmax = a;
    }
    const float sixg = 6.0f * g;
    const float t = bmax / sixg;
    const uint32_t sbyte = f32_to_e4m3_rne_sat(t);
    const float d = e4m3_to_f32<0>(sbyte) * g;
    uint32_t lo = 0u, hi = 0u;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; i++)
            lo |= f32_to_e2m1_rne_sat(w[i] / d) << (4 * i);
#pragma unroll
        for (int i = 0; i < 8; i++)
            hi |= f32_to_e2m1_rne_sat(w[8 + i] / d) << (4 * i);
    }
    *reinterpret_cast<uint2 *>(codes_out) = make_uint2(lo, hi);
    *scale_out = (uint8_t)sbyte;
}

hipError_t launch_pack(int K, int N, const float *W, uint8_t *Wq, uint8_t *Ws, float *gscale,
                       hipStream_t stream)
{
    (void)hipGetLastError();  // start from a clean error state
    uint32_t *slot = reinterpret_cast<uint32_t *>(gscale);
    const size_t count4 = (size_t)K * (size_t)N / 4;  // K % 16 == 0
    const size_t want = (count4 + 255) / 256;
    const unsigned amax_blocks = (unsigned)(want < 8192 ? (want ? want : 1) : 8192);
    hipLaunchKernelGGL(pack_clear_kernel, dim3(1), dim3(1), 0, stream, slot);
    hipLaunchKernelGGL(pack_amax_kernel, dim3(amax_blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(W), count4, slot);
    hipLaunchKernelGGL(pack_scale_kernel, dim3(1), dim3(1), 0, stream, gscale);
    const size_t threads = (size_t)(2 * num_chunks(K)) * (size_t)(kGroupCols * num_groups(N));
    const size_t qblocks = (threads + 255) / 256;
    hipLaunchKernelGGL(pack_quant_kernel, dim3((unsigned)qblocks), dim3(256), 0, stream, K, N, W,
                       Wq, Ws, gscale);
    return hipGetLastError();
}

}  // namespace nvfp4

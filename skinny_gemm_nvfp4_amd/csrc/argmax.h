// argmax.h -- greedy-token epilogue: the GEMM's outputs folded into one argmax per row.
//
// Greedy decode takes, for every row of X, the column of the largest logit of the lm_head GEMM
// ("SparkInfer" README: decode and speculative verification measured greedy, and a request
// speculating alone gets the tokens it would get without the drafter). The lm_head is a
// full-vocabulary GEMM read on every token ("Qwen3.8-27B-NVFP4-RTX5090" model card, section on
// why lm_head is NVFP4), so its M x N fp32 logits are the largest output of the pass; the argmax
// mode never writes them.
//
// Key. (value, column) is mapped to one unsigned 64-bit integer whose order is "larger value
// first, then smaller column": the high word is the fp32 bit pattern made monotone (sign bit
// flipped for non-negative values, all bits flipped for negative ones), the low word is
// ~column. -0 is taken as +0 and every NaN as the positive quiet NaN, so a NaN wins like any
// value above +inf. Every real key is non-zero, so 0 means "no output seen". The maximum of keys
// is associative and commutative: any fold order gives the same winner, so results are exact and
// reproducible however the writers split the columns.
//
// Fold. Each writer (a workgroup of the dot-product kernel, or a group of wavefronts of the
// matrix-core kernels) folds the outputs it owns into per-row keys, reduces them across its lanes
// and stores one key per row in its slot of the workspace; argmax_finalize_kernel then takes the
// maximum over a row's slots and writes the column and the fp32 value.
#pragma once

#include "device.h"

namespace nvfp4 {

typedef unsigned long long argkey_t;

__device__ __forceinline__ argkey_t argmax_key(float v, int col)
{
    uint32_t u = __float_as_uint(v);
    if (v != v)
        u = 0x7FC00000u;            // every NaN ranks as the positive quiet NaN
    else if (u == 0x80000000u)
        u = 0u;                     // -0 ranks as +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((argkey_t)u << 32) | (argkey_t)(~(uint32_t)col);
}

__device__ __forceinline__ float argmax_key_value(argkey_t k)
{
    const uint32_t u = (uint32_t)(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ int argmax_key_column(argkey_t k)
{
    return (int)~(uint32_t)k;
}

__device__ __forceinline__ argkey_t key_max(argkey_t a, argkey_t b) { return a > b ? a : b; }

__device__ __forceinline__ argkey_t shfl_xor_key(argkey_t k, int m)
{
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)k, m);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(k >> 32), m);
    return ((argkey_t)hi << 32) | lo;
}

// Maximum over the 16 lanes of each row of 16 (lanes 16 q .. 16 q + 15); every lane gets it.
__device__ __forceinline__ argkey_t key_max_16(argkey_t k)
{
    k = key_max(k, shfl_xor_key(k, 1));
    k = key_max(k, shfl_xor_key(k, 2));
    k = key_max(k, shfl_xor_key(k, 4));
    return key_max(k, shfl_xor_key(k, 8));
}

// Maximum over all 64 lanes; every lane gets it.
__device__ __forceinline__ argkey_t key_max_64(argkey_t k)
{
    k = key_max_16(k);
    k = key_max(k, shfl_xor_key(k, 16));
    return key_max(k, shfl_xor_key(k, 32));
}

// Row m of the workspace holds `slots` keys; one workgroup per row writes the winner's column to
// index[m] and its fp32 value to value[m].
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const argkey_t *keys, int slots,
                                                              int32_t *index, float *value)
{
    __shared__ argkey_t best[4];
    const int m = blockIdx.x;
    const argkey_t *row = keys + (size_t)m * (size_t)slots;
    argkey_t k = 0;
    // Eight loads in flight per thread (a row holds up to 16 keys per compute unit).
    for (int s0 = threadIdx.x; s0 < slots; s0 += 8 * 256) {
        argkey_t v[8];
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = s0 + 256 * i < slots ? row[s0 + 256 * i] : 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
            k = key_max(k, v[i]);
    }
    k = key_max_64(k);
    if ((threadIdx.x & (kWave - 1)) == 0)
        best[threadIdx.x / kWave] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
        k = key_max(key_max(best[0], best[1]), key_max(best[2], best[3]));
        index[m] = k == 0 ? -1 : argmax_key_column(k);
        value[m] = argmax_key_value(k);
    }
}

}  // namespace nvfp4

// device.h -- gfx950 device helpers shared by the NVFP4 kernels of libnvfp4.so.
//
// Decode primitives (all exact):
//   * E2M1 codes -> bf16 / fp32 through the gfx950 converters v_cvt_scalef32_pk_{bf16,f32}_fp4.
//     Their fp32 scale operand contributes only its exponent, so they are called with scale 1.0
//     and the E4M3 block scale is applied separately.
//   * E4M3 bytes -> fp32 through v_cvt_f32_fp8, which on gfx950 decodes the OCP E4M3FN format
//     (bias 7, max 448, NaN at 0x7F/0xFF), the block-scale format of NVFP4 ("Qwen3.8-27B-NVFP4-
//     RTX5090" model card, table "Recipe (NVIDIA ModelOpt)": NVFP4, group size 16).
//   * e2m1 * s has at most 2 + 4 significant bits, so it is exact in fp32 and in bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;          // lanes per wavefront on CDNA
constexpr int kTileN = 16;         // output columns n per workgroup tile
constexpr int kStepK = 256;        // k covered by one wave in one step (4 lane groups x 2 chunks x 32)
constexpr int kChunkK = 32;        // k per chunk: 16 bytes of codes, two 16-element blocks

// E4M3 byte SEL of w, decoded to fp32.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w)
{
    return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

// The two E2M1 codes of byte SEL of w (low nibble = element 0) as bf16, unscaled.
template <int SEL>
__device__ __forceinline__ bf16x2_t e2m1x2_to_bf16(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

// The two E2M1 codes of byte SEL of w as fp32, unscaled.
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_to_f32(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Eight codes of w (k ascending, low nibble first) times the block scale s, as bf16. Exact.
__device__ __forceinline__ bf16x8_t decode8_scaled(uint32_t w, float s)
{
    f32x2_t a = e2m1x2_to_f32<0>(w);
    f32x2_t b = e2m1x2_to_f32<1>(w);
    f32x2_t c = e2m1x2_to_f32<2>(w);
    f32x2_t d = e2m1x2_to_f32<3>(w);
    bf16x8_t r;
    r[0] = (__bf16)(a.x * s);
    r[1] = (__bf16)(a.y * s);
    r[2] = (__bf16)(b.x * s);
    r[3] = (__bf16)(b.y * s);
    r[4] = (__bf16)(c.x * s);
    r[5] = (__bf16)(c.y * s);
    r[6] = (__bf16)(d.x * s);
    r[7] = (__bf16)(d.y * s);
    return r;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u)
{
    return __builtin_bit_cast(bf16x2_t, u);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u)
{
    return __builtin_bit_cast(bf16x8_t, u);
}

// One chunk of one output column: 32 consecutive k, i.e. 16 code bytes and 2 scale bytes.
struct Chunk {
    uint32_t code[4];   // code[d] holds k = 8d .. 8d+7 of the chunk
    uint32_t scale;     // byte 0: block of k 0..15, byte 1: block of k 16..31
};

// Loads the chunk of row (wq_row, ws_row) that starts at k = kc (a multiple of 32).
// NARROW is for K % 32 == 16, where rows are only 8-byte aligned and the last chunk of a row may
// hold a single block. Blocks at or beyond K read as code 0 with scale byte 0.
template <bool NARROW>
__device__ __forceinline__ Chunk load_chunk(const uint8_t *wq_row, const uint8_t *ws_row, int kc,
                                            int K, bool row_ok)
{
    Chunk c;
    c.code[0] = c.code[1] = c.code[2] = c.code[3] = 0u;
    c.scale = 0u;
    if (!row_ok)
        return c;
    if (!NARROW) {
        if (kc < K) {  // K % 32 == 0: the chunk is either whole or absent
            u32x4_t v = *reinterpret_cast<const u32x4_t *>(wq_row + kc / 2);
            c.code[0] = v[0];
            c.code[1] = v[1];
            c.code[2] = v[2];
            c.code[3] = v[3];
            c.scale = *reinterpret_cast<const uint16_t *>(ws_row + kc / 16);
        }
    } else {
        if (kc < K) {
            u32x2_t v = *reinterpret_cast<const u32x2_t *>(wq_row + kc / 2);
            c.code[0] = v[0];
            c.code[1] = v[1];
            c.scale = ws_row[kc / 16];
        }
        if (kc + 16 < K) {
            u32x2_t v = *reinterpret_cast<const u32x2_t *>(wq_row + kc / 2 + 8);
            c.code[2] = v[0];
            c.code[3] = v[1];
            c.scale |= (uint32_t)ws_row[kc / 16 + 1] << 8;
        }
    }
    return c;
}

// Eight bf16 of X row m at k .. k+7 (16 bytes), or zeros if the row or the k range is outside.
// K % 16 == 0 and k % 8 == 0, so k < K implies k + 8 <= K.
__device__ __forceinline__ u32x4_t load_x8(const uint16_t *X, int m, int M, int k, int K)
{
    if (m < M && k < K)
        return *reinterpret_cast<const u32x4_t *>(X + (size_t)m * K + k);
    u32x4_t z = {0u, 0u, 0u, 0u};
    return z;
}

}  // namespace nvfp4

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
//
// Memory helpers: raw buffer descriptors, so that loads past a workgroup's range read zeros.
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

// Four words of 8 codes -> 16 bf16 pairs; pair 4 d + b holds k = 8 d + 2 b and 8 d + 2 b + 1.
__device__ __forceinline__ void decode32_bf16(const uint32_t code[4], bf16x2_t w[16])
{
#pragma unroll
    for (int d = 0; d < 4; d++) {
        w[4 * d + 0] = e2m1x2_to_bf16<0>(code[d]);
        w[4 * d + 1] = e2m1x2_to_bf16<1>(code[d]);
        w[4 * d + 2] = e2m1x2_to_bf16<2>(code[d]);
        w[4 * d + 3] = e2m1x2_to_bf16<3>(code[d]);
    }
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u)
{
    return __builtin_bit_cast(bf16x2_t, u);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u)
{
    return __builtin_bit_cast(bf16x8_t, u);
}

// ------------------------------------------------------------------------------------------
// Loads through raw buffer descriptors. A descriptor covers one workgroup's rows of an array
// (base pointer and byte count); a load whose offset is at or past the count returns zeros
// without touching memory. Ragged rows, ragged K and the prefetch past a wave's last window are
// all expressed that way, so the K loops carry no branches and no exec-masked loads, and the
// loads retire in the order they were issued.
// ------------------------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kRawBufferFlags = 0x00020000;     // word 3 of an unformatted gfx9 descriptor
constexpr int kAuxStream = 2;                    // "nt": read-once data
constexpr int kAuxNormal = 0;
constexpr uint32_t kOutOfRange = 0x80000000u;   // beyond every byte count used here

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRawBufferFlags);
}

__device__ __forceinline__ uint32_t off_if(bool valid, uint32_t off)
{
    return valid ? off : kOutOfRange;
}

// Wait until at most N vector memory operations of this wavefront are outstanding (they complete
// in issue order; direct-to-LDS loads count among them).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A buffer descriptor the compiler keeps in scalar registers: the direct-to-LDS loads need one,
// and a descriptor it cannot prove uniform costs a readfirstlane loop around every load.
__device__ __forceinline__ rsrc_t uniform_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return make_rsrc(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo), n);
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at dst + 16 l (dst the same in
// every lane), without passing through registers.
__device__ __forceinline__ void lds_load16(rsrc_t r, uint8_t *dst, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
}

// One chunk of one output column: 32 consecutive k, i.e. 16 code bytes and the aligned 4-byte
// word that holds the chunk's 2 scale bytes (and those of the neighbouring column of the group).
struct Chunk {
    uint32_t code[4];   // code[d] holds k = 8d .. 8d+7 of the chunk
    uint32_t scale;     // >> (16 * (column & 1)): byte 0 = block of k 0..15, byte 1 = k 16..31
};

// Sum of v over the 16 lanes that share lane & 3, in a fixed order (lane distance 4, 8, 16, 32),
// so every lane gets the same bits.
__device__ __forceinline__ float sum_lanes_stride4(float v)
{
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    const uint32_t u = __float_as_uint(v);
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const uint32_t u2 = __float_as_uint(v);
    auto p2 = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
    return __uint_as_float(p2[0]) + __uint_as_float(p2[1]);
}

// A value the compiler may keep in a scalar register (it is the same in every lane).
__device__ __forceinline__ int uniform(int v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

}  // namespace nvfp4

// launch.h -- internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

struct GemmArgs {
    const uint16_t *X;       // bf16 bits [M][K]
    const uint8_t *Wq;       // [N][K/2]
    const uint8_t *Ws;       // [N][K/16]
    const float *gscale;     // [1]
    float *Y;                // [M][N]
    int M, N, K;
};

enum Path { kPathAuto = 0, kPathDot = 1, kPathMfma = 2, kPathStream = 3, kPathMfmaStream = 4 };

// Largest M the dot-product kernel families are instantiated for.
constexpr int kDotMaxM = 8;

// Largest K: keeps every per-workgroup byte range of the buffer loads below 2^31.
constexpr int kMaxK = 1 << 22;

// Resolves path/split (0 = automatic) for this shape. Returns false for an unsupported pair.
// A persistent dot-product request whose X does not fit in LDS becomes the tiled dot-product
// path; a persistent matrix-core request with K % 128 != 0 becomes the tiled matrix-core path.
bool choose_config(int M, int N, int K, int *path, int *split);

// Launch the GEMM with a resolved path and split. Returns the hipError_t of the launch.
hipError_t launch_gemm(int path, int split, const GemmArgs &a, hipStream_t stream);

// Launch the three-kernel pack sequence (amax, tensor scale, quantise) on the stream.
hipError_t launch_pack(int K, int N, const float *W, uint8_t *Wq, uint8_t *Ws, float *gscale,
                       hipStream_t stream);

}  // namespace nvfp4

// launch.h -- internal interface between the C ABI (api.cpp) and the kernel launchers, and the
// packed-weight layout shared by the packer and the GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

struct GemmArgs {
    const uint16_t *X;       // bf16 bits [M][K]
    const uint8_t *Wq;       // [NG][CH][4][16]
    const uint8_t *Ws;       // [NG][CH][4][2]
    const float *gscale;     // [1]
    float *Y;                // [M][N]; unused when keys is set
    int M, N, K;
    // Argmax mode (nvfp4_gemm_argmax): instead of storing Y, each writer folds the outputs it
    // owns into one argmax key per row (argmax.h) and stores it at keys[m * key_slots + slot].
    unsigned long long *keys = nullptr;
    int key_slots = 0;
    // Layer neighbours (nvfp4_gemm_fused). gamma set (dot-product kernel only): X is replaced by
    // its RMSNorm, rounded to bf16, xhat = bf16((x * r) * gamma[k]) with r = 1 / sqrt(mean_k x^2
    // + eps) per row. H set (dot-product and 16-row kernels): instead of Y, H[m][j] =
    // bf16(SiLU(gate) * up) from the column pairs of the interleaved gate/up weight (columns
    // 8q + c and 8q + 4 + c, c < 4, give j = 4q + c); N % 8 == 0.
    const uint16_t *gamma = nullptr;   // bf16 [K]
    float eps = 0.0f;
    uint16_t *H = nullptr;             // bf16 [M][N / 2]
    // Caller-owned device scratch of nvfp4_gemm_fused (the normalised X when a kernel of its own
    // computes the RMSNorm).
    void *workspace = nullptr;
    size_t workspace_bytes = 0;
};

// Packed layout: 4-column groups, 32-k chunks. One chunk of one group is 4 x 16 code bytes
// (column-major inside the chunk: column j's 32 codes are bytes 16 j .. 16 j + 15) and 4 x 2
// scale bytes. Groups are contiguous runs of CH chunks.
constexpr int kGroupCols = 4;
constexpr int kChunkK = 32;
constexpr int kChunkCodeBytes = kGroupCols * 16;   // 64
constexpr int kChunkScaleBytes = kGroupCols * 2;   // 8

__host__ __device__ inline int num_groups(int N) { return (N + kGroupCols - 1) / kGroupCols; }

// The NG column groups dealt to G workgroups: NG / G each and one more to the first NG % G, so
// every workgroup streams the same weight bytes to within one group. Workgroup b owns groups
// [*first, *first + *count). 32-bit arithmetic only (a 64-bit division costs the kernel hundreds
// of scalar instructions before its first load).
__device__ __forceinline__ void group_range(int NG, int G, int b, int *first, int *count)
{
    const uint32_t q = (uint32_t)NG / (uint32_t)G;
    const uint32_t r = (uint32_t)NG - q * (uint32_t)G;
    *first = (int)((uint32_t)b * q + min((uint32_t)b, r));
    *count = (int)(q + ((uint32_t)b < r ? 1u : 0u));
}
__host__ __device__ inline int num_chunks(int K) { return (K + kChunkK - 1) / kChunkK; }

// Byte offset of the 16 code bytes of (column n, chunk c) and of the scale pair of the same.
__host__ __device__ inline size_t code_offset(int n, int c, int CH)
{
    return (((size_t)(n / kGroupCols) * (size_t)CH + (size_t)c) * kGroupCols + (size_t)(n % 4)) *
           16u;
}
__host__ __device__ inline size_t scale_offset(int n, int c, int CH)
{
    return (((size_t)(n / kGroupCols) * (size_t)CH + (size_t)c) * kGroupCols + (size_t)(n % 4)) *
           2u;
}

inline uint64_t codes_bytes(int N, int K)
{
    return (uint64_t)num_groups(N) * (uint64_t)num_chunks(K) * kChunkCodeBytes;
}
inline uint64_t scales_bytes(int N, int K)
{
    return (uint64_t)num_groups(N) * (uint64_t)num_chunks(K) * kChunkScaleBytes;
}

enum Path {
    kPathAuto = 0,
    kPathDot = 1,
    kPathMfma = 2,
    kPathBatch = 3,
    kPathInvariant = 5
};

// Largest M the dot-product kernel is instantiated for.
constexpr int kDotMaxM = 8;

// Largest K: keeps every per-workgroup byte range of the buffer loads below 2^31.
constexpr int kMaxK = 1 << 22;

// Resolves path/split (0 = automatic) for this shape. Returns false for an unsupported pair.
// A dot-product request whose X does not fit in LDS becomes the matrix-core path.
bool choose_config(int M, int N, int K, int *path, int *split);

// Lets kernel `fn` take `bytes` of dynamic LDS (above the 64 KB default it must opt in, once per
// kernel and device).
hipError_t allow_dynamic_lds(const void *fn, int bytes);

// Launch the GEMM with a resolved path and split. Returns the hipError_t of the launch.
hipError_t launch_gemm(int path, int split, const GemmArgs &a, hipStream_t stream);

// Largest number of argmax key slots per row for a device with `cus` compute units: the
// dot-product kernel writes one per wavefront (at most 16 per workgroup, one workgroup per
// compute unit); the other writers fewer.
constexpr int kArgmaxSlotsPerCu = 16;

// Argmax variant of launch_gemm: the same kernels and plan, outputs folded into per-row keys in
// `keys` ([M][key_slots], key_slots <= kArgmaxSlotsPerCu * compute units), then one key per row
// turned into index and value.
hipError_t launch_gemm_argmax(int path, int split, const GemmArgs &a, int32_t *index,
                              float *value, hipStream_t stream);

// nvfp4_gemm_argmax_noalloc keeps its keys in a static device array of kScratchKeys keys (4 MiB).
constexpr size_t kScratchKeys = (size_t)(4u << 20) / sizeof(unsigned long long);

// Rows that array holds on the current device: kScratchKeys / (kArgmaxSlotsPerCu * compute
// units), 128 on a 256-CU device.
int argmax_scratch_rows();

// Device address of that array on the current device (looked up once per device).
hipError_t argmax_scratch(unsigned long long **keys);

// Launch of nvfp4_gemm_fused: RMSNorm prologue (a.gamma) and/or SiLU(gate) * up epilogue (a.H).
// The normalised X goes to a.workspace when fused_workspace_bytes() is not zero.
hipError_t launch_gemm_fused(const GemmArgs &a, hipStream_t stream);

// Workspace bytes nvfp4_gemm_fused needs (0 when one kernel does everything).
size_t fused_workspace_bytes(bool norm, bool pair, int M, int N, int K);

// Compute units of the current device (cached per device).
int device_compute_units();

// Grouped (mixture-of-experts) GEMM: rows offsets[e] .. offsets[e+1] - 1 of X through expert e.
constexpr int kGroupedMaxExperts = 2048;

struct GroupedArgs {
    const uint16_t *X;        // bf16 [T][K], rows sorted by expert
    const int *offsets;       // [E + 1], device
    const uint8_t *Wq;        // E packed weights, each codes_bytes(N, K) bytes
    const uint8_t *Ws;        // E packed scales, each scales_bytes(N, K) bytes
    const float *gscale;      // [E]
    float *Y;                 // fp32 [T][N]
    int T, E, N, K;
};

// Rows of one expert per work item of the grouped kernel: `requested` (1, 2 or 4) or, for 0, a
// choice from the total rows T and the expert count E.
int grouped_rows_per_item(int T, int E, int requested);

// Launch the grouped (mixture-of-experts) GEMM. Largest E: kGroupedMaxExperts (grouped.h).
hipError_t launch_grouped(const GroupedArgs &a, int rows_per_item, hipStream_t stream);

// Launch the pack sequence (clear, amax, tensor scale, quantise) on the stream.
hipError_t launch_pack(int K, int N, const float *W, uint8_t *Wq, uint8_t *Ws, float *gscale,
                       hipStream_t stream);

}  // namespace nvfp4

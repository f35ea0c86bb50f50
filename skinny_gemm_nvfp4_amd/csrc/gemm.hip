// gemm.hip -- NVFP4 skinny GEMM kernels for gfx950: Y[M,N] = X[M,K] . dequant(W)[K,N].
//
// The operation is the per-token weight stream of decode and of speculative verification: every
// NVFP4 weight is read once per forward ("Qwen3.8-27B-NVFP4-RTX5090" model card, section "Why
// lm_head is NVFP4"), with M = 1 for plain decode and M = 16 or 128 when drafted tokens of one or
// eight requests are verified together ("SparkInfer" README, speculative decoding sections).
//
// Work split, shared by both kernel families
//   * A workgroup owns kTileN = 16 consecutive output columns n0 .. n0+15 and W wavefronts.
//   * In every wave, lane l = 16 g + r (r = 0..15, g = 0..3) works on column n0 + r.
//   * K is cut into steps of 256; wave w takes steps w, w+W, w+2W, ...
//   * In the step at k0, lane group g reads two chunks of 32 k (16 code bytes + 2 scale bytes):
//     chunk 0 at k0 + 32 g and chunk 1 at k0 + 128 + 32 g. For one column the four lanes read
//     64 contiguous bytes per load instruction, and a wave covers 16 columns x 256 k per step.
//   * The W partial results of a workgroup are summed through LDS in wave order, then multiplied
//     by the tensor scale g once and stored. Every sum has a fixed order, so results are
//     bit-reproducible.
//
// DOT family (M <= 8): E2M1 -> bf16 through the gfx950 converter, v_dot2_f32_bf16 against the
// matching bf16 pairs of X, one fp32 partial per 16-element block times its E4M3 scale.
// MFMA family (any M): each 8-code dword becomes the bf16 B operand e2m1 * s (exact) of
// v_mfma_f32_16x16x32_bf16; lane group g supplies MFMA k-slots 8g..8g+7, which map to the
// physical k of its own chunk, and the A operand (X) is read with the same mapping.
#include "device.h"
#include "launch.h"

namespace nvfp4 {

// Four words of 8 codes -> 16 bf16 pairs, pair index 4 d + b covers k = 8 d + 2 b, +1.
__device__ __forceinline__ void decode_chunk_bf16(const Chunk &c, bf16x2_t w[16])
{
#pragma unroll
    for (int d = 0; d < 4; d++) {
        w[4 * d + 0] = e2m1x2_to_bf16<0>(c.code[d]);
        w[4 * d + 1] = e2m1x2_to_bf16<1>(c.code[d]);
        w[4 * d + 2] = e2m1x2_to_bf16<2>(c.code[d]);
        w[4 * d + 3] = e2m1x2_to_bf16<3>(c.code[d]);
    }
}

template <int MR, int W, bool NARROW>
__global__ __launch_bounds__(kWave *W) void gemm_dot_kernel(GemmArgs a)
{
    __shared__ float red[W][MR][kTileN];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int K = a.K;
    const int n0 = blockIdx.x * kTileN;
    const int n = n0 + r;
    const bool row_ok = n < a.N;
    const uint8_t *wq_row = a.Wq + (size_t)(row_ok ? n : 0) * (size_t)(K / 2);
    const uint8_t *ws_row = a.Ws + (size_t)(row_ok ? n : 0) * (size_t)(K / 16);

    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; m++)
        acc[m] = 0.0f;

    const int nsteps = (K + kStepK - 1) / kStepK;
    for (int s = wave; s < nsteps; s += W) {
        const int k0 = s * kStepK;
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int kc = k0 + 128 * c + 32 * g;
            const Chunk ch = load_chunk<NARROW>(wq_row, ws_row, kc, K, row_ok);
            const float s0 = e4m3_to_f32<0>(ch.scale);
            const float s1 = e4m3_to_f32<1>(ch.scale);
            bf16x2_t w[16];
            decode_chunk_bf16(ch, w);
#pragma unroll
            for (int m = 0; m < MR; m++) {
                u32x4_t xv[4];
#pragma unroll
                for (int q = 0; q < 4; q++)
                    xv[q] = load_x8(a.X, m, a.M, kc + 8 * q, K);
                float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; i++)
                    p0 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xv[i / 4][i % 4]), p0,
                                                          false);
#pragma unroll
                for (int i = 8; i < 16; i++)
                    p1 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xv[i / 4][i % 4]), p1,
                                                          false);
                acc[m] = acc[m] + p0 * s0;
                acc[m] = acc[m] + p1 * s1;
            }
        }
    }

    // Sum the four lane groups of each column, then the W waves, in a fixed order.
#pragma unroll
    for (int m = 0; m < MR; m++) {
        float v = acc[m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0)
            red[wave][m][r] = v;
    }
    __syncthreads();
    const float gs = *a.gscale;
    for (int idx = threadIdx.x; idx < MR * kTileN; idx += kWave * W) {
        const int m = idx / kTileN;
        const int rr = idx % kTileN;
        if (m < a.M && n0 + rr < a.N) {
            float sum = red[0][m][rr];
#pragma unroll
            for (int w = 1; w < W; w++)
                sum += red[w][m][rr];
            a.Y[(size_t)m * a.N + n0 + rr] = sum * gs;
        }
    }
}

template <int MT, int W, bool NARROW>
__global__ __launch_bounds__(kWave *W) void gemm_mfma_kernel(GemmArgs a)
{
    __shared__ float red[W][kTileN][kTileN];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int K = a.K;
    const int n0 = blockIdx.x * kTileN;
    const int n = n0 + r;
    const bool row_ok = n < a.N;
    const int m_base = blockIdx.y * 16 * MT;
    const uint8_t *wq_row = a.Wq + (size_t)(row_ok ? n : 0) * (size_t)(K / 2);
    const uint8_t *ws_row = a.Ws + (size_t)(row_ok ? n : 0) * (size_t)(K / 16);

    f32x4_t acc[MT];
#pragma unroll
    for (int t = 0; t < MT; t++)
        acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int nsteps = (K + kStepK - 1) / kStepK;
    for (int s = wave; s < nsteps; s += W) {
        const int k0 = s * kStepK;
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int kc = k0 + 128 * c + 32 * g;
            const Chunk ch = load_chunk<NARROW>(wq_row, ws_row, kc, K, row_ok);
            const float s0 = e4m3_to_f32<0>(ch.scale);
            const float s1 = e4m3_to_f32<1>(ch.scale);
#pragma unroll
            for (int d = 0; d < 4; d++) {
                const bf16x8_t b = decode8_scaled(ch.code[d], d < 2 ? s0 : s1);
#pragma unroll
                for (int t = 0; t < MT; t++) {
                    const bf16x8_t x =
                        as_bf16x8(load_x8(a.X, m_base + 16 * t + r, a.M, kc + 8 * d, K));
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, b, acc[t], 0, 0, 0);
                }
            }
        }
    }

    // acc[t][i] is Y[m_base + 16 t + 4 g + i][n0 + r]. Sum the W waves in order, tile by tile.
    const float gs = *a.gscale;
    if (W == 1) {
#pragma unroll
        for (int t = 0; t < MT; t++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int m = m_base + 16 * t + 4 * g + i;
                if (m < a.M && row_ok)
                    a.Y[(size_t)m * a.N + n] = acc[t][i] * gs;
            }
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < MT; t++) {
        __syncthreads();  // the previous tile's readers are done with red
#pragma unroll
        for (int i = 0; i < 4; i++)
            red[wave][4 * g + i][r] = acc[t][i];
        __syncthreads();
        for (int idx = threadIdx.x; idx < kTileN * kTileN; idx += kWave * W) {
            const int row = idx / kTileN;
            const int col = idx % kTileN;
            const int m = m_base + 16 * t + row;
            if (m < a.M && n0 + col < a.N) {
                float sum = red[0][row][col];
#pragma unroll
                for (int w = 1; w < W; w++)
                    sum += red[w][row][col];
                a.Y[(size_t)m * a.N + n0 + col] = sum * gs;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Launch tables.
// ------------------------------------------------------------------------------------------
typedef void (*KernelFn)(GemmArgs);

#define NVFP4_SPLITS(KERN, R, NARROW) \
    { &KERN<R, 1, NARROW>, &KERN<R, 2, NARROW>, &KERN<R, 4, NARROW>, &KERN<R, 8, NARROW> }
#define NVFP4_TABLE(KERN, NARROW)                                                              \
    {                                                                                          \
        NVFP4_SPLITS(KERN, 1, NARROW), NVFP4_SPLITS(KERN, 2, NARROW),                          \
            NVFP4_SPLITS(KERN, 3, NARROW), NVFP4_SPLITS(KERN, 4, NARROW),                      \
            NVFP4_SPLITS(KERN, 5, NARROW), NVFP4_SPLITS(KERN, 6, NARROW),                      \
            NVFP4_SPLITS(KERN, 7, NARROW), NVFP4_SPLITS(KERN, 8, NARROW)                       \
    }

static const KernelFn kDotWide[8][4] = NVFP4_TABLE(gemm_dot_kernel, false);
static const KernelFn kDotNarrow[8][4] = NVFP4_TABLE(gemm_dot_kernel, true);
static const KernelFn kMfmaWide[8][4] = NVFP4_TABLE(gemm_mfma_kernel, false);
static const KernelFn kMfmaNarrow[8][4] = NVFP4_TABLE(gemm_mfma_kernel, true);

static int split_index(int split)
{
    switch (split) {
    case 1: return 0;
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
    default: return -1;
    }
}

bool choose_config(int M, int N, int K, int *path, int *split)
{
    if (*path == kPathAuto)
        *path = (M <= 4) ? kPathDot : kPathMfma;
    if (*path == kPathDot && M > kDotMaxM)
        return false;
    if (*path != kPathDot && *path != kPathMfma)
        return false;
    if (*split == 0) {
        // Enough waves to keep every CU streaming: aim for >= 2048 waves (8 per CU), with at
        // least two K steps per wave.
        const long long tiles = (N + kTileN - 1) / kTileN;
        const int steps = (K + kStepK - 1) / kStepK;
        int w = 1;
        while (w < 8 && tiles * w < 2048 && steps >= 4 * w)
            w *= 2;
        *split = w;
    }
    return split_index(*split) >= 0;
}

hipError_t launch_gemm(int path, int split, const GemmArgs &a, hipStream_t stream)
{
    const bool narrow = (a.K % 32) != 0;
    const int si = split_index(split);
    const dim3 block(kWave * split);
    const unsigned tiles = (unsigned)((a.N + kTileN - 1) / kTileN);
    KernelFn fn;
    dim3 grid;
    if (path == kPathDot) {
        fn = (narrow ? kDotNarrow : kDotWide)[a.M - 1][si];
        grid = dim3(tiles, 1, 1);
    } else {
        const int mt = a.M >= 128 ? 8 : (a.M + 15) / 16;
        const unsigned mchunks = (unsigned)((a.M + 16 * mt - 1) / (16 * mt));
        fn = (narrow ? kMfmaNarrow : kMfmaWide)[mt - 1][si];
        grid = dim3(tiles, mchunks, 1);
    }
    (void)hipGetLastError();  // start from a clean error state
    hipLaunchKernelGGL(fn, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4

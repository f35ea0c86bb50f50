// gemv.h -- NVFP4 x bf16 wavefront dot-product kernel for the smallest M (plain decode, M = 1).
//
// Decode at concurrency 1 streams every weight once per token, so the kernel is a read of the
// packed weights at HBM speed with the arithmetic hidden under it ("Qwen3.8-27B-NVFP4-RTX5090"
// model card, section "Why lm_head is NVFP4").
//
// Work split
//   * A wavefront is four quads of 16 lanes. Lane r of quad q owns 32 consecutive k (16 code
//     bytes, 2 scale bytes) in every window of kGemvWindow = 512 k: k = kw + 32 r .. kw + 32 r + 31.
//     One load instruction therefore reads 256 contiguous bytes of one weight row per quad.
//   * Quad q owns C consecutive output columns; a wavefront covers 4 C columns and a workgroup of
//     S wavefronts shares them, wave w taking windows w, w + S, w + 2 S, ... (split-K inside the
//     workgroup). The X values of a lane's k range are loaded once per window and reused for its
//     C columns.
//   * Per column the 32 codes are decoded E2M1 -> bf16 by the gfx950 converter (exact), paired
//     with X by v_dot2_f32_bf16 into one fp32 partial per 16-block, and the partial is multiplied
//     by the block's E4M3 scale.
//   * Two register sets alternate: every load of the next window (weights and X) is in flight
//     while the current window is multiplied. Loads retire in issue order, so waiting for the
//     current window never waits for the next one.
//   * The 16 lanes of a quad are summed by a butterfly, the S waves through LDS in wave order, and
//     the tensor scale g is applied once. Every sum has a fixed order: results are reproducible.
#pragma once

#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kGemvWindow = 512;

template <int MR, int C, bool NARROW>
struct GemvWindow {
    Chunk c[C];           // the lane's chunk of each of its C columns
    u32x4_t x[MR][4];     // X rows 0 .. MR-1 at the lane's 32 k

    // Issues every load of the window whose lane k range starts at kc.
    __device__ __forceinline__ void load(rsrc_t rq, rsrc_t rs, rsrc_t rx, const uint32_t (&qrow)[C],
                                         const uint32_t (&srow)[C], int kc, int K)
    {
#pragma unroll
        for (int j = 0; j < C; j++)
            c[j] = load_chunk<NARROW>(rq, rs, qrow[j], srow[j], kc, K);
#pragma unroll
        for (int m = 0; m < MR; m++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                x[m][i] = load_x8(rx, (uint32_t)(m * K + kc + 8 * i) * 2u, kc + 8 * i, K);
    }

    __device__ __forceinline__ void mul(float (&acc)[MR][C], const uint32_t (&srow)[C],
                                        int kc) const
    {
#pragma unroll
        for (int j = 0; j < C; j++) {
            const uint32_t sc = scale_pair<NARROW>(c[j].scale, srow[j], kc);
            const float s0 = e4m3_to_f32<0>(sc);
            const float s1 = e4m3_to_f32<1>(sc);
            bf16x2_t w[16];
            decode32_bf16(c[j].code, w);
#pragma unroll
            for (int m = 0; m < MR; m++) {
                float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; i++)
                    p0 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(x[m][i / 4][i % 4]), p0,
                                                          false);
#pragma unroll
                for (int i = 8; i < 16; i++)
                    p1 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(x[m][i / 4][i % 4]), p1,
                                                          false);
                acc[m][j] = __builtin_fmaf(p0, s0, acc[m][j]);
                acc[m][j] = __builtin_fmaf(p1, s1, acc[m][j]);
            }
        }
    }
};

template <int MR, int C, int S, bool NARROW>
__global__ __launch_bounds__(kWave *S) void gemv_kernel(GemmArgs a)
{
    typedef GemvWindow<MR, C, NARROW> Win;
    __shared__ float red[S > 1 ? S : 1][MR][4 * C];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;

    // This workgroup's rows of Wq / Ws, and all M rows of X (M <= 8 here).
    const int nfirst = blockIdx.x * (4 * C);
    const int nrows = min(4 * C, N - nfirst);
    const rsrc_t rq = make_rsrc(a.Wq + (size_t)nfirst * (size_t)(K / 2),
                                (uint32_t)nrows * (uint32_t)(K / 2));
    uint32_t sbias;
    const rsrc_t rs = scale_rsrc(a.Ws, (size_t)nfirst, nrows, K, &sbias);
    const rsrc_t rx = make_rsrc(a.X, (uint32_t)a.M * (uint32_t)K * 2u);
    uint32_t qrow[C], srow[C];
#pragma unroll
    for (int j = 0; j < C; j++) {
        qrow[j] = (uint32_t)(q * C + j) * (uint32_t)(K / 2);
        srow[j] = sbias + (uint32_t)(q * C + j) * (uint32_t)(K / 16);
    }

    float acc[MR][C];
#pragma unroll
    for (int m = 0; m < MR; m++)
#pragma unroll
        for (int j = 0; j < C; j++)
            acc[m][j] = 0.0f;

    const int nwin = (K + kGemvWindow - 1) / kGemvWindow;
    Win wa, wb;
    int win = wave;
    wa.load(rq, rs, rx, qrow, srow, win * kGemvWindow + 32 * r, K);
    while (win < nwin) {
        wb.load(rq, rs, rx, qrow, srow, (win + S) * kGemvWindow + 32 * r, K);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
        wa.mul(acc, srow, win * kGemvWindow + 32 * r);
        win += S;
        if (win >= nwin)
            break;
        wa.load(rq, rs, rx, qrow, srow, (win + S) * kGemvWindow + 32 * r, K);
        __builtin_amdgcn_sched_barrier(0);
        wb.mul(acc, srow, win * kGemvWindow + 32 * r);
        win += S;
    }

    // Butterfly over the 16 lanes of each quad: every lane ends with its quad's column sums.
#pragma unroll
    for (int m = 0; m < MR; m++)
#pragma unroll
        for (int j = 0; j < C; j++) {
            float v = acc[m][j];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            acc[m][j] = v;
        }

    const float gs = *a.gscale;
    const int col0 = nfirst + q * C;
    if (S == 1) {
        if (r == 0) {
#pragma unroll
            for (int m = 0; m < MR; m++)
#pragma unroll
                for (int j = 0; j < C; j++)
                    if (m < a.M && col0 + j < N)
                        a.Y[(size_t)m * N + col0 + j] = acc[m][j] * gs;
        }
        return;
    }
    if (r == 0) {
#pragma unroll
        for (int m = 0; m < MR; m++)
#pragma unroll
            for (int j = 0; j < C; j++)
                red[wave][m][q * C + j] = acc[m][j];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < MR * 4 * C; idx += kWave * S) {
        const int m = idx / (4 * C);
        const int c = idx % (4 * C);
        const int n = nfirst + c;
        if (m < a.M && n < N) {
            float sum = red[0][m][c];
#pragma unroll
            for (int w = 1; w < S; w++)
                sum += red[w][m][c];
            a.Y[(size_t)m * N + n] = sum * gs;
        }
    }
}

}  // namespace nvfp4

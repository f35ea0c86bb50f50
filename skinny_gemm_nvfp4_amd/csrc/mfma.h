// mfma.h -- NVFP4 x bf16 kernel on the gfx950 matrix cores, for M of 16 and more.
//
// Speculative verification multiplies the same weights by 1 + k drafted tokens of one request
// (M = 16) or of eight requests verified together (M = 128) ("SparkInfer" README, speculative
// decoding sections), so the rows of X form real 16-row MFMA tiles.
//
// Work split
//   * A workgroup owns 16 MT rows (blockIdx.y) x 16 NT columns (blockIdx.x) and S wavefronts,
//     wave w taking the 128-wide k windows w, w + S, ... (split-K inside the workgroup).
//   * Lane l = 16 q + r holds, per window and column tile t, the 32 codes of column
//     n0 + 16 t + r at k = kw + 32 q .. kw + 32 q + 31 (one 16-byte load) and their two scales.
//   * v_mfma_f32_16x16x32_bf16 sums over 32 k-slots; slot 8 q + j of step d (d = 0..3) is the
//     physical k = kw + 32 q + 8 d + j for every column, so word d of the lane's codes is its B
//     fragment for step d and X row m0 + 16 i + r at the same k is its A fragment. The sum over k
//     does not depend on the order of the slots, so this is the plain product.
//   * B is decoded to bf16 as e2m1 * s (exact: at most 6 significant bits) once and reused for the
//     MT row tiles; A is loaded once per step and reused for the NT column tiles.
//   * Two register sets alternate: every load of the next window (weights and X) is in flight
//     while the current window is multiplied. Loads retire in issue order, so waiting for the
//     current window never waits for the next one.
//   * The S partial tiles are summed through LDS in wave order; g is applied once.
#pragma once

#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kMfmaWindow = 128;

template <int MT, int NT, bool NARROW>
struct MfmaWindow {
    Chunk c[NT];          // the lane's chunk of column 16 t + r of each column tile t
    u32x4_t x[4][MT];     // A fragments: X row 16 i + r at k = kc + 8 d

    // Issues every load of the window whose lane k range starts at kc.
    __device__ __forceinline__ void load(rsrc_t rq, rsrc_t rs, rsrc_t rx,
                                         const uint32_t (&qrow)[NT], const uint32_t (&srow)[NT],
                                         const uint32_t (&xrow)[MT], int kc, int K)
    {
#pragma unroll
        for (int t = 0; t < NT; t++)
            c[t] = load_chunk<NARROW>(rq, rs, qrow[t], srow[t], kc, K);
#pragma unroll
        for (int d = 0; d < 4; d++)
#pragma unroll
            for (int i = 0; i < MT; i++)
                x[d][i] = load_x8(rx, xrow[i] + (uint32_t)(kc + 8 * d) * 2u, kc + 8 * d, K);
    }

    __device__ __forceinline__ void mul(f32x4_t (&acc)[MT][NT], const uint32_t (&srow)[NT],
                                        int kc) const
    {
        float s0[NT], s1[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const uint32_t sc = scale_pair<NARROW>(c[t].scale, srow[t], kc);
            s0[t] = e4m3_to_f32<0>(sc);
            s1[t] = e4m3_to_f32<1>(sc);
        }
#pragma unroll
        for (int d = 0; d < 4; d++)
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const bf16x8_t b = decode8_scaled(c[t].code[d], d < 2 ? s0[t] : s1[t]);
#pragma unroll
                for (int i = 0; i < MT; i++)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x[d][i]), b,
                                                                        acc[i][t], 0, 0, 0);
            }
    }
};

template <int MT, int NT, int S, bool NARROW>
__global__ __launch_bounds__(kWave *S) void mfma_kernel(GemmArgs a)
{
    typedef MfmaWindow<MT, NT, NARROW> Win;
    // Split-K partials, [S][MT * NT][4][64]; a single element when there is nothing to reduce.
    __shared__ float red[S > 1 ? S * MT * NT * 4 * kWave : 1];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int n0 = blockIdx.x * (16 * NT);
    const int m0 = blockIdx.y * (16 * MT);

    // This workgroup's rows of Wq / Ws and of X.
    const int nrows = min(16 * NT, N - n0);
    const int mrows = min(16 * MT, a.M - m0);
    const rsrc_t rq = make_rsrc(a.Wq + (size_t)n0 * (size_t)(K / 2),
                                (uint32_t)nrows * (uint32_t)(K / 2));
    uint32_t sbias;
    const rsrc_t rs = scale_rsrc(a.Ws, (size_t)n0, nrows, K, &sbias);
    const rsrc_t rx = make_rsrc(a.X + (size_t)m0 * (size_t)K, (uint32_t)mrows * (uint32_t)K * 2u);
    uint32_t qrow[NT], srow[NT], xrow[MT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        qrow[t] = (uint32_t)(16 * t + r) * (uint32_t)(K / 2);
        srow[t] = sbias + (uint32_t)(16 * t + r) * (uint32_t)(K / 16);
    }
#pragma unroll
    for (int i = 0; i < MT; i++)
        xrow[i] = (uint32_t)(16 * i + r) * (uint32_t)K * 2u;

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int t = 0; t < NT; t++)
            acc[i][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int nwin = (K + kMfmaWindow - 1) / kMfmaWindow;
    Win wa, wb;
    int win = wave;
    wa.load(rq, rs, rx, qrow, srow, xrow, win * kMfmaWindow + 32 * q, K);
    while (win < nwin) {
        wb.load(rq, rs, rx, qrow, srow, xrow, (win + S) * kMfmaWindow + 32 * q, K);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
        wa.mul(acc, srow, win * kMfmaWindow + 32 * q);
        win += S;
        if (win >= nwin)
            break;
        wa.load(rq, rs, rx, qrow, srow, xrow, (win + S) * kMfmaWindow + 32 * q, K);
        __builtin_amdgcn_sched_barrier(0);
        wb.mul(acc, srow, win * kMfmaWindow + 32 * q);
        win += S;
    }

    // acc[i][t][e] is Y[m0 + 16 i + 4 q + e][n0 + 16 t + r] before the tensor scale.
    const float gs = *a.gscale;
    if (S == 1) {
#pragma unroll
        for (int i = 0; i < MT; i++)
#pragma unroll
            for (int t = 0; t < NT; t++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int m = 16 * i + 4 * q + e;
                    if (m < mrows && 16 * t + r < nrows)
                        a.Y[(size_t)(m0 + m) * N + n0 + 16 * t + r] = acc[i][t][e] * gs;
                }
        return;
    }
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                red[((wave * MT * NT + i * NT + t) * 4 + e) * kWave + lane] = acc[i][t][e];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * NT * 4 * kWave; idx += kWave * S) {
        const int tile = idx / (4 * kWave);
        const int e = (idx / kWave) % 4;
        const int ln = idx % kWave;
        const int m = 16 * (tile / NT) + 4 * (ln >> 4) + e;
        const int n = 16 * (tile % NT) + (ln & 15);
        if (m < mrows && n < nrows) {
            float sum = red[(tile * 4 + e) * kWave + ln];
#pragma unroll
            for (int w = 1; w < S; w++)
                sum += red[((w * MT * NT + tile) * 4 + e) * kWave + ln];
            a.Y[(size_t)(m0 + m) * N + n0 + n] = sum * gs;
        }
    }
}

}  // namespace nvfp4

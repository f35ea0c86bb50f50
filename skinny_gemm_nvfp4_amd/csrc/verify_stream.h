// verify_stream.h -- persistent NVFP4 x bf16 matrix-core kernel for one 16-row block of X.
//
// Speculative verification of one request runs the target's projections on 1 + 15 drafted
// tokens at once ("SparkInfer" README, speculative decoding sections), so X has 16 rows: one
// v_mfma_f32_16x16x32_bf16 row tile. The kernel is bound by the weight stream, like decode.
//
// Work split
//   * One workgroup of W wavefronts per compute unit; workgroup b owns the columns
//     [b N / G, (b + 1) N / G) (equal weight bytes per compute unit) and one 16-row block of X
//     (blockIdx.y). Its columns form T tiles of 16; the tiles are taken TC at a time.
//   * K is cut into windows of 128; wavefront w owns the windows w, w + W, ... and, for those
//     windows, every tile of the chunk. It loads the window's X fragments once (16 rows x 128 k)
//     and reuses them for the TC tiles, so X is read once per compute unit in total.
//   * MFMA k-slot 8 q + e of step d (d = 0..3) is the physical k = kw + 32 d + 8 q + e for every
//     row and column: lane l = 16 q + r then reads X row r at kw + 32 d + 8 q, and the four
//     q-lanes of a row read 64 contiguous bytes. For the weights, lane (r, q) loads the 16 code
//     bytes of column r at k = kw + 32 q (the q-lanes of a row again read 64 contiguous bytes),
//     and a 4 x 4 transpose across the four lanes of the row (v_permlane32_swap, then
//     v_permlane16_swap) hands each lane the codes of its slots. The block scale of slot
//     8 q + e at step d is byte 2 d + q / 2 of the window's 8 scale bytes of the column.
//   * B = e2m1 * s decoded to bf16 (exact); the sum over k does not depend on the slot order, so
//     this is the plain product.
//   * Every load of the next window is in flight while the current one is multiplied. The weight
//     loads use the normal cache policy: a wavefront reads 64 of the 128 bytes of a line and the
//     other half belongs to another wavefront's window, which then hits in L2 instead of being
//     fetched again.
//   * The W partial tiles are summed through LDS in wavefront order and scaled by g once.
//     Results are reproducible.
// Requires K % 128 == 0 (the 8 scale bytes of a window are then one aligned 8-byte word).
#pragma once

#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kVerifyWindow = 128;

// LDS bytes of verify_stream_kernel<TC, W>: one 16 x 16 fp32 partial per wavefront and tile.
constexpr int verify_lds_bytes(int tc, int w)
{
    return w * tc * 4 * kWave * 4;
}

template <int TC>
struct VerifyWindow {
    u32x4_t x[4];      // A fragments of steps d = 0..3
    u32x4_t c[TC];     // the lane's 16 code bytes of column r of each tile (k = kw + 32 q)
    u32x2_t s[TC];     // the window's 8 scale bytes of column r of each tile

    __device__ __forceinline__ void load(rsrc_t rq, rsrc_t rs, rsrc_t rx, uint32_t vx,
                                         uint32_t vq, uint32_t vs, uint32_t tq, uint32_t ts,
                                         int w, bool live)
    {
#pragma unroll
        for (int d = 0; d < 4; d++)
            x[d] = __builtin_amdgcn_raw_buffer_load_b128(
                rx, off_if(live, vx + (uint32_t)(w * kVerifyWindow + 32 * d) * 2u), 0,
                kAuxNormal);
#pragma unroll
        for (int t = 0; t < TC; t++) {
            c[t] = __builtin_amdgcn_raw_buffer_load_b128(
                rq, off_if(live, vq + (uint32_t)t * tq + (uint32_t)w * 64u), 0, kAuxNormal);
            s[t] = __builtin_amdgcn_raw_buffer_load_b64(
                rs, off_if(live, vs + (uint32_t)t * ts + (uint32_t)w * 8u), 0, kAuxNormal);
        }
    }

    __device__ __forceinline__ void mul(f32x4_t (&acc)[TC], int nt, uint32_t qshift) const
    {
#pragma unroll
        for (int t = 0; t < TC; t++) {
            if (t < nt) {
                // 4 x 4 transpose across the lanes (r, 0..3): afterwards word d is the codes of
                // k = kw + 32 d + 8 q .. + 7, the B fragment of step d.
                uint32_t w0 = c[t][0], w1 = c[t][1], w2 = c[t][2], w3 = c[t][3];
                auto p = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
                w0 = p[0];
                w2 = p[1];
                p = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
                w1 = p[0];
                w3 = p[1];
                p = __builtin_amdgcn_permlane16_swap(w0, w1, false, false);
                w0 = p[0];
                w1 = p[1];
                p = __builtin_amdgcn_permlane16_swap(w2, w3, false, false);
                w2 = p[0];
                w3 = p[1];
                // Scale byte of step d: 2 d + q / 2 of the window's 8 bytes.
                const uint32_t lo = s[t][0] >> qshift;  // steps 0 (byte 0) and 1 (byte 2)
                const uint32_t hi = s[t][1] >> qshift;  // steps 2 and 3
                const uint32_t code[4] = {w0, w1, w2, w3};
                const float sc[4] = {e4m3_to_f32<0>(lo), e4m3_to_f32<2>(lo), e4m3_to_f32<0>(hi),
                                     e4m3_to_f32<2>(hi)};
#pragma unroll
                for (int d = 0; d < 4; d++)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(x[d]), decode8_scaled(code[d], sc[d]), acc[t], 0, 0, 0);
            }
        }
    }
};

template <int TC, int W>
__global__ __launch_bounds__(kWave *W) void verify_stream_kernel(GemmArgs a)
{
    extern __shared__ __align__(16) float red[];  // [W][TC][4][64]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int G = gridDim.x;
    const int c0 = (int)(((long long)blockIdx.x * N) / G);
    const int ncols = (int)(((long long)(blockIdx.x + 1) * N) / G) - c0;
    const int T = (ncols + 15) / 16;
    const int m0 = blockIdx.y * 16;
    const int mrows = min(16, a.M - m0);
    const int nwin = K / kVerifyWindow;

    const rsrc_t rq = make_rsrc(a.Wq + (size_t)c0 * (size_t)(K / 2),
                                (uint32_t)ncols * (uint32_t)(K / 2));
    uint32_t sbias;  // zero: K % 128 == 0 keeps the scale rows 8-byte aligned
    const rsrc_t rs = scale_rsrc(a.Ws, (size_t)c0, ncols, K, &sbias);
    const rsrc_t rx = make_rsrc(a.X + (size_t)m0 * (size_t)K, (uint32_t)mrows * (uint32_t)K * 2u);
    const uint32_t vx = ((uint32_t)r * (uint32_t)K + 8u * (uint32_t)q) * 2u;
    const uint32_t tq = 16u * (uint32_t)(K / 2);   // bytes per tile of codes
    const uint32_t ts = 16u * (uint32_t)(K / 16);  // bytes per tile of scales
    const uint32_t qshift = 8u * (uint32_t)(q >> 1);
    const float g = *a.gscale;

    for (int tc0 = 0; tc0 < T; tc0 += TC) {
        const int nt = min(TC, T - tc0);
        const uint32_t vq = (uint32_t)(16 * tc0 + r) * (uint32_t)(K / 2) + 16u * (uint32_t)q;
        const uint32_t vs = sbias + (uint32_t)(16 * tc0 + r) * (uint32_t)(K / 16);
        f32x4_t acc[TC];
#pragma unroll
        for (int t = 0; t < TC; t++)
            acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

        VerifyWindow<TC> wa, wb;
        int w = wave;
        wa.load(rq, rs, rx, vx, vq, vs, tq, ts, w, w < nwin);
        while (w < nwin) {
            wb.load(rq, rs, rx, vx, vq, vs, tq, ts, w + W, w + W < nwin);
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
            wa.mul(acc, nt, qshift);
            w += W;
            if (w >= nwin)
                break;
            wa.load(rq, rs, rx, vx, vq, vs, tq, ts, w + W, w + W < nwin);
            __builtin_amdgcn_sched_barrier(0);
            wb.mul(acc, nt, qshift);
            w += W;
        }

        // acc[t][e] is the partial Y[m0 + 4 q + e][c0 + 16 (tc0 + t) + r] of this wavefront.
#pragma unroll
        for (int t = 0; t < TC; t++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                red[((wave * TC + t) * 4 + e) * kWave + lane] = acc[t][e];
        __syncthreads();
        for (int idx = threadIdx.x; idx < nt * 4 * kWave; idx += kWave * W) {
            const int t = idx / (4 * kWave);
            const int e = (idx / kWave) % 4;
            const int ln = idx % kWave;
            const int row = 4 * (ln >> 4) + e;
            const int col = 16 * (tc0 + t) + (ln & 15);
            if (row < mrows && col < ncols) {
                float sum = red[(t * 4 + e) * kWave + ln];
                for (int v = 1; v < W; v++)
                    sum += red[((v * TC + t) * 4 + e) * kWave + ln];
                a.Y[(size_t)(m0 + row) * N + c0 + col] = sum * g;
            }
        }
        __syncthreads();  // red is reused by the next chunk
    }
}

}  // namespace nvfp4

// mfma_batch.h -- persistent NVFP4 x bf16 matrix-core kernel for up to 128 rows of X at once.
//
// Eight requests verifying 16 tokens each put 128 rows through every projection ("SparkInfer"
// README, speculative decoding sections); at that size the bf16 MFMA work, not the weight stream,
// bounds the kernel. Every weight is therefore decoded once per workgroup and multiplied against
// all row blocks of X while it sits in registers.
//
// Work split
//   * One workgroup per compute unit and slab of up to 128 rows (blockIdx.y); workgroup b owns
//     the 4-column groups [b NG / G, (b + 1) NG / G), i.e. T tiles of 16 columns (4 groups each).
//   * TW wavefronts, one per SIMD: wavefront w takes the tiles t = w + TW j (at most TCW of them
//     per pass), for every 128-k window.
//   * Every global load writes LDS directly (buffer_load ... lds), so nothing waits in registers:
//       - X: all rows of a window go to one slot of a ring of P windows shared by the workgroup.
//         Rows are 256 bytes; the 16-byte piece kp of row m sits at slot kp ^ (m & 7), so the
//         A-fragment reads (lane (r, q): row 16 rb + r, k = 32 q + 8 d) hit distinct banks.
//       - Weights: a ring of P windows per wavefront: the codes of tile j land lane-major (lane
//         l = 16 q + r: 16 bytes of column r, chunk q of the window, whole cache lines across
//         the wavefront), then the words holding the lanes' scale pairs.
//     Loads retire in issue order, so X and weights travel in one stream, P - 1 windows ahead:
//     every iteration issues the same number of loads (ranges past the end read zeros), window
//     it has landed at the fixed wait vmcnt((P - 2) * loads per iteration), and one barrier per
//     iteration both publishes X and frees the ring slots of the previous window.
//   * The decoded B fragments of a tile are reused for all row blocks (MB <= 8
//     v_mfma_f32_16x16x32_bf16 per fragment); Y = acc * g. Results are reproducible.
#pragma once

#include "device.h"
#include "launch.h"
#include "mfma_stream.h"

namespace nvfp4 {

constexpr int kBatchMaxBlocks = 8;                          // 16-row blocks: M <= 128
constexpr int kBatchRowBytes = 256;                         // one 128-k row of bf16
constexpr int kBatchXWinBytes = 16 * kBatchMaxBlocks * kBatchRowBytes;   // 32 KB per window
constexpr int kBatchTileBytes = kWave * 16 + kWave * 4;     // codes + scale words of a tile

// Loads per wavefront and iteration: X (1 KB each, the window split over TW wavefronts), then
// codes and scale words of TCW tiles.
constexpr int batch_x_loads(int tw)
{
    return (kBatchXWinBytes / 1024) / tw;
}
constexpr int batch_loads(int tcw, int tw)
{
    return batch_x_loads(tw) + 2 * tcw;
}

// LDS bytes of mfma_batch_kernel<TCW, TW, P>: the X ring, then the weight rings.
constexpr int mfma_batch_lds_bytes(int tcw, int tw, int p)
{
    return p * kBatchXWinBytes + tw * p * tcw * kBatchTileBytes;
}

// One window: decode the TCW tiles' B fragments step by step and multiply them against the MB
// row blocks of X in LDS. FULL: all 8 row blocks and all TCW tiles are live, so the A fragments
// of a step are read together and no guard sits between the MFMAs.
template <bool FULL, int TCW>
__device__ __forceinline__ void mul_window(f32x4_t (&acc)[kBatchMaxBlocks][TCW],
                                           const uint8_t *xb, const u32x4_t (&c)[TCW],
                                           const uint32_t (&s)[TCW], int MB, int nt, int r, int q,
                                           uint32_t sshift)
{
#pragma unroll
    for (int d = 0; d < 4; d++) {
        bf16x8_t bfrag[TCW];
#pragma unroll
        for (int j = 0; j < TCW; j++) {
            const uint32_t sw = s[j] >> sshift;
            const float sc = (d < 2) ? e4m3_to_f32<0>(sw) : e4m3_to_f32<1>(sw);
            bfrag[j] = decode8_scaled(c[j][d], sc);
        }
        const int piece = 4 * q + d;
        u32x4_t av[kBatchMaxBlocks];
#pragma unroll
        for (int b = 0; b < kBatchMaxBlocks; b++) {
            const int row = 16 * b + r;
            if (FULL || b < MB)
                av[b] = *reinterpret_cast<const u32x4_t *>(xb + row * kBatchRowBytes +
                                                           16 * (piece ^ (row & 7)));
        }
#pragma unroll
        for (int b = 0; b < kBatchMaxBlocks; b++)
#pragma unroll
            for (int j = 0; j < TCW; j++)
                if (FULL || (b < MB && j < nt))
                    acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(av[b]), bfrag[j], acc[b][j], 0, 0, 0);
    }
}

template <int TCW, int TW, int P>
__global__ __launch_bounds__(kWave *TW) void mfma_batch_kernel(GemmArgs a)
{
    constexpr int XL = batch_x_loads(TW);        // X loads per wavefront per iteration
    constexpr int LOADS = batch_loads(TCW, TW);  // all loads per wavefront per iteration
    static_assert(P >= 2 && (P - 2) * LOADS <= 63, "vmcnt counts at most 63 loads");
    static_assert(XL * TW * 1024 == kBatchXWinBytes, "X loads must tile the window");
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int m0 = blockIdx.y * 16 * kBatchMaxBlocks;   // row slab of this workgroup
    const int M = min(16 * kBatchMaxBlocks, a.M - m0);  // rows of the slab
    const int MB = (M + 15) / 16;
    const int CH = num_chunks(K);
    const int NG = num_groups(N);
    const int G = gridDim.x;
    const int g0 = (int)(((long long)blockIdx.x * NG) / G);
    const int ngroups = (int)(((long long)(blockIdx.x + 1) * NG) / G) - g0;
    const int c0 = kGroupCols * g0;
    const int ncols = min(N - c0, kGroupCols * ngroups);
    const int T = (ngroups + 3) / 4;
    const int nwin = (CH + 3) / 4;

    const uint32_t gq = (uint32_t)CH * kChunkCodeBytes;
    const uint32_t gs = (uint32_t)CH * kChunkScaleBytes;
    const rsrc_t rq = make_rsrc(a.Wq + (size_t)g0 * gq, (uint32_t)ngroups * gq);
    const rsrc_t rs = make_rsrc(a.Ws + (size_t)g0 * gs, (uint32_t)ngroups * gs);
    const rsrc_t rx = make_rsrc(a.X + (size_t)m0 * (size_t)K, (uint32_t)M * (uint32_t)K * 2u);
    const int gr = r >> 2;
    const uint32_t lq = (uint32_t)gr * gq + (uint32_t)q * kChunkCodeBytes + (uint32_t)(r & 3) * 16u;
    const uint32_t ls = (uint32_t)gr * gs + (uint32_t)q * kChunkScaleBytes + (uint32_t)(r & 2) * 2u;
    const uint32_t sshift = 16u * (uint32_t)(r & 1);
    const float g = *a.gscale;
    uint8_t *const ring = lds + P * kBatchXWinBytes + wave * (P * TCW * kBatchTileBytes);

    for (int tc0 = 0; tc0 < T; tc0 += TW * TCW) {
        // Tiles of this wavefront in this pass: tc0 + wave + TW j, j < nt.
        const int nt = max(0, min(TCW, (T - tc0 - wave + TW - 1) / TW));

        // X of window w into ring slot w % P: load p of this wavefront fills the 1 KB block
        // p * TW + wave of the slot, i.e. 4 rows.
        auto issue_x = [&](int w) {
            uint8_t *slotp = lds + (w % P) * kBatchXWinBytes;
#pragma unroll
            for (int p = 0; p < XL; p++) {
                const int blk = p * TW + wave;
                const int row = blk * 4 + (lane >> 4);
                const int kp = (lane & 15) ^ (row & 7);
                const int k = kMfmaWindow * w + 8 * kp;
                const bool v = w < nwin && row < M && k < K;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void *)(slotp + blk * 1024), 16,
                    off_if(v, ((uint32_t)row * (uint32_t)K + (uint32_t)k) * 2u), 0, 0,
                    kAuxNormal);
            }
        };
        // Weights of window w into this wavefront's ring slot w % P.
        auto issue_w = [&](int w) {
            const bool kv = w < nwin && 4 * w + q < CH;
            uint8_t *slotp = ring + (w % P) * (TCW * kBatchTileBytes);
#pragma unroll
            for (int j = 0; j < TCW; j++) {
                const int t = tc0 + wave + TW * j;
                const bool v = kv && j < nt && 4 * t + gr < ngroups;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rq, (__attribute__((address_space(3))) void *)(slotp + j * (kWave * 16)), 16,
                    off_if(v, lq + (uint32_t)t * (4u * gq) + (uint32_t)w * (4u * kChunkCodeBytes)),
                    0, 0, kAuxNormal);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs,
                    (__attribute__((address_space(3))) void *)(slotp + TCW * (kWave * 16) +
                                                               j * (kWave * 4)),
                    4, off_if(v, ls + (uint32_t)t * (4u * gs) + (uint32_t)w * (4u * kChunkScaleBytes)),
                    0, 0, kAuxNormal);
            }
        };

        f32x4_t acc[kBatchMaxBlocks][TCW];
#pragma unroll
        for (int b = 0; b < kBatchMaxBlocks; b++)
#pragma unroll
            for (int t = 0; t < TCW; t++)
                acc[b][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

        __syncthreads();   // the previous pass is done with every buffer
#pragma unroll
        for (int w = 0; w < P - 1; w++) {
            issue_x(w);
            issue_w(w);
        }
        for (int it = 0; it < nwin; it++) {
            // Window it has landed once only the P - 2 later windows' loads are pending; the
            // barrier then publishes its X and tells that every wavefront is done with window
            // it - 1, whose slots the loads of window it + P - 1 reuse. A plain s_barrier: a
            // fenced one would also wait for the loads still in flight.
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((P - 2) * LOADS) : "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            issue_x(it + P - 1);
            issue_w(it + P - 1);
            const uint8_t *slotp = ring + (it % P) * (TCW * kBatchTileBytes);
            u32x4_t c[TCW];
            uint32_t s[TCW];
#pragma unroll
            for (int j = 0; j < TCW; j++) {
                c[j] = *reinterpret_cast<const u32x4_t *>(slotp + j * (kWave * 16) + lane * 16);
                s[j] = *reinterpret_cast<const uint32_t *>(slotp + TCW * (kWave * 16) +
                                                           j * (kWave * 4) + lane * 4);
            }
            const uint8_t *xb = lds + (it % P) * kBatchXWinBytes;
            if (MB == kBatchMaxBlocks && nt == TCW)
                mul_window<true>(acc, xb, c, s, MB, nt, r, q, sshift);
            else
                mul_window<false>(acc, xb, c, s, MB, nt, r, q, sshift);
        }
        // Drain: the loads issued past the last window must land before LDS is reused.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
        for (int j = 0; j < TCW; j++) {
            const int colx = 16 * (tc0 + wave + TW * j) + r;
            if (j < nt && colx < ncols) {
#pragma unroll
                for (int b = 0; b < kBatchMaxBlocks; b++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int row = 16 * b + 4 * q + e;
                        if (row < M)
                            a.Y[(size_t)(m0 + row) * N + c0 + colx] = acc[b][j][e] * g;
                    }
            }
        }
    }
}

}  // namespace nvfp4

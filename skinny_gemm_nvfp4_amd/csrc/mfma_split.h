// mfma_split.h -- NVFP4 x bf16 matrix-core kernel for M >= 16 (speculative verification).
//
// Verification multiplies the same weights by the 1 + k drafted tokens of one request (M = 16)
// or of eight requests at once (M = 128) ("SparkInfer" README, speculative decoding sections).
//
// Work split
//   * A workgroup is 4 wavefronts. It owns 64 NTW consecutive columns (wave w: the NTW tiles of
//     16 columns starting at tile w NTW), 16 MT rows (blockIdx.z) and a range of 128-wide K
//     windows (split s = blockIdx.y of S).
//   * The four wavefronts step through the same windows together. The X tile of a window
//     (16 MT rows x 128 k) is staged once in LDS (double-buffered, one barrier per window) and
//     read by all four, so X costs no per-lane global loads.
//   * Lane l = 16 q + r holds, per window and tile, the 32 codes of column r at k = kw + 32 q
//     (one 16-byte load; the four q-lanes of a row read 64 contiguous bytes) and the two scale
//     bytes of those blocks (one 16-byte load per row covers two windows when K % 256 == 0).
//   * v_mfma_f32_16x16x32_bf16 sums over 32 k-slots; slot 8 q + e of step d is the physical
//     k = kw + 32 q + 8 d + e for every column, so word d of the lane's codes is its B fragment and
//     X row 16 i + r at the same k its A fragment. B = e2m1 * s in bf16 (exact), decoded once per
//     tile and reused for the MT row tiles; A is read once per step and reused for the NT tiles.
//   * The weights of the next window are in flight while the current one is multiplied.
//   * S == 1: the tile is scaled by g and stored. S > 1: each split writes its partial tile to a
//     workspace slot and bumps the tile's counter; the split that arrives last adds the S slots in
//     split order (= k order), scales by g, stores, and resets the counter to zero. Results are
//     therefore reproducible, and the workspace needs no clearing between calls.
#pragma once

#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kSplitWindow = 128;
constexpr int kSplitWaves = 4;
constexpr int kXRowBytes = kSplitWindow * 2 + 16;  // padded LDS row: 8 lanes hit 8 bank groups

// Dynamic LDS bytes of mfma_split_kernel<MT, ...>.
constexpr int split_lds_bytes(int mt)
{
    return 2 * 16 * mt * kXRowBytes;
}

// Workspace of the split-K reduction: `slots` floats and one counter per (column group, row
// block). Counters must be zero before the first call; every call leaves them zero.
struct SplitWork {
    float *slots;
    unsigned *counters;
};

// Registers of one pair of windows (256 k) for the lane's NTW tiles.
template <int NTW>
struct SplitPair {
    Chunk c[2][NTW];   // [window of the pair][tile]; the scale field is used when K % 256 != 0
    u32x4_t sc[NTW];   // K % 256 == 0: the row's 16 scale bytes of the two windows
};

template <int MT, int NTW, bool FAST, bool NARROW>
__global__ __launch_bounds__(kWave *kSplitWaves) void mfma_split_kernel(GemmArgs a, int S,
                                                                        SplitWork ws)
{
    // Two X buffers of 16 MT padded rows (dynamic LDS: split_lds_bytes(MT)).
    extern __shared__ __align__(16) uint8_t xs[];
    __shared__ unsigned arrive;
    constexpr int kXBuf = 16 * MT * kXRowBytes;
    constexpr int kThreads = kWave * kSplitWaves;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int n0 = blockIdx.x * (64 * NTW);
    const int m0 = blockIdx.z * (16 * MT);
    const int s = blockIdx.y;
    // Splits cut K at pairs of windows (FAST: K % 256 == 0, so every pair is whole).
    const int nwin = (K + kSplitWindow - 1) / kSplitWindow;
    const int npairs = (nwin + 1) / 2;
    const int pb = (int)(((long long)s * npairs) / S);
    const int pe = (int)(((long long)(s + 1) * npairs) / S);

    const int nrows = min(64 * NTW, N - n0);
    const int mrows = min(16 * MT, a.M - m0);
    const rsrc_t rq = make_rsrc(a.Wq + (size_t)n0 * (size_t)(K / 2),
                                (uint32_t)nrows * (uint32_t)(K / 2));
    uint32_t sbias;
    const rsrc_t rs = scale_rsrc(a.Ws, (size_t)n0, nrows, K, &sbias);
    const rsrc_t rx = make_rsrc(a.X + (size_t)m0 * (size_t)K, (uint32_t)mrows * (uint32_t)K * 2u);
    uint32_t qrow[NTW], srow[NTW];
#pragma unroll
    for (int j = 0; j < NTW; j++) {
        const uint32_t col = (uint32_t)(16 * (wave * NTW + j) + r);
        qrow[j] = col * (uint32_t)(K / 2);
        srow[j] = sbias + col * (uint32_t)(K / 16);
    }

    // X staging: thread t moves pieces t + 256 i (16 bytes each) of the 16 MT x 128 tile.
    auto load_x = [&](int w, u32x4_t (&v)[MT]) {
#pragma unroll
        for (int i = 0; i < MT; i++) {
            const int p = threadIdx.x + i * kThreads;
            const int k = w * kSplitWindow + 8 * (p & 15);
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(
                rx, off_if(k < K, ((uint32_t)(p >> 4) * (uint32_t)K + (uint32_t)k) * 2u), 0,
                kAuxNormal);
        }
    };
    auto store_x = [&](int buf, const u32x4_t (&v)[MT]) {
#pragma unroll
        for (int i = 0; i < MT; i++) {
            const int p = threadIdx.x + i * kThreads;
            *reinterpret_cast<u32x4_t *>(&xs[buf * kXBuf + (p >> 4) * kXRowBytes +
                                             16 * (p & 15)]) = v[i];
        }
    };
    auto load_pair = [&](int p, SplitPair<NTW> &sp) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int kc = (2 * p + h) * kSplitWindow + 32 * q;
#pragma unroll
            for (int j = 0; j < NTW; j++) {
                if (FAST) {
                    const u32x4_t c = __builtin_amdgcn_raw_buffer_load_b128(
                        rq, off_if(p < pe, qrow[j] + (uint32_t)kc / 2), 0, kAuxStream);
                    sp.c[h][j].code[0] = c[0];
                    sp.c[h][j].code[1] = c[1];
                    sp.c[h][j].code[2] = c[2];
                    sp.c[h][j].code[3] = c[3];
                } else {
                    sp.c[h][j] = load_chunk<NARROW>(rq, rs, qrow[j], srow[j], p < pe ? kc : K, K);
                }
            }
        }
        if (FAST) {
#pragma unroll
            for (int j = 0; j < NTW; j++)
                sp.sc[j] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, off_if(p < pe, srow[j] + (uint32_t)p * 16u), 0, kAuxStream);
        }
    };

    f32x4_t acc[MT][NTW];
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int j = 0; j < NTW; j++)
            acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Window h of the pair held in sp, X in LDS buffer h.
    auto mul = [&](const SplitPair<NTW> &sp, int h, int w) {
        float s0[NTW], s1[NTW];
#pragma unroll
        for (int j = 0; j < NTW; j++) {
            uint32_t pair;
            if (FAST) {
                // Byte 8 h + 2 q of the 16: dword 2 h + q / 2, half q % 2.
                const uint32_t word = (q >> 1) ? sp.sc[j][2 * h + 1] : sp.sc[j][2 * h];
                pair = word >> (16u * (uint32_t)(q & 1));
            } else {
                pair = scale_pair<NARROW>(sp.c[h][j].scale, srow[j], w * kSplitWindow + 32 * q);
            }
            s0[j] = e4m3_to_f32<0>(pair);
            s1[j] = e4m3_to_f32<1>(pair);
        }
        const uint8_t *xb = &xs[h * kXBuf + r * kXRowBytes + 64 * q];
#pragma unroll
        for (int d = 0; d < 4; d++) {
            bf16x8_t b[NTW];
#pragma unroll
            for (int j = 0; j < NTW; j++)
                b[j] = decode8_scaled(sp.c[h][j].code[d], d < 2 ? s0[j] : s1[j]);
#pragma unroll
            for (int i = 0; i < MT; i++) {
                const bf16x8_t x = as_bf16x8(
                    *reinterpret_cast<const u32x4_t *>(xb + i * 16 * kXRowBytes + 16 * d));
#pragma unroll
                for (int j = 0; j < NTW; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, b[j], acc[i][j], 0, 0,
                                                                        0);
            }
        }
    };

    SplitPair<NTW> cur, nxt;
    u32x4_t xv[MT];
    load_x(2 * pb, xv);
    load_pair(pb, cur);
    for (int p = pb; p < pe; p++) {
        // First window of the pair: its X into buffer 0, then start the next pair's weights
        // (two windows of arithmetic to arrive) and the second window's X.
        store_x(0, xv);
        load_pair(p + 1, nxt);
        load_x(2 * p + 1, xv);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        mul(cur, 0, 2 * p);
        // Second window: X into buffer 1, then the first X of the next pair.
        store_x(1, xv);
        load_x(2 * p + 2, xv);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        mul(cur, 1, 2 * p + 1);
        cur = nxt;
    }

    // acc[i][j][e] is the partial Y[m0 + 16 i + 4 q + e][n0 + 16 (wave NTW + j) + r].
    const float gs = *a.gscale;
    if (S == 1) {
#pragma unroll
        for (int i = 0; i < MT; i++)
#pragma unroll
            for (int j = 0; j < NTW; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int m = 16 * i + 4 * q + e;
                    const int n = 16 * (wave * NTW + j) + r;
                    if (m < mrows && n < nrows)
                        a.Y[(size_t)(m0 + m) * N + n0 + n] = acc[i][j][e] * gs;
                }
        return;
    }

    // Split-K: slot layout [group][split][i][j][e][256 threads].
    const size_t group = (size_t)blockIdx.z * gridDim.x + blockIdx.x;
    constexpr int kTileFloats = MT * NTW * 4 * kThreads;
    float *mine = ws.slots + (group * (size_t)S + (size_t)s) * kTileFloats;
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int j = 0; j < NTW; j++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                mine[((i * NTW + j) * 4 + e) * kThreads + threadIdx.x] = acc[i][j][e];
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        arrive = atomicAdd(&ws.counters[group], 1u);
    __syncthreads();
    if (arrive != (unsigned)(S - 1))
        return;
    __threadfence();
    const float *first = ws.slots + group * (size_t)S * kTileFloats;
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int j = 0; j < NTW; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int idx = ((i * NTW + j) * 4 + e) * kThreads + threadIdx.x;
                float sum = first[idx];
                for (int t = 1; t < S; t++)
                    sum += first[(size_t)t * kTileFloats + idx];
                const int m = 16 * i + 4 * q + e;
                const int n = 16 * (wave * NTW + j) + r;
                if (m < mrows && n < nrows)
                    a.Y[(size_t)(m0 + m) * N + n0 + n] = sum * gs;
            }
    if (threadIdx.x == 0)
        ws.counters[group] = 0u;
}

}  // namespace nvfp4

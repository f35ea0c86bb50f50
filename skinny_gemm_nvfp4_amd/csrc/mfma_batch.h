// mfma_batch.h -- persistent NVFP4 x bf16 matrix-core kernel for up to 128 rows of X at once.
//
// Eight requests verifying 16 tokens each put 128 rows through every projection ("SparkInfer"
// README, speculative decoding sections). At that size the bf16 MFMA work, not the weight stream,
// bounds the kernel, so every weight is decoded once per workgroup and multiplied against all
// row blocks of X while it sits in registers.
//
// Work split (one workgroup of 8 wavefronts per compute unit; workgroup b owns NG / G or
// NG / G + 1 consecutive 4-column groups (group_range), i.e. T tiles of 16 columns, for all of K
// and one slab of at most 16 MB rows of X; the tiles are taken PT = 4 TCW / KS at a time)
//   * K is cut into windows of 128 (4 chunks of 32). Every window passes through LDS once, in two
//     buffers, with one barrier per window:
//       - wavefronts 4 and 5 load X: rows 8 MB p .. 8 MB p + 8 MB - 1 of the window, as 16-byte
//         pieces, 1 to 3 windows ahead (fewer for more rows). Rows are 256 bytes in LDS; piece
//         kp of row m sits at slot kp ^ (m & 15), so the 16 rows of an A-fragment read hit 16
//         different slots.
//       - wavefronts 6 and 7 load the weights of the pass's tiles, kBatchWRing - 1 windows ahead:
//         lane l = 16 q + r of a tile takes the 16 code bytes of column r, chunk q (the 64 lanes
//         read four 256-byte pieces, i.e. whole cache lines) and the word that holds that
//         column's 2 scale bytes.
//     Each loader issues one kind of load, so the in-order completion of loads never makes one
//     stream wait for the other.
//   * Wavefronts 0..3 are the consumers (one per SIMD) and issue no global loads. Consumer
//     c = TS ks + ts takes tiles ts, ts + TS, ... of the pass (TS = 4 / KS) and, of each window,
//     the MFMA steps d = ks, ks + KS, ... Step d of lane (r, q) covers k = 32 q + 8 d .. + 7 of
//     the window: code dword d is its B fragment, scale byte d / 2 the block scale, and row
//     16 b + r of X at those k its A fragment of row block b (v_mfma_f32_16x16x32_bf16). Narrow
//     shapes (few tiles per workgroup) take KS = 2 or 4 so that all four matrix cores work.
//   * With KS = 1 a pass may end in NR remainder tiles (4 TCW + NR tiles): consumer c multiplies
//     MFMA step c of each remainder tile, so every consumer does the same work per window (a
//     workgroup of 9 tiles runs as 4 x 2 + 1 instead of 3, 2, 2, 2).
//   * Split K (gridDim.y = S > 1): workgroup (b, s) takes windows [s nwin / S, (s + 1) nwin / S)
//     and writes its unscaled partial sums to slice s of a workspace (a.Y, S x M x N floats);
//     batch_reduce_kernel adds the S slices in order and applies g. Narrow shapes (a few tiles
//     per compute unit) then read 1 / S of X per compute unit.
//   * B = e2m1 * s decoded to bf16 (exact). The KS partial sums of a tile (or the 4 of a
//     remainder tile) are added through LDS in a fixed order, then Y = sum * g. Results are
//     reproducible.
#pragma once

#include "argmax.h"
#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kBatchWindow = 128;
constexpr int kBatchMaxBlocks = 8;       // 16-row blocks: at most 128 rows per slab
constexpr int kBatchRowBytes = 256;      // one 128-k row of bf16 in LDS
constexpr int kBatchConsumers = 4;
constexpr int kBatchWaves = 8;
constexpr int kBatchTileBytes = kWave * 16;   // codes of one tile and window
constexpr int kBatchWRing = 5;           // weight windows held by a weight loader

// NR > 0 (KS = 1 only): NR remainder tiles per pass after the TS TCW full ones; consumer c takes
// MFMA step c of each of them, so that a pass of 4 TCW + NR tiles is balanced over the consumers.
template <int TCW, int MB, int KS, int NR = 0>
struct BatchShape {
    static_assert(NR == 0 || KS == 1, "remainder tiles need KS = 1");
    static constexpr int TS = kBatchConsumers / KS;   // tile lanes
    static constexpr int PT = TS * TCW + NR;          // tiles per pass
    static constexpr int NACC = TCW + NR;             // accumulator tiles per consumer
    static constexpr int NWP = (PT + 1) / 2;          // tiles per weight loader
    static constexpr int NXP = 2 * MB;                // X pieces per lane of an X loader
    static constexpr int XRING = MB >= 8 ? 2 : MB >= 4 ? 3 : 4;   // X windows per X loader
    static constexpr int NSTEP = 4 / KS;              // MFMA steps per window and consumer
    static constexpr int XBUF = 16 * MB * kBatchRowBytes;
    static constexpr int WBUF = PT * (kBatchTileBytes + kWave * 4);
    static constexpr int MAIN = 2 * XBUF + 2 * WBUF;
    static constexpr int RED_KS = (KS - 1) * TS * TCW * MB * kWave * 16;
    static constexpr int RED_NR = kBatchConsumers * NR * MB * kWave * 16;
    static constexpr int RED = RED_KS > RED_NR ? RED_KS : RED_NR;
    static constexpr int LDS = MAIN > RED ? MAIN : RED;
};

// Floats between the split-K slices of the workspace: M * N rounded up to 4 (16-byte slices).
__host__ __device__ inline size_t batch_slice_stride(int M, int N)
{
    return ((size_t)M * (size_t)N + 3) & ~(size_t)3;
}

// Byte position / 4 of code dword d inside a tile's 16 bytes in LDS: the order is d = 0, 2, 1, 3,
// so that the dwords of steps ks and ks + 2 (KS = 2) are adjacent.
__host__ __device__ constexpr int batch_dword_pos(int d)
{
    return d == 0 ? 0 : d == 1 ? 2 : d == 2 ? 1 : 3;
}

// Barrier for LDS hand-over. It waits for the wavefront's own LDS traffic only, not for its
// global loads in flight (a fenced __syncthreads would wait for those too).
__device__ __forceinline__ void batch_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The A fragments of step d for all MB row blocks.
template <int MB>
__device__ __forceinline__ void batch_read_a(u32x4_t (&av)[MB], const uint8_t *xb, int r, int q,
                                             int d)
{
    const int piece = 4 * q + d;
#pragma unroll
    for (int b = 0; b < MB; b++) {
        const int row = 16 * b + r;
        av[b] = *reinterpret_cast<const u32x4_t *>(xb + row * kBatchRowBytes +
                                                   16 * (piece ^ (row & 15)));
    }
}

// B fragments of step d (code dword i of each live tile) decoded to bf16 with their block scale.
template <int NT>
__device__ __forceinline__ void batch_decode(bf16x8_t (&bf)[NT], const uint32_t (&code)[NT],
                                             const uint32_t (&sw)[NT], int d)
{
#pragma unroll
    for (int j = 0; j < NT; j++) {
        // Steps 0 and 1 lie in the chunk's first block of 16 k, steps 2 and 3 in the second.
        const float sc = (d < 2) ? e4m3_to_f32<0>(sw[j]) : e4m3_to_f32<1>(sw[j]);
        bf[j] = decode8_scaled(code[j], sc);
    }
}

// One window of one consumer with NT live tiles: NSTEP steps of MB x NT MFMAs. The A fragments
// and the decoded B fragments of step i + 1 are prepared while step i multiplies: the
// scheduling groups interleave one MFMA with a few VALU instructions of the next decode (the
// matrix core runs an MFMA for 16 cycles, during which the wavefront can issue VALU work).
template <int TCW, int MB, int KS, int NT, int NR>
__device__ __forceinline__ void batch_window(f32x4_t (&acc)[MB][TCW + NR], const uint8_t *xb,
                                             const uint8_t *wb, int ts, int ks, int lane, int r,
                                             int q, uint32_t sshift)
{
    using S = BatchShape<TCW, MB, KS, NR>;
    // Code dword of step i of live tile j (read from LDS one step ahead) and its scale word.
    auto code_at = [&](int i, int j) -> uint32_t {
        const int d = ks + KS * i;
        return *reinterpret_cast<const uint32_t *>(wb + (ts + S::TS * j) * kBatchTileBytes +
                                                   lane * 16 + 4 * batch_dword_pos(d));
    };
    uint32_t code[2][NT];
    uint32_t sw[NT];
#pragma unroll
    for (int j = 0; j < NT; j++) {
        code[0][j] = code_at(0, j);
        sw[j] = *reinterpret_cast<const uint32_t *>(wb + S::PT * kBatchTileBytes +
                                                    (ts + S::TS * j) * (kWave * 4) + lane * 4) >>
                sshift;
    }
    // Remainder tiles: this consumer (ts, with TS = 4) multiplies their step ts only.
    bf16x8_t bfr[NR > 0 ? NR : 1];
    if constexpr (NR > 0) {
#pragma unroll
        for (int rr = 0; rr < NR; rr++) {
            const int p = S::TS * TCW + rr;
            const uint32_t c = *reinterpret_cast<const uint32_t *>(
                wb + p * kBatchTileBytes + lane * 16 +
                4 * (ts == 0 ? 0 : ts == 1 ? 2 : ts == 2 ? 1 : 3));
            const uint32_t w = *reinterpret_cast<const uint32_t *>(
                                   wb + S::PT * kBatchTileBytes + p * (kWave * 4) + lane * 4) >>
                               sshift;
            bfr[rr] = decode8_scaled(c, ts < 2 ? e4m3_to_f32<0>(w) : e4m3_to_f32<1>(w));
        }
    }
    // av[b] is refilled with step i + 1's fragment right after its last MFMA of step i.
    u32x4_t av[MB];
    u32x4_t ar[NR > 0 ? MB : 1];   // A fragments of step ts for the remainder tiles
    bf16x8_t bf[2][NT];
    batch_read_a<MB>(av, xb, r, q, ks);
    batch_decode<NT>(bf[0], code[0], sw, ks);
    if (S::NSTEP > 1) {
#pragma unroll
        for (int j = 0; j < NT; j++)
            code[1][j] = code_at(1, j);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kValuPerMfma = (20 + MB - 1) / MB;   // decode of one tile: about 20 VALU
#pragma unroll
    for (int i = 0; i < S::NSTEP; i++) {
        const int d = ks + KS * i;
        const bool more = i + 1 < S::NSTEP;
        if (more) {
            batch_decode<NT>(bf[(i + 1) & 1], code[(i + 1) & 1], sw, d + KS);
            if (i + 2 < S::NSTEP) {
#pragma unroll
                for (int j = 0; j < NT; j++)
                    code[i & 1][j] = code_at(i + 2, j);
            }
        }
        const int piece = 4 * q + d + KS;
        if constexpr (NR > 0) {
            if (i == S::NSTEP - 1)
                batch_read_a<MB>(ar, xb, r, q, ts);   // step ts, for the remainder tiles
        }
#pragma unroll
        for (int b = 0; b < MB; b++) {
#pragma unroll
            for (int j = 0; j < NT; j++)
                acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(av[b]), bf[i & 1][j], acc[b][j], 0, 0, 0);
            if (more) {
                const int row = 16 * b + r;
                av[b] = *reinterpret_cast<const u32x4_t *>(xb + row * kBatchRowBytes +
                                                           16 * (piece ^ (row & 15)));
            }
        }
        if (more) {
#pragma unroll
            for (int b = 0; b < MB; b++) {
#pragma unroll
                for (int j = 0; j < NT; j++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // next decode
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // next A of block b
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NR > 0) {
        // Remainder tiles: MFMA step ts of each, with the fragments read during the last step.
#pragma unroll
        for (int b = 0; b < MB; b++)
#pragma unroll
            for (int rr = 0; rr < NR; rr++)
                acc[b][TCW + rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(ar[b]), bfr[rr], acc[b][TCW + rr], 0, 0, 0);
    }
}

// All windows of one pass for a consumer with NT live tiles (NT = 0: barriers only).
template <int TCW, int MB, int KS, int NT, int NR>
__device__ __forceinline__ void batch_consume(f32x4_t (&acc)[MB][TCW + NR], const uint8_t *lds,
                                              int nwin, int ts, int ks, int lane, int r, int q,
                                              uint32_t sshift)
{
    using S = BatchShape<TCW, MB, KS, NR>;
    for (int it = 0; it < nwin; it++) {
        batch_barrier();   // window it is in buffer it & 1
        const int buf = it & 1;
        if constexpr (NT > 0)
            batch_window<TCW, MB, KS, NT, NR>(acc, lds + buf * S::XBUF,
                                          lds + 2 * S::XBUF + buf * S::WBUF, ts, ks, lane, r, q,
                                          sshift);
    }
}

// Loader pipeline shared by both kinds of loader: D - 1 windows in flight; window it is stored to
// buffer it & 1 and published by the barrier of window it.
template <int D, typename Win, typename Load, typename Store>
__device__ __forceinline__ void batch_produce(int nwin, Load &load, Store &store)
{
    Win ring[D];
#pragma unroll
    for (int u = 0; u < D - 1; u++)
        load(u, ring[u]);
    for (int it0 = 0; it0 < nwin; it0 += D) {
#pragma unroll
        for (int u = 0; u < D; u++) {
            const int it = it0 + u;
            if (it < nwin) {
                load(it + D - 1, ring[(u + D - 1) % D]);
                __builtin_amdgcn_sched_barrier(0);
                store(it & 1, ring[u]);
                batch_barrier();   // window it published
            }
        }
    }
}

template <int NWP>
struct BatchWWin {
    u32x4_t c[NWP];
    uint32_t s[NWP];
};

template <int NXP>
struct BatchXWin {
    u32x4_t x[NXP];
};

// ARGMAX: instead of storing Y, fold it into one argmax key per row and consumer (argmax.h),
// slot 4 blockIdx.x + consumer of a.keys; only for unsplit K (gridDim.y == 1).
template <int TCW, int MB, int KS, int NR = 0, bool ARGMAX = false>
__global__ __launch_bounds__(kWave *kBatchWaves) void mfma_batch_kernel(GemmArgs a)
{
    using S = BatchShape<TCW, MB, KS, NR>;
    constexpr int kExtraBarriers = (KS > 1 || NR > 0) ? 2 : 0;   // partial sums via LDS
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int M = a.M;   // rows of this slab: 16 (MB - 1) < M <= 16 MB
    const int CH = num_chunks(K);
    const int NG = num_groups(N);
    int g0, ngroups;
    group_range(NG, (int)gridDim.x, (int)blockIdx.x, &g0, &ngroups);
    const int c0 = kGroupCols * g0;
    const int ncols = min(N - c0, kGroupCols * ngroups);
    const int T = (ngroups + 3) / 4;
    const int nwin_all = (K + kBatchWindow - 1) / kBatchWindow;
    const int nslice = gridDim.y;   // K slices
    // nwin_all <= 2^15 and nslice <= 8: 32-bit products and divisions suffice.
    const int w0 = (int)(((uint32_t)blockIdx.y * (uint32_t)nwin_all) / (uint32_t)nslice);
    const int nwin =
        (int)(((uint32_t)(blockIdx.y + 1) * (uint32_t)nwin_all) / (uint32_t)nslice) - w0;

    // Each role runs its own loop over the passes (tiles tc0 .. tc0 + PT - 1), so that what it
    // precomputes stays inside its branch; all roles meet the same barriers in the same order.
    if (wave >= kBatchConsumers + 2) {
        // ---------------- weight loader: pass tiles p = wl, wl + 2, ... ----------------
        const int wl = wave - (kBatchConsumers + 2);
        const uint32_t gq = (uint32_t)CH * kChunkCodeBytes;
        const uint32_t gs = (uint32_t)CH * kChunkScaleBytes;
        const rsrc_t rq = make_rsrc(a.Wq + (size_t)g0 * gq, (uint32_t)ngroups * gq);
        const rsrc_t rs = make_rsrc(a.Ws + (size_t)g0 * gs, (uint32_t)ngroups * gs);
        const int gr = r >> 2;
        const uint32_t lq =
            (uint32_t)gr * gq + (uint32_t)q * kChunkCodeBytes + (uint32_t)(r & 3) * 16u;
        const uint32_t ls =
            (uint32_t)gr * gs + (uint32_t)q * kChunkScaleBytes + (uint32_t)(r & 2) * 2u;
        for (int tc0 = 0; tc0 < T; tc0 += S::PT) {
            // Window-0 offsets; a missing tile gets kOutOfRange, which stays out of range after
            // a window offset is added (every buffer here is far below 2^31 bytes).
            uint32_t coff[S::NWP], soff[S::NWP];
#pragma unroll
            for (int i = 0; i < S::NWP; i++) {
                const int p = wl + 2 * i;
                const int t = tc0 + p;
                const bool v = p < S::PT && 4 * t + gr < ngroups;
                coff[i] = off_if(v, lq + (uint32_t)t * (4u * gq));
                soff[i] = off_if(v, ls + (uint32_t)t * (4u * gs));
            }
            auto load = [&](int wl, BatchWWin<S::NWP> &dst) {
                const int w = w0 + wl;   // window of K
                const bool kv = wl < nwin && 4 * w + q < CH;
                const uint32_t cw = (uint32_t)w * (4u * kChunkCodeBytes);
                const uint32_t sw = (uint32_t)w * (4u * kChunkScaleBytes);
#pragma unroll
                for (int i = 0; i < S::NWP; i++) {
                    dst.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, off_if(kv, coff[i] + cw),
                                                                     0, kAuxNormal);
                    dst.s[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off_if(kv, soff[i] + sw),
                                                                    0, kAuxNormal);
                }
            };
            auto store = [&](int buf, const BatchWWin<S::NWP> &src) {
                uint8_t *wb = lds + 2 * S::XBUF + buf * S::WBUF;
#pragma unroll
                for (int i = 0; i < S::NWP; i++) {
                    const int p = wl + 2 * i;
                    if (p < S::PT) {
                        u32x4_t v;
#pragma unroll
                        for (int d = 0; d < 4; d++)
                            v[batch_dword_pos(d)] = src.c[i][d];
                        *reinterpret_cast<u32x4_t *>(wb + p * kBatchTileBytes + lane * 16) = v;
                        *reinterpret_cast<uint32_t *>(wb + S::PT * kBatchTileBytes +
                                                      p * (kWave * 4) + lane * 4) = src.s[i];
                    }
                }
            };
            batch_produce<kBatchWRing, BatchWWin<S::NWP>>(nwin, load, store);
            batch_barrier();   // the consumers are done with both buffers
            for (int e = 0; e < kExtraBarriers; e++)
                batch_barrier();   // partial sums written, then read
        }
    } else if (wave >= kBatchConsumers) {
        // ---------------- X loader: rows 8 MB xl .. 8 MB xl + 8 MB - 1 ----------------
        const int xl = wave - kBatchConsumers;
        // Rows past M lie beyond the descriptor and read zeros; k past K is cut per lane.
        const rsrc_t rx = make_rsrc(a.X, (uint32_t)M * (uint32_t)K * 2u);
        const int kp = lane & 15;
        const int row0 = 8 * MB * xl + (lane >> 4);   // row of piece i: row0 + 4 i
        const uint32_t xbase = ((uint32_t)row0 * (uint32_t)K + 8u * (uint32_t)kp) * 2u;
        const uint32_t xstep = 8u * (uint32_t)K;      // 4 rows
        uint32_t slot4[4];                           // LDS slot of piece i depends on i % 4
#pragma unroll
        for (int c = 0; c < 4; c++)
            slot4[c] = (uint32_t)row0 * kBatchRowBytes +
                       16u * (uint32_t)(kp ^ ((row0 + 4 * c) & 15));
        for (int tc0 = 0; tc0 < T; tc0 += S::PT) {
            auto load = [&](int wl, BatchXWin<S::NXP> &dst) {
                const int w = w0 + wl;   // window of K
                const bool v = wl < nwin && kBatchWindow * w + 8 * kp < K;
                const uint32_t cur = xbase + (uint32_t)w * (kBatchWindow * 2);
#pragma unroll
                for (int i = 0; i < S::NXP; i++)
                    dst.x[i] = __builtin_amdgcn_raw_buffer_load_b128(
                        rx, off_if(v, cur + (uint32_t)i * xstep), 0, kAuxNormal);
            };
            auto store = [&](int buf, const BatchXWin<S::NXP> &src) {
                uint8_t *xb = lds + buf * S::XBUF;
#pragma unroll
                for (int i = 0; i < S::NXP; i++)
                    *reinterpret_cast<u32x4_t *>(xb + slot4[i & 3] + 4 * i * kBatchRowBytes) =
                        src.x[i];
            };
            batch_produce<S::XRING, BatchXWin<S::NXP>>(nwin, load, store);
            batch_barrier();
            for (int e = 0; e < kExtraBarriers; e++)
                batch_barrier();
        }
    } else {
        // ---------------- consumer ----------------
        const int ts = wave % S::TS;
        const int ks = wave / S::TS;
        const uint32_t sshift = 16u * (uint32_t)(r & 1);
        // Split K: slice blockIdx.y of the workspace, unscaled; otherwise Y, times g.
        const rsrc_t ry = make_rsrc(a.Y + (size_t)blockIdx.y * batch_slice_stride(M, N),
                                    (uint32_t)M * (uint32_t)N * 4u);
        const float g = nslice > 1 ? 1.0f : *a.gscale;
        // Argmax mode: best[b][e] is the key of row 16 b + 4 q + e over the lane's columns.
        argkey_t best[ARGMAX ? MB : 1][4];
#pragma unroll
        for (int b = 0; b < (ARGMAX ? MB : 1); b++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                best[b][e] = 0;
        for (int tc0 = 0; tc0 < T; tc0 += S::PT) {
            const int nt = max(0, min(TCW, (T - tc0 - ts + S::TS - 1) / S::TS));
            f32x4_t acc[MB][S::NACC];
#pragma unroll
            for (int b = 0; b < MB; b++)
#pragma unroll
                for (int j = 0; j < S::NACC; j++)
                    acc[b][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (NR > 0 || nt >= TCW)   // with remainder tiles every slot runs (dead ones on zeros)
                batch_consume<TCW, MB, KS, TCW, NR>(acc, lds, nwin, ts, ks, lane, r, q, sshift);
            else if (TCW > 1 && nt == TCW - 1)
                batch_consume<TCW, MB, KS, (TCW > 1 ? TCW - 1 : 0), NR>(acc, lds, nwin, ts, ks,
                                                                        lane, r, q, sshift);
            else if (TCW > 2 && nt == TCW - 2)
                batch_consume<TCW, MB, KS, (TCW > 2 ? TCW - 2 : 0), NR>(acc, lds, nwin, ts, ks,
                                                                        lane, r, q, sshift);
            else
                batch_consume<TCW, MB, KS, 0, NR>(acc, lds, nwin, ts, ks, lane, r, q, sshift);
            batch_barrier();   // every wavefront is done with the buffers, which red reuses

            // acc[b][j][e] is the partial Y[16 b + 4 q + e][column 16 (tc0 + ts + TS j) + r] over
            // the steps of this consumer.
            float *red = reinterpret_cast<float *>(lds);   // [KS - 1][TS][TCW][MB][4][64]
            auto red_at = [&](int k2, int j, int b, int e) -> float & {
                return red[((((k2 - 1) * S::TS + ts) * TCW + j) * MB + b) * (4 * kWave) +
                           e * kWave + lane];
            };
            if (KS > 1) {
                if (ks > 0) {
#pragma unroll
                    for (int j = 0; j < TCW; j++)
                        if (j < nt)
#pragma unroll
                            for (int b = 0; b < MB; b++)
#pragma unroll
                                for (int e = 0; e < 4; e++)
                                    red_at(ks, j, b, e) = acc[b][j][e];
                }
                batch_barrier();   // partial sums written
            }
            if (ks == 0) {
                // Rows >= M lie beyond the descriptor (the whole offset is in the VGPR, which
                // the range check covers), so their stores are dropped; so are columns past the
                // workgroup's share.
#pragma unroll
                for (int j = 0; j < TCW; j++) {
                    const int colx = 16 * (tc0 + ts + S::TS * j) + r;
                    if (j < nt) {
                        const bool cv = colx < ncols;
                        const uint32_t vo =
                            ((uint32_t)(4 * q) * (uint32_t)N + (uint32_t)(c0 + colx)) * 4u;
#pragma unroll
                        for (int b = 0; b < MB; b++)
#pragma unroll
                            for (int e = 0; e < 4; e++) {
                                float v = acc[b][j][e];
                                for (int k2 = 1; k2 < KS; k2++)
                                    v += red_at(k2, j, b, e);
                                const uint32_t ro = (uint32_t)(16 * b + e) * (uint32_t)N * 4u;
                                if constexpr (ARGMAX) {
                                    if (cv)
                                        best[b][e] = key_max(best[b][e],
                                                             argmax_key(v * g, c0 + colx));
                                } else {
                                    __builtin_amdgcn_raw_buffer_store_b32(
                                        __float_as_uint(v * g), ry, off_if(cv, vo + ro), 0, 0);
                                }
                            }
                    }
                }
            }
            if (KS > 1)
                batch_barrier();   // partial sums read before the next pass refills the buffers
            if constexpr (NR > 0) {
                // Remainder tiles: every consumer's partial (its own MFMA step) into LDS, then
                // consumer rr adds the four of tile rr in consumer order.
                float *rred = reinterpret_cast<float *>(lds);   // [4][NR][MB][4][64]
#pragma unroll
                for (int rr = 0; rr < NR; rr++)
#pragma unroll
                    for (int b = 0; b < MB; b++)
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            rred[(((ts * NR + rr) * MB + b) * 4 + e) * kWave + lane] =
                                acc[b][TCW + rr][e];
                batch_barrier();   // partial sums written
                if (ts < NR) {
                    const int colx = 16 * (tc0 + S::TS * TCW + ts) + r;
                    const bool cv = colx < ncols;
                    const uint32_t vo =
                        ((uint32_t)(4 * q) * (uint32_t)N + (uint32_t)(c0 + colx)) * 4u;
#pragma unroll
                    for (int b = 0; b < MB; b++)
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            float v = 0.0f;
#pragma unroll
                            for (int c = 0; c < kBatchConsumers; c++)
                                v += rred[(((c * NR + ts) * MB + b) * 4 + e) * kWave + lane];
                            const uint32_t ro = (uint32_t)(16 * b + e) * (uint32_t)N * 4u;
                            if constexpr (ARGMAX) {
                                if (cv)
                                    best[b][e] =
                                        key_max(best[b][e], argmax_key(v * g, c0 + colx));
                            } else {
                                __builtin_amdgcn_raw_buffer_store_b32(
                                    __float_as_uint(v * g), ry, off_if(cv, vo + ro), 0, 0);
                            }
                        }
                }
                batch_barrier();   // partial sums read before the next pass refills the buffers
            }
        }
        if constexpr (ARGMAX) {
            // Every consumer writes all its rows' keys (0 where it stored nothing).
#pragma unroll
            for (int b = 0; b < (ARGMAX ? MB : 1); b++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const argkey_t k = key_max_16(best[b][e]);
                    const int row = 16 * b + 4 * q + e;
                    if (r == 0 && row < M)
                        a.keys[(size_t)row * a.key_slots + kBatchConsumers * blockIdx.x + wave] =
                            k;
                }
        }
    }
}

// Y = g * (P[0] + P[1] + ... + P[S - 1]) over count = M * N floats, slices in order (split K);
// slice s starts at P + s * stride (batch_slice_stride). Thread t takes elements 4 t .. 4 t + 3.
__global__ __launch_bounds__(256) void batch_reduce_kernel(const float *P, int S, long long count,
                                                          long long stride, const float *gscale,
                                                          float *Y)
{
    const long long e0 = 4 * ((long long)blockIdx.x * blockDim.x + threadIdx.x);
    if (e0 >= count)
        return;
    const float g = *gscale;
    if (e0 + 3 < count) {
        f32x4_t v = *reinterpret_cast<const f32x4_t *>(P + e0);
        for (int s = 1; s < S; s++)
            v += *reinterpret_cast<const f32x4_t *>(P + s * stride + e0);
#pragma unroll
        for (int i = 0; i < 4; i++)
            Y[e0 + i] = v[i] * g;
    } else {
        for (long long e = e0; e < count; e++) {
            float v = P[e];
            for (int s = 1; s < S; s++)
                v += P[s * stride + e];
            Y[e] = v * g;
        }
    }
}

// Split K in argmax mode: the outputs of batch_reduce_kernel (the same sums in the same order),
// folded into keys instead of stored. Workgroup (x, m) takes columns x * 256 + t, stepping by
// gridDim.x * 256, of row m and writes its key to keys[m * key_slots + x].
__global__ __launch_bounds__(256) void batch_reduce_argmax_kernel(const float *P, int S, int N,
                                                                  long long stride,
                                                                  const float *gscale,
                                                                  argkey_t *keys, int key_slots)
{
    __shared__ argkey_t best[4];
    const int m = blockIdx.y;
    const float g = *gscale;
    argkey_t k = 0;
    for (int c = blockIdx.x * 256 + threadIdx.x; c < N; c += gridDim.x * 256) {
        const long long e = (long long)m * N + c;
        float v = P[e];
        for (int s = 1; s < S; s++)
            v += P[s * stride + e];
        k = key_max(k, argmax_key(v * g, c));
    }
    k = key_max_64(k);
    if ((threadIdx.x & (kWave - 1)) == 0)
        best[threadIdx.x / kWave] = k;
    __syncthreads();
    if (threadIdx.x == 0)
        keys[(size_t)m * key_slots + blockIdx.x] =
            key_max(key_max(best[0], best[1]), key_max(best[2], best[3]));
}

}  // namespace nvfp4

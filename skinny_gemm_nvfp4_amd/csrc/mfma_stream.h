// mfma_stream.h -- persistent NVFP4 x bf16 matrix-core kernel, one 16-row block of X per workgroup.
//
// Speculative verification of one request runs the target's projections on 1 + 15 drafted
// tokens at once ("SparkInfer" README, speculative decoding sections), so X has 16 rows: one
// v_mfma_f32_16x16x32_bf16 row tile. The kernel is bound by the weight stream, like decode. More
// rows run as more 16-row blocks (blockIdx.y).
//
// Work split
//   * One workgroup of W wavefronts per compute unit and row block; workgroup b owns NG / G or
//     NG / G + 1 consecutive 4-column groups (group_range: equal weight bytes per compute unit).
//     Four consecutive groups form a tile of 16 columns; the tiles are taken in equal chunks of
//     at most TC.
//   * K is cut into windows of 128 (4 chunks of 32); wavefront w owns the windows w, w + W, ...
//     and, for those windows, every tile of the chunk.
//   * Lane l = 16 q + r holds column r of the tile: it loads the 16 code bytes of chunk q of the
//     window of that column (group r / 4, column r % 4 of the group). The 64 lanes together read
//     4 pieces of 256 contiguous bytes of the packed layout, i.e. whole cache lines. MFMA k-slot
//     8 q + e of step d (d = 0..3) is k = 128 w + 32 q + 8 d + e, so dword d of the lane's codes
//     is its B fragment of step d, with the scale of block 2 (4 w + q) + d / 2.
//   * X: the 16 rows x 128 k of a window go straight from memory into the wavefront's LDS
//     buffer of the window's ring slot (four direct-to-LDS loads of 1 KB; piece kp of row m at
//     slot kp ^ m, so that the 16 rows of an A fragment fall on different bank groups), and the
//     A fragments are read there: lane (r, q) takes row r at k = 32 q + 8 d. The loads of the
//     next window (those into LDS first, then the codes into registers) are in flight while the
//     current one is multiplied; X needs no registers (measured against staging it through registers: q/k/v
//     and o_proj at M = 32 14.2 -> 13.0 and 13.6 -> 12.4 us, o_proj at M = 8 8.6 -> 7.7, down at
//     M = 16 19.0 -> 18.6, the wide shapes even). With 4 wavefronts the scale bytes of a window
//     go into the slot the same way (one 1 KB load per 8 tiles instead of a 4-byte load per
//     tile: gate_up at M = 16 26.2 -> 25.2 us, lm_head at M = 8 106 -> 97).
//   * B = e2m1 * s decoded to bf16 (exact); the sum over k does not depend on the slot order, so
//     this is the plain product.
//   * The W partial tiles are summed through LDS in wavefront order and scaled by g once,
//     four adjacent outputs per thread where the output's alignment allows.
//     Results are reproducible.
//   * FAST (K % 128 == 0) needs no per-lane K test; otherwise lanes past the last chunk read zeros.
#pragma once

#include "argmax.h"
#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kMfmaWindow = 128;
constexpr int kXRowBytes = 256;                   // one 128-k row of bf16 X
constexpr int kXBufBytes = 16 * kXRowBytes;       // one window of 16 rows

// Whether a window's scale bytes go straight into LDS (one 1 KB load per 8 tiles) rather than
// into registers (one 4-byte load per tile): with 4 wavefronts, whose chunks are wide
// (measured: gate_up at M = 16 26.0 -> 24.9 us, lm_head 106 -> 102; with 8 wavefronts and 2
// tiles o_proj was 0.1-0.3 us slower, and 9 tiles would not fit in LDS).
constexpr bool mfma_scales_in_lds(int w) { return w == 4; }

// Direct-to-LDS scale loads per window.
constexpr int mfma_scale_loads(int tc, int w) { return mfma_scales_in_lds(w) ? (tc + 7) / 8 : 0; }

// Bytes of one ring slot of a wavefront: the window's X, then its tiles' scale bytes.
constexpr int mfma_slot_bytes(int tc, int w) { return kXBufBytes + 1024 * mfma_scale_loads(tc, w); }

// Windows in a wavefront's ring: one multiplied while the next is in flight (deeper rings
// measured slower: gate_up at M = 16 24.9 -> 26.9 us with 3, 28.2 with 4).
constexpr int kMfmaDepth = 2;

// LDS bytes of mfma_stream_kernel<TC, W, FAST>: the ring slots of every wavefront (the
// direct-to-LDS loads of the next window land there while a window is multiplied), then one
// 16 x 16 fp32 partial per wavefront and tile for the reduction.
constexpr int mfma_stream_lds_bytes(int tc, int w)
{
    return kMfmaDepth * mfma_slot_bytes(tc, w) * w + w * tc * 4 * kWave * 4;
}

template <int TC, bool SL>
struct MfmaWindow {
    static constexpr int NS = SL ? (TC + 7) / 8 : 0;
    u32x4_t c[TC];            // the lane's 16 code bytes of each tile
    uint32_t s[SL ? 1 : TC];  // without SL: the word holding the lane's 2 scale bytes of each tile

    // The window's loads, into ring slot `slot` (LDS) and these registers:
    //   * with SL, the scale bytes of its tiles straight into the slot (load j, lane l: tile
    //     8 j + l / 8, group (l / 2) % 4, chunks 2 (l % 2) and 2 (l % 2) + 1 of the window: 16
    //     bytes landing at 128 (l / 8) + 32 group + 16 (l % 2), i.e. tile-major, then group,
    //     chunk, column, block);
    //   * X straight into the slot (four 1 KB loads, load p holding rows 4 p .. 4 p + 3: lane l
    //     fetches the 16-byte piece (l % 16) ^ row of row 4 p + l / 16, which lands at slot
    //     l % 16 of the row);
    //   * the codes of each tile (and without SL its scale word) into registers.
    // xo[p] / xk[p]: the lane's X byte offset / k of load p at window 0; sv0 / sg / sh: its part
    // of the scale loads at window 0 (SL) or ls: its scale word's offset (without); lq: its code
    // offset within a tile-window at window 0; tq/ts: code/scale bytes per tile.
    template <bool FAST>
    __device__ __forceinline__ void load(rsrc_t rq, rsrc_t rs, rsrc_t rx, uint8_t *slot,
                                         uint32_t lq, uint32_t sv0, int sg, int sh, uint32_t ls,
                                         uint32_t tq, uint32_t ts, const uint32_t (&xo)[4],
                                         const int (&xk)[4], int lane, int w, bool live, int tc0,
                                         int nt, int ngroups, int gr, int q, int CH, int K)
    {
#pragma unroll
        for (int j = 0; j < NS; j++) {
            const int t = 8 * j + (lane >> 3);
            const bool v = live && t < nt && 4 * (tc0 + t) + sg < ngroups &&
                           (FAST || 4 * w + 2 * sh < CH);
            lds_load16(rs, slot + kXBufBytes + j * 1024,
                       off_if(v, sv0 + (uint32_t)(tc0 + t) * ts +
                                     (uint32_t)w * (4u * kChunkScaleBytes)));
        }
#pragma unroll
        for (int p = 0; p < 4; p++)
            lds_load16(rx, slot + p * 1024,
                       off_if(live && (FAST || kMfmaWindow * w + xk[p] < K),
                              xo[p] + (uint32_t)w * (kMfmaWindow * 2)));
        // The LDS loads go out first: the wait before a window's LDS operands counts the loads
        // into registers behind them (loads complete in issue order).
        __builtin_amdgcn_sched_barrier(0);
        const bool kv = live && (FAST || 4 * w + q < CH);
#pragma unroll
        for (int t = 0; t < TC; t++) {
            const bool v = kv && t < nt && 4 * (tc0 + t) + gr < ngroups;
            c[t] = __builtin_amdgcn_raw_buffer_load_b128(
                rq, off_if(v, lq + (uint32_t)(tc0 + t) * tq + (uint32_t)w * (4u * kChunkCodeBytes)),
                0, kAuxNormal);
            if constexpr (!SL)
                s[t] = __builtin_amdgcn_raw_buffer_load_b32(
                    rs, off_if(v, ls + (uint32_t)(tc0 + t) * ts +
                                      (uint32_t)w * (4u * kChunkScaleBytes)),
                    0, kAuxNormal);
        }
    }

    // sb: the lane's scale bytes of each tile (block of k 32 q .. + 15 in bits 0-7, of + 16 ..
    // + 31 in bits 8-15); with SL masked to zero for a chunk past K (the 16-byte scale load of
    // the window holding the end of K may bring the next group's bytes there; the codes are
    // zero).
    __device__ __forceinline__ void mul(f32x4_t (&acc)[TC], const u32x4_t (&a)[4],
                                        const uint32_t (&sb)[TC], int nt) const
    {
#pragma unroll
        for (int t = 0; t < TC; t++) {
            if (t < nt) {
                const uint32_t sw = sb[t];
                const float s_lo = e4m3_to_f32<0>(sw);   // k 32 q .. + 15 of the window
                const float s_hi = e4m3_to_f32<1>(sw);   // k 32 q + 16 .. + 31
#pragma unroll
                for (int d = 0; d < 4; d++)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(a[d]), decode8_scaled(c[t][d], d < 2 ? s_lo : s_hi), acc[t], 0,
                        0, 0);
            }
        }
    }
};

// The A fragments of a window from its X buffer: lane (r, q), step d: row r, piece 4 q + d (at
// slot (4 q + d) ^ r, so that the 16 rows of a fragment fall on different bank groups).
__device__ __forceinline__ void mfma_read_a(u32x4_t (&a)[4], const uint8_t *buf, int r, int q)
{
#pragma unroll
    for (int d = 0; d < 4; d++)
        a[d] = *reinterpret_cast<const u32x4_t *>(buf + r * kXRowBytes + 16 * ((4 * q + d) ^ r));
}

template <int TC, int W, bool FAST, int D = kMfmaDepth>
__global__ __launch_bounds__(kWave *W) void mfma_stream_kernel(GemmArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int CH = num_chunks(K);
    const int NG = num_groups(N);
    int g0, ngroups;
    if (a.H != nullptr) {
        // SiLU(gate) * up: whole pairs of groups per workgroup (gate 2p, up 2p + 1).
        group_range(NG >> 1, (int)gridDim.x, (int)blockIdx.x, &g0, &ngroups);
        g0 *= 2;
        ngroups *= 2;
    } else {
        group_range(NG, (int)gridDim.x, (int)blockIdx.x, &g0, &ngroups);
    }
    const int c0 = kGroupCols * g0;
    const int ncols = min(N - c0, kGroupCols * ngroups);
    const int T = (ngroups + 3) / 4;   // tiles of 16 columns
    const int m0 = blockIdx.y * 16;
    const int mrows = min(16, a.M - m0);
    const int nwin = (CH + 3) / 4;

    const uint32_t gq = (uint32_t)CH * kChunkCodeBytes;
    const uint32_t gs = (uint32_t)CH * kChunkScaleBytes;
    const rsrc_t rq = make_rsrc(a.Wq + (size_t)g0 * gq, (uint32_t)ngroups * gq);
    const rsrc_t rs = uniform_rsrc(a.Ws + (size_t)g0 * gs, (uint32_t)ngroups * gs);
    const rsrc_t rx = uniform_rsrc(a.X + (size_t)m0 * (size_t)K,
                                   (uint32_t)mrows * (uint32_t)K * 2u);
    const int gr = r >> 2;   // group of the lane's column within the tile
    const uint32_t lq = (uint32_t)gr * gq + (uint32_t)q * kChunkCodeBytes + (uint32_t)(r & 3) * 16u;
    // The lane's part of a window's scale loads: group sg, chunks 2 sh and 2 sh + 1.
    const int sg = (lane >> 1) & 3;
    const int sh = lane & 1;
    const uint32_t sv0 = (uint32_t)sg * gs + (uint32_t)sh * 16u;
    // Without SL: the lane's scale word (columns (r & 2), (r & 2) + 1 of chunk q), and its half.
    const uint32_t ls = (uint32_t)gr * gs + (uint32_t)q * kChunkScaleBytes + (uint32_t)(r & 2) * 2u;
    const uint32_t sshift = 16u * (uint32_t)(r & 1);
    // Its scale bytes within a slot's scale area: group r / 4, chunk q, column r % 4 (+ 128 t).
    const uint32_t sread = kXBufBytes + (uint32_t)(r >> 2) * 32u + (uint32_t)q * 8u +
                           (uint32_t)(r & 3) * 2u;
    const uint32_t tq = 4u * gq;
    const uint32_t ts = 4u * gs;
    // The lane's X pieces of a window: load p, row 4 p + lane / 16, piece (lane % 16) ^ row.
    uint32_t xo[4];
    int xk[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const int row = 4 * p + (lane >> 4);
        xk[p] = 8 * ((lane & 15) ^ row);
        xo[p] = ((uint32_t)row * (uint32_t)K + (uint32_t)xk[p]) * 2u;
    }
    constexpr bool SL = mfma_scales_in_lds(W);
    constexpr int SLOT = mfma_slot_bytes(TC, W);
    constexpr int NS = mfma_scale_loads(TC, W);
    static_assert(D == kMfmaDepth, "ring depth of the LDS plan");
    uint8_t *xb = lds + wave * D * SLOT;   // this wavefront's ring slot u: + u SLOT
    const float g = *a.gscale;
    // This wavefront's windows: wave, wave + W, ...; window i of the wavefront is wave + i W.
    const int nmine = (nwin - wave + W - 1) / W;

    // Argmax mode: every output this thread adds up below is in row 4 q + wave % 4 of the block
    // (W is a multiple of 4), so one key per thread.
    argkey_t best = 0;

    // The tiles are taken in ceil(T / TC) chunks of equal size (to within one tile), so that the
    // last chunk keeps about as many bytes in flight as the others (lm_head at M = 8 and 16,
    // 38 tiles per workgroup: 8, 8, 8, 8, 6 instead of 9, 9, 9, 9, 2, medians of five interleaved
    // runs 100.6 vs 102.6 us and 105.4 vs 107.8 us).
    // Whether the reduction stores 4 adjacent outputs per thread (16-byte Y, 8-byte H stores):
    // N a multiple of 4 (8 for H) and an aligned output. The argmax keys keep the loop with one
    // output per thread. Medians of four interleaved runs at M = 16 against one output per
    // thread: gate_up 24.7 -> 24.1 us, with SiLU * up 27.1 -> 26.2, lm_head 101.1 -> 99.5 (the
    // reduction and stores after the last window took 1.6 us of gate_up's 23.5).
    const bool vec = a.keys == nullptr &&
                     (a.H != nullptr ? (N & 7) == 0 && ((uintptr_t)a.H & 7) == 0
                                     : (N & 3) == 0 && ((uintptr_t)a.Y & 15) == 0);

    const int nch = (T + TC - 1) / TC;
    const int cs = T > 0 ? (T + nch - 1) / nch : TC;
    // Ring of D windows: D - 1 in flight while one is multiplied. Window i of a chunk sits in ring
    // slot i % D: its codes and scales in that slot's registers, its X in that slot's buffer.
    MfmaWindow<TC, SL> ring[D];
    auto load = [&](int i, int slot, int tc, int n) {
        const int w = wave + i * W;
        ring[slot].template load<FAST>(rq, rs, rx, xb + slot * SLOT, lq, sv0, sg, sh, ls, tq, ts,
                                       xo, xk, lane, w, i < nmine, tc, n, ngroups, gr, q, CH, K);
    };
    if (T > 0) {
#pragma unroll
        for (int i = 0; i < D - 1; i++)
            load(i, i, 0, min(cs, T));
    }
    for (int tc0 = 0; tc0 < T; tc0 += cs) {
        const int nt = min(cs, T - tc0);
        f32x4_t acc[TC];
#pragma unroll
        for (int t = 0; t < TC; t++)
            acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

        for (int i0 = 0; i0 < nmine; i0 += D) {
#pragma unroll
            for (int u = 0; u < D; u++) {
                const int i = i0 + u;
                if (i < nmine) {
                    // Window i's LDS loads have landed: after them went out only its loads into
                    // registers and the D - 2 windows behind it. Its LDS operands are read
                    // before the next window's loads go out, which write the slot of window i - 1.
                    constexpr int RL = SL ? TC : 2 * TC;   // register loads per window
                    wait_vm<RL + (D - 2) * (NS + 4 + RL)>();
                    const uint8_t *sl = xb + u * SLOT;
                    u32x4_t av[4];
                    mfma_read_a(av, sl, r, q);
                    uint32_t sb[TC];
                    if constexpr (SL) {
                        const uint32_t smask =
                            (FAST || 4 * (wave + i * W) + q < CH) ? 0xFFFFu : 0u;
#pragma unroll
                        for (int t = 0; t < TC; t++)
                            sb[t] = *reinterpret_cast<const uint16_t *>(
                                        sl + sread + (t >> 3) * 1024 + (t & 7) * 128) &
                                    smask;
                    }
                    load(i + D - 1, (u + D - 1) % D, tc0, nt);
                    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
                    if constexpr (!SL) {
#pragma unroll
                        for (int t = 0; t < TC; t++)
                            sb[t] = ring[u].s[t] >> sshift;
                    }
                    ring[u].mul(acc, av, sb, nt);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // The next chunk's leading windows go out before this chunk's reduction, so that the
        // weight stream does not drain between chunks (every slot's window has been multiplied).
        // Medians of seven interleaved runs against loading them after the reduction: lm_head
        // 97.5 vs 100.7 us at M = 8, 102.2 vs 105.8 at M = 16; N = 65536 (two chunks) 41.4 vs
        // 42.8 and 42.9 vs 43.9.
        if (tc0 + cs < T) {
#pragma unroll
            for (int i = 0; i < D - 1; i++)
                load(i, i, tc0 + cs, min(cs, T - tc0 - cs));
        } else {
            wait_vm<0>();   // the loads past the last window (zeros into the X buffers) landed
        }

        // acc[t][e] is the partial Y[m0 + 4 q + e][c0 + 16 (tc0 + t) + r] of this wavefront.
        float *red = reinterpret_cast<float *>(lds + W * D * SLOT);   // [W][TC][4][64]
#pragma unroll
        for (int t = 0; t < TC; t++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                red[((wave * TC + t) * 4 + e) * kWave + lane] = acc[t][e];
        __syncthreads();
        // Else one pass of the loop below covers the chunk (and instances with 4 TC <= W, whose
        // chunks are all that narrow, keep only that loop).
        const bool vc = 4 * TC > W && vec && 4 * nt > W;
        if (vc) {
            // Four adjacent columns per thread: wavefront wave takes tiles wave, wave + W, ...;
            // lane l adds up row 4 ((l / 4) % 4) + l / 16, columns 4 (l % 4) .. + 3 of the tile,
            // in the order of the loop below (wavefront 0 first), so the sums are the same.
            const int e = lane >> 4;
            const int qq = (lane >> 2) & 3;
            const int cc = lane & 3;
            const int row = 4 * qq + e;
            const int ln0 = 16 * qq + 4 * cc;
            for (int t = wave; t < nt; t += W) {
                const int colx = 16 * (tc0 + t) + 4 * cc;
                if (row >= mrows || colx >= ncols)
                    continue;
                const f32x4_t *rv = reinterpret_cast<const f32x4_t *>(red + (t * 4 + e) * kWave + ln0);
                if (a.H != nullptr) {
                    // Gate columns 4 cc .. + 3 (cc even) and their up partners in lanes + 4.
                    if ((cc & 1) != 0)
                        continue;
                    f32x4_t sg = rv[0], su = rv[1];
                    for (int v = 1; v < W; v++) {
                        sg += rv[v * TC * kWave];
                        su += rv[v * TC * kWave + 1];
                    }
                    uint16_t h[4];
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const float gate = sg[j] * g, up = su[j] * g;
                        h[j] = __builtin_bit_cast(uint16_t,
                                                  (__bf16)(gate / (1.0f + __expf(-gate)) * up));
                    }
                    const int n = c0 + colx;
                    *reinterpret_cast<uint2 *>(a.H + (size_t)(m0 + row) * (size_t)(N >> 1) +
                                               4 * (n >> 3)) =
                        make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                   (uint32_t)h[2] | ((uint32_t)h[3] << 16));
                } else {
                    f32x4_t s = rv[0];
                    for (int v = 1; v < W; v++)
                        s += rv[v * TC * kWave];
                    *reinterpret_cast<f32x4_t *>(a.Y + (size_t)(m0 + row) * N + c0 + colx) = s * g;
                }
            }
        }
        for (int idx = vc ? nt * 4 * kWave : threadIdx.x; idx < nt * 4 * kWave; idx += kWave * W) {
            const int t = idx / (4 * kWave);
            const int e = (idx / kWave) % 4;
            const int ln = idx % kWave;
            const int row = 4 * (ln >> 4) + e;
            const int colx = 16 * (tc0 + t) + (ln & 15);
            if (a.H != nullptr) {
                // SiLU(gate) * up: a gate column (colx % 8 < 4) and its up partner colx + 4 sit in
                // the same tile and lane row.
                if (row < mrows && colx < ncols && (colx & 4) == 0) {
                    float sg = red[(t * 4 + e) * kWave + ln];
                    float su = red[(t * 4 + e) * kWave + ln + 4];
                    for (int v = 1; v < W; v++) {
                        sg += red[((v * TC + t) * 4 + e) * kWave + ln];
                        su += red[((v * TC + t) * 4 + e) * kWave + ln + 4];
                    }
                    const float gate = sg * g, up = su * g;
                    const float h = gate / (1.0f + __expf(-gate)) * up;
                    const int n = c0 + colx;   // gate column 8 qp + cc -> j = 4 qp + cc
                    a.H[(size_t)(m0 + row) * (size_t)(N >> 1) + 4 * (n >> 3) + (n & 3)] =
                        __builtin_bit_cast(uint16_t, (__bf16)h);
                }
                continue;
            }
            if (row < mrows && colx < ncols) {
                float sum = red[(t * 4 + e) * kWave + ln];
                for (int v = 1; v < W; v++)
                    sum += red[((v * TC + t) * 4 + e) * kWave + ln];
                if (a.keys == nullptr)
                    a.Y[(size_t)(m0 + row) * N + c0 + colx] = sum * g;
                else
                    best = key_max(best, argmax_key(sum * g, c0 + colx));
            }
        }
        __syncthreads();  // red is reused by the next chunk
    }
    if (a.keys != nullptr) {
        // One key per row and group of 4 wavefronts: slot blockIdx.x (W / 4) + wave / 4.
        static_assert(W % 4 == 0, "rows per thread assume W % 4 == 0");
        best = key_max_16(best);
        const int row = 4 * q + wave % 4;
        if (r == 0 && row < mrows)
            a.keys[(size_t)(m0 + row) * a.key_slots + blockIdx.x * (W / 4) + wave / 4] = best;
    }
}

}  // namespace nvfp4

// mfma_slab.h -- persistent NVFP4 x bf16 matrix-core kernel for slabs of up to 128 rows of X.
//
// Eight requests verifying 16 tokens each put 128 rows through every projection ("SparkInfer"
// README, speculative decoding sections: up to eight requests speculate together, each verifying
// its drafted tokens in one pass). At that size the bf16 matrix-core work, not the weight stream,
// bounds the GEMM, so the kernel is built around what a compute unit can feed its four matrix
// cores with: each weight is decoded once per workgroup and multiplied against every row block
// of the slab while it sits in registers, and the A fragments (rows of X) are read from LDS as
// few times as possible.
//
// Work split
//   * The grid is S tile sets x P row groups, one workgroup each (S P <= compute units). Row
//     group p holds rows 16 RB p .. 16 RB p + 16 RB - 1 of the slab; tile set s holds NG / S or
//     NG / S + 1 consecutive 4-column groups (group_range), i.e. up to TW = 2 HT + NR tiles of
//     16 columns. Narrow weights take several row groups so that each compute unit streams less
//     of X; the row groups of one tile set get workgroup ids that are equal modulo 8, which the
//     dispatcher places on the same XCD, so the weights they share are fetched from HBM once and
//     served to the others by that XCD's L2.
//   * Workgroup of 4 wavefronts, one per SIMD. Consumer c = 2 ts + ks takes the main tiles ts,
//     ts + 2, ... (HT of them) and, of every 128-k window, the MFMA k-steps 2 ks and 2 ks + 1;
//     with NR = 1 the last tile's four k-steps go one to each consumer (step 2 ks + ts). Every
//     consumer thus multiplies the same number of tile-steps, and each weight is decoded once.
//   * Per 128-k window the whole workgroup stages X (16 RB rows x 256 bytes), the codes (1 KB
//     per tile) and the scales (128 bytes per tile) in LDS through direct-to-LDS buffer loads
//     (16 bytes per lane, no registers), D windows deep, with one barrier per window. The loads
//     of a window are dealt round robin to the four wavefronts, the same number to each; loads
//     past the end of a row, of K or of the workgroup's groups read zeros.
//   * Step d of lane (r, q) covers k = 32 q + 8 d .. + 7 of the window: dword d of the lane's 16
//     code bytes of column r, chunk q is its B fragment (decoded to bf16 with its block scale,
//     exact), and row 16 b + r of X at those k its A fragment of row block b
//     (v_mfma_f32_16x16x32_bf16). X rows sit in LDS with piece kp of row m at slot kp ^ (m & 15),
//     so the 16 rows of an A fragment hit 16 different bank groups.
//   * At the end of a pass the ks = 1 consumers' partial sums (and all four of the remainder
//     tile) meet the others' in LDS in a fixed order; Y = sum * g. Results are reproducible.
//     Weights with more tiles per workgroup than TW are done in several passes, each streaming
//     X again.
//   * MODE 0 stores Y; MODE 1 folds Y into argmax keys (argmax.h), one slot per consumer and
//     tile set; MODE 2 writes H = bf16(SiLU(gate) * up) of an interleaved gate/up weight (the
//     gate column's partner is 4 lanes away in the same tile).
#pragma once

#include "argmax.h"
#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kSlabWindow = 128;
constexpr int kSlabWaves = 4;
constexpr int kSlabRowBytes = 256;      // one 128-k row of bf16 X
constexpr int kSlabTileBytes = 1024;    // codes of one 16-column tile and window
constexpr int kSlabMaxLds = 160 * 1024;

enum SlabMode { kSlabStore = 0, kSlabArgmax = 1, kSlabSilu = 2 };

template <int RB, int HT, int NR>
struct SlabShape {
    static_assert(RB == 1 || RB == 2 || RB == 4 || RB == 8, "row blocks");
    static_assert(NR == 0 || NR == 1, "one remainder tile at most");
    static constexpr int TW = 2 * HT + NR;                     // tiles per pass
    static constexpr int XBYTES = 16 * RB * kSlabRowBytes;     // X of one window
    static constexpr int CBYTES = TW * kSlabTileBytes;
    static constexpr int NSC = (TW + 7) / 8;                   // scale loads per window
    static constexpr int BUF = XBYTES + CBYTES + NSC * 1024;
    static constexpr int SINK = 1024;                          // target of padding loads
    static constexpr int DMAX = (kSlabMaxLds - SINK) / BUF;
    static constexpr int D = DMAX >= 4 ? 4 : DMAX;             // windows in LDS
    static_assert(D >= 2, "slab buffers do not fit in LDS");
    static constexpr int NWL = TW + NSC;                       // code and scale loads
    static constexpr int NWPW = (NWL + kSlabWaves - 1) / kSlabWaves;
    static constexpr int LOADS = RB + NWPW;                    // loads per wavefront and window
    // End-of-pass exchange: ks = 1 partials [2][HT][RB][4][64], remainder [4][RB][4][64].
    static constexpr int RED_MAIN = 2 * HT * RB * 4 * kWave * 4;
    static constexpr int RED = RED_MAIN + (NR ? 4 * RB * 4 * kWave * 4 : 0);
    static constexpr int RING = D * BUF + SINK;
    static constexpr int LDS = (RING > RED) ? RING : RED;
};

struct SlabLayout {
    int sets;       // S: tile sets
    int rgroups;    // P: row groups of 16 RB rows
    int gunit;      // column groups dealt together (2: whole gate/up pairs)
    int xcd;        // 1: row groups of a set share an XCD (S % 8 == 0)
    int passes;     // tile passes of up to TW tiles
    int key_slots;  // argmax: keys per row of the workspace
};

// Wait until at most N vector memory operations of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void slab_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void slab_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A buffer descriptor the compiler keeps in scalar registers: the LDS-DMA loads need one, and a
// descriptor it cannot prove uniform costs a readfirstlane loop around every load.
__device__ __forceinline__ rsrc_t slab_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return make_rsrc(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo), n);
}

__device__ __forceinline__ void slab_lds_load16(rsrc_t r, uint8_t *dst, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
}

template <int RB, int HT, int NR, int MODE>
__global__ __launch_bounds__(kWave *kSlabWaves) void mfma_slab_kernel(GemmArgs a, SlabLayout L)
{
    using S = SlabShape<RB, HT, NR>;
    constexpr int TW = S::TW;
    constexpr int D = S::D;
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int ks = wave & 1;
    const int ts = wave >> 1;
    const int K = a.K;
    const int N = a.N;
    const int CH = num_chunks(K);
    const int NG = num_groups(N);

    // Workgroup -> (tile set, row group).
    int set, rg;
    {
        const int b = blockIdx.x;
        if (L.xcd) {
            const int idx = b >> 3;
            rg = idx % L.rgroups;
            set = (idx / L.rgroups) * 8 + (b & 7);
        } else {
            set = b / L.rgroups;
            rg = b - set * L.rgroups;
        }
    }
    int g0, ngroups;
    group_range(NG / L.gunit, L.sets, set, &g0, &ngroups);   // (gunit = 2: NG is even)
    g0 *= L.gunit;
    ngroups *= L.gunit;
    const int c0 = kGroupCols * g0;
    const int ncols = min(N - c0, kGroupCols * ngroups);
    const int m0 = rg * 16 * RB;
    const int mrows = min(16 * RB, a.M - m0);
    const int nwin = (K + kSlabWindow - 1) / kSlabWindow;

    const uint32_t gq = (uint32_t)CH * kChunkCodeBytes;
    const uint32_t gs = (uint32_t)CH * kChunkScaleBytes;
    const rsrc_t rq = slab_rsrc(a.Wq + (size_t)g0 * gq, (uint32_t)ngroups * gq);
    const rsrc_t rs = slab_rsrc(a.Ws + (size_t)g0 * gs, (uint32_t)ngroups * gs);
    const rsrc_t rx = slab_rsrc(a.X + (size_t)m0 * (size_t)K, (uint32_t)max(mrows, 0) *
                                                                   (uint32_t)K * 2u);
    const float g = *a.gscale;

    // ---- load side ----
    // Loads of window w of pass `pass` into ring buffer `buf`; every wavefront issues LOADS of
    // them per window whatever the window (past the pass's last window, past K, past the rows or
    // the groups they read zeros; padding loads write zeros into the sink), so waiting for a
    // window is a fixed count of outstanding loads.
    //   X: load i of this wavefront covers rows 4 u .. 4 u + 3 of the window, u = wave + 4 i;
    //      lane l fetches piece (l % 16) ^ (row & 15) of row 4 u + l / 16 into LDS slot l % 16.
    //   W: load v = wave + 4 j of the window's list: v < TW the codes of tile v (lane l: group
    //      l / 16 of the tile, 16-byte piece l % 16 of its 256 bytes, = LDS order); then the
    //      scales of tiles 8 (v - TW) .. + 7 (lane l: tile 8 (v - TW) + l / 8, group (l / 2) % 4,
    //      16-byte half l % 2 of its 32 bytes: chunks 2 (l % 2), 2 (l % 2) + 1 of the window).
    auto issue = [&](int pass, int w, int buf) {
        const bool live = w < nwin;
        uint8_t *base = lds + buf * S::BUF;
#pragma unroll
        for (int i = 0; i < RB; i++) {
            const int u = wave + kSlabWaves * i;
            const int m = 4 * u + (lane >> 4);
            const int kp = (lane & 15) ^ (m & 15);
            const bool v = live && kSlabWindow * w + 8 * kp < K;
            slab_lds_load16(rx, base + u * 1024,
                            off_if(v, (uint32_t)m * (uint32_t)K * 2u +
                                          (uint32_t)w * (kSlabWindow * 2) + (uint32_t)kp * 16u));
        }
#pragma unroll
        for (int j = 0; j < S::NWPW; j++) {
            const int v = wave + kSlabWaves * j;
            if (v < TW) {
                const int grp = 4 * (pass * TW + v) + (lane >> 4);
                const int chunk = 4 * w + ((lane & 15) >> 2);
                const bool ok = live && grp < ngroups && chunk < CH;
                slab_lds_load16(rq, base + S::XBYTES + v * kSlabTileBytes,
                                off_if(ok, (uint32_t)grp * gq + (uint32_t)w * 256u +
                                               (uint32_t)(lane & 15) * 16u));
            } else if (v < S::NWL) {
                const int tl = 8 * (v - TW) + (lane >> 3);
                const int grp = 4 * (pass * TW + tl) + ((lane >> 1) & 3);
                const int chunk = 4 * w + 2 * (lane & 1);
                const bool ok = live && tl < TW && grp < ngroups && chunk < CH;
                slab_lds_load16(rs, base + S::XBYTES + S::CBYTES + (v - TW) * 1024,
                                off_if(ok, (uint32_t)grp * gs + (uint32_t)w * 32u +
                                               (uint32_t)(lane & 1) * 16u));
            } else {
                slab_lds_load16(rq, lds + S::D * S::BUF, kOutOfRange);
            }
        }
    };

    // ---- consume side ----
    const uint32_t code_lane = (uint32_t)(r >> 2) * 256u + (uint32_t)q * 64u + (uint32_t)(r & 3) * 16u;
    const uint32_t scale_lane = (uint32_t)(r >> 2) * 32u + (uint32_t)q * 8u + (uint32_t)(r & 2) * 2u;
    const uint32_t sshift = 16u * (uint32_t)(r & 1) + 8u * (uint32_t)ks;

#pragma unroll
    for (int i = 0; i < D - 1; i++)
        issue(0, i, i);

    argkey_t best[MODE == kSlabArgmax ? RB : 1][4];
#pragma unroll
    for (int b = 0; b < (MODE == kSlabArgmax ? RB : 1); b++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            best[b][e] = 0;

    for (int pass = 0; pass < L.passes; pass++) {
        f32x4_t acc[HT][RB];
        f32x4_t racc[NR ? RB : 1];
#pragma unroll
        for (int j = 0; j < HT; j++)
#pragma unroll
            for (int b = 0; b < RB; b++)
                acc[j][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < (NR ? RB : 1); b++)
            racc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

        for (int w = 0; w < nwin; w++) {
            slab_wait_vm<(D - 2) * S::LOADS>();   // this wavefront's loads of window w landed
            slab_barrier();                      // ... everyone's; buffer (w - 1) % D is free
            issue(pass, w + D - 1, (w + D - 1) % D);
            const uint8_t *xb = lds + (w % D) * S::BUF;
            const uint8_t *cb = xb + S::XBYTES;
            const uint8_t *sb = cb + S::CBYTES;
            // Scale bytes of chunks past K may hold the next group's scales (a 16-byte load
            // spans two chunks); their codes are zero, and the scale is zeroed so that a NaN
            // scale there cannot reach the sum.
            const bool kvalid = 4 * w + q < CH;
            uint32_t code[HT][2];
            float sc[HT];
#pragma unroll
            for (int j = 0; j < HT; j++) {
                const int t = 2 * j + ts;
                const u32x2_t c2 = *reinterpret_cast<const u32x2_t *>(
                    cb + t * kSlabTileBytes + code_lane + 8 * ks);
                code[j][0] = c2[0];
                code[j][1] = c2[1];
                const uint32_t sw = *reinterpret_cast<const uint32_t *>(
                    sb + (t >> 3) * 1024 + (t & 7) * 128 + scale_lane);
                sc[j] = kvalid ? e4m3_to_f32<0>(sw >> sshift) : 0.0f;
            }
            uint32_t rcode = 0;
            float rsc = 0.0f;
            if constexpr (NR) {
                constexpr int t = 2 * HT;
                rcode = *reinterpret_cast<const uint32_t *>(cb + t * kSlabTileBytes + code_lane +
                                                            4 * (2 * ks + ts));
                const uint32_t sw = *reinterpret_cast<const uint32_t *>(
                    sb + (t >> 3) * 1024 + (t & 7) * 128 + scale_lane);
                rsc = kvalid ? e4m3_to_f32<0>(sw >> sshift) : 0.0f;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int step = 0; step < 2; step++) {
                const int d = 2 * ks + step;
                u32x4_t av[RB];
#pragma unroll
                for (int b = 0; b < RB; b++)
                    av[b] = *reinterpret_cast<const u32x4_t *>(
                        xb + (16 * b + r) * kSlabRowBytes + 16 * ((4 * q + d) ^ r));
#pragma unroll
                for (int j = 0; j < HT; j++) {
                    const bf16x8_t bfr = decode8_scaled(code[j][step], sc[j]);
#pragma unroll
                    for (int b = 0; b < RB; b++)
                        acc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[b]), bfr,
                                                                           acc[j][b], 0, 0, 0);
                }
                if constexpr (NR) {
                    if (ts == step) {
                        const bf16x8_t bfr = decode8_scaled(rcode, rsc);
#pragma unroll
                        for (int b = 0; b < RB; b++)
                            racc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(av[b]), bfr, racc[b], 0, 0, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- end of pass: partial sums meet in LDS ----
        slab_wait_vm<0>();   // the loads in flight (next pass, or zeros past the end) landed
        slab_barrier();      // every wavefront is done with the window buffers
        // The lane's exchange address is made opaque here, so that the compiler computes the
        // exchange addresses in the epilogue instead of hoisting all of them out of the pass
        // loop (where they would stay live, in registers, across every window).
        uint32_t red_lane = 4u * (uint32_t)lane;
        asm volatile("" : "+v"(red_lane));
        float *red = reinterpret_cast<float *>(lds + red_lane);
        auto red_main = [&](int tsx, int j, int b, int e) -> float & {
            return red[(((tsx * HT + j) * RB + b) * 4 + e) * kWave];
        };
        auto red_rem = [&](int c, int b, int e) -> float & {
            return red[S::RED_MAIN / 4 + ((c * RB + b) * 4 + e) * kWave];
        };
        if (ks == 1) {
#pragma unroll
            for (int j = 0; j < HT; j++)
#pragma unroll
                for (int b = 0; b < RB; b++) {
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        red_main(ts, j, b, e) = acc[j][b][e];
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        if constexpr (NR) {
#pragma unroll
            for (int b = 0; b < RB; b++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    red_rem(wave, b, e) = racc[b][e];
        }
        slab_barrier();

        // out(t, b, e, v): v is the unscaled sum of Y[m0 + 16 b + 4 q + e][c0 + 16 t + r].
        const rsrc_t ry = make_rsrc(MODE == kSlabStore ? (const void *)(a.Y + (size_t)m0 * N)
                                                       : (const void *)a.X,
                                    MODE == kSlabStore ? (uint32_t)max(mrows, 0) * (uint32_t)N * 4u
                                                       : 0u);
        auto out = [&](int t, int b, int e, float v) {
            const int col = 16 * t + r;
            const int row = 16 * b + 4 * q + e;
            if constexpr (MODE == kSlabStore) {
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(v * g), ry,
                    off_if(col < ncols, ((uint32_t)row * (uint32_t)N + (uint32_t)(c0 + col)) * 4u),
                    0, 0);
            } else if constexpr (MODE == kSlabArgmax) {
                if (col < ncols)
                    best[b][e] = key_max(best[b][e], argmax_key(v * g, c0 + col));
            } else {
                // SiLU(gate) * up: gate columns have (col & 4) == 0, their up partner is lane + 4.
                const float up = __shfl_xor(v, 4);
                if ((r & 4) == 0 && col < ncols && row < mrows) {
                    const float gt = v * g, u = up * g;
                    const float h = gt / (1.0f + __expf(-gt)) * u;
                    const int n = c0 + col;
                    a.H[(size_t)(m0 + row) * (size_t)(N >> 1) + 4 * (n >> 3) + (n & 3)] =
                        __builtin_bit_cast(uint16_t, (__bf16)h);
                }
            }
        };
        if (ks == 0) {
#pragma unroll
            for (int j = 0; j < HT; j++)
#pragma unroll
                for (int b = 0; b < RB; b++) {
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        out(pass * TW + 2 * j + ts, b, e, acc[j][b][e] + red_main(ts, j, b, e));
                    __builtin_amdgcn_sched_barrier(0);   // one fragment at a time
                }
        }
        if constexpr (NR) {
#pragma unroll
            for (int b = 0; b < RB; b++) {
                if ((b & 3) == wave) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float v = ((red_rem(0, b, e) + red_rem(1, b, e)) + red_rem(2, b, e)) +
                                        red_rem(3, b, e);
                        out(pass * TW + 2 * HT, b, e, v);
                    }
                }
            }
        }
        slab_barrier();   // the exchange area is reused by the next pass's windows
        if (pass + 1 < L.passes) {
#pragma unroll
            for (int i = 0; i < D - 1; i++)
                issue(pass + 1, i, i);
        }
    }

    if constexpr (MODE == kSlabArgmax) {
        // Every consumer writes a key for every row of the slab's group (0 where it saw nothing).
#pragma unroll
        for (int b = 0; b < RB; b++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const argkey_t k = key_max_16(best[b][e]);
                const int row = 16 * b + 4 * q + e;
                if (r == 0 && row < mrows)
                    a.keys[(size_t)(m0 + row) * L.key_slots + kSlabWaves * set + wave] = k;
            }
    }
}

}  // namespace nvfp4

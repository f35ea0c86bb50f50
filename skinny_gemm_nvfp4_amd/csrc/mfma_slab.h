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
//   * Workgroup of 8 wavefronts, two per SIMD (wavefront w runs on SIMD w % 4), so that one
//     wavefront's MFMAs run while the other of its SIMD decodes, reads LDS or waits. Consumer w
//     takes k-step ks = w % 4 of every 128-k window and the main tiles ts, ts + 2, ... (HT of
//     them), ts = w / 4; with NR = 1 the last tile's four k-steps go one to each SIMD, to its
//     X-loading wavefront (ts = 0): the weight loaders, whose loads take longer to issue and who
//     yield the SIMD to the older X loaders, are the last to finish a window (measured: o_proj
//     and down at M = 128 about 6% faster than with the remainder on ts = ks % 2). Every weight
//     is decoded once, every A fragment read from LDS by the two wavefronts of its k-step. Per
//     window a wavefront reads all its LDS operands first (codes, scale bytes, A fragments),
//     then goes tile by tile: the MFMAs of tile j for every row block, with the decode of tile
//     j + 1 placed between them; the other wavefront of its SIMD issues MFMAs while it decodes
//     or waits.
//   * Per 128-k window the whole workgroup stages X (16 RB rows x 256 bytes), the codes (1 KB
//     per tile) and the scales (128 bytes per tile) in LDS through direct-to-LDS buffer loads
//     (16 bytes per lane, no registers), with one barrier per window: X in a ring of 3 to 5
//     windows loaded by wavefronts 0-3, the weights (from HBM, higher latency) in a ring of 4 to
//     8 loaded by wavefronts 4-7, one loader of each kind per SIMD. Loads past the end of a row,
//     of K or of the workgroup's groups read zeros. A wavefront sends its loads one at a time
//     between its MFMAs of the window before: sent together after the barrier they queue in the
//     compute unit's load pipeline (several hundred cycles per window) and hold back the first
//     MFMAs.
//   * Step d of lane (r, q) covers k = 32 q + 8 d .. + 7 of the window: dword d of the lane's 16
//     code bytes of column r, chunk q is its B fragment (decoded to bf16 with its block scale,
//     exact), and row 16 b + r of X at those k its A fragment of row block b
//     (v_mfma_f32_16x16x32_bf16). X rows sit in LDS with piece kp of row m at slot kp ^ (m & 15),
//     so the 16 rows of an A fragment hit 16 different bank groups.
//   * At the end of a pass the four k-step partial sums of every output meet in LDS, 64 rows at
//     a time (LDS holds four k-steps' partials of 64 rows of 9 tiles): every wavefront writes
//     its partials to its k-step's area at once, then all 512 threads add the four areas in a
//     fixed order (((ks3 + ks2) + ks1) + ks0, the remainder tile's parts likewise) and write
//     whole rows (16-byte stores), Y = sum * g. Results are reproducible. (The k-steps had taken
//     turns adding into one tile, two wavefronts at a time: medians of two interleaved runs at
//     M = 128, gate_up 65.4 -> 59.8 us, lm_head 267 -> 249, q/k/v 26.2 -> 25.6.) Weights with
//     more tiles per workgroup than TW are done in several passes, each streaming X again.
//   * MODE 0 stores Y; MODE 1 folds Y into argmax keys (argmax.h), one slot per row and tile
//     set; MODE 2 writes H = bf16(SiLU(gate) * up) of an interleaved gate/up weight.
#pragma once

#include <type_traits>

#include "argmax.h"
#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kSlabWindow = 128;
constexpr int kSlabWaves = 8;
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
    static constexpr int WBYTES = CBYTES + NSC * 1024;         // weights of one window
    static constexpr int SINK = 1024;                          // target of padding loads
    // Ring depths from the LDS budget: X (from L2) as deep as room for 4 weight windows allows
    // (3 to 5 windows), then the weights (from HBM) in what is left (4 to 8). A window's loads
    // are issued D - 1 windows ahead of its use. (Deeper rings measured slower: 16 X and 24
    // weight windows took q/k/v at one row from 21 to 25 us.)
    static constexpr int XL = RB;                 // X loads per X wavefront and window
    static constexpr int NWL = TW + NSC;
    static constexpr int WL = (NWL + 3) / 4;      // weight loads per weight wavefront and window
    static constexpr int BUDGET = kSlabMaxLds - SINK;
    static constexpr int clampi(int v, int lo, int hi) { return v < lo ? lo : v > hi ? hi : v; }
    // Caps by instance, measured (medians of interleaved runs):
    //   * row groups of at most 32 rows with 8-9 tiles per pass (gate/up and the lm_head at small
    //     M) keep at most 4 and 6: the batch-invariant mode at one row gate_up 32.1 -> 30.3 us,
    //     lm_head 121.2 -> 118.2; at M = 32 gate_up 38.1 -> 37.2, the lm_head 145.3 -> 143.4 (the
    //     narrow shapes of those row groups were slower so: down 38.7 -> 42.4);
    //   * 64-row groups with at most 5 tiles per pass (q/k/v, o_proj and down at M = 128) keep 3
    //     and 4: q/k/v 25.9 -> 25.2, o_proj 23.6 -> 22.4, down 65.2 -> 63.2 (three runs; with 4 and
    //     6 down was slower, 65.0 -> 66.0);
    //   * 128-row groups with an even number of tiles per pass (the lm_head at M > 64) keep at
    //     most 4 weight windows: the lm_head at M = 128 251.4 -> 247.5 us, at M = 96 229.7 ->
    //     226.9 (four runs; gate/up, with a remainder tile, was even);
    //   * the others at most 5 and 8.
    static constexpr bool WIDE_SMALL = RB <= 2 && HT == 4;
    static constexpr bool NARROW_64 = RB == 4 && HT <= 2;
    static constexpr bool EVEN_128 = RB == 8 && NR == 0;
    static constexpr int XCAP = WIDE_SMALL ? 4 : NARROW_64 ? 3 : 5;
    static constexpr int WCAP = WIDE_SMALL ? 6 : (NARROW_64 || EVEN_128) ? 4 : 8;
    static constexpr int DX = clampi((BUDGET - 4 * WBYTES) / XBYTES, 3, XCAP);
    static constexpr int DW = clampi((BUDGET - DX * XBYTES) / WBYTES, 4, WCAP);
    static_assert(DX * XBYTES + DW * WBYTES <= BUDGET, "slab buffers do not fit in LDS");
    static constexpr int XOFF = 0;
    static constexpr int WOFF = DX * XBYTES;
    static constexpr int SINKOFF = WOFF + DW * WBYTES;
    // Waves 0-3 issue the X loads (16 RB rows, 4 per load: RB loads each per window), waves 4-7
    // the weight loads (codes then scales, the same count each, padded).
    static_assert((DX - 2) * XL < 64 && (DW - 2) * WL < 64, "vmcnt range");
    // End of a pass: the rows go through in NPH phases of PR = 16 PB rows (LDS holds the four
    // k-steps' partials of 64 rows of 9 tiles at most). In a phase, the partials of k-step k sit
    // in area k as a row-major tile [PR][YST] of floats (the row padding keeps the four rows a
    // fragment writes on different banks).
    static constexpr int PB = RB < 4 ? RB : 4;
    static constexpr int PR = 16 * PB;
    static constexpr int NPH = RB / PB;
    static constexpr int YST = 16 * TW + 4;
    static constexpr int AREA = PR * YST;         // floats of one k-step's area
    static constexpr int EPI = 4 * AREA * 4;
    static_assert(EPI <= kSlabMaxLds, "exchange areas do not fit in LDS");
    static constexpr int RING = SINKOFF + SINK;
    static constexpr int LDS = (RING > EPI) ? RING : EPI;
};

struct SlabLayout {
    int sets;       // S: tile sets
    int rgroups;    // P: row groups of 16 RB rows
    int gunit;      // column groups dealt together (2: whole gate/up pairs)
    int xcd;        // 1: row groups of a set share an XCD (S % 8 == 0)
    int passes;     // tile passes of up to TW tiles
    int key_slots;  // argmax: keys per row of the workspace (one per tile set)
    int vec;        // 1: Y (or H) rows may be written 16 (8) bytes at a time
};

__device__ __forceinline__ void slab_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int RB, int HT, int NR, int MODE>
__global__ __launch_bounds__(kWave *kSlabWaves) void mfma_slab_kernel(GemmArgs a, SlabLayout L)
{
    using S = SlabShape<RB, HT, NR>;
    constexpr int TW = S::TW;
    constexpr int kThreads = kWave * kSlabWaves;
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int ks = wave & 3;    // k-step of every window (= the SIMD)
    const int ts = wave >> 2;   // main tiles ts, ts + 2, ...
    const bool rem = NR != 0 && ts == 0;   // takes k-step ks of the remainder tile
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
    const rsrc_t rq = uniform_rsrc(a.Wq + (size_t)g0 * gq, (uint32_t)ngroups * gq);
    const rsrc_t rs = uniform_rsrc(a.Ws + (size_t)g0 * gs, (uint32_t)ngroups * gs);
    const rsrc_t rx = uniform_rsrc(a.X + (size_t)m0 * (size_t)K, (uint32_t)max(mrows, 0) *
                                                                   (uint32_t)K * 2u);
    const float g = *a.gscale;

    // ---- load side ----
    // Waves 0-3 load X windows into the X ring, waves 4-7 weight windows into the weight ring
    // (each load kind in waves of its own, so that waiting for a fast X load never waits for
    // older weight loads: loads complete in issue order). Every call issues the same number of
    // loads whatever the window (past the pass's last window they read zeros; padding loads write
    // zeros into the sink), so waiting for a window is a fixed count of outstanding loads. A
    // load's lane offset is a loop-invariant register plus a scalar part; rows past the group and
    // column groups past the workgroup's lie beyond the descriptors' ranges and read zeros by
    // themselves, so only the window holding the end of K masks lanes.
    //   X: load i of X wave xw covers rows 4 u .. 4 u + 3 of the window, u = xw + 4 i; lane l
    //      fetches piece (l % 16) ^ (row & 15) of row 4 u + l / 16 into LDS slot l % 16 (row & 15
    //      = (4 xw + l / 16) & 15 does not depend on i).
    //   W: load v = (wave - 4) + 4 j of the window's list: v < TW the codes of tile v (lane l:
    //      group l / 16 of the tile, 16-byte piece l % 16 of its 256 bytes, = LDS order); then
    //      the scales of tiles 8 (v - TW) .. + 7 (lane l: tile 8 (v - TW) + l / 8, group
    //      (l / 2) % 4, 16-byte half l % 2 of its 32 bytes: chunks 2 (l % 2), 2 (l % 2) + 1).
    const bool xwave = wave < 4;
    const int xw = wave & 3;
    const int xrow = 4 * xw + (lane >> 4);                    // row of load 0 (u = xw)
    const int xkp = (lane & 15) ^ (xrow & 15);
    const uint32_t xlane = (uint32_t)xrow * (uint32_t)K * 2u + (uint32_t)xkp * 16u;
    const uint32_t xstep = 16u * (uint32_t)K * 2u;            // 16 rows: load i to i + 1
    const uint32_t clane = (uint32_t)(lane >> 4) * gq + (uint32_t)(lane & 15) * 16u;
    const uint32_t slane = (uint32_t)(4 * (lane >> 3) + ((lane >> 1) & 3)) * gs +
                           (uint32_t)(lane & 1) * 16u;
    const int nfull = K / kSlabWindow;                        // windows with no K tail
    // A window's loads: a set-up per window, then one call per load, so that the loads can go
    // out one at a time between the MFMAs of the window before.
    struct XIssue {
        uint8_t *base;
        uint32_t lo;
    };
    auto x_setup = [&](int w, int slot) -> XIssue {
        // Only the window holding the end of K (and those past it) masks lanes.
        const uint32_t lo = (w < nfull || (w < nwin && kSlabWindow * w + 8 * xkp < K))
                                ? xlane + (uint32_t)w * (kSlabWindow * 2)
                                : kOutOfRange;
        // (kOutOfRange plus any row step stays beyond every descriptor's range.)
        return XIssue{lds + S::XOFF + slot * S::XBYTES, lo};
    };
    auto x_load = [&](const XIssue &x, int i) {
        lds_load16(rx, x.base + (xw + 4 * i) * 1024, x.lo + (uint32_t)i * xstep);
    };
    struct WIssue {
        uint8_t *base;
        uint32_t cl, sl;
    };
    auto w_setup = [&](int pass, int w, int slot) -> WIssue {
        const bool full = w < nfull;
        const bool live = w < nwin;
        const uint32_t cw0 = (uint32_t)(4 * pass * TW) * gq + (uint32_t)w * 256u;
        const uint32_t sw0 = (uint32_t)(4 * pass * TW) * gs + (uint32_t)w * 32u;
        // Lanes past K (and every lane past the last window) start at kOutOfRange; adding a
        // tile's offset keeps them beyond every descriptor's range.
        const uint32_t cl = (full || (live && 4 * w + ((lane & 15) >> 2) < CH)) ? clane + cw0
                                                                               : kOutOfRange;
        const uint32_t sl = (full || (live && 4 * w + 2 * (lane & 1) < CH)) ? slane + sw0
                                                                          : kOutOfRange;
        return WIssue{lds + S::WOFF + slot * S::WBYTES, cl, sl};
    };
    // Load j of a weight wave: item v = (wave - 4) + 4 j of the window's list. The kind of item
    // depends on the wave, so it is chosen by selects rather than branches (a branch would cut
    // the tile loop the load sits in into pieces the scheduler cannot interleave).
    auto w_load = [&](const WIssue &x, int j) {
        const int v = (wave - 4) + 4 * j;
        const bool code = v < TW;
        const bool scale = !code && v < S::NWL;
        uint8_t *dst = code    ? x.base + v * kSlabTileBytes
                       : scale ? x.base + S::CBYTES + (v - TW) * 1024
                               : lds + S::SINKOFF;
        const uint32_t off = code    ? x.cl + (uint32_t)(4 * v) * gq
                             : scale ? x.sl + (uint32_t)(32 * (v - TW)) * gs
                                     : kOutOfRange;
        lds_load16(code ? rq : rs, dst, off);
    };
    // The first windows of a pass: D - 1 windows ahead of their use, in each ring.
    auto prologue = [&](int pass) {
        if (xwave) {
#pragma unroll
            for (int i = 0; i < S::DX - 1; i++) {
                const XIssue x = x_setup(i, i);
#pragma unroll
                for (int l = 0; l < S::XL; l++)
                    x_load(x, l);
            }
        } else {
#pragma unroll
            for (int i = 0; i < S::DW - 1; i++) {
                const WIssue x = w_setup(pass, i, i);
#pragma unroll
                for (int l = 0; l < S::WL; l++)
                    w_load(x, l);
            }
        }
    };

    // ---- consume side ----
    // Lane (r, q) of k-step d: dword d of the 16 code bytes of column r, chunk q (k = 32 q + 8 d
    // .. + 7), whose block scale is byte d / 2 of the column's two for the chunk (scale bytes of
    // a tile and window: group r / 4 at 32 (r / 4), chunk q at + 8 q, column r % 4 at + 2 (r % 4)).
    const uint32_t code_lane = (uint32_t)(r >> 2) * 256u + (uint32_t)q * 64u +
                               (uint32_t)(r & 3) * 16u + 4u * (uint32_t)ks;
    const uint32_t scale_lane = (uint32_t)(r >> 2) * 32u + (uint32_t)q * 8u +
                                (uint32_t)(r & 3) * 2u + (uint32_t)(ks >> 1);
    // A fragment of k-step ks, row block b: row 16 b + r, 16-byte piece 4 q + ks (slot ^ r).
    const uint32_t a_lane = (uint32_t)r * kSlabRowBytes + 16u * (uint32_t)((4 * q + ks) ^ r);

    prologue(0);

    argkey_t best[S::NPH];   // greedy token: the key of this thread's row of each phase
#pragma unroll
    for (int h = 0; h < S::NPH; h++)
        best[h] = 0;

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

        // The window loop, one copy per loader role, so that the role's loads (known at compile
        // time) can be placed between the MFMAs: issued all at once after the barrier they queue
        // behind each other in the compute unit's load pipeline, and the waves issuing them
        // stall before their first MFMA.
        auto windows = [&](auto role) {
            constexpr bool XR = decltype(role)::value;
            constexpr int D = XR ? S::DX : S::DW;    // ring depth of this role's loads
            constexpr int NL = XR ? S::XL : S::WL;   // its loads per window
            for (int w = 0; w < nwin; w++) {
                wait_vm<(D - 2) * NL>();   // this wave's loads of window w landed
                slab_barrier();                 // ... everyone's; the slots of window w - 1 are free
                // The loads of window w + D - 1 (into the slot of window w - 1).
                const int lw = w + D - 1;
                XIssue xi{};
                WIssue wi{};
                if constexpr (XR)
                    xi = x_setup(lw, lw % D);
                else
                    wi = w_setup(pass, lw, lw % D);
                // Per-window LDS bases of this lane (made opaque so that the compiler adds the
                // per-tile and per-row-block offsets as immediates instead of keeping one address
                // register per tile across the loop).
                uint32_t xoff = (uint32_t)(S::XOFF + (w % S::DX) * S::XBYTES) + a_lane;
                uint32_t woff = (uint32_t)(S::WOFF + (w % S::DW) * S::WBYTES);
                uint32_t coff = woff + code_lane;
                uint32_t soff = woff + (uint32_t)S::CBYTES + scale_lane;
                asm volatile("" : "+v"(xoff), "+v"(coff), "+v"(soff));
                // Scale bytes of chunks past K may hold the next group's scales (a 16-byte load
                // spans two chunks); their codes are zero, and the scale byte is cleared so that
                // a NaN scale there cannot reach the sum (only in the window holding the end of
                // K). The clearing is a mask on the byte, not a condition on its conversion: a
                // condition splits the tile loop into blocks the scheduler cannot interleave. The
                // mask is applied where the byte is converted, not where it is read: applied at
                // the read, each read waited for the one before (registers reused under the
                // register budget), and the window's reads went out one at a time.
                const uint32_t smask = (w < nfull || 4 * w + q < CH) ? 0xFFu : 0u;
                constexpr int NT = HT + (NR ? 1 : 0);
                uint32_t cw[NT];
                uint32_t sb[NT];
                // Every LDS read of the window goes out before any arithmetic, the remainder
                // tile's too (its slot exists when NR = 1; a wave that does not own it ignores
                // the values).
#pragma unroll
                for (int j = 0; j < NT; j++) {
                    const int t = j < HT ? 2 * j + ts : 2 * HT;
                    cw[j] = *reinterpret_cast<const uint32_t *>(lds + coff + t * kSlabTileBytes);
                    sb[j] = lds[soff + (t >> 3) * 1024 + (t & 7) * 128];
                }
                u32x4_t av[RB];
#pragma unroll
                for (int b = 0; b < RB; b++)
                    av[b] =
                        *reinterpret_cast<const u32x4_t *>(lds + xoff + 16 * b * kSlabRowBytes);
                __builtin_amdgcn_sched_barrier(0);
                // Tile by tile: the B fragment of tile j + 1 is decoded while the MFMAs of tile
                // j run, a few decode instructions after each MFMA; main tile j also sends its
                // share of the next loads, spread over its MFMAs. The remainder tile's fragment
                // is decoded with the last main tile, before the branch on who owns it.
                bf16x8_t bcur = decode8_scaled(cw[0], e4m3_to_f32<0>(sb[0] & smask));
#pragma unroll
                for (int j = 0; j < NT; j++) {
                    if (j == HT && !rem)
                        break;
                    bf16x8_t bnext = bcur;
                    if (j + 1 < NT)
                        bnext = decode8_scaled(
                            cw[j + 1 < NT ? j + 1 : j],
                            e4m3_to_f32<0>(sb[j + 1 < NT ? j + 1 : j] & smask));
#pragma unroll
                    for (int b = 0; b < RB; b++) {
                        f32x4_t &c = j < HT ? acc[j < HT ? j : 0][b] : racc[NR ? b : 0];
                        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[b]), bcur, c, 0,
                                                                    0, 0);
                    }
                    const int l0 = j < HT ? j * NL / HT : 0;          // this tile's loads
                    const int l1 = j < HT ? (j + 1) * NL / HT : 0;
#pragma unroll
                    for (int l = l0; l < l1; l++) {
                        if constexpr (XR)
                            x_load(xi, l);
                        else
                            w_load(wi, l);
                    }
#pragma unroll
                    for (int b = 0; b < RB; b++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                        if (j + 1 < NT)
                            __builtin_amdgcn_sched_group_barrier(0x002, 16 / RB + 1, 0);
                        // the tile's loads after MFMAs b = (l - l0) RB / (l1 - l0)
                        for (int l = l0; l < l1; l++)
                            if ((l - l0) * RB / (l1 - l0) == b)
                                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (NR && j + 1 == HT)
                        asm volatile("" : "+v"(bnext));   // keeps the decode ahead of the branch
                    bcur = bnext;
                }
            }
        };
        if (xwave)
            windows(std::true_type{});
        else
            windows(std::false_type{});

        // ---- end of pass: the partial sums meet in LDS, a phase of PR rows at a time ----
        wait_vm<0>();   // the loads in flight (next pass, or zeros past the end) landed
        slab_barrier();      // every wavefront is done with the ring buffers
        // The lane's part of the LDS addresses is made opaque here, so that the compiler computes
        // the exchange addresses in the epilogue instead of hoisting them out of the pass loop
        // (where they would stay live, in registers, across every window).
        uint32_t lane_off = 4u * (uint32_t)((4 * q) * S::YST + r);
        asm volatile("" : "+v"(lane_off));
        float *ys = reinterpret_cast<float *>(lds + lane_off) + ks * S::AREA;   // + row * YST + col
        const float *area = reinterpret_cast<const float *>(lds);
        // Output (row, col) of the phase: ((ks 3 + ks 2) + ks 1) + ks 0, for four columns.
        auto sum4 = [&](int o) -> f32x4_t {
            const f32x4_t *p = reinterpret_cast<const f32x4_t *>(area + o);
            constexpr int A4 = S::AREA / 4;
            f32x4_t v = p[3 * A4] + p[2 * A4];
            v = v + p[A4];
            return v + p[0];
        };
        // The pass's columns: c0 + 16 TW pass + col.
        const int pc0 = c0 + 16 * TW * pass;                      // first column of the pass
        const int pcols = min(ncols - 16 * TW * pass, 16 * TW);   // columns of the pass
#pragma unroll
        for (int h = 0; h < S::NPH; h++) {
            // Every wavefront writes its partials of row blocks PB h .. PB h + PB - 1 to its
            // k-step's area (tiles 2 j + ts, and the remainder tile's k-step ks if it holds it),
            // all wavefronts at once: no reads, no rounds.
#pragma unroll
            for (int j = 0; j < HT; j++)
#pragma unroll
                for (int b = 0; b < S::PB; b++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        ys[(16 * b + e) * S::YST + 16 * (2 * j + ts)] = acc[j][S::PB * h + b][e];
            if constexpr (NR != 0) {
                if (rem) {
#pragma unroll
                    for (int b = 0; b < S::PB; b++)
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            ys[(16 * b + e) * S::YST + 16 * (2 * HT)] = racc[S::PB * h + b][e];
                }
            }
            slab_barrier();
            const int r0 = S::PR * h;                   // first row of the phase in the group
            const int prows = min(S::PR, mrows - r0);   // its rows that exist (may be <= 0)
            if constexpr (MODE == kSlabStore) {
                const rsrc_t ry =
                    make_rsrc(a.Y + (size_t)m0 * N, (uint32_t)mrows * (uint32_t)N * 4u);
                const int quads = (pcols + 3) >> 2;
                for (int idx = threadIdx.x; idx < prows * quads; idx += kThreads) {
                    const int row = idx / quads;
                    const int col = 4 * (idx - row * quads);
                    const f32x4_t v = sum4(row * S::YST + col);
                    const uint32_t off =
                        ((uint32_t)(r0 + row) * (uint32_t)N + (uint32_t)(pc0 + col)) * 4u;
                    if (L.vec && col + 3 < pcols) {
                        u32x4_t o;
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            o[e] = __float_as_uint(v[e] * g);
                        __builtin_amdgcn_raw_buffer_store_b128(o, ry, off, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (col + e < pcols)
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e] * g),
                                                                      ry, off + 4u * e, 0, 0);
                    }
                }
            } else if constexpr (MODE == kSlabSilu) {
                // Column block p of 8: gate columns 8 p .. 8 p + 3, up 8 p + 4 .. 8 p + 7 give
                // H[m][(pc0 >> 1) + 4 p .. + 3] (pc0 and pcols are multiples of 8).
                const int blocks = pcols >> 3;
                const size_t hstride = (size_t)(N >> 1);
                for (int idx = threadIdx.x; idx < prows * blocks; idx += kThreads) {
                    const int row = idx / blocks;
                    const int p8 = idx - row * blocks;
                    const f32x4_t gv = sum4(row * S::YST + 8 * p8);
                    const f32x4_t uv = sum4(row * S::YST + 8 * p8 + 4);
                    uint16_t hb[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float gt = gv[e] * g, u = uv[e] * g;
                        hb[e] = __builtin_bit_cast(uint16_t, (__bf16)(gt / (1.0f + __expf(-gt)) * u));
                    }
                    uint16_t *dst =
                        a.H + (size_t)(m0 + r0 + row) * hstride + (size_t)(pc0 >> 1) + 4 * p8;
                    if (L.vec) {
                        *reinterpret_cast<u32x2_t *>(dst) =
                            u32x2_t{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16),
                                    (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            dst[e] = hb[e];
                    }
                }
            } else {
                // Greedy token: TPR threads per row of the phase scan its columns (col = part,
                // part + TPR, ...) and fold them into one key; the key of that row over all
                // passes stays with those threads.
                constexpr int TPR = kThreads / S::PR;
                const int row = threadIdx.x / TPR;
                const int part = threadIdx.x - row * TPR;
                argkey_t k = 0;
                if (row < prows)
                    for (int col = part; col < pcols; col += TPR) {
                        const int o = row * S::YST + col;
                        const float y = ((area[o + 3 * S::AREA] + area[o + 2 * S::AREA]) +
                                         area[o + S::AREA]) +
                                        area[o];
                        k = key_max(k, argmax_key(y * g, pc0 + col));
                    }
#pragma unroll
                for (int d = 1; d < TPR; d <<= 1)
                    k = key_max(k, shfl_xor_key(k, d));
                best[h] = key_max(best[h], k);
            }
            slab_barrier();   // the areas are written again by the next phase or pass
        }
        if (pass + 1 < L.passes)
            prologue(pass + 1);
    }

    if constexpr (MODE == kSlabArgmax) {
        // One key per row and workgroup: slot `set` of the row.
        constexpr int TPR = kThreads / S::PR;
        const int row = threadIdx.x / TPR;
        if (threadIdx.x - row * TPR == 0) {
#pragma unroll
            for (int h = 0; h < S::NPH; h++)
                if (S::PR * h + row < mrows)
                    a.keys[(size_t)(m0 + S::PR * h + row) * L.key_slots + set] = best[h];
        }
    }
}

}  // namespace nvfp4

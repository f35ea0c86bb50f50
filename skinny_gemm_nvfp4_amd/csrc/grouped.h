// grouped.h -- grouped (mixture-of-experts) NVFP4 dot-product kernel: rows sorted by expert, each
// block of rows multiplied by its own expert's weights, in one launch with no host sync.
//
// The pages' engine runs mixture-of-experts models with a fused MoE FFN kernel and a router that
// dispatches tokens to experts without synchronising with the host ("SparkInfer" README, section
// "Layout & scoring", and its MoE model targets). At decode every token reads only its routed
// experts' weights, so the weight stream is a handful of small matrices with a few rows each:
// the same bandwidth-bound dot product as decode, cut into per-expert pieces whose sizes only the
// device knows.
//
// Work split
//   * The row counts come from the device array offsets[E + 1] (expert e owns rows offsets[e] ..
//     offsets[e+1] - 1 of X and Y). Each workgroup reads it once and builds, in LDS, the prefix
//     sums of the experts' row chunks (MR rows per chunk). An item is one (row chunk, 4-column
//     group) pair: the whole K of 4 columns of the chunk's expert, NG items per chunk.
//   * The items are dealt to all wavefronts of the grid in contiguous runs of equal length, so
//     every wavefront streams the same number of weight bytes whatever the routing. A wavefront
//     walks its run window by window (512 k: 1 KB of codes, one 16-byte load per lane, as the
//     dot-product kernel), with D windows in flight across item boundaries.
//   * Lane l takes column l % 4 of the group and chunk l / 4 of the window. LDSX: the workgroup
//     first copies the X rows of every chunk its items touch into LDS (a few rows: the launcher
//     sizes the space from T, E and the grid), 80 bytes per 32 k so that the lanes of a column
//     quad read one broadcast; otherwise each lane fetches its 64 bytes per row and window from
//     L2.
//   * At the end of an item the 16 lanes of each column are summed in a fixed order, times the
//     expert's g, and stored. No item is split between wavefronts, so there are no partial sums
//     to exchange, and a row's result does not depend on MR, the grid or the other rows.
//   * A chunk with fewer rows than MR (an expert with few rows) skips the dot products of the
//     missing rows, so a larger MR costs only the decode it shares: each expert's weights are
//     then read once for up to MR rows instead of once per row.
//   * Offsets are clamped to [0, T] and made non-decreasing (a running maximum), so the experts'
//     rows never overlap and add up to at most T: bad offsets move rows between experts, never
//     an access outside X, Y or the weights.
#pragma once

#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kGroupedWindow = 512;
constexpr int kGroupedSlot = 80;   // LDS bytes per 32-k chunk of a staged X row (64 used)

template <int MR, bool LDSX>
struct GroupedUnit {
    uint32_t code[4];
    uint32_t scale;
    u32x4_t x[LDSX ? 1 : MR][4];   // (L2 path) the lane's 32 k of each row: k = 8 p .. 8 p + 7
};

// LDSX: dynamic LDS holds xrows staged rows of row_bytes each, then xrows ints of row numbers.
template <int MR, int W, int D, bool FAST, bool LDSX>
__global__ __launch_bounds__(kWave *W) void grouped_gemv_kernel(GroupedArgs a, int xrows)
{
    extern __shared__ __align__(16) uint8_t xlds[];
    __shared__ int cum[kGroupedMaxExperts + 1];   // row chunks of experts < e
    __shared__ int rstart[kGroupedMaxExperts];    // first row of expert e (clamped)
    __shared__ int rcount[kGroupedMaxExperts];    // rows of expert e (>= 0)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int col = lane & 3;
    const int j = lane >> 2;
    const int T = a.T, E = a.E, N = a.N, K = a.K;
    const int NG = num_groups(N);
    const int CH = num_chunks(K);
    const int nwin = (K + kGroupedWindow - 1) / kGroupedWindow;
    const uint32_t gq = (uint32_t)CH * kChunkCodeBytes;    // code bytes per group
    const uint32_t gs = (uint32_t)CH * kChunkScaleBytes;   // scale bytes per group
    const size_t cb = (size_t)NG * gq;                      // code bytes per expert
    const size_t sb = (size_t)NG * gs;                      // scale bytes per expert

    // The offsets, clamped to [0, T], into cum[] first: one load per thread, all in flight at
    // once (the scan below reads them from LDS and overwrites cum[] only after its last read).
    for (int e = threadIdx.x; e <= E; e += kWave * W)
        cum[e] = min(max(a.offsets[e], 0), T);
    __syncthreads();

    // Prefix sums of the row chunks, by wavefront 0: lane l takes a contiguous run of experts.
    // Boundaries: the clamped offsets, then a running maximum (prefix max over the lanes' runs),
    // so expert e owns rows [b_e, b_{e+1}) with b non-decreasing.
    if (wave == 0) {
        const int per = (E + kWave - 1) / kWave;
        const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
        int lmax = 0;
        for (int e = e0; e < e1; e++)
            lmax = max(lmax, cum[e]);
        int pmax = lmax;   // inclusive prefix max over lanes
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int t = __shfl_up(pmax, d);
            if (lane >= d)
                pmax = max(pmax, t);
        }
        int bnd = __shfl_up(pmax, 1);   // max over the earlier lanes' runs
        if (lane == 0)
            bnd = 0;
        int local = 0;
        for (int e = e0; e < e1; e++) {
            const int r0 = max(bnd, cum[e]);
            bnd = max(r0, cum[e + 1]);
            const int n = bnd - r0;
            rstart[e] = r0;
            rcount[e] = n;
            local += (n + MR - 1) / MR;
        }
        int incl = local;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int t = __shfl_up(incl, d);
            if (lane >= d)
                incl += t;
        }
        int run = incl - local;
        for (int e = e0; e < e1; e++) {
            cum[e] = run;
            run += (rcount[e] + MR - 1) / MR;
        }
        if (lane == kWave - 1)
            cum[E] = incl;
    }
    __syncthreads();

    // This wavefront's run of items [i0, i1) out of chunks * NG (< 2^40 by the launcher).
    const long long items = (long long)cum[E] * NG;
    const long long V = (long long)gridDim.x * W;
    const long long v = (long long)blockIdx.x * W + wave;
    const long long i0 = items * v / V;
    const long long i1 = items * (v + 1) / V;

    // Item i: row chunk ci = i / NG of expert e (the last e with cum[e] <= ci), group i % NG.
    struct Item {
        int e, grp, row0, rows, slot;   // slot: the row chunk
    };
    auto item_at = [&](long long i) -> Item {
        Item it;
        const int ci = (int)(i / NG);
        it.grp = (int)(i - (long long)ci * NG);
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cum[mid] <= ci)
                lo = mid;
            else
                hi = mid - 1;
        }
        it.e = lo;
        const int first = (ci - cum[lo]) * MR;
        it.row0 = rstart[lo] + first;
        it.rows = min(MR, rcount[lo] - first);
        it.slot = ci;
        return it;
    };
    // The item after `it`: the next group of the same chunk, else group 0 of the next chunk,
    // whose expert is found by a binary search from it.e on (no 64-bit division).
    auto item_next = [&](Item &it) {
        if (++it.grp < NG)
            return;
        it.grp = 0;
        const int ci = ++it.slot;
        int lo = it.e, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cum[mid] <= ci)
                lo = mid;
            else
                hi = mid - 1;
        }
        it.e = lo;
        const int first = (ci - cum[lo]) * MR;
        it.row0 = rstart[lo] + first;
        it.rows = min(MR, rcount[lo] - first);
    };


    // Prefetch cursor: item ip (described by pit), window wp.
    long long ip = i0;
    int wp = 0;
    Item pit = item_at(ip);
    rsrc_t rq, rs, rx;
    auto set_sources = [&]() {
        rq = make_rsrc(a.Wq + (size_t)pit.e * cb + (size_t)pit.grp * gq, gq);
        rs = make_rsrc(a.Ws + (size_t)pit.e * sb + (size_t)pit.grp * gs, gs);
        if constexpr (!LDSX)
            rx = make_rsrc(a.X + (size_t)pit.row0 * (size_t)K,
                           (uint32_t)pit.rows * (uint32_t)K * 2u);
    };
    set_sources();
    const uint32_t vq = 16u * (uint32_t)lane;
    const uint32_t vs = 4u * (uint32_t)(lane >> 1);
    const uint32_t sshift = 16u * (uint32_t)(lane & 1);
    auto load_next = [&]() -> GroupedUnit<MR, LDSX> {
        GroupedUnit<MR, LDSX> u;
        const bool live = ip < i1 && (FAST || kGroupedWindow / kChunkK * wp + j < CH);
        const u32x4_t c = __builtin_amdgcn_raw_buffer_load_b128(
            rq, off_if(live, vq + (uint32_t)wp * (16u * kChunkCodeBytes)), 0, kAuxStream);
        u.code[0] = c[0];
        u.code[1] = c[1];
        u.code[2] = c[2];
        u.code[3] = c[3];
        u.scale = __builtin_amdgcn_raw_buffer_load_b32(
            rs, off_if(live, vs + (uint32_t)wp * (16u * kChunkScaleBytes)), 0, kAuxStream);
        if constexpr (!LDSX) {
            const int kc = kGroupedWindow * wp + kChunkK * j;   // first k of the lane's chunk
#pragma unroll
            for (int m = 0; m < MR; m++)
#pragma unroll
                for (int p = 0; p < 4; p++) {
                    const bool xv = live && m < pit.rows && kc + 8 * p < K;
                    u.x[m][p] = __builtin_amdgcn_raw_buffer_load_b128(
                        rx, off_if(xv, ((uint32_t)m * (uint32_t)K + (uint32_t)(kc + 8 * p)) * 2u),
                        0, kAuxNormal);
                }
        }
        if (++wp == nwin) {
            wp = 0;
            if (++ip < i1) {
                item_next(pit);
                set_sources();
            }
        }
        return u;
    };

    GroupedUnit<MR, LDSX> ring[D];
    if (i0 < i1) {
#pragma unroll
        for (int s = 0; s < D - 1; s++)
            ring[s] = load_next();
    }

    // LDSX: stage the rows of the chunks [cfirst, clast] this workgroup's items touch.
    const int row_bytes = nwin * (kGroupedWindow / kChunkK) * kGroupedSlot;
    int cfirst = 0;
    if constexpr (LDSX) {
        const long long I0 = items * ((long long)blockIdx.x * W) / V;
        const long long I1 = items * ((long long)(blockIdx.x + 1) * W) / V;
        if (I0 < I1) {
            cfirst = (int)(I0 / NG);
            const int nch = min((int)((I1 - 1) / NG) - cfirst + 1, xrows / MR);
            int *srow = reinterpret_cast<int *>(xlds + (size_t)xrows * row_bytes);
            for (int t = threadIdx.x; t < nch * MR; t += kWave * W) {
                const Item it = item_at((long long)(cfirst + t / MR) * NG);
                srow[t] = (t % MR) < it.rows ? it.row0 + t % MR : -1;
            }
            __syncthreads();
            const int row_pieces = nwin * (kGroupedWindow / 8);   // 16-byte pieces per row
            for (int idx = threadIdx.x; idx < nch * MR * row_pieces; idx += kWave * W) {
                const int t = idx / row_pieces;
                const int e = idx - t * row_pieces;
                const int row = srow[t];
                u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
                if (row >= 0 && 8 * e < K)
                    v = *reinterpret_cast<const u32x4_t *>(a.X + (size_t)row * K + 8 * e);
                *reinterpret_cast<u32x4_t *>(xlds + (size_t)t * row_bytes +
                                             (e >> 2) * kGroupedSlot + 16 * (e & 3)) = v;
            }
        }
        __syncthreads();
    }
    if (i0 >= i1)
        return;

    // Compute cursor: item ic (described by cit), window wc.
    long long ic = i0;
    int wc = 0;
    Item cit = item_at(ic);
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; m++)
        acc[m] = 0.0f;
    const long long units = (i1 - i0) * nwin;
    for (long long u = 0; u < units; u += D) {
#pragma unroll
        for (int s = 0; s < D; s++) {
            ring[(s + D - 1) % D] = load_next();
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
            if (u + s < units) {
                const GroupedUnit<MR, LDSX> &c = ring[s];
                const uint32_t sc = c.scale >> sshift;
                const float s0 = e4m3_to_f32<0>(sc);
                const float s1 = e4m3_to_f32<1>(sc);
                bf16x2_t w[16];
                decode32_bf16(c.code, w);
#pragma unroll
                for (int m = 0; m < MR; m++) {
                    // Rows past the chunk's last (an expert with fewer rows than MR) cost
                    // nothing: the weights are decoded once for the rows there are.
                    if (m > 0 && m >= cit.rows)
                        break;
                    u32x4_t xv[4];
                    if constexpr (LDSX) {
                        // row m of the item's chunk, window wc, the lane's 32-k chunk j
                        const uint8_t *xp = xlds +
                                            (size_t)((cit.slot - cfirst) * MR + m) * row_bytes +
                                            ((uint32_t)wc * 16u + (uint32_t)j) * kGroupedSlot;
#pragma unroll
                        for (int p = 0; p < 4; p++)
                            xv[p] = *reinterpret_cast<const u32x4_t *>(xp + 16 * p);
                    } else {
#pragma unroll
                        for (int p = 0; p < 4; p++)
                            xv[p] = c.x[m][p];
                    }
                    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        p0 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xv[i / 4][i % 4]),
                                                              p0, false);
#pragma unroll
                    for (int i = 8; i < 16; i++)
                        p1 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xv[i / 4][i % 4]),
                                                              p1, false);
                    acc[m] = __builtin_fmaf(p0, s0, acc[m]);
                    acc[m] = __builtin_fmaf(p1, s1, acc[m]);
                }
                if (++wc == nwin) {
                    // Item done: sum the 16 lanes of each column, times the expert's g.
                    const float g = a.gscale[cit.e];
                    const int n = kGroupCols * cit.grp + col;
#pragma unroll
                    for (int m = 0; m < MR; m++) {
                        const float v = sum_lanes_stride4(acc[m]);
                        acc[m] = 0.0f;
                        if (j == 0 && m < cit.rows && n < N)
                            a.Y[(size_t)(cit.row0 + m) * (size_t)N + n] = v * g;
                    }
                    wc = 0;
                    if (++ic < i1)
                        item_next(cit);
                }
            }
        }
    }
}

}  // namespace nvfp4

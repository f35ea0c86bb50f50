// gemv_stream.h -- persistent NVFP4 x bf16 dot-product kernel for the smallest M (decode).
//
// Decode at concurrency 1 reads every weight once per token and is bound by that read
// ("Qwen3.8-27B-NVFP4-RTX5090" model card, section "Why lm_head is NVFP4"). A streaming kernel
// reaches the HBM roof only if every compute unit keeps the same number of bytes in flight until
// the very end, so the work is split evenly by construction instead of by tile count:
//
//   * One workgroup of W wavefronts per compute unit (two for one row of a large weight: the
//     launcher's choice). With NG = q G + r 4-column groups,
//     workgroup b owns q + (b < r) consecutive groups from b q + min(b, r), so all hold the same
//     number of weight bytes (to within one group).
//   * A unit is one (group, 512-k window) pair: 16 chunks of 32 k x 4 columns, 1 KB of codes in
//     one contiguous piece of the packed layout. Lane l of a wavefront reads its 16 bytes at
//     16 l: column l % 4 of the group, chunk l / 4 of the window. The units of a workgroup,
//     ordered group-major, are dealt to the W wavefronts in W contiguous runs, shorter for the
//     second and later wavefronts of a SIMD, which the hardware serves later
//     (stream_run_start).
//   * X (all M rows, all of K) is staged once in LDS, so the weight loads are the only global
//     traffic of the loop. Each 32-k chunk of X sits in an 80-byte slot; the 16 chunks a
//     wavefront reads at once then fall into different bank groups, and each is broadcast to the
//     4 lanes of its column quad.
//   * A wavefront keeps D units in flight (a ring of D register sets filled through buffer loads
//     that return zeros past the end), accumulates its run in registers, and when the group
//     changes sums the 16 lanes of each column and writes the column partial to an LDS slot. A
//     group is split between at most L.slots consecutive wavefronts; the slots are added in
//     wavefront order (= k order) at the end, times the tensor scale g. Results are reproducible.
//   * FAST (K % 512 == 0) needs no per-lane K test; otherwise a lane whose chunk is past the
//     last one reads zeros instead of the next group's bytes.
//   * The set-up before the first weight load is kept short: a wavefront issues about one
//     instruction per four cycles, and every instruction before the loads delays the first
//     bytes. The launcher passes the split of the groups and 1 / nwin, so the set-up has no
//     64-bit and no generic integer division.
#pragma once

#include "argmax.h"
#include "device.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kStreamWindow = 512;
constexpr int kStreamSlot = 80;   // LDS bytes per 32-k chunk of X (64 used)

// LDS layout of the persistent kernel, computed by the launcher (which also sizes the dynamic
// LDS) and read by the kernel.
struct StreamLayout {
    int nwin;        // ceil(K / 512)
    int row_bytes;   // LDS bytes of one X row: 16 nwin chunks of kStreamSlot bytes
    int ngroups;     // most column groups of 4 any workgroup owns
    int slots;       // most wavefronts one group is split over
    int x_bytes;     // M * row_bytes
    int part_bytes;  // ngroups * slots * MR * 4 floats
    int gq, gr;      // NG = gunit (gq G + gr): workgroup b owns gunit (gq + (b < gr)) groups
    float rnwin;     // 1.0f / nwin
    int gunit;       // groups dealt together: 2 keeps the gate/up pairs of a workgroup whole
};

// Share of the units per wavefront. Wavefront w runs on SIMD w % 4, as the (w / 4)-th
// wavefront there; a SIMD's later wavefronts end their runs later (measured on gate_up at one
// row, 12 wavefronts of equal runs: the second and third of a SIMD 0.6-1.0 and 1.0-1.5 us after
// the first), so they get shorter runs: weight 32 - 2 (w / 4). C(w) is the weight of wavefronts
// 0 .. w - 1; with one wavefront per SIMD (W <= 4) the split is the plain even one.
__host__ __device__ inline uint32_t stream_weight_before(int w)
{
    const uint32_t f = (uint32_t)w >> 2, r = (uint32_t)w & 3u;
    return 4u * (32u * f - f * (f - 1u)) + r * (32u - 2u * f);
}

// First unit of wavefront w's run, of `units` < 2^21 units dealt to W <= 16 wavefronts.
__host__ __device__ inline int stream_run_start(int w, int W, uint32_t units)
{
    if (W <= 4)
        return (int)(((uint32_t)w * units) / (uint32_t)W);
    return (int)((stream_weight_before(w) * units) / stream_weight_before(W));
}

// The wavefront of the W whose run holds unit u.
inline int stream_owner(long long u, int W, long long units)
{
    int w = 0;
    while (w + 1 < W && stream_run_start(w + 1, W, (uint32_t)units) <= u)
        w++;
    return w;
}

// floor(x / d) for x < 2^22, given rd = 1.0f / d rounded to nearest. The float estimate is within
// one of the quotient and is corrected with the exact remainder.
__device__ __forceinline__ uint32_t div_small(uint32_t x, uint32_t d, float rd)
{
    uint32_t q = (uint32_t)((float)x * rd);
    const int r = (int)(x - q * d);
    if (r < 0)
        q--;
    else if (r >= (int)d)
        q++;
    return q;
}

template <int MR, int W, int D, bool FAST>
__global__ __launch_bounds__(kWave *W) void gemv_stream_kernel(GemmArgs a, StreamLayout L)
{
    extern __shared__ __align__(16) uint8_t lds[];
    float *part = reinterpret_cast<float *>(lds + L.x_bytes);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int col = lane & 3;   // column within the group
    const int j = lane >> 2;    // chunk within the window
    const int K = a.K;
    const int N = a.N;
    const int CH = num_chunks(K);
    const int b = blockIdx.x;
    const int g0 = L.gunit * (b * L.gq + min(b, L.gr));
    const int ngroups = L.gunit * (L.gq + (b < L.gr ? 1 : 0));
    const int c0 = kGroupCols * g0;
    const int ncols = min(N - c0, kGroupCols * ngroups);
    const int nwin = L.nwin;
    const uint32_t units = (uint32_t)ngroups * (uint32_t)nwin;   // < 2^21
    auto run_start = [&](int w) { return stream_run_start(w, W, units); };
    const int u0 = run_start(wave);
    const int u1 = run_start(wave + 1);
    const int gstart = (int)div_small((uint32_t)u0, (uint32_t)nwin, L.rnwin);

    const uint32_t gq = (uint32_t)CH * kChunkCodeBytes;    // code bytes per group
    const uint32_t gs = (uint32_t)CH * kChunkScaleBytes;   // scale bytes per group
    const rsrc_t rq = make_rsrc(a.Wq + (size_t)g0 * gq, (uint32_t)ngroups * gq);
    const rsrc_t rs = make_rsrc(a.Ws + (size_t)g0 * gs, (uint32_t)ngroups * gs);
    // Within a unit: the lane's 16 code bytes, and the 4-byte word holding its 2 scale bytes
    // (at 2 lane) together with those of lane ^ 1.
    const uint32_t vq = 16u * (uint32_t)lane;
    const uint32_t vs = 4u * (uint32_t)(lane >> 1);
    const uint32_t sshift = 16u * (uint32_t)(lane & 1);

    // Prefetch cursor: unit up = (gp, wp).
    int up = u0;
    int gp = gstart;
    int wp = u0 - gp * nwin;
    auto load_next = [&]() -> Chunk {
        Chunk c;
        const bool live = up < u1 && (FAST || kStreamWindow / kChunkK * wp + j < CH);
        const uint32_t uq = (uint32_t)gp * gq + (uint32_t)wp * (16u * kChunkCodeBytes);
        const uint32_t us = (uint32_t)gp * gs + (uint32_t)wp * (16u * kChunkScaleBytes);
        const u32x4_t v =
            __builtin_amdgcn_raw_buffer_load_b128(rq, off_if(live, vq + uq), 0, kAuxStream);
        c.code[0] = v[0];
        c.code[1] = v[1];
        c.code[2] = v[2];
        c.code[3] = v[3];
        c.scale = __builtin_amdgcn_raw_buffer_load_b32(rs, off_if(live, vs + us), 0, kAuxStream);
        up++;
        if (++wp == nwin) {
            wp = 0;
            gp++;
        }
        return c;
    };

    // Prologue. The X loads go first: loads retire in issue order, so the wait for X before the
    // LDS store must not also wait for the weights. Then the first D - 1 units of weights, so
    // that the stream is running while X lands in LDS and the workgroup synchronises.
    const rsrc_t rx = make_rsrc(a.X, (uint32_t)a.M * (uint32_t)K * 2u);
    const int row_pieces = nwin * (kStreamWindow / 8);  // 16-byte pieces per padded row
    const int xpieces = a.M * row_pieces;
    constexpr int kXPerThread = 4;                       // X pieces loaded ahead per thread
    u32x4_t xv0[kXPerThread];
#pragma unroll
    for (int i = 0; i < kXPerThread; i++) {
        const int idx = threadIdx.x + i * kWave * W;
        const int m = MR == 1 ? 0 : (int)div_small((uint32_t)idx >> 6, (uint32_t)nwin, L.rnwin);
        const int e = idx - m * row_pieces;
        const uint32_t src = ((uint32_t)m * (uint32_t)K + (uint32_t)e * 8u) * 2u;
        xv0[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rx, off_if(idx < xpieces && 8 * e < K, src), 0, kAuxNormal);
    }
    Chunk ring[D];
#pragma unroll
    for (int s = 0; s < D - 1; s++)
        ring[s] = load_next();

    // X into LDS (zeros past K), then the remaining pieces if X is larger, and clear the slots.
#pragma unroll
    for (int i = 0; i < kXPerThread; i++) {
        const int idx = threadIdx.x + i * kWave * W;
        if (idx < xpieces) {
            const int m =
                MR == 1 ? 0 : (int)div_small((uint32_t)idx >> 6, (uint32_t)nwin, L.rnwin);
            const int e = idx - m * row_pieces;
            *reinterpret_cast<u32x4_t *>(lds + m * L.row_bytes + (e >> 2) * kStreamSlot +
                                         16 * (e & 3)) = xv0[i];
        }
    }
    for (int idx = threadIdx.x + kXPerThread * kWave * W; idx < xpieces; idx += kWave * W) {
        const int m = (int)div_small((uint32_t)idx >> 6, (uint32_t)nwin, L.rnwin);
        const int e = idx - m * row_pieces;
        const uint32_t src = ((uint32_t)m * (uint32_t)K + (uint32_t)e * 8u) * 2u;
        const u32x4_t v =
            __builtin_amdgcn_raw_buffer_load_b128(rx, off_if(8 * e < K, src), 0, kAuxNormal);
        *reinterpret_cast<u32x4_t *>(lds + m * L.row_bytes + (e >> 2) * kStreamSlot +
                                     16 * (e & 3)) = v;
    }
    {
        const int nslots = L.ngroups * L.slots * MR * 4;
        for (int idx = threadIdx.x; idx < nslots; idx += kWave * W)
            part[idx] = 0.0f;
    }
    __syncthreads();

    if (a.gamma != nullptr) {
        // RMSNorm of the staged rows: per row r = 1 / sqrt(mean x^2 + eps); every x becomes
        // bf16((x * r) * gamma[k]) in place. The sum of squares: each thread adds its 8-value
        // pieces in order (fma), then a fixed butterfly over the wavefront, then the wavefronts in
        // order; its relative error stays below (K / 64 + 32) 2^-24.
        __shared__ float nss[W][MR];
        __shared__ float nr[MR];
        float ss[MR];
#pragma unroll
        for (int m = 0; m < MR; m++)
            ss[m] = 0.0f;
        auto piece = [&](int idx, int *m, int *e) {
            *m = MR == 1 ? 0 : (int)div_small((uint32_t)idx >> 6, (uint32_t)nwin, L.rnwin);
            *e = idx - *m * row_pieces;
        };
        for (int idx = threadIdx.x; idx < xpieces; idx += kWave * W) {
            int m, e;
            piece(idx, &m, &e);
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
                lds + m * L.row_bytes + (e >> 2) * kStreamSlot + 16 * (e & 3));
            float t = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float lo = __uint_as_float(v[i] << 16);
                const float hi = __uint_as_float(v[i] & 0xFFFF0000u);
                t = __builtin_fmaf(lo, lo, t);
                t = __builtin_fmaf(hi, hi, t);
            }
#pragma unroll
            for (int mm = 0; mm < MR; mm++)
                if (mm == m)
                    ss[mm] += t;
        }
#pragma unroll
        for (int m = 0; m < MR; m++) {
            float t = ss[m];
#pragma unroll
            for (int d = kWave / 2; d >= 1; d >>= 1)
                t += __shfl_xor(t, d);
            if (lane == 0)
                nss[wave][m] = t;
        }
        __syncthreads();
        if (threadIdx.x < MR) {
            float t = 0.0f;
            for (int w = 0; w < W; w++)
                t += nss[w][threadIdx.x];
            nr[threadIdx.x] = 1.0f / __builtin_sqrtf(t / (float)K + a.eps);
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < xpieces; idx += kWave * W) {
            int m, e;
            piece(idx, &m, &e);
            if (8 * e >= K)
                continue;   // padding stays zero
            u32x4_t *p = reinterpret_cast<u32x4_t *>(lds + m * L.row_bytes +
                                                     (e >> 2) * kStreamSlot + 16 * (e & 3));
            const u32x4_t v = *p;
            const u32x4_t gm = *reinterpret_cast<const u32x4_t *>(a.gamma + 8 * e);
            const float r = nr[m];
            u32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float x0 = __uint_as_float(v[i] << 16) * r;
                const float x1 = __uint_as_float(v[i] & 0xFFFF0000u) * r;
                bf16x2_t y;
                y[0] = (__bf16)(x0 * __uint_as_float(gm[i] << 16));
                y[1] = (__bf16)(x1 * __uint_as_float(gm[i] & 0xFFFF0000u));
                o[i] = __builtin_bit_cast(uint32_t, y);
            }
            *p = o;
        }
        __syncthreads();
    }

    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; m++)
        acc[m] = 0.0f;
    // Compute cursor: unit uc = (gc, wc); slot of the current group for this wavefront.
    int gc = gstart;
    int wc = u0 - gc * nwin;
    // Slot = number of earlier wavefronts whose runs reach into group gc.
    int slot = 0;
    for (int w = wave; w > 0 && run_start(w) > gc * nwin; w--)
        slot++;
    const uint32_t xlane = (uint32_t)j * kStreamSlot;

    auto flush = [&]() {
#pragma unroll
        for (int m = 0; m < MR; m++) {
            const float v = sum_lanes_stride4(acc[m]);
            acc[m] = 0.0f;
            if (j == 0)
                part[((gc * L.slots + slot) * MR + m) * 4 + col] = v;
        }
    };

    for (int u = u0; u < u1; u += D) {
#pragma unroll
        for (int s = 0; s < D; s++) {
            ring[(s + D - 1) % D] = load_next();
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
            if (u + s < u1) {
                const Chunk &c = ring[s];
                const uint32_t sc = c.scale >> sshift;
                const float s0 = e4m3_to_f32<0>(sc);
                const float s1 = e4m3_to_f32<1>(sc);
                bf16x2_t w[16];
                decode32_bf16(c.code, w);
                const uint8_t *xb = lds + xlane + (uint32_t)wc * (16u * kStreamSlot);
#pragma unroll
                for (int m = 0; m < MR; m++) {
                    const uint8_t *xm = xb + (m < a.M ? m : 0) * L.row_bytes;
                    u32x4_t xv[4];
#pragma unroll
                    for (int p = 0; p < 4; p++)
                        xv[p] = *reinterpret_cast<const u32x4_t *>(xm + 16 * p);
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
                    flush();
                    wc = 0;
                    gc++;
                    slot = 0;
                }
            }
        }
    }
    if (u0 < u1 && wc != 0)
        flush();  // the run ended inside a group
    __syncthreads();

    const float g = *a.gscale;
    if (a.H != nullptr) {
        // SiLU(gate) * up: the workgroup owns whole pairs of groups (gate group 2p, up group
        // 2p + 1; c0 is a multiple of 8), so column c's partner is c + 4.
        const int I = N >> 1;
        for (int m = 0; m < a.M && m < MR; m++)
            for (int pidx = threadIdx.x; pidx < (ncols >> 1); pidx += kWave * W) {
                const int c = 8 * (pidx >> 2) + (pidx & 3);
                float sg = 0.0f, su = 0.0f;
                for (int sl = 0; sl < L.slots; sl++) {
                    sg += part[(((c >> 2) * L.slots + sl) * MR + m) * 4 + (c & 3)];
                    su += part[((((c >> 2) + 1) * L.slots + sl) * MR + m) * 4 + (c & 3)];
                }
                const float gate = sg * g, up = su * g;
                const float h = gate / (1.0f + __expf(-gate)) * up;
                a.H[(size_t)m * I + (c0 >> 1) + 4 * (pidx >> 2) + (pidx & 3)] =
                    __builtin_bit_cast(uint16_t, (__bf16)h);
            }
        return;
    }
#pragma unroll
    for (int m = 0; m < MR; m++) {
        if (m >= a.M)
            break;
        argkey_t best = 0;
        for (int c = threadIdx.x; c < ncols; c += kWave * W) {
            const int grp = c >> 2;
            float sum = 0.0f;
            for (int sl = 0; sl < L.slots; sl++)
                sum += part[((grp * L.slots + sl) * MR + m) * 4 + (c & 3)];
            if (a.keys == nullptr)
                a.Y[(size_t)m * N + c0 + c] = sum * g;
            else
                best = key_max(best, argmax_key(sum * g, c0 + c));
        }
        if (a.keys != nullptr) {
            // Argmax mode: one key per row and workgroup (slot b of the row): the wavefronts'
            // keys meet in LDS, so the finalize kernel reads one key per compute unit.
            __shared__ argkey_t wkeys[W];
            best = key_max_64(best);
            if (lane == 0)
                wkeys[wave] = best;
            __syncthreads();
            if (threadIdx.x == 0) {
                argkey_t k = wkeys[0];
                for (int w = 1; w < W; w++)
                    k = key_max(k, wkeys[w]);
                a.keys[(size_t)m * a.key_slots + b] = k;
            }
            __syncthreads();   // wkeys is reused by the next row
        }
    }
}

}  // namespace nvfp4

// gemv_stream.h -- persistent NVFP4 x bf16 dot-product kernel for the smallest M (decode).
//
// Decode at concurrency 1 reads every weight once per token and is bound by that read
// ("Qwen3.8-27B-NVFP4-RTX5090" model card, section "Why lm_head is NVFP4"). A streaming kernel
// reaches the HBM roof only if every compute unit keeps the same number of bytes in flight until
// the very end, so the work is split evenly by construction instead of by tile count:
//
//   * One workgroup of W wavefronts per compute unit. Workgroup b owns the output columns
//     [b N / G, (b + 1) N / G) of the G workgroups, so all hold the same number of weight bytes
//     (to within one column).
//   * Its columns are cut into groups of 4 and K into windows of 512; a unit is one (group,
//     window) pair: quad q (16 lanes) of a wavefront reads 256 contiguous bytes of column 4 g + q,
//     lane r the 32 k = 512 w + 32 r .. + 31 of it. The units, ordered group-major, are dealt to
//     the W wavefronts in W contiguous runs of equal length (to within one unit).
//   * X (all M rows, all of K) is staged once in LDS, so the weight loads are the only global
//     traffic of the loop. Each 64-byte lane chunk sits in an 80-byte slot: eight consecutive
//     lanes then read eight different bank groups, and the four 16-byte pieces of a chunk are
//     immediate offsets of one address.
//   * A wavefront keeps D units in flight (a ring of D register sets filled through buffer loads
//     that return zeros past the end), accumulates its run in registers, and when the group
//     changes sums the 16 lanes of each quad and writes the column partial to an LDS slot. A
//     group is split between at most L.slots consecutive wavefronts; the slots are added in
//     wavefront order (= k order) at the end, times the tensor scale g. Results are reproducible.
//   * FAST (K % 512 == 0, hence the wide layout) needs no per-lane K test: every load offset is a
//     per-lane constant plus one wavefront-uniform term. Otherwise each lane checks its k range.
#pragma once

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
};

// First wavefront of the W whose run [u0(w), u0(w+1)), u0(w) = floor(w units / W), holds unit u.
__host__ __device__ inline int stream_owner(long long u, int W, long long units)
{
    return (int)(((u + 1) * W - 1) / units);
}

template <int MR, int W, int D, bool FAST, bool NARROW>
__global__ __launch_bounds__(kWave *W) void gemv_stream_kernel(GemmArgs a, StreamLayout L)
{
    extern __shared__ __align__(16) uint8_t lds[];
    float *part = reinterpret_cast<float *>(lds + L.x_bytes);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int G = gridDim.x;
    const int c0 = (int)(((long long)blockIdx.x * N) / G);
    const int ncols = (int)(((long long)(blockIdx.x + 1) * N) / G) - c0;
    const int ngroups = (ncols + 3) / 4;
    const int nwin = L.nwin;
    const long long units = (long long)ngroups * nwin;
    const int u0 = (int)(((long long)wave * units) / W);
    const int u1 = (int)(((long long)(wave + 1) * units) / W);

    const rsrc_t rq = make_rsrc(a.Wq + (size_t)c0 * (size_t)(K / 2),
                                (uint32_t)ncols * (uint32_t)(K / 2));
    uint32_t sbias;
    const rsrc_t rs = scale_rsrc(a.Ws, (size_t)c0, ncols, K, &sbias);
    const uint32_t qrow = (uint32_t)q * (uint32_t)(K / 2);           // this quad's column,
    const uint32_t srow = sbias + (uint32_t)q * (uint32_t)(K / 16);  // relative to group 0
    const uint32_t gq = 4u * (uint32_t)(K / 2);                       // bytes per group
    const uint32_t gs = 4u * (uint32_t)(K / 16);
    // FAST: the lane's offsets within a window are constants; the scale word holds lanes 2 p and
    // 2 p + 1 (K % 64 == 0 makes srow a multiple of 4 and sbias zero).
    const uint32_t vq = qrow + 16u * (uint32_t)r;
    const uint32_t vs = srow + 4u * (uint32_t)(r >> 1);
    const uint32_t sshift = 16u * (uint32_t)(r & 1);

    // Prefetch cursor: unit up = (gp, wp).
    int up = u0;
    int gp = u0 / nwin;
    int wp = u0 - gp * nwin;
    auto load_next = [&]() -> Chunk {
        Chunk c;
        const bool live = up < u1;
        if (FAST) {
            const uint32_t uq = live ? (uint32_t)gp * gq + (uint32_t)wp * 256u : kOutOfRange;
            const uint32_t us = live ? (uint32_t)gp * gs + (uint32_t)wp * 32u : kOutOfRange;
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rq, vq + uq, 0, kAuxStream);
            c.code[0] = v[0];
            c.code[1] = v[1];
            c.code[2] = v[2];
            c.code[3] = v[3];
            c.scale = __builtin_amdgcn_raw_buffer_load_b32(rs, vs + us, 0, kAuxStream);
        } else {
            const int kc = live ? wp * kStreamWindow + 32 * r : K;  // K: zeros
            c = load_chunk<NARROW>(rq, rs, qrow + (uint32_t)gp * gq, srow + (uint32_t)gp * gs,
                                   kc, K);
        }
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
        const int m = idx / row_pieces;
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
            const int m = idx / row_pieces;
            const int e = idx - m * row_pieces;
            *reinterpret_cast<u32x4_t *>(lds + m * L.row_bytes + (e >> 2) * kStreamSlot +
                                         16 * (e & 3)) = xv0[i];
        }
    }
    for (int idx = threadIdx.x + kXPerThread * kWave * W; idx < xpieces; idx += kWave * W) {
        const int m = idx / row_pieces;
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

    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; m++)
        acc[m] = 0.0f;
    // Compute cursor: unit uc = (gc, wc); slot of the current group for this wavefront.
    int gc = u0 / nwin;
    int wc = u0 - gc * nwin;
    int slot = (gc * nwin >= u0) ? 0 : wave - stream_owner((long long)gc * nwin, W, units);
    const uint32_t xlane = (uint32_t)r * kStreamSlot;

    auto flush = [&]() {
#pragma unroll
        for (int m = 0; m < MR; m++) {
            float v = acc[m];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            acc[m] = 0.0f;
            if (r == 0)
                part[((gc * L.slots + slot) * MR + m) * 4 + q] = v;
        }
    };

    for (int u = u0; u < u1; u += D) {
#pragma unroll
        for (int s = 0; s < D; s++) {
            ring[(s + D - 1) % D] = load_next();
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
            if (u + s < u1) {
                const Chunk &c = ring[s];
                const uint32_t sc =
                    FAST ? (c.scale >> sshift)
                         : scale_pair<NARROW>(c.scale, srow + (uint32_t)gc * gs,
                                              wc * kStreamWindow + 32 * r);
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
    for (int idx = threadIdx.x; idx < ncols * MR; idx += kWave * W) {
        const int m = idx / ncols;
        const int c = idx - m * ncols;
        if (m < a.M) {
            const int grp = c / 4;
            float sum = 0.0f;
            for (int sl = 0; sl < L.slots; sl++)
                sum += part[((grp * L.slots + sl) * MR + m) * 4 + (c & 3)];
            a.Y[(size_t)m * N + c0 + c] = sum * g;
        }
    }
}

}  // namespace nvfp4

/*
 * nvfp4.h -- C ABI of libnvfp4.so, the MI355X (gfx950) NVFP4 skinny-GEMM library.
 *
 * The library computes the decode / speculative-verify hot path of a single-model LLM engine:
 *
 *     Y[M,N] = X[M,K] . dequant(W)[K,N]
 *
 * with NVFP4 weights, bf16 activations, fp32 accumulation and fp32 output. M is small: 1 for
 * plain decode, 16 for the verify pass of one request with 15 drafted tokens, 128 when 8 requests
 * verify together ("SparkInfer" README, sections on speculative decoding and on up to eight
 * concurrent requests speculating together). Decode at concurrency 1 is bound by the weight
 * stream: every weight is read once per token ("Qwen3.8-27B-NVFP4-RTX5090" model card, section
 * "Why lm_head is NVFP4"). The weights are "NVFP4 W4A4, group size 16" stored as packed U8
 * tensors (same model card, table "Recipe (NVIDIA ModelOpt)" and section "Serving"); this library
 * keeps activations in bf16 (W4A16).
 *
 * NVFP4 as stored here
 *   - code: FP4 E2M1 (OCP MX v1.0): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 *     values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.
 *   - block scale: one FP8 E4M3 byte (OCP OFP8 "E4M3FN": bias 7, max 448, NaN = 0x7F/0xFF) per 16
 *     consecutive k of one output column n.
 *   - tensor scale g: one fp32 per weight matrix.
 *   - dequantised weight: w(k,n) = e2m1(code(k,n)) * e4m3(Ws[n][k/16]) * g.
 *
 * Layout (row-major: element (i,j) of an [R][C] array sits at offset i*C + j)
 *   W      fp32  [K][N]             input of nvfp4_pack
 *   Wq     uint8 [NG][CH][4][16]    codes, NG = ceil(N/4) groups of 4 columns, CH = ceil(K/32)
 *                                   chunks of 32 k: byte (g, c, j, i) holds the codes of column
 *                                   n = 4g + j at k = 32c + 2i (bits 3..0) and k = 32c + 2i + 1
 *                                   (bits 7..4)
 *   Wscale uint8 [NG][CH][4][2]     E4M3 scales: byte (g, c, j, b) is the scale of column 4g + j,
 *                                   block k/16 = 2c + b
 *   gscale fp32  [1]                g, in device memory
 *   X      bf16  [M][K]             passed as uint16_t bit patterns
 *   Y      fp32  [M][N]             fully overwritten
 * Bytes of columns n >= N and of k >= K (the padding up to 4 columns and 32 k) are zero, as
 * nvfp4_pack writes them; nvfp4_codes_bytes / nvfp4_scales_bytes give the array sizes.
 * Why this order: one 32-k chunk of 4 adjacent columns is 64 contiguous bytes, so the 16 chunks
 * of a 512-k window of a group are 1 KB in one piece (one 16-byte load per lane of a wavefront,
 * whole 128-byte lines), and a 16-column x 128-k tile is four 256-byte pieces; both kinds of
 * kernel read only whole cache lines. Scales follow the same order at 2 bytes per (column, chunk).
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer owned by the caller; the library keeps none of them past
 *     the call.
 *   - The library owns no device memory: every partial sum stays inside a workgroup (in
 *     registers and LDS), and the entry points that need scratch memory take it from the caller
 *     (nvfp4_gemm_argmax, nvfp4_gemm_fused), so a call never allocates, and calls on different
 *     streams or host threads never share memory unless the caller gives them the same buffers.
 *   - Sizes: 1 <= M, 1 <= N, 16 <= K <= 4194304 (2^22), K % 16 == 0, and every array must have
 *     fewer than 2^62 bytes. Anything else returns NVFP4_ERROR_INVALID_VALUE.
 *   - Alignment: X, Wq, Wscale and W must be 16-byte aligned, Y and gscale 4-byte aligned;
 *     otherwise NVFP4_ERROR_MISALIGNED. K % 512 == 0 takes the fastest loads; any K % 16 == 0 is
 *     correct.
 *   - Y must not overlap any input. Outputs of nvfp4_pack must not overlap W or each other.
 *   - Validation happens on the host before any HIP call: an error return has no side effects.
 *   - Calls are stream-ordered on `stream` (a hipStream_t; NULL is the null stream) and never
 *     synchronise. A failed kernel launch returns NVFP4_ERROR_LAUNCH; faults during execution
 *     surface at the caller's next synchronisation, as for any HIP kernel.
 *   - Results are deterministic: the same inputs give the same bits on every call, on any
 *     stream, eagerly or inside a captured graph.
 *   - Calls are re-entrant and thread-safe on the host. The only mutable global state is a
 *     per-device cache of the compute-unit count and of which kernels were allowed more LDS,
 *     both behind atomics or a mutex.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_SUCCESS = 0,
    NVFP4_ERROR_INVALID_VALUE = 1,  /* bad size, null pointer or unknown path */
    NVFP4_ERROR_MISALIGNED = 2,     /* a pointer breaks the alignment rules above */
    NVFP4_ERROR_LAUNCH = 3,         /* the HIP runtime refused a kernel launch */
    NVFP4_ERROR_SCRATCH_LIMIT = 4,  /* more rows than nvfp4_gemm_argmax_noalloc's scratch holds */
    /* Not statuses: they make the type span every int, so that any int a caller passes to
     * nvfp4_status_string is a valid value of it (a C++ enumeration only holds the values its
     * enumerators' bits can express). */
    NVFP4_STATUS_ENUM_MIN_ = -2147483647 - 1,
    NVFP4_STATUS_ENUM_MAX_ = 2147483647
} nvfp4_status_t;

/*
 * nvfp4_pack -- quantise fp32 W[K][N] to NVFP4 (codes Wq, block scales Wscale, tensor scale).
 *
 * The recipe of the workloads: g = amax(|W|) / (6*448); per block of 16 consecutive k of column n,
 * s = E4M3(block_amax / (6g)); code = E2M1(w / (s*g)). Each step is one fp32 operation rounded to
 * nearest-even, in that order (6*g is rounded before the division; s*g before w/(s*g)); both
 * roundings to E4M3 and E2M1 go to the nearest value, ties to the even code, saturating at 448 and
 * at 6. A tensor with g == 0 packs to all-zero bytes; a block whose s*g is 0 gets all-zero codes.
 * The page's checkpoint was quantised this way offline with NVIDIA ModelOpt ("Qwen3.8-27B-NVFP4-
 * RTX5090" model card, table "Recipe (NVIDIA ModelOpt)"); here it is the untimed set-up step.
 *
 *   K, N    sizes of W (K % 16 == 0)
 *   W       in:  fp32 [K][N], device
 *   Wq      out: uint8 [NG][CH][4][16] (nvfp4_codes_bytes(N, K) bytes), device; padding zeroed
 *   Wscale  out: uint8 [NG][CH][4][2] (nvfp4_scales_bytes(N, K) bytes), device; padding zeroed
 *   gscale  out: fp32 [1], device; it also holds the running amax while the call executes
 *   stream  hipStream_t
 */
nvfp4_status_t nvfp4_pack(int K, int N, const float *W, uint8_t *Wq, uint8_t *Wscale,
                          float *gscale, void *stream);

/*
 * nvfp4_gemm -- Y = X . dequant(Wq, Wscale, *gscale), fp32 accumulation, fp32 output.
 *
 * Each weight is decoded to the exact value e2m1(code) * e4m3(scale) (at most 6 significant bits,
 * so exact in bf16 and fp32); products with x are accumulated in fp32 and g is applied once to
 * each finished output. The tolerance the results meet against a double-precision sum is
 * |Y - Y_ref| <= 2e-3 * sum_k |x*w| + 1e-6 per output. The kernel is chosen from (M, N, K): a
 * wavefront dot product for the smallest M and bf16 MFMA tiles otherwise.
 *
 *   M, N, K  sizes (K % 16 == 0)
 *   X        in:  bf16 bits [M][K], device
 *   Wq       in:  uint8 [NG][CH][4][16], device (as written by nvfp4_pack, padding zero)
 *   Wscale   in:  uint8 [NG][CH][4][2], device
 *   gscale   in:  fp32 [1], device (read by the kernel; the host never reads it)
 *   Y        out: fp32 [M][N], device
 *   stream   hipStream_t
 */
nvfp4_status_t nvfp4_gemm(int M, int N, int K, const uint16_t *X, const uint8_t *Wq,
                          const uint8_t *Wscale, const float *gscale, float *Y, void *stream);

/* Kernel families nvfp4_gemm chooses between (for nvfp4_gemm_path). All are persistent: one
 * workgroup per compute unit (per 16-row block of X for NVFP4_PATH_MFMA; per row group and tile
 * set for NVFP4_PATH_BATCH), each with an equal share of the 4-column groups. nvfp4_gemm takes
 * DOT for M <= 4, MFMA for M <= 16 (and narrow weights up to M = 48) and BATCH above. */
typedef enum {
    NVFP4_PATH_AUTO = 0,  /* what nvfp4_gemm does */
    NVFP4_PATH_DOT = 1,   /* VALU: E2M1->bf16 decode, v_dot2_f32_bf16 against X staged in LDS,
                             fp32 partial * s; M <= 8 */
    NVFP4_PATH_MFMA = 2,  /* matrix cores: E2M1*s decoded to bf16, v_mfma_f32_16x16x32_bf16 on
                             one 16-row block of X per workgroup; any M */
    NVFP4_PATH_BATCH = 3, /* matrix cores, every weight decoded once per workgroup for slabs of
                             up to 128 rows of X: X, codes and scales staged in LDS by
                             direct-to-LDS loads, eight wavefronts (two per SIMD) splitting each
                             window's four k-steps; narrow weights cut the rows into row groups.
                             Any M, meant for M > 16. (Value 4 is not a path.) */
    NVFP4_PATH_INVARIANT = 5 /* batch-invariant mode: row m of Y is the same bits for every M
                             and whatever the other rows of X hold. A request verified alone
                             or with others then gets exactly the bits its own M = 1 call in
                             this mode gives it, which is what lets speculation leave the
                             greedy tokens unchanged ("SparkInfer" README, speculative decoding
                             sections). Every call that must agree, plain decode included, has
                             to use this mode: nvfp4_gemm at M = 1 picks another kernel and
                             other bits, and nvfp4_gemm_fused has no invariant mode. The slab
                             kernel for all M: its sum for an output runs over the 128-k
                             windows in order in each of four k-step lanes, then adds the lanes
                             in a fixed order, so no plan choice (row groups, tile sets, tiles
                             per pass) changes a row's bits, and each call takes the plan that
                             suits its rows; slower than NVFP4_PATH_AUTO at small M.
                             split must be 0. */
} nvfp4_path_t;

/*
 * nvfp4_gemm_path -- nvfp4_gemm with the kernel family forced, for testing and tuning.
 *
 * Same operation, arguments, rules and results as nvfp4_gemm. `path` is an nvfp4_path_t.
 * `split` tunes the kernel (0 picks it like nvfp4_gemm):
 *   NVFP4_PATH_DOT: wavefronts per workgroup, 4, 8, 12 or 16; M <= 8, else
 *     NVFP4_ERROR_INVALID_VALUE.
 *     If X does not fit in LDS (M * K too large) the call runs NVFP4_PATH_MFMA with its own split.
 *   NVFP4_PATH_MFMA: wavefronts per workgroup, 4 or 8.
 *   NVFP4_PATH_BATCH: rows per row group, 16, 32, 64 or 128 (the rows of a 128-row slab are
 *     cut into groups of that many, each with its own workgroups).
 *   NVFP4_PATH_INVARIANT: 0 only.
 * Any other value returns NVFP4_ERROR_INVALID_VALUE.
 */
nvfp4_status_t nvfp4_gemm_path(int path, int split, int M, int N, int K, const uint16_t *X,
                               const uint8_t *Wq, const uint8_t *Wscale, const float *gscale,
                               float *Y, void *stream);

/*
 * nvfp4_gemm_argmax -- greedy token per row of the GEMM, without writing Y.
 *
 * Greedy decode and greedy speculative verification take, for every row of X, the column of the
 * largest output of the lm_head GEMM ("SparkInfer" README: decode, DSpark and DFlash2 figures are
 * greedy, and a request speculating alone gets exactly the tokens it gets without the drafter).
 * The lm_head is a full-vocabulary GEMM on every token ("Qwen3.8-27B-NVFP4-RTX5090" model card,
 * section on why lm_head is NVFP4), so its M x N fp32 logits are the largest output of a pass;
 * here they stay in registers: each kernel folds its outputs into per-row (value, column) keys,
 * and a second small kernel picks the winner per row.
 *
 * Result, for the Y that nvfp4_gemm (or nvfp4_gemm_path with the same path and split) computes
 * from the same inputs, bit for bit:
 *   index[m] = the smallest n with Y[m][n] == max over n of Y[m][n]
 *   value[m] = that maximum (fp32)
 * Ranking: -0 equals +0 (a -0 maximum is returned as +0); NaN ranks above every number (NaN
 * inputs are outside the contract of the GEMM itself). Like nvfp4_gemm the result is
 * deterministic; with NVFP4_PATH_INVARIANT it is also the same for row m whatever M is.
 *
 *   M, N, K, X, Wq, Wscale, gscale   as for nvfp4_gemm
 *   index      out: int32 [M], device, 4-byte aligned
 *   value      out: fp32 [M], device, 4-byte aligned
 *   workspace  scratch owned by the caller: at least nvfp4_argmax_workspace_bytes(M) bytes of
 *              device memory, 8-byte aligned; its contents on entry do not matter and are left
 *              undefined. Calls that overlap in time must not share a workspace.
 *   workspace_bytes  its size; smaller than required returns NVFP4_ERROR_INVALID_VALUE
 *   stream     hipStream_t
 * Errors as for nvfp4_gemm.
 */
nvfp4_status_t nvfp4_gemm_argmax(int M, int N, int K, const uint16_t *X, const uint8_t *Wq,
                                 const uint8_t *Wscale, const float *gscale, int32_t *index,
                                 float *value, void *workspace, uint64_t workspace_bytes,
                                 void *stream);

/* nvfp4_gemm_argmax with the kernel family and its split forced (path and split exactly as for
 * nvfp4_gemm_path; the result matches nvfp4_gemm_path with the same two values). */
nvfp4_status_t nvfp4_gemm_argmax_path(int path, int split, int M, int N, int K,
                                      const uint16_t *X, const uint8_t *Wq,
                                      const uint8_t *Wscale, const float *gscale, int32_t *index,
                                      float *value, void *workspace, uint64_t workspace_bytes,
                                      void *stream);

/*
 * nvfp4_gemm_argmax_noalloc -- nvfp4_gemm_argmax for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture that must not call hipMalloc, tight serving
 * loops, and harnesses that forbid allocation.
 *
 * Same result as nvfp4_gemm_argmax with the same arguments (bit for bit: the same kernels and
 * plan). The per-row keys go to a 4 MiB array in device memory that the library holds for the
 * process's lifetime, one copy per GPU; its device address is looked up on the first call on each
 * device (with that device current). The call never calls hipMalloc, hipFree or any allocating
 * routine, and writes every key it reads, so nothing needs clearing between calls.
 *
 *   M, N, K, X, Wq, Wscale, gscale, index, value, stream   as for nvfp4_gemm_argmax
 * Limit: M <= 4 MiB / (8 * 16 * compute units), i.e. 128 rows on a 256-CU MI355X; more returns
 * NVFP4_ERROR_SCRATCH_LIMIT (use nvfp4_gemm_argmax with a workspace, or split the rows).
 * Concurrency: every call on one GPU shares the array; calls that overlap in time on one GPU
 * (other streams, other host threads, other graphs replaying) race and give undefined results.
 * Calls on different GPUs do not interfere. Other errors as for nvfp4_gemm_argmax.
 */
nvfp4_status_t nvfp4_gemm_argmax_noalloc(int M, int N, int K, const uint16_t *X,
                                         const uint8_t *Wq, const uint8_t *Wscale,
                                         const float *gscale, int32_t *index, float *value,
                                         void *stream);

/* Workspace bytes nvfp4_gemm_argmax needs for M rows on the current device:
 * 8 * 16 * (compute units) per row (room for 16 8-byte keys per compute unit; the kernels write
 * at most 4 per compute unit); 0 if M < 1. */
uint64_t nvfp4_argmax_workspace_bytes(int M);

/*
 * nvfp4_gemm_grouped -- grouped (mixture-of-experts) GEMM, one launch, no host synchronisation:
 *
 *     Y[t] = X[t] . dequant(Wq_e, Wscale_e, gscale[e])   for offsets[e] <= t < offsets[e+1]
 *
 * The pages' engine runs mixture-of-experts models with a fused MoE FFN kernel and a router that
 * dispatches tokens to experts on the device ("SparkInfer" README, section "Layout & scoring"; its
 * MoE targets). At decode each token reads only its routed experts, a few rows per expert: the
 * same bandwidth-bound dot product as nvfp4_gemm at M = 1, over pieces whose sizes only the device
 * knows. The rows of X arrive grouped by expert (the dispatch order of the router, which is not
 * part of this library); the kernel reads the row counts from `offsets` on the device and deals
 * the (row chunk, 4-column group) items evenly to every wavefront of the grid.
 *
 *   T        rows of X and Y (token-expert pairs); 0 is allowed and does nothing (the pointers
 *            are then not checked or used, so empty tensors' null pointers are fine)
 *   E        experts, 1 <= E <= 2048
 *   N, K     the shape of every expert's weight (K % 16 == 0, as for nvfp4_gemm)
 *   X        in:  bf16 bits [T][K], device, rows sorted by expert
 *   offsets  in:  int32 [E + 1], device: expert e owns rows offsets[e] .. offsets[e+1] - 1;
 *                 meant to be non-decreasing from 0 to T. Entries are clamped to [0, T] and made
 *                 non-decreasing by a running maximum (expert e owns rows b_e .. b_{e+1} - 1,
 *                 b_e = max over e' <= e of the clamped offsets[e']): bad offsets move rows
 *                 between experts (rows before b_0 or from b_E on are not written), never cause
 *                 an access out of range
 *   Wq       in:  E packed code arrays back to back, expert e at Wq + e * nvfp4_codes_bytes(N, K)
 *                 (each as nvfp4_pack writes it)
 *   Wscale   in:  E packed scale arrays, expert e at Wscale + e * nvfp4_scales_bytes(N, K)
 *   gscale   in:  fp32 [E], device: tensor scale of each expert
 *   Y        out: fp32 [T][N], device; every row some expert owns is fully written
 *   rows_per_item  rows of one expert taken together (each weight byte is read once per chunk of
 *                 this many rows): 1, 2 or 4, or 0 to choose from T and E. Results are the same
 *                 bits for every value.
 *   stream   hipStream_t
 * Accuracy as nvfp4_gemm (fp32 accumulation, g once per output). Sizes: T * ceil(N / 4) < 2^40
 * and E * nvfp4_codes_bytes(N, K) < 2^62, else NVFP4_ERROR_INVALID_VALUE. Alignment: X, Wq, Wscale
 * 16 bytes; offsets, gscale, Y 4 bytes. Deterministic; a row's result does not depend on the
 * other rows, on rows_per_item or on the grid.
 */
nvfp4_status_t nvfp4_gemm_grouped(int T, int E, int N, int K, const uint16_t *X,
                                  const int32_t *offsets, const uint8_t *Wq,
                                  const uint8_t *Wscale, const float *gscale, float *Y,
                                  int rows_per_item, void *stream);

/*
 * nvfp4_gemm_fused -- the GEMM with its decode-layer neighbours folded in: an RMSNorm of X
 * before it and/or the gated FFN activation SiLU(gate) * up after it.
 *
 * The pages' engine has RMSNorm and fused FFN kernels next to its decode GEMV ("SparkInfer"
 * README, section "Layout & scoring"). In a dense decoder layer the q/k/v and gate/up projections
 * read RMSNorm(hidden), and down_proj reads SiLU(gate) * up of the gate/up projection (the SiLU
 * gate is the reading taken for the model family's FFN). Folding them in saves the round trips of
 * the normalised activations and of the M x N gate/up output, and two launches.
 *
 * fuse = NVFP4_FUSE_RMSNORM, NVFP4_FUSE_SILU_MUL or both (bitwise or):
 *   NVFP4_FUSE_RMSNORM   X is replaced by xhat[m][k] = bf16((x[m][k] * r_m) * gamma[k]), rounded
 *                        to nearest even, with r_m = 1 / sqrt(mean_k x[m][k]^2 + eps) in fp32
 *                        (the sum of squares within a relative (K / 64 + 32) * 2^-24 of exact);
 *                        then the GEMM runs on xhat.
 *   NVFP4_FUSE_SILU_MUL  the weight is a fused gate/up matrix whose columns interleave in groups of
 *                        four: columns 8q .. 8q + 3 are gate columns 4q .. 4q + 3 and columns
 *                        8q + 4 .. 8q + 7 are up columns 4q .. 4q + 3 (N % 8 == 0, I = N / 2).
 *                        Instead of Y the call writes H[m][j] = bf16(SiLU(gate) * up), with gate
 *                        and up the fp32 outputs of columns 8q + c and 8q + 4 + c for
 *                        j = 4q + c, SiLU(v) = v / (1 + e^-v).
 *   M, N, K, X, Wq, Wscale, gscale   as for nvfp4_gemm
 *   gamma    in: bf16 bits [K], device, 16-byte aligned (RMSNorm only; else ignored)
 *   eps      RMSNorm epsilon, finite and >= 0 (e.g. 1e-6)
 *   out      out: fp32 Y [M][N] (4-byte aligned) without NVFP4_FUSE_SILU_MUL, bf16 bits
 *            H [M][N / 2] (2-byte aligned) with it; device
 *   workspace  scratch owned by the caller: at least nvfp4_fused_workspace_bytes(fuse, M, N, K)
 *              bytes of device memory, 16-byte aligned (NULL when that is 0); its contents on
 *              entry do not matter and are left undefined. Calls that overlap in time must not
 *              share a workspace.
 *   workspace_bytes  its size; smaller than required returns NVFP4_ERROR_INVALID_VALUE
 * Kernels: up to 4 rows the dot-product kernel does everything (X normalised once in LDS, the
 * epilogue on its column sums; no workspace). Above, RMSNorm is a row-wise kernel of its own
 * writing the bf16 xhat to the workspace (normalising X inside the matrix-core kernels would
 * repeat it in every workgroup); then the 16-row matrix-core kernel (M <= 16) or the slab kernel
 * (M > 16), each with the SiLU(gate) * up epilogue inside, so the fp32 gate/up output is never
 * written. Errors as for nvfp4_gemm.
 */
enum { NVFP4_FUSE_RMSNORM = 1, NVFP4_FUSE_SILU_MUL = 2 };

nvfp4_status_t nvfp4_gemm_fused(int fuse, int M, int N, int K, const uint16_t *X,
                                const uint16_t *gamma, float eps, const uint8_t *Wq,
                                const uint8_t *Wscale, const float *gscale, void *out,
                                void *workspace, uint64_t workspace_bytes, void *stream);

/* Workspace bytes nvfp4_gemm_fused needs for these arguments on the current device: 0 when one
 * kernel does everything (no RMSNorm, or up to 4 rows whose X fits in LDS), else the normalised
 * X, M * K * 2 bytes rounded up to 256. 0 for arguments nvfp4_gemm_fused would reject. */
uint64_t nvfp4_fused_workspace_bytes(int fuse, int M, int N, int K);

/* Bytes of Wq for an N x K weight: 64 * ceil(N/4) * ceil(K/32); 0 if N < 1 or K < 1. */
uint64_t nvfp4_codes_bytes(int N, int K);

/* Bytes of Wscale for an N x K weight: 8 * ceil(N/4) * ceil(K/32); 0 if N < 1 or K < 1. */
uint64_t nvfp4_scales_bytes(int N, int K);

/* Static description of a status code; never NULL. */
const char *nvfp4_status_string(nvfp4_status_t status);

/* ABI version of this header (bumped on any incompatible change). */
#define NVFP4_ABI_VERSION 7
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */

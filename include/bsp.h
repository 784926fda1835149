/*
 * bsp.h -- C ABI of the block-scaled precision library for MI355X (gfx950).
 *
 * Block-scaled low-precision quantization of mixture-of-experts layers and the
 * grouped expert GEMM that consumes it:
 *   - MXFP8: 32 consecutive E4M3 values share one E8M0 (power of two) scale,
 *     with rowwise and columnwise copies [alphasignal.ai, "LMSYS Drops Miles",
 *     Recipe 1; remio.ai, "Miles Blackwell RL ...", section "Un quantizzatore
 *     condiviso e il vero meccanismo"];
 *   - NVFP4: 16 E2M1 values share one E4M3 block scale under an FP32 outer
 *     scale, per token for activations and per expert for weights, with the
 *     optional "4/6" block-scale choice [hackernews.jp, "4ビットの教訓",
 *     baseline recipe; nopree.com, "End-to-End 4-Bit Training", sections
 *     先说为什么难 and 工程细节];
 *   - dequantize -> transpose -> requantize with stochastic rounding for the
 *     backward path [nopree.com, same page, section 第二个决定];
 *   - the block-scaled grouped expert GEMM (gate/up/down; forward, data and
 *     weight gradient) [alphasignal.ai, Recipe 1 and Recipe 2];
 *   - the BF16 grouped expert GEMM of the NVFP4 recipe's backward pass, on the
 *     original or on dequantized operands [remio.ai, section "Entrambe le
 *     ricette supportano ..."; alphasignal.ai, Recipe 2].
 *
 * Conventions shared by every call:
 *   - Pointers named in the comments as "device" point to GPU memory; sizes
 *     and scalars are host values.  The caller allocates and owns every buffer;
 *     the library allocates nothing.  Its state is a per-device cache of the
 *     grouped GEMM kernels' occupancy (workgroups per compute unit), a
 *     property of the device and the compiled code filled on first use and
 *     stored atomically: results never depend on it, and concurrent callers
 *     may share the library; and the static device scratch array of the
 *     allocation-free GEMM entry point (bsp_moe_grouped_gemm_blockscaled_noalloc,
 *     below), with its per-device address.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and never synchronize; results are ready when the
 *     stream reaches that point.  Calls on one stream are ordered.
 *   - All matrices are row-major.  NVFP4 codes pack two elements per byte,
 *     element 2j in the low nibble of byte j; MXFP8 codes are one byte each.
 *     Scales are canonical row-major byte arrays (no swizzle): NVFP4 E4M3
 *     [rows, K/16], MXFP8 E8M0 [rows, K/32].
 *   - Device pointers must be 16-byte aligned.  Arguments are validated on
 *     the host before anything is launched; an invalid call returns an error
 *     and enqueues nothing.  Inputs must be finite.
 *   - Bit-exactness: codes and scales are a pure function of the inputs
 *     (IEEE f32 arithmetic, no fast math), identical to the reference
 *     definition for every launch geometry.
 */
#ifndef BSP_H
#define BSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsp_status {
    BSP_OK = 0,
    BSP_ERR_INVALID_ARG = 1, /* null pointer, unknown enum or flag bit */
    BSP_ERR_SHAPE = 2,       /* size not positive or not a multiple of the block */
    BSP_ERR_ALIGNMENT = 3,   /* device pointer or leading dimension misaligned */
    BSP_ERR_UNSUPPORTED = 4, /* valid combination that is not implemented */
    BSP_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    BSP_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
    BSP_ERR_SCRATCH_LIMIT = 7 /* allocation-free call: the problem's workspace exceeds the static scratch */
} bsp_status;

enum { BSP_FMT_NVFP4 = 0, BSP_FMT_MXFP8 = 1 };
enum { BSP_DTYPE_F32 = 0, BSP_DTYPE_BF16 = 1 };
enum { BSP_GEMM_FPROP = 0, BSP_GEMM_DGRAD = 1, BSP_GEMM_WGRAD = 2 };

/* flags */
#define BSP_NVFP4_46 0x1u /* NVFP4: choose between the "6" and "4" block scales */
#define BSP_SR 0x2u       /* requant: stochastic rounding (else nearest even) */

int bsp_version(void);                    /* 100 * major + minor */
const char *bsp_status_string(int status); /* static string, never NULL */

/*
 * NVFP4 quantize with an FP32 outer scale
 * [remio.ai, section "Il supporto Miles Blackwell ora copre l'intero ciclo
 * RL": one FP32 scale per token; hackernews.jp, baseline recipe: the fused
 * per-token activation quantizer computes the token scale, the E4M3 block
 * scales and the packed FP4 values in one kernel; nopree.com, section
 * 工程细节: per-expert outer scale for weights, "4/6" for activations].
 *
 *   x       device bf16 [M, K] with row stride ldx (elements, ldx >= K, ldx % 8 == 0)
 *   M, K    M >= 1; K >= 16 and K % 16 == 0
 *   rows_per_scale  consecutive rows sharing one outer scale: 1 = per token;
 *           N = per expert when E matrices [N, K] are stacked as [E*N, K];
 *           M = per tensor.  Must divide M.
 *   codes   device u8 [M, K/2] (out)
 *   scales  device u8 [M, K/16] E4M3 (out)
 *   outer   device f32 [M / rows_per_scale] decode scales g = amax / 2688 (out)
 *   flags   0 or BSP_NVFP4_46
 * Per scope: g = amax / (6 * 448); per 16-block with maximum a:
 * s = E4M3(a / (6 g)) (RNE, saturating), codes = E2M1(x * (1 / (s g))) (RNE,
 * saturating); with BSP_NVFP4_46 the block instead takes s4 = E4M3(a / (4 g))
 * when that candidate's squared error (f32, fused multiply-adds in index
 * order) is strictly lower.  A zero or f32-subnormal s*g stores s = 0 and
 * signed-zero codes.
 */
bsp_status bsp_quantize_nvfp4_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                        int64_t rows_per_scale, uint8_t *codes, uint8_t *scales,
                                        float *outer, uint32_t flags, void *stream);

/*
 * MXFP8 quantize, rowwise and/or columnwise from the same bf16 input
 * [alphasignal.ai, Recipe 1: 32 consecutive E4M3 values share one E8M0 scale;
 * both row-wise and column-wise copies are made from the original input].
 *
 *   x            device bf16 [x_rows, K], row stride ldx (ldx >= K, ldx % 8 == 0)
 *   K            K % 32 == 0
 *   row_gather   device int32 [M] or NULL: row r of the quantized tensor is
 *                x[row_gather[r]] (an index outside [0, x_rows) reads as a
 *                zero row); NULL means M == x_rows and row r is x[r]
 *   M            rows of the quantized tensor
 *   batch        number of stacked independent matrices (>= 1): x is
 *                [batch, x_rows, K] (matrix stride x_rows * ldx) and every
 *                output gains a leading batch dimension ([batch, M, K],
 *                [batch, M, K/32], [batch, K, ld_colT], [batch, K, ld_colT/32]),
 *                e.g. the per-expert columnwise copies of stacked expert
 *                weights.  batch > 1 takes neither row_gather nor groups.
 *   codes_row    device u8 [M, K] or NULL      (blocks along K)
 *   scales_row   device u8 [M, K/32] E8M0 or NULL (both NULL or both set)
 *   codes_colT   device u8 [K, ld_colT] or NULL (blocks along M, stored transposed)
 *   scales_colT  device u8 [K, ld_colT/32] or NULL (both NULL or both set)
 *   ld_colT      columns of the transposed copy; ld_colT % 32 == 0.
 *                Ungrouped: ld_colT >= M and M % 32 == 0.
 *                Grouped: ld_colT >= roundup32(M + 31 G) (the value of
 *                bsp_mxfp8_grouped_cols(M, G) keeps rows line-aligned).
 *   group_offsets  device int64 [G+1] or NULL.  Rows [off[g], off[g+1]) form
 *                group g (0 = off[0] <= ... <= off[G] = M).  Columnwise blocks
 *                then stay inside a group: group g occupies transposed columns
 *                [P[g], P[g] + pad32(n_g)) with P the running sum of the padded
 *                sizes; padding columns hold code 0.  Columns from P[G] to
 *                ld_colT are left untouched.
 *   G            number of groups (>= 1 when group_offsets is set)
 *   flags        0
 * The block exponent is the smallest k with amax <= 448 * 2^k, kept within
 * [-127, 119]; codes = E4M3(x * 2^-k) (RNE, saturating).  At least one of the
 * two copies must be requested.
 */
bsp_status bsp_quantize_mxfp8(const uint16_t *x, int64_t x_rows, int64_t K, int64_t ldx, const int32_t *row_gather,
                              int64_t M, int64_t batch, uint8_t *codes_row, uint8_t *scales_row, uint8_t *codes_colT,
                              uint8_t *scales_colT, int64_t ld_colT, const int64_t *group_offsets, int64_t G,
                              uint32_t flags, void *stream);

/*
 * NVFP4 numerics variants [nopree.com, section 第二个决定: 16x16 block scales
 * survive a transpose, but one outlier among 256 values flattens the other
 * 255; hackernews.jp, recipe notes: the random Hadamard transform option].
 *
 * bsp_quantize_nvfp4_rht: per-token NVFP4 (standard, or 4/6 with
 * BSP_NVFP4_46) of the rows after a 16-point random Hadamard transform of
 * every 16-value block, in f32: negate element i where bit i of `signs`
 * (< 2^16) is set, Walsh-Hadamard butterflies (a, b) -> (a + b, a - b) at
 * distances 1, 2, 4, 8, scale by 1/4.  The transform is orthonormal, so two
 * operands transformed with the same signs along their common K multiply as
 * the originals (the GEMM takes them as they are); the outer scale is the
 * transformed row's.  Outputs as bsp_quantize_nvfp4_per_token with
 * rows_per_scale = 1; 16 <= K <= 8192, K % 16 == 0.
 *
 * bsp_quantize_nvfp4_2d: 16x16 2-D blocks under one per-tensor outer scale
 * g = amax / 2688 (outer [1]); tile (i, j)'s E4M3 scale s = E4M3(a / (6 g))
 * from the tile's amax, stored at scales[i * (K/16) + j] ([M/16, K/16]);
 * every 16-value row piece of the tile is then coded as a 1x16 block under
 * that scale (codes [M, K/2] as usual).  The transposed tensor's
 * quantization is the nibble transpose of the codes with the transposed
 * scales.  M % 16 == 0 (M/16 <= 65535), K % 16 == 0.
 */
bsp_status bsp_quantize_nvfp4_rht(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint32_t signs,
                                  uint8_t *codes, uint8_t *scales, float *outer, uint32_t flags, void *stream);
bsp_status bsp_quantize_nvfp4_2d(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint8_t *codes,
                                 uint8_t *scales, float *outer, void *stream);

/*
 * Dequantize NVFP4 or MXFP8 to f32 or bf16 [remio.ai, section "Entrambe le
 * ricette supportano ...": the dequantized backward rebuilds BF16 from the
 * exact low-precision values used in the forward; alphasignal.ai, Recipe 2].
 *
 *   fmt      BSP_FMT_NVFP4 or BSP_FMT_MXFP8
 *   codes, scales  device, layouts as produced by the quantizers ([M, K/2] +
 *            [M, K/16] for NVFP4; [M, K] + [M, K/32] for MXFP8)
 *   outer    device f32 [M / rows_per_scale] (NVFP4 only; NULL for MXFP8)
 *   out      device [M, K] of out_dtype (BSP_DTYPE_F32 or BSP_DTYPE_BF16)
 * NVFP4: y = value(q) * (s * g) in f32 (two rounded products, in that
 * order); MXFP8: y = value(q) * 2^k (exact).  bf16 output is the RNE of y.
 */
bsp_status bsp_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t M,
                          int64_t K, int64_t rows_per_scale, void *out, int out_dtype, void *stream);

/*
 * Dequantize -> transpose -> requantize NVFP4 with stochastic rounding
 * [nopree.com, "End-to-End 4-Bit Training", section 第二个决定: the forward's
 * 1x16 row blocks do not fit the gradient GEMM after the transpose, so the
 * tensor is dequantized to high precision, transposed and requantized with
 * stochastic rounding, which keeps the expectation].
 *
 *   codes, scales, outer  device rowwise NVFP4 [M, K] with per-row outer scales [M]
 *   M, K     M % 16 == 0, K % 16 == 0
 *   codesT   device u8 [K, M/2] (out; 16-blocks now run along M)
 *   scalesT  device u8 [K, M/16] (out)
 *   outerT   device f32 [1] (out): G = max_m outer[m]
 *   seed     key of the counter-based generator
 *   flags    BSP_SR for stochastic rounding, 0 for round to nearest even
 *   workspace  device, >= bsp_requant_workspace_size(M) bytes
 * Intermediate d = value(q) * (s * g) in f32; per output 16-block:
 * s' = E4M3(amax / (6 G)), v = |d| * (1 / (s' G)).  SR rounds v up to the next
 * E2M1 value iff u < frac * 65536, with frac the exact position of v between
 * its two grid neighbours and u the 16 bits of Philox4x32-10 (key = seed,
 * counter = (i / 8) in words 0-1) for output element i = k * M + m: word
 * (i % 8) / 2, low half for even i.  v >= 6 saturates to 6.
 */
bsp_status bsp_requant_transpose_sr(const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t M,
                                    int64_t K, uint8_t *codesT, uint8_t *scalesT, float *outerT, uint64_t seed,
                                    uint32_t flags, void *workspace, size_t ws_bytes, void *stream);

/*
 * The same for the weight gradient's token-blocked operands: the rows of each
 * expert group, read through the routing map, dequantized, transposed and
 * requantized on their own [nopree.com, section 第二个决定, per expert].
 *   codes, scales, outer  device rowwise NVFP4 [src_rows, K] with per-row
 *            outer scales [src_rows] (e.g. the forward's per-token X, or dY)
 *   gather   device int32 [R] or NULL (then src_rows == R): row r of the
 *            routed order reads source row gather[r]; an index outside
 *            [0, src_rows) reads as zeros
 *   group_offsets  device int64 [G+1], rows of the routed order per group
 *            (0 = off[0] <= ... <= off[G] = R); 1 <= G <= 2048
 *   codesT   device u8 [K, ldT/2], scalesT device u8 [K, ldT/16] (out):
 *            group g in columns [P[g], P[g] + pad32(n_g)), P the running sum
 *            of the 32-padded group sizes; padding columns hold zero codes
 *            and zero scales; columns from P[G] to ldT are left untouched
 *   ldT      multiple of 32, >= roundup32(R + 31 G) (bsp_mxfp8_grouped_cols
 *            gives a line-aligned value)
 *   outerT   device f32 [G] (out): G_g = max outer scale over group g's rows
 *   K % 16 == 0
 * Each group is requantized exactly as by bsp_requant_transpose_sr with its
 * own G_g; the SR bits of output element (k, p) are drawn at its index in
 * the output array, i = k*ldT + p.
 */
bsp_status bsp_requant_transpose_sr_grouped(const uint8_t *codes, const uint8_t *scales, const float *outer,
                                            int64_t src_rows, const int32_t *gather, const int64_t *group_offsets,
                                            int64_t G, int64_t R, int64_t K, uint8_t *codesT, uint8_t *scalesT,
                                            int64_t ldT, float *outerT, uint64_t seed, uint32_t flags, void *stream);

/*
 * The same for a batch of E tensors stacked along their rows, each on its
 * own [nopree.com, section 第二个决定, applied per expert]: the per-expert
 * weights of one projection become the data-gradient GEMM's B operand with
 * 16-blocks along the forward's output dimension.
 *   codes, scales  device rowwise NVFP4 of the stacked input [E*M, K]
 *   outer    device f32 [E*M / rows_per_scale]: row r's outer scale is
 *            outer[r / rows_per_scale] (rows_per_scale = M for per-expert
 *            weights); rows_per_scale divides M or is a multiple of M
 *            dividing E*M
 *   codesT   device u8 [E*K, M/2], scalesT device u8 [E*K, M/16] (out):
 *            tensor e's output at rows [e*K, (e+1)*K)
 *   outerT   device f32 [E] (out): G_e = max over tensor e's rows' outer scales
 *   E <= 65535; M % 16 == 0, K % 16 == 0
 *   workspace  device, >= bsp_requant_batched_workspace_size(E, M,
 *              rows_per_scale) bytes
 * Each tensor is requantized exactly as by bsp_requant_transpose_sr with its
 * own G_e; the SR bits of output element (e, k, m) are drawn at its index in
 * the stacked output, i = (e*K + k)*M + m.  bsp_requant_transpose_sr is
 * this call with E = 1, rows_per_scale = 1.
 */
bsp_status bsp_requant_transpose_sr_batched(const uint8_t *codes, const uint8_t *scales, const float *outer,
                                            int64_t rows_per_scale, int64_t E, int64_t M, int64_t K, uint8_t *codesT,
                                            uint8_t *scalesT, float *outerT, uint64_t seed, uint32_t flags,
                                            void *workspace, size_t ws_bytes, void *stream);

/*
 * Block-scaled grouped expert GEMM [alphasignal.ai, Recipe 1 (MXFP8 forward,
 * weight- and data-gradient GEMMs) and Recipe 2 (NVFP4 MoE experts, per-token
 * scaling fused into the GEMM epilogue); remio.ai, section "Un quantizzatore
 * condiviso": blocks must follow the reduction dimension].
 *
 * FPROP and DGRAD (same arithmetic; DGRAD takes the columnwise weight copy):
 *   C[r, n] = gA[t] * gB[e] * sum_k A[t, k] * B_e[n, k]
 *   with e the group holding row r (group_offsets, rows of C), t = a_gather[r]
 *   (or r when a_gather is NULL) and gA, gB the NVFP4 outer scales (1 for MXFP8).
 *     a_codes/a_scales  device A [a_rows, K] quantized along K
 *     a_outer   device f32 [a_rows] (NVFP4 per-token scales; NULL for MXFP8)
 *     a_gather  device int32 [M] or NULL (then a_rows == M)
 *     group_offsets  device int64 [G+1]: rows of C per group, off[G] == M
 *     M, N, K   rows of C, columns of C, reduction length (K % 32 == 0 for
 *               both formats: operand rows are fetched in 16-byte pieces);
 *               sizes below 2^31, and each operand's codes (A, one expert
 *               of B) and B's scales below 4 GiB, else BSP_ERR_SHAPE
 *     b_codes/b_scales  device B [G, N, K] quantized along K
 *     b_outer   device f32 [G] (NVFP4 per-expert scales; NULL for MXFP8)
 *     c         device [M, ldc] of c_dtype (BSP_DTYPE_F32 or BSP_DTYPE_BF16)
 * WGRAD: per group g, C_g[n, j] = gA[g] * gB[g] * sum over the group's
 *   padded token columns t of A[n, P[g] + t] * B[j, P[g] + t], where A [M, K]
 *   and B [N, K] are grouped columnwise copies (K = their ld_colT) and P the
 *   32-padded group starts; group_offsets are the unpadded token offsets.
 *   MXFP8: the copies made by bsp_quantize_mxfp8, a_outer and b_outer NULL.
 *   NVFP4 (the 4-bit backward [nopree.com, section 第二个决定]): the copies
 *   made by bsp_requant_transpose_sr_grouped, a_outer and b_outer their
 *   per-group outer scales [G].  C is [G, M, ldc] (group stride M * ldc).
 *   a_gather must be NULL and a_rows == M.
 * Accumulation is f32 on the MFMA units; the epilogue applies gA * gB and
 * rounds to c_dtype (RNE for bf16).
 *   workspace  device, >= bsp_gemm_workspace_size(fmt, mode, M, N, K, G)
 *              bytes, 16-byte aligned; holds the tile list (WGRAD: the padded
 *              group starts and the experts ordered by token count) and
 *              block-major copies of both operands' scales, rewritten by
 *              every call, so calls sharing one workspace must be
 *              stream-ordered
 */
bsp_status bsp_moe_grouped_gemm_blockscaled(int fmt, int mode, const uint8_t *a_codes, const uint8_t *a_scales,
                                            const float *a_outer, const int32_t *a_gather, int64_t a_rows,
                                            const int64_t *group_offsets, int64_t G, int64_t M, int64_t N,
                                            int64_t K, const uint8_t *b_codes, const uint8_t *b_scales,
                                            const float *b_outer, void *c, int c_dtype, int64_t ldc,
                                            void *workspace, size_t ws_bytes, void *stream);

/*
 * The same call with the GEMM's output tile edge chosen by the caller:
 * tile 0 is the library's choice (what bsp_moe_grouped_gemm_blockscaled
 * does: 256 once the problem has at least 512 such tiles, else 128), 128 or
 * 256 pins it; any other value returns BSP_ERR_INVALID_ARG.  Results do not
 * depend on the tile (the contract holds for every launch geometry); the pin
 * exists for tests, which run small problems with both tile shapes, and for
 * tuning.
 */
bsp_status bsp_moe_grouped_gemm_blockscaled_tiled(int fmt, int mode, const uint8_t *a_codes,
                                                  const uint8_t *a_scales, const float *a_outer,
                                                  const int32_t *a_gather, int64_t a_rows,
                                                  const int64_t *group_offsets, int64_t G, int64_t M, int64_t N,
                                                  int64_t K, const uint8_t *b_codes, const uint8_t *b_scales,
                                                  const float *b_outer, void *c, int c_dtype, int64_t ldc,
                                                  void *workspace, size_t ws_bytes, int tile, void *stream);

/*
 * Allocation-free form of bsp_moe_grouped_gemm_blockscaled, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments and results as
 * bsp_moe_grouped_gemm_blockscaled with the library's tile choice, minus the
 * workspace: the tile list, counters and scale planes live in a static
 * device array of BSP_GEMM_SCRATCH_BYTES (64 MiB) that each GPU the library
 * runs on holds until the process ends.  The call allocates nothing (no
 * hipMalloc or allocating library routine); on its first call on a device
 * it looks up that device's copy of the array (a HIP symbol query).
 *   - A problem whose bsp_gemm_workspace_size exceeds BSP_GEMM_SCRATCH_BYTES
 *     returns BSP_ERR_SCRATCH_LIMIT and enqueues nothing (e.g. the
 *     Qwen3-30B-A3B-shaped expert GEMMs fit, 18-37 MiB; a DeepSeek-V3 layer's
 *     257-expert forward GEMMs on one GPU, 122-249 MiB, do not).
 *   - Every call on a GPU shares that GPU's array and rewrites what it reads,
 *     so consecutive calls need nothing cleared; calls that overlap in time on
 *     one GPU (different streams without ordering, or several host threads)
 *     race on it and must be serialized by the caller.
 */
#define BSP_GEMM_SCRATCH_BYTES (64u << 20)
bsp_status bsp_moe_grouped_gemm_blockscaled_noalloc(int fmt, int mode, const uint8_t *a_codes,
                                                    const uint8_t *a_scales, const float *a_outer,
                                                    const int32_t *a_gather, int64_t a_rows,
                                                    const int64_t *group_offsets, int64_t G, int64_t M, int64_t N,
                                                    int64_t K, const uint8_t *b_codes, const uint8_t *b_scales,
                                                    const float *b_outer, void *c, int c_dtype, int64_t ldc,
                                                    void *stream);

/*
 * BF16 grouped expert GEMM for the backward pass of the NVFP4 MoE recipe,
 * which runs its data- and weight-gradient GEMMs in BF16 [remio.ai, section
 * "Entrambe le ricette supportano ...": either on the original high-precision
 * operands, or on operands dequantized (bsp_dequantize) from the exact NVFP4
 * values of the forward pass, which keeps the backward consistent with the
 * forward; alphasignal.ai, Recipe 2].  Both modes are this one call; they
 * differ only in the operands passed.  Operands are bf16, row-major, with
 * leading dimensions lda, ldb in elements (multiples of 8).
 *
 * FPROP and DGRAD, rows of C grouped by expert (e = group holding row r,
 * t = gather[r], or r when gather is NULL):
 *   FPROP: C[r, n] = sum_k A[t, k] * B_e[n, k],  B [G, N, ldb]: forward weight
 *   DGRAD: C[r, n] = sum_k A[t, k] * B_e[k, n],  B [G, K, ldb]: the forward
 *          weight as stored ([out, in] per expert), so no transposed copy is
 *          needed: dX = dY * W_e
 *     a        device bf16 [src_rows, lda >= K]; K % 8 == 0
 *     gather   device int32 [M] or NULL (then src_rows == M); a row with an
 *              index outside [0, src_rows) reads as zeros
 *     DGRAD: N % 8 == 0
 *     C        device [M, ldc] of c_dtype; group_offsets: rows of C per
 *              group, off[G] == M
 * WGRAD, reducing over the rows of each group:
 *   C_g[m, n] = sum_{r in [off[g], off[g+1])} A[r, m] * B[t, n],
 *   t = gather[r] (or r): dW_e = dY_e^T * X_e with the routed rows of X read
 *   through the routing map, and no transposed copies
 *     a        device bf16 [K, lda >= M] (K = off[G], rows in grouped order)
 *     b        device bf16 [src_rows, ldb >= N]
 *     gather   device int32 [K] or NULL (then src_rows == K); an index
 *              outside [0, src_rows) contributes nothing
 *     M % 8 == 0, N % 8 == 0; C device [G, M, ldc] (group stride M * ldc)
 * Accumulation is f32 on the MFMA units (V_MFMA_F32_32X32X16_BF16); bf16
 * output is the RNE of the f32 sum.  Sizes below 2^31, lda and ldb below
 * 2^26, A (FPROP/DGRAD) and one expert's B (FPROP) below 4 GiB, else
 * BSP_ERR_SHAPE.
 *   workspace  device, >= bsp_gemm_bf16_workspace_size(mode, M, N, K, G)
 *              bytes (the row-tile list, or for WGRAD the experts ordered by
 *              token count), rewritten by every call: calls sharing one
 *              workspace must be stream-ordered
 */
bsp_status bsp_moe_grouped_gemm_bf16(int mode, const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb,
                                     const int32_t *gather, int64_t src_rows, const int64_t *group_offsets,
                                     int64_t G, int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                                     void *workspace, size_t ws_bytes, void *stream);
/* The same with the tile edge chosen by the caller (0, 128 or 256), as
 * bsp_moe_grouped_gemm_blockscaled_tiled. */
bsp_status bsp_moe_grouped_gemm_bf16_tiled(int mode, const uint16_t *a, int64_t lda, const uint16_t *b,
                                           int64_t ldb, const int32_t *gather, int64_t src_rows,
                                           const int64_t *group_offsets, int64_t G, int64_t M, int64_t N, int64_t K,
                                           void *c, int c_dtype, int64_t ldc, void *workspace, size_t ws_bytes,
                                           int tile, void *stream);

/*
 * SwiGLU between the gate/up and down projections, then quantization of its
 * output for the down GEMM [hackernews.jp, baseline recipe: the activation
 * quantizer is fused with the per-token scale computation].
 *   h13     device [R, 2I] of in_dtype (f32 or bf16): gate = columns [0, I),
 *           up = columns [I, 2I)
 *   h_out   device bf16 [R, I] (out, may be NULL when fmt >= 0)
 *   fmt     -1 (only h), BSP_FMT_NVFP4 (per-token, flags may hold
 *           BSP_NVFP4_46) or BSP_FMT_MXFP8 (rowwise)
 *   codes, scales, outer  outputs as for the quantizers (outer NVFP4 only)
 * h = bf16(silu(gate) * up), silu(z) = z / (1 + exp(-z)) with exp evaluated
 * by one fixed f32 algorithm (Cody-Waite reduction by ln 2, degree-7 Taylor
 * polynomial, exact 2^n scaling), then quantized exactly as the quantizer
 * calls would quantize h.  I % 32 == 0.
 */
bsp_status bsp_swiglu_quantize(const void *h13, int in_dtype, int64_t R, int64_t I, uint16_t *h_out, int fmt,
                               uint8_t *codes, uint8_t *scales, float *outer, uint32_t flags, void *stream);

/* Host-only size helpers (pure functions, no HIP calls). */
bsp_status bsp_nvfp4_sizes(int64_t M, int64_t K, int64_t rows_per_scale, size_t *codes_bytes,
                           size_t *scales_bytes, size_t *outer_count);
bsp_status bsp_mxfp8_sizes(int64_t M, int64_t K, size_t *codes_bytes, size_t *scales_bytes);
/* Column count to allocate for a grouped columnwise copy (MXFP8 ld_colT, or
 * ldT of the grouped requant): roundup256(M + 31 * G).  Any multiple of 32 of
 * at least roundup32(M + 31 * G), an upper bound of the padded total
 * sum_g roundup32(n_g), is accepted; the multiple of 256 starts every row of
 * the transposed codes (ld bytes for MXFP8, ld / 2 for NVFP4) on a 128-byte
 * line, which the quantizers' row stores and the weight-gradient GEMM's
 * loads need to stay whole-line.  -1 for M < 0 or G < 1. */
int64_t bsp_mxfp8_grouped_cols(int64_t M, int64_t G);
/* Bytes of requant workspace for M rows: one f32 partial maximum of the outer
 * scales per 2048 rows (at most 1024 partials); 0 for M <= 0. */
size_t bsp_requant_workspace_size(int64_t M);
/* Bytes of workspace for the batched requant: per tensor, one f32 partial
 * maximum per 2048 outer scales (at most 1024); 0 for invalid arguments. */
size_t bsp_requant_batched_workspace_size(int64_t E, int64_t M, int64_t rows_per_scale);
/* Bytes of workspace for bsp_moe_grouped_gemm_blockscaled (0 for an unknown
 * format or mode, or sizes below 1). */
size_t bsp_gemm_workspace_size(int fmt, int mode, int64_t M, int64_t N, int64_t K, int64_t G);
/* Bytes of workspace for bsp_moe_grouped_gemm_bf16 (0 for invalid arguments). */
size_t bsp_gemm_bf16_workspace_size(int mode, int64_t M, int64_t N, int64_t K, int64_t G);

#ifdef __cplusplus
}
#endif
#endif /* BSP_H */

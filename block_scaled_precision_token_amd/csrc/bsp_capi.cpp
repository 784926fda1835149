// bsp_capi.cpp -- the exported C ABI: host-side validation, then launches on
// the caller's stream.  Validation happens before any HIP call, so a rejected
// call enqueues nothing and needs no GPU.
#include <hip/hip_runtime.h>

#include "bsp_internal.hpp"

#define BSP_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned16_or_null(const void *p) { return p == nullptr || aligned16(p); }

inline bsp_status hip_status(hipError_t e) { return e == hipSuccess ? BSP_OK : BSP_ERR_HIP; }
inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

BSP_EXPORT int bsp_version(void) { return 100; }

BSP_EXPORT const char *bsp_status_string(int status) {
    switch (status) {
        case BSP_OK: return "ok";
        case BSP_ERR_INVALID_ARG: return "invalid argument (null pointer, unknown enum or flag)";
        case BSP_ERR_SHAPE: return "invalid shape (size not positive or not a multiple of the block)";
        case BSP_ERR_ALIGNMENT: return "device pointer or leading dimension not 16-byte aligned";
        case BSP_ERR_UNSUPPORTED: return "unsupported combination";
        case BSP_ERR_WORKSPACE: return "workspace missing or too small";
        case BSP_ERR_HIP: return "HIP runtime error at launch";
        case BSP_ERR_SCRATCH_LIMIT: return "problem needs more workspace than the allocation-free call's static scratch";
        default: return "unknown status";
    }
}

BSP_EXPORT bsp_status bsp_nvfp4_sizes(int64_t M, int64_t K, int64_t rows_per_scale, size_t *codes_bytes,
                                      size_t *scales_bytes, size_t *outer_count) {
    if (!codes_bytes || !scales_bytes || !outer_count) return BSP_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0 || K % 16 || rows_per_scale <= 0 || M % rows_per_scale) return BSP_ERR_SHAPE;
    *codes_bytes = (size_t)(M * (K / 2));
    *scales_bytes = (size_t)(M * (K / 16));
    *outer_count = (size_t)(M / rows_per_scale);
    return BSP_OK;
}

BSP_EXPORT bsp_status bsp_mxfp8_sizes(int64_t M, int64_t K, size_t *codes_bytes, size_t *scales_bytes) {
    if (!codes_bytes || !scales_bytes) return BSP_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0 || K % 32) return BSP_ERR_SHAPE;
    *codes_bytes = (size_t)(M * K);
    *scales_bytes = (size_t)(M * (K / 32));
    return BSP_OK;
}

// Smallest accepted column count of a grouped transposed copy: the padded
// total sum_g roundup32(n_g) never exceeds roundup32(M + 31 G).
static int64_t grouped_cols_min(int64_t M, int64_t G) { return (M + 31 * G + 31) / 32 * 32; }

BSP_EXPORT int64_t bsp_mxfp8_grouped_cols(int64_t M, int64_t G) {
    if (M < 0 || G < 1) return -1;
    return (M + 31 * G + 255) / 256 * 256;
}

BSP_EXPORT size_t bsp_requant_workspace_size(int64_t M) {
    if (M <= 0) return 0;
    return (size_t)bsp::requant_partials(M) * sizeof(float);
}

BSP_EXPORT size_t bsp_requant_batched_workspace_size(int64_t E, int64_t M, int64_t rows_per_scale) {
    if (E <= 0 || M <= 0 || rows_per_scale <= 0) return 0;
    if (M % rows_per_scale && rows_per_scale % M) return 0;
    return (size_t)bsp::requant_workspace_floats(E, M, rows_per_scale) * sizeof(float);
}

BSP_EXPORT size_t bsp_gemm_workspace_size(int fmt, int mode, int64_t M, int64_t N, int64_t K, int64_t G) {
    if (M < 1 || N < 1 || K < 1 || G < 1) return 0;
    if (fmt != BSP_FMT_NVFP4 && fmt != BSP_FMT_MXFP8) return 0;
    if (mode != BSP_GEMM_FPROP && mode != BSP_GEMM_DGRAD && mode != BSP_GEMM_WGRAD) return 0;
    return (size_t)bsp::gemm_workspace_bytes(fmt, mode, M, N, K, G);
}

BSP_EXPORT size_t bsp_gemm_bf16_workspace_size(int mode, int64_t M, int64_t N, int64_t K, int64_t G) {
    if (M < 1 || N < 1 || K < 1 || G < 1) return 0;
    if (mode != BSP_GEMM_FPROP && mode != BSP_GEMM_DGRAD && mode != BSP_GEMM_WGRAD) return 0;
    return (size_t)bsp::gemm_bf16_workspace_bytes(mode, M, G);
}

BSP_EXPORT bsp_status bsp_quantize_nvfp4_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                                   int64_t rows_per_scale, uint8_t *codes, uint8_t *scales,
                                                   float *outer, uint32_t flags, void *stream) {
    if (!x || !codes || !scales || !outer) return BSP_ERR_INVALID_ARG;
    if (flags & ~BSP_NVFP4_46) return BSP_ERR_INVALID_ARG;
    if (M <= 0 || K < 16 || K % 16 || ldx < K || rows_per_scale <= 0 || M % rows_per_scale) return BSP_ERR_SHAPE;
    if (!aligned16(x) || ldx % 8 || !aligned16(codes) || !aligned16(scales) || !aligned16(outer))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_quantize_nvfp4(x, M, K, ldx, rows_per_scale, codes, scales, outer,
                                                 (flags & BSP_NVFP4_46) != 0, as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_quantize_nvfp4_rht(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint32_t signs,
                                             uint8_t *codes, uint8_t *scales, float *outer, uint32_t flags,
                                             void *stream) {
    if (!x || !codes || !scales || !outer) return BSP_ERR_INVALID_ARG;
    if (flags & ~BSP_NVFP4_46) return BSP_ERR_INVALID_ARG;
    if (signs > 0xFFFFu) return BSP_ERR_INVALID_ARG;
    if (M <= 0 || K < 16 || K % 16 || K > 8192 || ldx < K) return BSP_ERR_SHAPE;
    if (!aligned16(x) || ldx % 8 || !aligned16(codes) || !aligned16(scales) || !aligned16(outer))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_quantize_nvfp4_rht(x, M, K, ldx, signs, codes, scales, outer,
                                                     (flags & BSP_NVFP4_46) != 0, as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_quantize_nvfp4_2d(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint8_t *codes,
                                            uint8_t *scales, float *outer, void *stream) {
    if (!x || !codes || !scales || !outer) return BSP_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0 || M % 16 || K % 16 || ldx < K) return BSP_ERR_SHAPE;
    if (M / 16 > 65535) return BSP_ERR_SHAPE;
    if (!aligned16(x) || ldx % 8 || !aligned16(codes) || !aligned16(scales) || !aligned16(outer))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_quantize_nvfp4_2d(x, M, K, ldx, codes, scales, outer, as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_quantize_mxfp8(const uint16_t *x, int64_t x_rows, int64_t K, int64_t ldx,
                                         const int32_t *row_gather, int64_t M, int64_t batch, uint8_t *codes_row,
                                         uint8_t *scales_row, uint8_t *codes_colT, uint8_t *scales_colT,
                                         int64_t ld_colT, const int64_t *group_offsets, int64_t G, uint32_t flags,
                                         void *stream) {
    if (!x) return BSP_ERR_INVALID_ARG;
    if (flags != 0) return BSP_ERR_INVALID_ARG;
    if ((codes_row == nullptr) != (scales_row == nullptr)) return BSP_ERR_INVALID_ARG;
    if ((codes_colT == nullptr) != (scales_colT == nullptr)) return BSP_ERR_INVALID_ARG;
    if (!codes_row && !codes_colT) return BSP_ERR_INVALID_ARG;
    if (group_offsets && !codes_colT) return BSP_ERR_INVALID_ARG;
    if (M <= 0 || x_rows <= 0 || K < 32 || K % 32 || ldx < K) return BSP_ERR_SHAPE;
    if (!row_gather && M != x_rows) return BSP_ERR_SHAPE;
    if (batch < 1 || batch > 65535) return BSP_ERR_SHAPE;
    if (batch > 1 && (row_gather || group_offsets)) return BSP_ERR_UNSUPPORTED;
    if (codes_colT) {
        if (ld_colT <= 0 || ld_colT % 32) return BSP_ERR_SHAPE;
        if (group_offsets) {
            if (G < 1 || G > 2048) return BSP_ERR_SHAPE;
            if (ld_colT < grouped_cols_min(M, G)) return BSP_ERR_SHAPE;
        } else {
            if (M % 32 || ld_colT < M) return BSP_ERR_SHAPE;
        }
    }
    if (!aligned16(x) || ldx % 8 || !aligned16_or_null(codes_row) || !aligned16_or_null(scales_row) ||
        !aligned16_or_null(codes_colT) || !aligned16_or_null(scales_colT) || !aligned16_or_null(group_offsets) ||
        !aligned16_or_null(row_gather))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_quantize_mxfp8(x, x_rows, K, ldx, row_gather, M, codes_row, scales_row, codes_colT,
                                                 scales_colT, ld_colT, group_offsets, group_offsets ? G : 1, batch,
                                                 as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales, const float *outer,
                                     int64_t M, int64_t K, int64_t rows_per_scale, void *out, int out_dtype,
                                     void *stream) {
    if (!codes || !scales || !out) return BSP_ERR_INVALID_ARG;
    if (fmt != BSP_FMT_NVFP4 && fmt != BSP_FMT_MXFP8) return BSP_ERR_INVALID_ARG;
    if (out_dtype != BSP_DTYPE_F32 && out_dtype != BSP_DTYPE_BF16) return BSP_ERR_INVALID_ARG;
    if (fmt == BSP_FMT_NVFP4 && !outer) return BSP_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0) return BSP_ERR_SHAPE;
    if (fmt == BSP_FMT_NVFP4 && (K % 16 || rows_per_scale <= 0 || M % rows_per_scale)) return BSP_ERR_SHAPE;
    if (fmt == BSP_FMT_MXFP8 && K % 32) return BSP_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(out) || !aligned16_or_null(outer))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_dequantize(fmt, codes, scales, outer, M, K, fmt == BSP_FMT_NVFP4 ? rows_per_scale : 1,
                                             out, out_dtype, as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_requant_transpose_sr_batched(const uint8_t *codes, const uint8_t *scales,
                                                       const float *outer, int64_t rows_per_scale, int64_t E,
                                                       int64_t M, int64_t K, uint8_t *codesT, uint8_t *scalesT,
                                                       float *outerT, uint64_t seed, uint32_t flags, void *workspace,
                                                       size_t ws_bytes, void *stream) {
    if (!codes || !scales || !outer || !codesT || !scalesT || !outerT) return BSP_ERR_INVALID_ARG;
    if (flags & ~BSP_SR) return BSP_ERR_INVALID_ARG;
    if (E <= 0 || M <= 0 || K <= 0 || M % 16 || K % 16 || rows_per_scale <= 0) return BSP_ERR_SHAPE;
    if (E > 65535 || (M % rows_per_scale && rows_per_scale % M) || (E * M) % rows_per_scale) return BSP_ERR_SHAPE;
    if (!workspace || ws_bytes < bsp_requant_batched_workspace_size(E, M, rows_per_scale)) return BSP_ERR_WORKSPACE;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(outer) || !aligned16(codesT) || !aligned16(scalesT) ||
        !aligned16(outerT) || !aligned16(workspace))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_requant(codes, scales, outer, rows_per_scale, E, M, K, codesT, scalesT, outerT,
                                          seed, (flags & BSP_SR) != 0, reinterpret_cast<float *>(workspace),
                                          as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_requant_transpose_sr_grouped(const uint8_t *codes, const uint8_t *scales,
                                                       const float *outer, int64_t src_rows, const int32_t *gather,
                                                       const int64_t *group_offsets, int64_t G, int64_t R, int64_t K,
                                                       uint8_t *codesT, uint8_t *scalesT, int64_t ldT, float *outerT,
                                                       uint64_t seed, uint32_t flags, void *stream) {
    if (!codes || !scales || !outer || !group_offsets || !codesT || !scalesT || !outerT) return BSP_ERR_INVALID_ARG;
    if (flags & ~BSP_SR) return BSP_ERR_INVALID_ARG;
    if (G < 1 || G > 2048 || R <= 0 || K <= 0 || K % 16 || src_rows <= 0) return BSP_ERR_SHAPE;
    if (src_rows >= (1ll << 31) || R >= (1ll << 40)) return BSP_ERR_SHAPE;
    if (!gather && src_rows != R) return BSP_ERR_SHAPE;
    if (ldT % 32 || ldT < grouped_cols_min(R, G)) return BSP_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(outer) || !aligned16(group_offsets) ||
        !aligned16(codesT) || !aligned16(scalesT) || !aligned16(outerT) || !aligned16_or_null(gather))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_requant_grouped(codes, scales, outer, src_rows, gather, group_offsets, G, R, K,
                                                  codesT, scalesT, ldT, outerT, seed, (flags & BSP_SR) != 0,
                                                  as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_requant_transpose_sr(const uint8_t *codes, const uint8_t *scales, const float *outer,
                                               int64_t M, int64_t K, uint8_t *codesT, uint8_t *scalesT,
                                               float *outerT, uint64_t seed, uint32_t flags, void *workspace,
                                               size_t ws_bytes, void *stream) {
    return bsp_requant_transpose_sr_batched(codes, scales, outer, 1, 1, M, K, codesT, scalesT, outerT, seed, flags,
                                            workspace, ws_bytes, stream);
}

namespace {

// Argument checks shared by the grouped GEMM entry points (everything but the
// workspace), before any HIP call.
bsp_status gemm_args_status(int fmt, int mode, const uint8_t *a_codes, const uint8_t *a_scales, const float *a_outer,
                            const int32_t *a_gather, int64_t a_rows, const int64_t *group_offsets, int64_t G,
                            int64_t M, int64_t N, int64_t K, const uint8_t *b_codes, const uint8_t *b_scales,
                            const float *b_outer, void *c, int c_dtype, int64_t ldc) {
    if (!a_codes || !a_scales || !b_codes || !b_scales || !group_offsets || !c) return BSP_ERR_INVALID_ARG;
    if (fmt != BSP_FMT_NVFP4 && fmt != BSP_FMT_MXFP8) return BSP_ERR_INVALID_ARG;
    if (mode != BSP_GEMM_FPROP && mode != BSP_GEMM_DGRAD && mode != BSP_GEMM_WGRAD) return BSP_ERR_INVALID_ARG;
    if (c_dtype != BSP_DTYPE_F32 && c_dtype != BSP_DTYPE_BF16) return BSP_ERR_INVALID_ARG;
    if (fmt == BSP_FMT_NVFP4 && (!a_outer || !b_outer)) return BSP_ERR_INVALID_ARG;
    if (fmt == BSP_FMT_MXFP8 && (a_outer || b_outer)) return BSP_ERR_INVALID_ARG;
    if (mode == BSP_GEMM_WGRAD && a_gather) return BSP_ERR_INVALID_ARG;
    if (G < 1 || M <= 0 || N <= 0 || K <= 0) return BSP_ERR_SHAPE;
    if (ldc < N) return BSP_ERR_SHAPE;
    if (G >= (1ll << 23) || M >= (1ll << 40)) return BSP_ERR_SHAPE;
    if (fmt == BSP_FMT_MXFP8 && K % 32) return BSP_ERR_SHAPE;
    if (fmt == BSP_FMT_NVFP4 && K % 32) return BSP_ERR_SHAPE;   // rows of codes 16-byte aligned
    // The kernel keeps sizes, tile counts and per-lane byte offsets in 32 bits.
    {
        const int64_t lim31 = (1ll << 31) - 1, lim32 = 1ll << 32;
        if (M > lim31 || N > lim31 || K > lim31 || ldc > lim31 || a_rows > lim31) return BSP_ERR_SHAPE;
        const int64_t rowb = fmt == BSP_FMT_MXFP8 ? K : K / 2;     // code bytes per row
        const int64_t sr = fmt == BSP_FMT_MXFP8 ? K / 32 : K / 16;  // scale bytes per row
        if (a_rows * rowb >= lim32 || N * rowb >= lim32) return BSP_ERR_SHAPE;
        if (mode != BSP_GEMM_WGRAD && G * N * sr >= lim32) return BSP_ERR_SHAPE;
        if (((M + 127) / 128 + G) * ((N + 127) / 128) > lim31) return BSP_ERR_SHAPE;
    }
    if (mode != BSP_GEMM_WGRAD && !a_gather && a_rows != M) return BSP_ERR_SHAPE;
    if (mode == BSP_GEMM_WGRAD && a_rows != M) return BSP_ERR_SHAPE;
    if (a_rows <= 0) return BSP_ERR_SHAPE;
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) || !aligned16(b_scales) ||
        !aligned16(group_offsets) || !aligned16(c) || !aligned16_or_null(a_outer) ||
        !aligned16_or_null(b_outer) || !aligned16_or_null(a_gather))
        return BSP_ERR_ALIGNMENT;
    return BSP_OK;
}

}  // namespace

BSP_EXPORT bsp_status bsp_moe_grouped_gemm_blockscaled_tiled(int fmt, int mode, const uint8_t *a_codes,
                                                             const uint8_t *a_scales, const float *a_outer,
                                                             const int32_t *a_gather, int64_t a_rows,
                                                             const int64_t *group_offsets, int64_t G, int64_t M,
                                                             int64_t N, int64_t K, const uint8_t *b_codes,
                                                             const uint8_t *b_scales, const float *b_outer, void *c,
                                                             int c_dtype, int64_t ldc, void *workspace,
                                                             size_t ws_bytes, int tile, void *stream) {
    if (tile != 0 && tile != 128 && tile != 256) return BSP_ERR_INVALID_ARG;
    const bsp_status st = gemm_args_status(fmt, mode, a_codes, a_scales, a_outer, a_gather, a_rows, group_offsets, G,
                                           M, N, K, b_codes, b_scales, b_outer, c, c_dtype, ldc);
    if (st != BSP_OK) return st;
    if (!workspace || ws_bytes < bsp_gemm_workspace_size(fmt, mode, M, N, K, G)) return BSP_ERR_WORKSPACE;
    if (!aligned16(workspace)) return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_gemm(fmt, mode, a_codes, a_scales, a_outer, a_gather, a_rows, group_offsets, G, M, N, K,
                                       b_codes, b_scales, b_outer, c, c_dtype, ldc, workspace, tile,
                                       as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_moe_grouped_gemm_blockscaled_noalloc(int fmt, int mode, const uint8_t *a_codes,
                                                               const uint8_t *a_scales, const float *a_outer,
                                                               const int32_t *a_gather, int64_t a_rows,
                                                               const int64_t *group_offsets, int64_t G, int64_t M,
                                                               int64_t N, int64_t K, const uint8_t *b_codes,
                                                               const uint8_t *b_scales, const float *b_outer,
                                                               void *c, int c_dtype, int64_t ldc, void *stream) {
    const bsp_status st = gemm_args_status(fmt, mode, a_codes, a_scales, a_outer, a_gather, a_rows, group_offsets, G,
                                           M, N, K, b_codes, b_scales, b_outer, c, c_dtype, ldc);
    if (st != BSP_OK) return st;
    if (bsp_gemm_workspace_size(fmt, mode, M, N, K, G) > (size_t)BSP_GEMM_SCRATCH_BYTES) return BSP_ERR_SCRATCH_LIMIT;
    void *scratch = bsp::gemm_scratch();
    if (scratch == nullptr) return BSP_ERR_HIP;
    return hip_status(bsp::launch_gemm(fmt, mode, a_codes, a_scales, a_outer, a_gather, a_rows, group_offsets, G, M, N, K,
                                       b_codes, b_scales, b_outer, c, c_dtype, ldc, scratch, 0, as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_moe_grouped_gemm_blockscaled(int fmt, int mode, const uint8_t *a_codes,
                                                       const uint8_t *a_scales, const float *a_outer,
                                                       const int32_t *a_gather, int64_t a_rows,
                                                       const int64_t *group_offsets, int64_t G, int64_t M, int64_t N,
                                                       int64_t K, const uint8_t *b_codes, const uint8_t *b_scales,
                                                       const float *b_outer, void *c, int c_dtype, int64_t ldc,
                                                       void *workspace, size_t ws_bytes, void *stream) {
    return bsp_moe_grouped_gemm_blockscaled_tiled(fmt, mode, a_codes, a_scales, a_outer, a_gather, a_rows,
                                                  group_offsets, G, M, N, K, b_codes, b_scales, b_outer, c, c_dtype,
                                                  ldc, workspace, ws_bytes, 0, stream);
}

BSP_EXPORT bsp_status bsp_moe_grouped_gemm_bf16_tiled(int mode, const uint16_t *a, int64_t lda,
                                                      const uint16_t *b, int64_t ldb, const int32_t *gather,
                                                      int64_t src_rows, const int64_t *group_offsets, int64_t G,
                                                      int64_t M, int64_t N, int64_t K, void *c, int c_dtype,
                                                      int64_t ldc, void *workspace, size_t ws_bytes, int tile,
                                                      void *stream) {
    if (tile != 0 && tile != 128 && tile != 256) return BSP_ERR_INVALID_ARG;
    if (!a || !b || !group_offsets || !c) return BSP_ERR_INVALID_ARG;
    if (mode != BSP_GEMM_FPROP && mode != BSP_GEMM_DGRAD && mode != BSP_GEMM_WGRAD) return BSP_ERR_INVALID_ARG;
    if (c_dtype != BSP_DTYPE_F32 && c_dtype != BSP_DTYPE_BF16) return BSP_ERR_INVALID_ARG;
    if (G < 1 || M <= 0 || N <= 0 || K <= 0 || src_rows <= 0 || ldc < N) return BSP_ERR_SHAPE;
    if (G >= (1ll << 23)) return BSP_ERR_SHAPE;
    const bool wg = mode == BSP_GEMM_WGRAD;
    // Operand rows are fetched in 16-byte pieces (8 elements) along their
    // contiguous dimension: K for K-major operands, M or N for MN-major ones.
    if (wg) {
        if (M % 8 || N % 8 || lda < M || ldb < N) return BSP_ERR_SHAPE;
        if (!gather && src_rows != K) return BSP_ERR_SHAPE;
    } else {
        if (K % 8 || lda < K) return BSP_ERR_SHAPE;
        if (mode == BSP_GEMM_FPROP && ldb < K) return BSP_ERR_SHAPE;
        if (mode == BSP_GEMM_DGRAD && (N % 8 || ldb < N)) return BSP_ERR_SHAPE;
        if (!gather && src_rows != M) return BSP_ERR_SHAPE;
    }
    // The kernel keeps sizes, tile counts and per-lane byte offsets in 32 bits.
    {
        const int64_t lim31 = (1ll << 31) - 1, lim32 = 1ll << 32;
        if (M > lim31 || N > lim31 || K > lim31 || ldc > lim31 || src_rows > lim31) return BSP_ERR_SHAPE;
        if (lda >= (1ll << 26) || ldb >= (1ll << 26)) return BSP_ERR_SHAPE;
        if (!wg && (src_rows * lda * 2 >= lim32 || (mode == BSP_GEMM_FPROP && N * ldb * 2 >= lim32)))
            return BSP_ERR_SHAPE;
        const int64_t tiles = wg ? G * ((M + 127) / 128) * ((N + 127) / 128) : ((M + 127) / 128 + G) * ((N + 127) / 128);
        if (tiles > lim31) return BSP_ERR_SHAPE;
    }
    if (!workspace || ws_bytes < bsp_gemm_bf16_workspace_size(mode, M, N, K, G)) return BSP_ERR_WORKSPACE;
    if (lda % 8 || ldb % 8) return BSP_ERR_ALIGNMENT;
    if (!aligned16(a) || !aligned16(b) || !aligned16(group_offsets) || !aligned16(c) || !aligned16(workspace) ||
        !aligned16_or_null(gather))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_gemm_bf16(mode, a, lda, b, ldb, gather, src_rows, group_offsets, G, M, N, K, c,
                                            c_dtype, ldc, workspace, tile, as_stream(stream)));
}

BSP_EXPORT bsp_status bsp_moe_grouped_gemm_bf16(int mode, const uint16_t *a, int64_t lda, const uint16_t *b,
                                                int64_t ldb, const int32_t *gather, int64_t src_rows,
                                                const int64_t *group_offsets, int64_t G, int64_t M, int64_t N,
                                                int64_t K, void *c, int c_dtype, int64_t ldc, void *workspace,
                                                size_t ws_bytes, void *stream) {
    return bsp_moe_grouped_gemm_bf16_tiled(mode, a, lda, b, ldb, gather, src_rows, group_offsets, G, M, N, K, c,
                                           c_dtype, ldc, workspace, ws_bytes, 0, stream);
}

BSP_EXPORT bsp_status bsp_swiglu_quantize(const void *h13, int in_dtype, int64_t R, int64_t I, uint16_t *h_out,
                                          int fmt, uint8_t *codes, uint8_t *scales, float *outer, uint32_t flags,
                                          void *stream) {
    if (!h13) return BSP_ERR_INVALID_ARG;
    if (in_dtype != BSP_DTYPE_F32 && in_dtype != BSP_DTYPE_BF16) return BSP_ERR_INVALID_ARG;
    if (fmt != -1 && fmt != BSP_FMT_NVFP4 && fmt != BSP_FMT_MXFP8) return BSP_ERR_INVALID_ARG;
    if (fmt == -1 && !h_out) return BSP_ERR_INVALID_ARG;
    if (fmt >= 0 && (!codes || !scales)) return BSP_ERR_INVALID_ARG;
    if (fmt == BSP_FMT_NVFP4 && !outer) return BSP_ERR_INVALID_ARG;
    if (flags & ~BSP_NVFP4_46) return BSP_ERR_INVALID_ARG;
    if ((flags & BSP_NVFP4_46) && fmt != BSP_FMT_NVFP4) return BSP_ERR_INVALID_ARG;
    if (R <= 0 || I <= 0 || I % 32 || I > 8192) return BSP_ERR_SHAPE;
    if (!aligned16(h13) || !aligned16_or_null(h_out) || !aligned16_or_null(codes) || !aligned16_or_null(scales) ||
        !aligned16_or_null(outer))
        return BSP_ERR_ALIGNMENT;
    return hip_status(bsp::launch_swiglu(h13, in_dtype, R, I, h_out, fmt, (flags & BSP_NVFP4_46) != 0,
                                         fmt >= 0 ? codes : nullptr, fmt >= 0 ? scales : nullptr,
                                         fmt == BSP_FMT_NVFP4 ? outer : nullptr, as_stream(stream)));
}

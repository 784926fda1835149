// bsp_internal.hpp -- launch entry points shared between the kernel files and
// the C ABI shim.  Arguments are validated by the shim before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsp.h"

namespace bsp {

hipError_t launch_quantize_nvfp4(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int64_t rps, uint8_t *codes,
                                 uint8_t *scales, float *outer, bool m46, hipStream_t s);
hipError_t launch_quantize_nvfp4_rht(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint32_t signs,
                                     uint8_t *codes, uint8_t *scales, float *outer, bool m46, hipStream_t s);
hipError_t launch_quantize_nvfp4_2d(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint8_t *codes,
                                    uint8_t *scales, float *outer, hipStream_t s);
hipError_t launch_quantize_mxfp8(const uint16_t *x, int64_t x_rows, int64_t K, int64_t ldx, const int32_t *gather,
                                 int64_t M, uint8_t *codes_row, uint8_t *scales_row, uint8_t *codes_colT,
                                 uint8_t *scales_colT, int64_t ld_colT, const int64_t *group_offsets, int64_t G,
                                 int64_t batch, hipStream_t s);
hipError_t launch_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t M,
                             int64_t K, int64_t rps, void *out, int out_dtype, hipStream_t s);
int requant_partials(int64_t n);
int64_t requant_workspace_floats(int64_t E, int64_t M, int64_t rps);
hipError_t launch_requant(const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t rps, int64_t E,
                          int64_t M, int64_t K, uint8_t *codesT, uint8_t *scalesT, float *outerT, uint64_t seed,
                          bool sr, float *part, hipStream_t s);
hipError_t launch_requant_grouped(const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t src_rows,
                                  const int32_t *gather, const int64_t *group_offsets, int64_t G, int64_t R,
                                  int64_t K, uint8_t *codesT, uint8_t *scalesT, int64_t ldT, float *outerT,
                                  uint64_t seed, bool sr, hipStream_t s);
hipError_t launch_swiglu(const void *h13, int in_dtype, int64_t R, int64_t I, uint16_t *h_out, int fmt, bool m46,
                         uint8_t *codes, uint8_t *scales, float *outer, hipStream_t s);
int64_t gemm_tile_count(int64_t M, int64_t G);
constexpr int64_t kGemmSchedSlots = 16;   // spare counters and the listed tile count
int64_t gemm_workspace_bytes(int fmt, int mode, int64_t M, int64_t N, int64_t K, int64_t G);
hipError_t launch_gemm(int fmt, int mode, const uint8_t *a_codes, const uint8_t *a_scales, const float *a_outer,
                       const int32_t *a_gather, int64_t a_rows, const int64_t *group_offsets, int64_t G,
                       int64_t M, int64_t N,
                       int64_t K, const uint8_t *b_codes, const uint8_t *b_scales, const float *b_outer, void *c,
                       int c_dtype, int64_t ldc, void *workspace, int tile, hipStream_t s);
void *gemm_scratch();   // device address of the static GEMM scratch on the current device (nullptr: failed)
int64_t gemm_bf16_workspace_bytes(int mode, int64_t M, int64_t G);
hipError_t launch_gemm_bf16(int mode, const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb,
                            const int32_t *gather, int64_t src_rows, const int64_t *group_offsets, int64_t G,
                            int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc, void *workspace,
                            int tile, hipStream_t s);

}  // namespace bsp

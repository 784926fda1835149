// bsp_quant.hip -- memory-bound kernels of the block-scaled path for gfx950:
// NVFP4 quantize (per token / per scope, standard or 4/6), MXFP8 quantize
// (rowwise + columnwise from one read, optionally grouped), dequantize,
// dequantize -> transpose -> requantize with stochastic rounding, and
// SwiGLU fused with the quantization of its output.
//
// Every kernel reads its input once with 16-byte loads, keeps block
// reductions inside a lane (one lane owns whole 16/32-value blocks, so the
// amax of a block needs no cross-lane traffic), and writes codes and scales
// with coalesced stores.  All arithmetic is IEEE f32 (no contraction, correctly
// rounded division), so codes and scales do not depend on launch geometry.
#include "bsp_device.hpp"
#include "bsp_internal.hpp"

namespace bsp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// --------------------------------------------------------------------------
// NVFP4
// --------------------------------------------------------------------------

struct Nvfp4Block {
    uint32_t lo, hi;  // 16 nibbles, element 2j in the low nibble of byte j
    uint32_t s;       // E4M3 code
};

__device__ __forceinline__ void unpack16(const uint4 (&v)[2], float (&xf)[16]) {
    const uint32_t w[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        xf[2 * i] = bf16_lo(w[i]);
        xf[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ float absmax16(const float (&xf)[16]) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(xf[i]));
    return a;
}

// Codes of one block at effective decode scale eff = E4M3(s) * g: each value
// times one correctly rounded reciprocal of eff, converted by
// V_CVT_SCALEF32_PK_FP4_F32 at scale 1 (byte i of the word written in place).
// A zero or subnormal eff flushes the block: reciprocal 0, so every code
// keeps only its sign, and scale 0.
__device__ __forceinline__ Nvfp4Block nvfp4_codes(const float (&xf)[16], uint32_t s, float &eff) {
    const bool ok = eff >= kFlushBelow;
    const float r = ok ? 1.0f / eff : 0.0f;
    Nvfp4Block b;
    b.s = ok ? s : 0u;
    eff = ok ? eff : 0.0f;
    b.lo = 0u;
    b.hi = 0u;
#define BSP_FP4_PAIR(W, I, J) W = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(W, xf[I] * r, xf[I + 1] * r, 1.0f, J)
    BSP_FP4_PAIR(b.lo, 0, 0);
    BSP_FP4_PAIR(b.lo, 2, 1);
    BSP_FP4_PAIR(b.lo, 4, 2);
    BSP_FP4_PAIR(b.lo, 6, 3);
    BSP_FP4_PAIR(b.hi, 8, 0);
    BSP_FP4_PAIR(b.hi, 10, 1);
    BSP_FP4_PAIR(b.hi, 12, 2);
    BSP_FP4_PAIR(b.hi, 14, 3);
#undef BSP_FP4_PAIR
    return b;
}

// One candidate block scale with divisor D (6: standard; 4: the "4" of 4/6):
// s = E4M3(a / (D g)) by V_CVT_PK_FP8_F32 (identical to e4m3_encode on the
// clamped input), decoded by V_CVT_F32_FP8 (exact).  g = 0 gives s = 0.
__device__ __forceinline__ Nvfp4Block nvfp4_candidate(const float (&xf)[16], float a, float g, float D,
                                                      float &eff) {
    const uint32_t s = g > 0.0f ? e4m3x2_hw(a / (D * g), 0.0f) & 0xFFu : 0u;
    eff = __builtin_amdgcn_cvt_f32_fp8((int)s, 0) * g;
    return nvfp4_codes(xf, s, eff);
}

// Sum of squared reconstruction errors in index order with fused
// multiply-adds, d_i = x_i - value(q_i) * eff; the codes are decoded two at a
// time by V_CVT_SCALEF32_PK_F32_FP4 at scale 1 (exact).
__device__ __forceinline__ float nvfp4_sse(const float (&xf)[16], const Nvfp4Block &b, float eff) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 v[8];
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.lo, 1.0f, 0);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.lo, 1.0f, 1);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.lo, 1.0f, 2);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.lo, 1.0f, 3);
    v[4] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.hi, 1.0f, 0);
    v[5] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.hi, 1.0f, 1);
    v[6] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.hi, 1.0f, 2);
    v[7] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.hi, 1.0f, 3);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float d0 = __builtin_fmaf(-v[i].x, eff, xf[2 * i]);
        acc = __builtin_fmaf(d0, d0, acc);
        const float d1 = __builtin_fmaf(-v[i].y, eff, xf[2 * i + 1]);
        acc = __builtin_fmaf(d1, d1, acc);
    }
    return acc;
}

// 4/6: both candidate scales come from one two-value conversion.
template <bool M46>
__device__ __forceinline__ Nvfp4Block nvfp4_block(const float (&xf)[16], float g) {
    const float a = absmax16(xf);
    float eff6;
    if (!M46) return nvfp4_candidate(xf, a, g, 6.0f, eff6);
    const uint32_t s2 = g > 0.0f ? e4m3x2_hw(a / (6.0f * g), a / (4.0f * g)) : 0u;
    eff6 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 0) * g;
    float eff4 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 1) * g;
    const Nvfp4Block b6 = nvfp4_codes(xf, s2 & 0xFFu, eff6);
    const Nvfp4Block b4 = nvfp4_codes(xf, (s2 >> 8) & 0xFFu, eff4);
    const float e6 = nvfp4_sse(xf, b6, eff6);
    const float e4 = nvfp4_sse(xf, b4, eff4);
    return (e4 < e6) ? b4 : b6;
}

// 16-point random Hadamard transform of one block in f32: negate the
// elements whose bit is set in `signs`, Walsh-Hadamard butterflies (a, b) ->
// (a + b, a - b) at distances 1, 2, 4, 8, then scale by 1/4 (exact): an
// orthonormal transform, so two operands transformed along their common K
// give the same product.
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t signs) {
#pragma unroll
    for (int i = 0; i < 16; i++)
        if ((signs >> i) & 1u) v[i] = -v[i];
#pragma unroll
    for (int h = 1; h < 16; h *= 2)
#pragma unroll
        for (int j = 0; j < 16; j += 2 * h)
#pragma unroll
            for (int i = j; i < j + h; i++) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] *= 0.25f;
}

// Outer scope = one row, whole row kept in registers: LPR lanes per row (64,
// or 32 / 16 for short rows so that few lanes idle), lane l of a row owning
// the 16-value blocks starting at k = 16 LPR j + 16 l.  RHT: every block
// transformed first (the row's scale from the transformed values).
template <bool M46, int MAXIT, bool RHT = false, int LPR = 64, int NR = 1>
__global__ __launch_bounds__(256) void k_nvfp4_row(const uint16_t *__restrict__ x, int64_t M, int64_t K,
                                                   int64_t ldx, uint8_t *__restrict__ codes,
                                                   uint8_t *__restrict__ scales, float *__restrict__ outer,
                                                   uint32_t signs = 0) {
    // NR rows per lane group, RPW apart, all loaded before the first is
    // quantized (straight-line code): the later rows' loads overlap the
    // earlier rows' arithmetic, which matters when every workgroup of the
    // launch is resident at once (short tensors).
    constexpr int RPW = 64 / LPR;               // rows per wavefront and pass
    const int lane = threadIdx.x & (LPR - 1);
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW * NR + (threadIdx.x & 63) / LPR;
    if (row0 >= M) return;                      // whole row groups leave together
    uint4 v[NR][MAXIT][2];
#pragma unroll
    for (int q = 0; q < NR; q++) {
        // NR > 1: every load is issued, from a clamped (valid) address, so
        // that the count of loads in flight does not depend on the path and
        // the first row's wait leaves the later rows' loads outstanding;
        // pieces past M or K are never used
        const int64_t rq = row0 + q * RPW, row = NR > 1 && rq >= M ? M - 1 : rq;
#pragma unroll
        for (int j = 0; j < MAXIT; j++) {
            const int64_t kq = (int64_t)j * 16 * LPR + lane * 16, k0 = NR > 1 && kq >= K ? K - 16 : kq;
            if (NR > 1 || (row < M && k0 < K)) {
                v[q][j][0] = *reinterpret_cast<const uint4 *>(x + row * ldx + k0);
                v[q][j][1] = *reinterpret_cast<const uint4 *>(x + row * ldx + k0 + 8);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < NR; q++) {
        const int64_t row = row0 + q * RPW;
        if (row >= M) break;                    // uniform within the lane group
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < MAXIT; j++) {
            const int64_t k0 = (int64_t)j * 16 * LPR + lane * 16;
            if (k0 < K) {
                float xf[16];
                unpack16(v[q][j], xf);
                if (RHT) rht16(xf, signs);
                amax = fmaxf(amax, absmax16(xf));
            }
        }
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const float g = (amax == 0.0f) ? 0.0f : amax / 2688.0f;
        if (lane == 0) outer[row] = g;
#pragma unroll
        for (int j = 0; j < MAXIT; j++) {
            const int64_t k0 = (int64_t)j * 16 * LPR + lane * 16;
            if (k0 < K) {
                float xf[16];
                unpack16(v[q][j], xf);
                if (RHT) rht16(xf, signs);
                Nvfp4Block b = nvfp4_block<M46>(xf, g);
                *reinterpret_cast<uint2 *>(codes + row * (K / 2) + k0 / 2) = make_uint2(b.lo, b.hi);
                scales[row * (K / 16) + k0 / 16] = (uint8_t)b.s;
            }
        }
    }
}

// Per-token launch: lanes per row and blocks per lane from the block count
// nb = K / 16 (K <= 8192), so that at most a quarter of the lanes idle for
// the row lengths of the MoE layers (768 ... 8192).
template <bool M46, bool RHT>
static void launch_nvfp4_row(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint8_t *codes, uint8_t *scales,
                             float *outer, uint32_t signs, hipStream_t s) {
    const int64_t nb = K / 16;
    auto go = [&](auto kern, int lpr, int nr) {
        const int64_t rows_per_wg = 4 * (64 / lpr) * nr;
        kern<<<dim3((unsigned)((M + rows_per_wg - 1) / rows_per_wg)), 256, 0, s>>>(x, M, K, ldx, codes, scales,
                                                                                     outer, signs);
    };
    // K = 1537..2048 (the activations of the MoE layers): two rows per
    // wavefront while one each would keep at most ~8 workgroups per CU
    if (nb > 96 && nb <= 128) {
        if ((M + 3) / 4 <= 2048) go(k_nvfp4_row<M46, 2, RHT, 64, 2>, 64, 2);
        else go(k_nvfp4_row<M46, 2, RHT, 64>, 64, 1);
        return;
    }
    auto go1 = [&](auto kern, int lpr) { go(kern, lpr, 1); };
    if (nb <= 16) go1(k_nvfp4_row<M46, 1, RHT, 16>, 16);
    else if (nb <= 32) go1(k_nvfp4_row<M46, 1, RHT, 32>, 32);
    else if (nb <= 48) go1(k_nvfp4_row<M46, 3, RHT, 16>, 16);
    else if (nb <= 64) go1(k_nvfp4_row<M46, 1, RHT, 64>, 64);
    else if (nb <= 96) go1(k_nvfp4_row<M46, 3, RHT, 32>, 32);
    else if (nb <= 192) go1(k_nvfp4_row<M46, 3, RHT, 64>, 64);
    else go1(k_nvfp4_row<M46, 8, RHT, 64>, 64);
}

// 16x16 2-D blocks under one per-tensor outer scale (outer[0], computed
// before): workgroup (column tile of 256, band of 16 rows); thread 16 j + r
// owns row r of tile j (16 values), the tile's amax is a 16-lane maximum, and
// each row piece is quantized as a 1x16 block under the tile's scale.
__global__ __launch_bounds__(256) void k_nvfp4_2d(const uint16_t *__restrict__ x, int64_t K, int64_t ldx,
                                                  uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                  const float *__restrict__ outer) {
    const int t = threadIdx.x, j = t >> 4, r = t & 15;
    const int64_t row = (int64_t)blockIdx.y * 16 + r, k0 = (int64_t)blockIdx.x * 256 + 16 * j;
    const bool live = k0 < K;
    float xf[16];
    float a = 0.0f;
    if (live) {
        uint4 v[2];
        v[0] = *reinterpret_cast<const uint4 *>(x + row * ldx + k0);
        v[1] = *reinterpret_cast<const uint4 *>(x + row * ldx + k0 + 8);
        unpack16(v, xf);
        a = absmax16(xf);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
    if (!live) return;
    float eff;
    const Nvfp4Block b = nvfp4_candidate(xf, a, outer[0], 6.0f, eff);
    *reinterpret_cast<uint2 *>(codes + row * (K / 2) + k0 / 2) = make_uint2(b.lo, b.hi);
    if (r == 0) scales[(int64_t)blockIdx.y * (K / 16) + k0 / 16] = (uint8_t)b.s;
}

// Scope amax for scopes of several rows (or rows too long to keep in
// registers).  Block (scope, slice) reduces one contiguous slice of a scope
// and issues one atomic max of the non-negative f32 bit pattern (ordered like
// an unsigned integer) into `outer`, which holds zero on entry.
__global__ __launch_bounds__(256) void k_scope_amax(const uint16_t *__restrict__ x, int64_t K, int64_t ldx,
                                                    int64_t rows_per_scale, float *outer) {
    const int64_t scope = blockIdx.x;
    const int64_t nblk_row = K / 16;
    const int64_t nblk = rows_per_scale * nblk_row;
    const int64_t chunk = (nblk + gridDim.y - 1) / gridDim.y;
    const int64_t b0 = (int64_t)blockIdx.y * chunk;
    const int64_t b1 = b0 + chunk < nblk ? b0 + chunk : nblk;
    float a = 0.0f;
    for (int64_t b = b0 + threadIdx.x; b < b1; b += blockDim.x) {
        const int64_t r = scope * rows_per_scale + b / nblk_row, kb = b % nblk_row;
        uint4 v[2];
        v[0] = *reinterpret_cast<const uint4 *>(x + r * ldx + kb * 16);
        v[1] = *reinterpret_cast<const uint4 *>(x + r * ldx + kb * 16 + 8);
        float xf[16];
        unpack16(v, xf);
        a = fmaxf(a, absmax16(xf));
    }
    a = wave_max(a);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if (a > 0.0f) atomicMax(reinterpret_cast<unsigned int *>(outer + scope), __float_as_uint(a));
    }
}

__global__ void k_fill_f32(float *p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// outer[s] holds amax; turn it into the decode scale g = amax / 2688.
__global__ void k_amax_to_g(float *outer, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const float a = outer[i];
        outer[i] = (a == 0.0f) ? 0.0f : a / 2688.0f;
    }
}

// Quantize with precomputed outer scales: one lane per 16-value block.
template <bool M46>
__global__ __launch_bounds__(256) void k_nvfp4_blocks(const uint16_t *__restrict__ x, int64_t M, int64_t K,
                                                      int64_t ldx, int64_t rows_per_scale,
                                                      uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                      const float *__restrict__ outer) {
    const int64_t nblk_row = K / 16;
    const int64_t total = M * nblk_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nblk_row, kb = i - r * nblk_row;
        uint4 v[2];
        v[0] = *reinterpret_cast<const uint4 *>(x + r * ldx + kb * 16);
        v[1] = *reinterpret_cast<const uint4 *>(x + r * ldx + kb * 16 + 8);
        float xf[16];
        unpack16(v, xf);
        Nvfp4Block b = nvfp4_block<M46>(xf, outer[r / rows_per_scale]);
        *reinterpret_cast<uint2 *>(codes + r * (K / 2) + kb * 8) = make_uint2(b.lo, b.hi);
        scales[r * nblk_row + kb] = (uint8_t)b.s;
    }
}

static int grid_for(int64_t work, int per_block = 256, int cap = 65536) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    return (int)(g > cap ? cap : g);
}

hipError_t launch_quantize_nvfp4_rht(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint32_t signs,
                                     uint8_t *codes, uint8_t *scales, float *outer, bool m46, hipStream_t s) {
    if (m46) launch_nvfp4_row<true, true>(x, M, K, ldx, codes, scales, outer, signs, s);
    else launch_nvfp4_row<false, true>(x, M, K, ldx, codes, scales, outer, signs, s);
    return hipGetLastError();
}

static hipError_t launch_scope_outer(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int64_t rps, float *outer,
                                     hipStream_t s);

hipError_t launch_quantize_nvfp4_2d(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint8_t *codes,
                                    uint8_t *scales, float *outer, hipStream_t s) {
    const hipError_t e = launch_scope_outer(x, M, K, ldx, M, outer, s);
    if (e != hipSuccess) return e;
    k_nvfp4_2d<<<dim3((unsigned)((K + 255) / 256), (unsigned)(M / 16)), 256, 0, s>>>(x, K, ldx, codes, scales, outer);
    return hipGetLastError();
}

// Outer scales of scopes of rps rows: amax per scope, then g = amax / 2688.
static hipError_t launch_scope_outer(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int64_t rps, float *outer,
                                     hipStream_t s) {
    const int64_t nscope = M / rps;
    k_fill_f32<<<grid_for(nscope), 256, 0, s>>>(outer, nscope, 0.0f);
    const int64_t per_scope = rps * (K / 16);
    int64_t slices = (2048 + nscope - 1) / nscope;                     // about 2048 blocks in flight
    const int64_t max_slices = (per_scope + 1023) / 1024;              // at least 1024 16-blocks each
    slices = slices < max_slices ? slices : max_slices;
    slices = slices < 1 ? 1 : (slices > 65535 ? 65535 : slices);
    k_scope_amax<<<dim3((unsigned)nscope, (unsigned)slices), 256, 0, s>>>(x, K, ldx, rps, outer);
    k_amax_to_g<<<grid_for(nscope), 256, 0, s>>>(outer, nscope);
    return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int64_t rps, uint8_t *codes,
                                 uint8_t *scales, float *outer, bool m46, hipStream_t s) {
    if (rps == 1 && K <= 8192) {
        if (m46) launch_nvfp4_row<true, false>(x, M, K, ldx, codes, scales, outer, 0u, s);
        else launch_nvfp4_row<false, false>(x, M, K, ldx, codes, scales, outer, 0u, s);
        return hipGetLastError();
    }
    const hipError_t e = launch_scope_outer(x, M, K, ldx, rps, outer, s);
    if (e != hipSuccess) return e;
    const int64_t nblk = M * (K / 16);
    if (m46) k_nvfp4_blocks<true><<<grid_for(nblk, 256, 16384), 256, 0, s>>>(x, M, K, ldx, rps, codes, scales, outer);
    else k_nvfp4_blocks<false><<<grid_for(nblk, 256, 16384), 256, 0, s>>>(x, M, K, ldx, rps, codes, scales, outer);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// MXFP8
// --------------------------------------------------------------------------

// Quantize 32 values (f32) sharing one E8M0 scale; returns the scale code.
__device__ __forceinline__ uint32_t mxfp8_block(const float (&xf)[32], uint32_t (&q)[8]) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) a = fmaxf(a, fabsf(xf[i]));
    const int k = mx_block_exponent(a);
    // 2^-k is a normal f32 for k in [-127, 119]; the product is exact unless it
    // falls below 2^-126, far under E4M3's rounding threshold.
    const float inv = exp2i(-k);
#pragma unroll
    for (int w = 0; w < 8; w++)
        q[w] = e4m3x4_hw(xf[4 * w] * inv, xf[4 * w + 1] * inv, xf[4 * w + 2] * inv, xf[4 * w + 3] * inv);
    return (uint32_t)(k + 127);
}

constexpr int MX_TR = 128;  // tile rows (padded row space)
constexpr int MX_TC = 128;  // tile columns

// One 128 x 128 tile: rowwise blocks (32 along K) straight from registers and
// columnwise blocks (32 along rows) through LDS, from a single read of x.
// Loads and rowwise stores cover whole rows per instruction (16 lanes per
// 256-byte input row, 8 bytes of codes each); column codes are staged in LDS
// and written back in whole 128-byte rows.
// Grouped: tile rows live in the padded row space; 32-row block b belongs to
// the group g with P[g] <= 32 b < P[g + 1] and reads source row
// off[g] + (p - P[g]) (zero past the group).  The grouped grid is 1-D and
// XCD-aware: workgroup L runs tile v = (L % 8) * chunk + L / 8 of the
// column-major tile order (all row tiles of a column tile, then the next),
// so each XCD works through its own run of column tiles and the workgroups
// resident on it share one column slab of x in its L2 -- what a gathered
// input re-reads (every token appears once per routed copy).
template <bool ROW, bool COL, bool GROUPED, bool GATHER = GROUPED>
__global__ __launch_bounds__(256) void k_mxfp8_tile(const uint16_t *__restrict__ x, int64_t M, int64_t K,
                                                    int64_t ldx, uint8_t *__restrict__ codes_row,
                                                    uint8_t *__restrict__ scales_row, uint8_t *__restrict__ codes_colT,
                                                    uint8_t *__restrict__ scales_colT, int64_t ld_colT,
                                                    const int64_t *__restrict__ group_offsets, int G,
                                                    const int32_t *__restrict__ gather, int64_t x_rows) {
    // Tile rows map to rows of x through LDS tables only when they are not
    // the identity (groups or a gather); the plain form then needs 32 KB of
    // LDS in all, so five workgroups fit a compute unit.
    constexpr bool MAP = GROUPED || GATHER;
    __shared__ __attribute__((aligned(16))) uint16_t tile[COL ? MX_TR : 1][MX_TC];
    __shared__ int64_t rsrc[ROW && MAP ? MX_TR : 1];   // destination row of each tile row in codes_row (-1: none)
    __shared__ int64_t xsrc[MAP ? MX_TR : 1];           // row of x of each tile row (-1: zeros)
    __shared__ int64_t blk_src0[GROUPED ? MX_TR / 32 : 1], blk_end[GROUPED ? MX_TR / 32 : 1];
    __shared__ int64_t wsum[GROUPED ? 4 : 1];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int64_t p0, k0;
    if (GROUPED) {
        const int64_t gx = (K + MX_TC - 1) / MX_TC, gy = (ld_colT + MX_TR - 1) / MX_TR, n = gx * gy;
        const int64_t chunk = (n + 7) / 8, v = (int64_t)(blockIdx.x % 8) * chunk + blockIdx.x / 8;
        if (v >= n) return;
        k0 = (v / gy) * MX_TC;
        p0 = (v % gy) * MX_TR;
    } else {
        p0 = (int64_t)blockIdx.y * MX_TR;
        k0 = (int64_t)blockIdx.x * MX_TC;
    }
    int64_t ptotal = M;
    if (!GROUPED && gridDim.z > 1) {  // stacked independent matrices (no gather, no groups)
        const int64_t b = blockIdx.z;
        x += b * x_rows * ldx;
        if (codes_row) {
            codes_row += b * M * K;
            scales_row += b * M * (K / 32);
        }
        if (COL) {
            codes_colT += b * K * ld_colT;
            scales_colT += b * K * (ld_colT / 32);
        }
    }

    if (GROUPED) {
        // Thread t owns groups [t per, t per + per): a block-wide scan of their
        // padded sizes gives the padded start of its first group, and the
        // thread whose groups cover one of this tile's four 32-row blocks
        // resolves that block's first source row and group end.
        const int per = (G + 255) / 256;
        const int g0 = t * per, g1 = g0 + per < G ? g0 + per : G;
        int64_t local = 0;
        for (int g = g0; g < g1; g++) local += (group_offsets[g + 1] - group_offsets[g] + 31) / 32 * 32;
        const int64_t incl = wave_incl_scan(local, lane);
        if (lane == 63) wsum[wv] = incl;
        if (t < MX_TR / 32) {
            blk_src0[t] = 0;
            blk_end[t] = 0;
        }
        __syncthreads();
        int64_t run = incl - local;
        for (int w = 0; w < wv; w++) run += wsum[w];
        ptotal = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        if (local > 0 && run < p0 + MX_TR && run + local > p0) {
            for (int g = g0; g < g1; g++) {
                const int64_t o0 = group_offsets[g], o1 = group_offsets[g + 1];
                const int64_t pn = (o1 - o0 + 31) / 32 * 32;
#pragma unroll
                for (int b = 0; b < MX_TR / 32; b++) {
                    const int64_t pb = p0 + 32 * b;
                    if (pb >= run && pb < run + pn) {
                        blk_src0[b] = o0 + (pb - run);
                        blk_end[b] = o1 < M ? o1 : M;   // offsets past M are never read
                    }
                }
                run += pn;
            }
        }
        __syncthreads();
        if (p0 >= ptotal) return;
    }

    // ---- per-row sources: destination row of codes_row and row of x ----
    if constexpr (MAP) {
      if (t < MX_TR) {
        const int64_t p = p0 + t;
        int64_t src = -1;
        if (GROUPED) {
            const int b = t >> 5;
            const int64_t s_ = blk_src0[b] + (t & 31);
            if (p < ptotal && s_ >= 0 && s_ < blk_end[b]) src = s_;
        } else {
            if (p < M) src = p;
        }
        if constexpr (ROW) rsrc[t] = src;
        // physical row of x: the gathered row (out-of-range indices read as zeros)
        int64_t xrow = src;
        if (src >= 0 && gather) {
            xrow = gather[src];
            if (xrow < 0 || xrow >= x_rows) xrow = -1;
        }
        xsrc[t] = xrow;
      }
      __syncthreads();
    }
    // identity map: tile row r is row p0 + r (none past M)
    auto x_row = [&](int r) -> int64_t { return MAP ? xsrc[r] : (p0 + r < M ? p0 + r : -1); };
    auto dst_row = [&](int r) -> int64_t { return MAP ? rsrc[ROW && MAP ? r : 0] : (p0 + r < M ? p0 + r : -1); };

    // ---- load: lane l of wavefront w reads 16-byte chunk l % 16 of tile row
    // 32 w + 4 i + l / 16 (i = 0..7), so each load covers four whole 256-byte
    // rows.  A 32-value block is the chunks of four neighbouring lanes. ----
    const int ch = lane & 15, rq = lane >> 4;
    const int64_t kc = k0 + 8 * ch;
    const bool col_ok = kc < K;   // K % 32 == 0: a block's four lanes agree
    // A gathered x is read once per routed copy of each row: those loads keep
    // the default cache policy so the copies after the first hit in L2; an
    // x read once streams past the caches (non-temporal).
    const bool reread = GATHER && gather != nullptr;
    uint4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t xr = x_row(32 * wv + 4 * i + rq);
        raw[i] = make_uint4(0u, 0u, 0u, 0u);
        if (xr >= 0 && col_ok) {
            const u32x4 *px = reinterpret_cast<const u32x4 *>(x + xr * ldx + kc);
            const u32x4 v = reread ? *px : __builtin_nontemporal_load(px);
            raw[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
    if (ROW) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
            float xf[8];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xf[2 * j] = bf16_lo(w[j]);
                xf[2 * j + 1] = bf16_hi(w[j]);
            }
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) a = fmaxf(a, fabsf(xf[j]));
            a = fmaxf(a, __shfl_xor(a, 1, 64));
            a = fmaxf(a, __shfl_xor(a, 2, 64));
            const int k = mx_block_exponent(a);
            const float inv = exp2i(-k);   // see mxfp8_block
            const uint32_t q0 = e4m3x4_hw(xf[0] * inv, xf[1] * inv, xf[2] * inv, xf[3] * inv);
            const uint32_t q1 = e4m3x4_hw(xf[4] * inv, xf[5] * inv, xf[6] * inv, xf[7] * inv);
            const int64_t dr = dst_row(32 * wv + 4 * i + rq);
            if (dr >= 0 && col_ok) {
                __builtin_nontemporal_store(u32x2{q0, q1}, reinterpret_cast<u32x2 *>(codes_row + dr * K + kc));
                if ((ch & 3) == 0) scales_row[dr * (K / 32) + kc / 32] = (uint8_t)(k + 127);
            }
        }
    }
    if constexpr (!COL) return;   // rowwise copy only
#pragma unroll
    for (int i = 0; i < 8; i++) *reinterpret_cast<uint4 *>(&tile[32 * wv + 4 * i + rq][8 * ch]) = raw[i];
    __syncthreads();

    // ---- columns: thread t owns column t % 128, rows [64 (t / 128), +64): two 32-blocks ----
    const int c = t & 127, rh = t >> 7;
    const int64_t kcol = k0 + c;
    const int64_t plimit = GROUPED ? ptotal : M;
    uint32_t qcol[16];
    {
        uint32_t scs = 0;
        int nvalid = 0;
#pragma unroll
        for (int b = 0; b < 2; b++) {
            const int64_t pb = p0 + 64 * rh + 32 * b;
            float cf[32];
#pragma unroll
            for (int i = 0; i < 32; i++) cf[i] = __uint_as_float((uint32_t)tile[64 * rh + 32 * b + i][c] << 16);
            uint32_t q[8];
            const uint32_t sc = mxfp8_block(cf, q);
#pragma unroll
            for (int i = 0; i < 8; i++) qcol[8 * b + i] = q[i];
            if (pb < plimit) {
                scs |= sc << (8 * b);
                nvalid = b + 1;
            }
        }
        if (kcol < K && nvalid > 0) {
            uint8_t *sp = scales_colT + kcol * (ld_colT / 32) + (p0 + 64 * rh) / 32;
            if (nvalid == 2 && (reinterpret_cast<uintptr_t>(sp) & 1) == 0) {
                *reinterpret_cast<uint16_t *>(sp) = (uint16_t)scs;
            } else {
                for (int b = 0; b < nvalid; b++) sp[b] = (uint8_t)(scs >> (8 * b));
            }
        }
    }
    __syncthreads();   // the input tile is no longer read

    // ---- stage the column codes in LDS, then write them back with every
    // store instruction covering whole 128-byte rows (8 lanes per row):
    // lane-scattered 16-byte stores would cost one L2 request each ----
    // (16-byte piece q of staged row c sits at piece q ^ ((c >> 1) & 7): the
    // 64 lanes of a wavefront write rows 128 bytes apart, which without the
    // swizzle would put every lane's piece on the same two groups of banks)
    uint8_t *stage = reinterpret_cast<uint8_t *>(&tile[0][0]);
    {
        const int sw = (c >> 1) & 7;
#pragma unroll
        for (int i = 0; i < 4; i++)
            *reinterpret_cast<uint4 *>(stage + c * 128 + 16 * ((4 * rh + i) ^ sw)) =
                make_uint4(qcol[4 * i], qcol[4 * i + 1], qcol[4 * i + 2], qcol[4 * i + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int id = 256 * i + t, r = id >> 3, piece = id & 7;
        const uint4 v = *reinterpret_cast<const uint4 *>(stage + r * 128 + 16 * (piece ^ ((r >> 1) & 7)));
        if (k0 + r < K && p0 + 16 * piece < plimit)
            __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<u32x4 *>(codes_colT + (k0 + r) * ld_colT + p0 + 16 * piece));
    }
}

// Rowwise-only MXFP8: one lane per 32-value block.
__global__ __launch_bounds__(256) void k_mxfp8_row(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
                                                   uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                   const int32_t *__restrict__ gather, int64_t x_rows) {
    const int64_t nb = K / 32, total = M * nb;
    if (gridDim.z > 1) {  // stacked independent matrices
        const int64_t b = blockIdx.z;
        x += b * x_rows * ldx;
        codes += b * M * K;
        scales += b * M * nb;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nb, kb = i - r * nb;
        int64_t xr = r;
        if (gather) {
            xr = gather[r];
            if (xr < 0 || xr >= x_rows) xr = -1;
        }
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (xr < 0 ? 0 : xr) * ldx + kb * 32);
        float xf[32];
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const uint4 raw = xr < 0 ? make_uint4(0u, 0u, 0u, 0u) : src[v];
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xf[8 * v + 2 * j] = bf16_lo(w[j]);
                xf[8 * v + 2 * j + 1] = bf16_hi(w[j]);
            }
        }
        uint32_t q[8];
        const uint32_t sc = mxfp8_block(xf, q);
        uint4 *dst = reinterpret_cast<uint4 *>(codes + r * K + kb * 32);
        dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
        dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
        scales[i] = (uint8_t)sc;
    }
}

hipError_t launch_quantize_mxfp8(const uint16_t *x, int64_t x_rows, int64_t K, int64_t ldx, const int32_t *gather,
                                 int64_t M, uint8_t *codes_row, uint8_t *scales_row, uint8_t *codes_colT,
                                 uint8_t *scales_colT, int64_t ld_colT, const int64_t *group_offsets, int64_t G,
                                 int64_t batch, hipStream_t s) {
    const bool row = codes_row != nullptr, col = codes_colT != nullptr;
    const unsigned gx = (unsigned)((K + MX_TC - 1) / MX_TC);
    if (!col && M * K * batch < (int64_t(1) << 26)) {
        // a short rowwise-only tensor (less than one pass of 128 x 128 tiles
        // over the GPU's workgroup slots): one lane per block, more and
        // shorter work units
        const int gxr = grid_for(M * (K / 32), 256, batch > 1 ? 4096 : (1 << 20));
        k_mxfp8_row<<<dim3(gxr, 1, (unsigned)batch), 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row, gather,
                                                                   x_rows);
        return hipGetLastError();
    }
    if (!col) {   // rowwise only: the tile kernel without its column pass (whole-row loads and stores)
        const dim3 grid(gx, (unsigned)((M + MX_TR - 1) / MX_TR), (unsigned)batch);
        if (gather)
            k_mxfp8_tile<true, false, false, true><<<grid, 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row, nullptr,
                                                                       nullptr, 0, nullptr, 1, gather, x_rows);
        else
            k_mxfp8_tile<true, false, false, false><<<grid, 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row, nullptr,
                                                                        nullptr, 0, nullptr, 1, nullptr, x_rows);
        return hipGetLastError();
    }
    if (group_offsets) {
        // 1-D XCD-aware grid: 8 runs of ceil(tiles / 8) workgroups
        const int64_t tiles = (int64_t)gx * ((ld_colT + MX_TR - 1) / MX_TR);
        const unsigned nwg = (unsigned)(8 * ((tiles + 7) / 8));
        if (row)
            k_mxfp8_tile<true, true, true><<<dim3(nwg), 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row,
                                                                     codes_colT, scales_colT, ld_colT,
                                                                     group_offsets, (int)G, gather, x_rows);
        else
            k_mxfp8_tile<false, true, true><<<dim3(nwg), 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row,
                                                                      codes_colT, scales_colT, ld_colT,
                                                                      group_offsets, (int)G, gather, x_rows);
    } else {
        const unsigned gy = (unsigned)((M + MX_TR - 1) / MX_TR);
        const dim3 grid(gx, gy, (unsigned)batch);
        if (gather) {
            if (row)
                k_mxfp8_tile<true, true, false, true><<<grid, 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row,
                                                                          codes_colT, scales_colT, ld_colT, nullptr,
                                                                          1, gather, x_rows);
            else
                k_mxfp8_tile<false, true, false, true><<<grid, 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row,
                                                                           codes_colT, scales_colT, ld_colT, nullptr,
                                                                           1, gather, x_rows);
        } else {
            if (row)
                k_mxfp8_tile<true, true, false, false><<<grid, 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row,
                                                                           codes_colT, scales_colT, ld_colT,
                                                                           nullptr, 1, nullptr, x_rows);
            else
                k_mxfp8_tile<false, true, false, false><<<grid, 256, 0, s>>>(x, M, K, ldx, codes_row, scales_row,
                                                                            codes_colT, scales_colT, ld_colT,
                                                                            nullptr, 1, nullptr, x_rows);
        }
    }
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Dequantize
// --------------------------------------------------------------------------

// bf16 output: one lane per half block (8 values), so that a store
// instruction covers 1 KB of output contiguously; values decoded two at a
// time by V_CVT_SCALEF32_PK_F32_FP4 at scale 1 (exact), scaled in f32 and
// rounded to bf16 (RNE) in pairs, stored non-temporally (the output is a
// stream the GEMM reads later, far beyond the caches).
__global__ __launch_bounds__(256) void k_dequant_nvfp4_bf16(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            const float *__restrict__ outer, int64_t M, int64_t K,
                                                            int64_t rps, uint16_t *__restrict__ out) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    const int64_t nb = K / 16, total = 2 * M * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t blk = i >> 1, r = blk / nb;
        const float eff = e4m3_decode(scales[blk]) * outer[r / rps];
        const uint32_t c = reinterpret_cast<const uint32_t *>(codes)[i];
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const auto v = j == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0)
                         : j == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1)
                         : j == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2)
                                  : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
            w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[0] * eff, v[1] * eff}, bf2));
        }
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4 *>(out + i * 8));
    }
}

// f32 output: one lane per 16-value block.
__global__ __launch_bounds__(256) void k_dequant_nvfp4_f32(const uint8_t *__restrict__ codes,
                                                           const uint8_t *__restrict__ scales,
                                                           const float *__restrict__ outer, int64_t M, int64_t K,
                                                           int64_t rps, float *__restrict__ out) {
    const int64_t nb = K / 16, total = M * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nb;
        const float eff = e4m3_decode(scales[i]) * outer[r / rps];
        const uint2 c = *reinterpret_cast<const uint2 *>(codes + i * 8);
        float y[16];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            y[j] = e2m1_value((c.x >> (4 * j)) & 15u) * eff;
            y[8 + j] = e2m1_value((c.y >> (4 * j)) & 15u) * eff;
        }
        float4 *d = reinterpret_cast<float4 *>(out + i * 16);
#pragma unroll
        for (int j = 0; j < 4; j++) d[j] = make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
    }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant_mxfp8(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ scales, int64_t M, int64_t K,
                                                       void *__restrict__ out) {
    const int64_t nb = K / 32, total = M * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int k = (int)scales[i] - 127;
        const uint4 *cp = reinterpret_cast<const uint4 *>(codes + i * 32);
        const uint4 c0 = cp[0], c1 = cp[1];
        const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        float y[32];
#pragma unroll
        for (int j = 0; j < 32; j++) y[j] = ldexpf(e4m3_decode((w[j >> 2] >> (8 * (j & 3))) & 0xFFu), k);
        if (BF16) {
            uint4 *d = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + i * 32);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint32_t v[4];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    v[j] = f32_to_bf16(y[8 * q + 2 * j]) | (f32_to_bf16(y[8 * q + 2 * j + 1]) << 16);
                d[q] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        } else {
            float4 *d = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + i * 32);
#pragma unroll
            for (int j = 0; j < 8; j++) d[j] = make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
        }
    }
}

hipError_t launch_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t M,
                             int64_t K, int64_t rps, void *out, int out_dtype, hipStream_t s) {
    const bool bf = out_dtype == 1;
    if (fmt == 0) {
        if (bf)
            k_dequant_nvfp4_bf16<<<grid_for(2 * M * (K / 16), 256, 1 << 20), 256, 0, s>>>(
                codes, scales, outer, M, K, rps, reinterpret_cast<uint16_t *>(out));
        else
            k_dequant_nvfp4_f32<<<grid_for(M * (K / 16), 256, 1 << 20), 256, 0, s>>>(
                codes, scales, outer, M, K, rps, reinterpret_cast<float *>(out));
    } else {
        const int grid = grid_for(M * (K / 32), 256, 1 << 20);
        if (bf) k_dequant_mxfp8<true><<<grid, 256, 0, s>>>(codes, scales, M, K, out);
        else k_dequant_mxfp8<false><<<grid, 256, 0, s>>>(codes, scales, M, K, out);
    }
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Dequantize -> transpose -> requantize (stochastic rounding)
// --------------------------------------------------------------------------

constexpr int RQ_TM = 256;            // input rows (m) per tile: 16 output blocks of 16
constexpr int RQ_TK = 128;            // input columns (k) per tile: 16 groups of 8
constexpr int RQ_CS = RQ_TM + 4;      // word stride of the transposed code tile in LDS
constexpr int RQ_MAXPART = 1024;      // partial maxima of the outer scales
constexpr int RQ_PCHUNK = 2048;       // outer scales per partial-max block
// outer scales per tensor reduced inside the requant kernel (one load per
// thread; with 16384 the separate partial-maximum pass measured faster)
constexpr int64_t RQ_FUSE = 256;

// Partial maxima of the outer scales of each tensor of a batch (G_e = max
// over tensor e's partials, starting from 0).  Tensor e = blockIdx.y has rows
// [e M, (e + 1) M) and outer scale outer[row / rps], i.e. the entries
// [lo, hi) below.  Chunks are multiples of 4 floats; float4 loads where the
// chunk start is 16-byte aligned.
__global__ __launch_bounds__(256) void k_outer_partial_max(const float *__restrict__ outer, int64_t M, int64_t rps,
                                                           float *__restrict__ part) {
    const int64_t e = blockIdx.y;
    const int64_t lo = e * M / rps, hi = ((e + 1) * M - 1) / rps + 1, n = hi - lo;
    const int64_t chunk = ((n + gridDim.x - 1) / gridDim.x + 3) & ~(int64_t)3;
    const int64_t a = lo + (int64_t)blockIdx.x * chunk, b = a + chunk < hi ? a + chunk : hi;
    const bool vec = (lo & 3) == 0;
    float m = 0.0f;
    for (int64_t i = a + 4 * (int64_t)threadIdx.x; i < b; i += 4 * (int64_t)blockDim.x) {
        if (vec && i + 4 <= b) {
            const float4 v = *reinterpret_cast<const float4 *>(outer + i);
            m = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
        } else {
            for (int64_t j = i; j < b; j++) m = fmaxf(m, outer[j]);
        }
    }
    m = wave_max(m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[e * gridDim.x + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// a[15:0] * b[15:0] + c (low half of a) and a[31:16] * b[15:0] + c (high
// half): one V_MAD_U32_U16 each.
__device__ __forceinline__ uint32_t mad_u16_lo(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t d;
    asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
    return d;
}
__device__ __forceinline__ uint32_t mad_u16_hi(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t d;
    asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(d) : "v"(a), "s"(b), "v"(c));
    return d;
}

// floor(-y) as an int: V_CVT_FLR_I32_F32 with a negated operand, so that
// -result = ceil(y) in one instruction.
__device__ __forceinline__ int32_t neg_ceil_i32(float y) {
    int32_t f;
    asm("v_cvt_flr_i32_f32 %0, -%1" : "=v"(f) : "v"(y));
    return f;
}

// Stochastic rounding of x = d * r (r >= 0) onto the E2M1 grid with 16
// random bits u, passed as nw = ~word with u in its low (HI = false) or high
// half.  v = |x| is rounded up to the next grid value iff u < frac * 2^16,
// frac being v's exact position between its grid neighbours; v >= 6 gives 6.
// Returns the signed 4-bit code in bits 28-31 (lower bits are junk).
// Branch-free and exact:
//  - v in [1, 6]: the E2M1 value is v's exponent and top mantissa bit; frac *
//    2^22 is the 22 mantissa bits m below them.  Adding 2^22 - 1 - 64 u to
//    the bit pattern carries into bit 22 iff m > 64 u, i.e. iff u < frac *
//    2^16.  Bits 22 and up then read 252 + code.
//  - v < 1: the grid step is 0.5; with c = ceil(v * 2^17) (exact), floor(2 v)
//    plus the decision is (c + 65535 - u) >> 16, laid out as 252 + code from
//    bit 22 up as well.
// Adding 4 << 22 turns 252 + code into 256 + code, so bits 22-25 are the code
// with bit 25 clear.  Everything is computed shifted left by 6 (mod 2^32),
// which puts bits 22-25 at 28-31 with bit 31 clear for the sign of x; the
// random term 64 (65535 - u) << 6 is (~u & 0xFFFF) * 4096.
template <bool HI>
__device__ __forceinline__ uint32_t e2m1_sr_code_hi(float d, float r, uint32_t nw) {
    // |d * r| == |d| * r for r >= 0, and d * r keeps the sign of d (r = 0 too)
    const float x = d * r;
    const float v = fminf(fabsf(x), 6.0f);
    // (bits(v) + 0x0100003F) << 6 and (64 c + 0x3F000000 - 63 + 0x0100003F) << 6
    // = c << 12, with c = ceil(v * 2^17) <= 2^17
    const uint32_t pa = (__float_as_uint(v) << 6) + 0x40000FC0u;
    const uint32_t pb = (uint32_t)__mul24(neg_ceil_i32(v * 131072.0f), -4096);
    // select by mask: a plain ?: is turned into a divergent branch
    const uint32_t below = 0u - (uint32_t)(v < 1.0f);
    const uint32_t p = (pb & below) | (pa & ~below);
    const uint32_t t = HI ? mad_u16_hi(nw, 4096u, p) : mad_u16_lo(nw, 4096u, p);
    return t | (__float_as_uint(x) & 0x80000000u);
}

// Quantize one output block (16 values d of one output row k, m = mb ..
// mb + 15) and store its 8 code bytes at cp and its scale at sp.  blk is the
// Philox block of the block's first element, (k * M + mb) / 8.  rlut[s] is
// 1 / (E4M3(s) * G), or 0 where that product is below 2^-126 (the block is
// flushed: scale 0, every code keeps only its sign).  DIRECT: G differs
// between the blocks of a workgroup and the same value is computed in place.
template <bool SR, bool DIRECT = false>
__device__ __forceinline__ void requant_block(const float (&d)[16], float G, const float *rlut, uint64_t blk,
                                              uint8_t *cp, uint8_t *sp, uint32_t key0, uint32_t key1) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(d[i]));
    uint32_t s = 0u;
    float r = 0.0f;
    if (G > 0.0f) {
        s = e4m3x2_hw(a / (6.0f * G), 0.0f) & 0xFFu;  // a >= 0: s <= 0x7E
        if (DIRECT) {
            const float eff = __builtin_amdgcn_cvt_f32_fp8((int)s, 0) * G;
            r = eff >= kFlushBelow ? 1.0f / eff : 0.0f;
        } else {
            r = rlut[s];
        }
        s = r == 0.0f ? 0u : s;
    }
    uint32_t lo = 0u, hi = 0u;
    if (SR) {
        // k * M and mb are multiples of 16, so blk is even and the block's
        // two Philox blocks are blk and blk | 1: 8 x 16 bits each
        uint32_t rnd[8];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint32_t c[4] = {(uint32_t)blk | (uint32_t)h, (uint32_t)(blk >> 32), 0u, 0u};
            philox4x32_10(c, key0, key1);
#pragma unroll
            for (int w = 0; w < 4; w++) rnd[4 * h + w] = c[w];
        }
        // pack by funnel shifts, last element first: each step moves the
        // word up one nibble and brings the next code in at the bottom
        lo = e2m1_sr_code_hi<true>(d[7], r, ~rnd[3]) >> 28;
        hi = e2m1_sr_code_hi<true>(d[15], r, ~rnd[7]) >> 28;
#pragma unroll
        for (int q = 3; q >= 0; q--) {
            const uint32_t nw = ~rnd[q];
            if (q < 3) lo = __builtin_amdgcn_alignbit(lo, e2m1_sr_code_hi<true>(d[2 * q + 1], r, nw), 28);
            lo = __builtin_amdgcn_alignbit(lo, e2m1_sr_code_hi<false>(d[2 * q], r, nw), 28);
        }
#pragma unroll
        for (int q = 3; q >= 0; q--) {
            const uint32_t nw = ~rnd[4 + q];
            if (q < 3) hi = __builtin_amdgcn_alignbit(hi, e2m1_sr_code_hi<true>(d[8 + 2 * q + 1], r, nw), 28);
            hi = __builtin_amdgcn_alignbit(hi, e2m1_sr_code_hi<false>(d[8 + 2 * q], r, nw), 28);
        }
    } else {
        // d * r keeps the sign of d for the hardware conversion
#pragma unroll
        for (int i = 0; i < 4; i++) {
            lo |= e2m1x2_hw(d[2 * i] * r, d[2 * i + 1] * r) << (8 * i);
            hi |= e2m1x2_hw(d[8 + 2 * i] * r, d[8 + 2 * i + 1] * r) << (8 * i);
        }
    }
    *reinterpret_cast<uint2 *>(cp) = make_uint2(lo, hi);
    *sp = (uint8_t)s;
}

// Byte E of each of the 16 row words holds columns kbase + 2E (low nibble)
// and kbase + 2E + 1: decode both (exact at scale 1), scale, requantize.
// Output row kbase + e starts at block blk0 + e * bstep, code byte cp0 + e *
// cstep and scale byte sp0 + e * sstep.
template <bool SR, int E, bool DIRECT = false>
__device__ __forceinline__ void requant_pair(const uint32_t (&cw)[16], const float (&sf)[16], float G,
                                             const float *rlut, uint64_t blk0, uint64_t bstep, uint8_t *cp0,
                                             int64_t cstep, uint8_t *sp0, int64_t sstep, uint32_t key0,
                                             uint32_t key1) {
    float d0[16], d1[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], 1.0f, E);
        d0[i] = v[0] * sf[i];
        d1[i] = v[1] * sf[i];
    }
    requant_block<SR, DIRECT>(d0, G, rlut, blk0 + (2 * E) * bstep, cp0 + (2 * E) * cstep, sp0 + (2 * E) * sstep,
                              key0, key1);
    requant_block<SR, DIRECT>(d1, G, rlut, blk0 + (2 * E + 1) * bstep, cp0 + (2 * E + 1) * cstep,
                              sp0 + (2 * E + 1) * sstep, key0, key1);
}

// One 256 (m) x 128 (k) input tile per workgroup.  The code tile is stored
// transposed in LDS as words tc[kq][m] (the 8 nibbles of k = 8 kq .. 8 kq + 7
// of row m) and the effective scales s * g as tf[kb][m].  Thread (j, kq)
// then holds rows 16 j .. 16 j + 15 of its 8 columns and produces the 8
// output blocks (k, 16-row block j): for each k, the 16 lanes of one k write
// 128 contiguous bytes of output row k.
// A batch of tensors runs on blockIdx.y: tensor e reads rows [e M, (e+1) M)
// of the stacked input (outer scale of row r: outer[r / rps]) and writes
// [e K, (e+1) K) of the stacked output with its own G_e; its random bits are
// drawn at the element's index in the stacked output.
template <bool SR>
__global__ __launch_bounds__(256) void k_requant(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 const float *__restrict__ outer, int64_t rps, int64_t M, int64_t K,
                                                 uint8_t *__restrict__ codesT, uint8_t *__restrict__ scalesT,
                                                 float *__restrict__ outerT, const float *__restrict__ part, int npart,
                                                 uint32_t key0, uint32_t key1, int ntk, int ntiles) {
    __shared__ uint32_t tc[RQ_TK / 8][RQ_CS];
    __shared__ float tf[RQ_TK / 16][RQ_TM];
    __shared__ float red[4];
    __shared__ float rlut[128];
    const int t = threadIdx.x;
    const int64_t eb = blockIdx.y;
    codes += eb * M * (K / 2);
    scales += eb * M * (K / 16);
    codesT += eb * K * (M / 2);
    scalesT += eb * K * (M / 16);
    outerT += eb;
    part += eb * npart;
    // consecutive tiles (which share input cache lines) on one XCD
    int tile = (int)blockIdx.x;
    if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
    const int64_t m0 = (int64_t)(tile / ntk) * RQ_TM, k0 = (int64_t)(tile % ntk) * RQ_TK;

    {
        // G: the maximum of the tensor's partial maxima, or (a short outer
        // array) of its outer scales themselves, four at a time where aligned
        float g = 0.0f;
        int i0 = 0;
        if ((reinterpret_cast<uintptr_t>(part) & 15) == 0) {
            const int n4 = npart >> 2;
            for (int i = t; i < n4; i += 256) {
                const float4 v = reinterpret_cast<const float4 *>(part)[i];
                g = fmaxf(g, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
            }
            i0 = 4 * n4;
        }
        for (int i = i0 + t; i < npart; i += 256) g = fmaxf(g, part[i]);
        g = wave_max(g);
        if ((t & 63) == 0) red[t >> 6] = g;
    }

    // codes: thread t loads 16-byte pieces p = t & 3 (k0 + 32 p .. + 31) of
    // rows t / 4 + 64 it; K is a multiple of 16, so a piece is whole, half
    // or empty at the right edge
    const int64_t rowb = K / 2;
    if (m0 + RQ_TM <= M && k0 + RQ_TK <= K && (rowb & 15) == 0) {
        // interior tile: all four loads in flight before the LDS writes
        const int p = t & 3;
        const uint8_t *src = codes + (m0 + (t >> 2)) * rowb + k0 / 2 + 16 * p;
        uint4 v[4];
#pragma unroll
        for (int it = 0; it < 4; it++) v[it] = *reinterpret_cast<const uint4 *>(src + 64 * it * rowb);
#pragma unroll
        for (int it = 0; it < 4; it++) {
            const int r = (t >> 2) + 64 * it;
            tc[4 * p + 0][r] = v[it].x;
            tc[4 * p + 1][r] = v[it].y;
            tc[4 * p + 2][r] = v[it].z;
            tc[4 * p + 3][r] = v[it].w;
        }
    } else {
        const int p = t & 3;
        const int64_t kb = k0 + 32 * p;
#pragma unroll
        for (int it = 0; it < 4; it++) {
            const int r = (t >> 2) + 64 * it;
            const int64_t m = m0 + r;
            uint32_t w0 = 0u, w1 = 0u, w2 = 0u, w3 = 0u;
            if (m < M) {
                const uint8_t *src = codes + m * rowb + kb / 2;
                if (kb + 32 <= K) {
                    if ((rowb & 15) == 0) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(src);
                        w0 = v.x; w1 = v.y; w2 = v.z; w3 = v.w;
                    } else {
                        const uint2 a = reinterpret_cast<const uint2 *>(src)[0];
                        const uint2 b = reinterpret_cast<const uint2 *>(src)[1];
                        w0 = a.x; w1 = a.y; w2 = b.x; w3 = b.y;
                    }
                } else if (kb + 16 <= K) {
                    const uint2 a = *reinterpret_cast<const uint2 *>(src);
                    w0 = a.x; w1 = a.y;
                }
            }
            tc[4 * p + 0][r] = w0;
            tc[4 * p + 1][r] = w1;
            tc[4 * p + 2][r] = w2;
            tc[4 * p + 3][r] = w3;
        }
    }
    // effective scales of row m0 + t for the tile's 8 k blocks
    {
        const int64_t m = m0 + t;
        uint32_t sb[RQ_TK / 16];
#pragma unroll
        for (int b = 0; b < RQ_TK / 16; b++) sb[b] = 0u;
        float g = 0.0f;
        if (m < M) {
            g = outer[(eb * M + m) / rps];
            const int64_t sp = K / 16;
            const uint8_t *src = scales + m * sp + k0 / 16;
            const int64_t left = sp - k0 / 16;
            if (left >= RQ_TK / 16 && (sp & 7) == 0) {
                const uint2 v = *reinterpret_cast<const uint2 *>(src);
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    sb[b] = (v.x >> (8 * b)) & 0xFFu;
                    sb[4 + b] = (v.y >> (8 * b)) & 0xFFu;
                }
            } else {
#pragma unroll
                for (int b = 0; b < RQ_TK / 16; b++)
                    if (b < left) sb[b] = src[b];
            }
        }
#pragma unroll
        for (int b = 0; b < RQ_TK / 16; b++) tf[b][t] = e4m3_decode(sb[b]) * g;
    }
    __syncthreads();

    const float G = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (tile == 0 && t == 0) *outerT = G;
    if (t < 128) {
        // 1 / (E4M3(s) * G) per scale code s, 0 where the block is flushed
        const float eff = __builtin_amdgcn_cvt_f32_fp8(t, 0) * G;  // exact for s <= 0x7E
        rlut[t] = (t == 127 || !(eff >= kFlushBelow)) ? 0.0f : 1.0f / eff;
    }
    __syncthreads();
    const int lane = t & 63;
    const int j = lane & 15, kq = 4 * (t >> 6) + (lane >> 4);
    const int64_t mb = m0 + 16 * j, kbase = k0 + 8 * kq;
    if (mb >= M || kbase >= K) return;
    uint32_t cw[16];
    float sf[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const uint4 c = *reinterpret_cast<const uint4 *>(&tc[kq][16 * j + 4 * q]);
        const float4 f = *reinterpret_cast<const float4 *>(&tf[kq >> 1][16 * j + 4 * q]);
        cw[4 * q + 0] = c.x; cw[4 * q + 1] = c.y; cw[4 * q + 2] = c.z; cw[4 * q + 3] = c.w;
        sf[4 * q + 0] = f.x; sf[4 * q + 1] = f.y; sf[4 * q + 2] = f.z; sf[4 * q + 3] = f.w;
    }
    const uint64_t blk0 = (((uint64_t)eb * (uint64_t)K + (uint64_t)kbase) * (uint64_t)M + (uint64_t)mb) >> 3,
                   bstep = (uint64_t)M >> 3;
    uint8_t *cp0 = codesT + kbase * (M / 2) + mb / 2;
    uint8_t *sp0 = scalesT + kbase * (M / 16) + mb / 16;
    requant_pair<SR, 0>(cw, sf, G, rlut, blk0, bstep, cp0, M / 2, sp0, M / 16, key0, key1);
    requant_pair<SR, 1>(cw, sf, G, rlut, blk0, bstep, cp0, M / 2, sp0, M / 16, key0, key1);
    requant_pair<SR, 2>(cw, sf, G, rlut, blk0, bstep, cp0, M / 2, sp0, M / 16, key0, key1);
    requant_pair<SR, 3>(cw, sf, G, rlut, blk0, bstep, cp0, M / 2, sp0, M / 16, key0, key1);
}

// Grouped form, for the weight gradient's token-blocked operands: the rows of
// group g (rows [off[g], off[g+1]) of the routed order, read through the
// gather) become columns [P[g], P[g] + pad32(n_g)) of the output [K, ldT],
// each group requantized with its own G_g.  G_g = max outer scale over the
// group's rows, one workgroup per group.
// (Offsets are trusted only up to R, the length of the routed order.)
__global__ __launch_bounds__(256) void k_group_outer_max(const float *__restrict__ outer, int64_t src_rows,
                                                         const int32_t *__restrict__ gather,
                                                         const int64_t *__restrict__ off, int64_t R,
                                                         float *__restrict__ outerT) {
    const int64_t g = blockIdx.x, a = off[g], b = off[g + 1] < R ? off[g + 1] : R;
    // eight rows per thread and pass, their loads issued together: a large
    // group is a long chain of dependent (gather, then outer) loads otherwise
    constexpr int U = 8;
    float m = 0.0f;
    for (int64_t r0 = a + threadIdx.x; r0 < b; r0 += U * (int64_t)blockDim.x) {
        int64_t src[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t r = r0 + u * (int64_t)blockDim.x;
            src[u] = r < b ? (gather ? (int64_t)gather[r] : r) : -1;
        }
#pragma unroll
        for (int u = 0; u < U; u++)
            if (src[u] >= 0 && src[u] < src_rows) m = fmaxf(m, outer[src[u]]);
    }
    m = wave_max(m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) outerT[g] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One 256 (padded columns) x 128 (k) tile per workgroup, as k_requant, with
// the tile's rows mapped through the groups: 32-row block b of the tile lies
// in one group (P is 32-aligned), whose G_g every 16-block of it uses; rows
// past a group's tokens (padding) and bad gather indices read as zeros.  The
// SR bits of output element (k, p) are drawn at k * ldT + p.
template <bool SR>
__global__ __launch_bounds__(256) void k_requant_grouped(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, const float *__restrict__ outer,
    int64_t src_rows, const int32_t *__restrict__ gather, const int64_t *__restrict__ off, int G, int64_t R,
    int64_t K, int64_t ldT, uint8_t *__restrict__ codesT, uint8_t *__restrict__ scalesT,
    const float *__restrict__ outerT, uint32_t key0, uint32_t key1, int ntk) {
    __shared__ uint32_t tc[RQ_TK / 8][RQ_CS];
    __shared__ float tf[RQ_TK / 16][RQ_TM];
    __shared__ int64_t wsum[4];
    __shared__ int64_t blk_src0[RQ_TM / 32], blk_end[RQ_TM / 32];
    __shared__ float blk_G[RQ_TM / 32];
    __shared__ int64_t srow[RQ_TM];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t m0 = (int64_t)(blockIdx.x / ntk) * RQ_TM, k0 = (int64_t)(blockIdx.x % ntk) * RQ_TK;

    // Padded group starts: thread t owns groups [t per, t per + per); a
    // block-wide scan of their padded sizes gives the start of its first
    // group, and the thread whose groups cover one of the tile's 32-row
    // blocks resolves that block's first source row, group end and G_g.
    int64_t ptotal;
    {
        const int per = (G + 255) / 256;
        const int g0 = t * per, g1 = g0 + per < G ? g0 + per : G;
        int64_t local = 0;
        for (int g = g0; g < g1; g++) local += (off[g + 1] - off[g] + 31) / 32 * 32;
        const int64_t incl = wave_incl_scan(local, lane);
        if (lane == 63) wsum[wv] = incl;
        if (t < RQ_TM / 32) {
            blk_src0[t] = 0;
            blk_end[t] = 0;
            blk_G[t] = 0.0f;
        }
        __syncthreads();
        int64_t run = incl - local;
        for (int w = 0; w < wv; w++) run += wsum[w];
        const int64_t total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        ptotal = total < ldT ? total : ldT;   // never past the output's rows
        if (local > 0 && run < m0 + RQ_TM && run + local > m0) {
            for (int g = g0; g < g1; g++) {
                const int64_t o0 = off[g], o1 = off[g + 1];
                const int64_t pn = (o1 - o0 + 31) / 32 * 32;
#pragma unroll
                for (int b = 0; b < RQ_TM / 32; b++) {
                    const int64_t pb = m0 + 32 * b;
                    if (pb >= run && pb < run + pn && pb < ptotal) {
                        blk_src0[b] = o0 + (pb - run);
                        blk_end[b] = o1 < R ? o1 : R;
                        blk_G[b] = outerT[g];
                    }
                }
                run += pn;
            }
        }
        __syncthreads();
    }
    if (m0 >= ptotal) return;
    {
        const int b = t >> 5;
        const int64_t r = blk_src0[b] + (t & 31);
        int64_t src = -1;
        if (m0 + t < ptotal && r < blk_end[b]) {
            src = gather ? (int64_t)gather[r] : r;
            if (src < 0 || src >= src_rows) src = -1;
        }
        srow[t] = src;
    }
    __syncthreads();

    // codes of the tile's rows (16-byte pieces p = t & 3 of k0 + 32 p ..)
    const int64_t rowb = K / 2;
    {
        const int p = t & 3;
        const int64_t kb = k0 + 32 * p;
#pragma unroll
        for (int it = 0; it < 4; it++) {
            const int r = (t >> 2) + 64 * it;
            const int64_t src = srow[r];
            uint32_t w0 = 0u, w1 = 0u, w2 = 0u, w3 = 0u;
            if (src >= 0) {
                const uint8_t *sp = codes + src * rowb + kb / 2;
                if (kb + 32 <= K) {
                    if ((rowb & 15) == 0) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(sp);
                        w0 = v.x; w1 = v.y; w2 = v.z; w3 = v.w;
                    } else {
                        const uint2 a = reinterpret_cast<const uint2 *>(sp)[0];
                        const uint2 b = reinterpret_cast<const uint2 *>(sp)[1];
                        w0 = a.x; w1 = a.y; w2 = b.x; w3 = b.y;
                    }
                } else if (kb + 16 <= K) {
                    const uint2 a = *reinterpret_cast<const uint2 *>(sp);
                    w0 = a.x; w1 = a.y;
                }
            }
            tc[4 * p + 0][r] = w0;
            tc[4 * p + 1][r] = w1;
            tc[4 * p + 2][r] = w2;
            tc[4 * p + 3][r] = w3;
        }
    }
    // effective scales of tile row t for the tile's 8 k blocks
    {
        const int64_t src = srow[t];
        uint32_t sb[RQ_TK / 16];
#pragma unroll
        for (int b = 0; b < RQ_TK / 16; b++) sb[b] = 0u;
        float g = 0.0f;
        if (src >= 0) {
            g = outer[src];
            const int64_t sp = K / 16;
            const uint8_t *srcp = scales + src * sp + k0 / 16;
            const int64_t left = sp - k0 / 16;
#pragma unroll
            for (int b = 0; b < RQ_TK / 16; b++)
                if (b < left) sb[b] = srcp[b];
        }
#pragma unroll
        for (int b = 0; b < RQ_TK / 16; b++) tf[b][t] = e4m3_decode(sb[b]) * g;
    }
    __syncthreads();

    const int j = lane & 15, kq = 4 * wv + (lane >> 4);
    const int64_t mb = m0 + 16 * j, kbase = k0 + 8 * kq;
    if (mb >= ptotal || kbase >= K) return;
    const float G_ = blk_G[j >> 1];
    uint32_t cw[16];
    float sf[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const uint4 c = *reinterpret_cast<const uint4 *>(&tc[kq][16 * j + 4 * q]);
        const float4 f = *reinterpret_cast<const float4 *>(&tf[kq >> 1][16 * j + 4 * q]);
        cw[4 * q + 0] = c.x; cw[4 * q + 1] = c.y; cw[4 * q + 2] = c.z; cw[4 * q + 3] = c.w;
        sf[4 * q + 0] = f.x; sf[4 * q + 1] = f.y; sf[4 * q + 2] = f.z; sf[4 * q + 3] = f.w;
    }
    const uint64_t blk0 = ((uint64_t)kbase * (uint64_t)ldT + (uint64_t)mb) >> 3, bstep = (uint64_t)ldT >> 3;
    uint8_t *cp0 = codesT + kbase * (ldT / 2) + mb / 2;
    uint8_t *sp0 = scalesT + kbase * (ldT / 16) + mb / 16;
    requant_pair<SR, 0, true>(cw, sf, G_, nullptr, blk0, bstep, cp0, ldT / 2, sp0, ldT / 16, key0, key1);
    requant_pair<SR, 1, true>(cw, sf, G_, nullptr, blk0, bstep, cp0, ldT / 2, sp0, ldT / 16, key0, key1);
    requant_pair<SR, 2, true>(cw, sf, G_, nullptr, blk0, bstep, cp0, ldT / 2, sp0, ldT / 16, key0, key1);
    requant_pair<SR, 3, true>(cw, sf, G_, nullptr, blk0, bstep, cp0, ldT / 2, sp0, ldT / 16, key0, key1);
}

hipError_t launch_requant_grouped(const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t src_rows,
                                  const int32_t *gather, const int64_t *group_offsets, int64_t G, int64_t R,
                                  int64_t K, uint8_t *codesT, uint8_t *scalesT, int64_t ldT, float *outerT,
                                  uint64_t seed, bool sr, hipStream_t s) {
    k_group_outer_max<<<(unsigned)G, 256, 0, s>>>(outer, src_rows, gather, group_offsets, R, outerT);
    const int64_t ntk = (K + RQ_TK - 1) / RQ_TK, ntm = (ldT + RQ_TM - 1) / RQ_TM;
    if (ntk * ntm > INT32_MAX) return hipErrorInvalidValue;
    const int nt = (int)(ntk * ntm);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    if (sr)
        k_requant_grouped<true><<<nt, 256, 0, s>>>(codes, scales, outer, src_rows, gather, group_offsets, (int)G, R,
                                                   K, ldT, codesT, scalesT, outerT, k0, k1, (int)ntk);
    else
        k_requant_grouped<false><<<nt, 256, 0, s>>>(codes, scales, outer, src_rows, gather, group_offsets, (int)G, R,
                                                    K, ldT, codesT, scalesT, outerT, k0, k1, (int)ntk);
    return hipGetLastError();
}

// Outer scales per tensor of a batch of tensors of M rows, rps dividing M or
// a multiple of it.
static int64_t requant_scales_per_tensor(int64_t M, int64_t rps) { return M % rps == 0 ? M / rps : 1; }

int requant_partials(int64_t n) {
    n = (n + RQ_PCHUNK - 1) / RQ_PCHUNK;
    return (int)(n < 1 ? 1 : (n > RQ_MAXPART ? RQ_MAXPART : n));
}

int64_t requant_workspace_floats(int64_t E, int64_t M, int64_t rps) {
    return E * requant_partials(requant_scales_per_tensor(M, rps));
}

hipError_t launch_requant(const uint8_t *codes, const uint8_t *scales, const float *outer, int64_t rps, int64_t E,
                          int64_t M, int64_t K, uint8_t *codesT, uint8_t *scalesT, float *outerT, uint64_t seed,
                          bool sr, float *part, hipStream_t s) {
    // Up to RQ_FUSE outer scales per tensor (M / rps of them, contiguous per
    // tensor), each workgroup reduces them itself; beyond, a first kernel
    // reduces them to at most RQ_MAXPART partial maxima in the workspace.
    int np;
    const float *red_src;
    if (M % rps == 0 && M / rps <= RQ_FUSE) {
        np = (int)(M / rps);
        red_src = outer;
    } else {
        np = requant_partials(requant_scales_per_tensor(M, rps));
        k_outer_partial_max<<<dim3(np, (unsigned)E), 256, 0, s>>>(outer, M, rps, part);
        red_src = part;
    }
    const int64_t ntk = (K + RQ_TK - 1) / RQ_TK, ntm = (M + RQ_TM - 1) / RQ_TM;
    if (ntk * ntm > INT32_MAX) return hipErrorInvalidValue;
    const int nt = (int)(ntk * ntm);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const dim3 grid((unsigned)nt, (unsigned)E);
    if (sr)
        k_requant<true><<<grid, 256, 0, s>>>(codes, scales, outer, rps, M, K, codesT, scalesT, outerT, red_src, np,
                                             k0, k1, (int)ntk, nt);
    else
        k_requant<false><<<grid, 256, 0, s>>>(codes, scales, outer, rps, M, K, codesT, scalesT, outerT, red_src, np,
                                              k0, k1, (int)ntk, nt);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// SwiGLU + quantization of its output
// --------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ float load_elem(const T *p);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }

// 32 consecutive inputs starting at p (16-byte aligned) as f32, in 16-byte loads.
template <typename T>
__device__ __forceinline__ void load32(const T *p, float (&v)[32]);
template <>
__device__ __forceinline__ void load32<float>(const float *p, float (&v)[32]) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float4 f = q[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
}
template <>
__device__ __forceinline__ void load32<uint16_t>(const uint16_t *p, float (&v)[32]) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint4 u = q[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            v[8 * i + 2 * k] = bf16_lo(w[k]);
            v[8 * i + 2 * k + 1] = bf16_hi(w[k]);
        }
    }
}

// LPR lanes per row of h (64, or 32 / 16 / 8 for short rows so that lanes are
// not left idle); lane l of a row owns the 32-value chunks starting at
// i = 32 LPR j + 32 l (whole quantization blocks per lane).  Outputs whose
// per-lane pieces are not contiguous across lanes (h, MXFP8 codes) go through
// a per-wavefront LDS patch so that every store instruction writes a
// contiguous run.  FMT: -1 = h only, 0 = NVFP4 per token, 1 = MXFP8 rowwise.
template <typename T, int FMT, bool M46, int MAXIT, int LPR>
__global__ __launch_bounds__(256) void k_swiglu(const T *__restrict__ h13, int64_t R, int64_t I,
                                                uint16_t *__restrict__ h_out, uint8_t *__restrict__ codes,
                                                uint8_t *__restrict__ scales, float *__restrict__ outer) {
    // per wavefront: 64 lanes x (64 + 16) bytes (padding keeps the 64-byte
    // lane pieces on distinct banks)
    __shared__ __attribute__((aligned(16))) uint8_t stg[4][64 * 80];
    constexpr int RPW = 64 / LPR;               // rows per wavefront
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & (LPR - 1), sub = (threadIdx.x & 63) / LPR;
    const int64_t row = ((int64_t)blockIdx.x * 4 + wv) * RPW + sub;
    if (row >= R) return;                       // whole row groups leave together
    uint8_t *sw = stg[wv] + sub * (LPR * 80);
    const T *gp = h13 + row * 2 * I;
    const T *up = gp + I;
    float hv[MAXIT][32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXIT; j++) {
        const int64_t c0 = (int64_t)j * 32 * LPR;   // this chunk's first element
        const int64_t i0 = c0 + lane * 32;
        if (c0 >= I) break;                     // wave-uniform
        if (i0 < I) {
            float z[32], u[32];
            load32<T>(gp + i0, z);
            load32<T>(up + i0, u);
#pragma unroll
            for (int i = 0; i < 32; i++) {
                hv[j][i] = __uint_as_float(swiglu_bf16(z[i], u[i]) << 16);
                amax = fmaxf(amax, fabsf(hv[j][i]));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; i++) hv[j][i] = 0.0f;
        }
        if (h_out) {
            uint4 *d = reinterpret_cast<uint4 *>(sw + lane * 80);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; k++)
                    w[k] = (__float_as_uint(hv[j][8 * q + 2 * k]) >> 16) |
                           (__float_as_uint(hv[j][8 * q + 2 * k + 1]) & 0xFFFF0000u);
                d[q] = make_uint4(w[0], w[1], w[2], w[3]);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int m = LPR * k + lane;             // 16-byte piece of the chunk
                if (c0 + 8 * m < I) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(sw + 80 * (m >> 2) + 16 * (m & 3));
                    *reinterpret_cast<uint4 *>(h_out + row * I + c0 + 8 * m) = v;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    if (FMT < 0) return;
    if (FMT == 0) {
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const float g = (amax == 0.0f) ? 0.0f : amax / 2688.0f;
        if (lane == 0) outer[row] = g;
#pragma unroll
        for (int j = 0; j < MAXIT; j++) {
            const int64_t i0 = (int64_t)j * 32 * LPR + lane * 32;
            if (i0 < I) {
                uint32_t w4[4], sc = 0;
#pragma unroll
                for (int b = 0; b < 2; b++) {
                    float xf[16];
#pragma unroll
                    for (int i = 0; i < 16; i++) xf[i] = hv[j][16 * b + i];
                    Nvfp4Block nb = nvfp4_block<M46>(xf, g);
                    w4[2 * b] = nb.lo;
                    w4[2 * b + 1] = nb.hi;
                    sc |= nb.s << (8 * b);
                }
                // lane pieces are contiguous across lanes: one 16-byte and one 2-byte store
                *reinterpret_cast<uint4 *>(codes + row * (I / 2) + i0 / 2) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                *reinterpret_cast<uint16_t *>(scales + row * (I / 16) + i0 / 16) = (uint16_t)sc;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < MAXIT; j++) {
            const int64_t c0 = (int64_t)j * 32 * LPR;
            const int64_t i0 = c0 + lane * 32;
            if (c0 >= I) break;
            uint32_t q[8];
            const uint32_t sc = mxfp8_block(hv[j], q);
            if (i0 < I) scales[row * (I / 32) + i0 / 32] = (uint8_t)sc;
            uint4 *d = reinterpret_cast<uint4 *>(sw + lane * 48);
            d[0] = make_uint4(q[0], q[1], q[2], q[3]);
            d[1] = make_uint4(q[4], q[5], q[6], q[7]);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int m = LPR * k + lane;             // 16-byte piece of the code chunk
                if (c0 + 16 * m < I) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(sw + 48 * (m >> 1) + 16 * (m & 1));
                    *reinterpret_cast<uint4 *>(codes + row * I + c0 + 16 * m) = v;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <typename T, int FMT, bool M46>
static void swiglu_dispatch_it(const void *h13, int64_t R, int64_t I, uint16_t *h_out, uint8_t *codes,
                               uint8_t *scales, float *outer, hipStream_t s) {
    const T *in = reinterpret_cast<const T *>(h13);
    auto grid = [&](int lpr) { return dim3((unsigned)((R + 4 * (64 / lpr) - 1) / (4 * (64 / lpr)))); };
    // 32-value chunks per row: lanes per row and chunks per lane chosen so
    // that at most a third of the lanes idle (none for I = 768, 1536, 2048)
    const int64_t nc = (I + 31) / 32;
    if (nc <= 16) k_swiglu<T, FMT, M46, 1, 16><<<grid(16), 256, 0, s>>>(in, R, I, h_out, codes, scales, outer);
    else if (nc <= 24) k_swiglu<T, FMT, M46, 3, 8><<<grid(8), 256, 0, s>>>(in, R, I, h_out, codes, scales, outer);
    else if (nc <= 32) k_swiglu<T, FMT, M46, 1, 32><<<grid(32), 256, 0, s>>>(in, R, I, h_out, codes, scales, outer);
    else if (nc <= 48) k_swiglu<T, FMT, M46, 3, 16><<<grid(16), 256, 0, s>>>(in, R, I, h_out, codes, scales, outer);
    else if (nc <= 64) k_swiglu<T, FMT, M46, 1, 64><<<grid(64), 256, 0, s>>>(in, R, I, h_out, codes, scales, outer);
    else k_swiglu<T, FMT, M46, 4, 64><<<grid(64), 256, 0, s>>>(in, R, I, h_out, codes, scales, outer);
}

template <typename T>
static void swiglu_dispatch(const void *h13, int64_t R, int64_t I, uint16_t *h_out, int fmt, bool m46,
                            uint8_t *codes, uint8_t *scales, float *outer, hipStream_t s) {
    if (fmt < 0) swiglu_dispatch_it<T, -1, false>(h13, R, I, h_out, codes, scales, outer, s);
    else if (fmt == 0 && m46) swiglu_dispatch_it<T, 0, true>(h13, R, I, h_out, codes, scales, outer, s);
    else if (fmt == 0) swiglu_dispatch_it<T, 0, false>(h13, R, I, h_out, codes, scales, outer, s);
    else swiglu_dispatch_it<T, 1, false>(h13, R, I, h_out, codes, scales, outer, s);
}

hipError_t launch_swiglu(const void *h13, int in_dtype, int64_t R, int64_t I, uint16_t *h_out, int fmt, bool m46,
                         uint8_t *codes, uint8_t *scales, float *outer, hipStream_t s) {
    if (in_dtype == 0) swiglu_dispatch<float>(h13, R, I, h_out, fmt, m46, codes, scales, outer, s);
    else swiglu_dispatch<uint16_t>(h13, R, I, h_out, fmt, m46, codes, scales, outer, s);
    return hipGetLastError();
}

}  // namespace bsp

// bsp_gemm.hip -- block-scaled grouped expert GEMM on CDNA4 MFMA (gfx950).
//
// C = A * B^T per expert group, with both operands quantized in blocks along
// the reduction dimension K [alphasignal.ai, "LMSYS Drops Miles", Recipe 1
// and Recipe 2; remio.ai, section "Un quantizzatore condiviso": the blocks
// must follow the reduction dimension].
//
// MXFP8: 32 E4M3 values per E8M0 scale is exactly the operand format of
// gfx950's block-scaled MFMA (V_MFMA_SCALE_F32_32X32X64_F8F6F4): per 64-value
// K step each row has two 32-value blocks, each with the E8M0 byte supplied by
// one lane half, so codes and scales go to the matrix core unchanged (see
// load_mx_frag for the byte placement the instruction expects).
//
// NVFP4: the E4M3 scale covers 16 values and the matrix core only scales by
// powers of two per 32, so the operand value q * s (E2M1 times E4M3, at most
// 6 significant bits, magnitude in [2^-10, 2688]) is rebuilt exactly in fp16
// in registers and multiplied on the fp16 MFMA (V_MFMA_F32_32X32X16_F16); the
// FP32 outer scales (per token for A, per expert for B) are applied in the
// epilogue, so no separate scaling pass is needed.
//
// Tiling: 256 threads = 4 wavefronts in 2 x 2, each computing 64 x 64 of a
// 128 x 128 output tile as 2 x 2 MFMA 32 x 32 tiles, f32 accumulation.
// Row tiles never straddle two experts: a setup kernel lists the
// (expert, first row) of every 128-row tile from the device-side group
// offsets, so no host synchronization is needed.
#include "bsp_device.hpp"
#include "bsp_internal.hpp"

namespace bsp {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int GBM = 128, GBN = 128;

struct GemmArgs {
    const uint8_t *a_codes, *a_scales;
    const float *a_outer;
    const int32_t *a_gather;
    const int64_t *group_offsets;
    const uint8_t *b_codes, *b_scales;
    const float *b_outer;
    void *c;
    const int64_t *tiles;     // FPROP/DGRAD: [ntile_max] packed (group << 40) | row0; WGRAD: padded starts [G+1]
    int64_t G, M, N, K, ldc, a_rows;
};

// Tile list for the row-grouped form: tiles[i] = (g << 40) | first row, or -1.
__global__ void k_tile_list(const int64_t *__restrict__ off, int64_t G, int64_t ntile_max, int64_t *__restrict__ tiles) {
    __shared__ int64_t base[1025];
    // single workgroup: running tile counts (G <= 1024 per chunk loop)
    int64_t carry = 0;
    for (int64_t g0 = 0; g0 < G; g0 += 1024) {
        const int64_t n = (G - g0) < 1024 ? (G - g0) : 1024;
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int64_t rows = off[g0 + i + 1] - off[g0 + i];
            base[i + 1] = (rows + GBM - 1) / GBM;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            base[0] = carry;
            for (int i = 1; i <= n; i++) base[i] += base[i - 1];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int64_t g = g0 + i;
            const int64_t r0 = off[g];
            for (int64_t t = base[i]; t < base[i + 1] && t < ntile_max; t++)
                tiles[t] = (g << 40) | (r0 + (t - base[i]) * GBM);
        }
        carry = base[n];
        __syncthreads();
    }
    for (int64_t t = carry + threadIdx.x; t < ntile_max; t += blockDim.x) tiles[t] = -1;
}

// Padded group starts P (running sum of roundup32(n_g)) for the weight-gradient form.
__global__ void k_padded_starts(const int64_t *__restrict__ off, int64_t G, int64_t *__restrict__ P) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        int64_t run = 0;
        for (int64_t g = 0; g < G; g++) {
            P[g] = run;
            run += (off[g + 1] - off[g] + 31) / 32 * 32;
        }
        P[G] = run;
    }
}

// ---------------------------------------------------------------------------
// fragment loaders
// ---------------------------------------------------------------------------

// MXFP8 operand of V_MFMA_SCALE_F32_32X32X64_F8F6F4 for one row and the
// 64-value K step starting at k0.  The instruction works as two 32-value
// halves: bytes 0-15 of both lane halves form K block 0 (scaled by the E8M0
// byte of lane half 0) and bytes 16-31 form K block 1 (scaled by lane half
// 1's byte).  So lane half h holds K [k0 + 16h, +16) then [k0 + 32 + 16h, +16)
// and the scale of block k0/32 + h.  Blocks past kend read as zeros.
__device__ __forceinline__ void load_mx_frag(const uint8_t *codes, const uint8_t *scales, int64_t ld_codes,
                                             int64_t row, bool valid, int64_t k0, int64_t kend, int h, v8i &frag,
                                             int &scale) {
    const uint8_t *rp = codes + row * ld_codes;
    uint4 u0 = make_uint4(0u, 0u, 0u, 0u), u1 = u0;
    if (valid && k0 < kend) u0 = *reinterpret_cast<const uint4 *>(rp + k0 + 16 * h);
    if (valid && k0 + 32 < kend) u1 = *reinterpret_cast<const uint4 *>(rp + k0 + 32 + 16 * h);
    frag[0] = (int)u0.x; frag[1] = (int)u0.y; frag[2] = (int)u0.z; frag[3] = (int)u0.w;
    frag[4] = (int)u1.x; frag[5] = (int)u1.y; frag[6] = (int)u1.z; frag[7] = (int)u1.w;
    scale = (valid && k0 + 32 * h < kend) ? (int)scales[row * (ld_codes / 32) + k0 / 32 + h] : 127;
}

// 8 E2M1 nibbles (one 32-bit word, element 2j in the low nibble of byte j)
// -> 8 fp16 values as 4 words: the fp16 of every E2M1 value has a zero low
// byte, so the high byte comes from a byte-permute lookup of the magnitude
// plus the sign bit.
__device__ __forceinline__ void e2m1x8_to_f16(uint32_t w, uint32_t (&h)[4]) {
    const uint32_t lut_lo = 0x3E3C3800u;   // 0, 0.5, 1, 1.5 -> fp16 high bytes 00 38 3C 3E
    const uint32_t lut_hi = 0x46444240u;   // 2, 3, 4, 6     -> 40 42 44 46
    const uint32_t sel_e = w & 0x07070707u;
    const uint32_t sel_o = (w >> 4) & 0x07070707u;
    const uint32_t he = __builtin_amdgcn_perm(lut_hi, lut_lo, sel_e) | ((w << 4) & 0x80808080u);
    const uint32_t ho = __builtin_amdgcn_perm(lut_hi, lut_lo, sel_o) | (w & 0x80808080u);
    // word j = (element 2j, element 2j+1) = (he.byte j << 8) | (ho.byte j << 24)
    h[0] = __builtin_amdgcn_perm(ho, he, 0x040C000Cu);
    h[1] = __builtin_amdgcn_perm(ho, he, 0x050C010Cu);
    h[2] = __builtin_amdgcn_perm(ho, he, 0x060C020Cu);
    h[3] = __builtin_amdgcn_perm(ho, he, 0x070C030Cu);
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t hmul2(uint32_t a, h2 s) {
    h2 x = __builtin_bit_cast(h2, a);
    x = x * s;
    return __builtin_bit_cast(uint32_t, x);
}

// NVFP4: lane holds the 32 elements [kk, kk + 32) of one row (two 16-blocks)
// dequantized to fp16 as four 8-element MFMA operands.
__device__ __forceinline__ void load_nv_frag(const uint8_t *codes, const uint8_t *scales, int64_t K, int64_t row,
                                             bool valid, int64_t kk, v8h (&frag)[4]) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    float s0 = 0.0f, s1 = 0.0f;
    if (valid && kk < K) {
        const uint8_t *cp = codes + row * (K / 2) + kk / 2;
        const uint2 lo = *reinterpret_cast<const uint2 *>(cp);
        w[0] = lo.x; w[1] = lo.y;
        s0 = e4m3_decode(scales[row * (K / 16) + kk / 16]);
        if (kk + 16 < K) {
            const uint2 hi = *reinterpret_cast<const uint2 *>(cp + 8);
            w[2] = hi.x; w[3] = hi.y;
            s1 = e4m3_decode(scales[row * (K / 16) + kk / 16 + 1]);
        }
    }
    const h2 sv0 = {(_Float16)s0, (_Float16)s0};
    const h2 sv1 = {(_Float16)s1, (_Float16)s1};
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint32_t h[4];
        e2m1x8_to_f16(w[q], h);
        const h2 sv = (q < 2) ? sv0 : sv1;
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; j++) o[j] = hmul2(h[j], sv);
        frag[q] = __builtin_bit_cast(v8h, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------

template <int FMT, int MODE, bool BF16OUT>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lh = lane >> 5;

    int64_t g, row0, row_end, kbeg, kend;
    const uint8_t *bc, *bs;
    int64_t a_ld_rows;  // for WGRAD: row pitch of A and B in codes is ld_k
    (void)a_ld_rows;
    if (MODE == BSP_GEMM_WGRAD) {
        g = blockIdx.y;
        row0 = (int64_t)(blockIdx.x / ((p.N + GBN - 1) / GBN)) * GBM;
        row_end = p.M;
        kbeg = p.tiles[g];
        kend = kbeg + (p.group_offsets[g + 1] - p.group_offsets[g] + 31) / 32 * 32;
        kend = kend < p.K ? kend : p.K;  // offsets are trusted only up to the copies' width
        bc = p.b_codes;
        bs = p.b_scales;
    } else {
        const int64_t tile = p.tiles[blockIdx.y];
        if (tile < 0) return;
        g = tile >> 40;
        row0 = tile & ((1ll << 40) - 1);
        row_end = p.group_offsets[g + 1];
        row_end = row_end < p.M ? row_end : p.M;  // never past the rows of C
        kbeg = 0;
        kend = p.K;
        const int64_t bcs = (FMT == BSP_FMT_NVFP4) ? p.N * p.K / 2 : p.N * p.K;
        const int64_t bss = (FMT == BSP_FMT_NVFP4) ? p.N * p.K / 16 : p.N * p.K / 32;
        bc = p.b_codes + g * bcs;
        bs = p.b_scales + g * bss;
    }
    const int64_t ntn = (p.N + GBN - 1) / GBN;
    const int64_t col0 = (MODE == BSP_GEMM_WGRAD ? (int64_t)(blockIdx.x % ntn) : (int64_t)blockIdx.x) * GBN;

    // rows and columns this lane loads
    int64_t arow[2], brow[2];
    bool aval[2], bval[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t r = row0 + wm * 64 + i * 32 + lr;
        aval[i] = r < row_end;
        int64_t t = r;
        if (aval[i] && MODE != BSP_GEMM_WGRAD && p.a_gather) {
            t = (int64_t)p.a_gather[r];
            aval[i] = t >= 0 && t < p.a_rows;  // an out-of-range gather index reads as a zero row
        }
        arow[i] = aval[i] ? t : 0;
        const int64_t cn = col0 + wn * 64 + i * 32 + lr;
        bval[i] = cn < p.N;
        brow[i] = bval[i] ? cn : 0;
    }

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

    if (FMT == BSP_FMT_MXFP8) {
        const int64_t ldk = p.K;  // codes row pitch (FPROP: K; WGRAD: ld_colT)
        for (int64_t k0 = kbeg; k0 < kend; k0 += 64) {
            v8i af[2], bf[2];
            int as[2], bsc[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                load_mx_frag(p.a_codes, p.a_scales, ldk, arow[i], aval[i], k0, kend, lh, af[i], as[i]);
                load_mx_frag(bc, bs, ldk, brow[i], bval[i], k0, kend, lh, bf[i], bsc[i]);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0,
                                                                                as[i], 0, bsc[j]);
        }
    } else {
        for (int64_t k0 = 0; k0 < p.K; k0 += 64) {
            const int64_t kk = k0 + 32 * lh;
            v8h af[2][4], bf[2][4];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                load_nv_frag(p.a_codes, p.a_scales, p.K, arow[i], aval[i], kk, af[i]);
                load_nv_frag(bc, bs, p.K, brow[i], bval[i], kk, bf[i]);
            }
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i][q], bf[j][q], acc[i][j], 0, 0, 0);
        }
    }

    // epilogue: lane holds column (lane % 32) and rows 8 (e / 4) + 4 (lane / 32) + e % 4
    const float gb = (FMT == BSP_FMT_NVFP4) ? p.b_outer[g] : 1.0f;
    char *cbase = reinterpret_cast<char *>(p.c);
    const int64_t esz = BF16OUT ? 2 : 4;
    const int64_t goff = (MODE == BSP_GEMM_WGRAD) ? g * p.M * p.ldc : 0;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t cn = col0 + wn * 64 + j * 32 + lr;
            if (cn >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int64_t r = row0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
                if (r >= row_end) continue;
                float v = acc[i][j][e];
                if (FMT == BSP_FMT_NVFP4) {
                    const int64_t t = p.a_gather ? (int64_t)p.a_gather[r] : r;
                    v = (t >= 0 && t < p.a_rows) ? v * (p.a_outer[t] * gb) : 0.0f;
                }
                const int64_t off = goff + r * p.ldc + cn;
                if (BF16OUT) reinterpret_cast<uint16_t *>(cbase)[off] = (uint16_t)f32_to_bf16(v);
                else reinterpret_cast<float *>(cbase)[off] = v;
                (void)esz;
            }
        }
}

int64_t gemm_tile_count(int64_t M, int64_t G) { return (M + GBM - 1) / GBM + G; }

hipError_t launch_gemm(int fmt, int mode, const uint8_t *a_codes, const uint8_t *a_scales, const float *a_outer,
                       const int32_t *a_gather, int64_t a_rows, const int64_t *group_offsets, int64_t G, int64_t M, int64_t N,
                       int64_t K, const uint8_t *b_codes, const uint8_t *b_scales, const float *b_outer, void *c,
                       int c_dtype, int64_t ldc, void *workspace, hipStream_t s) {
    GemmArgs p;
    p.a_codes = a_codes; p.a_scales = a_scales; p.a_outer = a_outer; p.a_gather = a_gather;
    p.group_offsets = group_offsets; p.b_codes = b_codes; p.b_scales = b_scales; p.b_outer = b_outer;
    p.c = c; p.G = G; p.M = M; p.N = N; p.K = K; p.ldc = ldc; p.a_rows = a_rows;
    int64_t *ws = reinterpret_cast<int64_t *>(workspace);
    p.tiles = ws;
    const bool bf = c_dtype == BSP_DTYPE_BF16;
    dim3 block(256);
    if (mode == BSP_GEMM_WGRAD) {
        k_padded_starts<<<1, 64, 0, s>>>(group_offsets, G, ws);
        dim3 grid((unsigned)(((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN)), (unsigned)G);
        if (bf) k_gemm<BSP_FMT_MXFP8, BSP_GEMM_WGRAD, true><<<grid, block, 0, s>>>(p);
        else k_gemm<BSP_FMT_MXFP8, BSP_GEMM_WGRAD, false><<<grid, block, 0, s>>>(p);
        return hipGetLastError();
    }
    const int64_t nt = gemm_tile_count(M, G);
    k_tile_list<<<1, 256, 0, s>>>(group_offsets, G, nt, ws);
    dim3 grid((unsigned)((N + GBN - 1) / GBN), (unsigned)nt);
    if (fmt == BSP_FMT_MXFP8) {
        if (bf) k_gemm<BSP_FMT_MXFP8, BSP_GEMM_FPROP, true><<<grid, block, 0, s>>>(p);
        else k_gemm<BSP_FMT_MXFP8, BSP_GEMM_FPROP, false><<<grid, block, 0, s>>>(p);
    } else {
        if (bf) k_gemm<BSP_FMT_NVFP4, BSP_GEMM_FPROP, true><<<grid, block, 0, s>>>(p);
        else k_gemm<BSP_FMT_NVFP4, BSP_GEMM_FPROP, false><<<grid, block, 0, s>>>(p);
    }
    return hipGetLastError();
}

}  // namespace bsp

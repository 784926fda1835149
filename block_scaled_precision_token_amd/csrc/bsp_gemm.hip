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
// one lane half, so codes and scales go to the matrix core unchanged.
//
// NVFP4: the E4M3 scale covers 16 values and the matrix core only scales by
// powers of two per 32, so the operand value q * s (E2M1 times E4M3, at most
// 6 significant bits, magnitude in [2^-10, 2688]) is rebuilt exactly in fp16
// while the tile is staged into LDS (once per workgroup) and multiplied on
// the fp16 MFMA (V_MFMA_F32_32X32X16_F16); the FP32 outer scales (per token
// for A, per expert for B) are applied in the epilogue.
//
// Tiling: 256 threads = 4 wavefronts in 2 x 2.  Output tile BM x 128 (BM =
// 128; a 256-row variant exists behind a build switch).  K moves in
// 64-value stages through double-buffered LDS with register prefetch of the
// next stage.  Row tiles never straddle two experts: a setup kernel lists the
// (expert, first row) of every row tile from the device-side group offsets,
// so no host synchronization is needed.
//
// Tile order: workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  A workgroup's id is mapped to an XCD-contiguous chunk of
// the row-major tile sequence (row tile outer, column tile inner), so the
// workgroups in flight on one XCD are consecutive column tiles of the same
// row tiles: they share the activation tile, and successive row tiles of one
// expert re-read the same weight panels while they are still in that L2.
#include "bsp_device.hpp"
#include "bsp_internal.hpp"

namespace bsp {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBN = 128;   // output columns per workgroup
constexpr int GBK = 64;    // K values per LDS stage
constexpr int NXCD = 8;
constexpr int kMaxDevices = 64;

struct GemmArgs {
    const uint8_t *a_codes, *a_scales;
    const float *a_outer;
    const int32_t *a_gather;
    const int64_t *group_offsets;
    const uint8_t *b_codes, *b_scales;
    const float *b_outer;
    void *c;
    const int64_t *tiles;     // row-grouped form: packed (group << 40) | first row; WGRAD: padded starts [G+1]
    int64_t *sched;           // NXCD work-queue counters, then (row-grouped form) the listed row-tile count
    int64_t G, M, N, K, ldc, a_rows;
    int64_t ntm;              // row tiles (row-grouped form: tile-list length; WGRAD: G * ceil(M / BM))
    int64_t ntn;              // column tiles
};

// Row-tile list for the row-grouped form: tiles[i] = (g << 40) | first row, or -1.
__global__ void k_tile_list(const int64_t *__restrict__ off, int64_t G, int64_t M, int64_t bm, int64_t ntile_max,
                            int64_t *__restrict__ tiles, int64_t *__restrict__ sched) {
    __shared__ int64_t base[1025];
    int64_t carry = 0;
    for (int64_t g0 = 0; g0 < G; g0 += 1024) {
        const int64_t n = (G - g0) < 1024 ? (G - g0) : 1024;
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            int64_t lo = off[g0 + i], hi = off[g0 + i + 1];
            lo = lo < M ? lo : M;
            hi = hi < M ? hi : M;
            base[i + 1] = hi > lo ? (hi - lo + bm - 1) / bm : 0;
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
                tiles[t] = (g << 40) | (r0 + (t - base[i]) * bm);
        }
        carry = base[n];
        __syncthreads();
    }
    for (int64_t t = carry + threadIdx.x; t < ntile_max; t += blockDim.x) tiles[t] = -1;
    if (threadIdx.x < NXCD) sched[threadIdx.x] = 0;
    if (threadIdx.x == 0) sched[NXCD] = carry < ntile_max ? carry : ntile_max;
}

// Padded group starts P (running sum of roundup32(n_g)) for the weight-gradient form.
__global__ void k_padded_starts(const int64_t *__restrict__ off, int64_t G, int64_t *__restrict__ P,
                                int64_t *__restrict__ sched) {
    if (threadIdx.x < NXCD) sched[threadIdx.x] = 0;
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        int64_t run = 0;
        for (int64_t g = 0; g < G; g++) {
            P[g] = run;
            run += (off[g + 1] - off[g] + 31) / 32 * 32;
        }
        P[G] = run;
    }
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

__device__ __forceinline__ uint32_t hmul2(uint32_t a, h2 s) {
    h2 x = __builtin_bit_cast(h2, a);
    x = x * s;
    return __builtin_bit_cast(uint32_t, x);
}

// ---------------------------------------------------------------------------
// Stage loaders: global -> registers (prefetch) and registers -> LDS.
// ---------------------------------------------------------------------------

// MXFP8 stage = 64 K bytes per row = two 32-value blocks.  For a 128-row
// operand loader thread t takes row t/2, block t%2; for 256 rows, row t and
// both blocks.
template <int ROWS>
struct MxStage {
    static constexpr int NB = ROWS * 2 / 256;   // 32-byte blocks per thread (1 or 2)
    uint4 v[NB][2];
    uint32_t s[NB];
};

template <int ROWS>
__device__ __forceinline__ void mx_load(MxStage<ROWS> &st, const uint8_t *codes, const uint8_t *scales,
                                        int64_t ld, const int64_t *rowp, int64_t k0, int64_t kend) {
    const int t = threadIdx.x;
#pragma unroll
    for (int b = 0; b < MxStage<ROWS>::NB; b++) {
        const int blk = (MxStage<ROWS>::NB == 1) ? (t & 1) : b;
        const int64_t kk = k0 + 32 * blk;
        const int64_t r = rowp[0];
        if (r >= 0 && kk < kend) {
            const uint4 *q = reinterpret_cast<const uint4 *>(codes + r * ld + kk);
            st.v[b][0] = q[0];
            st.v[b][1] = q[1];
            st.s[b] = scales[r * (ld / 32) + kk / 32];
        } else {
            st.v[b][0] = make_uint4(0u, 0u, 0u, 0u);
            st.v[b][1] = st.v[b][0];
            st.s[b] = 127u;
        }
    }
}

// LDS row layout (MXFP8): 64 code bytes + 16 pad; scales [rows][2].
constexpr int MX_LDS_STRIDE = 80;

template <int ROWS>
__device__ __forceinline__ void mx_store(const MxStage<ROWS> &st, uint8_t *sc, uint8_t *ss) {
    const int t = threadIdx.x;
    const int row = (MxStage<ROWS>::NB == 1) ? (t >> 1) : t;
#pragma unroll
    for (int b = 0; b < MxStage<ROWS>::NB; b++) {
        const int blk = (MxStage<ROWS>::NB == 1) ? (t & 1) : b;
        uint4 *d = reinterpret_cast<uint4 *>(sc + row * MX_LDS_STRIDE + 32 * blk);
        d[0] = st.v[b][0];
        d[1] = st.v[b][1];
        ss[row * 2 + blk] = (uint8_t)st.s[b];
    }
}

// NVFP4 stage = 64 K values per row = 32 code bytes (four 16-blocks).  For a
// 128-row operand thread t takes row t/2, blocks 2(t%2) and 2(t%2)+1; for 256
// rows, row t and all four blocks.
template <int ROWS>
struct NvStage {
    static constexpr int NP = ROWS * 2 / 256;   // pairs of 16-blocks per thread (1 or 2)
    uint32_t w[NP][4];
    uint32_t s[NP][2];
};

template <int ROWS>
__device__ __forceinline__ void nv_load(NvStage<ROWS> &st, const uint8_t *codes, const uint8_t *scales, int64_t K,
                                        int64_t r, int64_t k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int b = 0; b < NvStage<ROWS>::NP; b++) {
        const int pair = (NvStage<ROWS>::NP == 1) ? (t & 1) : b;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int64_t kk = k0 + 32 * pair + 16 * h;
            if (r >= 0 && kk < K) {
                const uint2 c = *reinterpret_cast<const uint2 *>(codes + r * (K / 2) + kk / 2);
                st.w[b][2 * h] = c.x;
                st.w[b][2 * h + 1] = c.y;
                st.s[b][h] = scales[r * (K / 16) + kk / 16];
            } else {
                st.w[b][2 * h] = 0u;
                st.w[b][2 * h + 1] = 0u;
                st.s[b][h] = 0u;
            }
        }
    }
}

// LDS row layout (NVFP4): 64 fp16 + 8 pad.
constexpr int NV_LDS_STRIDE = 72;   // in halves

template <int ROWS>
__device__ __forceinline__ void nv_store(const NvStage<ROWS> &st, _Float16 *sh) {
    const int t = threadIdx.x;
    const int row = (NvStage<ROWS>::NP == 1) ? (t >> 1) : t;
#pragma unroll
    for (int b = 0; b < NvStage<ROWS>::NP; b++) {
        const int pair = (NvStage<ROWS>::NP == 1) ? (t & 1) : b;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const float sf = e4m3_decode(st.s[b][h]);
            const h2 sv = {(_Float16)sf, (_Float16)sf};
            uint32_t o[8];
#pragma unroll
            for (int q = 0; q < 2; q++) {
                uint32_t hh[4];
                e2m1x8_to_f16(st.w[b][2 * h + q], hh);
#pragma unroll
                for (int j = 0; j < 4; j++) o[4 * q + j] = hmul2(hh[j], sv);
            }
            uint4 *d = reinterpret_cast<uint4 *>(sh + row * NV_LDS_STRIDE + 32 * pair + 16 * h);
            d[0] = make_uint4(o[0], o[1], o[2], o[3]);
            d[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
}

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------

// One output tile: its expert, rows, K range and the operand rows this
// thread stages (fixed for the whole K loop).
struct TileCtx {
    int64_t g, row0, row_end, kbeg, kend, col0, arow, brow, nk;
    const uint8_t *bc, *bs;
};

template <int FMT, int MODE, int BM>
__device__ __forceinline__ void tile_setup(const GemmArgs &p, int64_t lin, TileCtx &c) {
    const int t = threadIdx.x;
    const int64_t ty = lin / p.ntn, tx = lin - ty * p.ntn;
    if (MODE == BSP_GEMM_WGRAD) {
        const int64_t mt_per_g = (p.M + BM - 1) / BM;
        c.g = ty / mt_per_g;
        c.row0 = (ty - c.g * mt_per_g) * BM;
        c.row_end = p.M;
        c.kbeg = p.tiles[c.g];
        c.kend = c.kbeg + (p.group_offsets[c.g + 1] - p.group_offsets[c.g] + 31) / 32 * 32;
        c.kend = c.kend < p.K ? c.kend : p.K;  // offsets are trusted only up to the copies' width
        c.bc = p.b_codes;
        c.bs = p.b_scales;
    } else {
        const int64_t tile = p.tiles[ty];       // valid: ty < the tile count the setup kernel wrote
        c.g = tile >> 40;
        c.row0 = tile & ((1ll << 40) - 1);
        c.row_end = p.group_offsets[c.g + 1];
        c.row_end = c.row_end < p.M ? c.row_end : p.M;  // never past the rows of C
        c.kbeg = 0;
        c.kend = p.K;
        const int64_t bcs = (FMT == BSP_FMT_NVFP4) ? p.N * p.K / 2 : p.N * p.K;
        const int64_t bss = (FMT == BSP_FMT_NVFP4) ? p.N * p.K / 16 : p.N * p.K / 32;
        c.bc = p.b_codes + c.g * bcs;
        c.bs = p.b_scales + c.g * bss;
    }
    c.col0 = tx * GBN;
    c.nk = c.kend > c.kbeg ? (c.kend - c.kbeg + GBK - 1) / GBK : 0;
    const int lrow = (BM == 128) ? (t >> 1) : t;
    const int64_t r = c.row0 + lrow;
    c.arow = -1;
    if (r < c.row_end) {
        c.arow = r;
        if (MODE != BSP_GEMM_WGRAD && p.a_gather) {
            c.arow = (int64_t)p.a_gather[r];
            if (c.arow < 0 || c.arow >= p.a_rows) c.arow = -1;  // an out-of-range gather index reads as a zero row
        }
    }
    const int64_t cn = c.col0 + (t >> 1);
    c.brow = cn < p.N ? cn : -1;
}

// Persistent workgroups.  Each XCD owns a work queue over a contiguous chunk
// of the row-major tile sequence (so concurrent tiles on one L2 share the
// activation tile and neighbouring weight panels) and, once it is empty,
// steals from the other XCDs' queues, which balances experts of very
// different sizes.  While a tile's epilogue runs, the first K stage of the
// next tile is already being fetched.
template <int FMT, int MODE, bool BF16OUT, int BM>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs p) {
    constexpr int WM = BM / 2;            // rows per wavefront
    constexpr int TI = WM / 32;           // 32-row MFMA tiles per wavefront
    constexpr int LDS_ROW = (FMT == BSP_FMT_MXFP8) ? MX_LDS_STRIDE : NV_LDS_STRIDE * 2;   // bytes
    constexpr int STAGE_BYTES = (BM + GBN) * LDS_ROW + ((FMT == BSP_FMT_MXFP8) ? (BM + GBN) * 2 : 0);
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];
    __shared__ int64_t s_lin;

    const int t = threadIdx.x;

    const int64_t ntm = (MODE == BSP_GEMM_WGRAD) ? p.ntm : p.sched[NXCD];   // row tiles actually listed
    const int64_t total = ntm * p.ntn;
    const int64_t chunk = (total + NXCD - 1) / NXCD;
    const int xcd = blockIdx.x % NXCD;
    auto grab = [&]() -> int64_t {
        if (t == 0) {
            int64_t got = -1;
            for (int d = 0; d < NXCD && got < 0; d++) {
                const int q = (xcd + d) % NXCD;
                const int64_t qbeg = q * chunk;
                const int64_t qlen = (total - qbeg) < chunk ? (total - qbeg) : chunk;
                if (qlen <= 0) continue;
                const int64_t i = (int64_t)atomicAdd(reinterpret_cast<unsigned long long *>(p.sched + q), 1ull);
                if (i < qlen) got = qbeg + i;
            }
            s_lin = got;
        }
        __syncthreads();
        // Uniform across the workgroup: move it to scalar registers so the
        // whole tile context is computed once per wavefront, not per lane.
        const uint64_t u = (uint64_t)s_lin;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
        __syncthreads();
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };

    const int64_t ldk = p.K;
    MxStage<BM> ma;
    MxStage<GBN> mb;
    NvStage<BM> na;
    NvStage<GBN> nb;
    auto load = [&](const TileCtx &c, int64_t stage) {
        if (FMT == BSP_FMT_MXFP8) {
            mx_load<BM>(ma, p.a_codes, p.a_scales, ldk, &c.arow, c.kbeg + stage * GBK, c.kend);
            mx_load<GBN>(mb, c.bc, c.bs, ldk, &c.brow, c.kbeg + stage * GBK, c.kend);
        } else {
            nv_load<BM>(na, p.a_codes, p.a_scales, p.K, c.arow, stage * GBK);
            nv_load<GBN>(nb, c.bc, c.bs, p.K, c.brow, stage * GBK);
        }
    };
    uint8_t *const lA0 = smem, *const lB0 = smem + BM * LDS_ROW;
    uint8_t *const lAs0 = smem + (BM + GBN) * LDS_ROW, *const lBs0 = lAs0 + BM * 2;   // MXFP8 scales
    auto store = [&](int buf) {
        if (FMT == BSP_FMT_MXFP8) {
            mx_store<BM>(ma, lA0 + buf * STAGE_BYTES, lAs0 + buf * STAGE_BYTES);
            mx_store<GBN>(mb, lB0 + buf * STAGE_BYTES, lBs0 + buf * STAGE_BYTES);
        } else {
            nv_store<BM>(na, reinterpret_cast<_Float16 *>(lA0 + buf * STAGE_BYTES));
            nv_store<GBN>(nb, reinterpret_cast<_Float16 *>(lB0 + buf * STAGE_BYTES));
        }
    };

    v16f acc[TI][2];
    TileCtx cur, nxt;
    int64_t lin = grab();
    bool have = lin >= 0;
    if (have) {
        tile_setup<FMT, MODE, BM>(p, lin, cur);
        if (cur.nk > 0) load(cur, 0);
    }
    while (have) {
        // Per-lane LDS offsets are rederived for every tile from an opaque
        // copy of the thread index; hoisted out of the tile loop they would
        // stay live through the epilogue and cost occupancy.
        int tq = threadIdx.x;
        asm volatile("" : "+v"(tq));
        const int lane = tq & 63, wave = tq >> 6;
        const int wm = wave >> 1, wn = wave & 1;
        const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

        // ---- K loop: double-buffered LDS, next stage prefetched in registers ----
        const int64_t nk = cur.nk;
        if (nk > 0) store(0);
        if (nk > 1) load(cur, 1);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; kt++) {
            const int buf = (int)(kt & 1);
            if (FMT == BSP_FMT_MXFP8) {
                const uint8_t *A = lA0 + buf * STAGE_BYTES, *B = lB0 + buf * STAGE_BYTES;
                const uint8_t *AS = lAs0 + buf * STAGE_BYTES, *BS = lBs0 + buf * STAGE_BYTES;
                // Row bytes [0, 32) hold K block 0 and [32, 64) block 1.  The
                // instruction wants lane half h to supply bytes [16h, 16h + 16) of
                // block 0 then of block 1 (offsets 16h and 32 + 16h), with the
                // E8M0 byte of block h.
                v8i af[TI], bf[2];
                int as[TI], bsc[2];
#pragma unroll
                for (int i = 0; i < TI; i++) {
                    const int r = wm * WM + 32 * i + lr;
                    const uint4 u0 = *reinterpret_cast<const uint4 *>(A + r * MX_LDS_STRIDE + 16 * lh);
                    const uint4 u1 = *reinterpret_cast<const uint4 *>(A + r * MX_LDS_STRIDE + 32 + 16 * lh);
                    af[i] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
                    as[i] = AS[r * 2 + lh];
                }
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int r = wn * 64 + 32 * j + lr;
                    const uint4 u0 = *reinterpret_cast<const uint4 *>(B + r * MX_LDS_STRIDE + 16 * lh);
                    const uint4 u1 = *reinterpret_cast<const uint4 *>(B + r * MX_LDS_STRIDE + 32 + 16 * lh);
                    bf[j] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
                    bsc[j] = BS[r * 2 + lh];
                }
#pragma unroll
                for (int i = 0; i < TI; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0,
                                                                                    0, as[i], 0, bsc[j]);
            } else {
                const _Float16 *A = reinterpret_cast<const _Float16 *>(lA0 + buf * STAGE_BYTES);
                const _Float16 *B = reinterpret_cast<const _Float16 *>(lB0 + buf * STAGE_BYTES);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    v8h af[TI], bf[2];
#pragma unroll
                    for (int i = 0; i < TI; i++)
                        af[i] = *reinterpret_cast<const v8h *>(A + (wm * WM + 32 * i + lr) * NV_LDS_STRIDE + 16 * q +
                                                               8 * lh);
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        bf[j] = *reinterpret_cast<const v8h *>(B + (wn * 64 + 32 * j + lr) * NV_LDS_STRIDE + 16 * q +
                                                               8 * lh);
#pragma unroll
                    for (int i = 0; i < TI; i++)
#pragma unroll
                        for (int j = 0; j < 2; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
                }
            }
            if (kt + 1 < nk) store(buf ^ 1);
            if (kt + 2 < nk) load(cur, kt + 2);
            __syncthreads();
        }

        // ---- next tile: its first stage is fetched while this epilogue runs ----
        lin = grab();
        const bool have_next = lin >= 0;
        if (have_next) {
            tile_setup<FMT, MODE, BM>(p, lin, nxt);
            if (nxt.nk > 0) load(nxt, 0);
        }
        // ---- epilogue ----
        // The MFMA leaves lane l with column l % 32 of a 32 x 32 block and rows
        // 8 (e / 4) + 4 (l / 32) + e % 4.  Each wavefront stages one 32 x 64
        // slice of its outputs in LDS (the stage buffers are free: the K loop
        // ended with a barrier), then writes whole rows with 16-byte
        // non-temporal stores, so the output streams past L2 instead of
        // evicting reusable operand panels.
        constexpr int ESZ = BF16OUT ? 2 : 4;
        constexpr int VEC = 16 / ESZ;                  // elements per 16-byte store
        constexpr int CHUNKS = 64 / VEC;               // 16-byte chunks per 64-column row
        const float gb = (FMT == BSP_FMT_NVFP4) ? p.b_outer[cur.g] : 1.0f;
        const int64_t goff = (MODE == BSP_GEMM_WGRAD) ? cur.g * p.M * p.ldc : 0;
        uint8_t *ep = smem + wave * (32 * 64 * ESZ);
        const bool vec_ok = (p.ldc % VEC) == 0;
#pragma unroll
        for (int i = 0; i < TI; i++) {
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int rin = 8 * (e >> 2) + 4 * lh + (e & 3);
                float sc = 1.0f;
                if (FMT == BSP_FMT_NVFP4) {
                    const int64_t r = cur.row0 + wm * WM + 32 * i + rin;
                    sc = 0.0f;
                    if (r < cur.row_end) {
                        const int64_t tt = p.a_gather ? (int64_t)p.a_gather[r] : r;
                        sc = (tt >= 0 && tt < p.a_rows) ? p.a_outer[tt] * gb : 0.0f;
                    }
                }
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const float v = acc[i][j][e] * sc;
                    const int cin = 32 * j + lr;
                    if (BF16OUT) reinterpret_cast<uint16_t *>(ep)[rin * 64 + cin] = (uint16_t)f32_to_bf16(v);
                    else reinterpret_cast<float *>(ep)[rin * 64 + cin] = v;
                }
            }
            __syncthreads();
#pragma unroll
            for (int pass = 0; pass < 32 * CHUNKS / 64; pass++) {
                const int idx = pass * 64 + lane;
                const int rin = idx / CHUNKS, ch = idx % CHUNKS;
                const int64_t r = cur.row0 + wm * WM + 32 * i + rin;
                const int64_t cn = cur.col0 + wn * 64 + ch * VEC;
                if (r >= cur.row_end || cn >= p.N) continue;
                const uint4 v = *reinterpret_cast<const uint4 *>(ep + (rin * 64 + ch * VEC) * ESZ);
                char *dst = reinterpret_cast<char *>(p.c) + (goff + r * p.ldc + cn) * ESZ;
                if (vec_ok && cn + VEC <= p.N) {
                    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(dst));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                    for (int q = 0; q < VEC && cn + q < p.N; q++) {
                        if (BF16OUT) reinterpret_cast<uint16_t *>(dst)[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
                        else reinterpret_cast<uint32_t *>(dst)[q] = w[q];
                    }
                }
            }
            __syncthreads();
        }
        cur = nxt;
        have = have_next;
    }
}

// Rows per tile.  Measured on the DeepSeek-V3-shaped forward GEMM, 128-row
// tiles (three wavefronts per SIMD) beat 256-row tiles (one wavefront per
// SIMD, fewer weight re-reads) by 1.2x: the kernel is latency-bound, so
// occupancy matters more than the extra panel fetches, which mostly hit L2.
// The 256-row variant is kept behind a build switch for such measurements.
#ifndef BSP_GEMM_BM256_BELOW_ROWS_PER_GROUP
#define BSP_GEMM_BM256_BELOW_ROWS_PER_GROUP 0
#endif
static int pick_bm(int mode, int64_t M, int64_t G) {
    if (mode == BSP_GEMM_WGRAD) return 128;
    return (M / G) < BSP_GEMM_BM256_BELOW_ROWS_PER_GROUP ? 256 : 128;
}

int64_t gemm_tile_count(int64_t M, int64_t G) { return (M + 127) / 128 + G; }

// Workgroups resident per XCD for one instantiation on the current device
// (compute units per XCD times workgroups per compute unit), cached per device.
template <typename Kern>
static int64_t resident_per_xcd(Kern kern, int *cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    if (cache[dev] == 0) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 256, 0) != hipSuccess || occ <= 0) occ = 1;
        cache[dev] = (cus + NXCD - 1) / NXCD * occ;
    }
    return cache[dev];
}

template <int FMT, int MODE, bool BF, int BM>
static void launch_one(const GemmArgs &p, hipStream_t s) {
    static int cache[kMaxDevices] = {};
    const int64_t per_xcd_max = resident_per_xcd(k_gemm<FMT, MODE, BF, BM>, cache);
    const int64_t total = p.ntm * p.ntn;            // upper bound of the tile count
    const int64_t per_xcd_need = (total + NXCD - 1) / NXCD;
    const int64_t per_xcd = per_xcd_need < per_xcd_max ? per_xcd_need : per_xcd_max;
    dim3 grid((unsigned)(per_xcd * NXCD)), block(256);
    k_gemm<FMT, MODE, BF, BM><<<grid, block, 0, s>>>(p);
}

template <int FMT, int MODE, int BM>
static void launch_k(const GemmArgs &p, bool bf, hipStream_t s) {
    if (bf) launch_one<FMT, MODE, true, BM>(p, s);
    else launch_one<FMT, MODE, false, BM>(p, s);
}

hipError_t launch_gemm(int fmt, int mode, const uint8_t *a_codes, const uint8_t *a_scales, const float *a_outer,
                       const int32_t *a_gather, int64_t a_rows, const int64_t *group_offsets, int64_t G,
                       int64_t M, int64_t N, int64_t K, const uint8_t *b_codes, const uint8_t *b_scales,
                       const float *b_outer, void *c, int c_dtype, int64_t ldc, void *workspace, hipStream_t s) {
    GemmArgs p;
    p.a_codes = a_codes; p.a_scales = a_scales; p.a_outer = a_outer; p.a_gather = a_gather;
    p.group_offsets = group_offsets; p.b_codes = b_codes; p.b_scales = b_scales; p.b_outer = b_outer;
    p.c = c; p.G = G; p.M = M; p.N = N; p.K = K; p.ldc = ldc; p.a_rows = a_rows;
    int64_t *ws = reinterpret_cast<int64_t *>(workspace);
    p.tiles = ws;
    // Work-queue counters follow the tile list (or the padded starts).
    p.sched = ws + (mode == BSP_GEMM_WGRAD ? G + 1 : gemm_tile_count(M, G));
    p.ntn = (N + GBN - 1) / GBN;
    const bool bf = c_dtype == BSP_DTYPE_BF16;
    if (mode == BSP_GEMM_WGRAD) {
        k_padded_starts<<<1, 64, 0, s>>>(group_offsets, G, ws, p.sched);
        p.ntm = G * ((M + 127) / 128);
        launch_k<BSP_FMT_MXFP8, BSP_GEMM_WGRAD, 128>(p, bf, s);
        return hipGetLastError();
    }
    const int bm = pick_bm(mode, M, G);
    p.ntm = (M + bm - 1) / bm + G;   // upper bound of the row-tile count
    k_tile_list<<<1, 256, 0, s>>>(group_offsets, G, M, bm, p.ntm, ws, p.sched);
#if BSP_GEMM_BM256_BELOW_ROWS_PER_GROUP > 0
    if (bm == 256) {
        if (fmt == BSP_FMT_MXFP8) launch_k<BSP_FMT_MXFP8, BSP_GEMM_FPROP, 256>(p, bf, s);
        else launch_k<BSP_FMT_NVFP4, BSP_GEMM_FPROP, 256>(p, bf, s);
        return hipGetLastError();
    }
#endif
    (void)bm;
    if (fmt == BSP_FMT_MXFP8) launch_k<BSP_FMT_MXFP8, BSP_GEMM_FPROP, 128>(p, bf, s);
    else launch_k<BSP_FMT_NVFP4, BSP_GEMM_FPROP, 128>(p, bf, s);
    return hipGetLastError();
}

}  // namespace bsp

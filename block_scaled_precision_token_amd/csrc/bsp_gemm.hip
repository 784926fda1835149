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
// powers of two per 32, so each wavefront rebuilds its operand fragments
// q * s exactly in fp16 (E2M1 times E4M3 has at most 6 significant bits and a
// magnitude in [2^-10, 2688]) and multiplies on the fp16 MFMA
// (V_MFMA_F32_32X32X16_F16); the FP32 outer scales (per token for A, per
// expert for B) are applied in the epilogue.
//
// Data movement.  Operand tiles stream from global memory straight into LDS
// with the gfx950 LDS-DMA loads (GLOBAL_LOAD_LDS_DWORDX4 for codes, _DWORD
// or _DWORDX4 for scales): no registers are spent on staging.  A ring of LDS
// stages keeps the next stages in flight while one is multiplied.  The
// forward and data-gradient forms stage 128 K values (MXFP8: 128 bytes of
// every operand row, whole 128-byte lines, in a ring of two stages; NVFP4: 64
// bytes, in a ring of four; BF16 64 values, 128 bytes, two stages): the
// per-CU count of outstanding memory requests is what bounds these loads, so
// bytes per request matter (8 % faster than 64-value stages on the
// DeepSeek-V3 MXFP8 shapes, 1-3 % on the Qwen3 NVFP4 and BF16 ones).  The
// weight-gradient forms stage half as many (64, BF16 32) in a ring of four.
// The ring runs across tile boundaries: the first stages of a workgroup's
// next tile are fetched while the current tile is finished and written back.
// Completion is tracked with explicit vmcnt waits (loads retire in order, so
// "at most n stages outstanding" means the oldest stage has landed) followed
// by a workgroup barrier; the epilogue's stores are issued so that the
// compiler's own counter model stays exact.
//
// LDS layout of a stage: per operand BT rows of code bytes (128 or 64 for
// MXFP8, 64 or 32 for NVFP4), the 16-byte chunks of row r stored at position
// chunk ^ swz(r) so that the 32 rows read by one fragment load hit distinct
// banks; then the
// stage's scale bytes as copied from the scale planes a setup kernel builds
// in the workspace: block-major ([scale block][row]) for MXFP8, in block
// pairs (a row's two scales of one lane half as a 16-bit word) for the NVFP4
// weight gradient, and in the order the lanes read them (one 8-byte chunk per
// lane and 32-row pair) for the NVFP4 row-grouped forms.
//
// Tiling: output tiles of BT x BT (256 on eight wavefronts, or 128 on four),
// each wavefront (BT / 2) x 64 outputs; wavefronts skip
// the 32-row blocks of a tile past its expert's rows.  Row tiles never
// straddle two experts: a setup kernel lists
// the (expert, first row) of every row tile from the device-side group
// offsets, so no host synchronization is needed.  Persistent workgroups walk a
// static tile sequence: for the row-grouped forms an XCD-contiguous chunk of
// the row-major tile order (workgroups resident on one XCD share activation
// rows and weight panels in that XCD's L2).  In the weight-gradient form a
// tile's cost is its expert's token count, which under skewed routing spans
// three orders of magnitude: a setup kernel orders the experts by token
// count, largest first, and workgroup b takes tiles b, 2P - 1 - b, 2P + b, ...
// of that order (P workgroups), so the longest tiles are spread first and the
// short ones fill in behind them.
#include <stdlib.h>

#include <atomic>

#include "bsp_device.hpp"
#include "bsp_internal.hpp"

namespace bsp {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int GBK = 64;    // K values per MFMA step of the block-scaled formats (a stage holds one or two)
constexpr int FMT_BF16 = 2;   // plain bf16 operands (internal format tag of the BF16 GEMM)
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
    const int32_t *order;     // WGRAD: experts by decreasing token count
    int64_t *sched;           // [NXCD] spare counters, then (row-grouped form) the listed row-tile count
    // Sizes fit 32 bits (checked at the C ABI), as do all tile and stage
    // counts; byte offsets are formed in 64 bits where they can exceed that.
    int32_t G, M, N, K, ldc, a_rows;
    int32_t ntm;              // row tiles (row-grouped form: upper bound; WGRAD: G * ceil(M / BT))
    int32_t ntn;              // column tiles
    // Scale planes in the workspace: plane[(z * nbp + block) * rp + row]
    // (NVFP4 forms: the same bytes in block pairs or lane order, k_scale_plane),
    // one byte per (block, row), rows of the A plane in tile-list order.
    const uint8_t *a_plane, *b_plane;
    int32_t a_rp, b_rp, nbp;
    // BF16 GEMM: bytes per operand row, and (weight-gradient form) the gather
    // of B's rows with B's row count.
    int32_t lda_b, ldb_b;
    const int32_t *b_gather;
    int32_t b_rows;
};

// Row-tile list for the row-grouped form: tiles[i] = (g << 40) | first row, or -1.
// One workgroup of 256 threads, per pass of 1024 groups: each thread counts
// the row tiles of four groups (the five offsets it needs loaded before any
// is used; the tile edge bm = 2^lbm makes the count a shift), a workgroup
// scan places the groups, and the pass's tiles are then written by all
// threads, each finding its tile's group by a binary search over the
// groups' first tiles in LDS (an expert with many row tiles would otherwise
// leave one thread writing all of them).
__global__ __launch_bounds__(256) void k_tile_list(const int64_t *__restrict__ off, int64_t G, int64_t M,
                                                   int lbm, int64_t ntile_max, int64_t *__restrict__ tiles,
                                                   int64_t *__restrict__ sched) {
    __shared__ int64_t wsum[4];
    __shared__ int64_t first[1024], row0[1024];
    const int t = threadIdx.x;
    const int64_t bm = (int64_t)1 << lbm;
    int64_t carry = 0;
    for (int64_t g0 = 0; g0 < G; g0 += 1024) {
        int64_t o[5];
#pragma unroll
        for (int q = 0; q < 5; q++) {
            const int64_t g = g0 + 4 * t + q;
            o[q] = g <= G ? off[g] : 0;
        }
        int64_t cnt[4], local = 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int64_t g = g0 + 4 * t + q;
            const int64_t lo = o[q] < M ? o[q] : M, hi = o[q + 1] < M ? o[q + 1] : M;
            cnt[q] = g < G && hi > lo ? (hi - lo + bm - 1) >> lbm : 0;
            local += cnt[q];
        }
        int64_t total;
        int64_t base = block256_excl_scan(local, wsum, total);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            first[4 * t + q] = base;
            row0[4 * t + q] = o[q];
            base += cnt[q];
        }
        __syncthreads();
        // tile i of the pass: group k = the last with first[k] <= i (it has tiles)
        for (int64_t i = t; i < total && carry + i < ntile_max; i += blockDim.x) {
            int lo = 0, hi = 1024;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (first[mid] <= i) lo = mid;
                else hi = mid;
            }
            tiles[carry + i] = ((g0 + lo) << 40) | (row0[lo] + (i - first[lo]) * bm);
        }
        __syncthreads();   // first / row0 are rewritten by the next pass
        carry += total;
    }
    for (int64_t i = carry + t; i < ntile_max; i += blockDim.x) tiles[i] = -1;
    if (t < NXCD) sched[t] = 0;
    if (t == 0) sched[NXCD] = carry < ntile_max ? carry : ntile_max;
}

// Weight-gradient form: the experts in order of decreasing token count (ties
// by index), by rank counting over the counts staged in LDS; past 4096
// experts the O(G^2) count is not worth it and the order stays the identity.
constexpr int kOrderMaxG = 4096;
__global__ __launch_bounds__(1024) void k_wgrad_order(const int64_t *__restrict__ off, int64_t G,
                                                      int32_t *__restrict__ order) {
    __shared__ int64_t cnt[kOrderMaxG];
    if (G > kOrderMaxG) {
        for (int64_t g = threadIdx.x; g < G; g += blockDim.x) order[g] = (int32_t)g;
        return;
    }
    const int n = (int)G;
    for (int g = threadIdx.x; g < n; g += blockDim.x) cnt[g] = off[g + 1] - off[g];
    __syncthreads();
    for (int g = threadIdx.x; g < n; g += blockDim.x) {
        const int64_t c = cnt[g];
        int rank = 0;
        for (int h = 0; h < n; h++) rank += (cnt[h] > c) || (cnt[h] == c && h < g);
        order[rank] = g;
    }
}

// Padded group starts P (running sum of roundup32(n_g)) for the weight-gradient
// form, by a workgroup scan over passes of 1024 groups (256 threads).
__global__ __launch_bounds__(256) void k_padded_starts(const int64_t *__restrict__ off, int64_t G,
                                                       int64_t *__restrict__ P, int64_t *__restrict__ sched) {
    __shared__ int64_t wsum[4];
    const int t = threadIdx.x;
    if (t < NXCD) sched[t] = 0;
    int64_t carry = 0;
    for (int64_t g0 = 0; g0 < G; g0 += 1024) {
        int64_t o[5], pn[4], local = 0;
#pragma unroll
        for (int q = 0; q < 5; q++) {
            const int64_t g = g0 + 4 * t + q;
            o[q] = g <= G ? off[g] : 0;
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int64_t g = g0 + 4 * t + q;
            pn[q] = g < G ? (o[q + 1] - o[q] + 31) / 32 * 32 : 0;
            local += pn[q];
        }
        int64_t total;
        int64_t run = carry + block256_excl_scan(local, wsum, total);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int64_t g = g0 + 4 * t + q;
            if (g < G) P[g] = run;
            run += pn[q];
        }
        carry += total;
    }
    if (t == 0) P[G] = carry;
}

// Scale planes.  The operands' scales arrive row-major ([rows][K / SBLK]);
// a K step needs SBLK-th bytes from every row of a tile, which as loads are
// one cache line per row.  Transposed to block-major planes, the bytes of a
// K step for the tile's rows are contiguous: a few lines per operand.
// plane[(z * nbp + b) * rp + r] = scale b of the source row of (z, r), or 0
// where (z, r) has no source row or b is past the row's blocks (the NVFP4
// forms place the same bytes in block pairs or lane order, below).
struct PlaneArgs {
    const uint8_t *src;
    int64_t src_rows;          // rows of src
    int32_t sr;                // scale bytes per source row (= blocks per row)
    uint8_t *plane;
    int32_t nbp, rp;           // padded blocks, row pitch of the plane
    int32_t rows_z;            // direct map: source row of (z, r) = z * rows_z + r for r < rows_z
    // tile-list map (row-grouped A): plane row r = slot * bt + i
    const int64_t *tiles, *sched, *off;
    const int32_t *gather;
    int32_t bt, M, a_rows;
    // 0: block-major as above; 1: lane order of the NVFP4 row-grouped GEMM
    // with tile edge bt; 2: block pairs of the NVFP4 weight-gradient GEMM
    // (see k_scale_plane)
    int32_t lane;
};

template <bool TILE_MAP>
__global__ __launch_bounds__(256) void k_scale_plane(PlaneArgs a) {
    __shared__ uint8_t tr[64][65];
    const int t = threadIdx.x;
    const int r0 = blockIdx.x * 64, b0 = blockIdx.y * 64, z = blockIdx.z;
    {
        const int rr = t >> 2, part = t & 3;
        const int r = r0 + rr;
        int64_t srow = -1;
        if (TILE_MAP) {
            const int slot = r / a.bt, i = r - slot * a.bt;
            if (slot < *a.sched) {
                const int64_t tile = a.tiles[slot];
                const int64_t g = tile >> 40, gr = (tile & ((1ll << 40) - 1)) + i;
                const int64_t re = a.off[g + 1] < a.M ? a.off[g + 1] : a.M;
                if (gr < re) {
                    const int64_t tok = a.gather ? (int64_t)a.gather[gr] : gr;
                    if (tok >= 0 && tok < a.a_rows) srow = tok;
                }
            }
        } else if (r < a.rows_z) {
            srow = (int64_t)z * a.rows_z + r;
        }
        const int bb = b0 + 16 * part;
        const uint8_t *src = a.src + srow * a.sr + bb;
        if (srow >= 0 && bb + 16 <= a.sr && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
            const uint4 v = *reinterpret_cast<const uint4 *>(src);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 16; k++) tr[rr][16 * part + k] = (uint8_t)(w4[k >> 2] >> (8 * (k & 3)));
        } else {
#pragma unroll
            for (int k = 0; k < 16; k++) tr[rr][16 * part + k] = (srow >= 0 && bb + k < a.sr) ? src[k] : 0;
        }
    }
    __syncthreads();
    if (a.lane == 2) {
        // Block pairs (NVFP4 weight-gradient GEMM): plane[(b / 2) 2 rp + 2 r +
        // (b & 1)], so a row's scales of blocks 2p and 2p + 1 are one 16-bit
        // word (groups start on even blocks, so a stage of 4 blocks is 2
        // whole pairs).  Thread (pair, 8-row piece) writes 16 bytes.
        const int pp = t >> 3, piece = t & 7;
        const int b = b0 + 2 * pp;
        if (b >= a.nbp) return;
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int rr = 8 * piece + 2 * k;
            v[k] = (uint32_t)tr[rr][2 * pp] | ((uint32_t)tr[rr][2 * pp + 1] << 8) |
                   ((uint32_t)tr[rr + 1][2 * pp] << 16) | ((uint32_t)tr[rr + 1][2 * pp + 1] << 24);
        }
        uint8_t *dst = a.plane + (int64_t)z * a.nbp * a.rp + (int64_t)(b / 2) * 2 * a.rp + 2 * (r0 + 8 * piece);
        *reinterpret_cast<uint4 *>(dst) = make_uint4(v[0], v[1], v[2], v[3]);
        return;
    }
    if (a.lane) {
        // Lane order (NVFP4 row-grouped GEMM): per tile of bt rows and stage
        // of 8 blocks, the stage's bt * 8 bytes hold one 8-byte chunk per
        // (64-row window w, lane row lr, lane half h), chunk (32 w + lr) 2 + h,
        // byte 4 s + 2 ii + e = scale of row 64 w + 32 ii + lr, block
        // 4 s + 2 h + e of the stage: a GEMM lane reads its scales of a stage
        // as whole chunks.  This block's 64 rows are one window: thread
        // (stage, lr) writes the two chunks of lr, 16 contiguous bytes.
        const int rt = r0 / a.bt, w = (r0 - rt * a.bt) / 64;
        const int lr = t & 31, stl = t >> 5;
        const int st = b0 / 8 + stl;
        if (st * 8 >= a.nbp) return;
        uint32_t v[4];
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int s = 0; s < 2; s++) {
                uint32_t d = 0;
#pragma unroll
                for (int ii = 0; ii < 2; ii++)
#pragma unroll
                    for (int e = 0; e < 2; e++)
                        d |= (uint32_t)tr[32 * ii + lr][8 * stl + 4 * s + 2 * h + e] << (8 * (2 * ii + e));
                v[2 * h + s] = d;
            }
        const int64_t o = (int64_t)z * a.nbp * a.rp + ((int64_t)rt * (a.nbp / 8) + st) * 8 * a.bt + (w * 32 + lr) * 16;
        *reinterpret_cast<uint4 *>(a.plane + o) = make_uint4(v[0], v[1], v[2], v[3]);
        return;
    }
    {
        const int bl = t >> 2, part = t & 3;
        const int b = b0 + bl;
        if (b < a.nbp) {
            uint32_t w4[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int i = 16 * part + 4 * q;
                w4[q] = (uint32_t)tr[i][bl] | ((uint32_t)tr[i + 1][bl] << 8) | ((uint32_t)tr[i + 2][bl] << 16) |
                        ((uint32_t)tr[i + 3][bl] << 24);
            }
            uint8_t *dst = a.plane + ((int64_t)z * a.nbp + b) * a.rp + r0 + 16 * part;
            *reinterpret_cast<uint4 *>(dst) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
    }
}

// ---------------------------------------------------------------------------
// Stage geometry, LDS-DMA and synchronization helpers.
// ---------------------------------------------------------------------------
// Square output tiles of BT x BT (BT = 128 or 256) on BT / 32 wavefronts in
// 2 x (BT / 64): each wavefront owns (BT / 2) x 64 outputs, i.e. TI x 2
// MFMA blocks of 32 x 32.
// BF16 stages hold 32 K values in the MXFP8 geometry (64 bytes per K-major
// row); an operand stored with its M or N dimension contiguous (MN-major,
// BF16 only) occupies the same bytes as 32 K rows of BT elements.
template <int FMT, int BT, bool WIDE = false>
struct Geo {
    static constexpr bool MX = FMT == BSP_FMT_MXFP8;
    static constexpr bool BF = FMT == FMT_BF16;
    static constexpr int BK = (BF ? 32 : GBK) * (WIDE ? 2 : 1);   // K values per stage
    static constexpr int NW = BT / 32;                 // wavefronts
    static constexpr int TI = BT / 64;                 // 32-row MFMA blocks per wavefront
    static constexpr int ROWB = MX ? BK : BF ? 2 * BK : BK / 2;   // code bytes per row per stage
    static constexpr int CH = ROWB / 16;               // 16-byte chunks per row
    static constexpr int CODE = BT * ROWB;             // one operand's codes per stage
    static constexpr int CIW = CODE / 1024 / NW;       // 1 KB DMA loads per wavefront per operand
    static constexpr int RPI = 64 / (BT / 8);          // MN-major K rows per wavefront DMA load
    static constexpr int KPW = CIW * RPI;              // MN-major K rows per wavefront per stage
    static constexpr int SBLK = MX ? 32 : 16;          // values per scale
    static constexpr int SPS = BF ? 0 : BK / SBLK;     // scales per row per stage
    static constexpr int SCLB = SPS * BT;              // scale bytes per operand per stage: [SPS][BT]
    static constexpr int A_SCL = 2 * CODE;
    static constexpr int B_SCL = 2 * CODE + SCLB;
    // scale DMA loads: one dword per lane (256 bytes) where the stage's scale
    // bytes fit one such load per wavefront, else 16 bytes per lane (1 KB)
    static constexpr int SCW = 2 * SCLB / 256 <= NW ? 4 : 16;
    static constexpr int SCI = 2 * SCLB / (64 * SCW);  // scale DMA loads per stage (both operands)
    static constexpr int OPS = 2 * CIW;                // code DMA loads per wavefront per stage (+1 for w < SCI)
    // a ring stage also serves as the epilogue's transpose patch (32 x 144 bytes per wavefront)
    static constexpr int SLOT = (2 * CODE + 2 * SCLB) > NW * 4608 ? (2 * CODE + 2 * SCLB) : NW * 4608;
    // ring stages: four where they fit the LDS, else two (the wide stage)
    static constexpr int NS = 4 * SLOT <= 152 * 1024 ? 4 : 2;
    static constexpr int VPC = MX ? 16 : 32;           // K values per 16-byte code chunk (block-scaled)
    static_assert(CIW >= 1 && SCI <= NW && SCI % 2 == 0, "DMA split over the wavefronts");
};

// The geometry of each GEMM form: the row-grouped forms (forward, data
// gradient) stage twice the K values of the weight-gradient form: 128 for
// the block-scaled formats (64 in the weight gradient), 64 for BF16 (32).  Every use
// (tile decoding, the kernel, the workspace layout) goes through this one
// definition, so the stage count of a tile and the stages the kernel loads
// agree.
template <int FMT, int MODE, int BT>
using GeoOf = Geo<FMT, BT, MODE != BSP_GEMM_WGRAD>;

// Chunk position of chunk c of row r is c ^ swz(r): a fragment load reads one
// chunk from each of 32 consecutive rows, and with this swizzle every group
// of 8 (or 16) rows served together lands on distinct LDS banks.
template <int CH>
__device__ __forceinline__ int swz(int r) {
    return CH == 8 ? (r & 7) : CH == 4 ? (((r >> 1) ^ (r >> 3)) & 3) : (((r >> 2) ^ (r >> 3)) & 1);
}
// MN-major stages: K row k holds BT / 8 chunks of 8 elements, chunk c stored
// at position c ^ swz_mn(k).  A transposed fragment read (below) touches 8 K
// rows, four consecutive ones twice, 64 bytes each; the XOR moves the four
// consecutive rows to distinct 64-byte bank windows.
__device__ __forceinline__ int swz_mn(int k) { return 4 * (k & 3); }

// LDS-DMA: every lane fetches `size` bytes from its own global address; the
// wavefront's data lands contiguously at M0 + lane * size.  Issued as inline assembly: the
// compiler would otherwise track these writes to LDS itself and, unable to
// follow the ring across loop iterations, wait for all of them before every
// LDS read.  Completion is covered by the explicit waits of the pipeline.
// M0 is a reserved register: the compiler sets it right before each of its
// own uses and keeps nothing in it, so the asm may overwrite it freely; the
// s_nop covers the M0-write to LDS-DMA hazard.
// The pipeline's vector-memory waits count these loads only, so the kernel
// must not spill to scratch (checked by a CPU test on the compiled code).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}
// base: wave-uniform 64-bit global address (SGPRs); voff: this lane's 32-bit
// byte offset from it; m0: the wave's LDS destination.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const uint8_t *base, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0)
                 : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t *base, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(m0)
                 : "memory");
}
// The same with a full 64-bit address per lane.
__device__ __forceinline__ void dma16v(const uint8_t *addr, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(m0) : "memory");
}
// Source of the chunks of a K stage that lie past the end of K.
__device__ __attribute__((aligned(16))) uint8_t kZeroChunk[16];

// s_waitcnt vmcnt(VM) lgkmcnt(LGKM) (expcnt untouched), gfx9 encoding.
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt() {
    static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}
// Workgroup barrier with no implied memory wait (a fence would wait for every
// outstanding LDS-DMA load); callers wait explicitly first.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until the oldest outstanding stage has landed: `ahead` younger stages
// (0..2) may stay in flight.
template <int OPS>
__device__ __forceinline__ void wait_stage(int ahead) {
    if (ahead >= 2) waitcnt<2 * OPS, 0>();
    else if (ahead == 1) waitcnt<OPS, 0>();
    else waitcnt<0, 0>();
}
// Wavefronts below `sci` issue one scale load per stage on top of OPS.
template <int OPS>
__device__ __forceinline__ void wait_stage_w(int ahead, bool scl) {
    if (scl) wait_stage<OPS + 1>(ahead);
    else wait_stage<OPS>(ahead);
}

// Output stores.  Issued as inline assembly so that the compiler's vmcnt
// bookkeeping, which would treat pending stores and loads as completing out
// of order and then wait for everything, only ever sees loads.  Store data
// registers are read at issue, so no wait is needed before reusing them.
__device__ __forceinline__ void st_nt16(void *p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off nt" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_b32(void *p, uint32_t v) {
    asm volatile("global_store_dword %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_b16(void *p, uint32_t v) {
    asm volatile("global_store_short %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

// Byte i (0..7) of a 64-bit word.
__device__ __forceinline__ uint32_t byte_of(uint64_t w, int i) { return (uint32_t)(w >> (8 * i)) & 0xFFu; }

// 8 E2M1 values (one dword, element 2j in the low nibble of byte j) times
// the fp16 scale s, exactly: V_CVT_SCALEF32_PK_F16_FP4 at scale 1 decodes two
// values, the packed fp16 multiply applies s (every product is representable).
__device__ __forceinline__ v8h nv_frag(uint32_t w, h2 s) {
    const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// The E4M3 pair in the low (HI false) or high half of w as two fp16 values,
// exactly (every E4M3 value is an fp16 value; scale 1).
template <bool HI>
__device__ __forceinline__ h2 e4m3_pair(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// One output tile: expert, rows [row0, row_end), columns from col0, K range.
struct Tile {
    int g, row0, row_end, col0, kbeg, kend;
    int nk;     // stages
    int slot;   // row-tile index (row-grouped form: position in the tile list)
};

// Load of a wave-uniform element through the scalar cache.  The tables read
// this way (tile list, group offsets, expert order, gathers) are written by
// earlier kernels, so the scalar cache, invalidated at kernel start, is
// coherent for them.  A vector load here would make the compiler wait for
// every outstanding vector-memory operation, the pipeline's LDS-DMA loads
// included, before using the value.
template <typename T>
__device__ __forceinline__ T sload(const T *p, int64_t i) {
    typedef const __attribute__((address_space(4))) T cT;
    return ((const cT *)p)[i];
}

template <int FMT, int MODE, int BT>
__device__ __forceinline__ Tile decode_tile(const GemmArgs &p, int lin) {
    constexpr int BK = GeoOf<FMT, MODE, BT>::BK;
    Tile T;
    const int ty = lin / p.ntn, tx = lin - ty * p.ntn;
    if (MODE == BSP_GEMM_WGRAD) {
        const int mt_per_g = (p.M + BT - 1) / BT;
        const int rank = ty / mt_per_g;
        T.g = __builtin_amdgcn_readfirstlane(sload(p.order, rank));
        T.row0 = (ty - rank * mt_per_g) * BT;
        T.row_end = p.M;
        // MXFP8: the group's padded token columns; BF16: the group's rows
        const int64_t o0 = sload(p.group_offsets, T.g), o1 = sload(p.group_offsets, T.g + 1);
        const int64_t kb = FMT == FMT_BF16 ? o0 : sload(p.tiles, T.g);
        const int64_t ke = FMT == FMT_BF16 ? o1 : kb + (o1 - o0 + 31) / 32 * 32;
        // offsets are trusted only up to the copies' width
        T.kbeg = (int)(kb < 0 ? 0 : kb < p.K ? kb : p.K);
        T.kend = (int)(ke < 0 ? 0 : ke < p.K ? ke : p.K);
        T.col0 = tx * BT;
        T.slot = ty;
    } else {
        // An expert's tiles occupy [t0 ntn, (t0 + nt) ntn) of the tile order
        // (t0: its first row tile, nt: its row-tile count); inside that range
        // the row tiles vary fastest, so the workgroups running an expert's
        // tiles at one time share its weight panels.
        const int64_t tile = sload(p.tiles, ty);   // valid: ty < the listed tile count
        T.g = __builtin_amdgcn_readfirstlane((int)(tile >> 40));
        const int64_t r0 = tile & ((1ll << 40) - 1);
        const int64_t rb = sload(p.group_offsets, T.g), re = sload(p.group_offsets, T.g + 1);
        // the row-tile count as the tile list counts it (rows clamped to M)
        const int64_t lo = rb < p.M ? rb : p.M, hi = re < p.M ? re : p.M;
        const int t0 = ty - (int)((r0 - rb) / BT);
        const int nt = hi > lo ? (int)((hi - lo + BT - 1) / BT) : 1;
        const int local = lin - t0 * p.ntn;
        const int tyc = t0 + local % nt;
        T.col0 = (local / nt) * BT;
        T.slot = tyc;
        T.row0 = (int)(rb + (int64_t)(tyc - t0) * BT);
        T.row_end = (int)(re < p.M ? re : p.M);   // never past the rows of C
        T.kbeg = 0;
        T.kend = p.K;
    }
    T.nk = T.kend > T.kbeg ? (T.kend - T.kbeg + BK - 1) / BK : 0;
    return T;
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int N>
struct IC {
    static constexpr int v = N;
};

template <int FMT, int MODE, bool BF16OUT, int BT>
__global__ __launch_bounds__(BT * 2) void k_gemm(GemmArgs p) {
    // The block-scaled row-grouped forms stage 128 K values (MXFP8: 128
    // bytes of every operand row, whole 128-byte L2 lines; NVFP4: 64 bytes):
    // fewer memory requests per byte than a 64-value stage, and the per-CU
    // count of outstanding requests is what bounds these loads.  MXFP8 then
    // needs a ring of two stages, NVFP4 keeps four (BF16 row-grouped forms: 64
    // values, 128 bytes, two stages); the weight-gradient forms stage half as
    // many (64, BF16 32) in a ring of four.
    using GG = GeoOf<FMT, MODE, BT>;
    constexpr int NS = GG::NS;
    // fragment-offset sets per stage: 64-value K steps (block-scaled), 32-value ones (BF16)
    constexpr int SUB = GG::BF ? GG::BK / 32 : GG::BK / GBK;
    constexpr int TI = GG::TI, SLOT_BYTES = GG::SLOT;
    constexpr bool MX = GG::MX, BF = GG::BF, NV = FMT == BSP_FMT_NVFP4;
    constexpr bool WG = MODE == BSP_GEMM_WGRAD;
    // NVFP4 row-grouped forms read scale planes in lane order, the weight-
    // gradient form in block pairs (k_scale_plane)
    constexpr bool NVL = NV && !WG, NVP = NV && WG;
    // BF16 operand layouts: the forward form takes both operands K-major; the
    // data-gradient form takes B as the forward weight is stored ([K, N] per
    // expert, N contiguous); the weight-gradient form reduces over rows, so
    // both operands arrive with M or N contiguous.
    constexpr bool A_MN = BF && WG, B_MN = BF && MODE != BSP_GEMM_FPROP;
    constexpr int RP = BT * 2;                         // bytes of an MN-major K row in LDS
    constexpr int SEEK = 1, FIN = 2;
    // Ring of NS K stages.
    __shared__ __attribute__((aligned(16))) uint8_t ring[NS * SLOT_BYTES];
    // Per tile (ordinal mod 8) and tile row: the A row read (-1: the row
    // reads as zero) and, for NVFP4, the row's outer scale times the expert's.
    // The producer runs at most 3 stages, hence at most 4 tiles, ahead.
    __shared__ int32_t rowtok[8][BT];
    __shared__ float rowmul[NV ? 8 : 1][BT];

    const int t = threadIdx.x, l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w / (GG::NW / 2), wn = w % (GG::NW / 2);   // 2 x (NW / 2) wavefronts
    const int lr = l & 31, lh = l >> 5;
    const uint32_t ring_lds = lds_addr(ring);

    // bytes per operand row
    const uint32_t ldA = BF ? (uint32_t)p.lda_b : MX ? p.K : p.K / 2;
    const uint32_t ldB = BF ? (uint32_t)p.ldb_b : ldA;

    // ---- static tile sequence of this workgroup ----
    int first, stride, last;
    if (WG) {
        first = blockIdx.x;
        stride = gridDim.x;   // P; the walk alternates direction every P tiles
        last = p.ntm * p.ntn;
    } else {
        const int total = (int)p.sched[NXCD] * p.ntn;   // listed row tiles x column tiles
        const int chunk = (total + NXCD - 1) / NXCD;
        const int x = blockIdx.x % NXCD;
        first = x * chunk + blockIdx.x / NXCD;
        stride = gridDim.x / NXCD;
        const int e = (x + 1) * chunk;
        last = e < total ? e : total;
    }

    // Next tile of this workgroup after `lin`: row-grouped forms lin + stride;
    // weight-gradient form the serpentine walk (lin = r P + x, x = b for even
    // rounds r and P - 1 - b for odd ones).
    auto next_tile = [&](int lin) __attribute__((always_inline)) -> int {
        if (!WG) return lin + stride;
        return lin + 2 * stride - 1 - 2 * (lin % stride);
    };

    // Fragment geometry (fixed per lane): LDS offsets inside a stage of the
    // code chunks and scale dwords this lane feeds to the MFMA.
    // Rows 32 apart share the swizzle, so one offset per operand serves all
    // of the wavefront's blocks (plus 32 * ROWB bytes per block).
    uint32_t fa0[SUB], fa1[SUB], fb0[SUB], fb1[SUB], fsa, fsb;
    // MN-major operands: base offset of this lane's transposed reads for each
    // 32-wide block (see mn_frag).
    uint32_t tra[A_MN ? TI : 1], trb[B_MN ? 2 : 1];
    {
        const int ra = wm * (BT / 2) + lr, rb = wn * 64 + lr;
        if (MX || BF) {
            // MFMA K step s of the stage: chunks 4 s + h and 4 s + 2 + h
#pragma unroll
            for (int s = 0; s < SUB; s++) {
                fa0[s] = ra * GG::ROWB + 16 * ((4 * s + lh) ^ swz<GG::CH>(ra));
                fa1[s] = ra * GG::ROWB + 16 * ((4 * s + 2 + lh) ^ swz<GG::CH>(ra));
                fb0[s] = GG::CODE + rb * GG::ROWB + 16 * ((4 * s + lh) ^ swz<GG::CH>(rb));
                fb1[s] = GG::CODE + rb * GG::ROWB + 16 * ((4 * s + 2 + lh) ^ swz<GG::CH>(rb));
            }
        } else {
            // NVFP4 K step s of the stage: chunk 2 s + h
#pragma unroll
            for (int s = 0; s < SUB; s++) {
                fa0[s] = fa1[s] = ra * GG::ROWB + 16 * ((2 * s + lh) ^ swz<GG::CH>(ra));
                fb0[s] = fb1[s] = GG::CODE + rb * GG::ROWB + 16 * ((2 * s + lh) ^ swz<GG::CH>(rb));
            }
        }
        // MXFP8 lane half h reads block h's byte; NVFP4 blocks 2h and 2h + 1
        // (row-grouped forms: the lane's chunk of the stage, k_scale_plane)
        if constexpr (NVL) {
            // the chunks of the lane's 64-row windows (A: TI / 2 of them, 512 bytes apart)
            fsa = GG::A_SCL + ((wm * (TI / 2)) * 32 + lr) * 16 + lh * 8;
            fsb = GG::B_SCL + (wn * 32 + lr) * 16 + lh * 8;
        } else if constexpr (NVP) {
            // the 16-bit word of block pair h of the lane's row
            fsa = GG::A_SCL + lh * 2 * BT + 2 * ra;
            fsb = GG::B_SCL + lh * 2 * BT + 2 * rb;
        } else {
            fsa = GG::A_SCL + (MX ? lh : 2 * lh) * BT + ra;
            fsb = GG::B_SCL + (MX ? lh : 2 * lh) * BT + rb;
        }
        // A transposed read (DS_READ_B64_TR_B16) works on groups of 16 lanes:
        // in-group lane 4 e + c gives the address of 4 consecutive elements
        // (piece c) of K row e, and in-group lane j receives element j of the
        // 16 columns from each of the 4 rows.  Lane group q = l / 16 serves
        // K rows 8 (q / 2) + 0..3 (lane half = K half) and columns
        // 16 (q % 2) + 0..15 of the block.
        const int q4 = l >> 4, e4 = (l >> 2) & 3, c4 = l & 3;
        auto tr_base = [&](int col) __attribute__((always_inline)) -> uint32_t {
            const int krow = 8 * (q4 >> 1) + e4;    // krow & 3 == e4
            const int chunk = (col >> 3) + 2 * (q4 & 1) + (c4 >> 1);
            return (uint32_t)(krow * RP + ((chunk ^ swz_mn(krow)) << 4) + 8 * (c4 & 1));
        };
#pragma unroll
        for (int i = 0; i < (A_MN ? TI : 1); i++) tra[i] = tr_base(wm * (BT / 2) + 32 * i);
#pragma unroll
        for (int j = 0; j < (B_MN ? 2 : 1); j++) trb[j] = GG::CODE + tr_base(wn * 64 + 32 * j);
    }

    // ---- producer state: next stage to fetch ----
    int p_lin = first;
    int p_ord = 0, p_kt = 0, p_nk = 0;
    bool p_done = false;
    Tile PT;
    const uint8_t *pca = nullptr, *pcb = nullptr;     // code bases of the tile (uniform)
    uint32_t poa[GG::CIW], pob[GG::CIW];              // this lane's code chunk offsets
    // Scale DMA (wavefronts w < SCI): operand and 64 SCW-byte piece of its
    // [SPS][BT] stage region; this lane covers block sbl, rows sr0..sr0+3.
    constexpr int SCH = GG::SCI > 0 ? GG::SCI / 2 : 1;
    const bool scl_w = GG::SCI > 0 && w < GG::SCI;
    const bool scl_b = w >= GG::SCI / 2;
    const int scl_o = 64 * GG::SCW * (w % SCH) + GG::SCW * l;
    // plane piece (block, or block pair for NVP) and offset in it of this lane's load
    const int sbl = scl_o / (NVP ? 2 * BT : BT), sr0 = scl_o % (NVP ? 2 * BT : BT);
    // lane offset in the plane (lane order: the stage's bytes are contiguous)
    const uint32_t psv = NVL ? (uint32_t)scl_o : (uint32_t)sbl * (NVP ? 2 : 1) * (scl_b ? p.b_rp : p.a_rp) + sr0;
    const uint8_t *psbase = nullptr;                   // plane at the tile's first block and row

    // A row of tile row r for the row-grouped form: its source row (or -1).
    // A row of tile row r for the row-grouped form: its source row (or -1).
    // (Vector loads: the compiler then waits for the pipeline's outstanding
    // loads once per tile; resolving the gather through scalar loads instead
    // measured slower, its code being much larger.)
    auto a_src = [&](const Tile &T, int r) __attribute__((always_inline)) -> int {
        const int gr = T.row0 + r;
        if (gr >= T.row_end) return -1;
        if (!p.a_gather) return gr;
        const int tok = p.a_gather[gr];
        return (tok >= 0 && tok < p.a_rows) ? tok : -1;
    };

    // BF16 producer set-up for tile PT.  K-major operands as for MXFP8 (unit u
    // = 64 (w CIW + j) + l covers row u / 4, chunk position u % 4; per-stage
    // offset 64 bytes); MN-major units cover K row u / (BT / 8), chunk
    // position u % (BT / 8).  Columns past the operand's width read its last
    // chunk (their outputs are discarded).
    auto bf_seek = [&](int ord) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < GG::CIW; j++) {
            const int u = 64 * (w * GG::CIW + j) + l;
            const int r = u / GG::CH, cp = u % GG::CH, c = cp ^ swz<GG::CH>(r);
            const int kr = u / (BT / 8), cm = (u % (BT / 8)) ^ swz_mn(kr);
            if constexpr (A_MN) {
                const int col = PT.row0 + 8 * cm < p.M - 8 ? PT.row0 + 8 * cm : p.M - 8;
                poa[j] = (uint32_t)kr * ldA + 2 * col;
            } else {
                const int s = a_src(PT, r);
                if (cp == 0) rowtok[ord][r] = s;
                poa[j] = (uint32_t)(s >= 0 ? s : 0) * ldA + 16 * c;
            }
            if constexpr (B_MN) {
                const int col = PT.col0 + 8 * cm < p.N - 8 ? PT.col0 + 8 * cm : p.N - 8;
                pob[j] = (WG ? 0u : (uint32_t)kr * ldB) + 2 * col;
            } else {
                const int n = PT.col0 + r < p.N ? PT.col0 + r : p.N - 1;
                pob[j] = (uint32_t)n * ldB + 16 * c;
            }
        }
        // A: weight-gradient form from the group's first row; B: the expert's
        // matrix ([N, K] forward form, [K, N] data-gradient form) or, in the
        // weight-gradient form, rows addressed one by one through the gather
        pca = p.a_codes + (WG ? (size_t)PT.kbeg * ldA : 0);
        pcb = p.b_codes + (WG ? 0 : (size_t)PT.g * (B_MN ? p.K : p.N) * ldB);
    };

    // Move the producer to the next tile with K work and set up this lane's
    // sources.  Tiles without K work (empty experts in the weight-gradient
    // form) are only written by the consumer.
    auto prod_seek = [&]() __attribute__((always_inline)) {
        while (p_lin < last) {
            PT = decode_tile<FMT, MODE, BT>(p, p_lin);
            if (PT.nk > 0) break;
            p_lin = next_tile(p_lin);
            p_ord++;
        }
        if (p_lin >= last) {
            p_done = true;
            return;
        }
        p_kt = 0;
        p_nk = PT.nk;
        const int ord = p_ord & 7;
        if constexpr (BF) {
            bf_seek(ord);
            return;
        }
        // weight-gradient form: code bytes from the group's first column
        pca = p.a_codes + (WG ? PT.kbeg / (MX ? 1 : 2) : 0);
        pcb = p.b_codes + (WG ? (size_t)(PT.kbeg / (MX ? 1 : 2)) : (size_t)PT.g * p.N * ldA);
        // codes: unit u = 64 (w CIW + j) + l covers row u / CH, chunk position u % CH
#pragma unroll
        for (int j = 0; j < GG::CIW; j++) {
            const int u = 64 * (w * GG::CIW + j) + l;
            const int r = u / GG::CH, cp = u % GG::CH;
            const int c = cp ^ swz<GG::CH>(r);
            int ar;
            if (WG) {
                ar = PT.row0 + r < p.M ? PT.row0 + r : PT.row0;
            } else {
                const int s = a_src(PT, r);
                if (cp == 0) {
                    rowtok[ord][r] = s;
                    if (NV) rowmul[NV ? ord : 0][r] = s >= 0 ? p.a_outer[s] * p.b_outer[PT.g] : 0.0f;
                }
                ar = s >= 0 ? s : 0;   // rows outside the tile or with a bad index read row 0, result discarded
            }
            const int n = PT.col0 + r < p.N ? PT.col0 + r : p.N - 1;
            poa[j] = (uint32_t)ar * ldA + 16 * c;
            pob[j] = (uint32_t)n * ldA + 16 * c;
        }
        {
            const int b0 = WG ? PT.kbeg / GG::SBLK : 0;
            if constexpr (NVL) {
                // lane order: tiles of BT rows, each nbp / SPS stages of SPS * BT bytes
                if (scl_b) psbase = p.b_plane + (size_t)PT.g * p.nbp * p.b_rp + (size_t)PT.col0 * p.nbp;
                else psbase = p.a_plane + (size_t)PT.slot * BT * p.nbp;
            } else if constexpr (NVP) {
                // block pairs: b0 is even (groups start on 32-token boundaries)
                if (scl_b) psbase = p.b_plane + (size_t)b0 * p.b_rp + 2 * PT.col0;
                else psbase = p.a_plane + (size_t)b0 * p.a_rp + 2 * PT.row0;
            } else {
                if (scl_b) psbase = p.b_plane + ((size_t)(WG ? 0 : PT.g) * p.nbp + b0) * p.b_rp + PT.col0;
                else psbase = p.a_plane + (size_t)b0 * p.a_rp + (WG ? PT.row0 : PT.slot * BT);
            }
        }
    };

    // BF16 stage fetch: 32 K values from k0.  K values past the tile's K end
    // (chunks of K-major rows, whole K rows of MN-major operands) load zeros.
    auto bf_issue = [&](uint32_t m0) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(PT.kbeg + p_kt * GG::BK);
        const int kend = __builtin_amdgcn_readfirstlane(PT.kend);
        const bool full = k0 + GG::BK <= kend;
        const uint32_t kb = p_kt * GG::ROWB;
        // K-major operand: chunk c of the row holds K values k0 + 8 c.
        auto kmajor = [&](const uint8_t *base, const uint32_t *off, uint32_t dst) __attribute__((always_inline)) {
            if (full) {
#pragma unroll
                for (int j = 0; j < GG::CIW; j++) dma16(base + kb, off[j], dst + (w * GG::CIW + j) * 1024);
            } else {
#pragma unroll
                for (int j = 0; j < GG::CIW; j++) {
                    const int u = 64 * (w * GG::CIW + j) + l;
                    const int c = (u % GG::CH) ^ swz<GG::CH>(u / GG::CH);
                    dma16v(k0 + 8 * c >= kend ? kZeroChunk : base + kb + off[j], dst + (w * GG::CIW + j) * 1024);
                }
            }
        };
        // MN-major operand with consecutive K rows: K row kr of the stage is
        // row (first + kr) of the matrix at `base`.
        auto mnmajor = [&](const uint8_t *base, const uint32_t *off, uint32_t dst) __attribute__((always_inline)) {
            if (full) {
#pragma unroll
                for (int j = 0; j < GG::CIW; j++) dma16(base, off[j], dst + (w * GG::CIW + j) * 1024);
            } else {
#pragma unroll
                for (int j = 0; j < GG::CIW; j++) {
                    const int kr = (64 * (w * GG::CIW + j) + l) / (BT / 8);
                    dma16v(k0 + kr >= kend ? kZeroChunk : base + off[j], dst + (w * GG::CIW + j) * 1024);
                }
            }
        };
        if constexpr (A_MN) mnmajor(uniform_ptr(pca + (size_t)p_kt * GG::BK * ldA), poa, m0);
        else kmajor(pca, poa, m0);
        if constexpr (!B_MN) {
            kmajor(pcb, pob, m0 + GG::CODE);
        } else if constexpr (!WG) {
            mnmajor(uniform_ptr(pcb + (size_t)k0 * ldB), pob, m0 + GG::CODE);
        } else {
            // Weight-gradient form: K row kr is row gather[k0 + kr] of B (or
            // row k0 + kr).  The wavefront's KPW indices come through scalar
            // loads (the pipeline's vector-memory waits count DMA loads only);
            // indices past the K end are clamped to the last row and their
            // chunks load zeros, as do rows with an index outside B.
            typedef const __attribute__((address_space(4))) int32_t cint32;
            const cint32 *gq = (const cint32 *)p.b_gather;
            int32_t tq[GG::KPW];
#pragma unroll
            for (int q = 0; q < GG::KPW; q++) {
                const int kr = k0 + GG::KPW * w + q;
                const int idx = kr < kend ? kr : kend - 1;
                tq[q] = p.b_gather ? gq[idx] : idx;
            }
#pragma unroll
            for (int j = 0; j < GG::CIW; j++) {
                const int sub = l / (BT / 8);
                int32_t tr = tq[j * GG::RPI];
#pragma unroll
                for (int q = 1; q < GG::RPI; q++) tr = sub == q ? tq[j * GG::RPI + q] : tr;
                const int kr = GG::KPW * w + j * GG::RPI + sub;
                const bool ok = k0 + kr < kend && tr >= 0 && tr < p.b_rows;
                dma16v(ok ? pcb + (size_t)tr * ldB + pob[j] : kZeroChunk,
                       m0 + GG::CODE + (w * GG::CIW + j) * 1024);
            }
        }
    };

    // Fetch the producer's next stage into ring stage `slot`.
    auto issue = [&](int slot) __attribute__((always_inline)) {
        // Opaque per call: hoisted out of the loop, the LDS addresses of every
        // ring stage and DMA would each hold a scalar register.
        uint32_t m0 = ring_lds + slot * SLOT_BYTES;
        asm volatile("" : "+s"(m0));
        if constexpr (BF) {
            bf_issue(m0);
            return;
        }
        const int k0 = PT.kbeg + p_kt * GG::BK;
        const uint32_t kb = p_kt * GG::ROWB, so = p_kt * GG::SPS;
        if (k0 + GG::BK <= PT.kend) {
#pragma unroll
            for (int j = 0; j < GG::CIW; j++) dma16(pca + kb, poa[j], m0 + (w * GG::CIW + j) * 1024);
#pragma unroll
            for (int j = 0; j < GG::CIW; j++) dma16(pcb + kb, pob[j], m0 + GG::CODE + (w * GG::CIW + j) * 1024);
        } else {
            // The stage runs past the K end: chunks past it load zeros, and
            // their scales (plane padding, or the next group's columns in
            // the weight-gradient form) are finite, so they add nothing and
            // the consumer needs no special case.
#pragma unroll
            for (int j = 0; j < GG::CIW; j++) {
                const int u = 64 * (w * GG::CIW + j) + l;
                const int c = (u % GG::CH) ^ swz<GG::CH>(u / GG::CH);
                const bool past = k0 + GG::VPC * c >= PT.kend;
                dma16v(past ? kZeroChunk : pca + kb + poa[j], m0 + (w * GG::CIW + j) * 1024);
                dma16v(past ? kZeroChunk : pcb + kb + pob[j], m0 + GG::CODE + (w * GG::CIW + j) * 1024);
            }
        }
        // scale bytes of the stage: SPS plane rows (padded past the K end)
        if (scl_w) {
            const uint8_t *sbase = uniform_ptr(psbase + (size_t)so * (NVL ? BT : scl_b ? p.b_rp : p.a_rp));
            const uint32_t sdst = m0 + (scl_b ? GG::B_SCL : GG::A_SCL) + 64 * GG::SCW * (w % SCH);
            if constexpr (GG::SCW == 4) dma4(sbase, psv, sdst);
            else dma16(sbase, psv, sdst);
        }
    };

    // ---- consumer state ----
    int c_lin = first;
    int c_ord = 0, c_kt = 0;
    bool c_done = first >= last;
    Tile CT;
    v16f acc[TI][2];

    auto cons_begin = [&]() __attribute__((always_inline)) {   // CT is set
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
    };

    // 32-row blocks of this wavefront's half of the consumer's tile that hold
    // rows of the group (uniform).  Small experts leave most of a row tile
    // empty: those blocks skip their MFMAs, fragment reads and epilogue.
    auto live_blocks = [&]() __attribute__((always_inline)) -> int {
        if (WG) return TI;
        const int rem = CT.row_end - CT.row0 - wm * (BT / 2);
        const int nb = (rem + 31) >> 5;
        return rem <= 0 ? 0 : (nb < TI ? nb : TI);
    };

    // Multiply the consumer's current stage, held in ring stage U.
    auto compute = [&](auto U) __attribute__((always_inline)) {
        // Opaque per call for the same reason (LDS offsets of stages 2 and 3
        // do not fit the instruction's immediate field).
        uint32_t soff = decltype(U)::v * SLOT_BYTES;
        asm volatile("" : "+s"(soff));
        const uint8_t *slot = ring + soff;
        const int nv = live_blocks();
        if (nv == 0) return;
        if constexpr (MX) {
            // Per 64-value MFMA K step s: lane half h supplies bytes
            // [16h, 16h + 16) of K block 2s, then of block 2s + 1 (chunks
            // 4s + h and 4s + 2 + h), with block (2s + h)'s E8M0 byte (only
            // the low byte of the scale operand is read).  Block i + 1's A
            // fragment is read before block i's MFMAs are issued (the empty
            // asm keeps the order), so the LDS reads run under the matrix
            // work; blocks past the group's rows skip their MFMAs.
#pragma unroll
          for (int s = 0; s < SUB; s++) {
            uint4 b0[2], b1[2], a0[TI], a1[TI];
            uint32_t bs[2], as[TI];
            const uint32_t sa = fsa + 2 * s * BT, sb = fsb + 2 * s * BT;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                b0[j] = *reinterpret_cast<const uint4 *>(slot + fb0[s] + 32 * GG::ROWB * j);
                b1[j] = *reinterpret_cast<const uint4 *>(slot + fb1[s] + 32 * GG::ROWB * j);
                bs[j] = slot[sb + 32 * j];
            }
            a0[0] = *reinterpret_cast<const uint4 *>(slot + fa0[s]);
            a1[0] = *reinterpret_cast<const uint4 *>(slot + fa1[s]);
            as[0] = slot[sa];
#pragma unroll
            for (int i = 0; i < TI; i++) {
                if (i + 1 < TI) {
                    a0[i + 1] = *reinterpret_cast<const uint4 *>(slot + fa0[s] + 32 * GG::ROWB * (i + 1));
                    a1[i + 1] = *reinterpret_cast<const uint4 *>(slot + fa1[s] + 32 * GG::ROWB * (i + 1));
                    as[i + 1] = slot[sa + 32 * (i + 1)];
                }
                asm volatile("" ::: "memory");
                if (i < nv) {
                    const v8i fa = {(int)a0[i].x, (int)a0[i].y, (int)a0[i].z, (int)a0[i].w,
                                    (int)a1[i].x, (int)a1[i].y, (int)a1[i].z, (int)a1[i].w};
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const v8i fb = {(int)b0[j].x, (int)b0[j].y, (int)b0[j].z, (int)b0[j].w,
                                        (int)b1[j].x, (int)b1[j].y, (int)b1[j].z, (int)b1[j].w};
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[i][j], 0, 0, 0,
                                                                                    (int)as[i], 0, (int)bs[j]);
                    }
                }
            }
          }
        } else if constexpr (BF) {
            // MFMA s covers K values 16 s + 0..15 of the stage, lane half h
            // supplying 16 s + 8 h + 0..7 of its row (A) or column (B):
            // K-major operands read chunk 2 s + h of the row (fa0 / fa1 as
            // for MXFP8), MN-major ones two transposed reads of 4 K rows.
            auto kfrag = [&](uint32_t off) __attribute__((always_inline)) -> v8bf {
                return __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4 *>(slot + off));
            };
            auto mfrag = [&](uint32_t off) __attribute__((always_inline)) -> v8bf {
                typedef __attribute__((address_space(3))) v4s lds_v4s;
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(slot + off));
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(slot + off + 4 * RP));
                return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            };
#pragma unroll
            for (int st = 0; st < GG::BK / 16; st++) {
                // MFMA step st = 2 sub + s2: K-major chunk 4 sub + 2 s2 + h
                const int sub = st >> 1, s2 = st & 1;
                v8bf fa[TI], fb[2];
#pragma unroll
                for (int j = 0; j < 2; j++)
                    fb[j] = B_MN ? mfrag(trb[B_MN ? j : 0] + 16 * st * RP)
                                 : kfrag((s2 ? fb1[sub] : fb0[sub]) + 32 * GG::ROWB * j);
                fa[0] = A_MN ? mfrag(tra[0] + 16 * st * RP) : kfrag(s2 ? fa1[sub] : fa0[sub]);
#pragma unroll
                for (int i = 0; i < TI; i++) {
                    if (i + 1 < TI)
                        fa[i + 1] = A_MN ? mfrag(tra[A_MN ? i + 1 : 0] + 16 * st * RP)
                                         : kfrag((s2 ? fa1[sub] : fa0[sub]) + 32 * GG::ROWB * (i + 1));
                    asm volatile("" ::: "memory");
                    if (i < nv) {
#pragma unroll
                        for (int j = 0; j < 2; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
                    }
                }
            }
        } else {
            // K order inside a 64-value step s of the stage: lane half h,
            // MFMA step q and element e take K = 64 s + 32 h + 8 q + e, the
            // same on both operands, so each lane reads one 16-byte chunk
            // (32 values, scale blocks 4s + 2h and 4s + 2h + 1).
            // Row-grouped forms: the lane's scales of the whole stage in
            // whole chunks (lane-ordered planes): dword s of the chunk of A's
            // window i / 2 (half i & 1) and of B's (half j) holds the E4M3
            // pair of blocks 4s + 2h + e.
            static_assert(!NVL || GG::SPS == 8, "lane-ordered planes hold stages of 8 blocks");
            uint32_t wsa[NVL ? TI : 1], wsb[2];
            if constexpr (NVL) {
#pragma unroll
                for (int ih = 0; ih < TI / 2; ih++) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(slot + fsa + 512 * ih);
                    wsa[2 * ih] = v.x;
                    wsa[2 * ih + 1] = v.y;
                }
                const uint2 v = *reinterpret_cast<const uint2 *>(slot + fsb);
                wsb[0] = v.x; wsb[1] = v.y;
            }
#pragma unroll
          for (int s = 0; s < SUB; s++) {
            uint4 ua[TI], ub[2];
            h2 sa[TI][2], sb[2][2];
            const uint32_t ssa = fsa + 4 * s * BT, ssb = fsb + 4 * s * BT;
#pragma unroll
            for (int i = 0; i < TI; i++) {
                if (i >= nv) break;
                ua[i] = *reinterpret_cast<const uint4 *>(slot + fa0[s] + 32 * GG::ROWB * i);
                if constexpr (NVL) {
                    const uint32_t wv = wsa[2 * (i / 2) + s];
                    const h2 pr = (i & 1) ? e4m3_pair<true>(wv) : e4m3_pair<false>(wv);
                    sa[i][0] = h2{pr.x, pr.x};
                    sa[i][1] = h2{pr.y, pr.y};
                } else if constexpr (NVP) {
                    static_assert(!NVP || SUB == 1, "block-pair planes: one 64-value step per stage");
                    const h2 pr = e4m3_pair<false>(*reinterpret_cast<const uint16_t *>(slot + fsa + 64 * i));
                    sa[i][0] = h2{pr.x, pr.x};
                    sa[i][1] = h2{pr.y, pr.y};
                } else {
                    const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)slot[ssa + 32 * i], 0);
                    const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)slot[ssa + BT + 32 * i], 0);
                    sa[i][0] = h2{s0, s0};
                    sa[i][1] = h2{s1, s1};
                }
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                ub[j] = *reinterpret_cast<const uint4 *>(slot + fb0[s] + 32 * GG::ROWB * j);
                if constexpr (NVL) {
                    const h2 pr = j ? e4m3_pair<true>(wsb[s]) : e4m3_pair<false>(wsb[s]);
                    sb[j][0] = h2{pr.x, pr.x};
                    sb[j][1] = h2{pr.y, pr.y};
                } else if constexpr (NVP) {
                    const h2 pr = e4m3_pair<false>(*reinterpret_cast<const uint16_t *>(slot + fsb + 64 * j));
                    sb[j][0] = h2{pr.x, pr.x};
                    sb[j][1] = h2{pr.y, pr.y};
                } else {
                    const _Float16 t0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)slot[ssb + 32 * j], 0);
                    const _Float16 t1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)slot[ssb + BT + 32 * j], 0);
                    sb[j][0] = h2{t0, t0};
                    sb[j][1] = h2{t1, t1};
                }
            }
            auto word = [](const uint4 &u, int q) __attribute__((always_inline)) -> uint32_t {
                return q == 0 ? u.x : q == 1 ? u.y : q == 2 ? u.z : u.w;
            };
            // B's fragments for step q + 1 are converted during step q and
            // each A fragment right before its two MFMAs, so that the
            // conversions issue between MFMAs and overlap them (a wavefront
            // issuing its MFMAs back to back could not convert meanwhile).
            // Block 0 is always live (nv >= 1 here); blocks past the group's
            // rows skip their conversions and MFMAs.
            v8h fb[2][2];
#pragma unroll
            for (int j = 0; j < 2; j++) fb[0][j] = nv_frag(word(ub[j], 0), sb[j][0]);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int c = q & 1;
                if (q < 3) {
#pragma unroll
                    for (int j = 0; j < 2; j++) fb[c ^ 1][j] = nv_frag(word(ub[j], q + 1), sb[j][(q + 1) >> 1]);
                }
#pragma unroll
                for (int i = 0; i < TI; i++) {
                    if (i > 0 && i >= nv) break;
                    const v8h fa = nv_frag(word(ua[i], q), sa[i][q >> 1]);
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb[c][j], acc[i][j], 0, 0, 0);
                }
                // request the interleave from the scheduler as well
#pragma unroll
                for (int m = 0; m < 2 * TI; m++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
                }
            }
          }
        }
    };

    // Write the consumer's tile.  The MFMA leaves lane l with column l % 32
    // of each 32 x 32 block and rows 8 (e / 4) + 4 (l / 32) + e % 4; the
    // transpose goes through an LDS patch in a ring stage no load targets.
    auto epilogue = [&](uint8_t *slot) __attribute__((always_inline)) {
        // Each wavefront stages a 32-row slice of its outputs in its own LDS
        // patch and writes it back in whole 128-byte row pieces: 32 x 64
        // columns for bf16 (both column blocks at once), 32 x 32 for f32.
        constexpr int ESZ = BF16OUT ? 2 : 4;
        constexpr int VEC = 16 / ESZ;                  // elements per 16-byte store
        constexpr int NJ = BF16OUT ? 2 : 1;            // column blocks per staged slice
        constexpr int RB = 32 * NJ * ESZ;              // bytes of a staged row piece (128)
        constexpr int STR = RB + 16;                   // padded LDS row stride
        constexpr int CPR = RB / 16;                   // 16-byte chunks per row piece
        uint8_t *ep = slot + w * (32 * STR);
        const int ord = c_ord & 7;
        const bool vec_ok = (p.ldc % VEC) == 0;
        const int64_t goff = WG ? (int64_t)CT.g * p.M * p.ldc : 0;
        // NVFP4 weight gradient: the group's outer scales of both operands
        const float gab = (WG && NV) ? sload(p.a_outer, CT.g) * sload(p.b_outer, CT.g) : 1.0f;
        const int nv = live_blocks();
        const int ncol = p.N;
#pragma unroll
        for (int i = 0; i < TI; i++) {
            if (i >= nv) break;
            float mul[16];
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int rt = wm * (BT / 2) + 32 * i + 8 * (e >> 2) + 4 * lh + (e & 3);
                if (WG) mul[e] = gab;
                else if (!NV) mul[e] = rowtok[ord][rt] >= 0 ? 1.0f : 0.0f;
                else mul[e] = rowmul[NV ? ord : 0][rt];
            }
#pragma unroll
            for (int j0 = 0; j0 < 2; j0 += NJ) {
                {
#pragma unroll
                    for (int jj = 0; jj < NJ; jj++) {
                        const int j = j0 + jj;
#pragma unroll
                        for (int e = 0; e < 16; e += 2) {
                            const int rin = 8 * (e >> 2) + 4 * lh + (e & 3);   // rows rin, rin + 1
                            const float v0 = mul[e] == 0.0f ? 0.0f : acc[i][j][e] * mul[e];
                            const float v1 = mul[e + 1] == 0.0f ? 0.0f : acc[i][j][e + 1] * mul[e + 1];
                            if (BF16OUT) {
                                // V_CVT_PK_BF16_F32: round to nearest even, like f32_to_bf16
                                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                                typedef float f2 __attribute__((ext_vector_type(2)));
                                const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v0, v1}, bf2));
                                *reinterpret_cast<uint16_t *>(ep + rin * STR + (32 * jj + lr) * 2) = (uint16_t)pk;
                                *reinterpret_cast<uint16_t *>(ep + (rin + 1) * STR + (32 * jj + lr) * 2) =
                                    (uint16_t)(pk >> 16);
                            } else {
                                *reinterpret_cast<float *>(ep + rin * STR + lr * 4) = v0;
                                *reinterpret_cast<float *>(ep + (rin + 1) * STR + lr * 4) = v1;
                            }
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();   // the patch is private to this wavefront
#pragma unroll
                for (int pass = 0; pass < 32 * CPR / 64; pass++) {
                    const int idx = pass * 64 + l;
                    const int rin = idx / CPR, ch = idx % CPR;
                    const int r = CT.row0 + wm * (BT / 2) + 32 * i + rin;
                    const int cn = CT.col0 + wn * 64 + 32 * j0 + ch * VEC;
                    const uint4 v = *reinterpret_cast<const uint4 *>(ep + rin * STR + ch * 16);
                    if (r < CT.row_end && cn < ncol) {
                        char *dst = reinterpret_cast<char *>(p.c) + (goff + (int64_t)r * p.ldc + cn) * ESZ;
                        if (vec_ok && cn + VEC <= ncol) {
                            st_nt16(dst, u32x4{v.x, v.y, v.z, v.w});
                        } else {
#pragma unroll
                            for (int q = 0; q < VEC; q++) {
                                const int d = BF16OUT ? q >> 1 : q;
                                const uint32_t wq = d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
                                if (cn + q < ncol) {
                                    if (BF16OUT) st_b16(dst + 2 * q, wq >> (16 * (q & 1)));
                                    else st_b32(dst + 4 * q, wq);
                                }
                            }
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
    };

    // Advance the consumer to its next tile.
    auto cons_next = [&]() __attribute__((always_inline)) {
        c_lin = next_tile(c_lin);
        c_ord++;
        if (c_lin >= last) {
            c_done = true;
            return;
        }
        CT = decode_tile<FMT, MODE, BT>(p, c_lin);
        c_kt = 0;
        cons_begin();
    };

    // ---- prologue: first tiles, first NS - 1 stages ----
    int p_q = 0, c_q = 0;   // stages issued / consumed
    prod_seek();
    waitcnt<63, 0>();
    barrier();   // row table of the first tile is visible
    if (!c_done) {
        CT = decode_tile<FMT, MODE, BT>(p, c_lin);
        cons_begin();
    }
    for (int s = 0; s < NS - 1 && !p_done; s++) {
        issue(s);
        p_q++;
        if (++p_kt == p_nk) {
            p_lin = next_tile(p_lin);
            p_ord++;
            prod_seek();
        }
    }

    // One pipeline step: the consumer's stage q sits in ring stage U = q % NS
    // and the producer refills ring stage (U + NS - 1) % NS, which held stage
    // q - 1, so NS - 1 stages stay in flight.
    auto step = [&](auto U) __attribute__((always_inline)) -> int {
        wait_stage_w<GG::OPS>(p_q - c_q - 1, scl_w);
        barrier();   // stage q landed for every wavefront; the ring stage of q - 1 is free
        int fl = 0;
        if (!p_done) {
            issue((decltype(U)::v + NS - 1) % NS);
            p_q++;
            if (++p_kt == p_nk) fl |= SEEK;
        }
        compute(U);
        c_q++;
        if (++c_kt == CT.nk) fl |= FIN;
        return fl;
    };

    // ---- main loop ----
    // Ring stages are compile-time constants inside the unrolled steps; the
    // walk leaves the unrolled sequence when the producer needs its next tile
    // or the consumer finished one, and re-enters at the stage it stopped.
    // A finished tile is written through the LDS of the stage just consumed;
    // tiles without K work (weight-gradient form only) use the ring stage that
    // precedes the next stage to consume, which no load targets at that point.
    while (!c_done) {
        int fl = 0;
        if (WG && CT.nk == 0) {
            fl = FIN;
        } else {
            const int u0 = c_q % NS;
            if constexpr (NS == 4) {
                if (u0 == 0) fl = step(IC<0>{});
                if (!fl && u0 <= 1) fl = step(IC<1>{});
                if (!fl && u0 <= 2) fl = step(IC<2>{});
                if (!fl) fl = step(IC<3>{});
            } else {
                if (u0 == 0) fl = step(IC<0>{});
                if (!fl) fl = step(IC<1>{});
            }
        }
        if (fl & SEEK) {
            p_lin = next_tile(p_lin);
            p_ord++;
            prod_seek();
        }
        if (fl & FIN) {
            waitcnt<63, 0>();
            barrier();   // every wavefront is done reading the stage
            epilogue(ring + ((c_q + NS - 1) % NS) * SLOT_BYTES);
            cons_next();
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
int64_t gemm_tile_count(int64_t M, int64_t G) { return (M + 127) / 128 + G; }

// Workspace: tile list (or padded group starts) and counters, then the A
// and B scale planes, each 256-byte aligned.
struct WsLayout {
    int64_t head, a_off, b_off, total;
    int32_t nbp, a_rp, b_rp;
};
static int64_t up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
static WsLayout ws_layout(int fmt, int mode, int64_t M, int64_t N, int64_t K, int64_t G) {
    WsLayout L;
    // scale blocks per stage, as the kernel's geometry stages them
    const int64_t sblk = fmt == BSP_FMT_MXFP8 ? 32 : 16;
    const bool wg = mode == BSP_GEMM_WGRAD;
    const int64_t sps = fmt == BSP_FMT_MXFP8
                            ? (wg ? GeoOf<BSP_FMT_MXFP8, BSP_GEMM_WGRAD, 256>::SPS
                                  : GeoOf<BSP_FMT_MXFP8, BSP_GEMM_FPROP, 256>::SPS)
                            : (wg ? GeoOf<BSP_FMT_NVFP4, BSP_GEMM_WGRAD, 256>::SPS
                                  : GeoOf<BSP_FMT_NVFP4, BSP_GEMM_FPROP, 256>::SPS);
    const int64_t nblk = K / sblk;
    L.nbp = (int32_t)(up(nblk, sps) + sps);   // K-tail stages read one padded step past the end
    const int64_t entries = (mode == BSP_GEMM_WGRAD ? G + 1 : gemm_tile_count(M, G)) + kGemmSchedSlots;
    // weight-gradient form: then the expert order, int32 [G]
    L.head = up(entries * 8 + (mode == BSP_GEMM_WGRAD ? G * 4 : 0), 256);
    L.a_rp = (int32_t)(mode == BSP_GEMM_WGRAD ? up(M, 256) : ((M + 255) / 256 + G) * 256);
    L.b_rp = (int32_t)up(N, 256);
    L.a_off = L.head;
    L.b_off = L.a_off + up((int64_t)L.nbp * L.a_rp, 256);
    L.total = L.b_off + up((mode == BSP_GEMM_WGRAD ? 1 : G) * (int64_t)L.nbp * L.b_rp, 256);
    return L;
}
int64_t gemm_workspace_bytes(int fmt, int mode, int64_t M, int64_t N, int64_t K, int64_t G) {
    return ws_layout(fmt, mode, M, N, K, G).total;
}

// Workgroups resident per XCD for one instantiation on the current device
// (compute units per XCD times workgroups per compute unit).  The value is a
// property of the device and the compiled kernel, so it is computed on first
// use per device and kept: every caller computes the same number, and the
// atomic store makes concurrent first calls harmless.
template <typename Kern>
static int64_t resident_per_xcd(Kern kern, int threads, std::atomic<int> *cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess || occ <= 0) occ = 1;
        v = (cus + NXCD - 1) / NXCD * occ;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int FMT, int MODE, bool BF, int BT>
static void launch_one(const GemmArgs &p, hipStream_t s) {
    static std::atomic<int> cache[kMaxDevices];
    const int64_t per_xcd_max = resident_per_xcd(k_gemm<FMT, MODE, BF, BT>, 2 * BT, cache);
    const int64_t total = (int64_t)p.ntm * p.ntn;   // upper bound of the tile count
    const int64_t per_xcd_need = (total + NXCD - 1) / NXCD;
    const int64_t per_xcd = per_xcd_need < per_xcd_max ? per_xcd_need : per_xcd_max;
    dim3 grid((unsigned)(per_xcd * NXCD)), block(2 * BT);
    k_gemm<FMT, MODE, BF, BT><<<grid, block, 0, s>>>(p);
}

template <int FMT, int MODE, int BT>
static void launch_k(const GemmArgs &p, bool bf, hipStream_t s) {
    if (bf) launch_one<FMT, MODE, true, BT>(p, s);
    else launch_one<FMT, MODE, false, BT>(p, s);
}

// Tile edge: 256 (eight wavefronts, half the operand traffic per output of a
// 128 tile) once there are enough tiles to occupy every compute unit twice
// over, else 128; `forced` (128 or 256, from the caller) pins the choice.
static int pick_tile(int64_t tiles256, int forced) {
    if (forced == 128 || forced == 256) return forced;
    return tiles256 >= 512 ? 256 : 128;
}

hipError_t launch_gemm(int fmt, int mode, const uint8_t *a_codes, const uint8_t *a_scales, const float *a_outer,
                       const int32_t *a_gather, int64_t a_rows, const int64_t *group_offsets, int64_t G,
                       int64_t M, int64_t N, int64_t K, const uint8_t *b_codes, const uint8_t *b_scales,
                       const float *b_outer, void *c, int c_dtype, int64_t ldc, void *workspace, int tile,
                       hipStream_t s) {
    const WsLayout L = ws_layout(fmt, mode, M, N, K, G);
    GemmArgs p = {};
    p.a_codes = a_codes; p.a_scales = a_scales; p.a_outer = a_outer; p.a_gather = a_gather;
    p.group_offsets = group_offsets; p.b_codes = b_codes; p.b_scales = b_scales; p.b_outer = b_outer;
    p.c = c; p.G = (int32_t)G; p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K; p.ldc = (int32_t)ldc;
    p.a_rows = (int32_t)a_rows;
    uint8_t *wsb = reinterpret_cast<uint8_t *>(workspace);
    int64_t *ws = reinterpret_cast<int64_t *>(workspace);
    p.tiles = ws;
    // The listed tile count follows the tile list (or the padded starts).
    p.sched = ws + (mode == BSP_GEMM_WGRAD ? G + 1 : gemm_tile_count(M, G));
    p.a_plane = wsb + L.a_off;
    p.b_plane = wsb + L.b_off;
    p.a_rp = L.a_rp; p.b_rp = L.b_rp; p.nbp = L.nbp;
    const bool bf = c_dtype == BSP_DTYPE_BF16;
    const int32_t sr = (int32_t)(K / (fmt == BSP_FMT_MXFP8 ? 32 : 16));
    const unsigned gy = (unsigned)((L.nbp + 63) / 64);

    PlaneArgs pb = {};
    pb.src = b_scales; pb.sr = sr; pb.plane = wsb + L.b_off; pb.nbp = L.nbp; pb.rp = L.b_rp; pb.rows_z = (int32_t)N;
    if (mode == BSP_GEMM_WGRAD) {
        const int bt = pick_tile(G * ((M + 255) / 256) * ((N + 255) / 256), tile);
        p.ntn = (int32_t)((N + bt - 1) / bt);
        p.ntm = (int32_t)(G * ((M + bt - 1) / bt));
        k_padded_starts<<<1, 256, 0, s>>>(group_offsets, G, ws, p.sched);
        int32_t *order = reinterpret_cast<int32_t *>(ws + G + 1 + kGemmSchedSlots);
        k_wgrad_order<<<1, 1024, 0, s>>>(group_offsets, G, order);
        p.order = order;
        PlaneArgs pa = {};
        pa.src = a_scales; pa.sr = sr; pa.plane = wsb + L.a_off; pa.nbp = L.nbp; pa.rp = L.a_rp;
        pa.rows_z = (int32_t)M;
        if (fmt == BSP_FMT_NVFP4) {
            pa.lane = 2;
            pb.lane = 2;
        }
        k_scale_plane<false><<<dim3((unsigned)(L.a_rp / 64), gy, 1), 256, 0, s>>>(pa);
        k_scale_plane<false><<<dim3((unsigned)(L.b_rp / 64), gy, 1), 256, 0, s>>>(pb);
        if (fmt == BSP_FMT_MXFP8) {
            if (bt == 256) launch_k<BSP_FMT_MXFP8, BSP_GEMM_WGRAD, 256>(p, bf, s);
            else launch_k<BSP_FMT_MXFP8, BSP_GEMM_WGRAD, 128>(p, bf, s);
        } else {
            if (bt == 256) launch_k<BSP_FMT_NVFP4, BSP_GEMM_WGRAD, 256>(p, bf, s);
            else launch_k<BSP_FMT_NVFP4, BSP_GEMM_WGRAD, 128>(p, bf, s);
        }
        return hipGetLastError();
    }
    const int bt = pick_tile(((M + 255) / 256 + G / 2) * ((N + 255) / 256), tile);
    p.ntn = (int32_t)((N + bt - 1) / bt);
    p.ntm = (int32_t)((M + bt - 1) / bt + G);   // upper bound of the row-tile count
    k_tile_list<<<1, 256, 0, s>>>(group_offsets, G, M, bt == 256 ? 8 : 7, p.ntm, ws, p.sched);
    PlaneArgs pa = {};
    pa.src = a_scales; pa.sr = sr; pa.plane = wsb + L.a_off; pa.nbp = L.nbp; pa.rp = L.a_rp;
    pa.tiles = ws; pa.sched = p.sched + NXCD; pa.off = group_offsets; pa.gather = a_gather;
    pa.bt = bt; pa.M = (int32_t)M; pa.a_rows = (int32_t)a_rows;
    if (fmt == BSP_FMT_NVFP4) {
        pa.lane = 1;
        pb.lane = 1;
        pb.bt = bt;
    }
    k_scale_plane<true><<<dim3((unsigned)((int64_t)p.ntm * bt / 64), gy, 1), 256, 0, s>>>(pa);
    k_scale_plane<false><<<dim3((unsigned)(L.b_rp / 64), gy, (unsigned)G), 256, 0, s>>>(pb);
    if (bt == 256) {
        if (fmt == BSP_FMT_MXFP8) launch_k<BSP_FMT_MXFP8, BSP_GEMM_FPROP, 256>(p, bf, s);
        else launch_k<BSP_FMT_NVFP4, BSP_GEMM_FPROP, 256>(p, bf, s);
    } else {
        if (fmt == BSP_FMT_MXFP8) launch_k<BSP_FMT_MXFP8, BSP_GEMM_FPROP, 128>(p, bf, s);
        else launch_k<BSP_FMT_NVFP4, BSP_GEMM_FPROP, 128>(p, bf, s);
    }
    return hipGetLastError();
}

// Device scratch of the allocation-free GEMM entry point: the workspace
// (tile list, counters, scale planes) of one call lives in this array instead
// of caller memory.  Each device holds its own copy, at its own address, for
// the life of the process; every call on a device rewrites the parts it reads
// (the setup kernels clear the counters), so nothing carries over between
// calls, and calls that overlap on one device race on it.
static __device__ __align__(256) uint8_t scratch[BSP_GEMM_SCRATCH_BYTES];

// Device address of `scratch` on the current device.  The host-side name is
// only a stand-in for the symbol, so the address is looked up once per device
// (with that device current) and kept; nullptr when the lookup fails.
void *gemm_scratch() {
    static std::atomic<void *> addr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        addr[dev].store(p, std::memory_order_release);
    }
    return p;
}

// BF16 grouped GEMM.  Workspace: the row-tile list and counters of the
// row-grouped forms; the expert order of the weight-gradient form.
int64_t gemm_bf16_workspace_bytes(int mode, int64_t M, int64_t G) {
    if (mode == BSP_GEMM_WGRAD) return up(G * 4, 256);
    return up((gemm_tile_count(M, G) + kGemmSchedSlots) * 8, 256);
}

hipError_t launch_gemm_bf16(int mode, const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb,
                            const int32_t *gather, int64_t src_rows, const int64_t *group_offsets, int64_t G,
                            int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc, void *workspace,
                            int tile, hipStream_t s) {
    GemmArgs p = {};
    const bool wg = mode == BSP_GEMM_WGRAD;
    p.a_codes = reinterpret_cast<const uint8_t *>(a);
    p.b_codes = reinterpret_cast<const uint8_t *>(b);
    p.group_offsets = group_offsets;
    p.a_gather = wg ? nullptr : gather;
    p.b_gather = wg ? gather : nullptr;
    p.a_rows = (int32_t)(wg ? K : src_rows);
    p.b_rows = (int32_t)(wg ? src_rows : 0);
    p.lda_b = (int32_t)(2 * lda);
    p.ldb_b = (int32_t)(2 * ldb);
    p.c = c; p.G = (int32_t)G; p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K; p.ldc = (int32_t)ldc;
    const bool bf = c_dtype == BSP_DTYPE_BF16;
    if (wg) {
        const int bt = pick_tile(G * ((M + 255) / 256) * ((N + 255) / 256), tile);
        p.ntn = (int32_t)((N + bt - 1) / bt);
        p.ntm = (int32_t)(G * ((M + bt - 1) / bt));
        int32_t *order = reinterpret_cast<int32_t *>(workspace);
        k_wgrad_order<<<1, 1024, 0, s>>>(group_offsets, G, order);
        p.order = order;
        if (bt == 256) launch_k<FMT_BF16, BSP_GEMM_WGRAD, 256>(p, bf, s);
        else launch_k<FMT_BF16, BSP_GEMM_WGRAD, 128>(p, bf, s);
        return hipGetLastError();
    }
    int64_t *ws = reinterpret_cast<int64_t *>(workspace);
    const int bt = pick_tile(((M + 255) / 256 + G / 2) * ((N + 255) / 256), tile);
    p.ntn = (int32_t)((N + bt - 1) / bt);
    p.ntm = (int32_t)((M + bt - 1) / bt + G);   // upper bound of the row-tile count
    p.tiles = ws;
    p.sched = ws + gemm_tile_count(M, G);
    k_tile_list<<<1, 256, 0, s>>>(group_offsets, G, M, bt == 256 ? 8 : 7, p.ntm, ws, p.sched);
    if (mode == BSP_GEMM_DGRAD) {
        if (bt == 256) launch_k<FMT_BF16, BSP_GEMM_DGRAD, 256>(p, bf, s);
        else launch_k<FMT_BF16, BSP_GEMM_DGRAD, 128>(p, bf, s);
    } else {
        if (bt == 256) launch_k<FMT_BF16, BSP_GEMM_FPROP, 256>(p, bf, s);
        else launch_k<FMT_BF16, BSP_GEMM_FPROP, 128>(p, bf, s);
    }
    return hipGetLastError();
}

}  // namespace bsp

// bf16 MFMA GEMMs of the projections around the decode:
//   q_lat[t][h][:] = q_nope[t][h][:] . W_UK[h]^T          huny.dev "DeepSeek MLA 해부" §3-1
//   u[t][h][:]     = o_lat[t][h][:] . W_UV[h]             §3-2 value equation
//   out[t][:]      = u[t][:] . W_O   (all heads at once)  §3-2 output equation
// and the weight products of the producers (h W^DKV, h W^DQ, h W^QR,
// c^Q W^UQ).  One kernel, C[z][m][n] = sum_k A[z][m][k] B[z](k, n) with fp32
// accumulation: A is always k-contiguous (activations); B is k-contiguous
// (W_UK[h] = B^T) or n-contiguous (the other weights).  At decode the token
// count T is small, so these products stream their weights: the kernel is
// built to keep HBM busy (direct-to-LDS copies, four stage buffers, two
// waves per SIMD) rather than to maximise MFMA reuse.
//
// Workgroup: a TM x 128 tile of C (TM = 128, or 64 when 128-row tiles would
// leave most CUs idle), K in 64-wide stages; 8 waves as 2 x 4 sub-tiles of
// TM/2 x 32 (4 waves as 2 x 2 of 64 x 64 for the short-K absorption), each
// sub-tile as 32 x 32 v_mfma_f32_32x32x16_bf16 blocks.  LDS tiles are filled
// by 1 KiB global_load_lds_dwordx4 copies whose lanes fetch XOR-swizzled
// 16-byte chunks, so that the fragment reads are free of bank conflicts:
//   k-contiguous tile [rows][64 k], 128 B rows: chunk c of row r at
//     position c ^ ((r >> 1) & 7)  (16 rows reading one chunk hit 16 bank groups);
//   n-contiguous tile [64 k][128 n], 256 B rows: chunk c of row k at
//     c ^ (4 (k & 3))  (a transposed read covers 4 rows x 64 B: all 64 banks).
// The n-contiguous B operand is read with ds_read_b64_tr_b16 (lane i of each
// 16-lane group receives element i % 4 of the 8 bytes read by lane 4s + i/4).
// Long K with few tiles is split over workgroups into fp32 partials that a
// small kernel sums (and, for the producers, rotates and stores); two
// products with one A share a launch.
#include "common.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int TILE_A = BM * BK * 2;          // 16 KiB
constexpr int TILE_B = BN * BK * 2;          // 16 KiB
constexpr int STAGE = TILE_A + TILE_B;       // 32 KiB
constexpr int C_PITCH = BN + 8;              // output staging pitch (elements)
// Stage buffers: NST_STREAM for products that stream a weight over a long K
// (copies run NST - 1 stages ahead: with one workgroup per CU, the bytes in
// flight per CU set the achievable HBM rate), NST_SHORT for K of at most two
// stages (64 KiB of LDS, two workgroups per CU).
constexpr int NST_STREAM = 4, NST_SHORT = 2;
constexpr int WV_STREAM = 8;   // waves of the streaming products
static_assert(NST_STREAM * STAGE <= 160 * 1024, "stage buffers exceed LDS");

struct GemmArgs {
    const uint16_t *A;   // A[z][m][k] = A + b * bsa + m * lda + k
    int64_t lda, bsa;
    const uint16_t *B;   // k-contiguous: B + b * bsb + n * ldb + k; else B + b * bsb + k * ldb + n
    int64_t ldb, bsb;
    void *C;             // C + b * bsc + s * css + m * ldc + n (bf16 or fp32 elements)
    int64_t ldc, bsc, css;
    int32_t M, N, K;     // K a multiple of 64; N a multiple of 8
    int32_t splits;      // z = b * splits + s; split s covers the 64-wide stages
                         // [s nk / splits, (s + 1) nk / splits) of the nk = K / 64
    int32_t ntiles;      // column tiles per workgroup, in turn (x * ntiles + j)
    // the fused absorption (gemm_bf16_kernel<..., ABS>): tile n0 of C is
    // head h = n0 / 128's q^C; W2 = W^UK [heads][N2 = 512][128], C2 = q~
    // [M][heads][N2]
    const uint16_t *W2;
    void *C2;
    int32_t N2, H2;
};

// One launch over the workgroups of up to two products of the same kind
// (one 1-D grid: units [0, units0) are product 0's, the rest product 1's).
// Workgroup u of a product takes column-tile group x, row tile y and batch /
// split z with u = x + tx (y + ty z), or with z_first u = x + tx (z + nz y)
// (nz = batch x splits): then the row tiles of one batch entry lie tx nz
// apart in the grid, on one XCD when that is a multiple of 8.
struct GemmPair {
    GemmArgs p0, p1;
    int32_t units0;
    int32_t tx0, ty0, tx1, ty1;
    int32_t z_first, nz;   // product 0 only (single-product launches)
};

__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, const void *src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(src)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N): at most N of this wave's copies may still be in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// wait for the oldest stage in flight while the y youngest (y <= MAXY) may
// still be copying, PER copies per stage
template <int MAXY, int PER>
__device__ __forceinline__ void wait_stage(int younger) {
    if constexpr (MAXY >= 3) { if (younger >= 3) { wait_vm<3 * PER>(); return; } }
    if constexpr (MAXY >= 2) { if (younger == 2) { wait_vm<2 * PER>(); return; } }
    if constexpr (MAXY >= 1) { if (younger == 1) { wait_vm<PER>(); return; } }
    wait_vm<0>();
}

// WV waves: 4 (2 x 2 waves of 64 x 64) or 8 (2 x 4 waves of TM/2 x 32, two
// waves per SIMD so that one wave's LDS reads overlap the other's MFMAs);
// TM rows per tile: 128, or 64 to give a product with few column tiles
// twice the workgroups (its weight tile is then read by two workgroups,
// which the dispatch order puts on one XCD).
// ABS: instead of storing C, a 64-row tile of q^C_h (its 128 columns are
// head h's) stays on chip as bf16 and is multiplied by W^UK_h^T (the
// absorbed query, huny.dev "DeepSeek MLA 해부" §3-1): the eight 16 KiB tiles
// of W^UK_h (128 columns of q~ x 64 k) are copied into the freed stage
// buffers after the q^C loop, and q~ is stored from the accumulators.
// (Copying half of them before the loop, past the stage buffers, measured
// no faster.)
constexpr int ABS_A2 = 8 * TILE_B;                      // q^C tile (16 KiB) after the W^UK_h tiles
constexpr int ABS_LDS = ABS_A2 + 2 * 64 * BK * 2;       // 144 KiB

template <bool B_KCONTIG, bool OUT_F32, int NST, int WV, int TM, bool ABS = false>
__global__ __launch_bounds__(64 * WV, NST <= NST_SHORT ? 2 : 1) void gemm_bf16_kernel(GemmPair G) {
    static_assert(!ABS || (!B_KCONTIG && !OUT_F32 && TM == 64 && WV == 8), "the fused absorption's shape");
    static_assert(!(OUT_F32 && NST <= NST_SHORT), "fp32 output staging needs the streaming stage buffers");
    static_assert(WV == 4 || WV == 8, "4 or 8 waves");
    static_assert(TM == 128 || (TM == 64 && WV == 8), "64-row tiles take 8 waves");
    static_assert(NST - 1 <= 4, "deeper pipelines need more wait cases");
    constexpr int AHEAD = NST - 1;          // stages copied ahead of the one computed
    constexpr int NT = 64 * WV;             // threads
    constexpr int TA = TM * BK * 2;         // A tile bytes
    constexpr int STG = TA + TILE_B;        // stage bytes
    constexpr int RA = TM / WV;             // A rows copied per wave
    constexpr int RB = BN / WV;             // k-contiguous B rows copied per wave
    constexpr int KB = BK / WV;             // n-contiguous B k rows copied per wave
    constexpr int CPA = RA / 8;             // 1 KiB copies of A per wave and stage
    constexpr int CPB = 16 / WV;            // 1 KiB copies of B per wave and stage
    constexpr int PER = CPA + CPB;          // copies per wave and stage
    constexpr int WNW = WV / 2;             // waves across n
    constexpr int TWN = BN / WNW;           // n width of a wave's sub-tile (64 or 32)
    constexpr int NJ = TWN / 32;            // 32-wide n blocks per wave
    constexpr int TWM = TM / 2;             // m height of a wave's sub-tile (64 or 32)
    constexpr int MI = TWM / 32;            // 32-row m blocks per wave
    static_assert(TM * C_PITCH * (OUT_F32 ? 4 : 2) <= NST * STG, "output staging exceeds the stage buffers");
    constexpr int LDS_BYTES = ABS && ABS_LDS > NST * STG ? ABS_LDS : NST * STG;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t smem_[LDS_BYTES];
    lds_u8 *smem = (lds_u8 *)smem_;
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool second = (int)blockIdx.x >= G.units0;
    const GemmArgs g = second ? G.p1 : G.p0;
    const int u = (int)blockIdx.x - (second ? G.units0 : 0);
    const int tx = second ? G.tx1 : G.tx0, ty = second ? G.ty1 : G.ty0;
    const int ux = u % tx;
    const int uy = G.z_first ? u / (tx * G.nz) : (u / tx) % ty;
    const int z = G.z_first ? (u / tx) % G.nz : u / (tx * ty), b = z / g.splits, s = z % g.splits;
    const int m0 = uy * TM;
    for (int tj = 0; tj < g.ntiles; ++tj) {
    const int n0 = (ux * g.ntiles + tj) * BN;
    if (n0 >= g.N) break;
    if (tj > 0) __syncthreads();   // the previous tile's epilogue is done with the LDS
    const int nk_all = g.K / BK;
    const int st0 = (int)((int64_t)s * nk_all / g.splits), nk = (int)((int64_t)(s + 1) * nk_all / g.splits) - st0;
    const int64_t k_begin = (int64_t)st0 * BK;

    // ---- copy offsets (bytes, relative to a per-stage scalar base)
    const uint16_t *a_base = g.A + (int64_t)b * g.bsa + (int64_t)m0 * g.lda + k_begin;
    const uint16_t *b_base = B_KCONTIG ? g.B + (int64_t)b * g.bsb + (int64_t)n0 * g.ldb + k_begin
                                       : g.B + (int64_t)b * g.bsb + k_begin * g.ldb + n0;
    uint32_t a_off[CPA], b_off[CPB];
#pragma unroll
    for (int d = 0; d < CPA; ++d) {
        // A: wave w copies tile rows RA w + 8d .. +7 (lane i: row + i/8, position i%8);
        // rows past M read row M-1 (their results are never stored)
        const int row = RA * wave + 8 * d + (lane >> 3), pos = lane & 7;
        const int mrow = min(m0 + row, g.M - 1) - m0;
        a_off[d] = (uint32_t)(((int64_t)mrow * g.lda + ((pos ^ ((row >> 1) & 7)) << 3)) * 2);
    }
#pragma unroll
    for (int d = 0; d < CPB; ++d) {
        if (B_KCONTIG) {
            // B: wave w copies tile rows RB w + 8d .. +7 as A;
            // columns past N read column N-1 (never stored)
            const int row = RB * wave + 8 * d + (lane >> 3), pos = lane & 7;
            const int nrow = min(n0 + row, g.N - 1) - n0;
            b_off[d] = (uint32_t)(((int64_t)nrow * g.ldb + ((pos ^ ((row >> 1) & 7)) << 3)) * 2);
        } else {
            // B: wave w copies k rows KB w + 4d .. +3 (lane i: row + i/16, position i%16);
            // 8-column chunks past N read the last chunk (never stored)
            const int krow = KB * wave + 4 * d + (lane >> 4), p16 = lane & 15;
            const int col = min(8 * (p16 ^ (4 * (krow & 3))), g.N - 8 - n0);
            b_off[d] = (uint32_t)(((int64_t)krow * g.ldb + col) * 2);
        }
    }
    auto issue = [&](int st) {
        const uint32_t lds = smem_addr + (st % NST) * STG;
        const uint16_t *as = a_base + (int64_t)st * BK;
        const uint16_t *bs = B_KCONTIG ? b_base + (int64_t)st * BK : b_base + (int64_t)st * BK * g.ldb;
#pragma unroll
        for (int d = 0; d < CPA; ++d) dma16(lds + (RA * wave + 8 * d) * (BK * 2), a_off[d], as);
#pragma unroll
        for (int d = 0; d < CPB; ++d) {
            const uint32_t row0 = B_KCONTIG ? (RB * wave + 8 * d) * (BK * 2) : (KB * wave + 4 * d) * (BN * 2);
            dma16(lds + TA + row0, b_off[d], bs);
        }
    };

    // ---- fragment read bases (bytes within a stage)
    const int wm = wave & 1, wn = wave >> 1;
    const int g32 = lane >> 5, l32 = lane & 31;
    uint32_t a_rd[MI];   // A rows TWM wm + 32 i + l32, chunk 2 ks + g32 -> a_rd[i] ^ (32 ks)
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int m = TWM * wm + 32 * i + l32;
        a_rd[i] = m * (BK * 2) + ((g32 ^ ((m >> 1) & 7)) << 4);
    }
    uint32_t b_rd[NJ];
    const int G = lane >> 4, w16 = lane & 15, q = w16 >> 2;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (B_KCONTIG) {
            const int n = TWN * wn + 32 * j + l32;
            b_rd[j] = TA + n * (BK * 2) + ((g32 ^ ((n >> 1) & 7)) << 4);
        } else {
            // k row 16 ks + 8 g + 4 hi + q (+16 ks * 256 B and 4 hi * 256 B as offsets);
            // n bytes 2 (TWN wn + 32 j) + 32 (G & 1) + 8 (w16 & 3): chunk TWN/8 wn + 4 j
            // + 2 (G & 1) + ((w16 & 3) >> 1) XORed with 4 q (k & 3 = q), byte 8 (w16 & 1)
            const int chunk = (TWN / 8) * wn + 4 * j + 2 * (G & 1) + ((w16 & 3) >> 1);
            b_rd[j] = TA + (8 * g32 + q) * (BN * 2) + ((chunk ^ (4 * q)) << 4) + 8 * (w16 & 1);
        }
    }

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

    // a K range that fits the stage buffers is copied at once; a longer one
    // AHEAD stages ahead, stage st + AHEAD into the buffer of stage st - 1
    const int pre = nk <= NST ? nk : AHEAD;
    for (int st = 0; st < pre; ++st) issue(st);
    for (int st = 0; st < nk; ++st) {
        // stage st landed for this wave (the later stages issued may be in flight)
        const int issued = max(pre, min(nk, st + AHEAD));
        wait_stage<AHEAD, PER>(issued - 1 - st);
        __syncthreads();   // every wave's copies visible; stage st-1's buffer is free
        if (st + AHEAD < nk && st + AHEAD >= pre) issue(st + AHEAD);
        lds_u8 *stg = smem + (st % NST) * STG;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[MI], bfr[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) af[i] = *(const bf16x8 *)(stg + (a_rd[i] ^ (32 * ks)));
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (B_KCONTIG) {
                    bfr[j] = *(const bf16x8 *)(stg + (b_rd[j] ^ (32 * ks)));
                } else {
                    lds_u8 *p = stg + b_rd[j] + 16 * ks * (BN * 2);
                    bfr[j].lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
                    bfr[j].hi = __builtin_bit_cast(
                        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * (BN * 2))));
                }
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    if constexpr (ABS) {
        // ---- q~[t][h][:] = q^C_h[t][:] . W^UK_h^T for the tile's 64 rows
        __syncthreads();   // every wave is done with the stage buffers
        const int h = n0 / BN;
        const uint16_t *wuk = g.W2 + (int64_t)h * g.N2 * BN;
        // tile (c, e) of W^UK_h: rows 128 c .. +127, k 64 e .. +63, as a
        // k-contiguous B tile at (2 c + e) * 16 KiB; wave w copies rows
        // RB w .. +15 of each (2 copies)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int c = t >> 1, e = t & 1;
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const int row = RB * wave + 8 * d + (lane >> 3), pos = lane & 7;
                const uint32_t off =
                    (uint32_t)(((128 * c + row) * BN + 64 * e + ((pos ^ ((row >> 1) & 7)) << 3)) * 2);
                dma16(smem_addr + t * TILE_B + (RB * wave + 8 * d) * (BK * 2), off, wuk);
            }
        }
        // q^C (bf16) as an A operand: k half e = n >> 6 of row m at
        // A2 + e * 8 KiB, in the A tile's swizzled layout
        constexpr int A2 = ABS_A2;
        uint16_t *a2 = (uint16_t *)(smem_ + A2);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = TWM * wm + 8 * (r >> 2) + 4 * g32 + (r & 3);
            const int n = TWN * wn + l32;
            const int byte = (n >> 6) * (TM * BK * 2) + m * (BK * 2) + ((((n & 63) >> 3) ^ ((m >> 1) & 7)) << 4) +
                             2 * (n & 7);
            a2[byte >> 1] = f32_to_bf16(acc[0][0][r]);
        }
        const uint32_t bk_rd = (uint32_t)((TWN * wn + l32) * (BK * 2) +
                                          ((g32 ^ (((TWN * wn + l32) >> 1) & 7)) << 4));
        f32x16 acc2[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc2[c] = f32x16{};
            // tiles 2c and 2c + 1 landed: the later tiles' copies may be in flight
            if (c == 0) wait_vm<12>();
            else if (c == 1) wait_vm<8>();
            else if (c == 2) wait_vm<4>();
            else wait_vm<0>();
            __syncthreads();   // every wave's copies (and, first, the q^C writes) are visible
            const int tb = 2 * c * TILE_B;
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int ks = 0; ks < BK / 16; ++ks) {
                    const bf16x8 af = *(const bf16x8 *)(smem + A2 + e * (TM * BK * 2) + (a_rd[0] ^ (32 * ks)));
                    const bf16x8 bf = *(const bf16x8 *)(smem + tb + e * TILE_B + (bk_rd ^ (32 * ks)));
                    acc2[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc2[c], 0, 0, 0);
                }
        }
        uint16_t *ql = (uint16_t *)g.C2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = m0 + TWM * wm + 8 * (r >> 2) + 4 * g32 + (r & 3);
            if (t < g.M) {
                uint16_t *row = ql + ((int64_t)t * g.H2 + h) * g.N2 + TWN * wn + l32;
#pragma unroll
                for (int c = 0; c < 4; ++c) row[128 * c] = f32_to_bf16(acc2[c][r]);
            }
        }
        return;
    }

    // ---- epilogue: the tile through LDS in the output type (bf16 rounded
    // here), then 16-byte row stores
    __syncthreads();   // every wave is done with the stage buffers
    float *ct = (float *)smem_;
    uint16_t *ct16 = (uint16_t *)smem_;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = TWM * wm + 32 * i + 8 * (r >> 2) + 4 * g32 + (r & 3);
                const int n = TWN * wn + 32 * j + l32;
                if constexpr (OUT_F32) ct[m * C_PITCH + n] = acc[i][j][r];
                else ct16[m * C_PITCH + n] = f32_to_bf16(acc[i][j][r]);
            }
    __syncthreads();
    const int64_t cb = (int64_t)b * g.bsc + (int64_t)s * g.css;
    for (int idx = threadIdx.x; idx < TM * (BN / 8); idx += NT) {
        const int m = idx / (BN / 8), c8 = idx % (BN / 8);
        if (m0 + m >= g.M) break;   // rows are visited in increasing order
        if (n0 + 8 * c8 >= g.N) continue;
        const int64_t off = cb + (int64_t)(m0 + m) * g.ldc + n0 + 8 * c8;
        if constexpr (OUT_F32) {
            float4 *dst = (float4 *)((float *)g.C + off);
            dst[0] = *(const float4 *)(ct + m * C_PITCH + 8 * c8);
            dst[1] = *(const float4 *)(ct + m * C_PITCH + 8 * c8 + 4);
        } else {
            *(uint4 *)((uint16_t *)g.C + off) = *(const uint4 *)(ct16 + m * C_PITCH + 8 * c8);
        }
    }
    }   // column tiles
}

// out[m][n] = bf16(sum over splits of ws[s][m][n]), 8 consecutive n per thread
__global__ __launch_bounds__(256) void split_sum_kernel(const float *__restrict__ ws, int32_t splits,
                                                        int64_t split_stride, int64_t n8,
                                                        uint16_t *__restrict__ out) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s) {
            const float4 *p = (const float4 *)(ws + s * split_stride + 8 * i);
            const float4 x = p[0], y = p[1];
            a[0] += x.x; a[1] += x.y; a[2] += x.z; a[3] += x.w;
            a[4] += y.x; a[5] += y.y; a[6] += y.z; a[7] += y.w;
        }
        uint4 pk;
        pk.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
        pk.z = (uint32_t)f32_to_bf16(a[4]) | ((uint32_t)f32_to_bf16(a[5]) << 16);
        pk.w = (uint32_t)f32_to_bf16(a[6]) | ((uint32_t)f32_to_bf16(a[7]) << 16);
        *(uint4 *)(out + 8 * i) = pk;
    }
}

// workgroups of one product: column-tile groups, row tiles, batch x splits
struct Units {
    int tx, ty, n;
};
Units units_of(const GemmArgs &g, int batch, int tm) {
    const int tiles = (g.N + BN - 1) / BN, nt = g.ntiles < 1 ? 1 : g.ntiles;
    Units u;
    u.tx = (tiles + nt - 1) / nt;
    u.ty = (g.M + tm - 1) / tm;
    u.n = u.tx * u.ty * batch * g.splits;
    return u;
}

template <bool B_KCONTIG, bool OUT_F32, int NST = NST_STREAM, int WV = WV_STREAM, int TM = BM>
hipError_t launch_gemm(const GemmArgs &g, int batch, hipStream_t st, bool z_first = false) {
    const Units u = units_of(g, batch, TM);
    GemmPair G{};
    G.p0 = g; G.p1 = g;
    G.units0 = u.n; G.tx0 = G.tx1 = u.tx; G.ty0 = G.ty1 = u.ty;
    G.z_first = z_first ? 1 : 0; G.nz = batch * g.splits;
    launch_timed((gemm_bf16_kernel<B_KCONTIG, OUT_F32, NST, WV, TM>), dim3((unsigned)u.n), dim3(64 * WV), 0, st,
                 G);
    return hipGetLastError();
}

// two products in one launch (batch 1 each), product 0's workgroups first
template <bool B_KCONTIG, bool OUT_F32, int NST = NST_STREAM, int WV = WV_STREAM>
hipError_t launch_gemm_pair(const GemmArgs &g0, const GemmArgs &g1, hipStream_t st) {
    const Units u0 = units_of(g0, 1, BM), u1 = units_of(g1, 1, BM);
    GemmPair G{};
    G.p0 = g0; G.p1 = g1;
    G.units0 = u0.n; G.tx0 = u0.tx; G.ty0 = u0.ty; G.tx1 = u1.tx; G.ty1 = u1.ty;
    launch_timed((gemm_bf16_kernel<B_KCONTIG, OUT_F32, NST, WV, BM>), dim3((unsigned)(u0.n + u1.n)), dim3(64 * WV), 0,
                 st, G);
    return hipGetLastError();
}

}  // namespace

// Split count for C[M][N] = A[M][K] B[K][N]: as many splits as keep the
// workgroups within one round on the device (256 compute units), at most 16,
// with at least 4 of the 64-wide stages per split.
int gemm_splits(int32_t M, int32_t N, int32_t K) {
    const int tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    const int nk = K / BK;
    int sp = 256 / tiles;
    sp = sp < 16 ? sp : 16;
    sp = sp < nk / 4 ? sp : nk / 4;
    return sp < 1 ? 1 : sp;
}

bool gemm_nn_mfma_ok(int32_t N, int32_t K) { return N % 8 == 0 && N >= 8 && K % BK == 0; }

// Splits of two products launched together whose workgroups should fit one
// round on the device: the smallest per-workgroup stage count S for which
// ceil(nk_i / S) splits of each product (at most 16, at least 4 stages
// each when the product has them) give at most 256 workgroups.
void gemm_pair_splits(int32_t M, int32_t N0, int32_t K0, int32_t N1, int32_t K1, int *s0, int *s1) {
    const int rows = (M + BM - 1) / BM;
    const int t0 = ((N0 + BN - 1) / BN) * rows, t1 = ((N1 + BN - 1) / BN) * rows;
    const int k0 = K0 / BK, k1 = K1 / BK;
    auto fit = [](int k, int S) {
        int sp = (k + S - 1) / S;
        sp = sp < 16 ? sp : 16;
        sp = sp < k / 4 ? sp : k / 4;
        return sp < 1 ? 1 : sp;
    };
    const int kmax = k0 > k1 ? k0 : k1;
    for (int S = 1; S <= kmax; ++S) {
        *s0 = fit(k0, S);
        *s1 = fit(k1, S);
        if (t0 * *s0 + t1 * *s1 <= 256) return;
    }
    *s0 = *s1 = 1;
}

// ws0 / ws1 as launch_gemm_nn_f32 for the two products A B0 and A B1 (one A,
// one launch)
hipError_t launch_gemm_nn_f32_pair(const void *A, int64_t lda, int32_t M, int32_t K, const void *B0, int64_t ldb0,
                                   float *ws0, int32_t N0, int splits0, const void *B1, int64_t ldb1, float *ws1,
                                   int32_t N1, int splits1, hipStream_t s) {
    GemmArgs g0{}, g1{};
    g0.A = g1.A = (const uint16_t *)A; g0.lda = g1.lda = lda;
    g0.B = (const uint16_t *)B0; g0.ldb = ldb0;
    g1.B = (const uint16_t *)B1; g1.ldb = ldb1;
    g0.C = ws0; g0.ldc = N0; g0.css = (int64_t)M * N0;
    g1.C = ws1; g1.ldc = N1; g1.css = (int64_t)M * N1;
    g0.M = g1.M = M; g0.K = g1.K = K;
    g0.N = N0; g1.N = N1;
    g0.splits = splits0; g1.splits = splits1;
    g0.ntiles = g1.ntiles = 1;
    return launch_gemm_pair<false, true>(g0, g1, s);
}

// ws[s][m][n] = sum over k in split s of A[m][k] B[k][n] (bf16 in, fp32 out),
// A k-contiguous with row stride lda, B n-contiguous with row stride ldb.
hipError_t launch_gemm_nn_f32(const void *A, int64_t lda, const void *B, int64_t ldb, float *ws,
                              int32_t M, int32_t N, int32_t K, int splits, hipStream_t s) {
    GemmArgs g{};
    g.A = (const uint16_t *)A; g.lda = lda; g.bsa = 0;
    g.B = (const uint16_t *)B; g.ldb = ldb; g.bsb = 0;
    g.C = ws; g.ldc = N; g.bsc = 0; g.css = (int64_t)M * N;
    g.M = M; g.N = N; g.K = K; g.splits = splits; g.ntiles = 1;
    return launch_gemm<false, true>(g, 1, s);
}

// As launch_gemm_nn_f32 for a short product (the cache row's): 64-row tiles
// and as many splits as put every workgroup's stages in flight at once
// (at most one round of 256 workgroups, at most 32 splits).
int gemm_splits_short(int32_t M, int32_t N, int32_t K) {
    const int tiles = ((N + BN - 1) / BN) * ((M + 63) / 64);
    const int nk = K / BK;
    int sp = (nk + NST_STREAM - 1) / NST_STREAM;
    sp = sp < 32 ? sp : 32;
    while (sp > 1 && tiles * sp > 256) --sp;
    return sp < 1 ? 1 : sp;
}

hipError_t launch_gemm_nn_f32_short(const void *A, int64_t lda, const void *B, int64_t ldb, float *ws,
                                    int32_t M, int32_t N, int32_t K, int splits, hipStream_t s) {
    GemmArgs g{};
    g.A = (const uint16_t *)A; g.lda = lda; g.bsa = 0;
    g.B = (const uint16_t *)B; g.ldb = ldb; g.bsb = 0;
    g.C = ws; g.ldc = N; g.bsc = 0; g.css = (int64_t)M * N;
    g.M = M; g.N = N; g.K = K; g.splits = splits; g.ntiles = 1;
    return launch_gemm<false, true, NST_STREAM, 8, 64>(g, 1, s);
}

// C[m][n] = bf16(A[m][k] B[k][n]), one split.
hipError_t launch_gemm_nn_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                               int64_t ldc, int32_t M, int32_t N, int32_t K, hipStream_t s) {
    GemmArgs g{};
    g.A = (const uint16_t *)A; g.lda = lda; g.bsa = 0;
    g.B = (const uint16_t *)B; g.ldb = ldb; g.bsb = 0;
    g.C = C; g.ldc = ldc; g.bsc = 0; g.css = 0;
    g.M = M; g.N = N; g.K = K; g.splits = 1; g.ntiles = 1;
    // few 128-row tiles: 64-row tiles double the workgroups
    const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    if (M > 64 && 2 * tiles <= 256) return launch_gemm<false, false, NST_STREAM, 8, 64>(g, 1, s);
    return launch_gemm<false, false>(g, 1, s);
}

// out[i] = bf16(sum_s ws[s][i]) for n8 groups of 8 elements
hipError_t launch_split_sum_bf16(const float *ws, int splits, int64_t split_stride, int64_t n8,
                                 void *out, hipStream_t s) {
    const int64_t nb = (n8 + 255) / 256;
    const unsigned grid = (unsigned)(nb < 4096 ? (nb < 1 ? 1 : nb) : 4096);
    launch_timed(split_sum_kernel, dim3(grid), dim3(256), 0, s, ws, splits, split_stride, n8,
                       (uint16_t *)out);
    return hipGetLastError();
}

bool absorb_q_mfma_ok(int32_t d_nope, int32_t d_c, mla_dtype_t dt) {
    return dt == MLA_DT_BF16 && d_nope % BK == 0 && d_c % BN == 0;
}

hipError_t launch_absorb_q_mfma(const void *q_nope, int64_t ld_q, const void *w_uk, void *q_lat,
                                int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c,
                                hipStream_t s) {
    GemmArgs g{};
    g.A = (const uint16_t *)q_nope; g.lda = ld_q; g.bsa = d_nope;
    g.B = (const uint16_t *)w_uk;   g.ldb = d_nope; g.bsb = (int64_t)d_c * d_nope;
    g.C = q_lat; g.ldc = (int64_t)n_h * d_c; g.bsc = d_c; g.css = 0;
    g.M = T; g.N = d_c; g.K = d_nope; g.splits = 1; g.ntiles = 1;
    // K = d_nope is at most two stages: one 128 x 128 tile per workgroup on
    // the short stage buffers, two workgroups per CU, every copy issued at
    // the start; eight waves (two per SIMD) measured faster than four, 64-row
    // tiles (twice the workgroups) slower
    if (d_nope <= NST_SHORT * BK) return launch_gemm<true, false, NST_SHORT, 8, BM>(g, n_h, s);
    return launch_gemm<true, false>(g, n_h, s);
}

bool q_up_absorb_ok(int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c, int32_t q_lora) {
    return d_nope == BN && d_c == 4 * BN && q_lora % BK == 0 && n_h >= 1 && T >= 1;
}

// q~[t][h][:] = (c^Q[t][:] W^UQ[:, 128 h .. 128 h + 127]) W^UK_h^T: one
// workgroup per (head, 64 query rows); the rows of one head run on one XCD
// (workgroup u = h + heads * row tile)
hipError_t launch_q_up_absorb(const void *cq, int64_t ld_cq, const void *w_uq, const void *w_uk, void *q_lat,
                              int32_t T, int32_t n_h, int32_t q_lora, hipStream_t s) {
    GemmArgs g{};
    g.A = (const uint16_t *)cq; g.lda = ld_cq;
    g.B = (const uint16_t *)w_uq; g.ldb = (int64_t)n_h * BN;
    g.M = T; g.N = n_h * BN; g.K = q_lora; g.splits = 1; g.ntiles = 1;
    g.W2 = (const uint16_t *)w_uk; g.C2 = q_lat; g.N2 = 4 * BN; g.H2 = n_h;
    const Units u = units_of(g, 1, 64);
    GemmPair G{};
    G.p0 = g; G.p1 = g;
    G.units0 = u.n; G.tx0 = G.tx1 = u.tx; G.ty0 = G.ty1 = u.ty;
    launch_timed((gemm_bf16_kernel<false, false, NST_STREAM, 8, 64, true>), dim3((unsigned)u.n), dim3(512), 0, s,
                 G);
    return hipGetLastError();
}

bool absorb_out_mfma_ok(int32_t n_h, int32_t d_c, int32_t d_v, int32_t d_model, mla_dtype_t dt) {
    return dt == MLA_DT_BF16 && d_c % BK == 0 && d_v % BN == 0 && ((int64_t)n_h * d_v) % BK == 0 &&
           d_model % BN == 0;
}

int64_t absorb_out_mfma_workspace(int32_t T, int32_t n_h, int32_t d_v, int32_t d_model) {
    const int sp = gemm_splits(T, d_model, n_h * d_v);
    return (int64_t)sp * T * d_model * 4;
}

hipError_t launch_absorb_out_mfma(const void *o_lat, const void *w_uv, const void *w_o,
                                  void *u_ws, void *out, float *ws, int32_t T, int32_t n_h,
                                  int32_t d_c, int32_t d_v, int32_t d_model, hipStream_t s) {
    // u[t][h][:] = o_lat[t][h][:] . W_UV[h]: one GEMM per head, B n-contiguous
    GemmArgs g1{};
    g1.A = (const uint16_t *)o_lat; g1.lda = (int64_t)n_h * d_c; g1.bsa = d_c;
    g1.B = (const uint16_t *)w_uv;  g1.ldb = d_v; g1.bsb = (int64_t)d_c * d_v;
    g1.C = u_ws; g1.ldc = (int64_t)n_h * d_v; g1.bsc = d_v; g1.css = 0;
    g1.M = T; g1.N = d_v; g1.K = d_c; g1.splits = 1; g1.ntiles = 1;
    // few 128-row tiles (one per head at T <= 128): 64-row tiles double the
    // workgroups, and the two of a head share an XCD (row tile slowest in the
    // grid, n_h * column tiles apart) so its W_UV tile comes from L2 the second time
    const int64_t tiles1 = (int64_t)n_h * ((d_v + BN - 1) / BN) * ((T + BM - 1) / BM);
    const bool t64 = T > 64 && 2 * tiles1 <= 256 && ((int64_t)n_h * ((d_v + BN - 1) / BN)) % 8 == 0;
    hipError_t e = t64 ? launch_gemm<false, false, NST_STREAM, 8, 64>(g1, n_h, s, true)
                       : launch_gemm<false, false>(g1, n_h, s);
    if (e != hipSuccess) return e;
    // out = u . W_O over K = n_h d_v, split into fp32 partials, then summed
    const int32_t K = n_h * d_v;
    const int sp = gemm_splits(T, d_model, K);
    GemmArgs g2{};
    g2.A = (const uint16_t *)u_ws; g2.lda = K; g2.bsa = 0;
    g2.B = (const uint16_t *)w_o;  g2.ldb = d_model; g2.bsb = 0;
    g2.C = ws; g2.ldc = d_model; g2.bsc = 0; g2.css = (int64_t)T * d_model;
    g2.M = T; g2.N = d_model; g2.K = K; g2.splits = sp; g2.ntiles = 1;
    e = launch_gemm<false, true>(g2, 1, s);
    if (e != hipSuccess) return e;
    const int64_t n8 = (int64_t)T * d_model / 8;
    const int64_t nb = (n8 + 255) / 256;
    const unsigned grid = (unsigned)(nb < 4096 ? nb : 4096);
    launch_timed(split_sum_kernel, dim3(grid), dim3(256), 0, s, (const float *)ws, sp,
                       (int64_t)T * d_model, n8, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace mla

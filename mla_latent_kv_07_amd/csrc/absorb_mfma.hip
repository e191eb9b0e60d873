// bf16 MFMA GEMMs for the absorptions around the decode:
//   q_lat[t][h][:] = q_nope[t][h][:] . W_UK[h]^T          huny.dev "DeepSeek MLA 해부" §3-1
//   u[t][h][:]     = o_lat[t][h][:] . W_UV[h]             §3-2 value equation
//   out[t][:]      = u[t][:] . W_O   (all heads at once)  §3-2 output equation
// One batched kernel, C[z][m][n] = sum_k A[z][m][k] B[z](k, n) with fp32
// accumulation: A is always k-contiguous (activations); B is k-contiguous
// (W_UK[h] = B^T) or n-contiguous (W_UV[h], W_O).  At decode the token count
// T is small, so these products stream their weights: the kernel is built to
// keep HBM busy (direct-to-LDS copies, four stage buffers) rather than to
// maximise MFMA reuse.
//
// Workgroup: 4 waves, a 128 x 128 tile of C, K in 64-wide stages.  Wave w
// computes the 64 x 64 sub-tile (64 (w & 1), 64 (w >> 1)) as 2 x 2
// v_mfma_f32_32x32x16_bf16 blocks.  LDS tiles are filled by 1 KiB
// global_load_lds_dwordx4 copies whose lanes fetch XOR-swizzled 16-byte
// chunks, so that the fragment reads are free of bank conflicts:
//   k-contiguous tile [128 rows][64 k], 128 B rows: chunk c of row r at
//     position c ^ ((r >> 1) & 7)  (16 rows reading one chunk hit 16 bank groups);
//   n-contiguous tile [64 k][128 n], 256 B rows: chunk c of row k at
//     c ^ (4 (k & 3))  (a transposed read covers 4 rows x 64 B: all 64 banks).
// The n-contiguous B operand is read with ds_read_b64_tr_b16 (lane i of each
// 16-lane group receives element i % 4 of the 8 bytes read by lane 4s + i/4).
// Long K with few tiles (W_O) is split over workgroups into fp32 partials
// that a small kernel sums and rounds.
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
constexpr int NSTAGE = 4;
constexpr int DMA_PER_STAGE = 8;             // per wave: 4 for A, 4 for B
constexpr int C_PITCH = BN + 8;              // fp32 staging pitch (floats)
static_assert(BM * C_PITCH * 4 <= NSTAGE * STAGE, "output staging exceeds the stage buffers");

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
    int32_t ntiles;      // column tiles per workgroup, in turn (blockIdx.x * ntiles + j)
};

__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, const void *src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(src)
                 : "memory", "m0");
}

template <bool B_KCONTIG, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem_[NSTAGE * STAGE];
    lds_u8 *smem = (lds_u8 *)smem_;
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int z = blockIdx.z, b = z / g.splits, s = z % g.splits;
    const int m0 = blockIdx.y * BM;
    for (int tj = 0; tj < g.ntiles; ++tj) {
    const int n0 = (blockIdx.x * g.ntiles + tj) * BN;
    if (n0 >= g.N) break;
    if (tj > 0) __syncthreads();   // the previous tile's epilogue is done with the LDS
    const int nk_all = g.K / BK;
    const int st0 = (int)((int64_t)s * nk_all / g.splits), nk = (int)((int64_t)(s + 1) * nk_all / g.splits) - st0;
    const int64_t k_begin = (int64_t)st0 * BK;

    // ---- copy offsets (bytes, relative to a per-stage scalar base)
    const uint16_t *a_base = g.A + (int64_t)b * g.bsa + (int64_t)m0 * g.lda + k_begin;
    const uint16_t *b_base = B_KCONTIG ? g.B + (int64_t)b * g.bsb + (int64_t)n0 * g.ldb + k_begin
                                       : g.B + (int64_t)b * g.bsb + k_begin * g.ldb + n0;
    uint32_t a_off[4], b_off[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        // A: wave w copies tile rows 32w + 8d .. +7 (lane i: row + i/8, position i%8);
        // rows past M read row M-1 (their results are never stored)
        const int row = 32 * wave + 8 * d + (lane >> 3), pos = lane & 7;
        const int mrow = min(m0 + row, g.M - 1) - m0;
        a_off[d] = (uint32_t)(((int64_t)mrow * g.lda + ((pos ^ ((row >> 1) & 7)) << 3)) * 2);
        if (B_KCONTIG) {
            // columns past N read column N-1 (never stored)
            const int nrow = min(n0 + row, g.N - 1) - n0;
            b_off[d] = (uint32_t)(((int64_t)nrow * g.ldb + ((pos ^ ((row >> 1) & 7)) << 3)) * 2);
        } else {
            // B: wave w copies k rows 16w + 4d .. +3 (lane i: row + i/16, position i%16);
            // 8-column chunks past N read the last chunk (never stored)
            const int krow = 16 * wave + 4 * d + (lane >> 4), p16 = lane & 15;
            const int col = min(8 * (p16 ^ (4 * (krow & 3))), g.N - 8 - n0);
            b_off[d] = (uint32_t)(((int64_t)krow * g.ldb + col) * 2);
        }
    }
    auto issue = [&](int st) {
        const uint32_t lds = smem_addr + (st & (NSTAGE - 1)) * STAGE;
        const uint16_t *as = a_base + (int64_t)st * BK;
        const uint16_t *bs = B_KCONTIG ? b_base + (int64_t)st * BK : b_base + (int64_t)st * BK * g.ldb;
#pragma unroll
        for (int d = 0; d < 4; ++d) dma16(lds + (32 * wave + 8 * d) * (BK * 2), a_off[d], as);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t row0 = B_KCONTIG ? (32 * wave + 8 * d) * (BK * 2) : (16 * wave + 4 * d) * (BN * 2);
            dma16(lds + TILE_A + row0, b_off[d], bs);
        }
    };

    // ---- fragment read bases (bytes within a stage)
    const int wm = wave & 1, wn = wave >> 1;
    const int g32 = lane >> 5, l32 = lane & 31;
    uint32_t a_rd[2];   // A rows 64 wm + 32 i + l32, chunk 2 ks + g32 -> a_rd[i] ^ (32 ks)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = 64 * wm + 32 * i + l32;
        a_rd[i] = m * (BK * 2) + ((g32 ^ ((m >> 1) & 7)) << 4);
    }
    uint32_t b_rd[2];
    const int G = lane >> 4, w16 = lane & 15, q = w16 >> 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (B_KCONTIG) {
            const int n = 64 * wn + 32 * j + l32;
            b_rd[j] = TILE_A + n * (BK * 2) + ((g32 ^ ((n >> 1) & 7)) << 4);
        } else {
            // k row 16 ks + 8 g + 4 hi + q (+16 ks * 256 B and 4 hi * 256 B as offsets);
            // n bytes 2 (64 wn + 32 j) + 32 (G & 1) + 8 (w16 & 3): chunk 8 wn + 4 j + 2 (G & 1)
            // + ((w16 & 3) >> 1) XORed with 4 q (k & 3 = q), byte 8 (w16 & 1)
            const int chunk = 8 * wn + 4 * j + 2 * (G & 1) + ((w16 & 3) >> 1);
            b_rd[j] = TILE_A + (8 * g32 + q) * (BN * 2) + ((chunk ^ (4 * q)) << 4) + 8 * (w16 & 1);
        }
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    for (int st = 0; st < 3 && st < nk; ++st) issue(st);
    for (int st = 0; st < nk; ++st) {
        // stage st landed for this wave (later stages may be in flight)
        const int younger = min(2, nk - 1 - st);
        if (younger >= 2)
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (younger == 1)
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // every wave's copies visible; stage st-1's buffer is free
        if (st + 3 < nk) issue(st + 3);
        lds_u8 *stg = smem + (st & (NSTAGE - 1)) * STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8 *)(stg + (a_rd[i] ^ (32 * ks)));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
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
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- epilogue: the fp32 tile through LDS, then 16-byte row stores
    __syncthreads();   // every wave is done with the stage buffers
    float *ct = (float *)smem_;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * g32 + (r & 3);
                const int n = 64 * wn + 32 * j + l32;
                ct[m * C_PITCH + n] = acc[i][j][r];
            }
    __syncthreads();
    const int64_t cb = (int64_t)b * g.bsc + (int64_t)s * g.css;
    for (int idx = threadIdx.x; idx < BM * (BN / 8); idx += 256) {
        const int m = idx / (BN / 8), c8 = idx % (BN / 8);
        if (m0 + m >= g.M) break;   // rows are visited in increasing order
        if (n0 + 8 * c8 >= g.N) continue;
        const float4 v0 = *(const float4 *)(ct + m * C_PITCH + 8 * c8);
        const float4 v1 = *(const float4 *)(ct + m * C_PITCH + 8 * c8 + 4);
        const int64_t off = cb + (int64_t)(m0 + m) * g.ldc + n0 + 8 * c8;
        if constexpr (OUT_F32) {
            float4 *dst = (float4 *)((float *)g.C + off);
            dst[0] = v0;
            dst[1] = v1;
        } else {
            uint4 pk;
            pk.x = (uint32_t)f32_to_bf16(v0.x) | ((uint32_t)f32_to_bf16(v0.y) << 16);
            pk.y = (uint32_t)f32_to_bf16(v0.z) | ((uint32_t)f32_to_bf16(v0.w) << 16);
            pk.z = (uint32_t)f32_to_bf16(v1.x) | ((uint32_t)f32_to_bf16(v1.y) << 16);
            pk.w = (uint32_t)f32_to_bf16(v1.z) | ((uint32_t)f32_to_bf16(v1.w) << 16);
            *(uint4 *)((uint16_t *)g.C + off) = pk;
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

template <bool B_KCONTIG, bool OUT_F32>
hipError_t launch_gemm(const GemmArgs &g, int batch, hipStream_t st) {
    const int tiles = (g.N + BN - 1) / BN, nt = g.ntiles < 1 ? 1 : g.ntiles;
    dim3 grid((unsigned)((tiles + nt - 1) / nt), (unsigned)((g.M + BM - 1) / BM), (unsigned)(batch * g.splits));
    launch_timed((gemm_bf16_kernel<B_KCONTIG, OUT_F32>), grid, dim3(256), 0, st, g);
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

// C[m][n] = bf16(A[m][k] B[k][n]), one split.
hipError_t launch_gemm_nn_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                               int64_t ldc, int32_t M, int32_t N, int32_t K, hipStream_t s) {
    GemmArgs g{};
    g.A = (const uint16_t *)A; g.lda = lda; g.bsa = 0;
    g.B = (const uint16_t *)B; g.ldb = ldb; g.bsb = 0;
    g.C = C; g.ldc = ldc; g.bsc = 0; g.css = 0;
    g.M = M; g.N = N; g.K = K; g.splits = 1; g.ntiles = 1;
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
    g.M = T; g.N = d_c; g.K = d_nope; g.splits = 1;
    // K = d_nope is two stages: one 128 x 128 tile per workgroup would take
    // two rounds of short workgroups; two tiles each (the query tile
    // re-read from L2) keep the heads within one round
    const int tiles = (d_c + BN - 1) / BN;
    g.ntiles = (int64_t)tiles * n_h > 256 && tiles > 1 ? 2 : 1;
    return launch_gemm<true, false>(g, n_h, s);
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
    hipError_t e = launch_gemm<false, false>(g1, n_h, s);
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

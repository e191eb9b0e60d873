// The producers of the decode's inputs, from the hidden states of the new
// tokens:
//   cache append      c = h W^DKV, k^R = RoPE(h W^KR), written into the token's
//                     slot of the paged cache (huny.dev "DeepSeek MLA 해부"
//                     §2-1 compression equation and §2-3 shared rotary key;
//                     vLLM MLA page, the kv_c_and_k_pe cache of "FlashMLAImpl")
//   query production  c^Q = h W^DQ, q^C = c^Q W^UQ (§2-2), q~ = q^C W^UK^T
//                     (§3-1 absorption), q^R = RoPE(h W^QR) (§2-3)
// Products run on the bf16 MFMA GEMM (split over K into fp32 partials when
// the output is small); a finishing kernel sums the partials and applies the
// rotation, the storage rounding and, for fp8 caches, the block scale.  On
// the MFMA path the queries take three launches: h W^QR with h W^DQ, the
// finish of both (q^R rotated, c^Q rounded to bf16), then c^Q W^UQ with the
// absorption by W^UK^T fused behind it (q^C never leaves the chip).
// RoPE frequencies are plain (theta_j = base^(-2j/d)) or YaRN-scaled; the
// huny page names YaRN for 128K+ contexts (§6, YaRN item) without a
// formula: the table follows the published YaRN NTK-by-parts interpolation.
#include <cmath>

#include "common.hpp"

namespace mla {

bool gemm_nn_mfma_ok(int32_t N, int32_t K);
int gemm_splits(int32_t M, int32_t N, int32_t K);
hipError_t launch_gemm_nn_f32(const void *A, int64_t lda, const void *B, int64_t ldb, float *ws,
                              int32_t M, int32_t N, int32_t K, int splits, hipStream_t s);
hipError_t launch_gemm_nn_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                               int64_t ldc, int32_t M, int32_t N, int32_t K, hipStream_t s);
hipError_t launch_split_sum_bf16(const float *ws, int splits, int64_t split_stride, int64_t n8,
                                 void *out, hipStream_t s);
bool q_up_absorb_ok(int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c, int32_t q_lora);
hipError_t launch_q_up_absorb(const void *cq, int64_t ld_cq, const void *w_uq, const void *w_uk, void *q_lat,
                              int32_t T, int32_t n_h, int32_t q_lora, hipStream_t s);
int gemm_splits_short(int32_t M, int32_t N, int32_t K);
hipError_t launch_gemm_nn_f32_short(const void *A, int64_t lda, const void *B, int64_t ldb, float *ws,
                                    int32_t M, int32_t N, int32_t K, int splits, hipStream_t s);
void gemm_pair_splits(int32_t M, int32_t N0, int32_t K0, int32_t N1, int32_t K1, int *s0, int *s1);
hipError_t launch_gemm_nn_f32_pair(const void *A, int64_t lda, int32_t M, int32_t K, const void *B0, int64_t ldb0,
                                   float *ws0, int32_t N0, int splits0, const void *B1, int64_t ldb1, float *ws1,
                                   int32_t N1, int splits1, hipStream_t s);

bool rope_table(const mla_rope_t *r, int32_t d_r, RopeTab *t) {
    if (!r || d_r < 2 || d_r % 2 || d_r / 2 > kMaxRopePairs) return false;
    if (!(r->base > 1.0) || !(r->factor > 0.0) || !(r->mscale > 0.0)) return false;
    const int half = d_r / 2;
    t->half = half;
    t->mscale = (float)r->mscale;
    for (int j = 0; j < half; ++j) {
        const double theta = std::pow(r->base, -2.0 * j / d_r);
        double th = theta;
        if (r->factor != 1.0) {
            if (!(r->orig_ctx > 0.0)) return false;
            // turns of pair j over the original context, and the ramp between
            // interpolation (theta / s) and the unchanged frequency
            const double turns = r->orig_ctx * theta / (2.0 * M_PI);
            double gamma;
            if (r->beta_fast > r->beta_slow)
                gamma = std::fmin(1.0, std::fmax(0.0, (turns - r->beta_slow) / (r->beta_fast - r->beta_slow)));
            else
                gamma = turns >= r->beta_fast ? 1.0 : 0.0;
            th = (1.0 - gamma) * theta / r->factor + gamma * theta;
        }
        t->theta[j] = th;
    }
    return true;
}

namespace {

// OCP E4M3 ("fn") from fp32: round to nearest even, |x| >= 448 saturates to
// +-448, NaN -> 0x7F, the sign of zero dropped (as x < 0 decides the sign).
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
    if (x != x) return 0x7F;
    const uint8_t sign = x < 0.f ? 0x80 : 0x00;
    const float a = fabsf(x);
    if (a >= 448.f) return sign | 0x7E;
    if (a < 0.015625f) {   // below 2^-6: subnormal steps of 2^-9 (8 steps reach 2^-6 = code 8)
        return sign | (uint8_t)__builtin_rintf(a * 512.f);
    }
    int e;
    const float m = frexpf(a, &e);            // a = m 2^e, m in [0.5, 1): exponent e - 1
    float q = __builtin_rintf(m * 16.f);      // 8..16: 1.mmm in eighths
    if (q == 16.f) { q = 8.f; ++e; }
    const int ef = e - 1 + 7;                 // biased exponent, 1..15
    if (ef > 15 || (ef == 15 && q > 14.f)) return sign | 0x7E;
    return sign | (uint8_t)((ef << 3) | ((int)q - 8));
}

// OCP E5M2 from fp32: round to nearest even, |x| >= 57344 saturates to
// +-57344 (as the e4m3 encoder saturates), NaN -> 0x7F, sign as x < 0.
__device__ __forceinline__ uint8_t f32_to_e5m2(float x) {
    if (x != x) return 0x7F;
    const uint8_t sign = x < 0.f ? 0x80 : 0x00;
    const float a = fabsf(x);
    if (a >= 57344.f) return sign | 0x7B;
    if (a < 6.103515625e-05f)   // below 2^-14: subnormal steps of 2^-16 (4 steps reach code 4)
        return sign | (uint8_t)__builtin_rintf(a * 65536.f);
    int e;
    const float m = frexpf(a, &e);            // a = m 2^e, m in [0.5, 1)
    float q = __builtin_rintf(m * 8.f);       // 4..8: 1.mm in quarters
    if (q == 8.f) { q = 4.f; ++e; }
    const int ef = e - 1 + 15;                // biased exponent, 1..30
    return sign | (uint8_t)((ef << 2) | ((int)q - 4));
}

__device__ __forceinline__ float e5m2_to_f32(uint8_t c) {
    const int e = (c >> 2) & 31, m = c & 3;
    if (e == 31) return m ? __builtin_nanf("") : ((c & 0x80) ? -__builtin_inff() : __builtin_inff());
    const float v = e == 0 ? (float)m * 1.52587890625e-05f : ldexpf(1.f + (float)m * 0.25f, e - 15);
    return (c & 0x80) ? -v : v;
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
    if ((c & 0x7F) == 0x7F) return __builtin_nanf("");
    const int e = (c >> 3) & 15, m = c & 7;
    const float v = e == 0 ? (float)m * 0.001953125f : ldexpf(1.f + (float)m * 0.125f, e - 7);
    return (c & 0x80) ? -v : v;
}

// sum over splits of ws[s * stride + i]: the first U splits' loads are all
// issued before the first add (one memory latency for the usual split
// counts), any further ones in turn
template <int U = 16>
__device__ __forceinline__ float split_sum(const float *__restrict__ ws, int64_t stride, int splits, int64_t i) {
    float v[U];
#pragma unroll
    for (int s = 0; s < U; ++s) v[s] = s < splits ? ws[s * stride + i] : 0.f;
#pragma unroll
    for (int w = U / 2; w > 0; w >>= 1)
#pragma unroll
        for (int s = 0; s < w; ++s) v[s] += v[s + w];
    for (int s = U; s < splits; ++s) v[0] += ws[s * stride + i];
    return v[0];
}

struct AppendArgs {
    const float *ws;          // fp32 partials: split s, token t, value f at ws[s split_stride + t ws_ld + f]
    int64_t split_stride;
    int64_t ws_ld;            // d_c + d_r, or wider when the row's columns share a partial buffer
    int32_t splits;
    uint8_t *pool;
    float *scales;
    int64_t block_bytes, num_blocks;
    const int32_t *bt;
    int32_t bt_stride;
    const int32_t *pos0;
    int32_t pos0_count;       // B
    int32_t q_len, d_c, d_r;
};

// fp8 caches (e4m3 or e5m2 latent + bf16 k^R, or the whole row in e4m3): one
// workgroup per sequence, its q_len tokens in order (positions outside the
// block table, p < 0 or p >= 64 bt_stride, or whose table entry is not a
// pool block id, are skipped).  The tokens that land
// in one block are handled together: the amax of their coded values sets or
// raises the block scale, earlier slots are re-encoded when it grows, then
// the codes are written.
template <int CODE>   // 0 e4m3 latent, 1 e5m2 latent, 2 e4m3 whole row
__device__ __forceinline__ void append_fp8_seq(const AppendArgs &a, const RopeTab &rt, int b) {
    constexpr bool ROWC = CODE == 2;
    constexpr float TOP = CODE == 1 ? 57344.f : 448.f;
    auto enc = [](float v) { return CODE == 1 ? f32_to_e5m2(v) : f32_to_e4m3(v); };
    auto dec = [](uint8_t c) { return CODE == 1 ? e5m2_to_f32(c) : e4m3_to_f32(c); };
    const int W = ROWC ? a.d_c + a.d_r : a.d_c;   // code bytes per token
    __shared__ float red[4];
    __shared__ float sh[3];
    const int tid = threadIdx.x;
    const int p0 = a.pos0[b];
    auto xval = [&](int t, int f) { return split_sum(a.ws, a.split_stride, a.splits, (int64_t)t * a.ws_ld + f); };
    auto block_of = [&](int p) { return (int64_t)a.bt[(int64_t)b * a.bt_stride + p / kBlock]; };
    // rotary pair j of token t at position p: rotated, times mscale
    auto rot = [&](int t, int p, int j, float &y0, float &y1) {
        const float x0 = xval(t, a.d_c + 2 * j), x1 = xval(t, a.d_c + 2 * j + 1);
        double sn, cs;
        sincos((double)p * rt.theta[j], &sn, &cs);
        const float c = (float)cs, s = (float)sn;
        y0 = (x0 * c - x1 * s) * rt.mscale;
        y1 = (x0 * s + x1 * c) * rt.mscale;
    };

    int i = 0;
    while (i < a.q_len) {
        const int p = p0 + i;
        const int i_end = p < 0 ? i + 1 : min(a.q_len, (p / kBlock + 1) * kBlock - p0);   // same block
        if (p < 0 || p / kBlock >= a.bt_stride) {   // outside the table: not written
            i = i_end;
            continue;
        }
        const int64_t blk = block_of(p);
        if (blk < 0 || blk >= a.num_blocks) {        // unallocated table slot: not written
            i = i_end;
            continue;
        }
        uint8_t *base = a.pool + blk * a.block_bytes;
        const int s0 = p % kBlock;
        // amax of the new latents in this block
        float m = 0.f;
        for (int k = i; k < i_end; ++k) {
            for (int f = tid; f < a.d_c; f += 256) m = fmaxf(m, fabsf(xval(b * a.q_len + k, f)));
            if constexpr (ROWC) {
                for (int j = tid; j < rt.half; j += 256) {
                    float y0, y1;
                    rot(b * a.q_len + k, p0 + k, j, y0, y1);
                    m = fmaxf(m, fmaxf(fabsf(y0), fabsf(y1)));
                }
            }
        }
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            const float old = a.scales[blk];
            float sc;
            bool grow = false;
            if (s0 == 0) {
                sc = amax > 0.f ? amax / TOP : 1.f;
            } else {
                sc = fmaxf(old, amax / TOP);
                grow = sc > old;
            }
            sh[0] = sc;
            sh[1] = grow ? old / sc : 1.f;
            sh[2] = grow ? 1.f : 0.f;
            a.scales[blk] = sc;
        }
        __syncthreads();
        const float sc = sh[0], ratio = sh[1];
        if (sh[2] != 0.f) {
            // re-encode the slots before the first new one at the larger scale
            for (int idx = tid; idx < s0 * W; idx += 256) base[idx] = enc(dec(base[idx]) * ratio);
        }
        for (int k = i; k < i_end; ++k) {
            const int t = b * a.q_len + k, pk = p0 + k, slot = pk % kBlock;
            for (int f = tid; f < a.d_c; f += 256) base[slot * W + f] = enc(xval(t, f) / sc);
            for (int j = tid; j < rt.half; j += 256) {
                float y0, y1;
                rot(t, pk, j, y0, y1);
                if constexpr (ROWC) {
                    base[slot * W + a.d_c + 2 * j] = enc(y0 / sc);
                    base[slot * W + a.d_c + 2 * j + 1] = enc(y1 / sc);
                } else {
                    uint16_t *kr = (uint16_t *)(base + (int64_t)kBlock * a.d_c + (int64_t)slot * a.d_r * 2);
                    kr[2 * j] = f32_to_bf16(y0);
                    kr[2 * j + 1] = f32_to_bf16(y1);
                }
            }
        }
        __syncthreads();   // red / sh are reused by the next block
        i = i_end;
    }
}

template <int CODE>
__global__ __launch_bounds__(256) void append_fp8_kernel(AppendArgs a, RopeTab rt) {
    append_fp8_seq<CODE>(a, rt, blockIdx.x);
}

// f32 / bf16 caches: one thread per (token, pair of row values); the rotary
// pairs turn by p theta_j (fp64 angle), then every value is rounded once.
template <int FMT>   // 0 f32, 1 bf16, 2 f16
__device__ __forceinline__ void append_row_pair(const AppendArgs &a, const RopeTab &rt, int64_t idx) {
    const int N = a.d_c + a.d_r, P2 = N / 2;
    if (idx >= (int64_t)a.q_len * a.pos0_count * P2) return;
    const int t = (int)(idx / P2), k = (int)(idx % P2);
    const int b = t / a.q_len, p = a.pos0[b] + t % a.q_len;
    if (p < 0 || p / kBlock >= a.bt_stride) return;   // outside the table: not written
    const int64_t blk = a.bt[(int64_t)b * a.bt_stride + p / kBlock];
    if (blk < 0 || blk >= a.num_blocks) return;       // unallocated table slot: not written
    const int64_t o = (int64_t)t * a.ws_ld + 2 * k;
    float y0 = split_sum<32>(a.ws, a.split_stride, a.splits, o);
    float y1 = split_sum<32>(a.ws, a.split_stride, a.splits, o + 1);
    if (2 * k >= a.d_c) {
        const int j = k - a.d_c / 2;
        double sn, cs;
        sincos((double)p * rt.theta[j], &sn, &cs);
        const float c = (float)cs, s = (float)sn;
        const float x0 = y0, x1 = y1;
        y0 = (x0 * c - x1 * s) * rt.mscale;
        y1 = (x0 * s + x1 * c) * rt.mscale;
    }
    uint8_t *row = a.pool + blk * a.block_bytes + (int64_t)(p % kBlock) * N * (FMT == 0 ? 4 : 2);
    if constexpr (FMT == 0) {
        *(float2 *)((float *)row + 2 * k) = make_float2(y0, y1);
    } else if constexpr (FMT == 1) {
        *(uint32_t *)((uint16_t *)row + 2 * k) = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
    } else {
        *(uint32_t *)((uint16_t *)row + 2 * k) = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y0) |
                                                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y1) << 16);
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void append_rows_kernel(AppendArgs a, RopeTab rt) {
    append_row_pair<FMT>(a, rt, blockIdx.x * 256ll + threadIdx.x);
}

// q^R: out[t][h][2j, 2j+1] = RoPE of the summed partials at token t's
// position, times mscale; item idx = (token, head, pair), angle p theta_j in
// fp64.  Positions: pos[t] (pos_q_len 1), or pos[t / q_len] + t % q_len when
// pos holds each sequence's first new position (pos_q_len = q_len).
template <typename OutT>
__device__ __forceinline__ void rope_q_item(int64_t idx, const float *__restrict__ ws, int64_t split_stride,
                                            int32_t splits, const int32_t *__restrict__ pos, int32_t pos_q_len,
                                            int32_t T, int32_t n_h, int32_t d_r, OutT *__restrict__ out,
                                            const RopeTab &rt) {
    const int64_t per_t = (int64_t)n_h * rt.half;
    if (idx >= T * per_t) return;
    const int t = (int)(idx / per_t), hj = (int)(idx % per_t);
    const int h = hj / rt.half, j = hj % rt.half;
    const int64_t o = (int64_t)t * n_h * d_r + (int64_t)h * d_r + 2 * j;
    const float x0 = split_sum(ws, split_stride, splits, o), x1 = split_sum(ws, split_stride, splits, o + 1);
    double sn, cs;
    const int p = pos[t / pos_q_len] + t % pos_q_len;
    sincos((double)p * rt.theta[j], &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float y0 = (x0 * c - x1 * s) * rt.mscale, y1 = (x0 * s + x1 * c) * rt.mscale;
    if constexpr (sizeof(OutT) == 2) {
        *(uint32_t *)(out + o) = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
    } else {
        out[o] = y0;
        out[o + 1] = y1;
    }
}

// The q^R items [256 blk, 256 blk + 256) of one 256-thread block: every
// head of a token turns by the same angles, so the block first forms the
// (cos, sin) of each (token, pair) it touches once, in LDS, then each
// thread rotates its item as rope_q_item does (the same values: the angle
// is the same fp64 product).
__device__ __forceinline__ void rope_q_block(int blk, const float *__restrict__ ws, int64_t split_stride,
                                             int32_t splits, const int32_t *__restrict__ pos, int32_t pos_q_len,
                                             int32_t T, int32_t n_h, int32_t d_r, uint16_t *__restrict__ out,
                                             const RopeTab &rt) {
    constexpr int TAB = 512;   // >= (256 / per_t + 2) * half entries for any per_t >= half
    __shared__ float2 cs_tab[TAB];
    const int half = rt.half;
    const int64_t per_t = (int64_t)n_h * half;
    const int64_t first = blk * 256ll, last = min(first + 255, (int64_t)T * per_t - 1);
    const int t0 = (int)(first / per_t), t1 = (int)(last / per_t);
    const int n_e = (t1 - t0 + 1) * half;
    for (int e = threadIdx.x; e < n_e; e += 256) {
        const int t = t0 + e / half, j = e % half;
        const int p = pos[t / pos_q_len] + t % pos_q_len;
        double sn, cs;
        sincos((double)p * rt.theta[j], &sn, &cs);
        cs_tab[e] = make_float2((float)cs, (float)sn);
    }
    __syncthreads();
    const int64_t idx = first + threadIdx.x;
    if (idx > last) return;
    const int t = (int)(idx / per_t), hj = (int)(idx % per_t);
    const int h = hj / half, j = hj % half;
    const int64_t o = (int64_t)t * n_h * d_r + (int64_t)h * d_r + 2 * j;
    const float x0 = split_sum(ws, split_stride, splits, o), x1 = split_sum(ws, split_stride, splits, o + 1);
    const float2 r = cs_tab[(t - t0) * half + j];
    const float y0 = (x0 * r.x - x1 * r.y) * rt.mscale, y1 = (x0 * r.y + x1 * r.x) * rt.mscale;
    *(uint32_t *)(out + o) = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
}

// one thread per (token, head, pair)
template <typename OutT>
__global__ __launch_bounds__(256) void rope_q_kernel(const float *__restrict__ ws, int64_t split_stride,
                                                     int32_t splits, const int32_t *__restrict__ pos,
                                                     int32_t T, int32_t n_h, int32_t d_r, OutT *__restrict__ out,
                                                     RopeTab rt) {
    rope_q_item(blockIdx.x * 256ll + threadIdx.x, ws, split_stride, splits, pos, 1, T, n_h, d_r, out, rt);
}

// Arguments of the finishing kernel of the low-rank query products.
struct FinishArgs {
    const float *ws1;          // h W^DQ partials: split s, token t, column c at ws1[(s T + t) ld1 + c]
    int32_t sp1, ld1, q_lora;
    uint16_t *cq;              // c^Q [T][q_lora], bf16
    int32_t nb_cq;             // blocks of the c^Q part
    const float *ws3;          // h W^QR partials [sp3][T][n_h d_r]
    int32_t sp3;
    const int32_t *pos;        // positions, as rope_q_item reads them (pos_q_len)
    int32_t pos_q_len, T, n_h, d_r;
    uint16_t *q_rope;          // q^R [T][n_h][d_r], bf16
    int32_t nb_rope;           // blocks of the q^R part
};

// The finishes of the low-rank query products in one launch.  APP >= 0
// (one decode step's producers): the first blocks finish the new cache rows,
// whose partials share the h W^DQ buffer: APP 0-2 one row-value pair per
// thread (append_row_pair, f32 / bf16 / f16 rows), APP 3-5 one block per
// sequence (append_fp8_seq, e4m3 / e5m2 latent, whole row in e4m3); they
// come first so that none of them trails the launch.  Then nb_cq blocks
// write c^Q = bf16(sum of the h W^DQ partials), 8 consecutive values per
// thread, and nb_rope blocks q^R = RoPE(sum of the h W^QR partials), one
// rotary pair per thread.
template <int APP>
__global__ __launch_bounds__(256) void q_finish_kernel(FinishArgs f, RopeTab rt, AppendArgs app) {
    int blk = blockIdx.x;
    if constexpr (APP >= 0) {
        const int nb_app = (int)gridDim.x - f.nb_cq - f.nb_rope;
        if (blk < nb_app) {
            if constexpr (APP >= 3) append_fp8_seq<APP - 3>(app, rt, blk);
            else append_row_pair<APP>(app, rt, blk * 256ll + threadIdx.x);
            return;
        }
        blk -= nb_app;
    }
    if (blk >= f.nb_cq) {
        rope_q_block(blk - f.nb_cq, f.ws3, (int64_t)f.T * f.n_h * f.d_r, f.sp3, f.pos, f.pos_q_len, f.T, f.n_h,
                     f.d_r, f.q_rope, rt);
        return;
    }
    const int64_t i = blk * 256ll + threadIdx.x;
    const int per_t = f.q_lora / 8;
    if (i >= (int64_t)f.T * per_t) return;
    const int t = (int)(i / per_t), c8 = (int)(i % per_t);
    const float *src = f.ws1 + (int64_t)t * f.ld1 + 8 * c8;
    const int64_t sstride = (int64_t)f.T * f.ld1;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // four splits' loads in flight per round
    for (int s0 = 0; s0 < f.sp1; s0 += 4) {
        float4 x[4], y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (s0 + k < f.sp1) {
                const float4 *p = (const float4 *)(src + (s0 + k) * sstride);
                x[k] = p[0];
                y[k] = p[1];
            } else {
                x[k] = y[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[0] += x[k].x; a[1] += x[k].y; a[2] += x[k].z; a[3] += x[k].w;
            a[4] += y[k].x; a[5] += y[k].y; a[6] += y[k].z; a[7] += y[k].w;
        }
    }
    uint4 pk;
    pk.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
    pk.z = (uint32_t)f32_to_bf16(a[4]) | ((uint32_t)f32_to_bf16(a[5]) << 16);
    pk.w = (uint32_t)f32_to_bf16(a[6]) | ((uint32_t)f32_to_bf16(a[7]) << 16);
    *(uint4 *)(f.cq + (int64_t)t * f.q_lora + 8 * c8) = pk;
}

template <typename T>
__device__ __forceinline__ float ldv(const T *p, int64_t i) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(p[i]);
    else return p[i];
}

// Generic C[z][m][n] = sum_k A[z][m][k] B[z](k, n) in fp32, one thread per
// output; B(k, n) = B[z * bsb + k * sbk + n * sbn].  For fp32 data and shapes
// the MFMA GEMM does not take.
template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const TA *__restrict__ A, int64_t lda, int64_t bsa,
                                                           const TB *__restrict__ B, int64_t sbk, int64_t sbn,
                                                           int64_t bsb, TC *__restrict__ C, int64_t ldc,
                                                           int64_t bsc, int32_t M, int32_t N, int32_t K,
                                                           int32_t batch) {
    const int64_t total = (int64_t)batch * M * N;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int n = (int)(i % N);
        const int m = (int)((i / N) % M);
        const int z = (int)(i / ((int64_t)M * N));
        const TA *a = A + z * bsa + (int64_t)m * lda;
        const TB *bb = B + z * bsb + (int64_t)n * sbn;
        float acc = 0.f;
        for (int k = 0; k < K; ++k) acc += ldv(a, k) * ldv(bb, (int64_t)k * sbk);
        if constexpr (sizeof(TC) == 2) C[z * bsc + (int64_t)m * ldc + n] = f32_to_bf16(acc);
        else C[z * bsc + (int64_t)m * ldc + n] = acc;
    }
}

unsigned grid_of(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

template <typename TA, typename TB, typename TC>
hipError_t gemm_generic(const TA *A, int64_t lda, int64_t bsa, const TB *B, int64_t sbk, int64_t sbn,
                        int64_t bsb, TC *C, int64_t ldc, int64_t bsc, int32_t M, int32_t N, int32_t K,
                        int32_t batch, hipStream_t s) {
    launch_timed((gemm_generic_kernel<TA, TB, TC>), dim3(grid_of((int64_t)batch * M * N)), dim3(256),
                       0, s, A, lda, bsa, B, sbk, sbn, bsb, C, ldc, bsc, M, N, K, batch);
    return hipGetLastError();
}

bool append_mfma(mla_dtype_t dt, int32_t d_model, int32_t N) {
    return dt == MLA_DT_BF16 && gemm_nn_mfma_ok(N, d_model);
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int64_t cache_append_workspace(int32_t T, int32_t d_model, int32_t d_c, int32_t d_r, mla_dtype_t dt) {
    const int32_t N = d_c + d_r;
    const int sp = append_mfma(dt, d_model, N) ? gemm_splits_short(T, N, d_model) : 1;
    return align256((int64_t)sp * T * N * 4);
}

hipError_t launch_cache_append(const void *h, const void *w_kv, mla_dtype_t dt, uint8_t *pool,
                               float *scales, int64_t block_bytes, int64_t num_blocks,
                               mla_dtype_t kv, const int32_t *bt, int32_t bt_stride,
                               const int32_t *pos0, int32_t B, int32_t q_len, int32_t d_model,
                               int32_t d_c, int32_t d_r, const RopeTab &rt, float *ws,
                               hipStream_t s) {
    const int32_t T = B * q_len, N = d_c + d_r;
    int sp = 1;
    hipError_t e;
    if (append_mfma(dt, d_model, N)) {
        sp = gemm_splits_short(T, N, d_model);
        e = launch_gemm_nn_f32_short(h, d_model, w_kv, N, ws, T, N, d_model, sp, s);
    } else if (dt == MLA_DT_BF16) {
        e = gemm_generic((const uint16_t *)h, d_model, 0, (const uint16_t *)w_kv, N, 1, 0, ws, N, 0, T, N,
                         d_model, 1, s);
    } else {
        e = gemm_generic((const float *)h, d_model, 0, (const float *)w_kv, N, 1, 0, ws, N, 0, T, N, d_model,
                         1, s);
    }
    if (e != hipSuccess) return e;
    AppendArgs a{};
    a.ws = ws; a.split_stride = (int64_t)T * N; a.ws_ld = N; a.splits = sp;
    a.pool = pool; a.scales = scales; a.block_bytes = block_bytes; a.num_blocks = num_blocks;
    a.bt = bt; a.bt_stride = bt_stride; a.pos0 = pos0; a.pos0_count = B; a.q_len = q_len;
    a.d_c = d_c; a.d_r = d_r;
    const unsigned rows_grid = (unsigned)(((int64_t)T * (N / 2) + 255) / 256);
    if (kv == MLA_DT_F32)
        launch_timed(append_rows_kernel<0>, dim3(rows_grid), dim3(256), 0, s, a, rt);
    else if (kv == MLA_DT_BF16)
        launch_timed(append_rows_kernel<1>, dim3(rows_grid), dim3(256), 0, s, a, rt);
    else if (kv == MLA_DT_F16)
        launch_timed(append_rows_kernel<2>, dim3(rows_grid), dim3(256), 0, s, a, rt);
    else if (kv == MLA_DT_FP8_E4M3)
        launch_timed(append_fp8_kernel<0>, dim3(B), dim3(256), 0, s, a, rt);
    else if (kv == MLA_DT_FP8_E5M2)
        launch_timed(append_fp8_kernel<1>, dim3(B), dim3(256), 0, s, a, rt);
    else
        launch_timed(append_fp8_kernel<2>, dim3(B), dim3(256), 0, s, a, rt);
    return hipGetLastError();
}

// ---------------------------------------------------------------- queries

namespace {

FinishArgs finish_args(const float *ws1, int sp1, int32_t ld1, int32_t q_lora, uint16_t *cq, const float *ws3,
                       int sp3, const int32_t *pos, int32_t pos_q_len, int32_t T, int32_t n_h, int32_t d_r,
                       uint16_t *q_rope) {
    FinishArgs f{};
    f.ws1 = ws1; f.sp1 = sp1; f.ld1 = ld1; f.q_lora = q_lora; f.cq = cq;
    f.nb_cq = (int32_t)(((int64_t)T * q_lora / 8 + 255) / 256);
    f.ws3 = ws3; f.sp3 = sp3; f.pos = pos; f.pos_q_len = pos_q_len; f.T = T; f.n_h = n_h; f.d_r = d_r;
    f.q_rope = q_rope;
    f.nb_rope = (int32_t)(((int64_t)T * n_h * (d_r / 2) + 255) / 256);
    return f;
}

struct QPlan {
    bool mfma;
    int sp1, sp3;                 // splits of h W^DQ and h W^QR
    int64_t off_cq, off_qc, off_w1, off_w3, total;
};

QPlan q_plan(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope, int32_t d_c,
             int32_t d_r, mla_dtype_t dt) {
    QPlan q{};
    const int32_t NQ = n_h * d_nope, NR = n_h * d_r;
    q.mfma = dt == MLA_DT_BF16 && gemm_nn_mfma_ok(q_lora, d_model) && gemm_nn_mfma_ok(NQ, q_lora) &&
             gemm_nn_mfma_ok(NR, d_model) && d_nope % 64 == 0 && d_c % 128 == 0;
    q.sp1 = q.sp3 = 1;
    // h W^QR and h W^DQ share one launch
    if (q.mfma) gemm_pair_splits(T, NR, d_model, q_lora, d_model, &q.sp3, &q.sp1);
    // c^Q and q^C: bf16 on the MFMA path (the next product's operand), fp32 otherwise
    const int eb = q.mfma ? 2 : 4;
    int64_t o = 0;
    q.off_cq = o; o = align256(o + (int64_t)T * q_lora * eb);
    q.off_qc = o; o = align256(o + (int64_t)T * NQ * eb);
    q.off_w1 = o; o = align256(o + (q.mfma ? (int64_t)q.sp1 * T * q_lora * 4 : 0));
    q.off_w3 = o; o = align256(o + (int64_t)q.sp3 * T * NR * 4);
    q.total = o;
    return q;
}

}  // namespace

int64_t project_q_workspace(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope,
                            int32_t d_c, int32_t d_r, mla_dtype_t dt) {
    return q_plan(T, d_model, q_lora, n_h, d_nope, d_c, d_r, dt).total;
}

hipError_t launch_project_q(const void *h, const void *w_dq, const void *w_uq, const void *w_qr,
                            const void *w_uk, mla_dtype_t dt, const int32_t *pos, int32_t T,
                            int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope, int32_t d_c,
                            int32_t d_r, const RopeTab &rt, void *q_lat, void *q_rope, void *ws,
                            hipStream_t s) {
    const QPlan q = q_plan(T, d_model, q_lora, n_h, d_nope, d_c, d_r, dt);
    const int32_t NQ = n_h * d_nope, NR = n_h * d_r;
    uint8_t *w = (uint8_t *)ws;
    hipError_t e;
    if (q.mfma) {
        // h W^QR and h W^DQ (split over d_model into fp32 partials) in one launch
        float *w1 = (float *)(w + q.off_w1), *w3 = (float *)(w + q.off_w3);
        e = launch_gemm_nn_f32_pair(h, d_model, T, d_model, w_qr, NR, w3, NR, q.sp3, w_dq, q_lora, w1, q_lora,
                                    q.sp1, s);
        if (e != hipSuccess) return e;
        // c^Q = bf16(sum of its partials) and q^R = RoPE(sum of its partials)
        const FinishArgs f = finish_args(w1, q.sp1, q_lora, q_lora, (uint16_t *)(w + q.off_cq), w3, q.sp3, pos,
                                         1, T, n_h, d_r, (uint16_t *)q_rope);
        launch_timed(q_finish_kernel<-1>, dim3((unsigned)(f.nb_cq + f.nb_rope)), dim3(256), 0, s, f, rt,
                     AppendArgs{});
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        // q~ = (c^Q W^UQ) W^UK^T per head, q^C kept on chip
        if (q_up_absorb_ok(T, n_h, d_nope, d_c, q_lora))
            return launch_q_up_absorb(w + q.off_cq, q_lora, w_uq, w_uk, q_lat, T, n_h, q_lora, s);
        // q^C = c^Q W^UQ
        e = launch_gemm_nn_bf16(w + q.off_cq, q_lora, w_uq, NQ, w + q.off_qc, NQ, T, NQ, q_lora, s);
        if (e != hipSuccess) return e;
        // q~ = q^C W^UK^T per head
        return launch_absorb_q(w + q.off_qc, NQ, w_uk, q_lat, T, n_h, d_nope, d_c, dt, s);
    } else {
        float *cq = (float *)(w + q.off_cq), *qc = (float *)(w + q.off_qc), *w3 = (float *)(w + q.off_w3);
        if (dt == MLA_DT_BF16) {
            const uint16_t *H = (const uint16_t *)h;
            e = gemm_generic(H, d_model, 0, (const uint16_t *)w_dq, q_lora, 1, 0, cq, q_lora, 0, T, q_lora, d_model, 1, s);
            if (e == hipSuccess)
                e = gemm_generic((const float *)cq, q_lora, 0, (const uint16_t *)w_uq, NQ, 1, 0, qc, NQ, 0, T, NQ, q_lora, 1, s);
            // q~[t][i][c] = sum_k q^C[t][i][k] W_UK[i][c][k]: batch over heads
            if (e == hipSuccess)
                e = gemm_generic((const float *)qc, NQ, d_nope, (const uint16_t *)w_uk, 1, d_nope,
                                 (int64_t)d_c * d_nope, (uint16_t *)q_lat, (int64_t)n_h * d_c, d_c, T, d_c,
                                 d_nope, n_h, s);
            if (e == hipSuccess)
                e = gemm_generic(H, d_model, 0, (const uint16_t *)w_qr, NR, 1, 0, w3, NR, 0, T, NR, d_model, 1, s);
        } else {
            const float *H = (const float *)h;
            e = gemm_generic(H, d_model, 0, (const float *)w_dq, q_lora, 1, 0, cq, q_lora, 0, T, q_lora, d_model, 1, s);
            if (e == hipSuccess)
                e = gemm_generic((const float *)cq, q_lora, 0, (const float *)w_uq, NQ, 1, 0, qc, NQ, 0, T, NQ, q_lora, 1, s);
            if (e == hipSuccess)
                e = gemm_generic((const float *)qc, NQ, d_nope, (const float *)w_uk, 1, d_nope,
                                 (int64_t)d_c * d_nope, (float *)q_lat, (int64_t)n_h * d_c, d_c, T, d_c,
                                 d_nope, n_h, s);
            if (e == hipSuccess)
                e = gemm_generic(H, d_model, 0, (const float *)w_qr, NR, 1, 0, w3, NR, 0, T, NR, d_model, 1, s);
        }
        if (e != hipSuccess) return e;
    }
    const float *w3 = (const float *)(w + q.off_w3);
    const unsigned rg = (unsigned)(((int64_t)T * n_h * (d_r / 2) + 255) / 256);
    if (dt == MLA_DT_BF16)
        launch_timed(rope_q_kernel<uint16_t>, dim3(rg), dim3(256), 0, s, w3, (int64_t)T * NR, q.sp3, pos,
                           T, n_h, d_r, (uint16_t *)q_rope, rt);
    else
        launch_timed(rope_q_kernel<float>, dim3(rg), dim3(256), 0, s, w3, (int64_t)T * NR, q.sp3, pos,
                           T, n_h, d_r, (float *)q_rope, rt);
    return hipGetLastError();
}

// ------------------------------------------------- one decode step's producers

namespace {

// The three down-projections of h, side by side in one weight
// [d_model][q_lora + d_c + d_r] (W^DQ, W^DKV, W^KR columns), are product 1
// of the paired launch, h W^QR product 0: the cache row's product rides in
// the query's launch, its finish in the query finish.
struct StepPlan {
    int sp1, sp3;
    int32_t N1;
    int64_t off_cq, off_w1, off_w3, total;
};

StepPlan step_plan(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_c, int32_t d_r) {
    StepPlan p{};
    p.N1 = q_lora + d_c + d_r;
    const int32_t NR = n_h * d_r;
    gemm_pair_splits(T, NR, d_model, p.N1, d_model, &p.sp3, &p.sp1);
    int64_t o = 0;
    p.off_cq = o; o = align256(o + (int64_t)T * q_lora * 2);
    p.off_w1 = o; o = align256(o + (int64_t)p.sp1 * T * p.N1 * 4);
    p.off_w3 = o; o = align256(o + (int64_t)p.sp3 * T * NR * 4);
    p.total = o;
    return p;
}

}  // namespace

bool project_step_ok(mla_dtype_t dt, int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope,
                     int32_t d_c, int32_t d_r) {
    const int32_t NQ = n_h * d_nope, NR = n_h * d_r;
    return dt == MLA_DT_BF16 && d_r > 0 && gemm_nn_mfma_ok(q_lora, d_model) && gemm_nn_mfma_ok(NQ, q_lora) &&
           gemm_nn_mfma_ok(NR, d_model) && gemm_nn_mfma_ok(q_lora + d_c + d_r, d_model) && d_nope % 64 == 0 &&
           d_c % 128 == 0 && (d_c + d_r) % 2 == 0 && q_up_absorb_ok(T, n_h, d_nope, d_c, q_lora);
}

int64_t project_step_workspace(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_c,
                               int32_t d_r) {
    return step_plan(T, d_model, q_lora, n_h, d_c, d_r).total;
}

hipError_t launch_project_step(const void *h, const void *w_dkvq, const void *w_uq, const void *w_qr,
                               const void *w_uk, uint8_t *pool, float *scales, int64_t block_bytes,
                               int64_t num_blocks, mla_dtype_t kv, const int32_t *bt, int32_t bt_stride,
                               const int32_t *pos0, int32_t B, int32_t q_len, int32_t d_model, int32_t q_lora,
                               int32_t n_h, int32_t d_c, int32_t d_r, const RopeTab &rt, void *q_lat,
                               void *q_rope, void *ws, hipStream_t s) {
    const int32_t T = B * q_len, NR = n_h * d_r;
    const StepPlan p = step_plan(T, d_model, q_lora, n_h, d_c, d_r);
    uint8_t *w = (uint8_t *)ws;
    float *w1 = (float *)(w + p.off_w1), *w3 = (float *)(w + p.off_w3);
    // h W^QR, and h [W^DQ | W^DKV | W^KR] (split over d_model into fp32 partials), in one launch
    hipError_t e = launch_gemm_nn_f32_pair(h, d_model, T, d_model, w_qr, NR, w3, NR, p.sp3, w_dkvq, p.N1, w1,
                                           p.N1, p.sp1, s);
    if (e != hipSuccess) return e;
    // c^Q, q^R and the new cache rows from their partials
    const FinishArgs f = finish_args(w1, p.sp1, p.N1, q_lora, (uint16_t *)(w + p.off_cq), w3, p.sp3, pos0, q_len,
                                     T, n_h, d_r, (uint16_t *)q_rope);
    AppendArgs a{};
    a.ws = w1 + q_lora; a.split_stride = (int64_t)T * p.N1; a.ws_ld = p.N1; a.splits = p.sp1;
    a.pool = pool; a.scales = scales; a.block_bytes = block_bytes; a.num_blocks = num_blocks;
    a.bt = bt; a.bt_stride = bt_stride; a.pos0 = pos0; a.pos0_count = B; a.q_len = q_len;
    a.d_c = d_c; a.d_r = d_r;
    const unsigned nb = (unsigned)(f.nb_cq + f.nb_rope);
    const unsigned rows = (unsigned)(((int64_t)T * ((d_c + d_r) / 2) + 255) / 256);
    switch (kv) {
    case MLA_DT_F32: launch_timed(q_finish_kernel<0>, dim3(nb + rows), dim3(256), 0, s, f, rt, a); break;
    case MLA_DT_BF16: launch_timed(q_finish_kernel<1>, dim3(nb + rows), dim3(256), 0, s, f, rt, a); break;
    case MLA_DT_F16: launch_timed(q_finish_kernel<2>, dim3(nb + rows), dim3(256), 0, s, f, rt, a); break;
    case MLA_DT_FP8_E4M3: launch_timed(q_finish_kernel<3>, dim3(nb + B), dim3(256), 0, s, f, rt, a); break;
    case MLA_DT_FP8_E5M2: launch_timed(q_finish_kernel<4>, dim3(nb + B), dim3(256), 0, s, f, rt, a); break;
    case MLA_DT_FP8_E4M3_ROW: launch_timed(q_finish_kernel<5>, dim3(nb + B), dim3(256), 0, s, f, rt, a); break;
    default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // q~ = (c^Q W^UQ) W^UK^T per head, q^C kept on chip
    return launch_q_up_absorb(w + p.off_cq, q_lora, w_uq, w_uk, q_lat, T, n_h, q_lora, s);
}

}  // namespace mla

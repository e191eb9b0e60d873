// Generic absorbed-MLA decode: any d_c <= 1024, d_r <= 256 (multiples of 4),
// fp32 / bf16 / fp16 / fp8 (e4m3 or e5m2 latent, or the whole row in e4m3)
// cache, fp32 / bf16 queries.  One wave per query row,
// one cached token at a time with a wavefront reduction for the 576-wide
// (d_c + d_r) dot product.  This is the path for the small fp32 layer and any
// shape the MFMA kernels are not instantiated for; the DeepSeek-V2 shape runs
// on decode_bf16.hip / decode_fp8.hip.
#include "common.hpp"

namespace mla {
namespace {

constexpr int kMaxC = 1024 / 64;  // latent features per lane
constexpr int kMaxR = 256 / 64;   // rotary features per lane

// E4M3 ("fn") code -> fp32, from the format: bias 7, 3 mantissa bits,
// exponent field 0 subnormal, S.1111.111 NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    const uint32_t s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    float v;
    if (e == 0)
        v = (float)m * 0.001953125f;  // m * 2^-9
    else if (e == 15 && m == 7)
        v = __uint_as_float(0x7fc00000u);
    else
        v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
    return s ? -v : v;
}

// E5M2 code -> fp32: bias 15, 2 mantissa bits, exponent field 0 subnormal,
// exponent 31 infinity (mantissa 0) or NaN.
__device__ __forceinline__ float e5m2_to_f32(uint32_t code) {
    const uint32_t s = (code >> 7) & 1u, e = (code >> 2) & 31u, m = code & 3u;
    float v;
    if (e == 0)
        v = (float)m * 1.52587890625e-05f;  // m * 2^-16
    else if (e == 31)
        v = __uint_as_float(m ? 0x7fc00000u : 0x7f800000u);
    else
        v = __uint_as_float(((e + 112u) << 23) | (m << 21));  // (1 + m/4) * 2^(e-15)
    return s ? -v : v;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

template <int KV>
__device__ __forceinline__ float load_c(const uint8_t *blk, int slot, int f, int d_c, int d_r) {
    if constexpr (KV == MLA_DT_F32)
        return ((const float *)blk)[(int64_t)slot * (d_c + d_r) + f];
    else if constexpr (KV == MLA_DT_BF16)
        return bf16_to_f32(((const uint16_t *)blk)[(int64_t)slot * (d_c + d_r) + f]);
    else if constexpr (KV == MLA_DT_F16)
        return f16_to_f32(((const uint16_t *)blk)[(int64_t)slot * (d_c + d_r) + f]);
    else if constexpr (KV == MLA_DT_FP8_E4M3_ROW)
        return e4m3_to_f32(blk[(int64_t)slot * (d_c + d_r) + f]);
    else if constexpr (KV == MLA_DT_FP8_E5M2)
        return e5m2_to_f32(blk[(int64_t)slot * d_c + f]);
    else
        return e4m3_to_f32(blk[(int64_t)slot * d_c + f]);
}

// rotary key value (for the whole-row e4m3 format: the code, before the block scale)
template <int KV>
__device__ __forceinline__ float load_r(const uint8_t *blk, int slot, int f, int d_c, int d_r) {
    if constexpr (KV == MLA_DT_F32)
        return ((const float *)blk)[(int64_t)slot * (d_c + d_r) + d_c + f];
    else if constexpr (KV == MLA_DT_BF16)
        return bf16_to_f32(((const uint16_t *)blk)[(int64_t)slot * (d_c + d_r) + d_c + f]);
    else if constexpr (KV == MLA_DT_F16)
        return f16_to_f32(((const uint16_t *)blk)[(int64_t)slot * (d_c + d_r) + d_c + f]);
    else if constexpr (KV == MLA_DT_FP8_E4M3_ROW)
        return e4m3_to_f32(blk[(int64_t)slot * (d_c + d_r) + d_c + f]);
    else
        return bf16_to_f32(((const uint16_t *)(blk + (int64_t)kBlock * d_c))[(int64_t)slot * d_r + f]);
}

template <typename QT>
__device__ __forceinline__ float load_q(const QT *p, int64_t i) {
    if constexpr (sizeof(QT) == 2)
        return bf16_to_f32(p[i]);
    else
        return p[i];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int KV, typename QT>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a) {
    // one workgroup per work item: {sequence * row_chunks + chunk, blocks, slot}
    const int item = blockIdx.x;
    if (item >= a.num_items) return;
    const int32_t *it = a.plan + plan_items_off() + 4 * item;
    const int b = it[0] / a.row_chunks, chunk = it[0] % a.row_chunks;
    const int blk0 = it[1], blk1 = it[2], slot = it[3];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int S = a.seq_lens[b];
    const QT *ql = (const QT *)a.q_lat;
    const QT *qr = (const QT *)a.q_rope;
    const uint8_t *pool = (const uint8_t *)a.pool;

    for (int r = chunk * kRowsPerChunk + wave; r < min(a.rows, (chunk + 1) * kRowsPerChunk); r += 4) {
        const int t = r / a.n_h;
        const int64_t grow = (int64_t)b * a.rows + r;  // global query row
        float qc[kMaxC], qrr[kMaxR], o[kMaxC];
#pragma unroll
        for (int j = 0; j < kMaxC; ++j) {
            const int f = lane + 64 * j;
            qc[j] = f < a.d_c ? load_q(ql, grow * a.d_c + f) : 0.f;
            o[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < kMaxR; ++j) {
            const int f = lane + 64 * j;
            qrr[j] = f < a.d_r ? load_q(qr, grow * a.d_r + f) : 0.f;
        }
        const int p_end = min(blk1 * kBlock, S - a.q_len + t + 1);
        float m = -INFINITY, l = 0.f;  // running max (log2 units) and sum
        for (int p = blk0 * kBlock; p < p_end; ++p) {
            int64_t blk = a.block_table[(int64_t)b * a.bt_stride + p / kBlock];
            blk = blk < 0 ? 0 : (blk >= a.num_pool_blocks ? a.num_pool_blocks - 1 : blk);
            const int sl = p % kBlock;
            const uint8_t *base = pool + blk * a.block_bytes;
            constexpr bool SCALED = KV == MLA_DT_FP8_E4M3 || KV == MLA_DT_FP8_E5M2 || KV == MLA_DT_FP8_E4M3_ROW;
            const float bs = SCALED ? a.block_scales[blk] : 1.0f;
            const float rs = KV == MLA_DT_FP8_E4M3_ROW ? bs : 1.0f;   // scale of the rotary values
            float c[kMaxC];
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxC; ++j) {
                const int f = lane + 64 * j;
                c[j] = f < a.d_c ? load_c<KV>(base, sl, f, a.d_c, a.d_r) * bs : 0.f;
                part += qc[j] * c[j];
            }
#pragma unroll
            for (int j = 0; j < kMaxR; ++j) {
                const int f = lane + 64 * j;
                if (f < a.d_r) part += qrr[j] * (load_r<KV>(base, sl, f, a.d_c, a.d_r) * rs);
            }
            const float s = wave_sum(part) * a.scale_log2;
            const float m_new = fmaxf(m, s);
            const float alpha = exp2f(m - m_new);  // 0 on the first token (m = -inf)
            const float w = exp2f(s - m_new);
            l = l * alpha + w;
#pragma unroll
            for (int j = 0; j < kMaxC; ++j) o[j] = o[j] * alpha + w * c[j];
            m = m_new;
        }
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        const float lse_v = l > 0.f ? (m + log2f(l)) * 0.6931471805599453f : -INFINITY;
        if (slot < 0) {
            QT *dst = (QT *)a.o_lat + grow * a.d_c;
#pragma unroll
            for (int j = 0; j < kMaxC; ++j) {
                const int f = lane + 64 * j;
                if (f < a.d_c) {
                    if constexpr (sizeof(QT) == 2)
                        dst[f] = f32_to_bf16(o[j] * inv);
                    else
                        dst[f] = o[j] * inv;
                }
            }
            if (lane == 0) a.lse[grow] = lse_v;
        } else if (a.partial_dtype == MLA_DT_BF16) {
            uint16_t *dst = (uint16_t *)a.o_part + ((int64_t)slot * a.rows + r) * a.d_c;
#pragma unroll
            for (int j = 0; j < kMaxC; ++j) {
                const int f = lane + 64 * j;
                if (f < a.d_c) dst[f] = f32_to_bf16(o[j] * inv);
            }
            if (lane == 0) a.lse_part[(int64_t)slot * a.rows + r] = lse_v;
        } else {
            float *dst = (float *)a.o_part + ((int64_t)slot * a.rows + r) * a.d_c;
#pragma unroll
            for (int j = 0; j < kMaxC; ++j) {
                const int f = lane + 64 * j;
                if (f < a.d_c) dst[f] = o[j] * inv;
            }
            if (lane == 0) a.lse_part[(int64_t)slot * a.rows + r] = lse_v;
        }
    }
}

template <int KV>
hipError_t launch_kv(const DecodeArgs &a, hipStream_t s) {
    dim3 grid((unsigned)a.num_items);
    if (a.q_dtype == MLA_DT_BF16)
        launch_timed((decode_generic_kernel<KV, uint16_t>), grid, dim3(256), 0, s, a);
    else
        launch_timed((decode_generic_kernel<KV, float>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_generic(const DecodeArgs &a, hipStream_t s) {
    switch (a.kv_dtype) {
    case MLA_DT_F32: return launch_kv<MLA_DT_F32>(a, s);
    case MLA_DT_BF16: return launch_kv<MLA_DT_BF16>(a, s);
    case MLA_DT_FP8_E4M3: return launch_kv<MLA_DT_FP8_E4M3>(a, s);
    case MLA_DT_F16: return launch_kv<MLA_DT_F16>(a, s);
    case MLA_DT_FP8_E5M2: return launch_kv<MLA_DT_FP8_E5M2>(a, s);
    case MLA_DT_FP8_E4M3_ROW: return launch_kv<MLA_DT_FP8_E4M3_ROW>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mla

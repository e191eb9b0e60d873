// Paged gather and the split-merge (LSE combine) kernels.
#include "common.hpp"

namespace mla {
namespace {

// out[b][p][:] = row bytes of logical token p of sequence b (bit-exact copy).
// For the fp8 block layout the row is stitched from the code row and the
// bf16 rotary-key row, which live in separate parts of the block.
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t *__restrict__ pool,
                                                     int64_t block_bytes, int32_t c_bytes,
                                                     int32_t r_bytes, int32_t split_rows,
                                                     const int32_t *__restrict__ bt,
                                                     int32_t bt_stride,
                                                     const int32_t *__restrict__ seq_lens,
                                                     int32_t max_tokens, uint8_t *__restrict__ out) {
    const int b = blockIdx.y;
    const int row_words = (c_bytes + r_bytes) >> 2;
    const int n = min(seq_lens[b], max_tokens);
    for (int p = blockIdx.x * 16; p < min(n, (int)blockIdx.x * 16 + 16); ++p) {
        const int64_t blk = bt[(int64_t)b * bt_stride + p / kBlock];
        const int slot = p % kBlock;
        const uint8_t *base = pool + blk * block_bytes;
        uint32_t *dst = (uint32_t *)(out + ((int64_t)b * max_tokens + p) * (c_bytes + r_bytes));
        if (!split_rows) {
            const uint32_t *src = (const uint32_t *)(base + (int64_t)slot * c_bytes);
            for (int w = threadIdx.x; w < row_words; w += blockDim.x) dst[w] = src[w];
        } else {
            const uint32_t *srcc = (const uint32_t *)(base + (int64_t)slot * c_bytes);
            const uint32_t *srcr = (const uint32_t *)(base + (int64_t)kBlock * c_bytes + (int64_t)slot * r_bytes);
            const int cw = c_bytes >> 2;
            for (int w = threadIdx.x; w < row_words; w += blockDim.x)
                dst[w] = w < cw ? srcc[w] : srcr[w - cw];
        }
    }
}

// One workgroup per (sequence, 2 rows); 128 threads per row stride over d_c.
template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o_part,
                                                      const float *__restrict__ lse_part,
                                                      const int32_t *__restrict__ split_off,
                                                      const int32_t *__restrict__ seq_flags,
                                                      int32_t rows, int32_t d_c,
                                                      OutT *__restrict__ o_lat,
                                                      float *__restrict__ lse) {
    const int b = blockIdx.y;
    const int r = blockIdx.x * 2 + (threadIdx.x >> 7);
    const int tid = threadIdx.x & 127;
    if (r >= rows) return;
    if (seq_flags && seq_flags[b] == 1) return;
    const int k0 = split_off[b], k1 = split_off[b + 1];
    const int64_t out_row = (int64_t)b * rows + r;
    float m = -INFINITY;
    for (int k = k0; k < k1; ++k) m = fmaxf(m, lse_part[(int64_t)k * rows + r]);
    OutT *dst = o_lat + out_row * d_c;
    if (m == -INFINITY) {
        for (int f = tid; f < d_c; f += 128) dst[f] = OutT(0);
        if (tid == 0) lse[out_row] = -INFINITY;
        return;
    }
    float wsum = 0.f;
    for (int k = k0; k < k1; ++k) wsum += expf(lse_part[(int64_t)k * rows + r] - m);
    const float inv = 1.0f / wsum;
    for (int f = tid; f < d_c; f += 128) {
        float acc = 0.f;
        for (int k = k0; k < k1; ++k) {
            const float lk = lse_part[(int64_t)k * rows + r];
            if (lk == -INFINITY) continue;
            acc += expf(lk - m) * o_part[((int64_t)k * rows + r) * d_c + f];
        }
        acc *= inv;
        if constexpr (sizeof(OutT) == 2)
            dst[f] = f32_to_bf16(acc);
        else
            dst[f] = acc;
    }
    if (tid == 0) lse[out_row] = m + logf(wsum);
}

}  // namespace

hipError_t launch_gather(const uint8_t *pool, int64_t block_bytes, int32_t c_bytes,
                         int32_t r_bytes, bool split_rows, const int32_t *bt, int32_t bt_stride,
                         const int32_t *seq_lens, int32_t B, int32_t max_tokens, uint8_t *out,
                         hipStream_t s) {
    dim3 grid((max_tokens + 15) / 16, B);
    hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, pool, block_bytes, c_bytes, r_bytes,
                       (int32_t)split_rows, bt, bt_stride, seq_lens, max_tokens, out);
    return hipGetLastError();
}

hipError_t launch_combine(const float *o_part, const float *lse_part, const int32_t *split_off,
                          const int32_t *seq_flags, int32_t B, int32_t rows, int32_t d_c,
                          void *o_lat, mla_dtype_t out_dt, float *lse, hipStream_t s) {
    dim3 grid((rows + 1) / 2, B);
    if (out_dt == MLA_DT_BF16)
        hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, dim3(256), 0, s, o_part, lse_part,
                           split_off, seq_flags, rows, d_c, (uint16_t *)o_lat, lse);
    else
        hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, o_part, lse_part,
                           split_off, seq_flags, rows, d_c, (float *)o_lat, lse);
    return hipGetLastError();
}

}  // namespace mla

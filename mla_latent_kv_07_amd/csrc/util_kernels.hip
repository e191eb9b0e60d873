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
                                                     int32_t max_tokens, int64_t num_blocks,
                                                     uint8_t *__restrict__ out) {
    const int b = blockIdx.y;
    const int row_words = (c_bytes + r_bytes) >> 2;
    // the host guarantees max_tokens <= 64 bt_stride, so p / 64 stays inside
    // the table row; ids outside the pool are clamped into it
    const int n = min(seq_lens[b], max_tokens);
    for (int p = blockIdx.x * 16; p < min(n, (int)blockIdx.x * 16 + 16); ++p) {
        int64_t blk = bt[(int64_t)b * bt_stride + p / kBlock];
        blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// One wave per output row (sequence b, row r); 4 rows per workgroup.  The
// split weights w_k = exp(lse_k - max) are computed once per row (lane k
// holds split k), then each lane accumulates 4 consecutive features per
// 256-feature stripe with 16-byte loads.  Requires d_c % 4 == 0, d_c <= 1024.
template <typename PartT>
__device__ __forceinline__ void load4(const PartT *p, float &a, float &b, float &c, float &d) {
    if constexpr (sizeof(PartT) == 2) {
        const uint2 v = *(const uint2 *)p;
        a = __uint_as_float(v.x << 16);
        b = __uint_as_float(v.x & 0xffff0000u);
        c = __uint_as_float(v.y << 16);
        d = __uint_as_float(v.y & 0xffff0000u);
    } else {
        const float4 v = *(const float4 *)p;
        a = v.x; b = v.y; c = v.z; d = v.w;
    }
}

template <typename PartT, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const PartT *__restrict__ o_part,
                                                      const float *__restrict__ lse_part,
                                                      const int32_t *__restrict__ split_off,
                                                      const int32_t *__restrict__ seq_flags,
                                                      int32_t rows, int32_t chunk_rows, int32_t d_c,
                                                      OutT *__restrict__ o_lat,
                                                      float *__restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.y;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    // the split list of the row's (sequence, row chunk)
    const int sc = b * ((rows + chunk_rows - 1) / chunk_rows) + r / chunk_rows;
    if (seq_flags && seq_flags[sc] == 1) return;
    const int k0 = split_off[sc], n = split_off[sc + 1] - k0;
    const int64_t out_row = (int64_t)b * rows + r;
    // running max over all splits (in chunks of 64 lanes)
    float m = -INFINITY;
    for (int c = 0; c < n; c += 64)
        if (c + lane < n) m = fmaxf(m, lse_part[(int64_t)(k0 + c + lane) * rows + r]);
    m = wave_max(m);
    OutT *dst = o_lat + out_row * d_c;
    if (m == -INFINITY) {
        for (int f = lane * 4; f < d_c; f += 256)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[f + j] = OutT(0);
        if (lane == 0) lse[out_row] = -INFINITY;
        return;
    }
    float wsum = 0.f;
    float acc[16];   // d_c <= 1024: up to 4 stripes of 256 features, 4 per lane
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    const int stripes = (d_c + 255) / 256;
    for (int c = 0; c < n; c += 64) {
        const float lk = c + lane < n ? lse_part[(int64_t)(k0 + c + lane) * rows + r] : -INFINITY;
        const float wk = lk == -INFINITY ? 0.f : expf(lk - m);
        wsum += wave_sum(wk);
        const int cn = min(64, n - c);
        for (int k = 0; k < cn; ++k) {
            const float w = __shfl(wk, k, 64);
            if (w == 0.f) continue;
            const PartT *src = o_part + ((int64_t)(k0 + c + k) * rows + r) * d_c;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j >= stripes) break;
                const int f = j * 256 + lane * 4;
                if (f < d_c) {
                    float v0, v1, v2, v3;
                    load4(src + f, v0, v1, v2, v3);
                    acc[4 * j + 0] += w * v0;
                    acc[4 * j + 1] += w * v1;
                    acc[4 * j + 2] += w * v2;
                    acc[4 * j + 3] += w * v3;
                }
            }
        }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int f = j * 256 + lane * 4;
        if (j < stripes && f < d_c) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (sizeof(OutT) == 2)
                    dst[f + e] = f32_to_bf16(acc[4 * j + e] * inv);
                else
                    dst[f + e] = acc[4 * j + e] * inv;
            }
        }
    }
    if (lane == 0) lse[out_row] = m + logf(wsum);
}

// 8 merged features of a lane, times inv, as bf16 (one 16-byte store) or fp32
template <typename OutT>
__device__ __forceinline__ void store_row(uint4 *dst, const float (&acc)[8], float inv) {
    if constexpr (sizeof(OutT) == 2) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pk[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
        *dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
        float4 *d4 = (float4 *)dst;
        d4[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        d4[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
}

// Fast path for bf16 partials of 512 latent features (the MFMA decode's
// split output): one wave per output row, lane owns features 8l..8l+7 (one
// 16-byte load per split).  The partial rows of up to 8 splits are requested
// before the split weights are known, so a row costs one memory round trip
// per 8 splits instead of one per split.
// FEW: every segment of the launch has at most 8 splits (the plan's
// max_splits), so only that path is compiled; it fits in 64 VGPRs, which
// lets 8 waves per SIMD run at once: batches with more rows than one round of
// waves at the general variant's 114 VGPRs (4 per SIMD, kCombineRound rows on
// 256 CUs) wait out fewer rounds of memory latency.  Within one round the
// general variant measured 0.1 us faster, so it keeps those.
constexpr int64_t kCombineRound = 256 * 16;
template <typename OutT, bool FEW = false>
__global__ __launch_bounds__(256, FEW ? 8 : 1) void combine512_kernel(const uint16_t *__restrict__ o_part,
                                                         const float *__restrict__ lse_part,
                                                         const int32_t *__restrict__ split_off,
                                                         const int32_t *__restrict__ seq_flags,
                                                         int32_t rows, int32_t chunk_rows,
                                                         OutT *__restrict__ o_lat,
                                                         float *__restrict__ lse) {
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.y;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    // the split list of the row's (sequence, row chunk), wave-uniform: read
    // through the scalar cache
    const int sc = __builtin_amdgcn_readfirstlane(b * ((rows + chunk_rows - 1) / chunk_rows) + r / chunk_rows);
    if (seq_flags && ((const __attribute__((address_space(4))) int32_t *)seq_flags)[sc] == 1) return;
    const int k0 = ((const __attribute__((address_space(4))) int32_t *)split_off)[sc];
    const int n = ((const __attribute__((address_space(4))) int32_t *)split_off)[sc + 1] - k0;
    const int64_t out_row = (int64_t)b * rows + r;
    const uint16_t *src0 = o_part + ((int64_t)k0 * rows + r) * 512 + lane * 8;
    const int64_t split_stride = (int64_t)rows * 512;

    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = u < n ? *(const uint4 *)(src0 + u * split_stride) : make_uint4(0, 0, 0, 0);
    uint4 *dst = (uint4 *)(o_lat + out_row * 512 + lane * 8);
    if (FEW || n <= U) {
        // at most U splits: their LSEs are wave-uniform, so scalar loads
        // beside the row loads, and the max and the weights take no
        // cross-lane step (the shuffle reductions cost ~0.7 us per wave)
        const __attribute__((address_space(4))) float *lse_s = (const __attribute__((address_space(4))) float *)lse_part;
        const int ru = __builtin_amdgcn_readfirstlane(r);   // the wave's row, as a scalar
        float lk[U], m = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            lk[u] = u < n ? lse_s[(int64_t)(k0 + u) * rows + ru] : -INFINITY;
            m = fmaxf(m, lk[u]);
        }
        if (m == -INFINITY) {
            *dst = make_uint4(0, 0, 0, 0);
            if constexpr (sizeof(OutT) == 4) dst[1] = make_uint4(0, 0, 0, 0);
            if (lane == 0) lse[out_row] = -INFINITY;
            return;
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float wsum = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = lk[u] == -INFINITY ? 0.f : __expf(lk[u] - m);
            wsum += w;
            if (w == 0.f) continue;   // split without visible tokens (or past n)
            const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += w * __uint_as_float(x[e] << 16);
                acc[2 * e + 1] += w * __uint_as_float(x[e] & 0xffff0000u);
            }
        }
        store_row<OutT>(dst, acc, 1.0f / wsum);
        if (lane == 0) lse[out_row] = m + __logf(wsum);
        return;
    }
    if constexpr (FEW) return;
    // lane j holds the lse of split j (the first 64), loaded with the rows
    const float l0 = lane < n ? lse_part[(int64_t)(k0 + lane) * rows + r] : -INFINITY;
    float m = l0;
    for (int c = 64; c < n; c += 64)
        if (c + lane < n) m = fmaxf(m, lse_part[(int64_t)(k0 + c + lane) * rows + r]);
    m = wave_max(m);
    if (m == -INFINITY) {
        *dst = make_uint4(0, 0, 0, 0);
        if constexpr (sizeof(OutT) == 4) dst[1] = make_uint4(0, 0, 0, 0);
        if (lane == 0) lse[out_row] = -INFINITY;
        return;
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    for (int c = 0; c < n; c += U) {
        if (c > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = c + u < n ? *(const uint4 *)(src0 + (c + u) * split_stride) : make_uint4(0, 0, 0, 0);
        }
        // lane u of the wave holds the weight of split c + u (the lse of the
        // first 64 splits is already in l0, on lane c + u)
        float lk;
        if (c < 64) {
            lk = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * ((c + lane) & 63), __float_as_int(l0)));
            lk = lane < U && c + lane < n ? lk : -INFINITY;
        } else {
            lk = lane < U && c + lane < n ? lse_part[(int64_t)(k0 + c + lane) * rows + r] : -INFINITY;
        }
        const float wk = lk == -INFINITY ? 0.f : __expf(lk - m);
        wsum += wave_sum(wk);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), u));
            if (w == 0.f) continue;   // split without visible tokens (or past n)
            const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += w * __uint_as_float(x[e] << 16);
                acc[2 * e + 1] += w * __uint_as_float(x[e] & 0xffff0000u);
            }
        }
    }
    store_row<OutT>(dst, acc, 1.0f / wsum);
    if (lane == 0) lse[out_row] = m + __logf(wsum);
}

// The same merge for segments with many splits (long sequences): one
// workgroup per output row, its four waves taking every fourth split, eight
// partial rows in flight per wave, the four sums added through LDS.  Every
// wave finds the max over all splits' LSEs itself.
template <typename OutT>
__global__ __launch_bounds__(256) void combine512_wide_kernel(const uint16_t *__restrict__ o_part,
                                                              const float *__restrict__ lse_part,
                                                              const int32_t *__restrict__ split_off,
                                                              const int32_t *__restrict__ seq_flags,
                                                              int32_t rows, int32_t chunk_rows,
                                                              OutT *__restrict__ o_lat,
                                                              float *__restrict__ lse) {
    constexpr int U = 8;
    __shared__ float red[4][9][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = blockIdx.x, b = blockIdx.y;
    const int sc = b * ((rows + chunk_rows - 1) / chunk_rows) + r / chunk_rows;
    if (seq_flags && seq_flags[sc] == 1) return;
    const int k0 = split_off[sc], n = split_off[sc + 1] - k0;
    const int64_t out_row = (int64_t)b * rows + r;
    const uint16_t *src0 = o_part + ((int64_t)k0 * rows + r) * 512 + lane * 8;
    const int64_t split_stride = (int64_t)rows * 512;

    float m = -INFINITY;
    for (int c = lane; c < n; c += 64) m = fmaxf(m, lse_part[(int64_t)(k0 + c) * rows + r]);
    m = wave_max(m);
    uint4 *dst = (uint4 *)(o_lat + out_row * 512 + lane * 8);
    if (m == -INFINITY) {
        if (wave == 0) {
            *dst = make_uint4(0, 0, 0, 0);
            if constexpr (sizeof(OutT) == 4) dst[1] = make_uint4(0, 0, 0, 0);
            if (lane == 0) lse[out_row] = -INFINITY;
        }
        return;
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int c = wave; c < n; c += 4 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = c + 4 * u < n ? *(const uint4 *)(src0 + (c + 4 * u) * split_stride) : make_uint4(0, 0, 0, 0);
        // lane u of the wave holds the weight of split c + 4 u
        const float lk = lane < U && c + 4 * lane < n ? lse_part[(int64_t)(k0 + c + 4 * lane) * rows + r] : -INFINITY;
        const float wk = lk == -INFINITY ? 0.f : __expf(lk - m);
        wsum += wave_sum(wk);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), u));
            if (w == 0.f) continue;   // split without visible tokens (or past n)
            const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += w * __uint_as_float(x[e] << 16);
                acc[2 * e + 1] += w * __uint_as_float(x[e] & 0xffff0000u);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][e][lane] = acc[e];
    red[wave][8][lane] = wsum;
    __syncthreads();
    if (wave != 0) return;
    float ws = 0.f;
#pragma unroll
    for (int v2 = 0; v2 < 4; ++v2) ws += red[v2][8][lane];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = red[0][e][lane] + red[1][e][lane] + red[2][e][lane] + red[3][e][lane];
    const float inv = 1.0f / ws;
    if constexpr (sizeof(OutT) == 2) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pk[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
        *dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
        float4 *d4 = (float4 *)dst;
        d4[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        d4[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
    if (lane == 0) lse[out_row] = m + __logf(ws);
}

}  // namespace

// Device checks (on request only): flag[0] counts offences; the first one's
// sequence, block index (-1: the sequence length itself) and value go to
// flag[1..3].  One thread per block-table entry; a sequence's length is
// checked by its entry 0.
__global__ __launch_bounds__(256) void table_check_kernel(const int32_t *__restrict__ bt, int64_t bt_stride,
                                                          const int32_t *__restrict__ seq_lens, int32_t B,
                                                          int64_t num_blocks, int32_t *__restrict__ flag) {
    auto record = [&](int b, int j, int v) {
        if (atomicAdd(&flag[0], 1) == 0) {
            flag[1] = b;
            flag[2] = j;
            flag[3] = v;
        }
    };
    const int64_t total = (int64_t)B * bt_stride;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int b = (int)(i / bt_stride);
        const int64_t j = i - (int64_t)b * bt_stride;
        const int S = seq_lens[b];
        if (S < 0 || (int64_t)S > kBlock * bt_stride) {
            if (j == 0) record(b, -1, S);
            continue;
        }
        if (j * kBlock < S) {
            const int id = bt[i];
            if (id < 0 || id >= num_blocks) record(b, (int)j, id);
        }
    }
}

hipError_t launch_table_check(const int32_t *bt, int64_t bt_stride, const int32_t *seq_lens, int32_t B,
                              int64_t num_blocks, int32_t *flag, hipStream_t s) {
    const int64_t nb = ((int64_t)B * bt_stride + 255) / 256;
    const unsigned grid = (unsigned)(nb < 1024 ? (nb < 1 ? 1 : nb) : 1024);
    launch_timed(table_check_kernel, dim3(grid), dim3(256), 0, s, bt, bt_stride, seq_lens, B, num_blocks, flag);
    return hipGetLastError();
}

// Shader-clock probe (a measurement helper, no step of the path): every wave
// runs a dependent chain of `iters` bf16 32x32x16 MFMAs; lane 0 of each
// workgroup records the shader cycles (s_memtime) and the 100 MHz real-time
// ticks (s_memrealtime) the chain took.  The volatile asm fences keep the
// chain between the two reads.
__global__ __launch_bounds__(256) void clock_probe_kernel(int64_t *__restrict__ out, int32_t iters) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
        b[i] = (__bf16)0.0f;
    }
    f32x16 acc = {};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    asm volatile("" : "+v"(acc));
    for (int i = 0; i < iters; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    asm volatile("s_nop 15" : "+v"(acc));
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = (int64_t)(t1 - t0);
        out[2 * blockIdx.x + 1] = (int64_t)(r1 - r0);
    }
    if (iters < 0) out[0] = (int64_t)acc[threadIdx.x & 15];   // keeps the chain (never taken)
}

hipError_t launch_clock_probe(int64_t *out, int32_t wgs, int32_t iters, hipStream_t s) {
    launch_timed(clock_probe_kernel, dim3(wgs), dim3(256), 0, s, out, iters);
    return hipGetLastError();
}

hipError_t launch_gather(const uint8_t *pool, int64_t block_bytes, int64_t num_blocks, int32_t c_bytes,
                         int32_t r_bytes, bool split_rows, const int32_t *bt, int32_t bt_stride,
                         const int32_t *seq_lens, int32_t B, int32_t max_tokens, uint8_t *out,
                         hipStream_t s) {
    dim3 grid((max_tokens + 15) / 16, B);
    launch_timed(gather_kernel, grid, dim3(256), 0, s, pool, block_bytes, c_bytes, r_bytes,
                       (int32_t)split_rows, bt, bt_stride, seq_lens, max_tokens, num_blocks, out);
    return hipGetLastError();
}

hipError_t launch_combine(const void *o_part, mla_dtype_t part_dt, const float *lse_part,
                          const int32_t *split_off, const int32_t *seq_flags, int32_t B,
                          int32_t rows, int32_t chunk_rows, int32_t d_c, void *o_lat,
                          mla_dtype_t out_dt, float *lse, int32_t max_splits, hipStream_t s) {
    dim3 grid((rows + 3) / 4, B);
    if (part_dt == MLA_DT_BF16 && d_c == 512 && max_splits > kWideCombineSplits) {
        // many splits per segment: a workgroup per row, four waves over the splits
        const dim3 wide((unsigned)rows, (unsigned)B);
        if (out_dt == MLA_DT_BF16)
            launch_timed(combine512_wide_kernel<uint16_t>, wide, dim3(256), 0, s, (const uint16_t *)o_part,
                         lse_part, split_off, seq_flags, rows, chunk_rows, (uint16_t *)o_lat, lse);
        else
            launch_timed(combine512_wide_kernel<float>, wide, dim3(256), 0, s, (const uint16_t *)o_part,
                         lse_part, split_off, seq_flags, rows, chunk_rows, (float *)o_lat, lse);
    } else if (part_dt == MLA_DT_BF16 && d_c == 512 && max_splits <= 8 && (int64_t)B * rows > kCombineRound) {
        if (out_dt == MLA_DT_BF16)
            launch_timed(combine512_kernel<uint16_t, true>, grid, dim3(256), 0, s, (const uint16_t *)o_part,
                         lse_part, split_off, seq_flags, rows, chunk_rows, (uint16_t *)o_lat, lse);
        else
            launch_timed(combine512_kernel<float, true>, grid, dim3(256), 0, s, (const uint16_t *)o_part,
                         lse_part, split_off, seq_flags, rows, chunk_rows, (float *)o_lat, lse);
    } else if (part_dt == MLA_DT_BF16 && d_c == 512) {
        if (out_dt == MLA_DT_BF16)
            launch_timed(combine512_kernel<uint16_t>, grid, dim3(256), 0, s,
                               (const uint16_t *)o_part, lse_part, split_off, seq_flags, rows,
                               chunk_rows, (uint16_t *)o_lat, lse);
        else
            launch_timed(combine512_kernel<float>, grid, dim3(256), 0, s,
                               (const uint16_t *)o_part, lse_part, split_off, seq_flags, rows,
                               chunk_rows, (float *)o_lat, lse);
    } else if (part_dt == MLA_DT_BF16) {
        if (out_dt == MLA_DT_BF16)
            launch_timed((combine_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s,
                               (const uint16_t *)o_part, lse_part, split_off, seq_flags, rows, chunk_rows, d_c,
                               (uint16_t *)o_lat, lse);
        else
            launch_timed((combine_kernel<uint16_t, float>), grid, dim3(256), 0, s,
                               (const uint16_t *)o_part, lse_part, split_off, seq_flags, rows, chunk_rows, d_c,
                               (float *)o_lat, lse);
    } else {
        if (out_dt == MLA_DT_BF16)
            launch_timed((combine_kernel<float, uint16_t>), grid, dim3(256), 0, s,
                               (const float *)o_part, lse_part, split_off, seq_flags, rows, chunk_rows, d_c,
                               (uint16_t *)o_lat, lse);
        else
            launch_timed((combine_kernel<float, float>), grid, dim3(256), 0, s,
                               (const float *)o_part, lse_part, split_off, seq_flags, rows, chunk_rows, d_c,
                               (float *)o_lat, lse);
    }
    return hipGetLastError();
}

}  // namespace mla

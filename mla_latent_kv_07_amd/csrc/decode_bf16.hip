// Absorbed MLA decode on MFMA for the DeepSeek-V2 shape: bf16 cache rows of
// [c (512) | k^R (64)], bf16 queries, fp32 accumulation.
//
// Workgroup = 4 waves = 128 query rows (heads x query tokens) of one
// sequence; wave w owns rows 32w..32w+31 for the whole work item and keeps
//   - its queries as MFMA B fragments in VGPRs (32 rows x 576, 144 VGPRs),
//   - O^T, the fp32 latent output sum (512 x 32 rows, 256 accumulators).
// The cached tokens stream through LDS one 64-token paged block at a time
// (the block is the tile), double-buffered with asynchronous direct-to-LDS
// loads; every tile is read from HBM once per workgroup and from LDS by all
// four waves:
//   score  S^T[64 tok x 32 rows] = K_tile[64 x 576] . Q^T        (MFMA 32x32x16)
//   p      = exp2(S*scale*log2e - m) with a lazily raised running max m
//   value  O^T[512 x 32] += V_tile^T[512 x 64] . P^T[64 x 32]    (MFMA 32x32x16)
// where V_tile is the c part of the same LDS rows, read transposed with
// ds_read_b64_tr_b16.  The score accumulator layout already is the value
// contraction's B operand, up to a fixed permutation of the 16 tokens of a
// k-step that both operands share, so P never moves between lanes.
//
// Score content + RoPE decomposition: huny.dev "DeepSeek MLA 해부" §2-3;
// W^UK absorption (the q_lat operand): §3-1; latent value sum: §3-2;
// MQA form over one latent head: vLLM MLA page, "MLA의 MQA 디코딩 경로".
#include "common.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int ROW_BYTES = D * 2;                 // 1152
constexpr int TILE_BYTES = kBlock * ROW_BYTES;   // 73728
constexpr int KSTEPS = D / 16;                   // 36 score k-steps
constexpr int MBLOCKS = DC / 32;                 // 16 value M-blocks

// 16-byte chunk swizzle inside each 128-byte group of a row: chunk c of token
// t is stored at chunk c ^ sigma(t).  sigma is a bijection on any 8 aligned
// consecutive tokens (conflict-free score reads: 8 lanes = 8 tokens, same
// chunk) and sigma>>1 is a bijection on any 4 aligned consecutive tokens
// (conflict-free transposed reads: 4 tokens x 2 chunks per 16 lanes).
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// Per-lane source offsets of the asynchronous tile copy.  Wave w copies LDS
// bytes [w*18K, (w+1)*18K) in 1 KiB steps; the lane whose LDS slot is
// (token t, stored chunk pc) reads global chunk pc ^ sigma(t) of token t.
// 9 KiB is exactly 8 rows, so steps k and k+9 differ by 9216 bytes and only
// nine offsets per lane are distinct.
struct TileLoadOffsets {
    int off[9];
};

__device__ __forceinline__ TileLoadOffsets tile_load_offsets(int wave, int lane) {
    TileLoadOffsets o;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int p = (wave * 18 + k) * 1024 + lane * 16;
        const int t = p / ROW_BYTES;
        const int pc = (p - t * ROW_BYTES) >> 4;
        o.off[k] = t * ROW_BYTES + ((pc ^ swz(t)) << 4);
    }
    return o;
}

// Issue the asynchronous copy of one 64-token block into an LDS tile.
__device__ __forceinline__ void issue_tile_load(const uint8_t *blk_base, lds_u8 *tile, int wave,
                                                const TileLoadOffsets &o) {
#pragma unroll
    for (int k = 0; k < 18; ++k) {
        const int region = (wave * 18 + k) * 1024;
        __builtin_amdgcn_global_load_lds((const void *)(blk_base + o.off[k % 9] + (k / 9) * 9216),
                                         (__attribute__((address_space(3))) void *)(tile + region),
                                         16, 0, 0);
    }
}

__device__ __forceinline__ float max_across_halves(float v) {
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeArgs a) {
    const int64_t num_blocks = a.num_pool_blocks;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * TILE_BYTES];
    lds_u8 *tiles = (lds_u8 *)smem;

    // workgroup -> (item, row chunk); the row chunks of one item sit 8 apart so
    // that they land on the same XCD and share the tile through its L2.
    const int rc = a.row_chunks;
    const int grp = blockIdx.x / (8 * rc), within = blockIdx.x % (8 * rc);
    const int chunk = within / 8;
    const int item = grp * 8 + within % 8;
    if (item >= a.num_items) return;
    const int32_t *it = a.plan + plan_items_off() + 4 * item;
    const int b = it[0], blk0 = it[1], blk1 = it[2], slot = it[3];
    const int ntiles = blk1 - blk0;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5;           // lane half
    const int ln = lane & 31;
    const int row = chunk * kRowsPerChunk + wave * 32 + ln;   // query row in the sequence
    const bool row_ok = row < a.rows;
    const int S = a.seq_lens[b];
    const int lim = row_ok ? S - a.q_len + row / a.n_h + 1 : 0;   // visible positions < lim
    const int64_t grow = (int64_t)b * a.rows + row;

    const uint8_t *pool = (const uint8_t *)a.pool;
    const int32_t *bt = a.block_table + (int64_t)b * a.bt_stride;
    auto block_ptr = [&](int blk) {
        int64_t id = bt[blk];
        id = id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
        return pool + id * (int64_t)TILE_BYTES;
    };

    const TileLoadOffsets tlo = tile_load_offsets(wave, lane);
    // first tile in flight before the query loads
    issue_tile_load(block_ptr(blk0), tiles, wave, tlo);

    // queries as B fragments: lane (row ln, half g) holds features 16ks+8g..+7
    bf16x8 qf[KSTEPS];
    {
        // rows past the end load row 0's queries; their scores are all masked
        const int64_t qrow = row_ok ? grow : (int64_t)b * a.rows;
        const bf16x8 *ql = (const bf16x8 *)((const uint16_t *)a.q_lat + qrow * DC);
        const bf16x8 *qr = (const bf16x8 *)((const uint16_t *)a.q_rope + qrow * DR);
#pragma unroll
        for (int ks = 0; ks < DC / 16; ++ks) qf[ks] = ql[2 * ks + g];
#pragma unroll
        for (int ks = 0; ks < DR / 16; ++ks) qf[DC / 16 + ks] = qr[2 * ks + g];
    }

    f32x16 oacc[MBLOCKS];
#pragma unroll
    for (int mb = 0; mb < MBLOCKS; ++mb) oacc[mb] = f32x16{};
    float m_run = -INFINITY;   // reference max (log2 units), lazily raised
    float l_lane = 0.f;        // this lane's share of the softmax denominator

    // Per-lane LDS read bases; every read below is base + a compile-time
    // offset.  Score reads: token ln (+32h), chunk 2ks+g, stored at chunk
    // (2ks+g) ^ sigma(ln); the XOR only touches the low 3 bits, so the bases
    // depend on ks & 3 and ks >> 2 adds 128 bytes.
    int kbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kbase[j] = ln * ROW_BYTES + (((2 * j + g) ^ swz(ln)) << 4);
    // Transposed value reads (ds_read_b64_tr_b16: lane i of each 16-lane group
    // receives element i%4 of the 8 bytes read by lanes 4s + i/4, s = 0..3):
    // lane (group G, index w) reads token 4(G/2) + w/4 of the k-step and the
    // 4 features 32mb + 16(G%2) + 4(w%4), i.e. chunk 4mb + 2(G%2) + (w%4)/2,
    // byte 8(w%2); both operands then agree on the token order of a k-step.
    const int grp16 = lane >> 4, w16 = lane & 15;
    const int tr_tok = 4 * (grp16 >> 1) + (w16 >> 2);
    const int tr_chunk = 2 * (grp16 & 1) + ((w16 & 3) >> 1);
    int vbase[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
        vbase[e] = tr_tok * ROW_BYTES + (((4 * e + tr_chunk) ^ swz(tr_tok)) << 4) + (w16 & 1) * 8;

    for (int ti = 0; ti < ntiles; ++ti) {
        lds_u8 *tile = tiles + (ti & 1) * TILE_BYTES;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's copies landed
        __syncthreads();                      // ... and everyone's; other buffer free
        const int p0 = (blk0 + ti) * kBlock;
        const int valid = S - p0;             // rows of this block holding tokens
        if (valid < kBlock) {
            // zero the tail rows so that P = 0 never meets NaN/garbage values
            for (int off = valid * ROW_BYTES + threadIdx.x * 16; off < TILE_BYTES; off += 256 * 16)
                *(uint4 *)(tile + off) = make_uint4(0, 0, 0, 0);
            __syncthreads();
        }
        if (ti + 1 < ntiles)
            issue_tile_load(block_ptr(blk0 + ti + 1), tiles + ((ti + 1) & 1) * TILE_BYTES, wave, tlo);

#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // ---- score: S^T[32 tokens x 32 rows] for tokens 32h..32h+31
            f32x16 sacc = {};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const bf16x8 kf = *(const bf16x8 *)(tile + kbase[ks & 3] + 128 * (ks >> 2) + h * 32 * ROW_BYTES);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc, 0, 0, 0);
            }
            // ---- online softmax; lane holds row ln, tokens 8(r/4)+4g+r%4
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int p = p0 + 32 * h + 8 * (r >> 2) + 4 * g + (r & 3);
                const float s = p < lim ? sacc[r] * a.scale_log2 : -INFINITY;
                sacc[r] = s;
                mx = fmaxf(mx, s);
            }
            mx = max_across_halves(mx);
            // raise the reference max only when a score exceeds it by 2^8
            const bool raise = mx > m_run + 8.0f;
            const float m_new = raise ? mx : m_run;
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            if (__ballot(raise && m_run != -INFINITY)) {
                // rare: keep the accumulators in AGPRs and rescale them one
                // block at a time (a plain multiply makes the compiler move
                // all 256 of them into VGPRs)
#pragma unroll
                for (int mb = 0; mb < MBLOCKS; ++mb) {
                    asm volatile("" : "+a"(oacc[mb]));
                    oacc[mb] *= alpha;
                    asm volatile("" : "+a"(oacc[mb]));
                }
            }
            l_lane *= alpha;
            m_run = m_new;
            const float m_ref = m_run == -INFINITY ? 0.f : m_run;
            bf16x8 pf[2];
            float psum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(sacc[r] - m_ref);
                psum += pv;
                pf[r >> 3][r & 7] = (__bf16)pv;
            }
            l_lane += psum;
            // ---- value: O^T[512 x 32] += V^T[512 x 16 tok] . P^T[16 tok x 32]
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int tok_off = (32 * h + 16 * s2) * ROW_BYTES;
#pragma unroll
                for (int mb = 0; mb < MBLOCKS; ++mb) {
                    lds_u8 *vp = tile + vbase[mb & 1] + tok_off + 128 * (mb >> 1);
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4 *)vp);
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4 *)(vp + 8 * ROW_BYTES));
                    bf16x8 vf;
                    vf.lo = __builtin_bit_cast(bf16x4, lo);
                    vf.hi = __builtin_bit_cast(bf16x4, hi);
                    oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s2], oacc[mb], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: lane (row ln, half g) holds features 32mb + 8(r/4) + 4g + (r%4)
    const float l_tot = l_lane + __shfl_xor(l_lane, 32, 64);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    if (!row_ok) return;
    if (slot < 0) {
        uint16_t *dst = (uint16_t *)a.o_lat + grow * DC;
#pragma unroll
        for (int mb = 0; mb < MBLOCKS; ++mb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = 32 * mb + 8 * q + 4 * g;
                bf16x4 v;
                v[0] = (__bf16)(oacc[mb][4 * q + 0] * inv);
                v[1] = (__bf16)(oacc[mb][4 * q + 1] * inv);
                v[2] = (__bf16)(oacc[mb][4 * q + 2] * inv);
                v[3] = (__bf16)(oacc[mb][4 * q + 3] * inv);
                *(bf16x4 *)(dst + f) = v;
            }
        }
        if (g == 0) a.lse[grow] = lse_v;
    } else {
        float *dst = a.o_part + ((int64_t)slot * a.rows + row) * DC;
#pragma unroll
        for (int mb = 0; mb < MBLOCKS; ++mb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = 32 * mb + 8 * q + 4 * g;
                *(float4 *)(dst + f) = make_float4(oacc[mb][4 * q] * inv, oacc[mb][4 * q + 1] * inv,
                                                   oacc[mb][4 * q + 2] * inv, oacc[mb][4 * q + 3] * inv);
            }
        }
        if (g == 0) a.lse_part[(int64_t)slot * a.rows + row] = lse_v;
    }
}

}  // namespace

hipError_t launch_decode_bf16_mfma(const DecodeArgs &a, hipStream_t s) {
    const int groups = (a.num_items + 7) / 8;
    dim3 grid((unsigned)groups * 8 * a.row_chunks);
    hipLaunchKernelGGL(decode_bf16_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_fp8_mfma(const DecodeArgs &a, hipStream_t s) {
    // fp8 MFMA path not instantiated yet: fall back to the generic kernel
    return launch_decode_generic(a, s);
}

}  // namespace mla

// Absorbed MLA decode on MFMA for the DeepSeek-V2 shape: bf16 cache rows of
// [c (512) | k^R (64)], bf16 queries, fp32 accumulation.
//
// Workgroup = 4 waves = 128 query rows (heads x query tokens) of one
// sequence; wave w owns rows 32w..32w+31 for the whole work item and keeps
//   - the latent part of its queries as MFMA B fragments in VGPRs
//     (32 rows x 512, 128 VGPRs); the rotary part sits in LDS (16 KB),
//   - O^T, the fp32 latent output sum (512 x 32 rows, 256 accumulators).
// Cached tokens stream through LDS in 32-token stages (half a paged block),
// four stage buffers deep, filled by asynchronous direct-to-LDS loads that
// run two stages ahead of the compute.  Every cached byte is read
// from HBM once per workgroup and from LDS by all four waves:
//   score  S^T[32 tok x 32 rows] = K[32 x 576] . Q^T           (MFMA 32x32x16)
//   p      = exp2(S*scale*log2e - m) with a lazily raised reference max m
//   value  O^T[512 x 32] += V^T[512 x 32] . P^T[32 x 32]       (MFMA 32x32x16)
// V is the latent part of the same LDS rows, read transposed with
// ds_read_b64_tr_b16; the score accumulator layout is already the value
// MFMA's B operand, up to a fixed permutation of the 16 tokens of a k-step
// that both operands share, so P never moves between lanes.
//
// Score = content + rotary part: huny.dev "DeepSeek MLA 해부" §2-3
// decomposition; absorbed query against the cached latent: §3-1; latent
// value sum: §3-2; one shared latent "head" (MQA form): vLLM MLA page,
// "MLA의 MQA 디코딩 경로".
#include <type_traits>

#include "common.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int DC = 512, DR = 64;
constexpr int ROW_BYTES = (DC + DR) * 2;        // 1152 bytes per cached token in HBM
constexpr int CB = DC * 2;                      // 1024: latent bytes of a token
constexpr int RB = DR * 2;                      // 128: rotary bytes of a token
constexpr int HALF = 32;                        // tokens per pipeline stage
constexpr int STAGE_BYTES = HALF * (CB + RB);   // 36864
constexpr int NSTAGE = 4;
constexpr int KC = DC / 16;                     // 32 latent score k-steps
constexpr int MBLOCKS = DC / 32;                // 16 value M-blocks
constexpr int O_PITCH = CB + 16;                // epilogue staging row pitch (bytes)
constexpr int PF = 4;                           // LDS fragment prefetch depth (MFMAs)

// LDS layout of a stage: latent rows [32][1024 B] then rotary rows [32][128 B].
// 16-byte chunk c of latent row t is stored at chunk c ^ sc(t) (the XOR stays
// inside the 16-chunk / 256-byte group), rotary chunk c of row t at c ^ sr(t).
// With 64 four-byte banks (256 B per cycle):
//  - score reads (16 lanes = 16 consecutive tokens, one chunk) need sc to be
//    a bijection on t mod 16;
//  - transposed value reads (32 lanes = 4 consecutive tokens x 4 chunks of a
//    4-chunk group) need sc >> 2 to be a bijection on t mod 4;
//  - rotary reads (16 tokens, one chunk, 128-byte rows) need (t & 1, sr(t))
//    distinct over 16 tokens.
__device__ __forceinline__ int sc(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int sr(int t) { return (t >> 1) & 7; }

// One asynchronous 1 KiB copy: global_load_lds_dwordx4 writes lane i's 16
// bytes to LDS at M0 + 16 i.  Issued as inline asm so that the compiler's
// wait-count pass does not see an LDS writer in flight (it would otherwise
// drain every LDS read with lgkmcnt(0)); completion is awaited explicitly
// (vmcnt + barrier) before a stage is read.  VMEM loads complete in order, so
// the compiler's own vmcnt waits stay correct: unseen extra loads can only
// make them over-wait.
__device__ __forceinline__ void dma16(lds_u8 *lds_dst, uint32_t voff, const uint8_t *src) {
    const uint32_t lds = (uint32_t)(uintptr_t)lds_dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(src)
                 : "memory", "m0");
}

constexpr int DMA_PER_STAGE = 9;   // per wave: 8 latent rows + 1 KiB of rotary rows

// Copy one stage (32 tokens starting at token tok0 of the block at blk_base).
// Wave w copies latent rows 8w..8w+7 (one instruction each) and the rotary
// rows of the same 8 tokens (one instruction).
__device__ __forceinline__ void issue_stage(const uint8_t *blk_base, int tok0, lds_u8 *stage,
                                            int wave, int lane) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int t = wave * 8 + k;
        dma16(stage + t * CB, (uint32_t)((tok0 + t) * ROW_BYTES + ((lane ^ sc(t)) << 4)), blk_base);
    }
    const int t = wave * 8 + (lane >> 3);
    dma16(stage + HALF * CB + wave * 8 * RB,
          (uint32_t)((tok0 + t) * ROW_BYTES + CB + (((lane & 7) ^ sr(t)) << 4)), blk_base);
}

// Loads of wave-uniform values (plan, block table, lengths) through the
// constant address space become scalar loads, which never wait on the
// vector-memory counter of the asynchronous stage copies.
__device__ __forceinline__ int32_t sload(const int32_t *p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem_[NSTAGE * STAGE_BYTES];
    lds_u8 *smem = (lds_u8 *)smem_;

    // workgroup -> (item, row chunk).  Workgroups are dealt to the 8 XCDs
    // round robin (XCD = blockIdx % 8); XCD x takes the contiguous run
    // x*G .. x*G+G-1 of the (item, chunk) units, so the splits of a sequence
    // and the row chunks of an item share one L2: the queries of a sequence
    // and each streamed block are fetched from HBM once.
    const int rc = a.row_chunks;
    const int G = gridDim.x / 8;
    const int unit = (blockIdx.x & 7) * G + (blockIdx.x >> 3);
    const int item = unit / rc, chunk = unit % rc;
    if (item >= a.num_items) return;
    const int64_t io = plan_items_off() + 4 * item;
    const int b = sload(a.plan, io), blk0 = sload(a.plan, io + 1), blk1 = sload(a.plan, io + 2),
              slot = sload(a.plan, io + 3);
    const int S = sload(a.seq_lens, b);
    const int nst = 2 * (blk1 - blk0);   // 32-token stages in this item
    // a stage holds tokens only if its first position is < S (the plan covers
    // ceil(S/64) blocks, so the second half of the last block may be empty)
    const int p_first = blk0 * kBlock;
    const int nst_live = min(nst, (S - p_first + HALF - 1) / HALF);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5;           // lane half
    const int ln = lane & 31;
    const int wrow = wave * 32 + ln;   // row inside the chunk
    const int row = chunk * kRowsPerChunk + wrow;
    const bool row_ok = row < a.rows;
    const int lim = row_ok ? S - a.q_len + row / a.n_h + 1 : 0;   // visible positions < lim
    const int64_t grow = (int64_t)b * a.rows + row;

    const uint8_t *pool = (const uint8_t *)a.pool;
    const int64_t bt_row = (int64_t)b * a.bt_stride;
    const int64_t num_blocks = a.num_pool_blocks;
    auto stage_src = [&](int st) {
        int64_t id = sload(a.block_table, bt_row + blk0 + (st >> 1));
        id = id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
        return pool + id * (int64_t)(kBlock * ROW_BYTES);
    };
    auto stage_buf = [&](int st) { return smem + (st & (NSTAGE - 1)) * STAGE_BYTES; };

    // stage 0 in flight, then the queries, then stage 1
    issue_stage(stage_src(0), 0, stage_buf(0), wave, lane);

    constexpr int KS = KC + DR / 16;   // 36 score k-steps: 32 latent + 4 rotary
    bf16x8 qf[KS];
    {
        // rows past the end load row 0's queries; their scores are all masked
        const int64_t qrow = row_ok ? grow : (int64_t)b * a.rows;
        const bf16x8 *ql = (const bf16x8 *)((const uint16_t *)a.q_lat + qrow * DC);
        const bf16x8 *qr = (const bf16x8 *)((const uint16_t *)a.q_rope + qrow * DR);
#pragma unroll
        for (int ks = 0; ks < KC; ++ks) qf[ks] = ql[2 * ks + g];
#pragma unroll
        for (int ks = 0; ks < DR / 16; ++ks) qf[KC + ks] = qr[2 * ks + g];
        // Consume the query registers here so that the compiler completes
        // these loads now (alongside stage 0's copy); otherwise it places
        // vmcnt waits on them inside the stage loop, where the count would
        // also drain the stage copies it does not know about.
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    }
    if (nst_live > 1) issue_stage(stage_src(1), HALF, stage_buf(1), wave, lane);

    f32x16 oacc[MBLOCKS];
#pragma unroll
    for (int mb = 0; mb < MBLOCKS; ++mb) oacc[mb] = f32x16{};
    float m_run = -INFINITY;   // reference max (log2 units), lazily raised
    float l_lane = 0.f;        // this lane's share of the softmax denominator

    // Per-lane LDS read bases; every read is base + stage offset + a
    // compile-time immediate.
    // Score, latent chunk 2ks+g of token ln: (2ks+g) ^ sc(ln) = 2ks ^ x with
    // x = g ^ sc(ln), so the base depends on ks & 7 and ks >> 3 adds 256 B.
    const int x = g ^ sc(ln);
    int kbase[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kbase[j] = ln * CB + (((2 * j) ^ x) << 4);
    const int rrow = HALF * CB + ln * RB, rx = g ^ sr(ln);        // rotary chunk 2j+g of token ln
    // Transposed value reads (ds_read_b64_tr_b16: lane i of each 16-lane group
    // receives element i%4 of the 8 bytes read by lanes 4s + i/4, s = 0..3).
    // Value k-step s2 takes the tokens {8 s2 + 4g + (0..3)} and the same +16
    // (score accumulator entries r = 4 s2 + (0..3) and 8 + 4 s2 + (0..3));
    // lane (group G, index w) reads token 8 s2 + 4(G/2) + w/4 (+16 for the
    // upper half) and features 32mb + 16(G%2) + 4(w%4): chunk
    // 4mb + 2(G%2) + (w%4)/2, byte 8(w%2).  sc() repeats every 16 tokens, so
    // the upper half is the lower address + 16 KiB.  Bases depend on mb & 3
    // (the XOR touches the low 4 chunk bits); mb >> 2 adds 256 B.
    const int grp16 = lane >> 4, w16 = lane & 15;
    const int tr_tok = 4 * (grp16 >> 1) + (w16 >> 2);
    const int tr_chunk = 2 * (grp16 & 1) + ((w16 & 3) >> 1);
    int vbase[2][4];   // [k-step][mb & 3]
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vbase[s2][e] = (8 * s2 + tr_tok) * CB + (((4 * e + tr_chunk) ^ sc(8 * s2 + tr_tok)) << 4) +
                           (w16 & 1) * 8;

    // value MFMAs of one stage: O^T[512 x 32] += V^T[512 x 32 tok] . P^T[32 tok x 32]
    // as two 16-token k-steps; transposed V fragments PF MFMAs ahead (LDS
    // latency under load is ~4 MFMA issue slots).
    auto value_stage = [&](lds_u8 *vst, const bf16x8 (&pv)[2], auto vpat_tag) {
        constexpr int vpat = decltype(vpat_tag)::value;
        auto vld = [&](int i) {
            const int s2 = i / MBLOCKS, mb = i % MBLOCKS;
            lds_u8 *lo = vst + vbase[s2][mb & 3] + 256 * (mb >> 2);
            lds_u8 *hi = lo + 16 * CB;
            bf16x8 vf;
            vf.lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)lo));
            vf.hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)hi));
            return vf;
        };
        bf16x8 vb[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) vb[j] = vld(j);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, vpat);
#pragma unroll
        for (int i = 0; i < 2 * MBLOCKS; ++i) {
            oacc[i % MBLOCKS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % PF], pv[i / MBLOCKS],
                                                                        oacc[i % MBLOCKS], 0, 0, 0);
            if (i + PF < 2 * MBLOCKS) vb[i % PF] = vld(i + PF);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, vpat);
            if (i + PF < 2 * MBLOCKS) __builtin_amdgcn_sched_group_barrier(0x100, 2, vpat);
        }
    };

    // One stage: wait for its copy, score it, softmax, value MFMAs.
    auto stage = [&](int st) {
        // stage st landed (stage st+1 may still be in flight) ...
        if (st + 1 < nst_live)
            asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // ... for every wave; stage st-2's buffer is free
        lds_u8 *stg = stage_buf(st);
        const int p0 = p_first + st * HALF;
        const int valid = S - p0;   // >= 1 for a live stage
        if (valid < HALF) {
            // zero the rows past the sequence end so that P = 0 never meets
            // NaN or stale data in the value MFMA
            for (int off = valid * CB + threadIdx.x * 16; off < HALF * CB; off += 256 * 16)
                *(uint4 *)(stg + off) = make_uint4(0, 0, 0, 0);
            for (int off = HALF * CB + valid * RB + threadIdx.x * 16; off < STAGE_BYTES; off += 256 * 16)
                *(uint4 *)(stg + off) = make_uint4(0, 0, 0, 0);
            __syncthreads();
        }
        if (st + 2 < nst_live)
            issue_stage(stage_src(st + 2), ((st + 2) & 1) * HALF, stage_buf(st + 2), wave, lane);

        // ---- score: S^T[32 tokens x 32 rows]; K fragments two k-steps ahead.
        // The score MFMAs are written as inline asm with VGPR operands: the
        // compiler gives every MFMA builtin an AGPR accumulator, and the 256
        // AGPRs are all taken by O^T.  Hazards the compiler cannot see are
        // covered by hand: the chain accumulates back to back into the same
        // registers (no wait states needed); s_nop 1 before each MFMA covers
        // a VALU write of an operand; s_nop 15 after the last one covers the
        // MFMA-result -> VALU-read latency (>= 12 wait states for 8 passes).
        f32x16 sacc;
        auto kld = [&](int ks) {
            return ks < KC ? *(const bf16x8 *)(stg + kbase[ks & 7] + 256 * (ks >> 3))
                           : *(const bf16x8 *)(stg + rrow + (((2 * ((ks - KC) & 3)) ^ rx) << 4));
        };
        bf16x8 kb[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) kb[j] = kld(j);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // the first MFMA writes the accumulator while reading its operands:
            // early clobber keeps them apart
            if (ks == 0)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                             : "=&v"(sacc) : "v"(kb[0]), "v"(qf[0]));
            else
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+v"(sacc) : "v"(kb[ks % PF]), "v"(qf[ks]));
            if (ks + PF < KS) kb[ks % PF] = kld(ks + PF);
        }
        asm volatile("s_nop 15" : "+v"(sacc));

        // ---- online softmax (lane holds row ln, tokens 8(r/4)+4g+r%4)
        const int lim_rel = lim - p0 - 4 * g;   // token offset t is visible iff t < lim_rel
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float sv = (8 * (r >> 2) + (r & 3)) < lim_rel ? sacc[r] : -INFINITY;
            sacc[r] = sv;
            mx = fmaxf(mx, sv);
        }
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx),
                                                             false, false);
            mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));   // max over lanes l, l^32
        }
        mx *= a.scale_log2;
        // raise the reference max only when a score exceeds it by 2^8
        const bool raise = mx > m_run + 8.0f;
        const float m_new = raise ? mx : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        bf16x8 pcur[2];
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], a.scale_log2, -m_ref));
            psum += pv;
            pcur[(r >> 2) & 1][((r >> 3) << 2) | (r & 3)] = (__bf16)pv;
        }
        if (__ballot(raise && m_run != -INFINITY)) {
            // rare: the value sum so far (through stage st-1) moves to the new
            // reference; accumulators stay in AGPRs and are rescaled block by
            // block (a plain multiply makes the compiler move all 256 to VGPRs)
#pragma unroll
            for (int mb = 0; mb < MBLOCKS; ++mb) {
                asm volatile("" : "+a"(oacc[mb]));
                oacc[mb] *= alpha;
                asm volatile("" : "+a"(oacc[mb]));
            }
        }
        l_lane = l_lane * alpha + psum;
        m_run = m_new;
        value_stage(stg, pcur, std::integral_constant<int, 1>{});
    };

    for (int st = 0; st < nst_live; ++st) stage(st);

    // ---- epilogue: O / l as bf16 rows staged through LDS, then 1 KiB
    // coalesced row stores (final o_lat, or this split's bf16 partial).
    float l_tot;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(l_lane), __float_as_int(l_lane),
                                                         false, false);
        l_tot = __int_as_float(sw[0]) + __int_as_float(sw[1]);   // sum over lanes l, l^32
    }
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    __syncthreads();   // every wave is done with the stage buffers
    lds_u8 *orow = smem + wrow * O_PITCH;
#pragma unroll
    for (int mb = 0; mb < MBLOCKS; ++mb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(oacc[mb][4 * q + e] * inv);
            *(bf16x4 *)(orow + (32 * mb + 8 * q + 4 * g) * 2) = v;
        }
    }
    // each wave stores its own 32 rows (no cross-wave dependency)
    uint8_t *dst_base = slot < 0 ? (uint8_t *)a.o_lat + ((int64_t)b * a.rows) * CB
                                 : (uint8_t *)a.o_part + ((int64_t)slot * a.rows) * CB;
    const int row0 = chunk * kRowsPerChunk + wave * 32;
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
        if (row0 + r >= a.rows) break;
        const uint4 v = *(const uint4 *)(smem + (wave * 32 + r) * O_PITCH + lane * 16);
        *(uint4 *)(dst_base + (int64_t)(row0 + r) * CB + lane * 16) = v;
    }
    if (row_ok && g == 0) {
        if (slot < 0)
            a.lse[grow] = lse_v;
        else
            a.lse_part[(int64_t)slot * a.rows + row] = lse_v;
    }
}

}  // namespace

hipError_t launch_decode_bf16_mfma(const DecodeArgs &a, hipStream_t s) {
    // a multiple of 8 workgroups, one per (item, row chunk) plus padding
    const int units = a.num_items * a.row_chunks;
    dim3 grid((unsigned)((units + 7) / 8) * 8);
    hipLaunchKernelGGL(decode_bf16_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_fp8_mfma(const DecodeArgs &a, hipStream_t s) {
    // fp8 MFMA path not instantiated yet: the generic kernel serves fp8 caches
    return launch_decode_generic(a, s);
}

}  // namespace mla

// Absorbed MLA decode on the 8-bit matrix cores for a paged cache of e4m3
// latents (one fp32 scale per 64-token block) with bf16 rotary keys, bf16
// queries and fp32 accumulation.
//
// The cached codes go into the MFMAs as stored (v_mfma_scale_f32_32x32x64_f8f6f4):
//   score  s = sigma_blk sigma_q (q8 . c8) + q^R . k^R
//   value  O += sigma_blk (P8 . c8)
// with
//   q8  the absorbed query of a row as two e4m3 terms, q~ ~= sigma_q (h + l/16),
//       sigma_q = max|q~| / 448 over the row (h alone leaves ~8 % error in
//       o_lat on N(0,1) data; with h + l/16 the query adds ~0.2 %);
//   P8  y = p 2^5 mant(sigma_blk) as two e4m3 terms, y ~= P_h + P_l (P_l the
//       unscaled residual y - P_h, within 2^-10 of it), with
//       sigma_blk = mant 2^e, mant in [1, 2): the value MFMA applies 2^(e-5)
//       through its E8M0 A-operand scale, so O gathers sum_p p c_p up to the
//       rounding of P (one term alone leaves ~4 % error in o_lat on N(0,1)
//       data; two leave ~0.3 %, the exact bf16 path's level).
// The rotary part stays on bf16 MFMAs: the rotary key is kept in 16 bits.
// (Paged fp8 latent cache with a per-block dynamic scale and a 16-bit
// rotary key: huny.dev "DeepSeek MLA 해부" §6, FP8 item; vLLM MLA page,
// "FP8 MLA 지원".  The pages fix the storage, not the arithmetic of the
// attention; quantising q~ and P for the 8-bit MFMAs is this kernel's
// choice.)
//
// Workgroup = 4 waves = 128 query rows of one sequence, as in the 16-bit
// kernel; wave w owns rows 32w..32w+31 and keeps
//   - h and l codes as 8-bit B fragments (2 x 64 VGPRs) and q^R as bf16 B
//     fragments (16 VGPRs),
//   - O^T, the fp32 latent output sum (512 x 32 rows, 256 accumulators).
// A stage is one paged block (64 tokens, 40,960 B), copied to LDS by
// asynchronous direct-to-LDS loads two stages ahead (three stage buffers):
//   score  S^T[32 tok x 32 rows] for 2 token tiles: 8 k-chunks x {h, l}
//          8-bit MFMAs (32x32x64) + 4 bf16 rotary MFMAs (32x32x16) per tile
//   p      exp2(S scale log2e - m), m raised lazily (p <= 4)
//   value  O^T[512 x 32] += V^T[512 x 64 tok] . P^T[64 tok x 32]: 16 x {P_h, P_l}
//          MFMAs on the same V fragments
// The 8-bit MFMA contracts over 64 k values: lane l holds row l % 32 of A
// (column of B) and 32 of them; any assignment of (lane half, byte) to k
// that A and B share is valid.  For the score, byte b of half g is latent
// feature 64 kc + 32 g + b.  For the value, byte b of half g is the token
// that score tile b / 16 keeps in accumulator b % 16 of half g, so the P
// codes of a lane are its own score entries and never move between lanes.
#include "common.hpp"
#include "lds_copy.hpp"

namespace mla {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int DC = 512, DR = 64;
constexpr int BT = kBlock;                   // 64 tokens per stage: one paged block
constexpr int LAT = BT * DC;                 // 32,768: the block's e4m3 latent codes
constexpr int RB = DR * 2;                   // 128: bf16 rotary key bytes of a token
constexpr int STAGE = LAT + BT * RB;         // 40,960: one block, as stored in HBM
constexpr int NST = 3;                       // stage buffers
constexpr int KC = DC / 64;                  // 8 latent k-chunks of the score
constexpr int KR = DR / 16;                  // 4 rotary k-steps
constexpr int MBLK = DC / 32;                // 16 value M-blocks
constexpr int PFV = 4;                       // value-fragment prefetch depth (M-blocks)
constexpr int RING_OFF = NST * STAGE;        // 4 block-scale slots, one per stage in flight
constexpr int RING_SLOT = 256;               // a slot: the scale as loaded by 64 lanes
constexpr int O_PITCH = 2 * DC + 16;         // epilogue staging row pitch (bytes)
// each row's visibility limit, read by the stage loop from LDS: held in a
// register it was spilled, and its reload waited on the stage copies in flight
constexpr int LIM_OFF = RING_OFF + 4 * RING_SLOT;
constexpr int LDS_BYTES = LIM_OFF + 4 * 128 > 128 * O_PITCH ? LIM_OFF + 4 * 128 : 128 * O_PITCH;
constexpr int COPIES = 11;                   // per wave and stage: 8 latent KiB, 2 rotary KiB, the scale
constexpr int E8M0_ONE = 127;                // E8M0 scale 2^0
constexpr int E8M0_16TH = 123;               // 2^-4: the l term of the query
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(COPIES <= 2 * KC, "two copy parts per score k-chunk");
static_assert(COPIES == 11, "the stage loop waits with vmcnt(11): one stage's copies per wave");
static_assert(STAGE % 8192 == 0, "stage offsets leave the XOR-ed address bits 4-8 clear");

// LDS layout of a stage (token t = 0..63 of the block):
//   latent  [64][512 B]: 16-byte chunk c of token t at chunk c ^ swz(t);
//   rotary  at LAT, token-major: token t's 128 B at (t >> 3) 1024 + (t & 7) 128,
//           its 16-byte chunk c in slot c ^ rot_swz(t).
// swz rotates the 4 low bits of t by two.  A score read (16 lanes = 16
// consecutive tokens, one chunk) then hits 16 distinct 16-byte bank groups,
// and so does a transposed value read (32 lanes = 8 tokens x 2 chunks): its
// tokens are 8 b + 4 g + c (b < 2, c < 4) with g fixed, whose swz values
// 4 c + 2 b + g differ in bits 1-3, and the two chunks 2 mb, 2 mb + 1 differ
// in bit 0.  Every read address is then a per-lane base XOR a compile-time
// constant in bits 4-8 plus compile-time multiples of 8 KiB.
__device__ __forceinline__ constexpr int swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
// Rotary slot swizzle (the 16-bit kernel's): over one 16-token score read the
// slots land in 16 distinct bank groups, and a copy's 16-lane quarter reads
// 2 cache lines.
__device__ __forceinline__ constexpr int rot_swz(int t) { return ((t & 7) >> 1) ^ (((t >> 3) & 1) << 2); }

// acc (=|+=) A . B on the 8-bit matrix core, E8M0 scales sa (A) and sb (B).
// Inline asm with VGPR operands: the compiler gives every MFMA builtin an
// AGPR accumulator, and the 256 AGPRs hold O^T.  Back-to-back accumulation
// into one register block needs no wait states; the operands come from LDS
// reads (waited by lgkmcnt) or stay resident.
__device__ __forceinline__ void mma8(f32x16 &acc, const i32x8 &a, const i32x8 &b, int sa, int sb, bool first) {
    if (first)
        asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
                     : "=&v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else
        asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                     : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// acc += A . B on bf16 (the rotary part); the first of a chain follows a
// VALU write of acc and takes the 2 wait states of an s_nop 1.
__device__ __forceinline__ void mma16(f32x16 &acc, const bf16x8 &a, const bf16x8 &b, bool nop) {
    if (nop)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Four floats -> e4m3 codes in bytes 0..3 (round to nearest even; every
// value passed here is within +-448).
__device__ __forceinline__ int pk8x4(float x0, float x1, float x2, float x3) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false), true);
}

__global__ __launch_bounds__(256, 1) void decode_f8mma_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem_[LDS_BYTES];
    lds_u8 *smem = (lds_u8 *)smem_;
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

    // workgroup -> work item {sequence * row_chunks + chunk, blocks, slot}
    const int item = sload(a.plan, plan_wg_off(a.num_items) + blockIdx.x);
    if (item < 0) return;
    const int64_t io = plan_items_off() + 4 * item;
    const int sc = sload(a.plan, io);
    const int b = sc / a.row_chunks, chunk = sc - b * a.row_chunks;
    const int blk0 = sload(a.plan, io + 1), blk1 = sload(a.plan, io + 2), slot = sload(a.plan, io + 3);
    const int S = sload(a.seq_lens, b);
    const int p_first = blk0 * BT;
    // every block of an item holds at least one position < S
    const int nst_live = max(0, min(blk1 - blk0, (S - p_first + BT - 1) / BT));

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5;           // lane half
    const int ln = lane & 31;
    const int wrow = wave * 32 + ln;   // row inside the chunk
    const int row = chunk * kRowsPerChunk + wrow;
    const bool row_ok = row < a.rows;
    const int lim = row_ok ? S - a.q_len + row / a.n_h + 1 : 0;   // visible positions < lim
    // (read back after the first barrier)
    if (g == 0) *(__attribute__((address_space(3))) int *)(smem + LIM_OFF + 4 * wrow) = lim;
    const int64_t grow = (int64_t)b * a.rows + row;

    const uint8_t *pool = (const uint8_t *)a.pool;
    const int64_t bt_row = (int64_t)b * a.bt_stride;
    const int64_t num_blocks = a.num_pool_blocks;
    auto stage_off = [](int st) { return (uint32_t)((st % NST) * STAGE); };

    // ---- copy of stage st (block blk0 + st) into buffer st % 3: wave w
    // copies latent KiB 8w..8w+7 (tokens 16w + 2k + h for lane half h: lane
    // i fills chunk i & 31, i.e. fetches chunk (i & 31) ^ swz(t)), rotary
    // KiB 2w, 2w+1 (tokens 8r + (i >> 3), slot i & 7), and the block scale.
    auto blk_id = [&](int st) -> int64_t {
        const int64_t id = sload(a.block_table, bt_row + blk0 + st);
        return id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
    };
    // part k (0..COPIES-1) of the copy of stage st, held by pool block id
    auto issue_part = [&](int st, int64_t id, int k) {
        const uint8_t *blk = pool + id * a.block_bytes;
        const uint32_t dst = smem_addr + stage_off(st);
        // per-lane offsets recomputed here, so that they are not held in
        // registers across the stage loop
        const int ol = opaque(lane);
        const int h = ol >> 5, u = (ol >> 3) & 7;
        if (k < 8) {
            // swz(2k + h) = 8 (k & 1) + 4 h + ((k >> 1) & 3)
            const uint32_t lat0 = (uint32_t)(512 * h + 16 * ((ol & 31) ^ (4 * h)));
            const int kib = 8 * wave + k;
            dma16(dst + 1024 * kib, lat0 ^ (uint32_t)(16 * (8 * (k & 1) + ((k >> 1) & 3))), blk + 1024 * kib);
        } else if (k < 10) {
            const int r = 2 * wave + (k - 8);   // rot_swz(8 r + u) = (u >> 1) ^ 4 (r & 1), r & 1 = k - 8
            dma16(dst + LAT + 1024 * r, (uint32_t)(128 * u + 16 * ((ol & 7) ^ (u >> 1) ^ (4 * (k - 8)))),
                  blk + LAT + 1024 * r);
        } else {
            // every lane fetches the block scale: a 256-byte ring slot holds 64
            // copies (no exec-mask branch among the score MFMAs)
            dma4_all(smem_addr + RING_OFF + RING_SLOT * (st & 3), (const uint8_t *)(a.block_scales + id));
        }
    };
    auto issue = [&](int st) {
        const int64_t id = blk_id(st);
#pragma unroll
        for (int k = 0; k < COPIES; ++k) issue_part(st, id, k);
    };
    auto sigma = [&](int st) {
        return *(const __attribute__((address_space(3))) float *)(smem + RING_OFF + RING_SLOT * (st & 3));
    };

    if (nst_live > 0) issue(0);
    if (nst_live > 1) issue(1);

    // ---- queries: sigma_q = max|q~| / 448 over the row (lanes ln and ln + 32
    // hold features with bit 5 = 0 and 1), then h = e4m3(q~ / sigma_q) and
    // l = e4m3(16 (q~ / sigma_q - h)) as B fragments: byte b of k-chunk kc is
    // feature 64 kc + 32 g + b.  Rows past the end read the last row (their
    // scores are masked).
    const int rr = min(row, a.rows - 1);
    const __bf16 *qrow = (const __bf16 *)a.q_lat + ((int64_t)b * a.rows + rr) * DC + 32 * g;
    i32x8 qh[KC], ql[KC];
    bf16x8 qr[KR];
    float sig_q;
    {
        float amax = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bf16x8 x = *(const bf16x8 *)(qrow + 64 * kc + 8 * v);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf((float)x[e]));
            }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(amax), __float_as_int(amax), false, false);
        amax = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
        sig_q = amax * (1.0f / 448.0f);
        const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bf16x8 x = *(const bf16x8 *)(qrow + 64 * kc + 8 * v);
                float y[8], r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (float)x[e] * inv;
                int w[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    w[d] = pk8x4(y[4 * d], y[4 * d + 1], y[4 * d + 2], y[4 * d + 3]);
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[d], false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[d], true);
                    r[4 * d] = (y[4 * d] - lo[0]) * 16.0f;
                    r[4 * d + 1] = (y[4 * d + 1] - lo[1]) * 16.0f;
                    r[4 * d + 2] = (y[4 * d + 2] - hi[0]) * 16.0f;
                    r[4 * d + 3] = (y[4 * d + 3] - hi[1]) * 16.0f;
                    qh[kc][2 * v + d] = w[d];
                    ql[kc][2 * v + d] = pk8x4(r[4 * d], r[4 * d + 1], r[4 * d + 2], r[4 * d + 3]);
                }
            }
        const __bf16 *qrr = (const __bf16 *)a.q_rope + ((int64_t)b * a.rows + rr) * DR + 8 * g;
#pragma unroll
        for (int j = 0; j < KR; ++j) qr[j] = *(const bf16x8 *)(qrr + 16 * j);
        // Consumed here, so that the compiler waits for these loads in the
        // prologue: a wait placed at their first use inside the stage loop
        // would run every iteration and, since loads complete in order, also
        // drain the stage copies in flight.
#pragma unroll
        for (int j = 0; j < KR; ++j) asm volatile("" : "+v"(qr[j]));
    }
    // E8M0 scale operands of the score chain, held in VGPRs written once here
    // (opaque, so that no VALU rematerialises them next to an MFMA)
    const int sc_one = opaque(E8M0_ONE), sc_16th = opaque(E8M0_16TH);

    f32x16 oacc[MBLK];
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) oacc[mb] = f32x16{};
    float m_run = -INFINITY;   // reference max (log2 units), lazily raised
    float l_lane = 0.f;        // this lane's share of the softmax denominator

    // Per-lane LDS read bases (stage offsets are multiples of 8 KiB):
    //  score latent, tile T, k-chunk kc, half-chunk hh: token 32 T + ln, chunk
    //    4 kc + 2 g + hh -> (kb ^ (64 kc + 16 hh)) + 16384 T
    //  score rotary, k-step j: chunk 2 j + g of token 32 T + ln ->
    //    (rb ^ 32 j) + 4096 T
    //  value, M-block mb, read j (ds_read_b64_tr_b8: lane 8 a + e of each
    //    16-lane group receives, as its byte s = 0..7, byte e of the 8 read by
    //    lane 2 s + a): byte 8 j + s of half g must be token 16 j + tv, tv =
    //    8 (s >> 2) + 4 g + (s & 3) (tile j >> 1, accumulator 8 (j & 1) + s),
    //    so lane 2 s + a of group G reads features 32 mb + 16 (G & 1) + 8 a
    //    .. + 7 of that token -> (vb ^ 32 mb) + 8192 j
    const int sw_ln = swz(ln & 15);
    const uint32_t kb = (uint32_t)(ln * DC + ((32 * g) ^ (16 * sw_ln)));
    const uint32_t rb = (uint32_t)(LAT + (ln >> 3) * 1024 + (ln & 7) * 128 + 16 * (g ^ rot_swz(ln)));
    uint32_t vb;
    {
        const int G = lane >> 4, i16 = lane & 15, s = i16 >> 1, aa = i16 & 1;
        const int tv = 8 * (s >> 2) + 4 * g + (s & 3);
        vb = (uint32_t)(tv * DC + 8 * aa + 16 * ((G & 1) ^ swz(tv)));
    }

    for (int st = 0; st < nst_live; ++st) {
        // this wave's copies of stage st have landed (stage st+1's may be in
        // flight); the barrier makes every wave's copies visible and frees
        // the buffer of stage st-1 for stage st+2
        if (st + 1 < nst_live)
            asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // stage st+2 goes to the buffer of stage st-1, in parts spread over
        // this iteration's score MFMAs (issued in one burst, the copies held
        // the wave at the memory pipeline while the matrix core idled; among
        // the value MFMAs they pushed the queries out of registers).  Past the
        // item's last stage the parts copy this stage's own block (just read,
        // so served from L2) into that free buffer, which is never read
        // again, so that the score loop needs no branch.
        const int64_t id2 = blk_id(st + 2 < nst_live ? st + 2 : st);
        const uint32_t so = stage_off(st);
        // positions past the sequence end: zero codes and keys, so that P = 0
        // never meets NaN or stale data in the value MFMA
        const int valid = S - (p_first + st * BT);
        if (valid < BT) {
            lds_u8 *stg = smem + so;
            for (int idx = threadIdx.x; idx < (BT - valid) * 32; idx += 256)
                *(uint4 *)(stg + (valid + (idx >> 5)) * DC + (idx & 31) * 16) = make_uint4(0, 0, 0, 0);
            for (int idx = threadIdx.x; idx < (BT - valid) * 8; idx += 256) {
                const int t = valid + (idx >> 3), c = idx & 7;
                *(uint4 *)(stg + LAT + (t >> 3) * 1024 + (t & 7) * 128 + c * 16) = make_uint4(0, 0, 0, 0);
            }
            __syncthreads();
        }
        const float sig = sigma(st);

        // ---- score: latent chunks on the 8-bit core, then the block and
        // query scales, then the rotary k-steps on bf16
        f32x16 s0, s1;
        {
            auto kld = [&](int T, int kc) {
                const uint32_t o = ((kb + so) ^ (uint32_t)(64 * kc)) + 16384 * T;
                i32x8 f;
                const i32x4 x0 = *(const i32x4 *)(smem + o);
                const i32x4 x1 = *(const i32x4 *)(smem + (o ^ 16u));
                f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
                f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
                return f;
            };
            auto rld = [&](int T, int j) {
                return *(const bf16x8 *)(smem + (((rb + so) ^ (uint32_t)(32 * j)) + 4096 * T));
            };
            bf16x8 r0[KR], r1[KR];
            i32x8 k0 = kld(0, 0), k1 = kld(1, 0);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                i32x8 n0, n1;
                if (kc + 1 < KC) {
                    n0 = kld(0, kc + 1);
                    n1 = kld(1, kc + 1);
                } else {
#pragma unroll
                    for (int j = 0; j < KR; ++j) { r0[j] = rld(0, j); r1[j] = rld(1, j); }
                }
                mma8(s0, k0, qh[kc], sc_one, sc_one, kc == 0);
                mma8(s1, k1, qh[kc], sc_one, sc_one, kc == 0);
                mma8(s0, k0, ql[kc], sc_one, sc_16th, false);
                if (2 * kc < COPIES) issue_part(st + 2, id2, 2 * kc);
                mma8(s1, k1, ql[kc], sc_one, sc_16th, false);
                if (2 * kc + 1 < COPIES) issue_part(st + 2, id2, 2 * kc + 1);
                if (kc + 1 < KC) { k0 = n0; k1 = n1; }
            }
            // 8-bit MFMA (16 passes) result -> VALU read: 19 wait states
            asm volatile("s_nop 15\n\ts_nop 3" : "+v"(s0), "+v"(s1));
            const float f = sig * sig_q;
            s0 *= f;
            s1 *= f;
#pragma unroll
            for (int j = 0; j < KR; ++j) {
                mma16(s0, r0[j], qr[j], j == 0);
                mma16(s1, r1[j], qr[j], j == 0);
            }
            // bf16 MFMA (8 passes) result -> VALU read: 11 wait states
            asm volatile("s_nop 15" : "+v"(s0), "+v"(s1));
        }

        // ---- softmax.  Entry q of tile T in lane half g is token
        // 32 T + 8 (q >> 2) + 4 g + (q & 3); it is visible iff its position
        // is < lim.
        const int lim_rel = *(const __attribute__((address_space(3))) int *)(smem + LIM_OFF + 4 * wrow) -
                            (p_first + st * BT) - 4 * g;
        if (__ballot(lim_rel < BT)) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int tq = 8 * (q >> 2) + (q & 3);
                s0[q] = tq < lim_rel ? s0[q] : -INFINITY;
                s1[q] = 32 + tq < lim_rel ? s1[q] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < 16; ++q) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s0[q], s1[q]));
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
            mx = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1])) * a.scale_log2;
        }
        // raise the reference max only when a score exceeds it by 2^2, so
        // that p <= 4 and p 2^5 mant(sigma) < 256 stays in e4m3 range
        const bool raise = mx > m_run + 2.0f;
        const float m_new = raise ? mx : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;

        // ---- P codes of y = p pm, pm = 2^5 mant(|sigma|) folded into the
        // exponent; the value MFMA scales by 2^(e-5).  A negative scale
        // negates the codes; a zero one (mant 1) zeroes them.
        // The denominator takes the exact sum of p: the two code terms carry
        // y to 2^-8, so that a row whose weight sits on one token still gets
        // that token to 2^-8.
        const float asig = __builtin_fabsf(sig);
        int e = asig != 0.f ? __builtin_amdgcn_frexp_expf(asig) - 1 : -122;
        e = e < -122 ? -122 : e;
        const float pm = 32.0f * (asig != 0.f ? __builtin_ldexpf(asig, -e) : 1.0f);
        const int sa = E8M0_ONE + e - 5;
        const float m_off = (m_new == -INFINITY ? 0.f : m_new) - __builtin_amdgcn_logf(pm);
        float ysum = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            s0[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[q], a.scale_log2, -m_off));
            s1[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[q], a.scale_log2, -m_off));
            ysum += s0[q] + s1[q];
        }
        const float psum = ysum / pm;
        if (!(sig > 0.f)) {   // wave-uniform, rare
            const float sg = sig < 0.f ? -1.0f : 0.0f;
            s0 *= sg;
            s1 *= sg;
        }
        i32x8 ph, pl;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const f32x16 &sv = w < 4 ? s0 : s1;
            const int q = 4 * (w & 3);
            ph[w] = pk8x4(sv[q], sv[q + 1], sv[q + 2], sv[q + 3]);
            const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(ph[w], false);
            const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(ph[w], true);
            pl[w] = pk8x4(sv[q] - h01[0], sv[q + 1] - h01[1], sv[q + 2] - h23[0], sv[q + 3] - h23[1]);
        }
        if (__ballot(raise && m_run != -INFINITY)) {
            // rare: the value sum so far moves to the new reference max;
            // accumulators stay in AGPRs and are rescaled block by block
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) {
                asm volatile("" : "+a"(oacc[mb]));
                oacc[mb] *= alpha;
                asm volatile("" : "+a"(oacc[mb]));
            }
        }
        l_lane = l_lane * alpha + psum;
        m_run = m_new;

        // ---- value: O^T[32 mb .. +31][rows] += V^T . P^T
        const uint32_t vbs = vb + so;
        auto vld = [&](int mb) {
            const uint32_t o = vbs ^ (uint32_t)(32 * mb);
            i32x8 f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(smem + o + 8192 * j));
                f[2 * j] = x[0];
                f[2 * j + 1] = x[1];
            }
            return f;
        };
        i32x8 vf[PFV];
#pragma unroll
        for (int j = 0; j < PFV; ++j) vf[j] = vld(j);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * PFV, 0);   // the prefetch reads first
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) {
            oacc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[mb % PFV], ph, oacc[mb], 0, 0, 0, sa, 0,
                                                                        E8M0_ONE);
            oacc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[mb % PFV], pl, oacc[mb], 0, 0, 0, sa, 0,
                                                                        E8M0_ONE);
            if (mb + PFV < MBLK) vf[mb % PFV] = vld(mb + PFV);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (mb + PFV < MBLK) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);

        }
    }

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
    // the copies issued past the last stage have landed, and every wave is
    // done with the stage buffers
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    lds_u8 *orow = smem + wrow * O_PITCH;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bf16x4 v;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) v[e4] = (__bf16)(oacc[mb][4 * q + e4] * inv);
            *(bf16x4 *)(orow + (32 * mb + 8 * q + 4 * g) * 2) = v;
        }
    }
    uint8_t *dst_base = slot < 0 ? (uint8_t *)a.o_lat + ((int64_t)b * a.rows) * (2 * DC)
                                 : (uint8_t *)a.o_part + ((int64_t)slot * a.rows) * (2 * DC);
    const int row0 = chunk * kRowsPerChunk + wave * 32;
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
        if (row0 + r >= a.rows) break;
        const uint4 v = *(const uint4 *)(smem + (wave * 32 + r) * O_PITCH + lane * 16);
        *(uint4 *)(dst_base + (int64_t)(row0 + r) * (2 * DC) + lane * 16) = v;
    }
    if (row_ok && g == 0) {
        if (slot < 0)
            a.lse[grow] = lse_v;
        else
            a.lse_part[(int64_t)slot * a.rows + row] = lse_v;
    }
}

}  // namespace

hipError_t launch_decode_f8mma(const DecodeArgs &a, hipStream_t s) {
    if (a.kv_dtype != MLA_DT_FP8_E4M3 || a.d_c != DC || a.d_r != DR || a.q_dtype != MLA_DT_BF16 ||
        a.block_bytes != STAGE)
        return hipErrorInvalidValue;
    launch_timed(decode_f8mma_kernel, dim3((unsigned)a.grid_wgs), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla

// Absorbed MLA decode on the 8-bit matrix cores, eight waves per workgroup:
// a paged cache of e4m3 latents (one fp32 scale per 64-token block) with
// bf16 rotary keys, bf16 queries and fp32 accumulation.
//
// The cached codes go into the MFMAs as stored (v_mfma_scale ..._f8f6f4):
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
// (Paged fp8 latent cache with a per-block dynamic scale and a 16-bit rotary
// key: huny.dev "DeepSeek MLA 해부" §6, FP8 item; vLLM MLA page, "FP8 MLA
// 지원".  The pages fix the storage, not the arithmetic of the attention;
// quantising q~ and P for the 8-bit MFMAs is this kernel's choice.)
//
// The split of the work: with one 32-row wave per SIMD (queries in 144
// VGPRs, O^T in 256 accumulators) the softmax and the P coding (exp2, e4m3
// conversions) ran with the matrix core idle.  Here a workgroup holds two
// waves per SIMD, each within 256 registers:
//   score  wave w owns query rows 16 w .. 16 w + 15: S^T[16 tok x 16 rows] for
//          4 token tiles, 4 k-chunks x {h, l} on v_mfma_scale 16x16x128 plus
//          2 bf16 rotary k-steps (16x16x32); its queries stay in 72 VGPRs;
//   p      the softmax of those rows, and their P codes written to LDS;
//   value  wave w owns latent features 64 w .. 64 w + 63 of all 128 rows:
//          O^T[64 x 128] += V^T[64 x 64 tok] . P^T[64 tok x 128] on
//          v_mfma_scale 32x32x64 (2 M-blocks x 4 row blocks x {P_h, P_l}),
//          128 accumulators.
// One wave's softmax then runs while the other wave of its SIMD issues
// MFMAs, and each V byte is read from LDS once per wave (the value A
// fragment is shared by the 4 row blocks; the P fragments come from LDS).
// A row's reference max lives with its score wave; when it rises, the score
// wave publishes the row's factor and every wave rescales its part of the
// row's O^T before adding the stage.
#include "common.hpp"
#include "lds_copy.hpp"

namespace mla {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) int lds_i32;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int DC = 512, DR = 64;
constexpr int BT = kBlock;                   // 64 tokens per stage: one paged block
constexpr int LAT = BT * DC;                 // 32,768: the block's e4m3 latent codes
constexpr int STAGE = LAT + BT * DR * 2;     // 40,960: one block, as stored in HBM
constexpr int NST = 3;                       // stage buffers
constexpr int WAVES = 8;
constexpr int ROWS = kRowsPerChunk;          // 128 query rows per workgroup
constexpr int SROWS = ROWS / WAVES;          // 16 score rows per wave
constexpr int KC = DC / 128;                 // 4 latent k-chunks of the score
constexpr int KR = DR / 32;                  // 2 rotary k-steps
constexpr int TILES = BT / 16;               // 4 token tiles
constexpr int MBW = DC / WAVES / 32;         // 2 value M-blocks per wave
constexpr int NB = ROWS / 32;                // 4 value row blocks
constexpr int P_PITCH = 144;                 // a row's P codes: 64 h, 64 l, 16 spare
constexpr int P_OFF = NST * STAGE;
constexpr int ALPHA_OFF = P_OFF + ROWS * P_PITCH;   // per row: this stage's rescale factor
constexpr int FLAG_OFF = ALPHA_OFF + ROWS * 4;      // per wave: a row of it was rescaled
constexpr int LIM_OFF = FLAG_OFF + 64;              // per row: visible positions < lim
constexpr int RING_OFF = LIM_OFF + ROWS * 4;        // 4 block-scale slots, one per stage in flight
constexpr int RING_SLOT = 256;                      // a slot: the scale as loaded by 64 lanes
constexpr int L_OFF = RING_OFF + 4 * RING_SLOT;     // per row: sigma_q (stage loop), then the
                                                    // softmax denominator (epilogue)
constexpr int QR_PITCH = DR * 2 + 16;               // a row's q^R, 16-byte padded
constexpr int QR_OFF = L_OFF + ROWS * 4;            // q^R rows (registers are short: see the kernel)
constexpr int LDS_BYTES = QR_OFF + ROWS * QR_PITCH;
constexpr int O_PITCH = 2 * DC + 16;                // epilogue staging row pitch (bytes)
constexpr int COPIES = 6;                    // per wave and stage: 4 latent KiB, 1 rotary KiB, the scale
constexpr int E8M0_ONE = 127;                // E8M0 scale 2^0
constexpr int E8M0_16TH = 123;               // 2^-4: the l term of the query
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(ROWS * O_PITCH <= ALPHA_OFF, "epilogue staging leaves the per-row words intact");
static_assert(COPIES == 6, "the stage loop waits with vmcnt(6): one stage's copies per wave");
static_assert(STAGE % 8192 == 0, "stage offsets leave the XOR-ed address bits 4-8 clear");
static_assert(LAT == 4 * WAVES * 1024 && BT * DR * 2 == WAVES * 1024, "copy split over the waves");

// LDS layout of a stage (token t = 0..63 of the block):
//   latent  [64][512 B]: 16-byte chunk c of token t at chunk c ^ swz(t);
//   rotary  at LAT, token-major: token t's 128 B at (t >> 3) 1024 + (t & 7) 128,
//           its 16-byte chunk c in slot c ^ rot_swz(t).
// swz rotates the 4 low bits of t by two.  A 16-lane pass of a score read
// (16 consecutive tokens, one chunk each) lands in 16 distinct 16-byte bank
// groups, and so does a transposed value read (32 lanes = 8 tokens x 2
// chunks).
__device__ __forceinline__ constexpr int swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ constexpr int rot_swz(int t) { return ((t & 7) >> 1) ^ (((t >> 3) & 1) << 2); }

// Four floats -> e4m3 codes in bytes 0..3 (round to nearest even; every
// value passed here is within +-448).
__device__ __forceinline__ int pk8x4(float x0, float x1, float x2, float x3) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false), true);
}

// max and sum over the four lanes r, r + 16, r + 32, r + 48 of a score row
__device__ __forceinline__ float row_max4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __builtin_fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __builtin_fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

__global__ __launch_bounds__(512, 1) void decode_f8w8_kernel(DecodeArgs a) {
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
    const int G = lane >> 4, r16 = lane & 15;   // score layout: lane group, row of the wave
    const int g = lane >> 5, ln = lane & 31;    // value layout: lane half, row of a row block
    const int srow = wave * SROWS + r16;        // score row inside the chunk
    const int row = chunk * ROWS + srow;
    const bool row_ok = row < a.rows;
    const int lim = row_ok ? S - a.q_len + row / a.n_h + 1 : 0;   // visible positions < lim
    // (read back by the stage loop, after the first barrier)
    if (G == 0) *(lds_i32 *)(smem + LIM_OFF + 4 * srow) = lim;

    const uint8_t *pool = (const uint8_t *)a.pool;
    const int64_t bt_row = (int64_t)b * a.bt_stride;
    const int64_t num_blocks = a.num_pool_blocks;
    auto stage_off = [](int st) { return (uint32_t)((st % NST) * STAGE); };

    // ---- copy of stage st (block blk0 + st) into buffer st % 3: wave w
    // copies latent KiB 4 w .. 4 w + 3 (KiB k holds tokens 2 k, 2 k + 1; lane
    // 32 h + p fills chunk position p of token 2 k + h, i.e. fetches chunk
    // p ^ swz(t)), rotary KiB w (tokens 8 w .. 8 w + 7; lane 8 u + s fills
    // slot s of token 8 w + u), and the block scale.
    auto blk_id = [&](int st) -> int64_t {
        const int64_t id = sload(a.block_table, bt_row + blk0 + st);
        return id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
    };
    auto issue_part = [&](int st, int64_t id, int k) {
        const uint8_t *blk = pool + id * a.block_bytes;
        const uint32_t dst = smem_addr + stage_off(st);
        // per-lane offsets recomputed here, so that they are not held in
        // registers across the stage loop
        const int ol = opaque(lane);
        if (k < 4) {
            const int kib = 4 * wave + k;
            const int h = ol >> 5, t = 2 * kib + h;
            dma16(dst + 1024 * kib, (uint32_t)(512 * h + 16 * ((ol & 31) ^ swz(t))), blk + 1024 * kib);
        } else if (k == 4) {
            const int u = (ol >> 3) & 7;   // rot_swz(8 w + u) = (u >> 1) ^ 4 (w & 1)
            dma16(dst + LAT + 1024 * wave, (uint32_t)(128 * u + 16 * ((ol & 7) ^ (u >> 1) ^ (4 * (wave & 1)))),
                  blk + LAT + 1024 * wave);
        } else {
            // every lane of every wave fetches the block scale into the same
            // 256-byte slot (equal values; no exec-mask branch)
            dma4_all(smem_addr + RING_OFF + RING_SLOT * (st & 3), (const uint8_t *)(a.block_scales + id));
        }
    };
    auto issue = [&](int st) {
        const int64_t id = blk_id(st);
#pragma unroll
        for (int k = 0; k < COPIES; ++k) issue_part(st, id, k);
    };
    auto sigma = [&](int st) { return *(const lds_f32 *)(smem + RING_OFF + RING_SLOT * (st & 3)); };

    if (nst_live > 0) issue(0);

    // ---- queries: sigma_q = max|q~| / 448 over the row (lane group G holds
    // features 128 G + 32 kc .. + 31 of every k-chunk kc), then
    // h = e4m3(q~ / sigma_q) and l = e4m3(16 (q~ / sigma_q - h)) as B
    // fragments of the 16x16x128 MFMA: byte b of k-chunk kc is feature
    // 128 G + 32 kc + b (the A fragments' order, chosen for the LDS banks:
    // see the score reads).  Rows past the end read the last row (their
    // scores are masked).
    // With O^T in 128 accumulators and the query codes in 64 VGPRs, a wave's
    // 256 registers leave no room for q^R and sigma_q across the stage loop
    // (held there, they were spilled and reloaded every stage, and each
    // reload's wait drained the stage copies in flight): they sit in LDS, in
    // the row's own words, and each lane reads back what its row wrote.
    const int rr = min(row, a.rows - 1);
    const __bf16 *qrow = (const __bf16 *)a.q_lat + ((int64_t)b * a.rows + rr) * DC + 128 * G;
    i32x8 qh[KC], ql[KC];
    {
        // the row's 256 bytes are loaded once and used by both passes (loaded
        // in each, the second pass's loads were issued one at a time, each
        // behind its own wait)
        bf16x8 qx[KC][4];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int v = 0; v < 4; ++v) qx[kc][v] = *(const bf16x8 *)(qrow + 32 * kc + 8 * v);
        float amax = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf((float)qx[kc][v][e]));
        amax = row_max4(amax);
        *(lds_f32 *)(smem + L_OFF + 4 * srow) = amax * (1.0f / 448.0f);   // sigma_q, equal in the row's 4 lanes
        const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bf16x8 x = qx[kc][v];
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (float)x[e] * inv;
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const int w = pk8x4(y[4 * d], y[4 * d + 1], y[4 * d + 2], y[4 * d + 3]);
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
                    qh[kc][2 * v + d] = w;
                    ql[kc][2 * v + d] = pk8x4((y[4 * d] - lo[0]) * 16.0f, (y[4 * d + 1] - lo[1]) * 16.0f,
                                              (y[4 * d + 2] - hi[0]) * 16.0f, (y[4 * d + 3] - hi[1]) * 16.0f);
                }
            }
        // q^R as B fragments of the 16x16x32 bf16 MFMA: lane group G holds
        // rotary features 32 j + 8 G .. + 7 of k-step j (16 bytes at
        // QR_OFF + srow QR_PITCH + 64 j + 16 G; the pitch puts a 16-lane
        // read's rows in 16 distinct bank groups)
        const __bf16 *qrr = (const __bf16 *)a.q_rope + ((int64_t)b * a.rows + rr) * DR + 8 * G;
#pragma unroll
        for (int j = 0; j < KR; ++j)
            *(bf16x8 *)(smem + QR_OFF + srow * QR_PITCH + 64 * j + 16 * G) = *(const bf16x8 *)(qrr + 32 * j);
    }
    // stage 1 after the queries: vector loads complete in order, so a copy
    // issued before them would hold back their first use
    if (nst_live > 1) issue(1);

    f32x16 oacc[MBW][NB];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[mb][nb] = f32x16{};
    float m_run = -INFINITY;   // this lane's score row: reference max (log2 units), lazily raised
    float l_lane = 0.f;        // this lane's share of that row's softmax denominator

    // Per-lane LDS read bases (stage offsets are multiples of 8 KiB):
    //  score latent, tile T, k-chunk kc, half hh: token 16 T + r16, chunk
    //    8 G + 2 kc + hh -> ((kb + so) ^ (32 kc + 16 hh)) + 8192 T.  (Lane
    //    group G in the chunk index's high bits: with G in bits 1-2 instead,
    //    i.e. chunk 8 kc + 2 G + hh, every 16-lane pass still covers the 16
    //    bank groups once, yet a microbenchmark of the read alone, eight
    //    waves per CU, measured 64 cycles per read against 44.9 for this
    //    order and for contiguous reads.)
    //  score rotary, tile T, k-step j: chunk 4 j + G of token 16 T + r16 ->
    //    ((rb + so) ^ 64 j) + 2048 T
    //  value, M-block mb (global, 0..15), read j (ds_read_b64_tr_b8, as
    //    probed on gfx950: lane 8 a + e of each 16-lane group receives, as
    //    its byte s = 0..7, byte e of the 8 read by lane 2 s + a): byte 8 j + s
    //    of half g is token 16 j + 8 (s >> 2) + 4 g + (s & 3), so lane 2 s + a
    //    of group G reads features 32 mb + 16 (G & 1) + 8 a .. + 7 of that
    //    token -> ((vb + so) ^ 32 mb) + 8192 j
    //  P codes: the value B fragment of row block nb and term t (h, l) is
    //    row 32 nb + ln, bytes 64 t + 32 g .. + 31, in the k order above; the
    //    score lane (G, r16) holds tokens 16 T + 4 G + i, whose k position is
    //    32 (G & 1) + 8 T + 4 (G >> 1) + i.
    const uint32_t kb = (uint32_t)(r16 * DC + 16 * ((8 * G) ^ swz(r16)));
    const uint32_t rb = (uint32_t)(LAT + (r16 >> 3) * 1024 + (r16 & 7) * 128 + 16 * (G ^ rot_swz(r16)));
    uint32_t vb;
    {
        const int i16 = lane & 15, s = i16 >> 1, aa = i16 & 1;
        const int tv = 8 * (s >> 2) + 4 * g + (s & 3);
        vb = (uint32_t)(tv * DC + 8 * aa + 16 * ((G & 1) ^ swz(tv)));
    }
    const uint32_t pw = (uint32_t)(P_OFF + srow * P_PITCH + 32 * (G & 1) + 4 * (G >> 1));
    const uint32_t pr = (uint32_t)(P_OFF + ln * P_PITCH + 32 * g);

    for (int st = 0; st < nst_live; ++st) {
        // this wave's copies of stage st have landed (stage st+1's may be in
        // flight); the barrier makes every wave's copies visible, and every
        // wave is done with stage st-1: its buffer takes stage st+2, and the
        // P codes, factors and flags may be rewritten
        if (st + 1 < nst_live)
            asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // Past the item's last stage the parts copy this stage's own block
        // (just read, so served from L2) into the free buffer, which is never
        // read again, so that the score loop needs no branch.
        const int64_t id2 = blk_id(st + 2 < nst_live ? st + 2 : st);
        const uint32_t so = stage_off(st);
        // positions past the sequence end: zero codes and keys, so that P = 0
        // never meets NaN or stale data in the value MFMA
        const int valid = S - (p_first + st * BT);
        if (valid < BT) {
            lds_u8 *stg = smem + so;
            for (int idx = threadIdx.x; idx < (BT - valid) * 32; idx += 512)
                *(uint4 *)(stg + (valid + (idx >> 5)) * DC + (idx & 31) * 16) = make_uint4(0, 0, 0, 0);
            for (int idx = threadIdx.x; idx < (BT - valid) * 8; idx += 512) {
                const int t = valid + (idx >> 3), c = idx & 7;
                *(uint4 *)(stg + LAT + (t >> 3) * 1024 + (t & 7) * 128 + c * 16) = make_uint4(0, 0, 0, 0);
            }
            __syncthreads();
        }
        const float sig = sigma(st);

        // ---- score: latent chunks on the 8-bit core (copy parts of stage
        // st+2 between them), then the block and query scales, then the
        // rotary k-steps on bf16
        f32x4 s[TILES];
        {
            // the XOR-ed bases are recomputed at each read (an opaque copy, so
            // that the compiler does not keep eight of them in registers)
            const uint32_t kbs = kb + so;
            auto kld = [&](int T, int kc) {
                const uint32_t o = ((uint32_t)opaque((int)kbs) ^ (uint32_t)(32 * kc)) + 8192 * T;
                const i32x4 x0 = *(const i32x4 *)(smem + o);
                const i32x4 x1 = *(const i32x4 *)(smem + (o ^ 16u));
                i32x8 f;
                f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
                f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
                return f;
            };
#pragma unroll
            for (int T = 0; T < TILES; ++T) s[T] = f32x4{};
            // each fragment is read one step ahead of its two MFMAs (the
            // schedule is pinned: left alone, the compiler read every fragment
            // right before its MFMAs and waited for it there)
            i32x8 kf = kld(0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int step = 0; step < KC * TILES; ++step) {
                const int kc = step / TILES, T = step % TILES;
                i32x8 kn;
                if (step + 1 < KC * TILES) kn = kld((step + 1) % TILES, (step + 1) / TILES);
                s[T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qh[kc], s[T], 0, 0, 0, E8M0_ONE, 0,
                                                                         E8M0_ONE);
                s[T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, ql[kc], s[T], 0, 0, 0, E8M0_ONE, 0,
                                                                         E8M0_16TH);
                if ((step & 1) == 0 && (step >> 1) < COPIES) issue_part(st + 2, id2, step >> 1);
                if (step + 1 < KC * TILES) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    kf = kn;
                }
            }
            const float f = sig * *(const lds_f32 *)(smem + L_OFF + 4 * srow);   // sigma_blk sigma_q
#pragma unroll
            for (int T = 0; T < TILES; ++T) s[T] *= f;
#pragma unroll
            for (int j = 0; j < KR; ++j) {
                const bf16x8 qr = *(const bf16x8 *)(smem + QR_OFF + srow * QR_PITCH + 64 * j + 16 * G);
                bf16x8 rf[TILES];
#pragma unroll
                for (int T = 0; T < TILES; ++T)
                    rf[T] = *(const bf16x8 *)(smem + (((uint32_t)opaque((int)(rb + so)) ^ (uint32_t)(64 * j)) + 2048 * T));
#pragma unroll
                for (int T = 0; T < TILES; ++T) s[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rf[T], qr, s[T], 0, 0, 0);
            }
        }

        // ---- softmax of this lane's row.  Entry i of tile T in lane group G
        // is token 16 T + 4 G + i; it is visible iff its position is < lim.
        const int lim_rel = *(const lds_i32 *)(smem + LIM_OFF + 4 * srow) - (p_first + st * BT) - 4 * G;
        if (__ballot(lim_rel < BT)) {
#pragma unroll
            for (int T = 0; T < TILES; ++T)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[T][i] = 16 * T + i < lim_rel ? s[T][i] : -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int T = 0; T < TILES; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, s[T][i]);
        mx = row_max4(mx) * a.scale_log2;
        // raise the reference max only when a score exceeds it by 2^2, so
        // that p <= 4 and p 2^5 mant(sigma) < 256 stays in e4m3 range; the
        // first raise of a row has nothing to rescale
        const bool raise = mx > m_run + 2.0f;
        const float m_new = raise ? mx : m_run;
        const float alpha = raise && m_run != -INFINITY ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;

        // ---- P codes of y = p pm, pm = 2^5 mant(|sigma|) folded into the
        // exponent; the value MFMA scales by 2^(e-5).  A negative scale
        // negates the codes; a zero one (mant 1) zeroes them.  The denominator
        // takes the exact sum of p.
        const float asig = __builtin_fabsf(sig);
        int e = asig != 0.f ? __builtin_amdgcn_frexp_expf(asig) - 1 : -122;
        e = e < -122 ? -122 : e;
        const float pm = 32.0f * (asig != 0.f ? __builtin_ldexpf(asig, -e) : 1.0f);
        const int sa = E8M0_ONE + e - 5;
        const float m_off = (m_new == -INFINITY ? 0.f : m_new) - __builtin_amdgcn_logf(pm);
        float ysum = 0.f;
#pragma unroll
        for (int T = 0; T < TILES; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[T][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[T][i], a.scale_log2, -m_off));
                ysum += s[T][i];
            }
        const float psum = ysum / pm;
        if (!(sig > 0.f)) {   // wave-uniform, rare
            const float sg = sig < 0.f ? -1.0f : 0.0f;
#pragma unroll
            for (int T = 0; T < TILES; ++T) s[T] *= sg;
        }
#pragma unroll
        for (int T = 0; T < TILES; ++T) {
            const int ph = pk8x4(s[T][0], s[T][1], s[T][2], s[T][3]);
            const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(ph, false);
            const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(ph, true);
            const int pl = pk8x4(s[T][0] - h01[0], s[T][1] - h01[1], s[T][2] - h23[0], s[T][3] - h23[1]);
            *(lds_i32 *)(smem + pw + 8 * T) = ph;
            *(lds_i32 *)(smem + pw + 64 + 8 * T) = pl;
        }
        const bool rescale = __ballot(alpha != 1.0f) != 0;
        if (G == 0) *(lds_f32 *)(smem + ALPHA_OFF + 4 * srow) = alpha;
        if (lane == 0) *(lds_i32 *)(smem + FLAG_OFF + 4 * wave) = rescale ? 1 : 0;
        l_lane = l_lane * alpha + psum;
        m_run = m_new;
        // every wave's P codes, factors and flags are in LDS
        __syncthreads();

        // ---- value: O^T[64 w + 32 mb ..][32 nb ..] += V^T . P^T (h and l)
        {
            const i32x4 f0 = *(const i32x4 *)(smem + FLAG_OFF);
            const i32x4 f1 = *(const i32x4 *)(smem + FLAG_OFF + 16);
            if ((f0[0] | f0[1] | f0[2] | f0[3] | f1[0] | f1[1] | f1[2] | f1[3]) != 0) {   // rare
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float al = *(const lds_f32 *)(smem + ALPHA_OFF + 4 * (32 * nb + ln));
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) oacc[mb][nb] *= al;
                }
            }
        }
        const uint32_t vbs = vb + so;
        auto vld = [&](int mb) {
            const uint32_t o = vbs ^ (uint32_t)(32 * (MBW * wave + mb));
            i32x8 f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(smem + o + 8192 * j));
                f[2 * j] = x[0];
                f[2 * j + 1] = x[1];
            }
            return f;
        };
        auto pld = [&](int nb, int t) {
            const uint32_t o = pr + nb * 32 * P_PITCH + 64 * t;
            const i32x4 x0 = *(const i32x4 *)(smem + o);
            const i32x4 x1 = *(const i32x4 *)(smem + o + 16);
            i32x8 f;
            f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
            f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
            return f;
        };
        i32x8 vf[MBW];
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) vf[mb] = vld(mb);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const i32x8 p_h = pld(nb, 0), p_l = pld(nb, 1);
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                oacc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[mb], p_h, oacc[mb][nb], 0, 0, 0, sa,
                                                                                0, E8M0_ONE);
                oacc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[mb], p_l, oacc[mb][nb], 0, 0, 0, sa,
                                                                                0, E8M0_ONE);
            }
        }
    }

    // ---- epilogue: O / l as bf16 rows staged through LDS, then 1 KiB
    // coalesced row stores (final o_lat, or this split's bf16 partial).
    const float l_row = row_sum4(l_lane);
    const float lse_v = l_row > 0.f ? (m_run + __log2f(l_row)) * 0.6931471805599453f : -INFINITY;
    if (G == 0) *(lds_f32 *)(smem + L_OFF + 4 * srow) = l_row;
    // the copies issued past the last stage have landed, every wave is done
    // with the stage buffers and P codes, and every row's denominator is in
    // LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l = *(const lds_f32 *)(smem + L_OFF + 4 * (32 * nb + ln));
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        lds_u8 *orow = smem + (32 * nb + ln) * O_PITCH;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x4 v;
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) v[e4] = (__bf16)(oacc[mb][nb][4 * q + e4] * inv);
                *(bf16x4 *)(orow + (32 * (MBW * wave + mb) + 8 * q + 4 * g) * 2) = v;
            }
    }
    __syncthreads();
    uint8_t *dst_base = slot < 0 ? (uint8_t *)a.o_lat + ((int64_t)b * a.rows) * (2 * DC)
                                 : (uint8_t *)a.o_part + ((int64_t)slot * a.rows) * (2 * DC);
    const int row0 = chunk * ROWS + wave * SROWS;
#pragma unroll 4
    for (int r = 0; r < SROWS; ++r) {
        if (row0 + r >= a.rows) break;
        const uint4 v = *(const uint4 *)(smem + (wave * SROWS + r) * O_PITCH + lane * 16);
        *(uint4 *)(dst_base + (int64_t)(row0 + r) * (2 * DC) + lane * 16) = v;
    }
    if (row_ok && G == 0) {
        const int64_t grow = (int64_t)b * a.rows + row;
        if (slot < 0)
            a.lse[grow] = lse_v;
        else
            a.lse_part[(int64_t)slot * a.rows + row] = lse_v;
    }
}

}  // namespace

hipError_t launch_decode_f8w8(const DecodeArgs &a, hipStream_t s) {
    if (a.kv_dtype != MLA_DT_FP8_E4M3 || a.d_c != DC || a.d_r != DR || a.q_dtype != MLA_DT_BF16 ||
        a.block_bytes != STAGE)
        return hipErrorInvalidValue;
    launch_timed(decode_f8w8_kernel, dim3((unsigned)a.grid_wgs), dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla

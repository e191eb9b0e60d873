// Absorbed MLA decode on MFMA for the DeepSeek-V2 shape (latent 512, rotary
// 64, bf16 queries, fp32 accumulation) over a paged cache of bf16 rows
// [c (512) | k^R (64)], or of e4m3 latents with one scale per 64-token block
// plus bf16 rotary keys (decode_mfma_kernel<true>, see below).
//
// Workgroup = 4 waves = 128 query rows (heads x query tokens) of one
// sequence; wave w owns rows 32w..32w+31 for the whole work item and keeps
//   - its queries as MFMA B fragments in VGPRs (32 rows x 576, 144 VGPRs),
//   - O^T, the fp32 latent output sum (512 x 32 rows, 256 accumulators).
// Cached tokens stream through LDS in 32-token stages (half a paged block),
// four stage buffers deep, filled by asynchronous direct-to-LDS loads that
// run two stages ahead of the compute.  Every cached byte is read
// from HBM once per workgroup and from LDS by all four waves:
//   score  S^T[32 tok x 32 rows] = K[32 x 576] . Q^T           (MFMA 32x32x16)
//   p      = exp2(S*scale*log2e - m) with a lazily raised reference max m
//            (raised only when a score passes it by a wide margin)
//   value  O^T[512 x 32] += V^T[512 x 32] . P^T[32 x 32]       (MFMA 32x32x16)
// V is the latent part of the same LDS rows, read transposed with
// ds_read_b64_tr_b16; the score accumulator layout is already the value
// MFMA's B operand, so P never moves between lanes.
// The stage loop is software pipelined: while the matrix pipe runs the score
// MFMAs of stage i+1, the same wave turns stage i's scores into
// probabilities, one slice of the softmax after each MFMA.
//
// Score = content + rotary part: huny.dev "DeepSeek MLA 해부" §2-3
// decomposition; absorbed query against the cached latent: §3-1; latent
// value sum: §3-2; one shared latent "head" (MQA form): vLLM MLA page,
// "MLA의 MQA 디코딩 경로".
#include <type_traits>

#include "common.hpp"
#include "lds_copy.hpp"

namespace mla {

// Cache formats of the MFMA decode (template tags): 16-bit rows (bf16 or
// fp16), or 8-bit codes with one scale per block (e4m3 / e5m2 latent with bf16
// rotary keys, or the whole row in e4m3).
namespace kv {
struct Bf16 { static constexpr bool fp8 = false, half = false, row = false, e5m2 = false; };
struct F16 { static constexpr bool fp8 = false, half = true, row = false, e5m2 = false; };
struct E4m3 { static constexpr bool fp8 = true, half = false, row = false, e5m2 = false; };
struct E5m2 { static constexpr bool fp8 = true, half = false, row = false, e5m2 = true; };
struct E4m3Row { static constexpr bool fp8 = true, half = false, row = true, e5m2 = false; };
}  // namespace kv

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int DC = 512, DR = 64;
constexpr int ROW_BYTES = (DC + DR) * 2;        // 1152 bytes per cached token in HBM
constexpr int CB = DC * 2;                      // 1024: latent bytes of a token
constexpr int RB = DR * 2;                      // 128: rotary bytes of a token
constexpr int HALF = 32;                        // tokens per pipeline stage
constexpr int LPITCH = CB + 16;                 // 1040: LDS pitch of a latent row
constexpr int LAT_BYTES = HALF * LPITCH;        // 33280
constexpr int STAGE_BYTES = LAT_BYTES + HALF * RB;   // 37376
constexpr int NSTAGE = 4;
constexpr int KC = DC / 16;                     // 32 latent score k-steps
constexpr int KS = KC + DR / 16;                // 36 score k-steps
constexpr int MBLOCKS = DC / 32;                // 16 value M-blocks
constexpr int O_PITCH = CB + 16;                // epilogue staging row pitch (bytes)
constexpr int PF = 8;                           // value-fragment prefetch depth (MFMAs)
constexpr int PFK = 3;                          // score-fragment prefetch depth (MFMAs)
template <bool FP8> constexpr int copy_at() { return FP8 ? 0 : 2; }   // stage copies: 0 top, 1 score MFMAs, 2 value MFMAs
// fp8 caches: each stage's e4m3 latent (32 x 512 B) and bf16 rotary rows
// (32 x 128 B) land in one of two staging buffers, and are converted once per
// workgroup into a bf16 stage buffer of the layout above (three of them).
constexpr int FP8_LAT = HALF * DC;              // 16384
constexpr int FP8_STAGE = FP8_LAT + HALF * RB;  // 20480
constexpr int NSTAGE8 = 3;
template <bool FP8>
constexpr int lds_bytes() { return FP8 ? NSTAGE8 * STAGE_BYTES + 2 * FP8_STAGE : NSTAGE * STAGE_BYTES; }
// After the stage buffers: the pool ids of an item's first TAB_IDS blocks
// (read once in the prologue, so that the stage loop issues no scalar memory
// load), then for 8-bit caches a ring of 4 block-scale slots, one per stage in
// flight, each filled by the stage's own copy.
constexpr int TAB_IDS = 1024;
template <bool FP8>
constexpr int tab_off() { return lds_bytes<FP8>(); }
template <bool FP8>
constexpr int ring_off() { return tab_off<FP8>() + 4 * TAB_IDS; }
template <bool FP8>
constexpr int lds_total() { return ring_off<FP8>() + (FP8 ? 16 : 0); }
static_assert(lds_total<false>() <= 160 * 1024 && lds_total<true>() <= 160 * 1024, "stage buffers exceed LDS");
static_assert(4 * 18432 <= 2 * STAGE_BYTES, "query halves exceed stage buffers 0-1");
static_assert(LAT_BYTES % 128 == 0 && STAGE_BYTES % 128 == 0, "rotary reads XOR bits 5-6 of their offsets");
static_assert(2 * STAGE_BYTES <= NSTAGE8 * STAGE_BYTES, "fp8: query halves overlap the staging buffers");
static_assert(4 * 32 * O_PITCH <= lds_bytes<true>() && 4 * 32 * O_PITCH <= lds_bytes<false>(),
              "epilogue staging exceeds the LDS allocation");

// LDS layout of a stage (slot t = token t of the stage):
//   latent rows  [32][1040 B]: bytes 0..1023 of slot t = c of token t;
//   rotary part  [32 tokens][8 slots][16 B], token-major: token t's 128 B at
//                LAT_BYTES + (t >> 3) * 1024 + (t & 7) * 128, its 16-byte
//                chunk c in slot c ^ rot_swz(t).
// Row i of the score MFMA (A-operand lane i) reads slot tok_of(i), where
// i = 8a + 4h + e  ->  16 (a >> 1) + 4 e + 2 (a & 1) + h.
// With 64 four-byte banks (256 B per cycle), the 16-byte pitch step makes
// the 16 slots of a score read land in 16 distinct 16-byte bank groups, and
// a transposed value read (32 lanes = 4 slots x 64 B) gets 4 slots spaced 4
// apart, i.e. 64 B apart in bank space: every bank exactly once.  Every LDS
// read is then a per-lane base plus a compile-time offset.
__device__ __forceinline__ constexpr int tok_of(int i) {
    return 16 * (i >> 4) + 4 * (i & 3) + 2 * ((i >> 3) & 1) + ((i >> 2) & 1);
}
// Chunk swizzle of the rotary part.  One 16-lane pass of a score read takes
// chunk c of 16 tokens: t & 7 = 0..7 of two 8-token groups.  Token t's slot
// lands in 16-byte bank group 8 (t & 1) + (c ^ rot_swz(t)); over the 4 tokens
// of one parity in a group rot_swz takes 4 values that differ in bits 0-1, and
// the two groups differ in bit 2, so the 16 reads hit 16 distinct bank groups.
// The copy fills a token's 128 B from 8 consecutive lanes, so each 16-lane
// quarter of a copy reads 2 cache lines; a chunk-major layout made every
// quarter touch 8 lines and cost the copy four times the issue time of a
// contiguous one.
__device__ __forceinline__ constexpr int rot_swz(int t) { return ((t & 7) >> 1) ^ (((t >> 3) & 1) << 2); }

// The copy of one stage is split into parts (one instruction each) so that
// the stage loop can spread them over the score MFMAs.
constexpr int DMA_PER_STAGE = 9;    // 16-bit rows, per wave: 8 latent rows + 1 KiB of rotary parts
constexpr int DMA_PER_STAGE8 = 6;   // 8-bit codes, per wave: the block scale + 5 KiB

// Part k of a 16-bit stage whose first token is at src0 (token row pointer in
// HBM).  Wave w copies latent row 8w + k for k < 8 (one 1 KiB instruction;
// lane i reads bytes 16i..16i+15, voff = l16 = 16 i) and, for k = 8, the
// rotary parts of the same 8 tokens (lane i = 8u + p fills slot p of token
// 8w + u, i.e. reads its chunk p ^ rot_swz(8w + u); voff = rot_off).
__device__ __forceinline__ void stage_part(const uint8_t *src0, uint32_t stage_lds, int wave,
                                           uint32_t l16, uint32_t rot_off, int k) {
    if (k < 8) {
        const int t = wave * 8 + k;
        dma16(stage_lds + t * LPITCH, l16, src0 + t * ROW_BYTES);
    } else {
        dma16(stage_lds + LAT_BYTES + wave * 1024, rot_off, src0);
    }
}

// Part k of an 8-bit stage (32 tokens of a block) into a staging buffer:
// k = 0 the block scale (lane 0 of every wave, into the stage's ring slot);
// e4m3 / e5m2 latent: k = 1..4 latent bytes 4 KiB w + 1 KiB (k - 1) (two
// 512-byte rows per instruction), k = 5 the 8 rotary rows 8w..8w+7.
__device__ __forceinline__ void stage_part_fp8(const uint8_t *codes0, const uint8_t *rope0, const uint8_t *scale,
                                               uint32_t staging_lds, uint32_t ring_lds, int wave, int lane, int k) {
    const uint32_t l16 = (uint32_t)lane << 4;
    if (k == 0)
        dma4_lane0(ring_lds, scale, lane);
    else if (k < 5)
        dma16(staging_lds + (4 * wave + k - 1) * 1024, l16, codes0 + (4 * wave + k - 1) * 1024);
    else
        dma16(staging_lds + FP8_LAT + wave * 1024, l16, rope0 + wave * 1024);
}

// Whole-row e4m3 cache: one stage is 32 contiguous rows of 576 codes (18 KiB)
// of the block's [64][576]; after the scale (k = 0), wave w copies KiB
// 4w + k - 1 for k = 1..4 and KiB 16 + (w & 1) for k = 5 (waves 2 and 3
// repeat the last copies of waves 0 and 1: same bytes, same place), so every
// wave issues as many copies as for the split layout.
__device__ __forceinline__ void stage_part_row(const uint8_t *rows0, const uint8_t *scale, uint32_t staging_lds,
                                               uint32_t ring_lds, int wave, int lane, int k) {
    const uint32_t l16 = (uint32_t)lane << 4;
    if (k == 0) {
        dma4_lane0(ring_lds, scale, lane);
    } else {
        const int kib = k < 5 ? 4 * wave + k - 1 : 16 + (wave & 1);
        dma16(staging_lds + kib * 1024, l16, rows0 + kib * 1024);
    }
}
static_assert(HALF * (DC + DR) <= 18 * 1024 && 18 * 1024 <= FP8_STAGE, "row stage copy");

// FP8: the cache stores e4m3 (or e5m2) latents with one fp32 scale per
// 64-token block and bf16 rotary keys.  Codes are converted exactly to bf16
// (the scale is a per-stage scalar): the score chain runs the 4 rotary
// k-steps first, scales that partial sum by 1/sigma, then adds the latent
// k-steps, so that sigma * acc = sigma (q~ . c8) + q^R . k^R; the
// probabilities are produced already multiplied by sigma (value MFMAs then
// sum (sigma p) c8 = p c) and the denominator takes psum / sigma.  With the
// whole row in e4m3 the rotary codes carry the same scale, so the chain has
// no 1/sigma step.  (fp8 cache: huny.dev "DeepSeek MLA 해부" §6 FP8 item;
// vLLM MLA page, "FP8 MLA 지원".)
// F16: rows of IEEE fp16 run the same pipeline on fp16 MFMAs; the bf16
// queries are rounded to fp16 once in the prologue (exact for magnitudes in
// [2^-14, 65504]; larger ones saturate) and the probabilities are fp16.
template <typename KV>
__global__ __launch_bounds__(256, 1) void decode_mfma_kernel(DecodeArgs a) {
    constexpr bool FP8 = KV::fp8, ROW = KV::row, H16 = KV::half;
    constexpr int COPY_AT = copy_at<FP8>();
    // Lazy reference max (log2 units): a row's reference m is raised only
    // when a stage's max passes it by RAISE_T, and then to that max plus
    // RAISE_H, so p = 2^(s - m) <= 2^RAISE_T.  A raise rescales the wave's
    // whole O^T (256 products per lane), so it must stay rare.  fp16
    // probabilities (65504 at most) and 8-bit caches (the block scale rides
    // in the exp2 argument, down to 2^-64) keep p <= 2^8 with no headroom;
    // bf16 ones have fp32's exponent range: p <= 2^40, and the max token's
    // p = 2^-24 after a raise, so that outlier keys (scores tens of units
    // above the rest) raise once instead of at every new record.  The fp32
    // sums overflow only for |v| near 2^(128 - 40 - 17) = 2^71 over 2^17
    // tokens, and products p v underflow only for |v| below about 2^-100.
    constexpr float RAISE_T = (FP8 || H16) ? 8.0f : 40.0f;
    constexpr float RAISE_H = (FP8 || H16) ? 0.0f : 24.0f;
    __shared__ __attribute__((aligned(1024))) uint8_t smem_[lds_total<FP8>()];
    lds_u8 *smem = (lds_u8 *)smem_;
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

    // Every kernel argument that the first copies depend on, in one round
    // trip: left alone, the compiler loaded each where it was first needed,
    // and the prologue waited on the scalar cache five times before its first
    // copy.
    asm volatile("" ::"s"(a.plan), "s"(a.seq_lens), "s"(a.block_table), "s"(a.q_lat), "s"(a.q_rope), "s"(a.pool),
                 "s"(a.num_items), "s"(a.row_chunks), "s"(a.bt_stride), "s"(a.rows), "s"(a.num_pool_blocks),
                 "s"(a.q_len), "s"(a.n_h));
    // workgroup -> work item {sequence * row_chunks + chunk, blocks, slot},
    // from the plan's dispatch table (longest items first on each XCD; -1
    // pads the grid)
    const int item = sload(a.plan, plan_wg_off(a.num_items) + blockIdx.x);
    if (item < 0) return;
    const int64_t io = plan_items_off() + 4 * item;
    const int sc = sload(a.plan, io);
    const int b = sc / a.row_chunks, chunk = sc - b * a.row_chunks;
    const int blk0 = sload(a.plan, io + 1), blk1 = sload(a.plan, io + 2), slot = sload(a.plan, io + 3);
    // the sequence length: loaded here, waited for after the first query
    // copies are issued (see the queries below), which do not need it
    const int S_load = sload(a.seq_lens, b);
    int S, nst_live;
    const int nst = 2 * (blk1 - blk0);   // 32-token stages in this item
    const int p_first = blk0 * kBlock;

    // wave index as a wave-uniform (scalar) value: the stage copies use it in
    // their scalar source pointers and LDS destinations
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5;           // lane half
    const int ln = lane & 31;
    const int wrow = wave * 32 + ln;   // row inside the chunk
    const int row = chunk * kRowsPerChunk + wrow;
    const bool row_ok = row < a.rows;
    const int64_t grow = (int64_t)b * a.rows + row;

    const uint8_t *pool = (const uint8_t *)a.pool;
    const int64_t bt_row = (int64_t)b * a.bt_stride;
    const int64_t num_blocks = a.num_pool_blocks;
    auto blk_id = [&](int st) {
        int64_t id = sload(a.block_table, bt_row + blk0 + (st >> 1));
        return id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
    };
    // pool id of the block holding stage st, from the LDS table once the
    // prologue has filled it (a scalar load for blocks past its end)
    const int ntab = min(blk1 - blk0, TAB_IDS);
    const __attribute__((address_space(3))) int32_t *tab =
        (const __attribute__((address_space(3))) int32_t *)(smem + tab_off<FP8>());
    // (raw: the table entry of stage st as read into a VGPR, tab_raw(st))
    auto tab_raw = [&](int st) { return tab[min(st >> 1, TAB_IDS - 1)]; };
    auto blk_id_tab = [&](int st, int raw) -> int64_t {
        if ((st >> 1) < ntab) return __builtin_amdgcn_readfirstlane(raw);
        return blk_id(st);
    };
    // block scale of stage st (8-bit caches): its ring slot, filled by the
    // stage's copy
    auto sigma = [&](int st) {
        return *(const __attribute__((address_space(3))) float *)(smem + ring_off<FP8>() + 4 * (st & 3));
    };
    // The arithmetic takes the magnitude of a block scale: its sign and a
    // zero are applied to the codes when they are converted (negated, or
    // zeroed with magnitude 1).  Magnitudes below 2^-64 are raised to 2^-64:
    // the rotary partial sum is divided by the scale and the probabilities
    // carry it, and this keeps both inside fp32's range (such a block's
    // latent values are below 448 * 2^-64 either way).
    auto sig_mag = [](float s) { return s == 0.f ? 1.f : __builtin_fmaxf(__builtin_fabsf(s), 0x1p-64f); };
    // xor mask (sign flip of both bf16 halves) and zero flag of stage st's
    // converted codes
    auto code_xor = [&](int st) { return sigma(st) < 0.f ? 0x80008000u : 0u; };
    auto code_zero = [&](int st) { return sigma(st) == 0.f; };
    auto stage_off = [&](int st) {
        // bf16: stage st in buffer (st + 2) mod 4 (buffers 0-1 hold the queries
        // while stages 0-1 are copied)
        return FP8 ? (uint32_t)((st % NSTAGE8) * STAGE_BYTES) : (uint32_t)(((st + 2) & (NSTAGE - 1)) * STAGE_BYTES);
    };
    auto staging_off = [&](int st) { return (uint32_t)(NSTAGE8 * STAGE_BYTES + (st & 1) * FP8_STAGE); };
    const uint32_t l16 = lane << 4;
    auto rot_voff = [&](int ln_) {
        const int t = wave * 8 + (ln_ >> 3);
        return (uint32_t)(t * ROW_BYTES + CB + 16 * ((ln_ & 7) ^ rot_swz(t)));
    };
    // part k of the copy of stage st, held by pool block id
    constexpr int NPARTS = FP8 ? DMA_PER_STAGE8 : DMA_PER_STAGE;
    auto issue_part = [&](int st, int64_t id, int k) {
        if constexpr (FP8) {
            const uint8_t *blk = pool + id * a.block_bytes;
            const uint8_t *scale = (const uint8_t *)a.block_scales + 4 * id;
            const uint32_t ring = smem_addr + ring_off<FP8>() + 4 * (st & 3);
            if constexpr (ROW)
                stage_part_row(blk + (st & 1) * HALF * (DC + DR), scale, smem_addr + staging_off(st), ring, wave,
                               opaque(lane), k);
            else
                stage_part_fp8(blk + (st & 1) * FP8_LAT, blk + kBlock * DC + (st & 1) * HALF * RB, scale,
                               smem_addr + staging_off(st), ring, wave, opaque(lane), k);
        } else {
            const uint8_t *src0 = pool + id * (int64_t)(kBlock * ROW_BYTES) + (st & 1) * HALF * ROW_BYTES;
            // the two per-lane offsets are recomputed where they are used
            // (held across the loop, they were spilled)
            const int ol = opaque(lane);
            stage_part(src0, smem_addr + stage_off(st), wave, (uint32_t)ol << 4, rot_voff(ol), k);
        }
    };
    auto issue = [&](int st, int64_t id) {
#pragma unroll
        for (int k = 0; k < NPARTS; ++k) issue_part(st, id, k);
    };

    // ---- queries -> VGPRs (MFMA B fragments: lane (ln, g) holds, for k-step
    // ks, bytes 32 ks + 16 g .. +15 of row ln's 1152), in two halves of 16
    // rows so that the copies of stages 0 and 1 start with the first half.
    // Each wave copies a half into its own 18 KiB region of stage buffers 0-1
    // (stages 0 and 1 go to buffers 2-3) with coalesced 1 KiB copies: latent
    // row r with its 16-byte chunks XOR-swizzled by r & 15 (lane i fetches
    // chunk i ^ (r & 15)), so that 16 rows reading one chunk hit 16 distinct
    // bank groups; the rotary parts as [r >> 3][chunk][r & 7].  Lanes of rows
    // 0-15 read the first half, lanes of rows 16-31 the second.  Rows past
    // the end of the sequence's rows read its last row (their scores are
    // masked).  VMEM loads complete in order, so waiting for the second half
    // also waits for stages 0 and 1.
    bf16x8 qf[KS];
    {
        const uint32_t qreg = smem_addr + wave * 18432;
        const int row_base = chunk * kRowsPerChunk + wave * 32;   // first row of this wave
        const int64_t seq_row0 = (int64_t)b * a.rows;
        const uint8_t *qlat = (const uint8_t *)a.q_lat + seq_row0 * CB;
        const uint8_t *qrope = (const uint8_t *)a.q_rope + seq_row0 * RB;
        auto copy_half = [&](int h) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = min(row_base + 16 * h + r, a.rows - 1);
                dma16(qreg + r * CB, l16 ^ (uint32_t)(r << 4), qlat + (int64_t)rr * CB);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                // lane i = 8 c + u: chunk c of row 16 h + 8 q + u
                const int rr = min(row_base + 16 * h + 8 * q + (lane & 7), a.rows - 1);
                dma16(qreg + 16 * CB + q * 1024, (uint32_t)(rr * RB + 16 * (lane >> 3)), qrope);
            }
        };
        lds_u8 *qw = smem + wave * 18432;
        const int lr = ln & 15;
        auto read_half = [&]() {
#pragma unroll
            for (int ks = 0; ks < KC; ++ks)
                qf[ks] = *(const bf16x8 *)(qw + lr * CB + (((2 * ks + g) ^ lr) << 4));
#pragma unroll
            for (int j = 0; j < DR / 16; ++j)
                qf[KC + j] = *(const bf16x8 *)(qw + 16 * CB + (lr >> 3) * 1024 + (2 * j + g) * 128 + (lr & 7) * 16);
        };
        // the block-id table: plain loads issued before any copy (so the
        // wait the compiler places before the table writes, after every copy
        // has landed, holds nothing back)
        int tv[TAB_IDS / 256];
#pragma unroll
        for (int k = 0; k < TAB_IDS / 256; ++k) {
            const int j = (int)threadIdx.x + 256 * k;
            tv[k] = j < ntab ? a.block_table[bt_row + blk0 + j] : 0;
        }
        copy_half(0);
        // a stage holds tokens only if its first position is < S (the plan
        // covers ceil(S/64) blocks, so the second half of the last block may
        // be empty)
        S = S_load;
        asm volatile("" : "+s"(S));
        nst_live = min(nst, (S - p_first + HALF - 1) / HALF);
        issue(0, blk_id(0));
        if (nst_live > 1) issue(1, blk_id(1));
        // the first half has landed when at most the stage copies are in flight
        if (nst_live > 1) {
            if constexpr (FP8) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
        } else {
            if constexpr (FP8) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        }
        if (ln < 16) read_half();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the region is refilled
        copy_half(1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // second half, stages 0 and 1
        {
            __attribute__((address_space(3))) int32_t *tw =
                (__attribute__((address_space(3))) int32_t *)(smem + tab_off<FP8>());
#pragma unroll
            for (int k = 0; k < TAB_IDS / 256; ++k) {
                // every entry is written (0 past the item's blocks), so that
                // no load stays outstanding for the compiler past this point
                const int j = (int)threadIdx.x + 256 * k;
                tw[j] = tv[k] < 0 ? 0 : (tv[k] >= num_blocks ? (int)(num_blocks - 1) : tv[k]);
            }
        }
        if (ln >= 16) read_half();
        if constexpr (H16) {
            // fp16 cache: the queries as fp16 (saturating)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = fminf(fmaxf((float)qf[ks][e], -65504.f), 65504.f);
                    qf[ks][e] = __builtin_bit_cast(__bf16, (_Float16)f);
                }
        }
    }
    // every wave holds its queries (the query regions are free) and every
    // wave's copies of stages 0 and 1 are visible
    __syncthreads();
    const int lim = row_ok ? S - a.q_len + row / a.n_h + 1 : 0;   // visible positions < lim
    f32x16 oacc[MBLOCKS];
#pragma unroll
    for (int mb = 0; mb < MBLOCKS; ++mb) oacc[mb] = f32x16{};
    float m_run = -INFINITY;   // reference max (log2 units), lazily raised
    float l_lane = 0.f;        // this lane's share of the softmax denominator

    // Per-lane LDS read bases (a stage offset is added once per stage; every
    // read adds a compile-time offset).
    //  score, latent k-step ks: slot tok_of(ln), chunk 2 ks + g -> kb0 + 32 ks
    //  score, rotary k-step KC + j: chunk 2 j + g of token tq = tok_of(ln), in
    //  slot (2 j + g) ^ rot_swz(tq) = 2 j ^ (g ^ rot_swz(tq)): rb0 holds the
    //  token's base + 16 (g ^ rot_swz(tq)) (a stage offset keeps bits 0-6
    //  clear), the k-step applies ^ 32 j
    //  value (ds_read_b64_tr_b16: lane i of each 16-lane group receives element
    //  i % 4 of the 8 bytes read by lane 4s + i/4, s = 0..3): k-step s2 needs,
    //  for lane half g, the tokens tok_of(8 s2 + 4 g + e) = 4 e + 2 s2 + g and,
    //  for the upper 8 k, 16 + the same; lane (group G, index w) reads slot
    //  4 (w >> 2) + 2 s2 + (G >> 1) (+16), features 32 mb + 16 (G & 1) + 4 (w & 3)
    //  -> vb0 + 2 LPITCH s2 + 64 mb (+ 16 LPITCH).
    const int tq = tok_of(ln);
    const uint32_t kb0 = tq * LPITCH + 16 * g;
    const uint32_t rb0 = LAT_BYTES + (tq >> 3) * 1024 + (tq & 7) * 128 + 16 * (g ^ rot_swz(tq));
    const int grp16 = lane >> 4, w16 = lane & 15;
    const uint32_t vb0 = (4 * (w16 >> 2) + (grp16 >> 1)) * LPITCH + 32 * (grp16 & 1) + 8 * (w16 & 3);

    auto kld = [&](uint32_t kbs, uint32_t rbs, int ks) {
        return ks < KC ? *(const bf16x8 *)(smem + kbs + 32 * ks)
                       : *(const bf16x8 *)(smem + (rbs ^ (uint32_t)(32 * (ks - KC))));
    };
    auto vld = [&](uint32_t vbs, int i) {
        const int s2 = i / MBLOCKS, mb = i % MBLOCKS;
        lds_u8 *lo = smem + vbs + 2 * LPITCH * s2 + 64 * mb;
        bf16x8 vf;
        vf.lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)lo));
        vf.hi = __builtin_bit_cast(bf16x4,
                                   __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lo + 16 * LPITCH)));
        return vf;
    };
    // order of the score k-steps: fp8 runs the 4 rotary k-steps first
    auto kstep = [](int i) { return FP8 ? (i < DR / 16 ? KC + i : i - DR / 16) : i; };

    // ---- score MFMAs: S^T[32 tokens x 32 rows] += K[32 x 16] . Q^T[16 x 32].
    // Written as inline asm with VGPR operands: the compiler gives every MFMA
    // builtin an AGPR accumulator, and the 256 AGPRs are all taken by O^T.
    // Hazards the compiler cannot see are covered by hand: the chain
    // accumulates back to back into the same registers (no wait states
    // needed); its operands come from LDS reads (waited by lgkmcnt) or stay
    // resident, so inside the stage loop only a VALU write of the
    // accumulator needs the 2 wait states of an s_nop 1 (the fp8 rescale
    // after the rotary k-steps; the first MFMA takes one too).  The chain of
    // stage 0 keeps a nop before every MFMA: the compiler may place the
    // fp16 conversion of a query fragment right before its first use.  An
    // s_nop 15 after a chain covers the MFMA-result -> VALU-read latency
    // (>= 10 wait states for an 8-pass MFMA).  A nop before every MFMA cost
    // ~130 cycles per stage of issue.
    auto score_mfma = [&](f32x16 &acc, const bf16x8 &kf, int i, bool all_nops) {
        const bool nop = all_nops || i == 0 || (FP8 && !ROW && i == DR / 16);
        // the first MFMA writes the accumulator while reading its operands:
        // early clobber keeps them apart
        if constexpr (H16) {
            if (i == 0)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0"
                             : "=&v"(acc) : "v"(kf), "v"(qf[kstep(0)]));
            else if (nop)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                             : "+v"(acc) : "v"(kf), "v"(qf[kstep(i)]));
            else
                asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                             : "+v"(acc) : "v"(kf), "v"(qf[kstep(i)]));
        } else {
            if (i == 0)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                             : "=&v"(acc) : "v"(kf), "v"(qf[kstep(0)]));
            else if (nop)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+v"(acc) : "v"(kf), "v"(qf[kstep(i)]));
            else
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+v"(acc) : "v"(kf), "v"(qf[kstep(i)]));
        }
    };
    // fp8: after the rotary k-steps, divide the partial sum by the block scale
    auto rope_to_latent_scale = [&](f32x16 &acc, float inv_sigma) {
        asm volatile("s_nop 15" : "+v"(acc));
        acc *= inv_sigma;
    };

    // Rows past the sequence end in a partial stage are zeroed in LDS so that
    // P = 0 never meets NaN or stale data in the value MFMA (their scores are
    // masked to -inf, so the score MFMA may read either).
    auto zero_tail = [&](int st) {
        const int valid = S - (p_first + st * HALF);   // >= 1 for a live stage
        if (valid < HALF) {
            lds_u8 *stg = smem + stage_off(st);
            for (int idx = threadIdx.x; idx < (HALF - valid) * 64; idx += 256)
                *(uint4 *)(stg + (valid + (idx >> 6)) * LPITCH + (idx & 63) * 16) = make_uint4(0, 0, 0, 0);
            for (int idx = threadIdx.x; idx < (HALF - valid) * 8; idx += 256) {
                const int t = valid + (idx >> 3), c = idx & 7;
                *(uint4 *)(stg + LAT_BYTES + (t >> 3) * 1024 + (t & 7) * 128 + c * 16) = make_uint4(0, 0, 0, 0);
            }
        }
    };
    // fp8: staging buffer of stage st -> its bf16 stage buffer, by all 256
    // threads: latent codes converted exactly (scale 1), rotary rows copied,
    // rows past the sequence end written as zeros.
    // codes 0-1 (lo) or 2-3 (hi) of a packed word -> two bf16 (exact; scale 1)
    auto cvt_lo = [](uint32_t w) {
        if constexpr (KV::e5m2)
            return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false));
        else
            return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    };
    auto cvt_hi = [](uint32_t w) {
        if constexpr (KV::e5m2)
            return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true));
        else
            return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    };
    // latent codes of token t: [t][512] (split layout) or the first 512 of [t][576]
    constexpr int CODE_PITCH = ROW ? DC + DR : DC;
    // The staged bytes a thread converts, in five parts: part j < 4 is
    // 16-byte chunk tid + 256 j of the 16 KiB of latent codes, part 4 a
    // piece of the rotary part.
    auto convert_load = [&](int st, int j) {
        const lds_u8 *src = smem + staging_off(st);
        const int tid = opaque(threadIdx.x);
        if (j < 4) {
            const int i = tid + 256 * j;
            const int t = i >> 5, c16 = i & 31;
            return *(const uint4 *)(src + (ROW ? t * CODE_PITCH + c16 * 16 : i * 16));
        }
        const int t = tid >> 3, c = tid & 7;
        if constexpr (ROW) {
            const uint2 w = *(const uint2 *)(src + t * CODE_PITCH + DC + c * 8);   // rotary codes 8c..8c+7
            return make_uint4(w.x, w.y, 0, 0);
        } else {
            return *(const uint4 *)(src + FP8_LAT + t * RB + c * 16);
        }
    };
    // xr / zr: the stage's code_xor / code_zero (a negative scale negates
    // the converted codes, a zero scale zeroes them; the rotary part of the
    // split layout is bf16 and carries no scale)
    auto convert_part = [&](int st, const uint4 &in, int j, uint32_t xr, bool zr) {
        const int valid = S - (p_first + st * HALF);
        lds_u8 *dst = smem + stage_off(st);
        const int tid = opaque(threadIdx.x);
        if (j < 4) {
            const int i = tid + 256 * j;
            const int t = i >> 5, c16 = i & 31;
            uint32_t o[8];
            const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = cvt_lo(w[e]) ^ xr;
                o[2 * e + 1] = cvt_hi(w[e]) ^ xr;
            }
            const bool live = t < valid && !zr;
            uint4 *d = (uint4 *)(dst + t * LPITCH + c16 * 32);
            d[0] = live ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(0, 0, 0, 0);
            d[1] = live ? make_uint4(o[4], o[5], o[6], o[7]) : make_uint4(0, 0, 0, 0);
        } else {
            const int t = tid >> 3, c = tid & 7;
            uint4 v = in;
            bool live = t < valid;
            if constexpr (ROW) {
                v = make_uint4(cvt_lo(in.x) ^ xr, cvt_hi(in.x) ^ xr, cvt_lo(in.y) ^ xr, cvt_hi(in.y) ^ xr);
                live = live && !zr;
            }
            *(uint4 *)(dst + LAT_BYTES + (t >> 3) * 1024 + (t & 7) * 128 + (c ^ rot_swz(t)) * 16) =
                live ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto convert = [&](int st) {
        const uint32_t xr = code_xor(st);
        const bool zr = code_zero(st);
        uint4 in[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) in[j] = convert_load(st, j);
#pragma unroll
        for (int j = 0; j < 5; ++j) convert_part(st, in[j], j, xr, zr);
    };

    // ---- prologue: score of stage 0
    float sig_cur = 1.f, sig_next = 1.f;   // block scales of stages st, st+1 (fp8)
    if constexpr (FP8) {
        // stages 0 and 1 landed in the staging buffers and are converted;
        // stage 2 then takes stage 0's staging buffer
        convert(0);
        if (nst_live > 1) convert(1);
        __syncthreads();
        if (nst_live > 2) issue(2, blk_id_tab(2, tab_raw(2)));
        sig_cur = sig_mag(sigma(0));
    } else {
        if (nst_live > 2) issue(2, blk_id_tab(2, tab_raw(2)));
        zero_tail(0);
    }
    f32x16 sA, sB;
    {
        const uint32_t kbs = kb0 + stage_off(0), rbs = rb0 + stage_off(0);
        bf16x8 kb[PFK];
#pragma unroll
        for (int j = 0; j < PFK; ++j) kb[j] = kld(kbs, rbs, kstep(j));
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            score_mfma(sA, kb[i % PFK], i, true);
            if (i + PFK < KS) kb[i % PFK] = kld(kbs, rbs, kstep(i + PFK));
            if (FP8 && !ROW && i == DR / 16 - 1) rope_to_latent_scale(sA, 1.0f / sig_cur);
        }
        asm volatile("s_nop 15" : "+v"(sA));
    }

    // ---- one pipelined iteration: scores of stage st (cur, complete) become
    // probabilities while stage st+1's score MFMAs fill nxt; then stage st's
    // value MFMAs.
    // raw: on entry the table entry of stage st+3 (read one iteration ahead,
    // so its LDS latency is hidden); on exit that of stage st+4
    auto iteration = [&](int st, f32x16 &cur, f32x16 &nxt, int &raw) {
        const bool has_next = st + 1 < nst_live;
        // stage st+3 is copied in parts spread over this iteration's score
        // MFMAs
        const bool iss = st + 3 < nst_live;
        const int64_t id3 = iss ? blk_id_tab(st + 3, raw) : 0;
        auto copy_slot = [&](int i, int n) {   // slot i of n MFMAs: one copy part
            const int spread = n / NPARTS;
            if (i % spread == 1 && i / spread < NPARTS) {
                if (iss) issue_part(st + 3, id3, i / spread);
            }
        };
        if constexpr (FP8) {
            // stage st+1 was converted during iteration st-1 (or in the
            // prologue); every wave has finished iteration st-1, so the
            // staging buffer and scale slot of stage st+1 may be refilled
            // with stage st+3
            __syncthreads();
            if constexpr (COPY_AT == 0) { if (iss) issue(st + 3, id3); }
            if (has_next) sig_next = sig_mag(sigma(st + 1));
        } else {
            if (has_next) {
                // stage st+1 landed for this wave (stage st+2 may be in flight)
                if (st + 2 < nst_live)
                    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            // every wave's copy of stage st+1 is visible, and every wave has
            // finished iteration st-1, so stage st-1's buffer may be refilled
            __syncthreads();
            if constexpr (COPY_AT == 0) { if (iss) issue(st + 3, id3); }
            if (has_next) zero_tail(st + 1);
        }
        const uint32_t kbs = kb0 + stage_off(st + 1), rbs = rb0 + stage_off(st + 1);
        bf16x8 kb[PFK];
        if (has_next) {
#pragma unroll
            for (int j = 0; j < PFK; ++j) kb[j] = kld(kbs, rbs, kstep(j));
        }

        // mask: entry r of lane half g is token tok_of(8 (r >> 2) + 4 g + (r & 3))
        // = 16 (r >> 3) + 4 (r & 3) + 2 ((r >> 2) & 1) + g of the stage, visible
        // iff < lim - p0 (only the last stage of a sequence, causal query pairs
        // and rows past the end need it)
        const int lim_rel = lim - (p_first + st * HALF) - g;
        if (__ballot(lim_rel < HALF - 1)) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                cur[r] = (16 * (r >> 3) + 4 * (r & 3) + 2 * ((r >> 2) & 1)) < lim_rel ? cur[r] : -INFINITY;
        }

        // fp8: the scores are sigma * cur and the probabilities are produced
        // multiplied by sigma (exp2 argument + log2 sigma)
        const float s_l2 = FP8 ? a.scale_log2 * sig_cur : a.scale_log2;
        const float l2sig = FP8 ? __builtin_amdgcn_logf(sig_cur) : 0.f;
        float mx = -INFINITY, m_new = m_run, m_off = 0.f, alpha = 1.f, psum = 0.f;
        bool raise = false;
        bf16x8 pcur[2];
        bf16x8 vb[PF];
        // Slice k of the softmax of stage st.  Each slice holds at most three
        // independent VALU ops; the exp2 pipeline is skewed (fma of entry r,
        // exp2 of r-1 and the sum of r-2 in one slice) so no slice waits on
        // its own results.
        auto softmax_slice = [&](int k) {
            if (k < 8) {
                mx = __builtin_fmaxf(mx, __builtin_fmaxf(cur[2 * k], cur[2 * k + 1]));
            } else if (k == 8) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx),
                                                                 false, false);
                mx = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1])) * s_l2;
                // raise the reference max only when a score passes it by RAISE_T
                raise = mx > m_run + RAISE_T;
                m_new = raise ? mx + RAISE_H : m_run;
                m_off = (m_new == -INFINITY ? 0.f : m_new) - l2sig;
            } else if (k < 28) {
                if (k == 9) alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                const int r = k - 10;
                if (r >= 2 && r < 18) psum += cur[r - 2];
                if (r >= 1 && r < 17) cur[r - 1] = __builtin_amdgcn_exp2f(cur[r - 1]);
                if (r >= 0 && r < 16) cur[r] = __builtin_fmaf(cur[r], s_l2, -m_off);
            } else {
                const int r = 2 * (k - 28);   // entries r, r+1 -> one packed pair of P
                if constexpr (H16) {
                    // one packed fp32 -> fp16 conversion per pair
                    const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{cur[r], cur[r + 1]}, f16x2));
                    pcur[(r >> 2) & 1][((r >> 3) << 2) | (r & 3)] = __builtin_bit_cast(__bf16, (uint16_t)u);
                    pcur[(r >> 2) & 1][((r >> 3) << 2) | (r & 3) + 1] = __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));
                } else {
                    pcur[(r >> 2) & 1][((r >> 3) << 2) | (r & 3)] = (__bf16)cur[r];
                    pcur[(r >> 2) & 1][((r >> 3) << 2) | (r & 3) + 1] = (__bf16)cur[r + 1];
                }
            }
        };

        if (has_next) {
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                score_mfma(nxt, kb[i % PFK], i, false);
                if (i + PFK < KS) kb[i % PFK] = kld(kbs, rbs, kstep(i + PFK));
                if (FP8 && !ROW && i == DR / 16 - 1) rope_to_latent_scale(nxt, 1.0f / sig_next);
                softmax_slice(i);
                if constexpr (COPY_AT == 1) copy_slot(i, KS);
                __builtin_amdgcn_sched_barrier(0);
            }
            asm volatile("s_nop 15" : "+v"(nxt));
        } else {
#pragma unroll
            for (int k = 0; k < KS; ++k) softmax_slice(k);
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
        l_lane = l_lane * alpha + (FP8 ? psum / sig_cur : psum);
        m_run = m_new;

        // fp8: stage st+2 is converted during the value MFMAs, into the
        // buffer of stage st-1 (free since the barrier at the top).  Every
        // wave waits for its copy of stage st+2 (stage st+3's may still be in
        // flight); the barrier makes all copies visible; the staged bytes are
        // converted in five parts between them, each part read one slot
        // ahead; the next iteration's barrier publishes the result.
        raw = tab_raw(st + 4);
        const bool conv = FP8 && st + 2 < nst_live;
        uint4 cin[2];
        uint32_t cxr = 0;
        bool czr = false;
        if constexpr (FP8) {
            if (conv) {
                if (COPY_AT != 2 && st + 3 < nst_live)
                    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();   // every wave's copy of stage st+2 has landed
                cin[0] = convert_load(st + 2, 0);
                cxr = code_xor(st + 2);
                czr = code_zero(st + 2);
            }
        }

        // value MFMAs: O^T[512 x 32] += V^T[512 x 32 tok] . P^T[32 tok x 32]
        // as two 16-token k-steps, V fragments PF MFMAs ahead
        const uint32_t vbs = vb0 + stage_off(st);
#pragma unroll
        for (int j = 0; j < PF; ++j) vb[j] = vld(vbs, j);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);   // the prefetch reads first
#pragma unroll
        for (int i = 0; i < 2 * MBLOCKS; ++i) {
            if constexpr (H16)
                oacc[i % MBLOCKS] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, vb[i % PF]), __builtin_bit_cast(f16x8, pcur[i / MBLOCKS]),
                    oacc[i % MBLOCKS], 0, 0, 0);
            else
                oacc[i % MBLOCKS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % PF], pcur[i / MBLOCKS],
                                                                            oacc[i % MBLOCKS], 0, 0, 0);
            if (i + PF < 2 * MBLOCKS) vb[i % PF] = vld(vbs, i + PF);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i + PF < 2 * MBLOCKS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            if constexpr (COPY_AT == 2) {
                __builtin_amdgcn_sched_barrier(0);
                copy_slot(i, 2 * MBLOCKS);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (FP8) {
                if (i % 6 == 4) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (conv) {
                        const int j = i / 6;
                        if (j < 4) cin[(j + 1) & 1] = convert_load(st + 2, j + 1);
                        convert_part(st + 2, cin[j & 1], j, cxr, czr);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if constexpr (FP8) sig_cur = sig_next;
    };

    // two iterations per trip so that the score accumulators swap roles
    // without register copies
    int raw = tab_raw(3);
    for (int st = 0; st < nst_live; st += 2) {
        iteration(st, sA, sB, raw);
        if (st + 1 < nst_live) iteration(st + 1, sB, sA, raw);
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

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
    // one workgroup per dispatch-table entry (a multiple of 8)
    dim3 grid((unsigned)a.grid_wgs);
    switch (a.kv_dtype) {
    case MLA_DT_BF16: launch_timed(decode_mfma_kernel<kv::Bf16>, grid, dim3(256), 0, s, a); break;
    case MLA_DT_F16: launch_timed(decode_mfma_kernel<kv::F16>, grid, dim3(256), 0, s, a); break;
    case MLA_DT_FP8_E4M3: launch_timed(decode_mfma_kernel<kv::E4m3>, grid, dim3(256), 0, s, a); break;
    case MLA_DT_FP8_E5M2: launch_timed(decode_mfma_kernel<kv::E5m2>, grid, dim3(256), 0, s, a); break;
    case MLA_DT_FP8_E4M3_ROW:
        launch_timed(decode_mfma_kernel<kv::E4m3Row>, grid, dim3(256), 0, s, a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mla

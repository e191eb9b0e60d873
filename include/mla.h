/*
 * mla.h — C ABI of the absorbed Multi-head Latent Attention decode library
 * for AMD MI355X (gfx950).
 *
 * What it computes (the pages on DeepSeek MLA):
 *   - every cached token is one row [c (d_c) | k^R (d_r)], the low-rank latent
 *     and the shared rotary key (blog.huny.dev "DeepSeek MLA 해부" §2-1 and
 *     §2-3; donmain.dev "KV Cache를 10분의 1로 줄인 MLA의 트릭", section
 *     "위치 정보와 압축의 충돌": 512 + 64 = 576);
 *   - the query's content part is absorbed through W^UK once per token
 *     (huny §3-1 absorption equation): mla_absorb_q;
 *   - all heads then attend MQA-style to the one latent "head"
 *     (blog.secrett2633.cloud "[vLLM] Multi-head Latent Attention", section
 *     "MLA의 MQA 디코딩 경로") with score q~.c + q^R.k^R (huny §2-3
 *     decomposition equation) and a softmax: mla_decode;
 *   - the latent output sum_j A c_j is mapped back through W^UV and W^O
 *     (huny §3-2 value and output equations): mla_absorb_out.
 *
 * Conventions shared by every call:
 *   - Pointers are device pointers unless the name ends in _host.
 *   - The caller owns every buffer; the library allocates nothing and keeps
 *     no device state between calls, apart from mla_decode_noalloc's scratch
 *     and the device checks' flag (mla_set_debug), both file-scope device
 *     arrays.
 *   - Calls are asynchronous on `stream`; host-side argument checks run before
 *     any launch and a failing check launches nothing.
 *   - Every call returns an mla_status_t; mla_last_error() returns a
 *     thread-local message for the last failure on the calling thread.
 *   - No C++ exception crosses the ABI.  Calls are thread-safe.
 *   - Row-major layouts throughout; "T" is the number of query tokens
 *     (B * q_len, sequence-major: token index = b * q_len + t).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *mla_stream_t; /* == hipStream_t */

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, empty cache, missing plan */
    MLA_ERR_UNSUPPORTED = 2,  /* block size != 64, dtype or dims not instantiated */
    MLA_ERR_ALIGN = 3,        /* pointer or row not 16-byte aligned */
    MLA_ERR_WORKSPACE = 4,    /* workspace smaller than the plan needs */
    MLA_ERR_HIP = 5,          /* a HIP launch or runtime call failed */
    MLA_ERR_DEVICE_CHECK = 6  /* device checks on (mla_set_debug): the block table or
                                 sequence lengths on the device are out of range */
} mla_status_t;

typedef enum {
    MLA_DT_F32 = 0,
    MLA_DT_BF16 = 1,
    MLA_DT_FP8_E4M3 = 2,      /* OCP E4M3 ("fn": no infinities, S.1111.111 = NaN) */
    MLA_DT_F16 = 3,           /* IEEE binary16 (cache rows only) */
    MLA_DT_FP8_E5M2 = 4,      /* OCP E5M2 latent codes (cache only; huny §6 "E4M3 or E5M2") */
    MLA_DT_FP8_E4M3_ROW = 5   /* the whole [c | k^R] row as E4M3 codes (cache only) */
} mla_dtype_t;

/* Tokens per paged block.  The pages' decode kernel accepts only 64-token
 * blocks, sized to its tile (vLLM MLA page, "FlashMLABackend: 하드웨어 요구사항");
 * here too a block is exactly one decode tile. */
#define MLA_BLOCK_SIZE 64

/*
 * Paged latent cache (huny §6 PagedAttention item; vLLM MLA page, the combined
 * kv_c_and_k_pe cache of "FlashMLAImpl").  `base` holds num_blocks blocks of
 * 64 token rows each:
 *   kv_dtype F32 / BF16: block = [64][d_c + d_r] rows of [c | k^R] in that type
 *                        (bf16 at d_c=512, d_r=64: 73,728 B per block);
 *   kv_dtype F16:        as BF16 with IEEE fp16 rows (a kv-cache dtype of the
 *                        vLLM MLA page, "FlashMLABackend").
 *   kv_dtype FP8_E4M3:   block = c codes [64][d_c] (e4m3) followed by k^R
 *                        [64][d_r] in bf16 (the rotary key keeps 16-bit
 *                        precision, huny §6 FP8 item; 40,960 B per block), and
 *                        block_scales[num_blocks] (fp32) holds the one
 *                        dequantisation scale of each block: c = code * scale.
 *   kv_dtype FP8_E5M2:   as FP8_E4M3 with e5m2 latent codes (huny §6).
 *   kv_dtype FP8_E4M3_ROW: block = [64][d_c + d_r] e4m3 codes of the whole
 *                        row, one scale per block for both parts:
 *                        [c | k^R] = code * scale (36,864 B per block).
 * Blocks are 256-byte aligned when base is (block bytes are multiples of 256
 * for the instantiated dims).  Rows past a sequence's length may hold
 * anything, including NaN: no result depends on them.
 *
 * flags (0 or MLA_CACHE_FP8_EXACT) choose the arithmetic of mla_decode over
 * an FP8_E4M3 cache at d_c = 512, d_r = 64 with BF16 queries.  The pages fix
 * the fp8 storage, not this arithmetic.
 *   0 (default): the codes go into 8-bit MFMAs as stored.  Each query row
 *     becomes two e4m3 terms, q~ ~= sigma_q (h + l/16) with
 *     sigma_q = max|q~| / 448.  The probabilities become two e4m3 terms of
 *     y = p 2^5 mant(|block scale|), y ~= h + l (l the residual); the exponent of the block
 *     scale rides on the value MFMA's E8M0 operand scale.  The rotary part
 *     stays on bf16.
 *   MLA_CACHE_FP8_EXACT: codes are decoded exactly to bf16, and bf16 MFMAs
 *     run the 16-bit pipeline (probabilities rounded to bf16).
 * Both keep the error within a few 1e-3 of each output row's norm on N(0,1)
 * data (two e4m3 terms carry q~ and P to ~2^-8).  The 8-bit path's score
 * error grows with the logits: a block whose scale dwarfs its data's
 * absmax / 448 (logits far beyond the rest) is better decoded exactly.
 * Block scales must be finite (any sign; zero allowed).  Both arithmetics
 * bound tiny scales to keep their fp32 intermediates in range: the 8-bit
 * path clamps the exponent at -122 (the mantissa then shrinks), the exact
 * path (and the e5m2 / whole-row formats, which always take it) raises
 * magnitudes below 2^-64 to 2^-64 — a block with such a scale holds latent
 * values below 448 * 2^-64, negligible next to any block of ordinary scale.
 * Every other format and shape ignores flags.
 */
#define MLA_CACHE_FP8_EXACT 1

typedef struct {
    const void *base;
    const float *block_scales;  /* FP8_E4M3 only, else NULL */
    int64_t num_blocks;
    int32_t block_size;         /* must be MLA_BLOCK_SIZE */
    int32_t d_c;                /* latent width */
    int32_t d_r;                /* rotary key width */
    mla_dtype_t kv_dtype;
    int32_t flags;              /* 0 or MLA_CACHE_FP8_EXACT (see above) */
} mla_cache_desc_t;

/*
 * Split-KV plan (the tile-scheduler metadata of the vLLM MLA page,
 * get_mla_metadata / num_splits in "MLA의 MQA 디코딩 경로" and "FP8 MLA 지원").
 * Filled by mla_decode_plan on the host.
 */
typedef struct {
    int32_t B, q_len, n_h, d_c;
    int32_t num_items;      /* work items: block ranges of one (sequence, row chunk) */
    int32_t row_chunks;     /* query-row chunks per sequence (128 rows each) */
    int32_t num_partials;   /* partial-result slots (items of split segments) */
    int32_t needs_combine;  /* 1 if mla_decode launches the LSE combine */
    int32_t max_splits;     /* largest item count of any (sequence, row chunk) */
    int32_t blocks_per_item;/* largest block count of any item */
    int32_t partial_dtype;  /* element type of the partial outputs in the workspace:
                               BF16 for the MFMA shapes (d_c 512, d_r 64, bf16/fp8
                               cache), F32 otherwise */
    int64_t plan_ints;      /* int32 entries of the device plan */
    int64_t workspace_bytes;/* partial-result workspace mla_decode needs */
    int32_t grid_wgs;       /* workgroups of the MFMA decode launch (dispatch-table entries) */
    int32_t kv_dtype;       /* cache format the plan was built for (mla_dtype_t) */
    int32_t d_r;            /* rotary width the plan was built for */
    int32_t max_seq_blocks; /* largest ceil(seq_lens[b] / 64): mla_decode needs
                               bt_stride >= this */
} mla_plan_t;

/*
 * mla_decode_plan — host only, pure, makes no HIP call.
 *
 * Cuts the work, every (sequence, row chunk) segment of ceil(seq_len/64)
 * blocks, into work items (contiguous block ranges) for `num_cus` compute
 * units: the segments, in order, are packed into at most num_cus bins so
 * that the largest bin cost is minimal (cost of an item = its 32-token
 * stages + 6 for its prologue and epilogue; a bin takes whole segments while
 * they fit, then whole blocks of the next), and the pieces of that packing
 * are the items.  Items run one per workgroup; a dispatch table orders them
 * longest first per XCD (workgroup k runs on XCD k % 8), by simulating
 * list scheduling on num_cus/8 compute units per XCD.
 *
 * seq_lens_host [B]: tokens per sequence, counting the q_len query tokens
 *                    (each query token's own row is already in the cache).
 * plan_host:         int32 array of plan_capacity entries, or NULL to only
 *                    size the plan (info is filled either way).
 * Layout written (int32): header[8] = {num_items, B, row_chunks,
 *                 num_partials, grid_wgs, 0, 0, 0},
 *                 items[num_items][4] = {b * row_chunks + chunk, blk_begin,
 *                 blk_end, slot (-1 = final)} (a segment of an empty
 *                 sequence has one item with blk_begin == blk_end),
 *                 wg_item[grid_wgs] (item of each decode workgroup, -1 = none),
 *                 split_off[B * row_chunks + 1] (partial slots of segment
 *                 s = b * row_chunks + chunk are split_off[s] .. split_off[s+1]-1),
 *                 seq_flags[B * row_chunks] (1 = decode writes the segment's
 *                 final output directly).
 * The caller copies plan_host to device memory (plan_ints int32 entries)
 * and passes it to mla_decode with the same seq_lens.
 * Errors: INVALID_ARG for B < 1, q_len < 1, n_h < 1, negative lengths,
 * num_cus < 1, a too-small plan_capacity; UNSUPPORTED for dtypes.
 */
mla_status_t mla_decode_plan(const int32_t *seq_lens_host, int32_t B, int32_t q_len,
                             int32_t n_h, int32_t d_c, int32_t d_r, mla_dtype_t kv_dtype,
                             int32_t num_cus, int32_t *plan_host, int64_t plan_capacity,
                             mla_plan_t *info);

/*
 * mla_decode — absorbed MLA decode over the paged latent cache.
 *
 * For query row (b, t, h): visible positions p <= seq_lens[b] - q_len + t
 * (speculative multi-token queries are causal within the step, vLLM MLA
 * page "FlashMLAImpl", reshape for spec decode);
 *   s_p   = scale * (q_lat[b,t,h] . c_p + q_rope[b,t,h] . k^R_p)
 *   o_lat = sum_p softmax(s)_p c_p       (latent-space value sum, huny §3-2)
 *   lse   = ln sum_p exp(s_p)            (natural log; vLLM MLA page,
 *                                         can_return_lse_for_decode)
 * A row with no visible position gets o_lat = 0 and lse = -inf.
 *
 * q_lat  [T][n_h][d_c], q_rope [T][n_h][d_r] in q_dtype (F32 or BF16); the
 *        pages pass q as the pair (q_nope_absorbed, q_pe) — here two pointers.
 * cache  see mla_cache_desc_t.  Fast paths: every kv dtype but F32 with q BF16,
 *        d_c = 512, d_r = 64 (MFMA); every other supported combination runs a
 *        generic kernel (d_c <= 1024, d_r <= 256, d_c and d_r multiples of 4).
 * block_table [B][bt_stride] int32 pool block ids; entries past
 *        ceil(seq_lens[b]/64) are never read.  bt_stride must cover the
 *        longest planned sequence (bt_stride >= plan->max_seq_blocks).  Ids
 *        outside [0, num_blocks) are clamped into it (no fault; a correct
 *        table holds none).
 * seq_lens [B] int32 (device), the same values the plan was built from
 *        (the kernels read at most the planned blocks of each sequence).
 * scale  softmax scale; the pages give none — the absorbed score keeps the
 *        un-absorbed logits, so pass 1/sqrt(d_nope + d_r) for those.
 * plan / plan_dev  from mla_decode_plan (host struct, device copy).
 * workspace  >= plan->workspace_bytes (may be NULL if that is 0), 256-B aligned.
 * o_lat  [T][n_h][d_c] in q_dtype; lse [T][n_h] fp32.
 * Errors: INVALID_ARG (nulls, sizes, num_blocks < 1, a plan built for
 * another B / q_len / n_h / d_c / d_r / kv dtype, bt_stride below
 * plan->max_seq_blocks), UNSUPPORTED (block_size != 64, dims/dtypes), ALIGN,
 * WORKSPACE, HIP.
 */
mla_status_t mla_decode(const void *q_lat, const void *q_rope, mla_dtype_t q_dtype,
                        const mla_cache_desc_t *cache, const int32_t *block_table,
                        int32_t bt_stride, const int32_t *seq_lens, int32_t B, int32_t q_len,
                        int32_t n_h, float scale, const mla_plan_t *plan,
                        const int32_t *plan_dev, void *workspace, int64_t workspace_bytes,
                        void *o_lat, float *lse, mla_stream_t stream);

/*
 * mla_decode_noalloc — mla_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and results, with the
 * split partials in a scratch array the library holds in device memory
 * instead of a caller workspace.  It calls no hipMalloc / hipFree and no
 * allocating routine.  Limit: plan->workspace_bytes <=
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB: every configuration of 256 work items
 * of up to 256 query rows), else MLA_ERR_WORKSPACE before any HIP call.
 * Each GPU the library runs on holds one scratch array (64 MiB) until the
 * process ends; its address is looked up once per device on the first call
 * there (with that device current).  Every call on a GPU shares that GPU's
 * scratch, which keeps the last call's contents (nothing in it has to start
 * at zero): calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.  Arguments and other errors
 * are those of mla_decode without workspace / workspace_bytes.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64 << 20)
mla_status_t mla_decode_noalloc(const void *q_lat, const void *q_rope, mla_dtype_t q_dtype,
                                const mla_cache_desc_t *cache, const int32_t *block_table,
                                int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                                int32_t q_len, int32_t n_h, float scale, const mla_plan_t *plan,
                                const int32_t *plan_dev, void *o_lat, float *lse,
                                mla_stream_t stream);

/*
 * mla_decode_partial / mla_decode_finish — mla_decode in its two launches.
 * mla_decode_partial runs the split decode kernel alone: sequences with one
 * split get their final o_lat / lse, the others leave normalised partials
 * and their lse in the workspace.  mla_decode_finish then runs the LSE
 * combine for the plan (nothing if plan->needs_combine is 0), writing the
 * remaining rows of o_lat (out_dtype = the query dtype) and lse.  Calling
 * both, in order, on one stream is exactly mla_decode; they exist so that a
 * caller can place other work or timing events between the two launches.
 * Arguments and errors are those of mla_decode.
 */
mla_status_t mla_decode_partial(const void *q_lat, const void *q_rope, mla_dtype_t q_dtype,
                                const mla_cache_desc_t *cache, const int32_t *block_table,
                                int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                                int32_t q_len, int32_t n_h, float scale, const mla_plan_t *plan,
                                const int32_t *plan_dev, void *workspace,
                                int64_t workspace_bytes, void *o_lat, float *lse,
                                mla_stream_t stream);
mla_status_t mla_decode_finish(const mla_plan_t *plan, const int32_t *plan_dev, void *workspace,
                               int64_t workspace_bytes, mla_dtype_t out_dtype, void *o_lat,
                               float *lse, mla_stream_t stream);

/*
 * mla_combine_lse — merge per-split partial results (the num_splits
 * reduction named on the vLLM MLA page, "FP8 MLA 지원").  For each sequence b
 * and row r, with slots k in [split_off[b], split_off[b+1]):
 *   M = max_k lse_k;  w_k = exp(lse_k - M);
 *   o = sum_k w_k o_k / sum_k w_k;  lse = M + ln sum_k w_k.
 * Slots with lse = -inf carry no weight; a sequence whose slots are all -inf
 * (or that has none) gets o = 0, lse = -inf.
 * o_part [P][rows][d_c] fp32 (normalised partial outputs, 16-byte aligned;
 * d_c a multiple of 4, at most 1024), lse_part [P][rows] fp32, split_off [B+1] int32, seq_flags [B] int32 or NULL: sequences with
 * flag 1 are skipped (their output is already final).  rows = q_len * n_h.
 * o_lat [B*rows][d_c] in out_dtype (F32 or BF16); lse [B*rows] fp32.
 */
mla_status_t mla_combine_lse(const float *o_part, const float *lse_part,
                             const int32_t *split_off, const int32_t *seq_flags, int32_t B,
                             int32_t rows, int32_t d_c, void *o_lat, mla_dtype_t out_dtype,
                             float *lse, mla_stream_t stream);

/*
 * mla_absorb_q — W^UK query absorption (huny §3-1; donmain "위치 정보와
 * 압축의 충돌", q~ = W^UK^T q):
 *   q_lat[t][h][:] = q_nope[t][h][:] . W_UK[h]^T
 * q_nope [T][n_h][d_nope] with token stride ld_q elements (>= n_h*d_nope),
 * w_uk [n_h][d_c][d_nope] (W^UK_i maps the latent to head i's key,
 * k = c W^UK_i), q_lat [T][n_h][d_c].  dt F32 or BF16 for all three;
 * accumulation in fp32.  BF16 with d_c % 32 == 0 and d_nope % 16 == 0 runs
 * on MFMA.
 */
mla_status_t mla_absorb_q(const void *q_nope, int64_t ld_q, const void *w_uk, void *q_lat,
                          int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c,
                          mla_dtype_t dt, mla_stream_t stream);

/*
 * mla_absorb_out — map the latent output back (huny §3-2 value and output
 * equations):
 *   u[t][h][:] = o_lat[t][h][:] . W_UV[h]          (W_UV [n_h][d_c][d_v])
 *   out[t][:]  = sum_h u[t][h][:] . W_O[h*d_v:(h+1)*d_v][:]  (W_O [n_h*d_v][d_model])
 * u_ws [T][n_h][d_v] receives u (caller-provided, same dtype); out [T][d_model].
 * f32_ws: fp32 scratch of at least mla_absorb_out_workspace() bytes (split-K
 * partial sums of out); may be NULL when that is 0.
 * dt F32 or BF16; accumulation in fp32.
 */
int64_t mla_absorb_out_workspace(int32_t T, int32_t n_h, int32_t d_v, int32_t d_model,
                                 mla_dtype_t dt);
mla_status_t mla_absorb_out(const void *o_lat, const void *w_uv, const void *w_o, void *u_ws,
                            void *out, void *f32_ws, int64_t f32_ws_bytes, int32_t T,
                            int32_t n_h, int32_t d_c, int32_t d_v, int32_t d_model,
                            mla_dtype_t dt, mla_stream_t stream);

/*
 * mla_gather_paged — copy each sequence's logical rows out of the pool:
 *   out[b][p][:] = row bytes of token p of sequence b, p < seq_lens[b]
 * (block bt[b][p/64], slot p%64).  Row bytes: (d_c + d_r) * elem for F32 /
 * BF16; for FP8_E4M3 the d_c code bytes followed by the 2*d_r bytes of the
 * bf16 rotary key.  out is [B][max_tokens][row bytes]; rows past seq_lens[b]
 * are not written.  Bit-exact byte copy.  max_tokens must not exceed
 * 64 * bt_stride (INVALID_ARG); block ids outside [0, num_blocks) are
 * clamped into it.
 */
mla_status_t mla_gather_paged(const mla_cache_desc_t *cache, const int32_t *block_table,
                              int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                              int32_t max_tokens, void *out, mla_stream_t stream);

/*
 * Rotary embedding of the decoupled RoPE parts (huny §2-3 rotary key and
 * rotary query; donmain "위치 정보와 압축의 충돌").  Adjacent pairs
 * (2j, 2j+1) of a d_r-wide vector at position p turn by p * theta'_j and the
 * result is multiplied by mscale.
 *   factor == 1: plain RoPE, theta'_j = base^(-2j/d_r).
 *   factor  > 1: YaRN.  The huny page (§6, YaRN item) names the method for
 *     128K+ contexts and asks that base and scaling factor match the model,
 *     with no formula; this follows the published YaRN "NTK-by-parts" rule:
 *     pair j turns r_j = orig_ctx * theta_j / (2 pi) times over the original
 *     context; gamma_j = clamp((r_j - beta_slow) / (beta_fast - beta_slow), 0, 1);
 *     theta'_j = (1 - gamma_j) theta_j / factor + gamma_j theta_j.
 *     YaRN's magnitude factor (0.1 ln(factor) + 1 in the published method)
 *     is the caller's mscale; a model that folds it into the softmax scale
 *     passes 1 here.
 * Angles are formed and rotated from fp64 p * theta'_j.
 */
typedef struct {
    double base;        /* > 1, e.g. 10000 */
    double factor;      /* > 0; 1 = plain RoPE */
    double orig_ctx;    /* original context length (factor != 1) */
    double beta_fast;   /* pairs turning >= beta_fast times keep theta_j */
    double beta_slow;   /* pairs turning <= beta_slow times use theta_j / factor */
    double mscale;      /* > 0; multiplies every rotated vector */
} mla_rope_t;

/* theta'_j for j < d_r/2 into theta_host (host only, no HIP call).
 * INVALID_ARG on NULLs, d_r odd, < 2 or > 256, or out-of-range fields. */
mla_status_t mla_rope_freqs(const mla_rope_t *rope, int32_t d_r, double *theta_host);

/*
 * mla_cache_append — write the cache rows of q_len new tokens per sequence
 * (huny §2-1 compression equation c = h W^DKV and §2-3 shared rotary key
 * k^R = RoPE(h W^KR); the row [c | k^R] is the kv_c_and_k_pe cache row of
 * the vLLM MLA page, "FlashMLAImpl"):
 *   token t = b * q_len + i of sequence b, at position p = pos0[b] + i:
 *   [c | k^R] = h[t] . w_kv, k^R rotated at p (see mla_rope_t), stored in
 *   slot p % 64 of block block_table[b][p / 64].
 * h [T][d_model], w_kv [d_model][d_c + d_r] (W^DKV then W^KR columns), both
 * dt (F32 or BF16); accumulation in fp32; pos0 [B] int32 (device).  The block
 * table must already hold blocks for every written position; a token whose
 * table entry lies outside [0, num_blocks) (an unallocated slot such as -1)
 * is not written, nor is a token at p < 0 or p >= 64 bt_stride, so no other
 * block is touched.  Storage: F32 / BF16 rows rounded once to
 * nearest even.  FP8_E4M3 (huny §6 FP8 item: a dynamic scale per block; the
 * pages give no update rule — the reading here): a block whose slot 0 is
 * written by this call takes scale amax|c| / 448 over the tokens written
 * into it (1 if 0); otherwise scale' = max(scale, amax / 448), and when it
 * grows the codes of the slots before the first written one are re-encoded
 * at scale' (code' = e4m3(value(code) * scale / scale')).  New codes are
 * e4m3(c / scale') (nearest even, saturating at 448); k^R is bf16.
 * cache->base and cache->block_scales are written (the descriptor's const
 * describes the decode's use).  Sequences of one call must be distinct.
 * workspace: >= mla_cache_append_workspace() bytes, 256-byte aligned (fp32
 * partial products).  rope may be NULL only when d_r == 0.
 * Errors: INVALID_ARG, UNSUPPORTED (dt, cache format), ALIGN, WORKSPACE, HIP.
 */
int64_t mla_cache_append_workspace(int32_t T, int32_t d_model, int32_t d_c, int32_t d_r,
                                   mla_dtype_t dt);
mla_status_t mla_cache_append(const void *h, const void *w_kv, mla_dtype_t dt,
                              const mla_cache_desc_t *cache, const int32_t *block_table,
                              int32_t bt_stride, const int32_t *pos0, int32_t B, int32_t q_len,
                              int32_t d_model, const mla_rope_t *rope, void *workspace,
                              int64_t workspace_bytes, mla_stream_t stream);

/*
 * mla_project_q — the decode's query inputs straight from the hidden states
 * (huny §2-2 low-rank query c^Q = h W^DQ, q^C_i = c^Q W^UQ_i; §2-3 rotary
 * query q^R_i = RoPE(h W^QR_i), read from h as written there; §3-1 absorption
 * q~_i = q^C_i W^UK_i^T):
 *   q_lat [T][n_h][d_c] = q~,  q_rope [T][n_h][d_r] = q^R rotated at pos[t].
 * h [T][d_model], w_dq [d_model][q_lora], w_uq [q_lora][n_h d_nope] (head i
 * = columns i d_nope ..), w_qr [d_model][n_h d_r], w_uk [n_h][d_c][d_nope];
 * all dt (F32 or BF16), pos [T] int32 (device).  fp32 accumulation; on the
 * bf16 MFMA path c^Q and q^C are rounded to bf16 between the products.
 * W^UQ and W^UK stay two products: the merged W^UQ W^UK^T would hold
 * n_h * q_lora * d_c weights against q_lora * n_h * d_nope + n_h * d_c *
 * d_nope (201 MB against 67 MB at the DeepSeek-V2 shape).
 * workspace >= mla_project_q_workspace() bytes, 256-byte aligned.
 */
int64_t mla_project_q_workspace(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h,
                                int32_t d_nope, int32_t d_c, int32_t d_r, mla_dtype_t dt);
mla_status_t mla_project_q(const void *h, const void *w_dq, const void *w_uq, const void *w_qr,
                           const void *w_uk, mla_dtype_t dt, const int32_t *pos, int32_t T,
                           int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope,
                           int32_t d_c, int32_t d_r, const mla_rope_t *rope, void *q_lat,
                           void *q_rope, void *workspace, int64_t workspace_bytes,
                           mla_stream_t stream);

/*
 * mla_project_step — one decode step's producers from the same hidden states:
 * the queries of mla_project_q and the cache rows of mla_cache_append in
 * three launches instead of five.  Both read h through a down-projection
 * (huny §2-2 c^Q = h W^DQ, §2-1 c = h W^DKV, §2-3 k^R = RoPE(h W^KR)), so
 * the three weights come side by side in one matrix and share one product
 * with h W^QR (§2-3 rotary query); one finishing launch sums the partials
 * into c^Q, q^R and the cache rows; c^Q W^UQ with the W^UK absorption
 * follows (§3-1).
 *   token t = b * q_len + i of sequence b sits at p = pos0[b] + i: q^R of t is
 *   rotated at p and its cache row [c | k^R] goes to slot p % 64 of block
 *   block_table[b][p / 64], exactly as mla_cache_append writes it (same
 *   storage rules, scale rule and skipped positions for every cache format).
 * h [B q_len][d_model]; w_dkvq [d_model][q_lora + d_c + d_r] = the columns of
 * W^DQ, then W^DKV, then W^KR (d_c, d_r from the cache descriptor); w_uq,
 * w_qr, w_uk, q_lat, q_rope as in mla_project_q (T = B q_len).  All BF16,
 * fp32 accumulation, c^Q rounded to bf16 before W^UQ.  q_lat and q_rope are
 * bit-identical to mla_project_q's for the same inputs; the cache rows take
 * another split of the d_model sum than mla_cache_append's (fp32 partials),
 * so they may differ from its rows by rounding.  Sequences of one call must
 * be distinct.  One rope configuration serves q^R and k^R.
 * Shapes: the bf16 MFMA path of mla_project_q (d_model and q_lora multiples
 * of 64, n_h d_nope and n_h d_r multiples of 8, d_nope a multiple of 64, d_c
 * of 128, q_lora + d_c + d_r a multiple of 8); mla_project_step_workspace()
 * returns 0 for any other shape or dtype, and the call UNSUPPORTED (use the
 * two separate calls).
 * workspace >= mla_project_step_workspace() bytes, 256-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGN, WORKSPACE, HIP.
 */
int64_t mla_project_step_workspace(int32_t B, int32_t q_len, int32_t d_model, int32_t q_lora,
                                   int32_t n_h, int32_t d_nope, int32_t d_c, int32_t d_r,
                                   mla_dtype_t dt);
mla_status_t mla_project_step(const void *h, const void *w_dkvq, const void *w_uq, const void *w_qr,
                              const void *w_uk, mla_dtype_t dt, const mla_cache_desc_t *cache,
                              const int32_t *block_table, int32_t bt_stride, const int32_t *pos0,
                              int32_t B, int32_t q_len, int32_t d_model, int32_t q_lora, int32_t n_h,
                              int32_t d_nope, const mla_rope_t *rope, void *q_lat, void *q_rope,
                              void *workspace, int64_t workspace_bytes, mla_stream_t stream);

/*
 * mla_clock_probe — measurement helper, not a step of the path: `wgs`
 * workgroups of 4 waves each run a dependent chain of `iters` bf16
 * 32x32x16 MFMAs, and out[2k], out[2k+1] (int64, device) receive the shader
 * cycles (s_memtime) and 100 MHz real-time ticks (s_memrealtime) workgroup k
 * spent in it, so that out[2k] / out[2k+1] * 100 MHz is the shader clock
 * under matrix-core load.  INVALID_ARG for NULL out, wgs outside [1, 65536]
 * or iters outside [1, 2^24]; ALIGN for an out not 8-byte aligned.
 */
mla_status_t mla_clock_probe(int64_t *out, int32_t wgs, int32_t iters, mla_stream_t stream);

/*
 * mla_set_launch_events — measurement helper, not a step of the path: the
 * next `pairs` kernel launches that the decode entry points make on the
 * calling thread (the decode kernel, then the combine when one runs) record
 * their own start and stop times into events[2k] and events[2k+1]
 * (hipEvent_t created with timing; hipEventElapsedTime between the two gives
 * the kernel's duration).  The timestamps come from the kernel's dispatch
 * (hipExtLaunchKernel), so no marker enters the stream between launches.
 * Pairs a call does not consume are dropped by the next call to this
 * function.  INVALID_ARG for pairs outside [0, 16] or NULL events.
 * mla_launch_events_used returns how many of the pairs set last have been
 * consumed by launches on the calling thread.
 */
mla_status_t mla_set_launch_events(void *const *events, int32_t pairs);
int32_t mla_launch_events_used(void);

/*
 * mla_set_debug / mla_debug — device checks of the data the host cannot see
 * (block ids and slots of a device-resident block table; the block and its
 * 64 slots per position are the paged layout of vLLM MLA page,
 * "FlashMLABackend: 하드웨어 요구사항").  When on,
 * mla_decode, mla_decode_partial, mla_decode_noalloc and mla_gather_paged,
 * after their host checks, first run a check kernel on `stream` over the
 * device block table and sequence lengths and wait for it; if any sequence
 * length is negative or above 64 * bt_stride, or any table entry for a
 * position below its sequence's length lies outside [0, num_blocks), the
 * call launches nothing else and returns MLA_ERR_DEVICE_CHECK, naming the
 * first offence in mla_last_error().  The checked calls synchronize the
 * stream (not for graph capture) and share one flag per device, so checked
 * calls that overlap on one GPU race.  Off by default; the environment
 * variable MLA_DEBUG set to a non-zero integer turns it on at the first
 * call that consults it.  mla_set_debug(0 | 1) overrides; mla_debug returns
 * the current state.
 */
mla_status_t mla_set_debug(int32_t on);
int32_t mla_debug(void);

/* Bytes of the whole pool described by `cache` (0 on bad arguments). */
int64_t mla_cache_bytes(const mla_cache_desc_t *cache);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char *mla_last_error(void);

/* Library version string. */
const char *mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */

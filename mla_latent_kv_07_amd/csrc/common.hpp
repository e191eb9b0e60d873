// Internal declarations shared by the host layer and the kernels of libmla.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

constexpr int kBlock = MLA_BLOCK_SIZE;   // tokens per paged block == decode tile
constexpr int kRowsPerChunk = 128;       // query rows handled by one workgroup

// Everything a decode kernel needs, resolved and validated on the host.
struct DecodeArgs {
    const void *q_lat;
    const void *q_rope;
    const void *pool;
    const float *block_scales;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const int32_t *plan;       // device plan (header, items, split_off, seq_flags)
    void *o_part;              // [num_partials][rows][d_c] in partial_dtype
    float *lse_part;           // [num_partials][rows]
    void *o_lat;
    float *lse;
    int64_t block_bytes;
    int64_t num_pool_blocks;   // block ids are clamped to [0, num_pool_blocks)
    int32_t bt_stride, B, q_len, n_h, d_c, d_r;
    int32_t rows;              // q_len * n_h
    int32_t num_items, row_chunks, grid_wgs;
    float scale_log2;          // scale * log2(e)
    mla_dtype_t q_dtype, kv_dtype, partial_dtype;
    int32_t cache_flags;       // mla_cache_desc_t::flags
};

// Plan layout (int32 entries): header[8] = {num_items, B, row_chunks,
// num_partials, grid_wgs, 0, 0, 0}; items[num_items][4] = {b * row_chunks +
// chunk, blk_begin, blk_end, slot}; wg_item[grid_wgs] (the item of each MFMA
// decode workgroup, -1 for none); split_off[B * row_chunks + 1];
// seq_flags[B * row_chunks].
constexpr int kPlanHeader = 8;
__host__ __device__ inline int64_t plan_items_off() { return kPlanHeader; }
__host__ __device__ inline int64_t plan_wg_off(int32_t num_items) { return kPlanHeader + 4 * (int64_t)num_items; }
__host__ __device__ inline int64_t plan_split_off(int32_t num_items, int32_t grid_wgs) {
    return plan_wg_off(num_items) + grid_wgs;
}
__host__ __device__ inline int64_t plan_flags_off(int32_t num_items, int32_t grid_wgs, int32_t num_seg) {
    return plan_split_off(num_items, grid_wgs) + num_seg + 1;
}

// Measurement hook (mla_set_launch_events): the start / stop events the
// next kernel launch on this thread records its own timestamps into (none:
// nullptr), consumed in order by the launch sites below.
struct LaunchTiming {
    hipEvent_t start, stop;
};
LaunchTiming next_launch_timing();

// A kernel launch that takes the next pair of measurement events, if any
// (hipExtLaunchKernel stamps them from the kernel's own dispatch: no extra
// packet enters the stream).
template <typename F, typename... Args>
inline void launch_timed(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
    const LaunchTiming t = next_launch_timing();
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, t.start, t.stop, 0u, args...);
}

hipError_t launch_decode_generic(const DecodeArgs &a, hipStream_t s);
// MFMA decode of the DeepSeek-V2 shape (d_c 512, d_r 64, bf16 queries) for
// every 16-bit and 8-bit cache format
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s);
// the same shape over an e4m3 latent cache on the 8-bit matrix cores (eight
// waves per workgroup, two per SIMD)
hipError_t launch_decode_f8w8(const DecodeArgs &a, hipStream_t s);
// split_off / seq_flags are indexed by b * ceil(rows / chunk_rows) + r / chunk_rows
// segments with more splits than this merge on a workgroup per row
constexpr int kWideCombineSplits = 16;
hipError_t launch_combine(const void *o_part, mla_dtype_t part_dt, const float *lse_part,
                          const int32_t *split_off, const int32_t *seq_flags, int32_t B,
                          int32_t rows, int32_t chunk_rows, int32_t d_c, void *o_lat,
                          mla_dtype_t out_dt, float *lse, int32_t max_splits, hipStream_t s);
hipError_t launch_gather(const uint8_t *pool, int64_t block_bytes, int64_t num_blocks, int32_t c_bytes,
                         int32_t r_bytes, bool split_rows, const int32_t *bt, int32_t bt_stride,
                         const int32_t *seq_lens, int32_t B, int32_t max_tokens, uint8_t *out,
                         hipStream_t s);
hipError_t launch_table_check(const int32_t *bt, int64_t bt_stride, const int32_t *seq_lens, int32_t B,
                              int64_t num_blocks, int32_t *flag, hipStream_t s);
hipError_t launch_clock_probe(int64_t *out, int32_t wgs, int32_t iters, hipStream_t s);
hipError_t launch_absorb_q(const void *q_nope, int64_t ld_q, const void *w_uk, void *q_lat,
                           int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c, mla_dtype_t dt,
                           hipStream_t s);
int64_t absorb_out_workspace(int32_t T, int32_t n_h, int32_t d_v, int32_t d_model,
                             mla_dtype_t dt);
hipError_t launch_absorb_out(const void *o_lat, const void *w_uv, const void *w_o, void *u_ws,
                             void *out, float *ws, int32_t T, int32_t n_h, int32_t d_c,
                             int32_t d_v, int32_t d_model, mla_dtype_t dt, hipStream_t s);

// RoPE frequency table of one call (plain or YaRN), passed by value.
constexpr int kMaxRopePairs = 128;
struct RopeTab {
    double theta[kMaxRopePairs];   // angle per position of pair j
    float mscale;                  // factor on every rotated vector
    int32_t half;                  // d_r / 2
};
bool rope_table(const mla_rope_t *r, int32_t d_r, RopeTab *t);

int64_t cache_append_workspace(int32_t T, int32_t d_model, int32_t d_c, int32_t d_r, mla_dtype_t dt);
hipError_t launch_cache_append(const void *h, const void *w_kv, mla_dtype_t dt, uint8_t *pool,
                               float *scales, int64_t block_bytes, int64_t num_blocks,
                               mla_dtype_t kv, const int32_t *bt, int32_t bt_stride,
                               const int32_t *pos0, int32_t B, int32_t q_len, int32_t d_model,
                               int32_t d_c, int32_t d_r, const RopeTab &rt, float *ws,
                               hipStream_t s);
int64_t project_q_workspace(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope,
                            int32_t d_c, int32_t d_r, mla_dtype_t dt);
hipError_t launch_project_q(const void *h, const void *w_dq, const void *w_uq, const void *w_qr,
                            const void *w_uk, mla_dtype_t dt, const int32_t *pos, int32_t T,
                            int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope, int32_t d_c,
                            int32_t d_r, const RopeTab &rt, void *q_lat, void *q_rope, void *ws,
                            hipStream_t s);
bool project_step_ok(mla_dtype_t dt, int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope,
                     int32_t d_c, int32_t d_r);
int64_t project_step_workspace(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_c,
                               int32_t d_r);
hipError_t launch_project_step(const void *h, const void *w_dkvq, const void *w_uq, const void *w_qr,
                               const void *w_uk, uint8_t *pool, float *scales, int64_t block_bytes,
                               int64_t num_blocks, mla_dtype_t kv, const int32_t *bt, int32_t bt_stride,
                               const int32_t *pos0, int32_t B, int32_t q_len, int32_t d_model, int32_t q_lora,
                               int32_t n_h, int32_t d_c, int32_t d_r, const RopeTab &rt, void *q_lat,
                               void *q_rope, void *ws, hipStream_t s);

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace mla

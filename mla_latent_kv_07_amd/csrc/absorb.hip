// Query absorption (W^UK) and output absorption (W^UV, then W^O).
//   q_lat[t][h][:] = q_nope[t][h][:] . W_UK[h]^T        huny.dev "DeepSeek MLA 해부" §3-1
//   u[t][h][:]     = o_lat[t][h][:] . W_UV[h]           §3-2 value equation
//   out[t][:]      = sum_h u[t][h][:] . W_O[h-block]    §3-2 output equation
// This file holds the generic (any shape, fp32 or bf16, fp32 accumulation)
// kernels; the bf16 MFMA kernels for the DeepSeek-V2 shape are in
// absorb_mfma.hip and are preferred by the launchers when the shape allows.
#include "common.hpp"

namespace mla {

bool absorb_q_mfma_ok(int32_t d_nope, int32_t d_c, mla_dtype_t dt);
hipError_t launch_absorb_q_mfma(const void *q_nope, int64_t ld_q, const void *w_uk, void *q_lat,
                                int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c,
                                hipStream_t s);
bool absorb_out_mfma_ok(int32_t n_h, int32_t d_c, int32_t d_v, int32_t d_model, mla_dtype_t dt);
int64_t absorb_out_mfma_workspace(int32_t T, int32_t n_h, int32_t d_v, int32_t d_model);
hipError_t launch_absorb_out_mfma(const void *o_lat, const void *w_uv, const void *w_o,
                                  void *u_ws, void *out, float *ws, int32_t T, int32_t n_h,
                                  int32_t d_c, int32_t d_v, int32_t d_model, hipStream_t s);

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i) {
    if constexpr (sizeof(T) == 2)
        return bf16_to_f32(p[i]);
    else
        return p[i];
}

template <typename T>
__device__ __forceinline__ void st(T *p, int64_t i, float v) {
    if constexpr (sizeof(T) == 2)
        p[i] = f32_to_bf16(v);
    else
        p[i] = v;
}

// one thread per output (t, h, c)
template <typename T>
__global__ __launch_bounds__(256) void absorb_q_generic(const T *__restrict__ q_nope, int64_t ld_q,
                                                        const T *__restrict__ w_uk,
                                                        T *__restrict__ q_lat, int32_t T_,
                                                        int32_t n_h, int32_t d_nope, int32_t d_c) {
    const int64_t total = (int64_t)T_ * n_h * d_c;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int c = (int)(i % d_c);
        const int h = (int)((i / d_c) % n_h);
        const int64_t t = i / ((int64_t)d_c * n_h);
        const T *q = q_nope + t * ld_q + (int64_t)h * d_nope;
        const T *w = w_uk + ((int64_t)h * d_c + c) * d_nope;
        float acc = 0.f;
        for (int k = 0; k < d_nope; ++k) acc += ld(q, k) * ld(w, k);
        st(q_lat, i, acc);
    }
}

// u[t][h][v] = sum_c o[t][h][c] W_UV[h][c][v]; one thread per (t, h, v)
template <typename T>
__global__ __launch_bounds__(256) void absorb_uv_generic(const T *__restrict__ o_lat,
                                                         const T *__restrict__ w_uv,
                                                         T *__restrict__ u, int32_t T_,
                                                         int32_t n_h, int32_t d_c, int32_t d_v) {
    const int64_t total = (int64_t)T_ * n_h * d_v;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int v = (int)(i % d_v);
        const int h = (int)((i / d_v) % n_h);
        const int64_t t = i / ((int64_t)d_v * n_h);
        const T *o = o_lat + (t * n_h + h) * d_c;
        const T *w = w_uv + (int64_t)h * d_c * d_v + v;
        float acc = 0.f;
        for (int c = 0; c < d_c; ++c) acc += ld(o, c) * ld(w, (int64_t)c * d_v);
        st(u, i, acc);
    }
}

// out[t][d] = sum_k u[t][k] W_O[k][d], k over n_h * d_v; one thread per (t, d)
template <typename T>
__global__ __launch_bounds__(256) void absorb_o_generic(const T *__restrict__ u,
                                                        const T *__restrict__ w_o,
                                                        T *__restrict__ out, int32_t T_,
                                                        int32_t K, int32_t d_model) {
    const int64_t total = (int64_t)T_ * d_model;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int d = (int)(i % d_model);
        const int64_t t = i / d_model;
        const T *ur = u + t * K;
        float acc = 0.f;
        for (int k = 0; k < K; ++k) acc += ld(ur, k) * ld(w_o, (int64_t)k * d_model + d);
        st(out, i, acc);
    }
}

unsigned grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    return (unsigned)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

}  // namespace

hipError_t launch_absorb_q(const void *q_nope, int64_t ld_q, const void *w_uk, void *q_lat,
                           int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c, mla_dtype_t dt,
                           hipStream_t s) {
    if (absorb_q_mfma_ok(d_nope, d_c, dt))
        return launch_absorb_q_mfma(q_nope, ld_q, w_uk, q_lat, T, n_h, d_nope, d_c, s);
    const unsigned grid = grid_for((int64_t)T * n_h * d_c);
    if (dt == MLA_DT_BF16)
        launch_timed(absorb_q_generic<uint16_t>, dim3(grid), dim3(256), 0, s,
                           (const uint16_t *)q_nope, ld_q, (const uint16_t *)w_uk,
                           (uint16_t *)q_lat, T, n_h, d_nope, d_c);
    else
        launch_timed(absorb_q_generic<float>, dim3(grid), dim3(256), 0, s,
                           (const float *)q_nope, ld_q, (const float *)w_uk, (float *)q_lat, T,
                           n_h, d_nope, d_c);
    return hipGetLastError();
}

int64_t absorb_out_workspace(int32_t T, int32_t n_h, int32_t d_v, int32_t d_model,
                             mla_dtype_t dt) {
    if (dt == MLA_DT_BF16 && absorb_out_mfma_ok(n_h, 512, d_v, d_model, dt))
        return absorb_out_mfma_workspace(T, n_h, d_v, d_model);
    return 0;
}

hipError_t launch_absorb_out(const void *o_lat, const void *w_uv, const void *w_o, void *u_ws,
                             void *out, float *ws, int32_t T, int32_t n_h, int32_t d_c,
                             int32_t d_v, int32_t d_model, mla_dtype_t dt, hipStream_t s) {
    if (absorb_out_mfma_ok(n_h, d_c, d_v, d_model, dt))
        return launch_absorb_out_mfma(o_lat, w_uv, w_o, u_ws, out, ws, T, n_h, d_c, d_v, d_model, s);
    const unsigned g1 = grid_for((int64_t)T * n_h * d_v);
    const unsigned g2 = grid_for((int64_t)T * d_model);
    if (dt == MLA_DT_BF16) {
        launch_timed(absorb_uv_generic<uint16_t>, dim3(g1), dim3(256), 0, s,
                           (const uint16_t *)o_lat, (const uint16_t *)w_uv, (uint16_t *)u_ws, T,
                           n_h, d_c, d_v);
        launch_timed(absorb_o_generic<uint16_t>, dim3(g2), dim3(256), 0, s,
                           (const uint16_t *)u_ws, (const uint16_t *)w_o, (uint16_t *)out, T,
                           n_h * d_v, d_model);
    } else {
        launch_timed(absorb_uv_generic<float>, dim3(g1), dim3(256), 0, s,
                           (const float *)o_lat, (const float *)w_uv, (float *)u_ws, T, n_h, d_c,
                           d_v);
        launch_timed(absorb_o_generic<float>, dim3(g2), dim3(256), 0, s, (const float *)u_ws,
                           (const float *)w_o, (float *)out, T, n_h * d_v, d_model);
    }
    return hipGetLastError();
}

}  // namespace mla

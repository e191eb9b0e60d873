// bf16 MFMA kernels for the absorption GEMMs (DeepSeek-V2 shape).
// Not instantiated yet: the launchers fall back to the generic kernels.
#include "common.hpp"

namespace mla {

bool absorb_q_mfma_ok(int32_t, int32_t, mla_dtype_t) { return false; }
hipError_t launch_absorb_q_mfma(const void *, int64_t, const void *, void *, int32_t, int32_t,
                                int32_t, int32_t, hipStream_t) {
    return hipErrorInvalidValue;
}
bool absorb_out_mfma_ok(int32_t, int32_t, int32_t, int32_t, mla_dtype_t) { return false; }
int64_t absorb_out_mfma_workspace(int32_t, int32_t, int32_t, int32_t) { return 0; }
hipError_t launch_absorb_out_mfma(const void *, const void *, const void *, void *, void *,
                                  float *, int32_t, int32_t, int32_t, int32_t, int32_t,
                                  hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace mla

// No-op launchers with the signatures of kernels.hpp, so that api.cpp's host
// code (argument validation, error reporting, dispatch on dtype) can be built
// and run under the host sanitizers without any device code.  Workspace sizes
// are fixed small values: api_driver.cpp only exercises the validation paths.
#include <hip/hip_runtime.h>

#include "../../padding_free_expert_amd/csrc/kernels.hpp"

namespace xmoe {

hipError_t launch_route(int, const void *, const void *, int64_t, int, int, int, float, const float *, const float *,
                        int32_t *, float *, float *, void *, hipStream_t) { return hipSuccess; }
size_t route_workspace(int64_t T, int, int E, int dt) { return dt == kBF16 ? static_cast<size_t>(T * E * 4) : 0; }
size_t route_bwd_workspace(int64_t T, int, int E, int) { return static_cast<size_t>(T * E * 2 + 64); }
hipError_t launch_route_bwd(int, const void *, const void *, const float *, const int32_t *, const float *, int,
                            int64_t, int, int, int, float, bool, void *, float *, void *, hipStream_t) {
    return hipSuccess;
}
size_t pft_workspace(int64_t T, int E) { return static_cast<size_t>(2 * ((T + 255) / 256) * E * 4 + 256); }
hipError_t launch_build_pft(const int32_t *, const float *, int64_t, int, int, int, const PftPtrs &, void *,
                            hipStream_t) { return hipSuccess; }
hipError_t launch_build_pft_static(const int32_t *, const float *, int64_t, int, int, const PftPtrs &, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_build_pilots(const int32_t *, int64_t, int, int, int, const PilotPtrs &, void *, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_ep_send_plan(const int32_t *, int, int, int32_t *, int32_t *, hipStream_t) { return hipSuccess; }
size_t ep_recv_plan_workspace(int G, int el) { return static_cast<size_t>(2 * G * el * 4 + 64); }
hipError_t launch_ep_recv_plan(const int32_t *, int, int, int64_t, int32_t *, int32_t *, int32_t *, int32_t *, void *,
                               hipStream_t) { return hipSuccess; }
hipError_t launch_dispatch(int, const void *, const int32_t *, int64_t, int, int, void *, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_scatter_rows(int, const void *, int64_t, int, const int32_t *, int64_t, void *, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_gather_sum(int, const void *, const int32_t *, const float *, int64_t, int, int, const void *, void *,
                             hipStream_t) { return hipSuccess; }
hipError_t launch_combine_bwd(int, const void *, const void *, const int32_t *, const float *, int64_t, int, int, void *,
                              float *, hipStream_t) { return hipSuccess; }
hipError_t launch_ffn_up(int, const void *, const int32_t *, int64_t, const void *, const void *, const int32_t *, int,
                         int64_t, int, int, void *, void *, hipStream_t) { return hipSuccess; }
hipError_t launch_ffn_down(int, const void *, const void *, const int32_t *, int, int64_t, int, int, void *, bool,
                           hipStream_t) { return hipSuccess; }
hipError_t launch_ffn_bwd_dact(int, const void *, const int32_t *, int64_t, const float *, const void *, const void *,
                               const int32_t *, int, int64_t, int, int, void *, hipStream_t) { return hipSuccess; }
hipError_t launch_ffn_bwd_dx(int, const void *, const void *, const void *, const int32_t *, int, int64_t, int, int,
                             void *, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_ffn_bwd_dw13(int, const void *, const int32_t *, int64_t, const void *, const int32_t *, int, int64_t,
                               int, int, void *, void *, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_ffn_bwd_dw2(int, const void *, const void *, const int32_t *, int, int64_t, int, int, void *, int,
                              bool, hipStream_t) { return hipSuccess; }
hipError_t launch_ffn_bwd(int, const void *, const void *, const void *, const void *, const void *, const void *,
                          const void *, const int32_t *, int, int64_t, int, int, void *, void *, bool, void *, void *,
                          void *, int, bool, hipStream_t) { return hipSuccess; }

}  // namespace xmoe

// Internal launchers of libxmoe (C++ linkage; the C ABI lives in api.cpp).
// Each launcher enqueues its kernels on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xmoe {

// dtype tags as in the C ABI
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

struct PftPtrs {
    int32_t *token_ids, *expert_ids, *tokens_per_expert, *expert_offsets;
    float *combine_weights;
    int32_t *slot_to_row;
};

// router
hipError_t launch_route(int dt, const void *x, const void *wg, int64_t T, int d, int E, int k, float inv_tau,
                        const float *logit_bias, const float *select_bias, int32_t *topk_ids, float *topk_w,
                        float *logits, void *ws, hipStream_t s);
size_t route_workspace(int64_t T, int d, int E, int dt);
size_t route_bwd_workspace(int64_t T, int d, int E, int dt);
hipError_t launch_route_bwd(int dt, const void *x, const void *wg, const float *logits, const int32_t *topk_ids,
                            const float *dtopk_w, int ldw, int64_t T, int d, int E, int k, float inv_tau,
                            bool accumulate, void *dx, float *dwg, void *ws, hipStream_t s);

// Padding-Free Token buffer
size_t pft_workspace(int64_t T, int E);
// E experts in all; each token has k routed slots then n_always slots for the
// last n_always experts, weight 1
hipError_t launch_build_pft(const int32_t *topk_ids, const float *topk_w, int64_t T, int E, int k, int n_always,
                            const PftPtrs &pft, void *ws, hipStream_t s);

// The same build with the library's own static scratch (kPftScratchBytes on
// each device) in place of a workspace: for callers that cannot allocate.
// hipErrorInvalidValue when pft_workspace(T, E) exceeds the scratch.
constexpr size_t kPftScratchBytes = size_t(4) << 20;
hipError_t launch_build_pft_static(const int32_t *topk_ids, const float *topk_w, int64_t T, int E, int k,
                                   const PftPtrs &pft, hipStream_t s);

// pilot tokens (Redundancy-Bypassing Dispatch, stage 1); workspace pft_workspace(T, E / experts_per_node)
struct PilotPtrs {
    int32_t *pilot_token_ids, *pilot_node_ids, *node_counts, *node_offsets, *slot_to_pilot;
};
hipError_t launch_build_pilots(const int32_t *topk_ids, int64_t T, int E, int k, int experts_per_node,
                               const PilotPtrs &pl, void *ws, hipStream_t s);

// expert-parallel plans
hipError_t launch_ep_send_plan(const int32_t *expert_offsets, int E, int G, int32_t *send_counts,
                               int32_t *send_displs, hipStream_t s);
size_t ep_recv_plan_workspace(int G, int el);
hipError_t launch_ep_recv_plan(const int32_t *recv_counts, int G, int el, int64_t n, int32_t *local_offsets,
                               int32_t *recv_displs, int32_t *local_to_recv, int32_t *recv_to_local, void *ws,
                               hipStream_t s);

// row movement
hipError_t launch_dispatch(int dt, const void *x, const int32_t *slot_to_row, int64_t T, int d, int k, void *xs,
                           hipStream_t s);
// dst[index[i]] = src[i] for i < n (indices outside [0, dst_rows) skipped)
hipError_t launch_scatter_rows(int dt, const void *src, int64_t n, int d, const int32_t *index, int64_t dst_rows,
                               void *dst, hipStream_t s);
hipError_t launch_gather_sum(int dt, const void *src, const int32_t *slot_to_row, const float *weights, int64_t T,
                             int d, int k, const void *add, void *out, hipStream_t s);
hipError_t launch_combine_bwd(int dt, const void *dy, const void *ye, const int32_t *slot_to_row,
                              const float *weights, int64_t T, int d, int k, void *dye, float *dtopk_w,
                              hipStream_t s);

// expert FFN
// row_map: NULL (rows of xs) or the PFT token_ids (rows of x, which has map_rows rows)
hipError_t launch_ffn_up(int dt, const void *xs, const int32_t *row_map, int64_t map_rows, const void *w1,
                         const void *w3, const int32_t *offsets, int E, int64_t rows, int d, int h, void *act,
                         void *h13, hipStream_t s);
// accumulate: ye += act . W2 (else ye =)
hipError_t launch_ffn_down(int dt, const void *act, const void *w2, const int32_t *offsets, int E, int64_t rows,
                           int d, int h, void *ye, bool accumulate, hipStream_t s);
// the four products of the expert backward, each on its own stream if the caller wants
// row_map (may be nullptr): A row r is dye[row_map[r]] (dye has map_rows rows);
// row_scale (may be nullptr): dA row r times row_scale[r] before the SwiGLU backward
hipError_t launch_ffn_bwd_dact(int dt, const void *dye, const int32_t *row_map, int64_t map_rows,
                               const float *row_scale, const void *w2, const void *h13, const int32_t *offsets, int E,
                               int64_t rows, int d, int h, void *dh13, hipStream_t s);
hipError_t launch_ffn_bwd_dx(int dt, const void *dh13, const void *w1, const void *w3, const int32_t *offsets, int E,
                             int64_t rows, int d, int h, void *dxs, bool accumulate, hipStream_t s);
// row_map (may be nullptr): k row r of an expert reads xs[row_map[r]] (xs has map_rows rows)
// grad_dt: dtype of the weight gradients (kF32 with bf16 inputs: unrounded
// sums); accumulate (fp32 gradients only): dW += the sums
hipError_t launch_ffn_bwd_dw13(int dt, const void *xs, const int32_t *row_map, int64_t map_rows, const void *dh13,
                               const int32_t *offsets, int E, int64_t rows, int d, int h, void *dw1, void *dw3,
                               int grad_dt, bool accumulate, hipStream_t s);
hipError_t launch_ffn_bwd_dw2(int dt, const void *act, const void *dye, const int32_t *offsets, int E, int64_t rows,
                              int d, int h, void *dw2, int grad_dt, bool accumulate, hipStream_t s);
hipError_t launch_ffn_bwd(int dt, const void *xs, const void *w1, const void *w3, const void *w2, const void *act,
                          const void *h13, const void *dye, const int32_t *offsets, int E, int64_t rows, int d,
                          int h, void *dh13, void *dxs, bool accumulate_dxs, void *dw1, void *dw3, void *dw2,
                          int grad_dt, bool accumulate_dw, hipStream_t s);

}  // namespace xmoe

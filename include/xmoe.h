/*
 * xmoe.h -- C ABI of libxmoe.so, the padding-free MoE layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer follows the X-MoE pages:
 *   - "5.4 MoE模型在分布式训练中的应用", section 训练流程: gate scores per token,
 *     dispatch tokens to experts, each expert processes its tokens, combine the
 *     results back to the owning token; the backward runs the reverse path.
 *   - X-MoE article (adg.csdn.net), section 2.1.1 "PFT数据结构创新": the
 *     Padding-Free Token buffer (PFT) replaces fixed-capacity expert buffers:
 *     token_ids, expert_ids, tokens_per_expert, combine_weights and the token
 *     rows themselves; no padding and no dropped tokens.
 *   - same article, section 2.1.2 "跨平台核函数优化": a gather that copies row
 *     token_ids[r] of the input into row r, and expert GEMMs over each expert's
 *     own rows only (no alignment to a maximum capacity).
 *
 * Conventions shared by every entry point:
 *   - Every array argument is caller-owned DEVICE memory (except the xmoe_pft
 *     struct itself, a host struct of device pointers read during the call).
 *     The library never allocates, frees or synchronises; it keeps no state
 *     beyond its loaded kernels and a per-device architecture check.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Each call
 *     validates its arguments on the host, enqueues its kernels on `stream`
 *     and returns without waiting.
 *   - Matrices are row-major and densely packed.  Sizes are int64_t or int32_t
 *     as declared; all address arithmetic is 64-bit.
 *   - Errors: a call that fails validation returns before launching anything
 *     and has no side effect: XMOE_ERR_INVALID_VALUE (NULL required pointer,
 *     size out of range, k > E, ...), XMOE_ERR_UNSUPPORTED (dtype, a size that
 *     is not a multiple of 8 where 16-byte vectors need it, a pointer not
 *     16-byte aligned, a device that is not gfx950), XMOE_ERR_WORKSPACE
 *     (workspace too small).  A launch failure returns XMOE_ERR_HIP.  Faults
 *     inside kernels surface at the caller's next synchronisation, as for any
 *     HIP work.  xmoe_last_error() returns the calling thread's last message.
 *   - Outputs must not alias inputs unless stated.  Calls are thread-safe;
 *     calls on different streams may overlap when their buffers do not alias.
 *   - dtype XMOE_BF16: bf16 inputs and outputs, fp32 accumulation, one
 *     round-to-nearest-even per stored value.  XMOE_F32: fp32 throughout.
 *     Router scores, probabilities and weights are always fp32.
 *   - Results are deterministic: no floating-point atomics; every sum runs in
 *     a fixed order, so identical inputs give bitwise identical outputs.
 *
 * Notation: T tokens, d model width, E routed experts, h expert hidden width,
 * k experts per token, R = T*k PFT rows.
 */
#ifndef XMOE_H_
#define XMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    XMOE_OK = 0,
    XMOE_ERR_INVALID_VALUE = 1,
    XMOE_ERR_UNSUPPORTED = 2,
    XMOE_ERR_WORKSPACE = 3,
    XMOE_ERR_HIP = 4
} xmoe_status;

typedef enum { XMOE_F32 = 0, XMOE_BF16 = 1 } xmoe_dtype;

/*
 * The Padding-Free Token buffer (X-MoE article, section 2.1.1), one row per
 * (token, chosen expert) pair, rows ordered by (expert ascending, token
 * ascending) -- the order the article's per-expert GEMM visits them
 * (section 2.1.2).  All pointers are device arrays owned by the caller.
 *   token_ids[r]          input position of row r                     [R]
 *   expert_ids[r]         expert of row r                             [R]
 *   tokens_per_expert[e]  rows of expert e (0 allowed)                [E]
 *   expert_offsets[e]     first row of expert e; [E] == R             [E+1]
 *   combine_weights[r]    router weight of row r (fp32)               [R]
 *   slot_to_row[t*k+j]    row holding token t's j-th choice           [R]
 * slot_to_row is the inverse of (token_ids, slot); it lets the combine and the
 * dispatch work token by token without atomics.  The PFT's token rows ("x" on
 * the page) are the separate `xs` buffer of xmoe_dispatch.
 */
typedef struct {
    int32_t *token_ids;
    int32_t *expert_ids;
    int32_t *tokens_per_expert;
    int32_t *expert_offsets;
    float *combine_weights;
    int32_t *slot_to_row;
} xmoe_pft;

/* Last error message of the calling thread ("" after success). */
const char *xmoe_last_error(void);

/* Library ABI version (major*100 + minor). */
int xmoe_version(void);

/*
 * Query device `ordinal`: *is_gfx950 = 1 when its architecture is gfx950.
 * Returns XMOE_ERR_HIP if the device cannot be queried.
 */
xmoe_status xmoe_query_device(int ordinal, int *is_gfx950);

/* ------------------------------------------------------------------ forward */

/*
 * Gate ("5.4 MoE模型在分布式训练中的应用", section 训练流程, step a: gate scores
 * per token; X-MoE notes "略读笔记90", section 需求: large top-k routing).
 *   z = x[t] . wg                    (x [T,d], wg [d,E], fp32 accumulation)
 *   s = z * inv_temperature + logit_bias[e]             -> logits [T,E] (fp32)
 *   p = softmax over the E experts of s
 *   sel = s + select_bias[e]         (selection only; never in the weights)
 *   topk_ids[t, j] = the j-th largest sel, ties to the lower expert index
 *   topk_w[t, j]   = p[t, topk_ids[t, j]]   (not renormalised)
 * logit_bias / select_bias: fp32 [E] or NULL.  logits (fp32 [T,E]) is required:
 * it is the softmax input the backward needs.  With XMOE_F32 each logit is one
 * fused multiply-add per feature in ascending order; with XMOE_BF16 the sum
 * runs on bf16 matrix cores with fp32 accumulation.
 * With XMOE_BF16 and E <= 64 one kernel forms each block of tokens' logits over
 * the whole of d (a few fixed ranges of d, added in a fixed order) and selects
 * in place; it needs no workspace.  With XMOE_BF16 and E > 64 the reduction over
 * d is split into a few ranges whose fp32 partial sums go to `workspace`
 * (caller-owned device memory of at least xmoe_route_workspace_size bytes,
 * 16-byte aligned, no initialisation needed, dead after the call) and are added
 * in range order.  Both are deterministic.  XMOE_F32 needs no workspace.  Where
 * xmoe_route_workspace_size is 0, workspace may be NULL.
 * Limits: 1 <= k <= E <= 1024, d >= 1; bf16 needs d % 8 == 0 and E % 8 == 0.
 */
xmoe_status xmoe_route(const void *x, const void *wg, xmoe_dtype dtype, int64_t T, int32_t d,
                       int32_t E, int32_t k, float inv_temperature, const float *logit_bias,
                       const float *select_bias, int32_t *topk_ids, float *topk_w, float *logits,
                       void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes xmoe_route needs for these sizes (0: none needed, or invalid). */
size_t xmoe_route_workspace_size(int64_t T, int32_t d, int32_t E, xmoe_dtype dtype);

/* Workspace bytes xmoe_build_pft needs for these sizes (0 if invalid). */
size_t xmoe_build_pft_workspace_size(int64_t T, int32_t E, int32_t k);

/*
 * Build the PFT (X-MoE article, section 2.1.1) from a routing result: a
 * per-block expert histogram, an exclusive scan, then a stable scatter that
 * gives row r = offsets[e] + (number of earlier tokens that chose e).  Fills
 * every field of *pft; combine_weights are bit-for-bit copies of topk_w.
 * Every token appears exactly k times; nothing is padded or dropped.
 * topk_ids must be valid (each in [0,E), distinct within a token); for invalid
 * ids the buffer contents are unspecified but every write stays in bounds.
 * workspace: device, >= xmoe_build_pft_workspace_size(T,E,k) bytes, 16-byte
 * aligned; its contents need no initialisation and are dead after the call.
 * Limits: 1 <= k <= E <= 1024, T*k < 2^31.
 */
xmoe_status xmoe_build_pft(const int32_t *topk_ids, const float *topk_w, int64_t T, int32_t E,
                           int32_t k, const xmoe_pft *pft, void *workspace, size_t ws_bytes,
                           void *stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: xmoe_build_pft
 * with no workspace argument.  The three kernels use the library's own static
 * scratch of xmoe_build_pft_noalloc_max_bytes() bytes (4 MiB) instead, one copy
 * per device, held until the process ends; the call allocates and frees
 * nothing and leaves no state the next call depends on (every count it reads
 * it has written first).  Calls that overlap on one device (two streams, or two
 * host threads) share that scratch and race: serialise them.  Sizes needing
 * more scratch than that (xmoe_build_pft_workspace_size(T, E, k) above the
 * maximum; at E = 1024 that is beyond 130816 tokens) return XMOE_ERR_UNSUPPORTED
 * before anything is launched.  Otherwise the same arguments, limits and
 * results, bit for bit, as xmoe_build_pft.
 */
size_t xmoe_build_pft_noalloc_max_bytes(void);
xmoe_status xmoe_build_pft_noalloc(const int32_t *topk_ids, const float *topk_w, int64_t T, int32_t E,
                                   int32_t k, const xmoe_pft *pft, void *stream);

/*
 * The same buffer with shared experts carried as experts every token is
 * routed to with weight 1 (the shared expert beside the routed ones of
 * "5.4 MoE模型在分布式训练中的应用", section 实际案例, held in the X-MoE
 * article's section 2.1.1 buffer): E_routed + n_shared experts; each
 * token has its k routed slots (topk_ids, topk_w [T,k], ids in [0, E_routed);
 * others are skipped) followed by n_shared slots for experts
 * E_routed .. E_routed + n_shared - 1, weight 1.  The pft is sized as for
 * E = E_routed + n_shared experts and k + n_shared slots per token (rows
 * R = T*(k + n_shared); slot_to_row [T, k + n_shared]).  workspace:
 * >= xmoe_build_pft_workspace_size(T, E_routed + n_shared, k + n_shared).
 */
xmoe_status xmoe_build_pft_shared(const int32_t *topk_ids, const float *topk_w, int64_t T, int32_t E_routed,
                                  int32_t k, int32_t n_shared, const xmoe_pft *pft, void *workspace,
                                  size_t ws_bytes, void *stream);

/*
 * Dispatch = the PFT gather (X-MoE article, section 2.1.2):
 *   xs[r, :] = x[token_ids[r], :]   for every PFT row r     (xs [R,d])
 * Carried out token by token through slot_to_row (each input row is read once
 * and written to its k rows), which writes exactly the same rows.  Exact copy.
 * Needs pft->slot_to_row.  d % 8 == 0 (bf16) or d % 4 == 0 (fp32).
 */
xmoe_status xmoe_dispatch(const void *x, xmoe_dtype dtype, int64_t T, int32_t d, int32_t k,
                          const xmoe_pft *pft, void *xs, void *stream);

/*
 * Up-projection of the SwiGLU experts over the expert-sorted rows (X-MoE
 * article, section 2.1.2: each expert multiplies only its own rows, no
 * padding).  For each expert e and each row r in [offsets[e], offsets[e+1]):
 *   H1 = xs[r] . w1[e],  H3 = xs[r] . w3[e]   (w1, w3 [E,d,h])
 *   act[r] = silu(H1) * H3,  silu(a) = a / (1 + exp(-a))           (act [rows,h])
 *   h13[r] = [H1 | H3] rounded to the dtype, if h13 != NULL       (h13 [rows,2h])
 * act may be NULL when h13 is given: only the pre-activations are written (as
 * when a backward recomputes them instead of keeping them).
 * expert_offsets: DEVICE int32 [E+1], non-decreasing, offsets[0] == 0,
 * offsets[E] == rows (segments are clamped to [0, rows]).  The launch is sized
 * on the host from `rows` and E alone; the tile scheduler reads the offsets on
 * the device, so nothing is copied back.  Empty experts cost nothing.
 * Limits: d, h multiples of 8 and at most 2^20; E <= 1024; rows < 2^31.
 */
xmoe_status xmoe_expert_ffn_up(const void *xs, const void *w1, const void *w3, xmoe_dtype dtype,
                               const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d,
                               int32_t h, void *act, void *h13, void *stream);

/*
 * Down-projection (X-MoE article, section 2.1.2: each expert's own rows):
 * ye[r] = act[r] . w2[e] for the rows of expert e (w2 [E,h,d], act [rows,h],
 * ye [rows,d]).  accumulate != 0: ye[r] += act[r] . w2[e] (ye read, the sum
 * rounded once to the dtype); 0: ye is overwritten.  Same offsets and limits
 * as xmoe_expert_ffn_up.
 */
xmoe_status xmoe_expert_ffn_down(const void *act, const void *w2, xmoe_dtype dtype,
                                 const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d,
                                 int32_t h, void *ye, int32_t accumulate, void *stream);

/*
 * Up-projection with the dispatch gather fused into the operand loads (X-MoE
 * article, section 2.1.2: the PFT's token_ids name each row's source token):
 * the same products as xmoe_expert_ffn_up with xs[r] replaced by
 * x[token_ids[r]], so the expert-sorted copy xs is never materialised.
 * x [T,d]; token_ids: DEVICE int32 [rows] with values in [0, T) (the PFT's
 * token_ids satisfy this; bf16 reads outside x return 0, fp32 reads are not
 * checked).  Results are bitwise those of xmoe_dispatch + xmoe_expert_ffn_up.
 * Limits as xmoe_expert_ffn_up, plus T * d * element size < 2^31 bytes.
 */
xmoe_status xmoe_expert_ffn_up_gather(const void *x, const int32_t *token_ids, const void *w1,
                                      const void *w3, xmoe_dtype dtype,
                                      const int32_t *expert_offsets, int32_t E, int64_t T,
                                      int64_t rows, int32_t d, int32_t h, void *act, void *h13,
                                      void *stream);

/*
 * Whole expert FFN with the gather fused: xmoe_expert_ffn_up_gather followed
 * by xmoe_expert_ffn_down (accumulate as there).  Same arguments and limits as
 * those two calls.
 */
xmoe_status xmoe_expert_ffn_gather(const void *x, const int32_t *token_ids, const void *w1,
                                   const void *w3, const void *w2, xmoe_dtype dtype,
                                   const int32_t *expert_offsets, int32_t E, int64_t T,
                                   int64_t rows, int32_t d, int32_t h, void *act, void *h13,
                                   void *ye, int32_t accumulate, void *stream);

/*
 * Whole expert FFN ("5.4 MoE模型在分布式训练中的应用", section 训练流程: each
 * expert processes the tokens dispatched to it; X-MoE article, section 2.1.2:
 * over each expert's own rows, no padding): xmoe_expert_ffn_up followed by
 * xmoe_expert_ffn_down.  act [rows,h] is required (it is the down-projection's
 * input and the backward's); h13 may be NULL for a forward-only pass.
 * accumulate != 0: ye += the expert outputs (one rounding of the sum), so
 * several FFNs can add into one output; 0: ye is overwritten.
 * Shared (always-on) experts run through the same call with E = 1,
 * offsets = {0, T}, xs = x: either one call per shared expert, the second with
 * accumulate = 1, or -- faster -- one call of width n*h_s with the n experts'
 * weights side by side along the hidden axis (the same sum: a SwiGLU FFN of
 * width n*h_s is the sum of the n FFNs of its column blocks).
 */
xmoe_status xmoe_expert_ffn(const void *xs, const void *w1, const void *w3, const void *w2,
                            xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E,
                            int64_t rows, int32_t d, int32_t h, void *act, void *h13, void *ye,
                            int32_t accumulate, void *stream);

/*
 * Combine ("5.4 MoE模型在分布式训练中的应用", section 专家并行: results return to
 * the owning token; X-MoE article, section 2.1.1: combine_weights):
 *   y[t] = sum_{j=0..k-1} combine_weights[r_j] * ye[r_j]  (+ y_add[t]),
 *   r_j = slot_to_row[t*k + j]
 * summed in fp32 in slot order and rounded once.  y_add [T,d] may be NULL
 * (the shared experts' output goes here).  No atomics.
 */
xmoe_status xmoe_combine(const void *ye, const xmoe_pft *pft, int64_t T, int32_t d, int32_t k,
                         xmoe_dtype dtype, const void *y_add, void *y, void *stream);

/* ----------------------------------------------------------------- backward */

/*
 * Backward of the combine ("5.4 MoE模型在分布式训练中的应用", section 训练流程:
 * the backward runs the forward's steps in reverse; the combine there is the
 * weighted sum of section 专家并行 with the X-MoE article's combine_weights,
 * section 2.1.1) for the upstream gradient dy [T,d]:
 *   dye[r]        = combine_weights[r] * dy[token_ids[r]]          (dye [R,d])
 *   dtopk_w[t, j] = < dy[t], ye[slot_to_row[t*k+j]] >              (fp32 [T,k])
 * Token by token: dy[t] is read once.
 */
xmoe_status xmoe_combine_bwd(const void *dy, const void *ye, const xmoe_pft *pft, int64_t T,
                             int32_t d, int32_t k, xmoe_dtype dtype, void *dye, float *dtopk_w,
                             void *stream);

/*
 * Backward of the SwiGLU experts ("5.4 MoE模型在分布式训练中的应用", section
 * 训练流程: the reverse path through the experts; X-MoE article, section 2.1.2:
 * each expert over its own rows), per expert, given dye [rows,d]:
 *   dA  = dye . w2[e]^T
 *   dH1 = dA * H3 * sig(H1) * (1 + H1 * (1 - sig(H1))),  dH3 = dA * silu(H1)
 *         -> dh13 = [dH1 | dH3]                                   (dh13 [rows,2h])
 *   dxs = dH1 . w1[e]^T + dH3 . w3[e]^T                           (dxs [rows,d])
 *   dw1[e] = xs_e^T . dH1,  dw3[e] = xs_e^T . dH3                (dw1, dw3 [E,d,h])
 *   dw2[e] = act_e^T . dye_e                                      (dw2 [E,h,d])
 * with H1, H3 from the forward's h13 and act from its act.
 * accumulate_dxs != 0: dxs += (one rounding of the sum); 0: overwritten.
 * grad_dt: dtype of dw1, dw3, dw2 -- the input dtype, or XMOE_F32 with bf16
 * inputs (the fp32 sums are stored without rounding).  accumulate_dw != 0
 * adds the sums to the caller's gradients (fp32 only: grad_dt must be
 * XMOE_F32, else XMOE_ERR_UNSUPPORTED), e.g. over micro-batches; 0 writes
 * them.  Experts with no rows get zeros (accumulate_dw: unchanged).
 * Same offsets and limits as xmoe_expert_ffn_up.
 */
xmoe_status xmoe_expert_ffn_bwd(const void *xs, const void *w1, const void *w3, const void *w2,
                                const void *act, const void *h13, const void *dye,
                                xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E,
                                int64_t rows, int32_t d, int32_t h, void *dh13, void *dxs,
                                int32_t accumulate_dxs, void *dw1, void *dw3, void *dw2,
                                xmoe_dtype grad_dt, int32_t accumulate_dw, void *stream);

/*
 * The four products of xmoe_expert_ffn_bwd ("5.4 MoE模型在分布式训练中的应用",
 * section 训练流程, the reverse path; X-MoE article, section 2.1.2, per expert)
 * as separate calls, so that a caller can run the weight gradients on another
 * stream beside the data gradients (same definitions, arguments, limits,
 * flags and results):
 *   _dact : dh13 from dye, w2 and the saved h13       (needs nothing else)
 *   _dx   : dxs from dh13, w1, w3; accumulate as accumulate_dxs  (after _dact)
 *   _dw13 : dw1, dw3 from xs and dh13; grad_dt, accumulate as above (after _dact)
 *   _dw2  : dw2 from act and dye; grad_dt, accumulate as above   (independent)
 */
xmoe_status xmoe_expert_ffn_bwd_dact(const void *dye, const void *w2, const void *h13,
                                     xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E,
                                     int64_t rows, int32_t d, int32_t h, void *dh13, void *stream);
/*
 * xmoe_expert_ffn_bwd_dact fed by the upstream gradient itself
 * ("5.4 MoE模型在分布式训练中的应用", section 训练流程: the reverse path runs
 * from the layer output back through the weighted combine into the experts;
 * X-MoE article, section 2.1.2: the PFT's token_ids name each row's source
 * token and combine_weights its gate weight):
 *   dA[r] = row_weights[r] * (dy[token_ids[r]] . w2[e]^T),  then dH1, dH3 as _dact
 * The combine backward's dye rows (w_r * dy[t]) are thus never materialised;
 * the weight multiplies the fp32 product instead of being rounded into dye
 * first, so results agree with xmoe_combine_bwd + xmoe_expert_ffn_bwd_dact to
 * rounding, not bitwise.  dy [T,d]; token_ids: DEVICE int32 [rows] with values
 * in [0, T); row_weights: DEVICE fp32 [rows] (the PFT's token_ids and
 * combine_weights).  Limits as xmoe_expert_ffn_bwd_dact, plus T * d * element
 * size < 2^31 bytes.
 */
xmoe_status xmoe_expert_ffn_bwd_dact_gather(const void *dy, const int32_t *token_ids,
                                            const float *row_weights, const void *w2, const void *h13,
                                            xmoe_dtype dtype, const int32_t *expert_offsets,
                                            int32_t E, int64_t T, int64_t rows, int32_t d, int32_t h,
                                            void *dh13, void *stream);
xmoe_status xmoe_expert_ffn_bwd_dx(const void *dh13, const void *w1, const void *w3,
                                   xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E,
                                   int64_t rows, int32_t d, int32_t h, void *dxs, int32_t accumulate,
                                   void *stream);
xmoe_status xmoe_expert_ffn_bwd_dw13(const void *xs, const void *dh13, xmoe_dtype dtype,
                                     const int32_t *expert_offsets, int32_t E, int64_t rows,
                                     int32_t d, int32_t h, void *dw1, void *dw3, xmoe_dtype grad_dt,
                                     int32_t accumulate, void *stream);
/*
 * xmoe_expert_ffn_bwd_dw13 with the dispatch gather fused into the loads of
 * xs (X-MoE article, section 2.1.2: the PFT's token_ids name each row's source
 * token): dw1[e] = xs_e^T . dH1 and dw3[e] = xs_e^T . dH3 with xs[r] replaced
 * by x[token_ids[r]], so the backward needs no expert-sorted copy of x.
 * x [T,d]; token_ids: DEVICE int32 [rows] with values in [0, T) (bf16 reads
 * outside x return 0, fp32 reads are not checked).  Results are bitwise those
 * of xmoe_dispatch + xmoe_expert_ffn_bwd_dw13.  Limits as
 * xmoe_expert_ffn_bwd_dw13, plus T * d * element size < 2^31 bytes.
 */
xmoe_status xmoe_expert_ffn_bwd_dw13_gather(const void *x, const int32_t *token_ids, const void *dh13,
                                            xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E,
                                            int64_t T, int64_t rows, int32_t d, int32_t h, void *dw1,
                                            void *dw3, xmoe_dtype grad_dt, int32_t accumulate,
                                            void *stream);
xmoe_status xmoe_expert_ffn_bwd_dw2(const void *act, const void *dye, xmoe_dtype dtype,
                                    const int32_t *expert_offsets, int32_t E, int64_t rows,
                                    int32_t d, int32_t h, void *dw2, xmoe_dtype grad_dt,
                                    int32_t accumulate, void *stream);

/*
 * Backward of the dispatch ("5.4 MoE模型在分布式训练中的应用", section 训练流程,
 * the reverse path; the transpose of the X-MoE article's section 2.1.2 gather):
 *   dx[t] = sum_{j=0..k-1} dxs[slot_to_row[t*k+j]]  (+ dx_add[t])
 * summed in fp32 in slot order, rounded once; no atomics.  dx_add [T,d] may be
 * NULL (the shared experts' input gradient goes here).
 */
xmoe_status xmoe_dispatch_bwd(const void *dxs, const xmoe_pft *pft, int64_t T, int32_t d,
                              int32_t k, xmoe_dtype dtype, const void *dx_add, void *dx,
                              void *stream);

/* Workspace bytes xmoe_route_bwd needs (0 if invalid). */
size_t xmoe_route_bwd_workspace_size(int64_t T, int32_t d, int32_t E, xmoe_dtype dtype);

/*
 * Backward of the gate ("5.4 MoE模型在分布式训练中的应用", section 训练流程: the
 * reverse path reaches the gate's scores) through the probabilities (the top-k
 * selection is piecewise constant and carries no gradient; the biases get
 * none):
 *   p = softmax(logits[t]),  g[t,e] = dtopk_w[t,j] if e == topk_ids[t,j] else 0
 *   c_t = sum_j p[t, topk_ids[t,j]] * dtopk_w[t,j]
 *   dz[t,e] = p[t,e] * (g[t,e] - c_t) * inv_temperature
 *   dx[t] += dz[t] . wg^T        (read-modify-write of dx [T,d])
 *   dwg = x^T . dz               (fp32 [d,E], fixed-order split-T sum)
 * With XMOE_BF16, dz is rounded to bf16 for the two matrix-core products
 * (fp32 accumulation).  workspace: device, >= xmoe_route_bwd_workspace_size.
 * dtopk_w: row t at dtopk_w + t*ldw (ldw >= k; ldw > k reads the routed slots
 * of a buffer with more slots per token, such as one that also holds shared
 * experts).  accumulate != 0: dx += dz . wg^T as above; 0: dx = dz . wg^T.
 */
xmoe_status xmoe_route_bwd(const void *x, const void *wg, const float *logits,
                           const int32_t *topk_ids, const float *dtopk_w, int32_t ldw, xmoe_dtype dtype,
                           int64_t T, int32_t d, int32_t E, int32_t k, float inv_temperature,
                           int32_t accumulate, void *dx, float *dwg, void *workspace, size_t ws_bytes,
                           void *stream);

/* ------------------------------------------------------------------------
 * Pilot tokens of Redundancy-Bypassing Dispatch, stage 1
 * (X-MoE article, adg.csdn.net, section 2.2.1 "分层冗余消除算法", Pilot Token选择):
 *   node(e) = e / experts_per_node;   pilots = {(t, node(topk_ids[t,j]))}
 * i.e. a token's k destinations deduplicated per node.  Listed by node, then
 * token (the Padding-Free Token buffer's order with the node as the key).
 * Outputs (DEVICE, int32, caller-owned; N = E / experts_per_node,
 * P = node_offsets[N] <= T * min(k, N)):
 *   pilot_token_ids [>= P], pilot_node_ids [>= P]   -- pilot p carries token
 *       pilot_token_ids[p] to node pilot_node_ids[p];
 *   node_counts [N], node_offsets [N+1]             -- node n's pilots are
 *       [node_offsets[n], node_offsets[n+1]);
 *   slot_to_pilot [T*k]                            -- the pilot that carries
 *       slot (t, j) to its expert's node.
 * Sizing pilot_token_ids / pilot_node_ids for T*k rows is always enough.
 * topk_ids: DEVICE int32 [T,k]; ids outside [0, E) are skipped (their slot
 * gets -1).  experts_per_node must divide E; E <= 1024.  workspace: device,
 * 16-byte aligned, >= xmoe_build_pilots_workspace_size.  No host sync.
 */
size_t xmoe_build_pilots_workspace_size(int64_t T, int32_t E, int32_t k, int32_t experts_per_node);
xmoe_status xmoe_build_pilots(const int32_t *topk_ids, int64_t T, int32_t E, int32_t k, int32_t experts_per_node,
                              int32_t *pilot_token_ids, int32_t *pilot_node_ids, int32_t *node_counts,
                              int32_t *node_offsets, int32_t *slot_to_pilot, void *workspace, size_t ws_bytes,
                              void *stream);

/* ------------------------------------------------------------------------
 * Expert-parallel plans ("5.4 MoE模型在分布式训练中的应用", section 专家并行:
 * 数据流, All-to-All通信步骤; the X-MoE article, section 2.1.1, sends the
 * Padding-Free Token rows with an alltoallv and no padding).  G ranks; rank q
 * holds the E/G consecutive experts [q*E/G, (q+1)*E/G).  This library plans
 * and rearranges; the exchange itself (RCCL alltoallv of the counts, then of
 * the rows) is the caller's.
 *
 * xmoe_ep_send_plan: from a rank's Padding-Free Token buffer, the rows it sends
 * to each rank -- one contiguous run each, since the buffer is expert-sorted:
 *   send_counts[q] = expert_offsets[(q+1)E/G] - expert_offsets[qE/G]   [G]
 *   send_displs[q] = expert_offsets[qE/G]                              [G+1]
 * (DEVICE int32, caller-owned).  G must divide E; E <= 1024.
 */
xmoe_status xmoe_ep_send_plan(const int32_t *expert_offsets, int32_t E, int32_t G, int32_t *send_counts,
                              int32_t *send_displs, void *stream);

/*
 * xmoe_ep_recv_plan: the receiver's layout.  recv_counts: DEVICE int32
 * [G, E_local], row s = the tokens_per_expert source s sends for this rank's
 * E_local experts.  Rows arrive source-major (source s, its experts ascending,
 * its row order) and are regrouped expert-major (local expert e, then source
 * s, then the same order), which the grouped expert GEMMs read:
 *   local_offsets [E_local+1]  expert e's rows in the expert-major layout;
 *   recv_displs   [G+1]        source s's rows in the arrival layout;
 *   local_to_recv [n_recv]     arrival index of expert-major row m;
 *   recv_to_local [n_recv]     its inverse.
 * n_recv (host) must equal the sum of recv_counts (the caller knows it: the
 * alltoallv needs it); rows past n_recv are never written, so a wrong n_recv
 * gives a wrong but memory-safe plan.  G * E_local <= 1024.  workspace: device,
 * 16-byte aligned, >= xmoe_ep_recv_plan_workspace_size.
 * Regroup with xmoe_scatter_rows(recv, ..., recv_to_local, ...) and send the
 * expert outputs back with xmoe_scatter_rows(out, ..., local_to_recv, ...).
 */
size_t xmoe_ep_recv_plan_workspace_size(int32_t G, int32_t E_local);
xmoe_status xmoe_ep_recv_plan(const int32_t *recv_counts, int32_t G, int32_t E_local, int64_t n_recv,
                              int32_t *local_offsets, int32_t *recv_displs, int32_t *local_to_recv,
                              int32_t *recv_to_local, void *workspace, size_t ws_bytes, void *stream);

/*
 * Row scatter: dst[index[i], :] = src[i, :] for i < n; index values outside
 * [0, dst_rows) are skipped.  src [n, d], dst [dst_rows, d], row-major, DEVICE,
 * 16-byte aligned; index DEVICE int32 [n].  d a multiple of 8.  With a
 * permutation index this is the EP regroup (and, with the inverse, the
 * ungroup).  Overlapping src and dst are not allowed.
 */
xmoe_status xmoe_scatter_rows(const void *src, xmoe_dtype dtype, int64_t n, int32_t d, const int32_t *index,
                              int64_t dst_rows, void *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* XMOE_H_ */

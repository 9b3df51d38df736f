// C ABI of libxmoe: argument validation, architecture check and kernel launch.
// Every check runs on the host before anything is enqueued, so a rejected call
// has no side effect.  Semantics of each entry point are documented in xmoe.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/xmoe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

xmoe_status fail(xmoe_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

xmoe_status ok() {
    g_err.clear();
    return XMOE_OK;
}

xmoe_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(XMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Architecture check of the current device, cached per device ordinal.
constexpr int kMaxDevices = 64;
int g_arch[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::mutex g_arch_mu;

xmoe_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(XMOE_ERR_HIP, "no current HIP device");
    {
        std::lock_guard<std::mutex> lk(g_arch_mu);
        if (g_arch[dev] == 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
                return fail(XMOE_ERR_HIP, "cannot query device %d", dev);
            g_arch[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        }
        if (g_arch[dev] != 1) return fail(XMOE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    }
    return XMOE_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, st, ...)                  \
    do {                                        \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

#define CHECK_DEVICE()                          \
    do {                                        \
        xmoe_status _s = check_device();        \
        if (_s != XMOE_OK) return _s;           \
    } while (0)

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

// a * b <= limit for a, b >= 0, without forming a product that could overflow
// (callers may pass any int64 size; the checks must stay defined for all)
bool within(int64_t a, int64_t b, int64_t limit) { return a >= 0 && b >= 0 && (b == 0 || a <= limit / b); }

xmoe_status check_dtype(xmoe_dtype dt) {
    if (dt != XMOE_F32 && dt != XMOE_BF16) return fail(XMOE_ERR_UNSUPPORTED, "unknown dtype %d", static_cast<int>(dt));
    return XMOE_OK;
}

xmoe_status check_pft(const xmoe_pft *pft, bool need_s2r, bool need_w, bool need_all) {
    if (!pft) return fail(XMOE_ERR_INVALID_VALUE, "pft is NULL");
    if (need_s2r && !pft->slot_to_row) return fail(XMOE_ERR_INVALID_VALUE, "pft->slot_to_row is NULL");
    if (need_w && !pft->combine_weights) return fail(XMOE_ERR_INVALID_VALUE, "pft->combine_weights is NULL");
    if (need_all && (!pft->token_ids || !pft->expert_ids || !pft->tokens_per_expert || !pft->expert_offsets ||
                     !pft->combine_weights || !pft->slot_to_row))
        return fail(XMOE_ERR_INVALID_VALUE, "a pft field is NULL");
    return XMOE_OK;
}

xmoe_status check_rows_common(int64_t T, int32_t d, int32_t k) {
    REQUIRE(T >= 0, XMOE_ERR_INVALID_VALUE, "T must be >= 0");
    REQUIRE(k >= 1 && k <= 1024, XMOE_ERR_INVALID_VALUE, "k must be in [1, 1024]");
    REQUIRE(within(T, k, kMaxRows), XMOE_ERR_INVALID_VALUE, "T*k must be < 2^31");
    REQUIRE(d >= 1, XMOE_ERR_INVALID_VALUE, "d must be >= 1");
    REQUIRE(d % 8 == 0, XMOE_ERR_UNSUPPORTED, "d must be a multiple of 8");
    return XMOE_OK;
}

xmoe_status check_ffn_sizes(const int32_t *offsets, int32_t E, int64_t rows, int32_t d, int32_t h) {
    REQUIRE(offsets, XMOE_ERR_INVALID_VALUE, "expert_offsets is NULL");
    REQUIRE(E >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E must be in [1, 1024]");
    REQUIRE(rows >= 0 && rows <= kMaxRows, XMOE_ERR_INVALID_VALUE, "rows must be in [0, 2^31)");
    REQUIRE(d >= 1 && h >= 1, XMOE_ERR_INVALID_VALUE, "d and h must be >= 1");
    REQUIRE(d % 8 == 0 && h % 8 == 0, XMOE_ERR_UNSUPPORTED, "d and h must be multiples of 8");
    // tiles address up to 256 rows of [H1|H3] or of d columns with 32-bit offsets
    REQUIRE(d <= (1 << 20) && h <= (1 << 20), XMOE_ERR_UNSUPPORTED, "d and h must be at most 2^20");
    return XMOE_OK;
}

// Weight-gradient dtype: the input dtype, or fp32 with bf16 inputs (unrounded
// sums).  Accumulating into the gradients needs fp32 gradients.
xmoe_status check_grad_dt(xmoe_dtype dtype, xmoe_dtype grad_dt, int32_t accumulate) {
    if (grad_dt != XMOE_F32 && grad_dt != XMOE_BF16)
        return fail(XMOE_ERR_UNSUPPORTED, "unknown grad_dt %d", static_cast<int>(grad_dt));
    if (dtype == XMOE_F32 && grad_dt != XMOE_F32)
        return fail(XMOE_ERR_UNSUPPORTED, "fp32 inputs need grad_dt = XMOE_F32");
    if (accumulate && grad_dt != XMOE_F32)
        return fail(XMOE_ERR_UNSUPPORTED, "accumulating weight gradients needs grad_dt = XMOE_F32");
    return XMOE_OK;
}

#define TRY(expr)                         \
    do {                                  \
        xmoe_status _s = (expr);          \
        if (_s != XMOE_OK) return _s;     \
    } while (0)

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

xmoe::PftPtrs to_ptrs(const xmoe_pft *p) {
    return {p->token_ids, p->expert_ids, p->tokens_per_expert, p->expert_offsets, p->combine_weights, p->slot_to_row};
}

// x is read through the row map with 32-bit buffer offsets
xmoe_status check_gather(const void *x, const int32_t *token_ids, int64_t T, int64_t rows, int32_t d,
                         xmoe_dtype dtype) {
    REQUIRE(rows == 0 || (x && token_ids), XMOE_ERR_INVALID_VALUE, "x and token_ids are required");
    REQUIRE(T >= 0 && (rows == 0 || T >= 1), XMOE_ERR_INVALID_VALUE, "T must be >= 1 when there are rows to gather");
    REQUIRE(within(T, static_cast<int64_t>(d) * (dtype == XMOE_BF16 ? 2 : 4), (int64_t{1} << 31) - 1),
            XMOE_ERR_UNSUPPORTED,
            "x must be smaller than 2^31 bytes to be gathered");
    REQUIRE(aligned16(x), XMOE_ERR_UNSUPPORTED, "x must be 16-byte aligned");
    return XMOE_OK;
}
}  // namespace

extern "C" {

const char *xmoe_last_error(void) { return g_err.c_str(); }

int xmoe_version(void) { return 200; }

xmoe_status xmoe_query_device(int ordinal, int *is_gfx950) {
    REQUIRE(is_gfx950, XMOE_ERR_INVALID_VALUE, "is_gfx950 is NULL");
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, ordinal);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    *is_gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    return ok();
}

size_t xmoe_route_workspace_size(int64_t T, int32_t d, int32_t E, xmoe_dtype dtype) {
    if (T < 0 || T > kMaxRows || d < 1 || E < 1 || E > 1024 || (dtype != XMOE_BF16 && dtype != XMOE_F32)) return 0;
    return xmoe::route_workspace(T, d, E, dtype);
}

xmoe_status xmoe_route(const void *x, const void *wg, xmoe_dtype dtype, int64_t T, int32_t d, int32_t E, int32_t k,
                       float inv_temperature, const float *logit_bias, const float *select_bias, int32_t *topk_ids,
                       float *topk_w, float *logits, void *workspace, size_t ws_bytes, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(wg && (T == 0 || (x && topk_ids && topk_w && logits)), XMOE_ERR_INVALID_VALUE,
            "a required pointer is NULL");
    REQUIRE(T >= 0 && d >= 1, XMOE_ERR_INVALID_VALUE, "T must be >= 0 and d >= 1");
    REQUIRE(E >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E must be in [1, 1024]");
    REQUIRE(k >= 1 && k <= E, XMOE_ERR_INVALID_VALUE, "k must be in [1, E]");
    REQUIRE(T <= kMaxRows && within(T, E, kMaxRows * 8), XMOE_ERR_INVALID_VALUE, "T too large");
    if (dtype == XMOE_BF16) {
        REQUIRE(d % 8 == 0 && E % 8 == 0, XMOE_ERR_UNSUPPORTED, "bf16 routing needs d and E multiples of 8");
        REQUIRE(aligned16(x) && aligned16(wg), XMOE_ERR_UNSUPPORTED, "x and wg must be 16-byte aligned");
    }
    const size_t need = xmoe::route_workspace(T, d, E, dtype);
    REQUIRE(need == 0 || (workspace && aligned16(workspace)), XMOE_ERR_WORKSPACE,
            "workspace is NULL or not 16-byte aligned");
    REQUIRE(ws_bytes >= need, XMOE_ERR_WORKSPACE, "workspace too small (see xmoe_route_workspace_size)");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_route(dtype, x, wg, T, d, E, k, inv_temperature, logit_bias, select_bias, topk_ids,
                                         topk_w, logits, workspace, S(stream)),
                      "xmoe_route launch");
}

size_t xmoe_build_pft_workspace_size(int64_t T, int32_t E, int32_t k) {
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || !within(T, k, kMaxRows)) return 0;
    return xmoe::pft_workspace(T, E);
}

xmoe_status xmoe_build_pft(const int32_t *topk_ids, const float *topk_w, int64_t T, int32_t E, int32_t k,
                           const xmoe_pft *pft, void *workspace, size_t ws_bytes, void *stream) {
    REQUIRE(T == 0 || (topk_ids && topk_w), XMOE_ERR_INVALID_VALUE, "topk_ids and topk_w are required");
    REQUIRE(T >= 0, XMOE_ERR_INVALID_VALUE, "T must be >= 0");
    REQUIRE(E >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E must be in [1, 1024]");
    REQUIRE(k >= 1 && k <= E, XMOE_ERR_INVALID_VALUE, "k must be in [1, E]");
    REQUIRE(within(T, k, kMaxRows), XMOE_ERR_INVALID_VALUE, "T*k must be < 2^31");
    TRY(check_pft(pft, T > 0, T > 0, T > 0));
    REQUIRE(pft->tokens_per_expert && pft->expert_offsets, XMOE_ERR_INVALID_VALUE,
            "pft->tokens_per_expert and pft->expert_offsets are required");
    REQUIRE(workspace && aligned16(workspace), XMOE_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
    REQUIRE(ws_bytes >= xmoe::pft_workspace(T, E), XMOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes,
            xmoe::pft_workspace(T, E));
    CHECK_DEVICE();
    return hip_status(xmoe::launch_build_pft(topk_ids, topk_w, T, E, k, 0, to_ptrs(pft), workspace, S(stream)),
                      "xmoe_build_pft launch");
}

size_t xmoe_build_pft_noalloc_max_bytes(void) { return xmoe::kPftScratchBytes; }

xmoe_status xmoe_build_pft_noalloc(const int32_t *topk_ids, const float *topk_w, int64_t T, int32_t E, int32_t k,
                                   const xmoe_pft *pft, void *stream) {
    REQUIRE(T == 0 || (topk_ids && topk_w), XMOE_ERR_INVALID_VALUE, "topk_ids and topk_w are required");
    REQUIRE(T >= 0, XMOE_ERR_INVALID_VALUE, "T must be >= 0");
    REQUIRE(E >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E must be in [1, 1024]");
    REQUIRE(k >= 1 && k <= E, XMOE_ERR_INVALID_VALUE, "k must be in [1, E]");
    REQUIRE(within(T, k, kMaxRows), XMOE_ERR_INVALID_VALUE, "T*k must be < 2^31");
    TRY(check_pft(pft, T > 0, T > 0, T > 0));
    REQUIRE(pft->tokens_per_expert && pft->expert_offsets, XMOE_ERR_INVALID_VALUE,
            "pft->tokens_per_expert and pft->expert_offsets are required");
    REQUIRE(xmoe::pft_workspace(T, E) <= xmoe::kPftScratchBytes, XMOE_ERR_UNSUPPORTED,
            "T and E need %zu bytes of scratch, more than the %zu the library holds per device "
            "(use xmoe_build_pft with a workspace)",
            xmoe::pft_workspace(T, E), xmoe::kPftScratchBytes);
    CHECK_DEVICE();
    return hip_status(xmoe::launch_build_pft_static(topk_ids, topk_w, T, E, k, to_ptrs(pft), S(stream)),
                      "xmoe_build_pft_noalloc launch");
}

xmoe_status xmoe_build_pft_shared(const int32_t *topk_ids, const float *topk_w, int64_t T, int32_t E_routed,
                                  int32_t k, int32_t n_shared, const xmoe_pft *pft, void *workspace, size_t ws_bytes,
                                  void *stream) {
    REQUIRE(n_shared >= 0, XMOE_ERR_INVALID_VALUE, "n_shared must be >= 0");
    const int64_t E = static_cast<int64_t>(E_routed) + n_shared, ks = static_cast<int64_t>(k) + n_shared;
    REQUIRE(T == 0 || (topk_ids && topk_w), XMOE_ERR_INVALID_VALUE, "topk_ids and topk_w are required");
    REQUIRE(T >= 0, XMOE_ERR_INVALID_VALUE, "T must be >= 0");
    REQUIRE(E_routed >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E_routed >= 1 and E_routed + n_shared <= 1024");
    REQUIRE(k >= 1 && k <= E_routed, XMOE_ERR_INVALID_VALUE, "k must be in [1, E_routed]");
    REQUIRE(within(T, ks, kMaxRows), XMOE_ERR_INVALID_VALUE, "T*(k+n_shared) must be < 2^31");
    TRY(check_pft(pft, T > 0, T > 0, T > 0));
    REQUIRE(pft->tokens_per_expert && pft->expert_offsets, XMOE_ERR_INVALID_VALUE,
            "pft->tokens_per_expert and pft->expert_offsets are required");
    const size_t need = xmoe::pft_workspace(T, static_cast<int>(E));
    REQUIRE(workspace && aligned16(workspace), XMOE_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
    REQUIRE(ws_bytes >= need, XMOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
    CHECK_DEVICE();
    return hip_status(xmoe::launch_build_pft(topk_ids, topk_w, T, static_cast<int>(E), k, n_shared, to_ptrs(pft),
                                             workspace, S(stream)),
                      "xmoe_build_pft_shared launch");
}

xmoe_status xmoe_dispatch(const void *x, xmoe_dtype dtype, int64_t T, int32_t d, int32_t k, const xmoe_pft *pft,
                          void *xs, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(T == 0 || (x && xs), XMOE_ERR_INVALID_VALUE, "x and xs are required");
    TRY(check_rows_common(T, d, k));
    TRY(check_pft(pft, T > 0, false, false));
    REQUIRE(aligned16(x) && aligned16(xs), XMOE_ERR_UNSUPPORTED, "x and xs must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_dispatch(dtype, x, pft->slot_to_row, T, d, k, xs, S(stream)), "xmoe_dispatch launch");
}

xmoe_status xmoe_expert_ffn_up(const void *xs, const void *w1, const void *w3, xmoe_dtype dtype,
                               const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d, int32_t h, void *act,
                               void *h13, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w1 && w3 && (rows == 0 || (xs && (act || h13))), XMOE_ERR_INVALID_VALUE,
            "xs, w1, w3 and act or h13 are required");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(xs) && aligned16(w1) && aligned16(w3) && aligned16(act) && aligned16(h13),
            XMOE_ERR_UNSUPPORTED, "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_up(dtype, xs, nullptr, 0, w1, w3, expert_offsets, E, rows, d, h, act, h13,
                                          S(stream)),
                      "xmoe_expert_ffn_up launch");
}

xmoe_status xmoe_expert_ffn_down(const void *act, const void *w2, xmoe_dtype dtype, const int32_t *expert_offsets,
                                 int32_t E, int64_t rows, int32_t d, int32_t h, void *ye, int32_t accumulate,
                                 void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w2 && (rows == 0 || (act && ye)), XMOE_ERR_INVALID_VALUE, "act, w2 and ye are required");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(act) && aligned16(w2) && aligned16(ye), XMOE_ERR_UNSUPPORTED, "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_down(dtype, act, w2, expert_offsets, E, rows, d, h, ye, accumulate != 0,
                                            S(stream)),
                      "xmoe_expert_ffn_down launch");
}


xmoe_status xmoe_expert_ffn_up_gather(const void *x, const int32_t *token_ids, const void *w1, const void *w3,
                                      xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E, int64_t T,
                                      int64_t rows, int32_t d, int32_t h, void *act, void *h13, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w1 && w3 && (rows == 0 || act || h13), XMOE_ERR_INVALID_VALUE, "w1, w3 and act or h13 are required");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    TRY(check_gather(x, token_ids, T, rows, d, dtype));
    REQUIRE(aligned16(w1) && aligned16(w3) && aligned16(act) && aligned16(h13), XMOE_ERR_UNSUPPORTED,
            "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_up(dtype, x, token_ids, T, w1, w3, expert_offsets, E, rows, d, h, act, h13,
                                          S(stream)),
                      "xmoe_expert_ffn_up_gather launch");
}

xmoe_status xmoe_expert_ffn_gather(const void *x, const int32_t *token_ids, const void *w1, const void *w3,
                                   const void *w2, xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E,
                                   int64_t T, int64_t rows, int32_t d, int32_t h, void *act, void *h13, void *ye,
                                   int32_t accumulate, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w1 && w3 && w2 && (rows == 0 || (act && ye)), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    TRY(check_gather(x, token_ids, T, rows, d, dtype));
    REQUIRE(aligned16(w1) && aligned16(w3) && aligned16(w2) && aligned16(act) && aligned16(h13) && aligned16(ye),
            XMOE_ERR_UNSUPPORTED, "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    hipError_t e = xmoe::launch_ffn_up(dtype, x, token_ids, T, w1, w3, expert_offsets, E, rows, d, h, act, h13,
                                       S(stream));
    if (e != hipSuccess) return hip_status(e, "xmoe_expert_ffn_gather up-projection launch");
    return hip_status(xmoe::launch_ffn_down(dtype, act, w2, expert_offsets, E, rows, d, h, ye, accumulate != 0,
                                            S(stream)),
                      "xmoe_expert_ffn_gather down-projection launch");
}

xmoe_status xmoe_expert_ffn(const void *xs, const void *w1, const void *w3, const void *w2, xmoe_dtype dtype,
                            const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d, int32_t h, void *act,
                            void *h13, void *ye, int32_t accumulate, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w1 && w3 && w2 && (rows == 0 || (xs && act && ye)), XMOE_ERR_INVALID_VALUE,
            "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(xs) && aligned16(w1) && aligned16(w3) && aligned16(w2) && aligned16(act) && aligned16(h13) &&
                aligned16(ye),
            XMOE_ERR_UNSUPPORTED, "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    hipError_t e = xmoe::launch_ffn_up(dtype, xs, nullptr, 0, w1, w3, expert_offsets, E, rows, d, h, act, h13, S(stream));
    if (e != hipSuccess) return hip_status(e, "xmoe_expert_ffn up-projection launch");
    return hip_status(xmoe::launch_ffn_down(dtype, act, w2, expert_offsets, E, rows, d, h, ye, accumulate != 0,
                                            S(stream)),
                      "xmoe_expert_ffn down-projection launch");
}

xmoe_status xmoe_combine(const void *ye, const xmoe_pft *pft, int64_t T, int32_t d, int32_t k, xmoe_dtype dtype,
                         const void *y_add, void *y, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(T == 0 || (ye && y), XMOE_ERR_INVALID_VALUE, "ye and y are required");
    TRY(check_rows_common(T, d, k));
    TRY(check_pft(pft, T > 0, T > 0, false));
    REQUIRE(aligned16(ye) && aligned16(y) && aligned16(y_add), XMOE_ERR_UNSUPPORTED, "rows must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_gather_sum(dtype, ye, pft->slot_to_row, pft->combine_weights, T, d, k, y_add, y,
                                              S(stream)),
                      "xmoe_combine launch");
}

xmoe_status xmoe_combine_bwd(const void *dy, const void *ye, const xmoe_pft *pft, int64_t T, int32_t d, int32_t k,
                             xmoe_dtype dtype, void *dye, float *dtopk_w, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(T == 0 || (dy && ye && dye && dtopk_w), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_rows_common(T, d, k));
    TRY(check_pft(pft, T > 0, T > 0, false));
    REQUIRE(aligned16(dy) && aligned16(ye) && aligned16(dye), XMOE_ERR_UNSUPPORTED, "rows must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_combine_bwd(dtype, dy, ye, pft->slot_to_row, pft->combine_weights, T, d, k, dye,
                                               dtopk_w, S(stream)),
                      "xmoe_combine_bwd launch");
}

xmoe_status xmoe_expert_ffn_bwd(const void *xs, const void *w1, const void *w3, const void *w2, const void *act,
                                const void *h13, const void *dye, xmoe_dtype dtype, const int32_t *expert_offsets,
                                int32_t E, int64_t rows, int32_t d, int32_t h, void *dh13, void *dxs,
                                int32_t accumulate_dxs, void *dw1, void *dw3, void *dw2, xmoe_dtype grad_dt,
                                int32_t accumulate_dw, void *stream) {
    TRY(check_dtype(dtype));
    TRY(check_grad_dt(dtype, grad_dt, accumulate_dw));
    REQUIRE(w1 && w3 && w2 && dw1 && dw3 && dw2 && (rows == 0 || (xs && act && h13 && dye && dh13 && dxs)),
            XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(xs) && aligned16(w1) && aligned16(w3) && aligned16(w2) && aligned16(act) && aligned16(h13) &&
                aligned16(dye) && aligned16(dh13) && aligned16(dxs) && aligned16(dw1) && aligned16(dw3) &&
                aligned16(dw2),
            XMOE_ERR_UNSUPPORTED, "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_bwd(dtype, xs, w1, w3, w2, act, h13, dye, expert_offsets, E, rows, d, h, dh13,
                                           dxs, accumulate_dxs != 0, dw1, dw3, dw2, grad_dt, accumulate_dw != 0,
                                           S(stream)),
                      "xmoe_expert_ffn_bwd launch");
}

xmoe_status xmoe_expert_ffn_bwd_dact(const void *dye, const void *w2, const void *h13, xmoe_dtype dtype,
                                     const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d, int32_t h,
                                     void *dh13, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w2 && (rows == 0 || (dye && h13 && dh13)), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(dye) && aligned16(w2) && aligned16(h13) && aligned16(dh13), XMOE_ERR_UNSUPPORTED,
            "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_bwd_dact(dtype, dye, nullptr, 0, nullptr, w2, h13, expert_offsets, E, rows, d, h,
                                                dh13, S(stream)),
                      "xmoe_expert_ffn_bwd_dact launch");
}

xmoe_status xmoe_expert_ffn_bwd_dact_gather(const void *dy, const int32_t *token_ids, const float *row_weights,
                                            const void *w2, const void *h13, xmoe_dtype dtype,
                                            const int32_t *expert_offsets, int32_t E, int64_t T, int64_t rows,
                                            int32_t d, int32_t h, void *dh13, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w2 && (rows == 0 || (row_weights && h13 && dh13)), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    TRY(check_gather(dy, token_ids, T, rows, d, dtype));
    REQUIRE(aligned16(w2) && aligned16(h13) && aligned16(dh13), XMOE_ERR_UNSUPPORTED, "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_bwd_dact(dtype, dy, token_ids, T, row_weights, w2, h13, expert_offsets, E, rows,
                                                d, h, dh13, S(stream)),
                      "xmoe_expert_ffn_bwd_dact_gather launch");
}

xmoe_status xmoe_expert_ffn_bwd_dx(const void *dh13, const void *w1, const void *w3, xmoe_dtype dtype,
                                   const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d, int32_t h,
                                   void *dxs, int32_t accumulate, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(w1 && w3 && (rows == 0 || (dh13 && dxs)), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(dh13) && aligned16(w1) && aligned16(w3) && aligned16(dxs), XMOE_ERR_UNSUPPORTED,
            "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_bwd_dx(dtype, dh13, w1, w3, expert_offsets, E, rows, d, h, dxs, accumulate != 0,
                                              S(stream)),
                      "xmoe_expert_ffn_bwd_dx launch");
}

xmoe_status xmoe_expert_ffn_bwd_dw13(const void *xs, const void *dh13, xmoe_dtype dtype,
                                     const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d, int32_t h,
                                     void *dw1, void *dw3, xmoe_dtype grad_dt, int32_t accumulate, void *stream) {
    TRY(check_dtype(dtype));
    TRY(check_grad_dt(dtype, grad_dt, accumulate));
    REQUIRE(dw1 && dw3 && (rows == 0 || (xs && dh13)), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(xs) && aligned16(dh13) && aligned16(dw1) && aligned16(dw3), XMOE_ERR_UNSUPPORTED,
            "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_bwd_dw13(dtype, xs, nullptr, 0, dh13, expert_offsets, E, rows, d, h, dw1, dw3,
                                                grad_dt, accumulate != 0, S(stream)),
                      "xmoe_expert_ffn_bwd_dw13 launch");
}

xmoe_status xmoe_expert_ffn_bwd_dw13_gather(const void *x, const int32_t *token_ids, const void *dh13,
                                            xmoe_dtype dtype, const int32_t *expert_offsets, int32_t E, int64_t T,
                                            int64_t rows, int32_t d, int32_t h, void *dw1, void *dw3,
                                            xmoe_dtype grad_dt, int32_t accumulate, void *stream) {
    TRY(check_dtype(dtype));
    TRY(check_grad_dt(dtype, grad_dt, accumulate));
    REQUIRE(dw1 && dw3 && (rows == 0 || dh13), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    TRY(check_gather(x, token_ids, T, rows, d, dtype));
    REQUIRE(aligned16(dh13) && aligned16(dw1) && aligned16(dw3), XMOE_ERR_UNSUPPORTED,
            "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_bwd_dw13(dtype, x, token_ids, T, dh13, expert_offsets, E, rows, d, h, dw1, dw3,
                                                grad_dt, accumulate != 0, S(stream)),
                      "xmoe_expert_ffn_bwd_dw13_gather launch");
}

xmoe_status xmoe_expert_ffn_bwd_dw2(const void *act, const void *dye, xmoe_dtype dtype,
                                    const int32_t *expert_offsets, int32_t E, int64_t rows, int32_t d, int32_t h,
                                    void *dw2, xmoe_dtype grad_dt, int32_t accumulate, void *stream) {
    TRY(check_dtype(dtype));
    TRY(check_grad_dt(dtype, grad_dt, accumulate));
    REQUIRE(dw2 && (rows == 0 || (act && dye)), XMOE_ERR_INVALID_VALUE, "a required pointer is NULL");
    TRY(check_ffn_sizes(expert_offsets, E, rows, d, h));
    REQUIRE(aligned16(act) && aligned16(dye) && aligned16(dw2), XMOE_ERR_UNSUPPORTED,
            "matrices must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ffn_bwd_dw2(dtype, act, dye, expert_offsets, E, rows, d, h, dw2, grad_dt,
                                               accumulate != 0, S(stream)),
                      "xmoe_expert_ffn_bwd_dw2 launch");
}

xmoe_status xmoe_dispatch_bwd(const void *dxs, const xmoe_pft *pft, int64_t T, int32_t d, int32_t k, xmoe_dtype dtype,
                              const void *dx_add, void *dx, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(T == 0 || (dxs && dx), XMOE_ERR_INVALID_VALUE, "dxs and dx are required");
    TRY(check_rows_common(T, d, k));
    TRY(check_pft(pft, T > 0, false, false));
    REQUIRE(aligned16(dxs) && aligned16(dx) && aligned16(dx_add), XMOE_ERR_UNSUPPORTED,
            "rows must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_gather_sum(dtype, dxs, pft->slot_to_row, nullptr, T, d, k, dx_add, dx, S(stream)),
                      "xmoe_dispatch_bwd launch");
}

size_t xmoe_route_bwd_workspace_size(int64_t T, int32_t d, int32_t E, xmoe_dtype dtype) {
    if (T < 0 || T > kMaxRows || d < 1 || E < 1 || E > 1024 || (dtype != XMOE_F32 && dtype != XMOE_BF16)) return 0;
    return xmoe::route_bwd_workspace(T, d, E, dtype);
}

xmoe_status xmoe_route_bwd(const void *x, const void *wg, const float *logits, const int32_t *topk_ids,
                           const float *dtopk_w, int32_t ldw, xmoe_dtype dtype, int64_t T, int32_t d, int32_t E,
                           int32_t k, float inv_temperature, int32_t accumulate, void *dx, float *dwg,
                           void *workspace, size_t ws_bytes, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(wg && dwg && (T == 0 || (x && logits && topk_ids && dtopk_w && dx)), XMOE_ERR_INVALID_VALUE,
            "a required pointer is NULL");
    REQUIRE(T >= 0 && T <= kMaxRows && d >= 1, XMOE_ERR_INVALID_VALUE, "T must be in [0, 2^31) and d >= 1");
    REQUIRE(E >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E must be in [1, 1024]");
    REQUIRE(k >= 1 && k <= E, XMOE_ERR_INVALID_VALUE, "k must be in [1, E]");
    REQUIRE(ldw >= k, XMOE_ERR_INVALID_VALUE, "ldw must be >= k");
    REQUIRE(within(T, ldw, kMaxRows), XMOE_ERR_INVALID_VALUE, "T*ldw must be < 2^31");
    if (dtype == XMOE_BF16) {
        REQUIRE(d % 8 == 0 && E % 8 == 0, XMOE_ERR_UNSUPPORTED, "bf16 needs d and E multiples of 8");
        REQUIRE(aligned16(x) && aligned16(wg) && aligned16(dx), XMOE_ERR_UNSUPPORTED,
                "x, wg and dx must be 16-byte aligned");
    }
    const size_t need = xmoe::route_bwd_workspace(T, d, E, dtype);
    REQUIRE(workspace && aligned16(workspace), XMOE_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
    REQUIRE(ws_bytes >= need, XMOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
    CHECK_DEVICE();
    return hip_status(xmoe::launch_route_bwd(dtype, x, wg, logits, topk_ids, dtopk_w, ldw, T, d, E, k, inv_temperature,
                                             accumulate != 0, dx, dwg, workspace, S(stream)),
                      "xmoe_route_bwd launch");
}

/* ---------------------------------------------- pilot tokens and EP plans */

size_t xmoe_build_pilots_workspace_size(int64_t T, int32_t E, int32_t k, int32_t experts_per_node) {
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || !within(T, k, kMaxRows) ||
        experts_per_node < 1 || E % experts_per_node != 0)
        return 0;
    return xmoe::pft_workspace(T, E / experts_per_node);
}

xmoe_status xmoe_build_pilots(const int32_t *topk_ids, int64_t T, int32_t E, int32_t k, int32_t experts_per_node,
                              int32_t *pilot_token_ids, int32_t *pilot_node_ids, int32_t *node_counts,
                              int32_t *node_offsets, int32_t *slot_to_pilot, void *workspace, size_t ws_bytes,
                              void *stream) {
    REQUIRE(T >= 0, XMOE_ERR_INVALID_VALUE, "T must be >= 0");
    REQUIRE(E >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E must be in [1, 1024]");
    REQUIRE(k >= 1 && k <= E, XMOE_ERR_INVALID_VALUE, "k must be in [1, E]");
    REQUIRE(within(T, k, kMaxRows), XMOE_ERR_INVALID_VALUE, "T*k must be < 2^31");
    REQUIRE(experts_per_node >= 1 && E % experts_per_node == 0, XMOE_ERR_INVALID_VALUE,
            "experts_per_node must divide E");
    REQUIRE(node_counts && node_offsets, XMOE_ERR_INVALID_VALUE, "node_counts and node_offsets are required");
    REQUIRE(T == 0 || (topk_ids && pilot_token_ids && pilot_node_ids && slot_to_pilot), XMOE_ERR_INVALID_VALUE,
            "topk_ids, pilot_token_ids, pilot_node_ids and slot_to_pilot are required");
    const size_t need = xmoe::pft_workspace(T, E / experts_per_node);
    REQUIRE(workspace && aligned16(workspace), XMOE_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
    REQUIRE(ws_bytes >= need, XMOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
    CHECK_DEVICE();
    const xmoe::PilotPtrs pl{pilot_token_ids, pilot_node_ids, node_counts, node_offsets, slot_to_pilot};
    return hip_status(xmoe::launch_build_pilots(topk_ids, T, E, k, experts_per_node, pl, workspace, S(stream)),
                      "xmoe_build_pilots launch");
}

xmoe_status xmoe_ep_send_plan(const int32_t *expert_offsets, int32_t E, int32_t G, int32_t *send_counts,
                              int32_t *send_displs, void *stream) {
    REQUIRE(expert_offsets && send_counts && send_displs, XMOE_ERR_INVALID_VALUE,
            "expert_offsets, send_counts and send_displs are required");
    REQUIRE(E >= 1 && E <= 1024, XMOE_ERR_INVALID_VALUE, "E must be in [1, 1024]");
    REQUIRE(G >= 1 && E % G == 0, XMOE_ERR_INVALID_VALUE, "G must divide E");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ep_send_plan(expert_offsets, E, G, send_counts, send_displs, S(stream)),
                      "xmoe_ep_send_plan launch");
}

size_t xmoe_ep_recv_plan_workspace_size(int32_t G, int32_t E_local) {
    if (G < 1 || E_local < 1 || static_cast<int64_t>(G) * E_local > 1024) return 0;
    return xmoe::ep_recv_plan_workspace(G, E_local);
}

xmoe_status xmoe_ep_recv_plan(const int32_t *recv_counts, int32_t G, int32_t E_local, int64_t n_recv,
                              int32_t *local_offsets, int32_t *recv_displs, int32_t *local_to_recv,
                              int32_t *recv_to_local, void *workspace, size_t ws_bytes, void *stream) {
    REQUIRE(recv_counts && local_offsets && recv_displs, XMOE_ERR_INVALID_VALUE,
            "recv_counts, local_offsets and recv_displs are required");
    REQUIRE(G >= 1 && E_local >= 1 && static_cast<int64_t>(G) * E_local <= 1024, XMOE_ERR_INVALID_VALUE,
            "G >= 1, E_local >= 1 and G*E_local <= 1024 are required");
    REQUIRE(n_recv >= 0 && n_recv <= kMaxRows, XMOE_ERR_INVALID_VALUE, "n_recv must be in [0, 2^31)");
    REQUIRE(n_recv == 0 || (local_to_recv && recv_to_local), XMOE_ERR_INVALID_VALUE,
            "local_to_recv and recv_to_local are required");
    const size_t need = xmoe::ep_recv_plan_workspace(G, E_local);
    REQUIRE(workspace && aligned16(workspace), XMOE_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
    REQUIRE(ws_bytes >= need, XMOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
    CHECK_DEVICE();
    return hip_status(xmoe::launch_ep_recv_plan(recv_counts, G, E_local, n_recv, local_offsets, recv_displs,
                                                local_to_recv, recv_to_local, workspace, S(stream)),
                      "xmoe_ep_recv_plan launch");
}

xmoe_status xmoe_scatter_rows(const void *src, xmoe_dtype dtype, int64_t n, int32_t d, const int32_t *index,
                              int64_t dst_rows, void *dst, void *stream) {
    TRY(check_dtype(dtype));
    REQUIRE(n >= 0 && n <= kMaxRows && dst_rows >= 0 && dst_rows <= kMaxRows, XMOE_ERR_INVALID_VALUE,
            "n and dst_rows must be in [0, 2^31)");
    REQUIRE(n == 0 || (src && index && dst), XMOE_ERR_INVALID_VALUE, "src, index and dst are required");
    REQUIRE(d >= 1, XMOE_ERR_INVALID_VALUE, "d must be >= 1");
    REQUIRE(d % 8 == 0, XMOE_ERR_UNSUPPORTED, "d must be a multiple of 8");
    REQUIRE(aligned16(src) && aligned16(dst), XMOE_ERR_UNSUPPORTED, "src and dst must be 16-byte aligned");
    CHECK_DEVICE();
    return hip_status(xmoe::launch_scatter_rows(dtype, src, n, d, index, dst_rows, dst, S(stream)),
                      "xmoe_scatter_rows launch");
}

}  // extern "C"

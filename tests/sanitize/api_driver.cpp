// Drives every entry point of the C ABI through its host-side validation
// (built with the host sanitizers, device work stubbed out): invalid
// arguments must be rejected with the documented status and a message, and
// calls that pass validation must stop at the device check (no GPU here) with
// XMOE_ERR_HIP or XMOE_ERR_UNSUPPORTED, never touching memory.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/xmoe.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                                       \
    do {                                                                                         \
        const int _got = (call);                                                                 \
        if (_got != (want)) {                                                                    \
            std::printf("FAIL %s:%d %s -> %d (want %d): %s\n", __FILE__, __LINE__, #call, _got, \
                        static_cast<int>(want), xmoe_last_error());                              \
            ++g_fail;                                                                            \
        }                                                                                        \
    } while (0)
// passes validation, then the device check fails (no GPU) or reports a non-gfx950 device
#define EXPECT_DEVICE(call)                                                                      \
    do {                                                                                         \
        const int _got = (call);                                                                 \
        if (_got != XMOE_ERR_HIP && _got != XMOE_ERR_UNSUPPORTED) {                              \
            std::printf("FAIL %s:%d %s -> %d (want a device error)\n", __FILE__, __LINE__, #call, _got); \
            ++g_fail;                                                                            \
        }                                                                                        \
        if (std::strlen(xmoe_last_error()) == 0) ++g_fail;                                       \
    } while (0)

int main() {
    // 16-byte aligned stand-ins: validation never dereferences them
    alignas(16) static char buf[4096];
    void *p = buf;
    const int32_t *ip = reinterpret_cast<const int32_t *>(buf);
    const float *fp = reinterpret_cast<const float *>(buf);
    int32_t *op = reinterpret_cast<int32_t *>(buf);
    float *of = reinterpret_cast<float *>(buf);
    xmoe_pft pft = {op, op, op, op, of, op};
    const xmoe_dtype bf = XMOE_BF16, f32 = XMOE_F32;

    EXPECT(xmoe_route(nullptr, nullptr, bf, 10, 8, 8, 2, 1.f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                      nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT(xmoe_route(p, p, bf, 10, 8, 8, 9, 1.f, nullptr, nullptr, op, of, of, nullptr, 0, nullptr),
           XMOE_ERR_INVALID_VALUE);
    EXPECT(xmoe_route(p, p, static_cast<xmoe_dtype>(7), 10, 8, 8, 2, 1.f, nullptr, nullptr, op, of, of, nullptr, 0,
                      nullptr), XMOE_ERR_UNSUPPORTED);
    EXPECT(xmoe_route(p, p, bf, 10, 64, 8, 2, 1.f, nullptr, nullptr, op, of, of, nullptr, 0, nullptr),
           XMOE_ERR_WORKSPACE);
    EXPECT_DEVICE(xmoe_route(p, p, bf, 4, 64, 8, 2, 1.f, fp, fp, op, of, of, p, 4096, nullptr));
    EXPECT_DEVICE(xmoe_route(p, p, f32, 4, 64, 8, 2, 1.f, nullptr, nullptr, op, of, of, nullptr, 0, nullptr));
    size_t ws = xmoe_build_pft_workspace_size(1000, 16, 4);
    EXPECT(xmoe_build_pft(ip, fp, 1000, 16, 4, &pft, p, 8, nullptr), XMOE_ERR_WORKSPACE);
    EXPECT(xmoe_build_pft(ip, fp, 10, 16, 17, &pft, p, ws, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT(xmoe_build_pft(ip, fp, 10, 16, 4, nullptr, p, ws, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT_DEVICE(xmoe_build_pft(ip, fp, 10, 16, 4, &pft, p, 4096, nullptr));
    EXPECT(xmoe_build_pft_noalloc(ip, fp, 130817, 1024, 8, &pft, nullptr), XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_build_pft_noalloc(ip, fp, 100, 64, 6, &pft, nullptr));
    EXPECT(xmoe_build_pft_shared(ip, fp, 100, 64, 6, -1, &pft, p, 1 << 20, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT(xmoe_dispatch(p, bf, int64_t{1} << 30, 64, 8, &pft, p, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT(xmoe_dispatch(p, bf, 10, 12, 2, &pft, p, nullptr), XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_dispatch(p, bf, 10, 64, 2, &pft, p, nullptr));
    EXPECT(xmoe_expert_ffn_up(p, p, p, bf, ip, 4, 100, 64, 12, p, nullptr, nullptr), XMOE_ERR_UNSUPPORTED);
    EXPECT(xmoe_expert_ffn_up(p, p, p, bf, nullptr, 4, 100, 64, 64, p, nullptr, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT(xmoe_expert_ffn_up(buf + 2, p, p, bf, ip, 4, 100, 64, 64, p, nullptr, nullptr), XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_expert_ffn_up(p, p, p, bf, ip, 4, 100, 64, 64, p, nullptr, nullptr));
    EXPECT_DEVICE(xmoe_expert_ffn_down(p, p, bf, ip, 4, 100, 64, 64, p, 1, nullptr));
    EXPECT_DEVICE(xmoe_expert_ffn(p, p, p, p, bf, ip, 4, 100, 64, 64, p, p, p, 0, nullptr));
    EXPECT(xmoe_expert_ffn_up_gather(p, ip, p, p, bf, ip, 4, int64_t{1} << 17, 100, 8192, 64, p, nullptr, nullptr),
           XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_expert_ffn_gather(p, ip, p, p, p, bf, ip, 4, 100, 100, 64, 64, p, p, p, 0, nullptr));
    EXPECT(xmoe_combine(p, &pft, 10, 64, 0, bf, nullptr, p, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT_DEVICE(xmoe_combine(p, &pft, 10, 64, 2, bf, p, p, nullptr));
    EXPECT_DEVICE(xmoe_combine_bwd(p, p, &pft, 10, 64, 2, bf, p, of, nullptr));
    EXPECT(xmoe_expert_ffn_bwd(p, p, p, p, p, p, p, bf, ip, 4, 100, 64, 64, p, p, 0, p, p, p, bf, 1, nullptr),
           XMOE_ERR_UNSUPPORTED);
    EXPECT(xmoe_expert_ffn_bwd(p, p, p, p, p, p, p, f32, ip, 4, 100, 64, 64, p, p, 0, p, p, p, bf, 0, nullptr),
           XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_expert_ffn_bwd(p, p, p, p, p, p, p, bf, ip, 4, 100, 64, 64, p, p, 1, p, p, p, f32, 1, nullptr));
    EXPECT_DEVICE(xmoe_expert_ffn_bwd_dact(p, p, p, bf, ip, 4, 100, 64, 64, p, nullptr));
    EXPECT(xmoe_expert_ffn_bwd_dact_gather(p, ip, nullptr, p, p, bf, ip, 4, 100, 100, 64, 64, p, nullptr),
           XMOE_ERR_INVALID_VALUE);
    EXPECT(xmoe_expert_ffn_bwd_dact_gather(p, ip, fp, p, p, bf, ip, 4, int64_t{1} << 17, 100, 8192, 64, p, nullptr),
           XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_expert_ffn_bwd_dact_gather(p, ip, fp, p, p, bf, ip, 4, 100, 100, 64, 64, p, nullptr));
    EXPECT_DEVICE(xmoe_expert_ffn_bwd_dx(p, p, p, bf, ip, 4, 100, 64, 64, p, 1, nullptr));
    EXPECT(xmoe_expert_ffn_bwd_dw13(p, p, bf, ip, 4, 100, 64, 64, p, p, static_cast<xmoe_dtype>(9), 0, nullptr),
           XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_expert_ffn_bwd_dw13(p, p, bf, ip, 4, 100, 64, 64, p, p, f32, 1, nullptr));
    EXPECT_DEVICE(xmoe_expert_ffn_bwd_dw13_gather(p, ip, p, bf, ip, 4, 100, 100, 64, 64, p, p, bf, 0, nullptr));
    EXPECT(xmoe_expert_ffn_bwd_dw2(p, p, bf, ip, 4, 100, 64, 64, p, bf, 1, nullptr), XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_expert_ffn_bwd_dw2(p, p, bf, ip, 4, 100, 64, 64, p, f32, 0, nullptr));
    EXPECT_DEVICE(xmoe_dispatch_bwd(p, &pft, 10, 64, 2, bf, p, p, nullptr));
    EXPECT(xmoe_route_bwd(p, p, fp, ip, fp, 3, bf, 100, 64, 64, 6, 1.f, 1, p, of, p, 1 << 20, nullptr),
           XMOE_ERR_INVALID_VALUE);
    EXPECT_DEVICE(xmoe_route_bwd(p, p, fp, ip, fp, 6, bf, 10, 64, 64, 6, 1.f, 1, p, of, p, 1 << 20, nullptr));
    EXPECT(xmoe_build_pilots(ip, 100, 64, 6, 5, op, op, op, op, op, p, 1 << 20, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT_DEVICE(xmoe_build_pilots(ip, 100, 64, 6, 8, op, op, op, op, op, p, 1 << 20, nullptr));
    EXPECT(xmoe_ep_send_plan(ip, 64, 6, op, op, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT_DEVICE(xmoe_ep_send_plan(ip, 64, 8, op, op, nullptr));
    EXPECT(xmoe_ep_recv_plan(ip, 64, 32, 10, op, op, op, op, p, 1 << 20, nullptr), XMOE_ERR_INVALID_VALUE);
    EXPECT_DEVICE(xmoe_ep_recv_plan(ip, 8, 8, 10, op, op, op, op, p, 1 << 20, nullptr));
    EXPECT(xmoe_scatter_rows(p, bf, 10, 12, ip, 10, p, nullptr), XMOE_ERR_UNSUPPORTED);
    EXPECT_DEVICE(xmoe_scatter_rows(p, bf, 10, 16, ip, 10, p, nullptr));
    int is950 = -1;
    (void)xmoe_query_device(0, &is950);
    EXPECT(xmoe_query_device(0, nullptr), XMOE_ERR_INVALID_VALUE);
    std::printf("%s: %d failures\n", g_fail ? "FAILED" : "ok", g_fail);
    return g_fail ? 1 : 0;
}

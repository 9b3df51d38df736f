// Random arguments for every entry point of the C ABI, through the host-side
// validation only (device work stubbed out, no GPU visible): whatever the
// sizes, flags and pointers, a call must return one of the documented
// statuses, leave a message when it fails, and do nothing the host sanitizers
// flag (no signed overflow in the size arithmetic, no read of the pointers).
// Values are drawn from the edges of each parameter's range.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/xmoe.h"

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t next() {  // splitmix64
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
template <typename T, size_t N>
T pick(const T (&v)[N]) { return v[next() % N]; }

const int64_t kI64[] = {0, 1, 2, 7, 8, 255, 256, 4096, 65535, (int64_t{1} << 31) - 1, int64_t{1} << 31,
                        int64_t{1} << 32, int64_t{1} << 40, int64_t{1} << 62, std::numeric_limits<int64_t>::max(),
                        -1, -7, std::numeric_limits<int64_t>::min()};
const int32_t kI32[] = {0, 1, 2, 3, 7, 8, 12, 16, 64, 96, 1023, 1024, 1025, 4096, 7168, 1 << 20, (1 << 20) + 8,
                        std::numeric_limits<int32_t>::max(), -1, -8, std::numeric_limits<int32_t>::min()};
const size_t kSz[] = {0, 16, 4096, size_t{1} << 32, std::numeric_limits<size_t>::max()};
const float kF[] = {1.0f, 0.5f, 0.0f, -1.0f};

alignas(16) char g_buf[4096];
void *ptr() {
    switch (next() % 4) {
        case 0: return nullptr;
        case 1: return g_buf + 2;  // misaligned
        default: return g_buf;
    }
}
template <typename T>
T *tp() { return static_cast<T *>(ptr()); }
xmoe_dtype dt() {
    const int v[] = {XMOE_BF16, XMOE_BF16, XMOE_F32, 7};
    return static_cast<xmoe_dtype>(pick(v));
}
int64_t I64() { return pick(kI64); }
int32_t I32() { return pick(kI32); }
size_t SZ() { return pick(kSz); }
float F() { return pick(kF); }
xmoe_pft g_pft;
const xmoe_pft *pft() {
    if (next() % 5 == 0) return nullptr;
    g_pft = {tp<int32_t>(), tp<int32_t>(), tp<int32_t>(), tp<int32_t>(), tp<float>(), tp<int32_t>()};
    return &g_pft;
}

int g_fail = 0;
void check(int st, const char *name) {
    if (st < XMOE_OK || st > XMOE_ERR_HIP) {
        std::printf("FAIL %s returned %d\n", name, st);
        ++g_fail;
    } else if (st != XMOE_OK && std::strlen(xmoe_last_error()) == 0) {
        std::printf("FAIL %s returned %d with no message\n", name, st);
        ++g_fail;
    }
}
#define CALL(f, ...) check(f(__VA_ARGS__), #f)

}  // namespace

int main() {
    for (int it = 0; it < 4000; ++it) {
        CALL(xmoe_route, ptr(), ptr(), dt(), I64(), I32(), I32(), I32(), F(), tp<float>(), tp<float>(), tp<int32_t>(),
             tp<float>(), tp<float>(), ptr(), SZ(), nullptr);
        (void)xmoe_route_workspace_size(I64(), I32(), I32(), dt());
        (void)xmoe_build_pft_workspace_size(I64(), I32(), I32());
        CALL(xmoe_build_pft, tp<int32_t>(), tp<float>(), I64(), I32(), I32(), pft(), ptr(), SZ(), nullptr);
        CALL(xmoe_build_pft_noalloc, tp<int32_t>(), tp<float>(), I64(), I32(), I32(), pft(), nullptr);
        CALL(xmoe_build_pft_shared, tp<int32_t>(), tp<float>(), I64(), I32(), I32(), I32(), pft(), ptr(), SZ(), nullptr);
        CALL(xmoe_dispatch, ptr(), dt(), I64(), I32(), I32(), pft(), ptr(), nullptr);
        CALL(xmoe_expert_ffn_up, ptr(), ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I32(), I32(), ptr(), ptr(),
             nullptr);
        CALL(xmoe_expert_ffn_down, ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I32(), I32(), ptr(), I32(), nullptr);
        CALL(xmoe_expert_ffn_up_gather, ptr(), tp<int32_t>(), ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I64(),
             I32(), I32(), ptr(), ptr(), nullptr);
        CALL(xmoe_expert_ffn_gather, ptr(), tp<int32_t>(), ptr(), ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(),
             I64(), I32(), I32(), ptr(), ptr(), ptr(), I32(), nullptr);
        CALL(xmoe_expert_ffn, ptr(), ptr(), ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I32(), I32(), ptr(),
             ptr(), ptr(), I32(), nullptr);
        CALL(xmoe_combine, ptr(), pft(), I64(), I32(), I32(), dt(), ptr(), ptr(), nullptr);
        CALL(xmoe_combine_bwd, ptr(), ptr(), pft(), I64(), I32(), I32(), dt(), ptr(), tp<float>(), nullptr);
        CALL(xmoe_expert_ffn_bwd, ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(),
             I32(), I32(), ptr(), ptr(), I32(), ptr(), ptr(), ptr(), dt(), I32(), nullptr);
        CALL(xmoe_expert_ffn_bwd_dact, ptr(), ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I32(), I32(), ptr(),
             nullptr);
        CALL(xmoe_expert_ffn_bwd_dact_gather, ptr(), tp<int32_t>(), tp<float>(), ptr(), ptr(), dt(), tp<int32_t>(),
             I32(), I64(), I64(), I32(), I32(), ptr(), nullptr);
        CALL(xmoe_expert_ffn_bwd_dx, ptr(), ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I32(), I32(), ptr(),
             I32(), nullptr);
        CALL(xmoe_expert_ffn_bwd_dw13, ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I32(), I32(), ptr(), ptr(),
             dt(), I32(), nullptr);
        CALL(xmoe_expert_ffn_bwd_dw13_gather, ptr(), tp<int32_t>(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I64(),
             I32(), I32(), ptr(), ptr(), dt(), I32(), nullptr);
        CALL(xmoe_expert_ffn_bwd_dw2, ptr(), ptr(), dt(), tp<int32_t>(), I32(), I64(), I32(), I32(), ptr(), dt(),
             I32(), nullptr);
        CALL(xmoe_dispatch_bwd, ptr(), pft(), I64(), I32(), I32(), dt(), ptr(), ptr(), nullptr);
        (void)xmoe_route_bwd_workspace_size(I64(), I32(), I32(), dt());
        CALL(xmoe_route_bwd, ptr(), ptr(), tp<float>(), tp<int32_t>(), tp<float>(), I32(), dt(), I64(), I32(), I32(),
             I32(), F(), I32(), ptr(), tp<float>(), ptr(), SZ(), nullptr);
        (void)xmoe_build_pilots_workspace_size(I64(), I32(), I32(), I32());
        CALL(xmoe_build_pilots, tp<int32_t>(), I64(), I32(), I32(), I32(), tp<int32_t>(), tp<int32_t>(), tp<int32_t>(),
             tp<int32_t>(), tp<int32_t>(), ptr(), SZ(), nullptr);
        CALL(xmoe_ep_send_plan, tp<int32_t>(), I32(), I32(), tp<int32_t>(), tp<int32_t>(), nullptr);
        (void)xmoe_ep_recv_plan_workspace_size(I32(), I32());
        CALL(xmoe_ep_recv_plan, tp<int32_t>(), I32(), I32(), I64(), tp<int32_t>(), tp<int32_t>(), tp<int32_t>(),
             tp<int32_t>(), ptr(), SZ(), nullptr);
        CALL(xmoe_scatter_rows, ptr(), dt(), I64(), I32(), tp<int32_t>(), I64(), ptr(), nullptr);
    }
    std::printf("fuzz: %d failures\n", g_fail);
    return g_fail == 0 ? 0 : 1;
}

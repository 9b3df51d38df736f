// Expert-parallel plans around the padding-free layer.
//
// "5.4 MoE模型在分布式训练中的应用", section 专家并行 (数据流, All-to-All通信步骤):
// each of G ranks holds a block of experts; dispatch sends every rank the
// tokens routed to its experts, the rank runs them, combine sends the results
// back.  The X-MoE article (adg.csdn.net), section 2.1.1 "PFT数据结构创新",
// moves the Padding-Free Token rows with an alltoallv and no padding.  Rank q
// holds the E/G consecutive experts [q*E/G, (q+1)*E/G), so the rows for rank q
// are one contiguous run of the expert-sorted buffer: the send plan is the
// buffer's offsets at every E/G-th expert.
//
// A receiver gets its rows source-major (source s, then the source's experts
// ascending, then the source's row order) and lays them out expert-major
// (local expert e, then source s, then the same order) for its grouped GEMM.
// With C[s][e] the rows s sends for local expert e, block (s, e) starts at
//   arrival:       recv_displs[s]    + sum_{e' < e} C[s][e']
//   expert-major:  local_offsets[e]  + sum_{s' < s} C[s'][e]
// and row i of the block keeps its place i in both.  The exchange itself (two
// alltoallv over RCCL: the counts, then the rows) lies outside this library.
#include "common.hpp"
#include "kernels.hpp"

namespace xmoe {

namespace {

constexpr int kMaxCells = 1024;  // G * E_local = the experts of the layer

__global__ __launch_bounds__(256) void ep_send_plan_kernel(const int32_t *__restrict__ off, int E, int G,
                                                           int32_t *__restrict__ counts, int32_t *__restrict__ displs) {
    const int el = E / G;
    for (int q = threadIdx.x; q <= G; q += blockDim.x) {
        const int a = off[q * el];
        if (q < G) counts[q] = off[(q + 1) * el] - a;
        displs[q] = a;
    }
}

// Exclusive scan over the 1024 threads of the block (v of thread i -> sum of
// v over threads < i); `tot` receives the sum of all.
__device__ int block_exscan(int v, int *tmp, int *tot) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
    }
    if (lane == 63) tmp[wv] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wv) before += tmp[w];
        all += tmp[w];
    }
    __syncthreads();
    *tot = all;
    return before + inc - v;
}

// One block of 1024 threads.  Writes local_offsets, recv_displs and the two
// block starts of every (s, e) cell (arrival, expert-major) to `cell`.
__global__ __launch_bounds__(1024) void ep_recv_scan_kernel(const int32_t *__restrict__ C, int G, int el,
                                                            int32_t *__restrict__ local_offsets,
                                                            int32_t *__restrict__ recv_displs,
                                                            int32_t *__restrict__ cell) {
    __shared__ int c[kMaxCells];
    __shared__ int tmp[16];
    const int ncell = G * el;
    for (int i = threadIdx.x; i < ncell; i += blockDim.x) c[i] = C[i] < 0 ? 0 : C[i];
    __syncthreads();
    // per source: the row total and the arrival start of each of its cells
    int rsum = 0;
    if (static_cast<int>(threadIdx.x) < G)
        for (int e = 0; e < el; ++e) rsum += c[threadIdx.x * el + e];
    int tot;
    const int rdisp = block_exscan(rsum, tmp, &tot);
    if (static_cast<int>(threadIdx.x) < G) {
        recv_displs[threadIdx.x] = rdisp;
        if (static_cast<int>(threadIdx.x) == G - 1) recv_displs[G] = tot;
        int run = rdisp;
        for (int e = 0; e < el; ++e) {
            cell[2 * (threadIdx.x * el + e)] = run;
            run += c[threadIdx.x * el + e];
        }
    }
    // per local expert: the row total and the expert-major start of each cell
    int csum = 0;
    if (static_cast<int>(threadIdx.x) < el)
        for (int s = 0; s < G; ++s) csum += c[s * el + threadIdx.x];
    const int loff = block_exscan(csum, tmp, &tot);
    if (static_cast<int>(threadIdx.x) < el) {
        local_offsets[threadIdx.x] = loff;
        if (static_cast<int>(threadIdx.x) == el - 1) local_offsets[el] = tot;
        int run = loff;
        for (int s = 0; s < G; ++s) {
            cell[2 * (s * el + threadIdx.x) + 1] = run;
            run += c[s * el + threadIdx.x];
        }
    }
}

// One block per (s, e) cell: row i of the cell is arrival row a0 + i and
// expert-major row l0 + i.  Rows at or past n are not written.
__global__ __launch_bounds__(256) void ep_recv_map_kernel(const int32_t *__restrict__ C, int el, int64_t n,
                                                          const int32_t *__restrict__ cell,
                                                          int32_t *__restrict__ local_to_recv,
                                                          int32_t *__restrict__ recv_to_local) {
    const int id = blockIdx.x;
    const int cnt = C[id] < 0 ? 0 : C[id];
    const int64_t a0 = cell[2 * id], l0 = cell[2 * id + 1];
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
        const int64_t a = a0 + i, l = l0 + i;
        if (a < n && l < n) {
            local_to_recv[l] = static_cast<int32_t>(a);
            recv_to_local[a] = static_cast<int32_t>(l);
        }
    }
}

}  // namespace

hipError_t launch_ep_send_plan(const int32_t *expert_offsets, int E, int G, int32_t *send_counts,
                               int32_t *send_displs, hipStream_t s) {
    hipLaunchKernelGGL(ep_send_plan_kernel, dim3(1), dim3(256), 0, s, expert_offsets, E, G, send_counts, send_displs);
    return hipGetLastError();
}

size_t ep_recv_plan_workspace(int G, int el) { return static_cast<size_t>(2) * G * el * sizeof(int32_t) + 256; }

hipError_t launch_ep_recv_plan(const int32_t *recv_counts, int G, int el, int64_t n, int32_t *local_offsets,
                               int32_t *recv_displs, int32_t *local_to_recv, int32_t *recv_to_local, void *ws,
                               hipStream_t s) {
    int32_t *cell = static_cast<int32_t *>(ws);
    hipLaunchKernelGGL(ep_recv_scan_kernel, dim3(1), dim3(1024), 0, s, recv_counts, G, el, local_offsets, recv_displs,
                       cell);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || n <= 0) return err;
    hipLaunchKernelGGL(ep_recv_map_kernel, dim3(static_cast<unsigned>(G * el)), dim3(256), 0, s, recv_counts, el, n,
                       cell, local_to_recv, recv_to_local);
    return hipGetLastError();
}

}  // namespace xmoe

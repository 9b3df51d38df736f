// Padding-Free Token buffer construction.
//
// X-MoE article (adg.csdn.net), section 2.1.1 "PFT数据结构创新": instead of
// fixed-capacity expert buffers, a compact buffer records, per routed
// (token, expert) pair, the token's position, the expert, the combine weight
// and the per-expert token counts -- nothing padded, nothing dropped.  The
// row order is the one the article's per-expert GEMM (section 2.1.2) visits:
// experts ascending, tokens in input order within an expert.
//
// Three kernels, no host synchronisation and no global atomics:
//   1. count:   each block takes 256 consecutive tokens and marks, in an LDS
//               bitmap of E x 256 bits, which of its tokens chose each expert;
//               the popcount of an expert's 256 bits is the block's count.
//   2. scan:    one block turns the [blocks x E] counts into tokens_per_expert,
//               the exclusive scan expert_offsets, and each block's first row
//               per expert.
//   3. scatter: each block rebuilds its bitmap; the row of (t, e) is the
//               block's base for e plus the number of lower tokens of the block
//               whose bit for e is set -- a stable (expert, token) order.
//
// The same kernels build the pilot tokens of Redundancy-Bypassing Dispatch
// (X-MoE article, section 2.2.1 "分层冗余消除算法", Pilot Token选择): the key
// of a slot is then its expert's node, e / experts_per_node, and the bitmap
// keeps one bit per (node, token) however many of the token's experts sit on
// that node -- the per-node deduplication -- so the rows are the (token, node)
// pilots, listed by node, then token, and every slot of a token bound for one
// node gets the same pilot row.
//
// Shared experts can ride in the same buffer as experts every token is routed
// to with weight 1: with n_always > 0 each token has, after its k routed slots,
// n_always more slots for the last n_always experts (E - n_always + i).
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace xmoe {

// Library-owned scratch for callers that cannot allocate (launch_build_pft_static):
// the per-block counts and bases of the three kernels below.  Each device that
// runs the library holds one copy until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host the name is a stand-in, not
// a device address): it looks up the device address once per device with
// hipGetSymbolAddress and passes that.
static __device__ __align__(256) char scratch[kPftScratchBytes];

namespace {

constexpr int kChunk = 256;          // tokens per block
constexpr int kWords = kChunk / 32;  // bitmap words per expert
constexpr int kMaxE = 1024;

// key of an expert id: e / div (div = 1: the expert; experts per node: the node)
__device__ __forceinline__ int key_of(int e, int div) { return div == 1 ? e : e / div; }

// expert of slot j of token t: routed slots from ids, then the always-routed ones
__device__ __forceinline__ int slot_expert(const int32_t *__restrict__ ids, int64_t t, int j, int k, int E, int na) {
    if (j >= k) return E - na + (j - k);
    const int e = ids[t * k + j];
    return e < E - na ? e : -1;  // a routed id among the always-routed experts is invalid
}

__device__ void build_bitmap(uint32_t *bm, const int32_t *__restrict__ ids, int64_t T, int E, int k, int na,
                             int div) {
    const int nk = E / div;
    for (int i = threadIdx.x; i < nk * kWords; i += blockDim.x) bm[i] = 0u;
    __syncthreads();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kChunk + threadIdx.x;
    if (t < T) {
        const uint32_t bit = 1u << (threadIdx.x & 31);
        const int w = threadIdx.x >> 5;
        for (int j = 0; j < k + na; ++j) {
            const int e = slot_expert(ids, t, j, k, E, na);
            if (e >= 0 && e < E) atomicOr(&bm[key_of(e, div) * kWords + w], bit);
        }
    }
    __syncthreads();
}

// BY_NODE (a compile-time copy of the same code) only names the pilot build's
// launches apart from the buffer build's in a profile.
template <bool BY_NODE>
__global__ __launch_bounds__(kChunk) void pft_count_kernel(const int32_t *__restrict__ ids, int64_t T, int E, int k,
                                                           int na, int div, int32_t *__restrict__ counts) {
    __shared__ uint32_t bm[kMaxE * kWords];
    build_bitmap(bm, ids, T, E, k, na, div);
    const int nk = E / div;
    for (int e = threadIdx.x; e < nk; e += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWords; ++w) c += __popc(bm[e * kWords + w]);
        counts[static_cast<int64_t>(blockIdx.x) * nk + e] = c;
    }
}

// One block of 1024 threads.  Each key (expert or node) gets P = min(64,
// 1024 / E_p) consecutive lanes of one wave (E_p = E rounded up to a power of
// two); lane `part` of key e sums the counts of its range of token blocks with
// independent loads, a segmented scan over the key's lanes places the ranges,
// and a block-wide scan over the key totals gives the key offsets.
template <bool BY_NODE>
__global__ __launch_bounds__(1024) void pft_scan_kernel(const int32_t *__restrict__ counts, int nblk, int E,
                                                        int32_t *__restrict__ base, int32_t *__restrict__ tpe,
                                                        int32_t *__restrict__ offsets) {
    __shared__ int wave_tot[16];
    int ep = 1;
    while (ep < E) ep <<= 1;
    const int P = min(64, 1024 / ep);
    const int e = threadIdx.x / P, part = threadIdx.x % P;
    const bool live = e < E;
    const int per = (nblk + P - 1) / P;
    const int b0 = min(nblk, part * per), b1 = min(nblk, b0 + per);
    int mine = 0;
    if (live)
        for (int b = b0; b < b1; ++b) mine += counts[static_cast<int64_t>(b) * E + e];
    // segmented scan over the key's P lanes (P divides 64, so they share a wave)
    int inc = mine;
    for (int off = 1; off < P; off <<= 1) {
        const int v = __shfl_up(inc, off, P);
        if (part >= off) inc += v;
    }
    const int total = __shfl(inc, P - 1, P);  // the key's count
    const int before_part = inc - mine;
    // exclusive scan of the key totals: lane part 0 of each key contributes
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int v0 = part == 0 && live ? total : 0;
    int winc = v0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(winc, off, 64);
        if (lane >= off) winc += v;
    }
    if (lane == 63) wave_tot[wv] = winc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    const int off_e = __shfl(before + winc - v0, 0, P);  // the key's offset, from its lane 0
    if (live) {
        if (part == 0) {
            tpe[e] = total;
            offsets[e] = off_e;
            if (e == E - 1) offsets[E] = off_e + total;
        }
        int run = off_e + before_part;
        for (int b = b0; b < b1; ++b) {
            const int64_t i = static_cast<int64_t>(b) * E + e;
            base[i] = run;
            run += counts[i];
        }
    }
}

template <bool BY_NODE>
__global__ __launch_bounds__(kChunk) void pft_scatter_kernel(const int32_t *__restrict__ ids,
                                                          const float *__restrict__ wt, int64_t T, int E, int k,
                                                          int na, int div, const int32_t *__restrict__ base,
                                                          int32_t *__restrict__ tok, int32_t *__restrict__ eid,
                                                          float *__restrict__ cw, int32_t *__restrict__ s2r) {
    __shared__ uint32_t bm[kMaxE * kWords];
    build_bitmap(bm, ids, T, E, k, na, div);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kChunk + threadIdx.x;
    if (t >= T) return;
    const int ks = k + na;  // slots per token
    const int64_t R = T * ks;
    const int nk = E / div;
    const int wd = threadIdx.x >> 5;
    const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
    for (int j = 0; j < ks; ++j) {
        const int e = slot_expert(ids, t, j, k, E, na);
        int64_t r = -1;
        int key = -1;
        if (e >= 0 && e < E) {
            key = key_of(e, div);
            int rank = __popc(bm[key * kWords + wd] & below);
            for (int q = 0; q < wd; ++q) rank += __popc(bm[key * kWords + q]);
            r = base[static_cast<int64_t>(blockIdx.x) * nk + key] + rank;
            if (r >= R) r = -1;
        }
        s2r[t * ks + j] = static_cast<int32_t>(r);
        if (r >= 0) {  // a token's slots bound for one key write the same row with the same values
            if (tok) tok[r] = static_cast<int32_t>(t);
            if (eid) eid[r] = key;
            if (cw) cw[r] = j >= k ? 1.0f : (wt ? wt[t * k + j] : 0.0f);
        }
    }
}

}  // namespace

size_t pft_workspace(int64_t T, int E) {
    const int64_t nblk = (T + kChunk - 1) / kChunk;
    return static_cast<size_t>(2 * nblk * E) * sizeof(int32_t) + 256;
}

namespace {

// Stable counting sort of the slots by key (expert, or node when div > 1).
template <bool BY_NODE>
hipError_t keyed_sort(const int32_t *ids, const float *w, int64_t T, int E, int k, int na, int div, int32_t *tok,
                      int32_t *keyid,
                      int32_t *count_per_key, int32_t *offsets, float *cw, int32_t *s2r, void *ws, hipStream_t s) {
    const int64_t nblk = (T + kChunk - 1) / kChunk;
    const int nk = E / div;
    int32_t *counts = static_cast<int32_t *>(ws);
    int32_t *base = counts + nblk * nk;
    if (nblk > 0) {
        hipLaunchKernelGGL(pft_count_kernel<BY_NODE>, dim3(static_cast<unsigned>(nblk)), dim3(kChunk), 0, s, ids, T, E, k, na,
                           div, counts);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(pft_scan_kernel<BY_NODE>, dim3(1), dim3(1024), 0, s, counts, static_cast<int>(nblk), nk, base,
                       count_per_key, offsets);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nblk == 0) return err;
    hipLaunchKernelGGL(pft_scatter_kernel<BY_NODE>, dim3(static_cast<unsigned>(nblk)), dim3(kChunk), 0, s, ids, w, T, E, k, na,
                       div, base, tok, keyid, cw, s2r);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build_pft(const int32_t *ids, const float *w, int64_t T, int E, int k, int n_always,
                            const PftPtrs &pft, void *ws, hipStream_t s) {
    return keyed_sort<false>(ids, w, T, E, k, n_always, 1, pft.token_ids, pft.expert_ids, pft.tokens_per_expert, pft.expert_offsets,
                      pft.combine_weights, pft.slot_to_row, ws, s);
}

namespace {
constexpr int kMaxScratchDevices = 64;
void *g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t pft_scratch_address(void **out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // first call on this device (it is current): the device address of its copy
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_build_pft_static(const int32_t *ids, const float *w, int64_t T, int E, int k,
                                   const PftPtrs &pft, hipStream_t s) {
    if (pft_workspace(T, E) > kPftScratchBytes) return hipErrorInvalidValue;
    void *ws = nullptr;
    hipError_t err = pft_scratch_address(&ws);
    if (err != hipSuccess) return err;
    // the kernels write every count and base before reading it: nothing to clear
    return launch_build_pft(ids, w, T, E, k, 0, pft, ws, s);
}

hipError_t launch_build_pilots(const int32_t *ids, int64_t T, int E, int k, int experts_per_node,
                               const PilotPtrs &pl, void *ws, hipStream_t s) {
    return keyed_sort<true>(ids, nullptr, T, E, k, 0, experts_per_node, pl.pilot_token_ids, pl.pilot_node_ids, pl.node_counts,
                      pl.node_offsets, nullptr, pl.slot_to_pilot, ws, s);
}

}  // namespace xmoe

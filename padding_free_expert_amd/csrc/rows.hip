// Row-movement kernels: the dispatch gather, the combine, and their transposes.
//
// X-MoE article (adg.csdn.net), section 2.1.2: the gather copies row
// token_ids[r] of the input into row r of the expert-sorted buffer, one program
// per row over the hidden dimension.  Here the work is organised per token
// instead: a wavefront owns token t, reads its row once and writes (or reads)
// its k buffer rows slot_to_row[t*k + j].  Every row is moved exactly once, as
// whole 16-byte vectors per lane (the article's section 3.1 asks for contiguous
// accesses of at least 64 bytes; a wavefront moves 1 KiB per instruction), and
// sums over the k slots run in slot order in fp32 -- no atomics, deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace xmoe {

namespace {

constexpr int kWaves = 4;      // tokens per 256-thread block
constexpr int kUnroll = 4;     // 16-byte vectors in flight per lane

// 16-byte store marked non-temporal.  Measured per kernel in the layer: it
// speeds up the dispatch copy (35 -> 26 us at the DeepSeek-MoE-16B shape) and
// the gather-sums, and slows the combine backward, which keeps plain stores.
__device__ __forceinline__ void nt_store16(uint4 v, uint4 *p) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(p));
}

template <typename T>
__global__ __launch_bounds__(256) void dispatch_kernel(const T *__restrict__ x, const int32_t *__restrict__ s2r,
                                                       int64_t ntok, int d, int k, int64_t R, T *__restrict__ xs) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (t >= ntok) return;
    const int lane = threadIdx.x & 63;
    constexpr int V = Elem<T>::kVec;
    const int nvec = d / V;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + t * d);
    for (int jb = 0; jb < k; jb += 64) {
        const int nj = min(64, k - jb);
        const int r_lane = lane < nj ? s2r[t * k + jb + lane] : -1;
        // the trip count is the same for every lane: each lane must be active
        // when the others read its slot row with a shuffle (a read from an
        // inactive lane does not return that lane's value)
        for (int cb = 0; cb < nvec; cb += 64 * kUnroll) {
            const int c0 = cb + lane;
            uint4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + 64 * u;
                if (c < nvec) v[u] = src[c];
            }
            for (int j = 0; j < nj; ++j) {
                const int r = __shfl(r_lane, j, 64);
                if (r < 0 || r >= R) continue;
                uint4 *dst = reinterpret_cast<uint4 *>(xs + static_cast<int64_t>(r) * d);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int c = c0 + 64 * u;
                    if (c < nvec) nt_store16(v[u], &dst[c]);
                }
            }
        }
    }
}

// out[t] = sum_j w_j * src[slot_to_row[t*k+j]] (+ add[t]); w_j = weights[r_j] or 1.
template <typename T, bool WEIGHTED>
__global__ __launch_bounds__(256) void gather_sum_kernel(const T *__restrict__ src, const int32_t *__restrict__ s2r,
                                                         const float *__restrict__ wts, int64_t ntok, int d, int k,
                                                         int64_t R, const T *__restrict__ add, T *__restrict__ out) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (t >= ntok) return;
    const int lane = threadIdx.x & 63;
    constexpr int V = Elem<T>::kVec;
    const int nvec = d / V;
    // a wave-uniform trip count, as in the dispatch: every lane loads its slot
    // and takes part in the shuffles, also where d / V < k
    for (int cb = 0; cb < nvec; cb += 64 * kUnroll) {
        const int c0 = cb + lane;
        float acc[kUnroll][V];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[u][e] = 0.0f;
        for (int jb = 0; jb < k; jb += 64) {
            const int nj = min(64, k - jb);
            int r_lane = -1;
            float w_lane = 0.0f;
            if (lane < nj) {
                r_lane = s2r[t * k + jb + lane];
                if (r_lane >= 0 && r_lane < R) w_lane = WEIGHTED ? wts[r_lane] : 1.0f;
                else r_lane = -1;
            }
            for (int j = 0; j < nj; ++j) {
                const int r = __shfl(r_lane, j, 64);
                const float w = __shfl(w_lane, j, 64);
                if (r < 0) continue;
                const uint4 *row = reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(r) * d);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int c = c0 + 64 * u;
                    if (c < nvec) {
                        float f[V];
                        Elem<T>::unpack(row[c], f);
#pragma unroll
                        for (int e = 0; e < V; ++e) acc[u][e] = __builtin_fmaf(w, f[e], acc[u][e]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = c0 + 64 * u;
            if (c < nvec) {
                if (add) {
                    float f[V];
                    Elem<T>::unpack(reinterpret_cast<const uint4 *>(add + t * d)[c], f);
#pragma unroll
                    for (int e = 0; e < V; ++e) acc[u][e] += f[e];
                }
                nt_store16(Elem<T>::pack(acc[u]), &reinterpret_cast<uint4 *>(out + t * d)[c]);
            }
        }
    }
}

// dye[r_j] = w_j * dy[t];  dtopk_w[t, j] = <dy[t], ye[r_j]>  (slots in groups of 8)
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T *__restrict__ dy, const T *__restrict__ ye,
                                                          const int32_t *__restrict__ s2r,
                                                          const float *__restrict__ wts, int64_t ntok, int d, int k,
                                                          int64_t R, T *__restrict__ dye, float *__restrict__ dw) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (t >= ntok) return;
    const int lane = threadIdx.x & 63;
    constexpr int V = Elem<T>::kVec;
    constexpr int J = 8;
    const int nvec = d / V;
    const uint4 *g = reinterpret_cast<const uint4 *>(dy + t * d);
    for (int jb = 0; jb < k; jb += J) {
        int r[J];
        float w[J], part[J];
#pragma unroll
        for (int jj = 0; jj < J; ++jj) {
            const int j = jb + jj;
            r[jj] = j < k ? s2r[t * k + j] : -1;
            if (r[jj] < 0 || r[jj] >= R) r[jj] = -1;
            w[jj] = r[jj] >= 0 ? wts[r[jj]] : 0.0f;
            part[jj] = 0.0f;
        }
        for (int c = lane; c < nvec; c += 64) {
            float gv[V];
            Elem<T>::unpack(g[c], gv);
#pragma unroll
            for (int jj = 0; jj < J; ++jj) {
                if (r[jj] < 0) continue;
                const int64_t rb = static_cast<int64_t>(r[jj]) * d;
                float yv[V], ov[V];
                Elem<T>::unpack(reinterpret_cast<const uint4 *>(ye + rb)[c], yv);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    part[jj] = __builtin_fmaf(gv[e], yv[e], part[jj]);
                    ov[e] = w[jj] * gv[e];
                }
                reinterpret_cast<uint4 *>(dye + rb)[c] = Elem<T>::pack(ov);
            }
        }
#pragma unroll
        for (int jj = 0; jj < J; ++jj) {
            const float s = wave_sum(part[jj]);
            if (lane == 0 && jb + jj < k) dw[t * k + jb + jj] = s;
        }
    }
}

inline unsigned token_blocks(int64_t T) { return static_cast<unsigned>((T + kWaves - 1) / kWaves); }

}  // namespace

hipError_t launch_dispatch(int dt, const void *x, const int32_t *s2r, int64_t T, int d, int k, void *xs,
                           hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int64_t R = T * k;
    if (dt == kBF16)
        hipLaunchKernelGGL(dispatch_kernel<bf16_t>, dim3(token_blocks(T)), dim3(256), 0, s,
                           static_cast<const bf16_t *>(x), s2r, T, d, k, R, static_cast<bf16_t *>(xs));
    else
        hipLaunchKernelGGL(dispatch_kernel<float>, dim3(token_blocks(T)), dim3(256), 0, s,
                           static_cast<const float *>(x), s2r, T, d, k, R, static_cast<float *>(xs));
    return hipGetLastError();
}

// One row per source index: the dispatch copy with one destination per row.
hipError_t launch_scatter_rows(int dt, const void *src, int64_t n, int d, const int32_t *index, int64_t dst_rows,
                               void *dst, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (dt == kBF16)
        hipLaunchKernelGGL(dispatch_kernel<bf16_t>, dim3(token_blocks(n)), dim3(256), 0, s,
                           static_cast<const bf16_t *>(src), index, n, d, 1, dst_rows, static_cast<bf16_t *>(dst));
    else
        hipLaunchKernelGGL(dispatch_kernel<float>, dim3(token_blocks(n)), dim3(256), 0, s,
                           static_cast<const float *>(src), index, n, d, 1, dst_rows, static_cast<float *>(dst));
    return hipGetLastError();
}

hipError_t launch_gather_sum(int dt, const void *src, const int32_t *s2r, const float *weights, int64_t T, int d,
                             int k, const void *add, void *out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int64_t R = T * k;
    const dim3 grid(token_blocks(T)), block(256);
    if (dt == kBF16) {
        auto *a = static_cast<const bf16_t *>(add);
        if (weights)
            hipLaunchKernelGGL((gather_sum_kernel<bf16_t, true>), grid, block, 0, s, static_cast<const bf16_t *>(src),
                               s2r, weights, T, d, k, R, a, static_cast<bf16_t *>(out));
        else
            hipLaunchKernelGGL((gather_sum_kernel<bf16_t, false>), grid, block, 0, s, static_cast<const bf16_t *>(src),
                               s2r, weights, T, d, k, R, a, static_cast<bf16_t *>(out));
    } else {
        auto *a = static_cast<const float *>(add);
        if (weights)
            hipLaunchKernelGGL((gather_sum_kernel<float, true>), grid, block, 0, s, static_cast<const float *>(src), s2r,
                               weights, T, d, k, R, a, static_cast<float *>(out));
        else
            hipLaunchKernelGGL((gather_sum_kernel<float, false>), grid, block, 0, s, static_cast<const float *>(src), s2r,
                               weights, T, d, k, R, a, static_cast<float *>(out));
    }
    return hipGetLastError();
}

hipError_t launch_combine_bwd(int dt, const void *dy, const void *ye, const int32_t *s2r, const float *weights,
                              int64_t T, int d, int k, void *dye, float *dtopk_w, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int64_t R = T * k;
    if (dt == kBF16)
        hipLaunchKernelGGL(combine_bwd_kernel<bf16_t>, dim3(token_blocks(T)), dim3(256), 0, s,
                           static_cast<const bf16_t *>(dy), static_cast<const bf16_t *>(ye), s2r, weights, T, d, k, R,
                           static_cast<bf16_t *>(dye), dtopk_w);
    else
        hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3(token_blocks(T)), dim3(256), 0, s,
                           static_cast<const float *>(dy), static_cast<const float *>(ye), s2r, weights, T, d, k, R,
                           static_cast<float *>(dye), dtopk_w);
    return hipGetLastError();
}

}  // namespace xmoe

// Router (gate) forward and backward.
//
// "5.4 MoE模型在分布式训练中的应用", section 训练流程: every device computes the
// gate scores of its own tokens; X-MoE notes "略读笔记90", section 需求:
// fine-grained experts are used with a large top-k.  The pages give no gate
// formula; the one implemented is a softmax over the E experts of
// s = (x . Wg) * inv_tau + logit_bias, the top-k of s + select_bias with ties to
// the lower expert index, and the chosen probabilities as (unrenormalised)
// combine weights.
//
// Forward: one product x . Wg (bf16: split over d, fp32 partial sums) whose
// column tile spans all experts, then softmax + top-k with 8-32 lanes per
// token (k rounds of an arg-max over the token's lanes under the order (sel
// desc, index asc)).  Backward: the same lane layout forms dz = p * (g - c) *
// inv_tau; two products then give dx += dz . Wg^T and the split-T partials of
// Wg's gradient, which a last kernel sums in a fixed order.
#include <algorithm>

#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

namespace xmoe {

namespace {

constexpr int kWaves = 4;

// expert of value q in lane r of a token's LT lanes (16-byte chunks r, r + LT, ...)
template <int LT>
__device__ __forceinline__ int lane_expert(int r, int q) {
    return 4 * (r + LT * (q >> 2)) + (q & 3);
}

// A token's E values held by its LT lanes (lane r: QQ values, expert of value
// q = lane_expert(r, q)) written to row[0..E), 16 bytes at a time when E % 4 == 0.
template <int LT, int QQ>
__device__ __forceinline__ void store_row(float *row, const float (&s)[QQ], int r, int E) {
    if (E % 4 == 0) {
#pragma unroll
        for (int q = 0; q < QQ; q += 4)
            if (lane_expert<LT>(r, q) < E)
                *reinterpret_cast<float4 *>(row + lane_expert<LT>(r, q)) = make_float4(s[q], s[q + 1], s[q + 2], s[q + 3]);
    } else {
#pragma unroll
        for (int q = 0; q < QQ; ++q)
            if (lane_expert<LT>(r, q) < E) row[lane_expert<LT>(r, q)] = s[q];
    }
}

// Softmax and top-k of one token whose scaled, biased logits s (lane layout of
// store_row) sit in its LT lanes: the maximum and the denominator reduce over
// those lanes, then k rounds of an arg-max of s + select_bias under the order
// (value desc, expert index asc); the winner's lane writes the id and the
// probability exp(s - max) / den.  Every lane of the wavefront takes part in the
// shuffles; only live tokens write.
template <int LT, int QQ>
__device__ __forceinline__ void topk_select(const float (&s)[QQ], bool live, int r, int64_t t, int E, int k,
                                            const float *__restrict__ sbias, int32_t *__restrict__ ids,
                                            float *__restrict__ w) {
    float sel[QQ];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < QQ; ++q) {
        const int e = lane_expert<LT>(r, q);
        sel[q] = -INFINITY;
        if (live && e < E) {
            sel[q] = sbias ? __fadd_rn(s[q], sbias[e]) : s[q];
            mx = fmaxf(mx, s[q]);
        }
    }
#pragma unroll
    for (int off = LT / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float den = 0.0f;
#pragma unroll
    for (int q = 0; q < QQ; ++q)
        if (lane_expert<LT>(r, q) < E) den += expf(s[q] - mx);
#pragma unroll
    for (int off = LT / 2; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
    uint32_t taken = 0u;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = 0x7fffffff;  // no candidate
#pragma unroll
        for (int q = 0; q < QQ; ++q) {
            const int e = lane_expert<LT>(r, q);
            if (e < E && !((taken >> q) & 1u) && (bi == 0x7fffffff || sel[q] > bv)) {
                bv = sel[q];
                bi = e;
            }
        }
#pragma unroll
        for (int off = LT / 2; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if (live && r == (bi >> 2) % LT) {
            const int qb = ((bi >> 2) / LT) * 4 + (bi & 3);
            float sb = 0.0f;
#pragma unroll
            for (int q = 0; q < QQ; ++q)
                if (q == qb) sb = s[q];
            taken |= 1u << qb;
            ids[t * k + j] = bi;
            w[t * k + j] = expf(sb - mx) / den;
        }
    }
}

// LT lanes per token (8, 16 or 32), 64 / LT tokens per wavefront; lane r of a
// token holds QQ experts as 16-byte chunks r, r + LT, r + 2 LT, ... of the
// token's row (expert of value q: 4 (r + LT (q / 4)) + q % 4, ascending in q),
// so that every load and store instruction covers one contiguous run of the
// row; the vectors are used when E is a multiple of 4 (QQ always is).  When `part` is set, the
// logits are first formed from nparts fp32 partial sums of z (a split of the
// d reduction, summed in part order), then scaled and biased with one IEEE
// operation each and written to `logits`.  The softmax and the top-k (k
// rounds of an arg-max under the order (sel desc, index asc)) reduce over the
// token's LT lanes only: log2(LT) butterfly steps per round instead of six.
template <int LT, int QQ>
__global__ __launch_bounds__(256) void topk_softmax_kernel(float *__restrict__ logits, const float *__restrict__ part,
                                                           int nparts, int64_t part_stride, float scale,
                                                           const float *__restrict__ lbias,
                                                           const float *__restrict__ sbias, int64_t T, int E, int k,
                                                           int32_t *__restrict__ ids, float *__restrict__ w) {
    static_assert(LT == 8 || LT == 16 || LT == 32, "lanes per token");
    static_assert(QQ % 4 == 0 && QQ <= 32, "whole 16-byte vectors; one bit per value in the taken mask");
    constexpr int TPW = 64 / LT;
    const int lane = threadIdx.x & 63;
    const int r = lane % LT;
    auto ex = [&](int q) { return 4 * (r + LT * (q >> 2)) + (q & 3); };  // expert of value q
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6)) * TPW + lane / LT;
    const bool live = t < T;  // every lane stays for the shuffles; a token's lanes are all live or all not
    float s[QQ];
#pragma unroll
    for (int q = 0; q < QQ; ++q) s[q] = -INFINITY;
    // z (or the logits) of this lane's experts
    const float *src = part ? part : logits;
    if (live) {
        if (E % 4 == 0) {
#pragma unroll
            for (int q = 0; q < QQ; q += 4)
                if (ex(q) < E) {
                    const float4 v = *reinterpret_cast<const float4 *>(src + t * E + ex(q));
                    s[q] = v.x; s[q + 1] = v.y; s[q + 2] = v.z; s[q + 3] = v.w;
                }
            if (part)
                for (int pi = 1; pi < nparts; ++pi) {
#pragma unroll
                    for (int q = 0; q < QQ; q += 4)
                        if (ex(q) < E) {
                            const float4 v = *reinterpret_cast<const float4 *>(part + pi * part_stride + t * E + ex(q));
                            s[q] += v.x; s[q + 1] += v.y; s[q + 2] += v.z; s[q + 3] += v.w;
                        }
                }
        } else {
#pragma unroll
            for (int q = 0; q < QQ; ++q)
                if (ex(q) < E) {
                    float z = src[t * E + ex(q)];
                    if (part)
                        for (int pi = 1; pi < nparts; ++pi) z += part[pi * part_stride + t * E + ex(q)];
                    s[q] = z;
                }
        }
    }
    if (part && live) {
#pragma unroll
        for (int q = 0; q < QQ; ++q) {
            const int e = ex(q);
            if (e < E) {
                float v = __fmul_rn(s[q], scale);
                if (lbias) v = __fadd_rn(v, lbias[e]);
                s[q] = v;
            }
        }
        store_row<LT, QQ>(logits + t * E, s, r, E);
    }
    topk_select<LT, QQ>(s, live, r, t, E, k, sbias, ids, w);
}

// One launch for bf16 routing with up to 64 experts: a block takes TB tokens
// (16 or 32) and forms their E logits over the whole of d on the matrix cores,
// then runs the softmax and top-k on them in place, so no partial sums leave
// the chip.  With TB = 16 the products' rows 16..31 read whatever the ring
// holds there and are dropped.
// Each of the NWV waves reduces its own share of d (32-deep k blocks w,
// w + NWV, ...) through a private S-slot LDS ring filled by LDS DMA (x rows
// k-contiguous, Wg rows expert-contiguous, read with the transposing LDS
// read), so the k loop has no block-wide barrier.  The waves' fp32 partial
// tiles then meet in LDS and are added in wave order (deterministic), scaled
// and biased with one IEEE operation each, written to `logits`, and handed to
// topk_select with LT = 64 * NWV / TB lanes per token.
template <int EP, int NWV, int S, int TB>
__global__ __launch_bounds__(64 * NWV) void route_fused_kernel(const bf16_t *__restrict__ x,
                                                               const bf16_t *__restrict__ wg, int64_t T, int d,
                                                               int E, int k, float scale,
                                                               const float *__restrict__ lbias,
                                                               const float *__restrict__ sbias,
                                                               float *__restrict__ logits, int32_t *__restrict__ ids,
                                                               float *__restrict__ w) {
    constexpr int BK = 32;
    constexpr int LT = 64 * NWV / TB, QQ = ((EP / LT) + 3) / 4 * 4, TN = EP / 32;
    static_assert(EP == 64 || EP == 128, "one or two 64-expert column blocks");
    static_assert(TB == 16 || TB == 32, "one 32-row product, all or half of it used");
    static_assert(LT == 8 || LT == 16 || LT == 32, "lanes per token");
    using PA = DmaPlan<TB, BK, true, 1>;    // this wave's TB x-rows x 32 k
    using PB = DmaPlan<EP, BK, false, 1>;   // 32 k-rows of Wg x EP experts
    constexpr int kA = PA::kBytes, kStage = kA + PB::kBytes, kL = PA::kN + PB::kN;
    static_assert(kL * (S - 1) <= 63, "vmcnt range");
    constexpr int kRing = NWV * S * kStage, kPart = NWV * TB * EP * 4;
    constexpr int kLds = kRing > kPart ? kRing : kPart;
    static_assert(kLds <= 160 * 1024 - 64, "one block per compute unit");
    __shared__ __align__(1024) char smem[kLds];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * TB;
    const int rows = static_cast<int>(T - row0 < TB ? T - row0 : TB);
    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem)) + wave * S * kStage;
    PA pa;
    PB pb;
    pa.init(0, lane, d, 0, rows, d);   // rows past T and k past d load zeros
    pb.init(0, lane, E, 0, E, d);      // experts past E and k past d load zeros
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(x + row0 * d, static_cast<int64_t>(rows) * d * 2);
    const int nkb = (d + BK - 1) / BK;
    const int cnt = nkb > wave ? (nkb - wave + NWV - 1) / NWV : 0;  // this wave's k blocks
    // this wave's k block j into the slot at dst (j >= cnt: out-of-range loads
    // that write zeros to a slot nobody reads and keep the count uniform)
    auto issue = [&](int j, uint32_t dst) {
        const bool live = j < cnt;
        const int k0 = live ? (wave + j * NWV) * BK : 0;
        const int kc = live ? k0 : INT_MAX;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(wg + static_cast<int64_t>(k0) * E,
                                                    static_cast<int64_t>(d - k0) * E * 2);
#pragma unroll
        for (int i = 0; i < PA::kN; ++i) pa.issue(ra, kc, 2 * k0, dst, 0, i);
#pragma unroll
        for (int i = 0; i < PB::kN; ++i) pb.issue(rb, kc, 0, dst + kA, 0, i);
    };
    uint32_t fa[2], fb[TN];
#pragma unroll
    for (int h = 0; h < 2; ++h) fa[h] = FragAddr<32, BK, true>::kc(0, lane, 16 * h);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = FragAddr<EP, BK, false>::mn(32 * j, lane);
    f32x16_t acc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
#pragma unroll
    for (int st = 0; st < S - 1; ++st) issue(st, ring + st * kStage);
    for (int j = 0; j < cnt; ++j) {
        // the slot of block j - 1, whose fragments this wave has consumed
        issue(j + S - 1, ring + ((j + S - 1) % S) * kStage);
        wait_vmem<kL * (S - 1)>();  // block j has landed (a wave reads only its own slots)
        const uint32_t sa = ring + (j % S) * kStage;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8_t fA = lds_read_frag16(sa + fa[h]);
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) {
                const uint32_t a = sa + kA + fb[jj] + 16 * h * PB::kRowBytes;
                const s16x4_t lo = lds_read_tr(a), hi = lds_read_tr(a + 4 * PB::kRowBytes);
                const bf16x8_t fB = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fB, fA, acc[jj], 0, 0, 0);
            }
        }
    }
    wait_vmem<0>();   // no load may still target the ring
    __syncthreads();  // every wave is done with its ring: the partial tiles reuse the LDS
    // accumulator r of lane l: token l % 32, expert 32 jj + 8 (r / 4) + 4 (l / 32) + r % 4
    float *const part = reinterpret_cast<float *>(smem);
    if ((lane & 31) < TB) {
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4 *>(part + (wave * TB + (lane & 31)) * EP + 32 * jj + 8 * g + 4 * (lane >> 5)) =
                    make_float4(acc[jj][4 * g], acc[jj][4 * g + 1], acc[jj][4 * g + 2], acc[jj][4 * g + 3]);
    }
    __syncthreads();
    const int r = threadIdx.x % LT, tok = threadIdx.x / LT;
    const int64_t t = row0 + tok;
    const bool live = t < T;  // a token's LT lanes are all live or all not
    float s[QQ];
#pragma unroll
    for (int q = 0; q < QQ; ++q) {
        const int e = lane_expert<LT>(r, q);
        s[q] = -INFINITY;
        if (live && e < E) {
            float z = part[tok * EP + e];
#pragma unroll
            for (int v = 1; v < NWV; ++v) z += part[(v * TB + tok) * EP + e];
            z = __fmul_rn(z, scale);
            if (lbias) z = __fadd_rn(z, lbias[e]);
            s[q] = z;
        }
    }
    if (live) store_row<LT, QQ>(logits + t * E, s, r, E);
    topk_select<LT, QQ>(s, live, r, t, E, k, sbias, ids, w);
}

// dz = p * (g - c) * inv_tau per token (p = softmax of the logits, g the
// slots' weight gradients scattered to their experts, c = sum of p * g), with
// the top-k kernel's layout: LT lanes per token, lane r holding the 16-byte
// chunks r, r + LT, ... of the token's row.  The token's slots arrive LT at a
// time, one per lane, and are broadcast within the token's lanes.
template <int LT, int QQ, typename OutT>
__global__ __launch_bounds__(256) void route_dz_kernel(const float *__restrict__ logits,
                                                       const int32_t *__restrict__ ids,
                                                       const float *__restrict__ dw, int ldw, int64_t T, int E,
                                                       int k, float inv_tau, OutT *__restrict__ dz) {
    static_assert(LT == 8 || LT == 16 || LT == 32, "lanes per token");
    static_assert(QQ % 4 == 0, "whole 16-byte chunks");
    constexpr int TPW = 64 / LT;
    const int lane = threadIdx.x & 63;
    const int r = lane % LT, g0 = lane - r;  // lane r of the token's group starting at g0
    auto ex = [&](int q) { return 4 * (r + LT * (q >> 2)) + (q & 3); };
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6)) * TPW + lane / LT;
    const bool live = t < T;  // a token's lanes are all live or all not
    float p[QQ], g[QQ];
#pragma unroll
    for (int q = 0; q < QQ; ++q) {
        p[q] = -INFINITY;
        g[q] = 0.0f;
    }
    if (live) {
        if (E % 4 == 0) {
#pragma unroll
            for (int q = 0; q < QQ; q += 4)
                if (ex(q) < E) {
                    const float4 v = *reinterpret_cast<const float4 *>(logits + t * E + ex(q));
                    p[q] = v.x; p[q + 1] = v.y; p[q + 2] = v.z; p[q + 3] = v.w;
                }
        } else {
#pragma unroll
            for (int q = 0; q < QQ; ++q)
                if (ex(q) < E) p[q] = logits[t * E + ex(q)];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < QQ; ++q) mx = fmaxf(mx, p[q]);
#pragma unroll
    for (int off = LT / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float den = 0.0f;
#pragma unroll
    for (int q = 0; q < QQ; ++q) {
        p[q] = ex(q) < E && live ? expf(p[q] - mx) : 0.0f;
        den += p[q];
    }
#pragma unroll
    for (int off = LT / 2; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
    for (int jb = 0; jb < k; jb += LT) {
        const int nj = min(LT, k - jb);
        const int e_lane = live && r < nj ? ids[t * k + jb + r] : -1;
        const float g_lane = live && r < nj ? dw[t * ldw + jb + r] : 0.0f;
        for (int j = 0; j < nj; ++j) {
            const int ej = __shfl(e_lane, g0 + j, 64);
            const float gj = __shfl(g_lane, g0 + j, 64);
#pragma unroll
            for (int q = 0; q < QQ; ++q)
                if (ex(q) == ej) g[q] = gj;
        }
    }
    float c = 0.0f;
#pragma unroll
    for (int q = 0; q < QQ; ++q) {
        p[q] /= den;
        c += p[q] * g[q];
    }
#pragma unroll
    for (int off = LT / 2; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    if (!live) return;
#pragma unroll
    for (int q = 0; q < QQ; ++q)
        if (ex(q) < E) Elem<OutT>::store(dz, t * E + ex(q), p[q] * (g[q] - c) * inv_tau);
}

__global__ __launch_bounds__(256) void sum_partials_kernel(const float *__restrict__ part, int S, int64_t n,
                                                           float *__restrict__ out) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
        float acc = 0.0f;
        for (int s = 0; s < S; ++s) acc += part[s * n + i];
        out[i] = acc;
    }
}

// Column tile of the two skinny products with E columns (the logits x . Wg
// and Wg's gradient x^T . dz): one tile spans all E experts (up to 256), so x,
// by far the largest operand, is read once.  With 64-column tiles, E = 160
// read every row of x three times, in blocks that run on different XCDs.
inline int col_tile(int E) { return E <= 64 ? 64 : E <= 128 ? 128 : 256; }

// Lanes per token of the top-k and dz kernels: at most 32 experts a lane, and
// enough lanes that the launch gives each SIMD a few wavefronts (8 lanes from
// 32768 tokens on, 16 from 16384, else 32).
inline int lanes_per_token(int64_t T, int E) {
    const int lt_e = E <= 256 ? 8 : E <= 512 ? 16 : 32;
    const int lt_t = T >= 32768 ? 8 : T >= 16384 ? 16 : 32;
    return std::max(lt_e, lt_t);
}

// split count of the reduction over tokens for Wg's gradient: enough blocks to
// fill the chip, at least 1024 tokens per split
inline int rbwd_splits(int64_t T, int d, int E) {
    const int bn = col_tile(E);
    const int64_t tiles = ((d + 127) / 128) * ((E + bn - 1) / bn);
    int64_t S = (512 + tiles - 1) / tiles;
    const int64_t maxS = (T + 255) / 256;
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    if (S > 64) S = 64;
    return static_cast<int>(S);
}

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

}  // namespace

// bf16 logits: the d reduction is split into kparts ranges so that the skinny
// product (T x d times d x E) still gives each compute unit a block; the
// partial sums land in the workspace and the top-k kernel adds them in order.
// (Aiming at two blocks per compute unit doubles the partial sums written and
// read again: 4-10% slower at 128-256 experts with 32-deep k blocks, 14-25%
// slower with the 64-deep ones, which fit one block per compute unit.)
int route_kparts(int64_t T, int d, int E) {
    const int bn = col_tile(E);
    const int64_t tiles = ((T + 127) / 128) * ((E + bn - 1) / bn);
    int64_t kp = (256 + tiles - 1) / tiles;
    const int64_t maxkp = d / 256;  // each part at least 256 of d
    if (kp > maxkp) kp = maxkp;
    if (kp < 1) kp = 1;
    if (kp > 16) kp = 16;
    return static_cast<int>(kp);
}

// bf16 routing with up to 64 experts runs as the one fused kernel (with 128,
// the whole Wg that every 32-token block reads made it slower than the split
// product and the top-k kernel: 50 against 38 us at 16384 tokens, d = 2048)
static bool route_fused(int E, int dt) { return dt == kBF16 && E <= 64; }

size_t route_workspace(int64_t T, int d, int E, int dt) {
    if (dt != kBF16 || T <= 0 || route_fused(E, dt)) return 0;
    return static_cast<size_t>(route_kparts(T, d, E)) * static_cast<size_t>(T) * E * 4;
}

hipError_t launch_route(int dt, const void *x, const void *wg, int64_t T, int d, int E, int k, float inv_tau,
                        const float *logit_bias, const float *select_bias, int32_t *topk_ids, float *topk_w,
                        float *logits, void *ws, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (route_fused(E, dt)) {
        // 16 tokens a block: at 4096 tokens every compute unit gets one (13.6
        // against 14.3 us with 32 tokens a block, whose Wg reads are halved)
        constexpr int TB = 16;
        const dim3 grid(static_cast<unsigned>((T + TB - 1) / TB));
        hipLaunchKernelGGL((route_fused_kernel<64, 8, 3, TB>), grid, dim3(512), 0, s, static_cast<const bf16_t *>(x),
                           static_cast<const bf16_t *>(wg), T, d, E, k, inv_tau, logit_bias, select_bias, logits,
                           topk_ids, topk_w);
        return hipGetLastError();
    }
    GemmArgs p{};
    p.group_mode = GM_ROWS;
    p.offsets = nullptr;
    p.G = 1;
    p.extent = T;
    p.kchunk = static_cast<int>(T);
    p.N = E;
    p.K = d;
    p.nphase = 1;
    p.A0 = x;
    p.lda = d;
    p.B0 = wg;
    p.ldb = E;
    p.ldc = E;
    p.scale = inv_tau;
    p.col_bias = logit_bias;
    hipError_t err;
    float *part = nullptr;
    int kparts = 1;
    if (dt == kBF16) {
        kparts = route_kparts(T, d, E);
        part = static_cast<float *>(ws);
        p.C0 = part;
        p.kparts = kparts;
        p.kpart_len = ((d / kparts + 31) / 32) * 32;
        p.c_gstride = T * E;
        // 64-deep k blocks: each x row then brings whole 128-byte lines per
        // block (half lines with 32), one block per compute unit.  Alone, 32768
        // tokens of d = 4096 at 160 experts 115.6 -> 101.6 us (route with its
        // top-k), 8192 of d = 7168 at 256 experts 61.0 -> 58.5 us, 16384 of
        // d = 2048 at 128 experts 38.8 -> 37.5 us; bitwise the same logits
        switch (col_tile(E)) {
            case 128: err = launch_gemm_dma<128, 128, 64, 2, 2, 1, true, false, 3, EPI_STORE, float, 1>(p, s); break;
            // E <= 192: four waves side by side over the 256 columns, so the
            // wave whose 64 columns all lie past E skips its products
            default:
                err = E <= 192 ? launch_gemm_dma<128, 256, 64, 1, 4, 1, true, false, 3, EPI_STORE, float, 1>(p, s)
                               : launch_gemm_dma<128, 256, 64, 2, 2, 1, true, false, 3, EPI_STORE, float, 1>(p, s);
                break;
        }
    } else {
        p.C0 = logits;
        err = launch_gemm_f32<1, true, false, EPI_ROUTER>(p, s);
    }
    if (err != hipSuccess) return err;
    const int64_t ps = T * E;
    // a lane holds QQ, a multiple of 4, experts
    const int lt = lanes_per_token(T, E);
    const int qq = ((E + lt - 1) / lt + 3) / 4 * 4;
#define XMOE_TOPK(LT, QQ)                                                                                   \
    hipLaunchKernelGGL((topk_softmax_kernel<LT, QQ>),                                                       \
                       dim3(static_cast<unsigned>((T + kWaves * (64 / LT) - 1) / (kWaves * (64 / LT)))), dim3(256), \
                       0, s, logits, part, kparts, ps, inv_tau, logit_bias, select_bias, T, E, k, topk_ids, topk_w)
#define XMOE_TOPK_QQ(LT)                                                                                    \
    switch (qq) {                                                                                           \
        case 4: XMOE_TOPK(LT, 4); break;                                                                    \
        case 8: XMOE_TOPK(LT, 8); break;                                                                    \
        case 12: XMOE_TOPK(LT, 12); break;                                                                  \
        case 16: XMOE_TOPK(LT, 16); break;                                                                  \
        case 20: XMOE_TOPK(LT, 20); break;                                                                  \
        case 24: XMOE_TOPK(LT, 24); break;                                                                  \
        case 28: XMOE_TOPK(LT, 28); break;                                                                  \
        default: XMOE_TOPK(LT, 32); break;                                                                  \
    }
    if (lt == 8) {
        XMOE_TOPK_QQ(8)
    } else if (lt == 16) {
        XMOE_TOPK_QQ(16)
    } else {
        XMOE_TOPK_QQ(32)
    }
#undef XMOE_TOPK_QQ
#undef XMOE_TOPK
    return hipGetLastError();
}

size_t route_bwd_workspace(int64_t T, int d, int E, int dt) {
    const int S = rbwd_splits(T, d, E);
    const size_t dz = align256(static_cast<size_t>(T) * E * (dt == kBF16 ? 2 : 4));
    const size_t part = align256(static_cast<size_t>(S) * d * E * 4);
    return dz + part;
}

template <typename OutT>
static void launch_dz(int E, hipStream_t s, const float *logits, const int32_t *ids, const float *dw, int ldw,
                      int64_t T, int k, float inv_tau, OutT *dz) {
    const int lt = lanes_per_token(T, E);
    const int qq = ((E + lt - 1) / lt + 3) / 4 * 4;
#define XMOE_DZ(LT, QQ)                                                                                       \
    hipLaunchKernelGGL((route_dz_kernel<LT, QQ, OutT>),                                                       \
                       dim3(static_cast<unsigned>((T + kWaves * (64 / LT) - 1) / (kWaves * (64 / LT)))),      \
                       dim3(256), 0, s, logits, ids, dw, ldw, T, E, k, inv_tau, dz)
#define XMOE_DZ_QQ(LT)                                                                                        \
    switch (qq) {                                                                                             \
        case 4: XMOE_DZ(LT, 4); break;                                                                        \
        case 8: XMOE_DZ(LT, 8); break;                                                                        \
        case 12: XMOE_DZ(LT, 12); break;                                                                      \
        case 16: XMOE_DZ(LT, 16); break;                                                                      \
        case 20: XMOE_DZ(LT, 20); break;                                                                      \
        case 24: XMOE_DZ(LT, 24); break;                                                                      \
        case 28: XMOE_DZ(LT, 28); break;                                                                      \
        default: XMOE_DZ(LT, 32); break;                                                                      \
    }
    if (lt == 8) {
        XMOE_DZ_QQ(8)
    } else if (lt == 16) {
        XMOE_DZ_QQ(16)
    } else {
        XMOE_DZ_QQ(32)
    }
#undef XMOE_DZ_QQ
#undef XMOE_DZ
}

hipError_t launch_route_bwd(int dt, const void *x, const void *wg, const float *logits, const int32_t *topk_ids,
                            const float *dtopk_w, int ldw, int64_t T, int d, int E, int k, float inv_tau,
                            bool accumulate, void *dx, float *dwg, void *ws, hipStream_t s) {
    const int S = rbwd_splits(T, d, E);
    const size_t dz_bytes = align256(static_cast<size_t>(T) * E * (dt == kBF16 ? 2 : 4));
    void *dz = ws;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + dz_bytes);
    hipError_t err;
    if (T > 0) {
        if (dt == kBF16)
            launch_dz<bf16_t>(E, s, logits, topk_ids, dtopk_w, ldw, T, k, inv_tau, static_cast<bf16_t *>(dz));
        else
            launch_dz<float>(E, s, logits, topk_ids, dtopk_w, ldw, T, k, inv_tau, static_cast<float *>(dz));
        if ((err = hipGetLastError()) != hipSuccess) return err;

        // dx[t] += dz[t] . Wg^T (or dx[t] = ... without accumulate) : A = dz [T,E]
        // (k-contiguous), B(k=e, n=i) = Wg[i*E + e]
        GemmArgs a{};
        a.group_mode = GM_ROWS;
        a.G = 1;
        a.extent = T;
        a.kchunk = static_cast<int>(T);
        a.N = d;
        a.K = E;
        a.nphase = 1;
        a.A0 = dz;
        a.lda = E;
        a.B0 = wg;
        a.ldb = E;
        a.C0 = dx;
        a.ldc = d;
        // bf16 (E is a multiple of 8): the pipelined kernel, whose epilogue brings
        // the dx tile into LDS by DMA, adds and writes it back in row chunks
        if (accumulate)
            err = dt != kBF16 ? launch_gemm_f32<1, true, true, EPI_ACCUM>(a, s)
                              : launch_gemm_dma<128, 256, 32, 2, 2, 1, true, true, 3, EPI_ACCUM, bf16_t, 2>(a, s);
        else
            err = dt != kBF16 ? launch_gemm_f32<1, true, true, EPI_STORE>(a, s)
                              : launch_gemm_dma<128, 256, 32, 2, 2, 1, true, true, 3, EPI_STORE, bf16_t, 2>(a, s);
        if (err != hipSuccess) return err;
    }
    // partial[s] = x[chunk s]^T . dz[chunk s] : A(m=i, k=t) = x[t*d + i], B(k=t, n=e) = dz[t*E + e]
    GemmArgs b{};
    b.group_mode = GM_KSPLIT;
    b.offsets = nullptr;
    b.G = S;
    b.extent = T;
    b.kchunk = static_cast<int>((T + S - 1) / S);
    b.M = d;
    b.N = E;
    b.nphase = 1;
    b.A0 = x;
    b.lda = d;
    b.B0 = dz;
    b.ldb = E;
    b.C0 = part;
    b.ldc = E;
    b.c_gstride = static_cast<int64_t>(d) * E;
    if (dt != kBF16)
        err = launch_gemm_f32<1, false, false, EPI_STORE>(b, s);
    else
        switch (col_tile(E)) {
            case 64: err = launch_gemm_dma<128, 64, 32, 2, 2, 1, false, false, 3, EPI_STORE, float, 2>(b, s); break;
            case 128: err = launch_gemm_dma<128, 128, 32, 2, 2, 1, false, false, 3, EPI_STORE, float, 2>(b, s); break;
            default:
                err = E <= 192 ? launch_gemm_dma<128, 256, 32, 1, 4, 1, false, false, 3, EPI_STORE, float, 2>(b, s)
                               : launch_gemm_dma<128, 256, 32, 2, 2, 1, false, false, 3, EPI_STORE, float, 2>(b, s);
                break;
        }
    if (err != hipSuccess) return err;
    const int64_t n = static_cast<int64_t>(d) * E;
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 4096));
    hipLaunchKernelGGL(sum_partials_kernel, dim3(blocks), dim3(256), 0, s, part, S, n, dwg);
    return hipGetLastError();
}

}  // namespace xmoe

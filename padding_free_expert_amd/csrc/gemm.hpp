// Grouped GEMM for the padding-free expert FFN, the router and their gradients.
//
// One problem descriptor covers every product the layer needs:
//   GM_ROWS   - the rows of C are cut into groups by device-side offsets
//               (one group per expert, as the X-MoE article's per-expert GEMM in
//               section 2.1.2, "跨平台核函数优化", multiplies each expert's own rows
//               without padding).  Group g owns rows [off[g], off[g+1]) of A and C
//               and its own B (B + g*b_gstride).  Used by the expert forward, the
//               expert data-gradient, and the dense router products (G = 1).
//   GM_KSPLIT - the reduction dimension is cut into groups (offsets, or uniform
//               chunks of kchunk when offsets == nullptr); group g writes its own
//               C (C + g*c_gstride).  Used by the expert weight gradients (K = the
//               expert's rows, zero rows -> zero gradient) and the split-T router
//               weight gradient.
// Tiles are scheduled on the device from the offsets: the grid is sized on the
// host from an upper bound and blocks without a tile exit at once.  Nothing is
// read back to the host and no row is padded.
//
// Operand layouts (template flags):  A(m,k) = A[m*lda + k] (A_KC) or A[k*lda + m];
// B(k,n) = B[n*ldb + k] (B_KC) or B[k*ldb + n].  Shared-memory tiles are always
// stored k-contiguous so that every matrix-core operand is one 16-byte LDS read;
// operands that arrive MN-contiguous are transposed in registers on the way in.
#pragma once

#include "common.hpp"

namespace xmoe {

enum { GM_ROWS = 0, GM_KSPLIT = 1 };
enum { EPI_STORE = 0, EPI_ACCUM = 1, EPI_SWIGLU = 2, EPI_SWIGLU_BWD = 3, EPI_ROUTER = 4 };

struct GemmArgs {
    int group_mode;
    const int32_t *offsets;  // [G+1] device (may be nullptr for uniform GM_KSPLIT)
    int G;
    int64_t extent;          // GM_ROWS: total rows; GM_KSPLIT: total reduction length
    int M, N, K;             // GM_ROWS uses N, K; GM_KSPLIT uses M, N
    int kchunk;              // uniform GM_KSPLIT chunk
    int nphase;              // 2: C = A0.B0 + A1.B1 (GM_ROWS only)
    const void *A0, *A1;
    const void *B0, *B1, *Bx;  // Bx: second B sharing A (two outputs)
    int64_t lda, ldb, b_gstride;
    void *C0, *Cx;
    int64_t ldc, c_gstride;
    const void *aux;         // EPI_SWIGLU_BWD: saved [H1|H3]
    void *aux_out;           // EPI_SWIGLU: [H1|H3] to save (optional)
    int64_t ld_aux;
    int hoff;                // column offset of the H3 half in [H1|H3]
    float scale;             // EPI_ROUTER
    const float *col_bias;   // EPI_ROUTER (optional)
};

// ---------------------------------------------------------------- epilogues

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

template <int EPI, typename OutT>
__device__ __forceinline__ void epilogue(const GemmArgs &p, int64_t cbase_row, int64_t cbase_off, int m,
                                         int n, float v0, float v1) {
    // cbase_row: first C row of the group (GM_ROWS) ; cbase_off: group offset (GM_KSPLIT)
    const int64_t row = cbase_row + m;
    if constexpr (EPI == EPI_STORE) {
        Elem<OutT>::store(static_cast<OutT *>(p.C0), cbase_off + row * p.ldc + n, v0);
        if (p.Cx) Elem<OutT>::store(static_cast<OutT *>(p.Cx), cbase_off + row * p.ldc + n, v1);
    } else if constexpr (EPI == EPI_ACCUM) {
        OutT *c = static_cast<OutT *>(p.C0);
        const int64_t i = cbase_off + row * p.ldc + n;
        Elem<OutT>::store(c, i, Elem<OutT>::load(c, i) + v0);
    } else if constexpr (EPI == EPI_SWIGLU) {
        // v0 = H1, v1 = H3 at the same (row, n)
        Elem<OutT>::store(static_cast<OutT *>(p.C0), row * p.ldc + n, silu_f(v0) * v1);
        if (p.aux_out) {
            OutT *s = static_cast<OutT *>(p.aux_out);
            Elem<OutT>::store(s, row * p.ld_aux + n, v0);
            Elem<OutT>::store(s, row * p.ld_aux + p.hoff + n, v1);
        }
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        const OutT *s = static_cast<const OutT *>(p.aux);
        const float h1 = Elem<OutT>::load(s, row * p.ld_aux + n);
        const float h3 = Elem<OutT>::load(s, row * p.ld_aux + p.hoff + n);
        const float sg = 1.0f / (1.0f + __expf(-h1));
        OutT *o = static_cast<OutT *>(p.C0);
        Elem<OutT>::store(o, row * p.ldc + n, v0 * h3 * sg * (1.0f + h1 * (1.0f - sg)));
        Elem<OutT>::store(o, row * p.ldc + p.hoff + n, v0 * h1 * sg);
    } else {  // EPI_ROUTER: s = z * scale (+ bias[n]), each an IEEE fp32 operation
        float s = __fmul_rn(v0, p.scale);
        if (p.col_bias) s = __fadd_rn(s, p.col_bias[n]);
        static_cast<float *>(p.C0)[row * p.ldc + n] = s;
    }
}

// ------------------------------------------------------------ tile scheduler

struct Tile {
    int g;          // group
    int mt, nt;     // tile coordinates inside the group
    int64_t base;   // GM_ROWS: first row of the group; GM_KSPLIT: first k of the group
    int Mg, Kg;     // extents of the group
};

__device__ __forceinline__ void seg_bounds(const GemmArgs &p, int g, int64_t *lo, int64_t *hi) {
    int64_t a, b;
    if (p.offsets) {
        a = p.offsets[g];
        b = p.offsets[g + 1];
    } else {
        a = static_cast<int64_t>(g) * p.kchunk;
        b = a + p.kchunk;
    }
    a = a < 0 ? 0 : (a > p.extent ? p.extent : a);
    b = b < a ? a : (b > p.extent ? p.extent : b);
    *lo = a;
    *hi = b;
}

// Resolve this block's tile.  Returns false when the block has no tile.
// GM_ROWS: block -> (global m-tile, n-tile); the global m-tile is located among
// the groups by a prefix sum of per-group tile counts computed by wave 0.
template <int BM, int BN>
__device__ bool resolve_tile(const GemmArgs &p, Tile *t) {
    const int tiles_n = (p.N + BN - 1) / BN;
    if (p.group_mode == GM_KSPLIT) {
        const int tiles_m = (p.M + BM - 1) / BM;
        const int per_g = tiles_m * tiles_n;
        const int g = blockIdx.x / per_g;
        if (g >= p.G) return false;
        const int rem = blockIdx.x - g * per_g;
        int64_t lo, hi;
        seg_bounds(p, g, &lo, &hi);
        t->g = g;
        t->mt = rem / tiles_n;
        t->nt = rem - t->mt * tiles_n;
        t->base = lo;
        t->Mg = p.M;
        t->Kg = static_cast<int>(hi - lo);
        return true;
    }
    __shared__ int s_res[2];
    const int mt_global = blockIdx.x / tiles_n;
    const int lane = threadIdx.x;
    if (threadIdx.x == 0) s_res[0] = -1;
    __syncthreads();
    if (threadIdx.x < 64) {
        const int per = (p.G + 63) / 64;
        const int g0 = min(lane * per, p.G), g1 = min(g0 + per, p.G);
        int cnt = 0;
        for (int g = g0; g < g1; ++g) {
            int64_t lo, hi;
            seg_bounds(p, g, &lo, &hi);
            cnt += static_cast<int>((hi - lo + BM - 1) / BM);
        }
        int inc = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(inc, off, 64);
            if (lane >= off) inc += v;
        }
        const int exc = inc - cnt;
        if (mt_global >= exc && mt_global < inc) {
            int b = exc;
            for (int g = g0; g < g1; ++g) {
                int64_t lo, hi;
                seg_bounds(p, g, &lo, &hi);
                const int n = static_cast<int>((hi - lo + BM - 1) / BM);
                if (mt_global < b + n) {
                    s_res[0] = g;
                    s_res[1] = mt_global - b;
                    break;
                }
                b += n;
            }
        }
    }
    __syncthreads();
    const int g = s_res[0];
    if (g < 0) return false;
    int64_t lo, hi;
    seg_bounds(p, g, &lo, &hi);
    t->g = g;
    t->mt = s_res[1];
    t->nt = blockIdx.x - mt_global * tiles_n;
    t->base = lo;
    t->Mg = static_cast<int>(hi - lo);
    t->Kg = p.K;
    return true;
}

template <int BM, int BN>
inline int64_t gemm_grid(const GemmArgs &p) {
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    if (p.group_mode == GM_KSPLIT) return static_cast<int64_t>(p.G) * ((p.M + BM - 1) / BM) * tiles_n;
    return ((p.extent + BM - 1) / BM + p.G) * tiles_n;
}

// Per-group operand base pointers (element offsets).
template <typename T>
struct GroupPtrs {
    const T *A0, *A1;  // k phase 0 / 1
    const T *B0, *B1;
    const T *Bx;
    int64_t crow;   // first C row (GM_ROWS)
    int64_t coff;   // C element offset of the group (GM_KSPLIT)
};

template <typename T>
__device__ __forceinline__ GroupPtrs<T> group_ptrs(const GemmArgs &p, const Tile &t) {
    GroupPtrs<T> q;
    if (p.group_mode == GM_ROWS) {
        q.A0 = static_cast<const T *>(p.A0) + t.base * p.lda;
        q.A1 = p.A1 ? static_cast<const T *>(p.A1) + t.base * p.lda : nullptr;
        q.B0 = static_cast<const T *>(p.B0) + static_cast<int64_t>(t.g) * p.b_gstride;
        q.B1 = p.B1 ? static_cast<const T *>(p.B1) + static_cast<int64_t>(t.g) * p.b_gstride : nullptr;
        q.Bx = p.Bx ? static_cast<const T *>(p.Bx) + static_cast<int64_t>(t.g) * p.b_gstride : nullptr;
        q.crow = t.base;
        q.coff = 0;
    } else {
        q.A0 = static_cast<const T *>(p.A0) + t.base * p.lda;
        q.A1 = nullptr;
        q.B0 = static_cast<const T *>(p.B0) + t.base * p.ldb;
        q.B1 = nullptr;
        q.Bx = p.Bx ? static_cast<const T *>(p.Bx) + t.base * p.ldb : nullptr;
        q.crow = 0;
        q.coff = static_cast<int64_t>(t.g) * p.c_gstride;
    }
    return q;
}

// ------------------------------------------------------ bf16 matrix-core path

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 8x8 transpose of 16-bit elements held as 8 rows of 16 bytes: out[j] gets
// element j of every input row (input row i -> 16-bit lane i of out[j]).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i][0] = in[i].x; w[i][1] = in[i].y; w[i][2] = in[i].z; w[i][3] = in[i].w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(w[2 * q + 1][j >> 1], w[2 * q][j >> 1], sel);
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Global -> register staging of one operand tile of R (m or n) x BK (k) elements,
// and register -> LDS store in the k-contiguous [R][BK+8] layout.
template <int R, int BK, bool KC>
struct TileLoader;

// K-contiguous operand: element (r, k) at base[r*ld + k]
template <int R, int BK>
struct TileLoader<R, BK, true> {
    static constexpr int kChunks = R * BK / 8;
    static constexpr int kIter = (kChunks + 255) / 256;
    uint4 v[kIter];
    __device__ __forceinline__ void load(const bf16_t *base, int64_t ld, int r0, int rmax, int k0, int kmax) {
#pragma unroll
        for (int i = 0; i < kIter; ++i) {
            const int c = threadIdx.x + 256 * i;
            const int r = c / (BK / 8), kc = c % (BK / 8);
            const int gr = r0 + r, gk = k0 + kc * 8;
            v[i] = make_uint4(0, 0, 0, 0);
            if ((kChunks % 256 == 0 || c < kChunks) && gr < rmax && gk < kmax)
                v[i] = *reinterpret_cast<const uint4 *>(base + static_cast<int64_t>(gr) * ld + gk);
        }
    }
    __device__ __forceinline__ void store(bf16_t *lds) const {
#pragma unroll
        for (int i = 0; i < kIter; ++i) {
            const int c = threadIdx.x + 256 * i;
            if (kChunks % 256 == 0 || c < kChunks) {
                const int r = c / (BK / 8), kc = c % (BK / 8);
                *reinterpret_cast<uint4 *>(lds + r * (BK + 8) + kc * 8) = v[i];
            }
        }
    }
};

// MN-contiguous operand: element (r, k) at base[k*ld + r]; moved as 8x8 blocks.
template <int R, int BK>
struct TileLoader<R, BK, false> {
    static constexpr int kBlocks = (R / 8) * (BK / 8);
    static constexpr int kIter = (kBlocks + 255) / 256;
    uint4 v[kIter][8];
    __device__ __forceinline__ void load(const bf16_t *base, int64_t ld, int r0, int rmax, int k0, int kmax) {
#pragma unroll
        for (int i = 0; i < kIter; ++i) {
            const int b = threadIdx.x + 256 * i;
            const int rb = b % (R / 8), kb = b / (R / 8);
            const int gr = r0 + rb * 8;
            const bool ok = (kBlocks % 256 == 0 || b < kBlocks) && gr < rmax;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int gk = k0 + kb * 8 + q;
                v[i][q] = make_uint4(0, 0, 0, 0);
                if (ok && gk < kmax) v[i][q] = *reinterpret_cast<const uint4 *>(base + static_cast<int64_t>(gk) * ld + gr);
            }
        }
    }
    __device__ __forceinline__ void store(bf16_t *lds) const {
#pragma unroll
        for (int i = 0; i < kIter; ++i) {
            const int b = threadIdx.x + 256 * i;
            if (kBlocks % 256 == 0 || b < kBlocks) {
                const int rb = b % (R / 8), kb = b / (R / 8);
                uint4 t[8];
                transpose8x8(v[i], t);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<uint4 *>(lds + (rb * 8 + j) * (BK + 8) + kb * 8) = t[j];
            }
        }
    }
};

// BM x BN tile per 256-thread block (4 waves as WGM x WGN), BK-deep k steps,
// double-buffered LDS, v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
// NB = 2 multiplies the same A tile by two B matrices (the up-projection's W1
// and W3, or the weight gradient's dH1 and dH3).
template <int BM, int BN, int BK, int WGM, int WGN, int NB, bool A_KC, bool B_KC, int EPI, typename OutT>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs p) {
    static_assert(WGM * WGN == 4, "four waves per block");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tile must be a multiple of 32");
    constexpr int LDK = BK + 8;
    __shared__ __align__(16) bf16_t As[2][BM * LDK];
    __shared__ __align__(16) bf16_t Bs[2][NB][BN * LDK];

    Tile t;
    if (!resolve_tile<BM, BN>(p, &t)) return;
    const GroupPtrs<bf16_t> q = group_ptrs<bf16_t>(p, t);
    const int m0 = t.mt * BM, n0 = t.nt * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    f32x16_t acc[NB][TM][TN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.0f;

    const int ktiles = (t.Kg + BK - 1) / BK;
    const int nph = (p.group_mode == GM_ROWS) ? p.nphase : 1;
    const int total = ktiles * nph;

    TileLoader<BM, BK, A_KC> la;
    TileLoader<BN, BK, B_KC> lb[NB];

    auto load_stage = [&](int it) {
        const int ph = it >= ktiles ? 1 : 0;
        const int k0 = (it - ph * ktiles) * BK;
        la.load(ph ? q.A1 : q.A0, p.lda, m0, t.Mg, k0, t.Kg);
        lb[0].load(ph ? q.B1 : q.B0, p.ldb, n0, p.N, k0, t.Kg);
        if constexpr (NB == 2) lb[1].load(q.Bx, p.ldb, n0, p.N, k0, t.Kg);
    };
    auto store_stage = [&](int buf) {
        la.store(As[buf]);
        lb[0].store(Bs[buf][0]);
        if constexpr (NB == 2) lb[1].store(Bs[buf][1]);
    };

    if (total > 0) {
        load_stage(0);
        store_stage(0);
        __syncthreads();
    }
    for (int it = 0; it < total; ++it) {
        const int buf = it & 1;
        if (it + 1 < total) load_stage(it + 1);
        const bf16_t *as = As[buf] + (wm * WTM + (lane & 31)) * LDK + (lane >> 5) * 8;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8_t af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8_t *>(as + i * 32 * LDK + kk);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const bf16_t *bs = Bs[buf][b] + (wn * WTN + (lane & 31)) * LDK + (lane >> 5) * 8;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const bf16x8_t bf = *reinterpret_cast<const bf16x8_t *>(bs + j * 32 * LDK + kk);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf, acc[b][i][j], 0, 0, 0);
                }
            }
        }
        if (it + 1 < total) store_stage(buf ^ 1);
        __syncthreads();
    }

    // accumulator (i, j, r): row = 8*(r/4) + 4*(lane/32) + r%4, col = lane%32 of the 32x32 block
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int n = n0 + wn * WTN + j * 32 + (lane & 31);
                if (m < t.Mg && n < p.N)
                    epilogue<EPI, OutT>(p, q.crow, q.coff, m, n, acc[0][i][j][r],
                                        NB == 2 ? acc[NB - 1][i][j][r] : 0.0f);
            }
}

template <int BM, int BN, int BK, int WGM, int WGN, int NB, bool A_KC, bool B_KC, int EPI, typename OutT>
inline hipError_t launch_gemm_mfma(const GemmArgs &p, hipStream_t stream) {
    const int64_t grid = gemm_grid<BM, BN>(p);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, WGM, WGN, NB, A_KC, B_KC, EPI, OutT>), dim3(static_cast<unsigned>(grid)),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ------------------------------------------------------------- fp32 path
//
// Plain FMA tiles (64x64 per block, 4x4 per thread).  Every output is summed
// in ascending k with one fused multiply-add per term, so the fp32 router's
// logits follow exactly that order.

template <int NB, bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM];
    __shared__ float Bs[NB][BK][BN];
    Tile t;
    if (!resolve_tile<BM, BN>(p, &t)) return;
    const GroupPtrs<float> q = group_ptrs<float>(p, t);
    const int m0 = t.mt * BM, n0 = t.nt * BN;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    float acc[NB][4][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.0f;
    const int nph = (p.group_mode == GM_ROWS) ? p.nphase : 1;
    for (int ph = 0; ph < nph; ++ph) {
        const float *A = ph ? q.A1 : q.A0;
        const float *B0 = ph ? q.B1 : q.B0;
        for (int k0 = 0; k0 < t.Kg; k0 += BK) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = threadIdx.x + 256 * i;  // 0..1023 over the 16x64 tile
                const int kk = e / BM, mm = e % BM;
                const int gm = m0 + mm, gk = k0 + kk;
                float va = 0.0f;
                if (gm < t.Mg && gk < t.Kg)
                    va = A_KC ? A[static_cast<int64_t>(gm) * p.lda + gk] : A[static_cast<int64_t>(gk) * p.lda + gm];
                As[kk][mm] = va;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int gn = n0 + mm;
                    float vb = 0.0f;
                    const float *Bm = b ? q.Bx : B0;
                    if (gn < p.N && gk < t.Kg)
                        vb = B_KC ? Bm[static_cast<int64_t>(gn) * p.ldb + gk] : Bm[static_cast<int64_t>(gk) * p.ldb + gn];
                    Bs[b][kk][mm] = vb;
                }
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < BK; ++kk) {
                float a[4], bv[NB][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[b][j] = Bs[b][kk][tx * 4 + j];
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[b][i][j] = __builtin_fmaf(a[i], bv[b][j], acc[b][i][j]);
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < t.Mg && n < p.N)
                epilogue<EPI, float>(p, q.crow, q.coff, m, n, acc[0][i][j], acc[NB - 1][i][j]);
        }
}

template <int NB, bool A_KC, bool B_KC, int EPI>
inline hipError_t launch_gemm_f32(const GemmArgs &p, hipStream_t stream) {
    const int64_t grid = gemm_grid<64, 64>(p);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_f32_kernel<NB, A_KC, B_KC, EPI>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace xmoe

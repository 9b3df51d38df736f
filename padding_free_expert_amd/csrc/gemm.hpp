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

#include <climits>
#include <type_traits>

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
    // EPI_SWIGLU_BWD (optional): dA of rows-space row r is multiplied by
    // row_scale[r] before the SwiGLU backward (the combine weight of a row
    // whose A operand is the unweighted upstream gradient)
    const float *row_scale;
    void *aux_out;           // EPI_SWIGLU: [H1|H3] to save (optional)
    int64_t ld_aux;
    int hoff;                // column offset of the H3 half in [H1|H3]
    float scale;             // EPI_ROUTER
    const float *col_bias;   // EPI_ROUTER (optional)
    // GM_ROWS with a k-contiguous A (bf16 pipelined and fp32 kernels only):
    // when a_map is set, row r of the rows-space reads A0 row a_map[r] (A0 has
    // a_map_rows rows), i.e. the dispatch gather happens in the operand loads.
    // GM_KSPLIT with an mn-contiguous A (fp32 kernel, or the pipelined kernel's
    // KMAP variant): k row r reads A0 row a_map[r] the same way.
    const int32_t *a_map;
    int64_t a_map_rows;
    // GM_ROWS split over k (pipelined kernel only): block b works on k range
    // part b % kparts of length kpart_len and writes C + part * c_gstride
    // (partial sums, EPI_STORE); kparts <= 1 means no split.
    int kparts;
    int kpart_len;
    // fp32 outputs with EPI_STORE: nonzero adds the products to C (C0 and Cx)
    // instead of overwriting it (one fp32 addition per element)
    int accum;
    // tiles per XCD run of the block -> tile map: 0 = kXcdRun; -1 = GM_KSPLIT:
    // half of one group's tiles, so that two XCDs share a group's operands
    // (GM_ROWS: the mean group's tiles)
    int xcd_run;
};

// ---------------------------------------------------------------- epilogues

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

template <int EPI, typename OutT>
__device__ __forceinline__ void epilogue(const GemmArgs &p, int64_t cbase_row, int64_t cbase_off, int m,
                                         int n, float v0, float v1) {
    // cbase_row: first C row of the group (GM_ROWS) ; cbase_off: group offset (GM_KSPLIT)
    const int64_t row = cbase_row + m;
    if constexpr (EPI == EPI_STORE) {
        const int64_t i = cbase_off + row * p.ldc + n;
        if (std::is_same<OutT, float>::value && p.accum) {
            OutT *c0 = static_cast<OutT *>(p.C0);
            Elem<OutT>::store(c0, i, Elem<OutT>::load(c0, i) + v0);
            if (p.Cx) {
                OutT *cx = static_cast<OutT *>(p.Cx);
                Elem<OutT>::store(cx, i, Elem<OutT>::load(cx, i) + v1);
            }
        } else {
            Elem<OutT>::store(static_cast<OutT *>(p.C0), i, v0);
            if (p.Cx) Elem<OutT>::store(static_cast<OutT *>(p.Cx), i, v1);
        }
    } else if constexpr (EPI == EPI_ACCUM) {
        OutT *c = static_cast<OutT *>(p.C0);
        const int64_t i = cbase_off + row * p.ldc + n;
        Elem<OutT>::store(c, i, Elem<OutT>::load(c, i) + v0);
    } else if constexpr (EPI == EPI_SWIGLU) {
        // v0 = H1, v1 = H3 at the same (row, n)
        if (p.C0) Elem<OutT>::store(static_cast<OutT *>(p.C0), row * p.ldc + n, silu_f(v0) * v1);
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
        const float da = p.row_scale ? v0 * p.row_scale[row] : v0;
        OutT *o = static_cast<OutT *>(p.C0);
        Elem<OutT>::store(o, row * p.ldc + n, da * h3 * sg * (1.0f + h1 * (1.0f - sg)));
        Elem<OutT>::store(o, row * p.ldc + p.hoff + n, da * h1 * sg);
    } else {  // EPI_ROUTER: s = z * scale (+ bias[n]), each an IEEE fp32 operation
        float s = __fmul_rn(v0, p.scale);
        if (p.col_bias) s = __fadd_rn(s, p.col_bias[n]);
        static_cast<float *>(p.C0)[row * p.ldc + n] = s;
    }
}

// ------------------------------------------------------------ tile scheduler

struct Tile {
    int g;          // group
    int m0, nt;     // first row of the tile inside the group; column tile
    int64_t base;   // GM_ROWS: first row of the group; GM_KSPLIT: first k of the group
    int Mg, Kg;     // row extent of the group and K extent
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

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2.  Tiles that share operands are numbered
// consecutively (a group's tiles together; within a GM_ROWS group the m-tiles
// of one n-tile, which read the same weight slice at the same k, are adjacent),
// and the block -> tile map gives every XCD runs of kXcdRun consecutive tiles:
// the tiles that run at the same time on one XCD then share their operands
// through that XCD's L2 instead of each XCD fetching them from HBM.  The map
// is a bijection on [0, nblocks).
constexpr int kXcds = 8;
constexpr int kXcdRun = 32;

__device__ __forceinline__ int xcd_tile_order(int b, int nblocks, int run = kXcdRun) {
    const int W = kXcds * run;
    const int full = nblocks / W * W;
    if (b >= full) return b;
    const int xcd = b % kXcds, local = b / kXcds;
    return (local / run) * W + xcd * run + local % run;
}

// the run length of a launch (see GemmArgs::xcd_run)
template <int BM, int BN>
__device__ __forceinline__ int xcd_run_of(const GemmArgs &p) {
    if (p.xcd_run > 0) return p.xcd_run;
    if (p.xcd_run == 0) return kXcdRun;
    const int tiles_n = (p.N + BN - 1) / BN;
    if (p.group_mode == GM_KSPLIT) return (((p.M + BM - 1) / BM) * tiles_n + 1) / 2;
    const int64_t per = (p.extent + static_cast<int64_t>(BM) * p.G - 1) / (static_cast<int64_t>(BM) * p.G);
    return static_cast<int>(per > 0 ? per : 1) * tiles_n;
}

// Resolve this block's tile.  Returns false when the block has no tile.
// GM_ROWS: the group is located by a prefix sum of per-group m-tile counts
// computed by wave 0 (group g owns tiles [exc*tiles_n, inc*tiles_n)).
template <int BM, int BN>
__device__ bool resolve_tile(const GemmArgs &p, Tile *t, int block, int nblocks) {
    const int tiles_n = (p.N + BN - 1) / BN;
    if (p.group_mode == GM_KSPLIT) {
        const int tiles_m = (p.M + BM - 1) / BM;
        const int per_g = tiles_m * tiles_n;
        const int bid = xcd_tile_order(block, nblocks, xcd_run_of<BM, BN>(p));
        const int g = bid / per_g;
        if (g >= p.G) return false;
        const int rem = bid - g * per_g;
        int64_t lo, hi;
        seg_bounds(p, g, &lo, &hi);
        const int mt = rem / tiles_n;
        t->g = g;
        t->m0 = mt * BM;
        t->nt = rem - mt * tiles_n;
        t->base = lo;
        t->Mg = p.M;
        t->Kg = static_cast<int>(hi - lo);
        return true;
    }
    __shared__ int s_res[3];
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
        const int bid = xcd_tile_order(block, nblocks, xcd_run_of<BM, BN>(p));
        const int mt_global = bid / tiles_n;   // past the last group's tiles: no tile
        if (mt_global >= exc && mt_global < inc) {
            int b = exc;
            for (int g = g0; g < g1; ++g) {
                int64_t lo, hi;
                seg_bounds(p, g, &lo, &hi);
                const int n = static_cast<int>((hi - lo + BM - 1) / BM);
                if (mt_global < b + n) {
                    // the group's tiles are bid in [b*tiles_n, (b+n)*tiles_n), m-tile fastest
                    const int local = bid - b * tiles_n;
                    s_res[0] = g;
                    s_res[1] = local % n;
                    s_res[2] = local / n;
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
    const int mt = s_res[1];
    t->g = g;
    t->nt = s_res[2];
    t->base = lo;
    t->Kg = p.K;
    t->m0 = mt * BM;
    t->Mg = static_cast<int>(hi - lo);
    return true;
}

template <int BM, int BN>
inline int64_t gemm_grid(const GemmArgs &p) {
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    if (p.group_mode == GM_KSPLIT) return static_cast<int64_t>(p.G) * ((p.M + BM - 1) / BM) * tiles_n;
    return ((p.extent + BM - 1) / BM + p.G) * tiles_n * (p.kparts > 1 ? p.kparts : 1);
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

// ------------------------------------------------------- bf16 helpers

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
// The operands' tile edges (rows past a group's end, k past K) are expressed
// as an out-of-range offset, so loads need no branches.
constexpr int kOob = 0x7ffffff0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint32_t n = bytes >= 0x7ffffff0 ? 0x7ffffff0u : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(n), 0x00020000);
}

// Epilogue on 4 consecutive output columns n..n+3 of row m (all in range).
template <int EPI, typename OutT>
__device__ __forceinline__ void epilogue4(const GemmArgs &p, int64_t crow, int64_t coff, int m, int n,
                                          const float (&v0)[4], const float (&v1)[4]) {
    const int64_t row = crow + m;
    if constexpr (EPI == EPI_ROUTER) {
        float4 o;
        float *po = &o.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s = __fmul_rn(v0[i], p.scale);
            if (p.col_bias) s = __fadd_rn(s, p.col_bias[n + i]);
            po[i] = s;
        }
        *reinterpret_cast<float4 *>(static_cast<float *>(p.C0) + row * p.ldc + n) = o;
    } else if constexpr (std::is_same<OutT, float>::value) {
        float *c = static_cast<float *>(p.C0) + coff + row * p.ldc + n;
        if constexpr (EPI == EPI_ACCUM) {
            float4 o = *reinterpret_cast<float4 *>(c);
            o.x += v0[0]; o.y += v0[1]; o.z += v0[2]; o.w += v0[3];
            *reinterpret_cast<float4 *>(c) = o;
        } else if (p.accum) {
            float4 o = *reinterpret_cast<float4 *>(c);
            o.x += v0[0]; o.y += v0[1]; o.z += v0[2]; o.w += v0[3];
            *reinterpret_cast<float4 *>(c) = o;
            if (p.Cx) {
                float4 *cx = reinterpret_cast<float4 *>(static_cast<float *>(p.Cx) + coff + row * p.ldc + n);
                float4 u = *cx;
                u.x += v1[0]; u.y += v1[1]; u.z += v1[2]; u.w += v1[3];
                *cx = u;
            }
        } else {
            *reinterpret_cast<float4 *>(c) = make_float4(v0[0], v0[1], v0[2], v0[3]);
            if (p.Cx)
                *reinterpret_cast<float4 *>(static_cast<float *>(p.Cx) + coff + row * p.ldc + n) =
                    make_float4(v1[0], v1[1], v1[2], v1[3]);
        }
    } else {
        typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
        typedef float f4 __attribute__((ext_vector_type(4)));
        auto pack = [](const float (&a)[4]) {
            const f4 t = {a[0], a[1], a[2], a[3]};
            return __builtin_convertvector(t, bf4);
        };
        auto unpack = [](bf4 b, float (&a)[4]) {
            const f4 t = __builtin_convertvector(b, f4);
            a[0] = t[0]; a[1] = t[1]; a[2] = t[2]; a[3] = t[3];
        };
        __bf16 *C0 = static_cast<__bf16 *>(p.C0);
        if constexpr (EPI == EPI_STORE) {
            *reinterpret_cast<bf4 *>(C0 + coff + row * p.ldc + n) = pack(v0);
            if (p.Cx) *reinterpret_cast<bf4 *>(static_cast<__bf16 *>(p.Cx) + coff + row * p.ldc + n) = pack(v1);
        } else if constexpr (EPI == EPI_ACCUM) {
            bf4 *c = reinterpret_cast<bf4 *>(C0 + coff + row * p.ldc + n);
            float a[4];
            unpack(*c, a);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] += v0[i];
            *c = pack(a);
        } else if constexpr (EPI == EPI_SWIGLU) {
            // act = silu(H1) * H3 from the fp32 accumulators
            float a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-v0[i]));
                a[i] = v0[i] * sg * v1[i];
            }
            if (C0) *reinterpret_cast<bf4 *>(C0 + row * p.ldc + n) = pack(a);
            if (p.aux_out) {
                __bf16 *s = static_cast<__bf16 *>(p.aux_out) + row * p.ld_aux + n;
                *reinterpret_cast<bf4 *>(s) = pack(v0);
                *reinterpret_cast<bf4 *>(s + p.hoff) = pack(v1);
            }
        } else {  // EPI_SWIGLU_BWD: v0 = dA (times the row's scale, if any)
            const __bf16 *s = static_cast<const __bf16 *>(p.aux) + row * p.ld_aux + n;
            float h1[4], h3[4], g1[4], g3[4];
            unpack(*reinterpret_cast<const bf4 *>(s), h1);
            unpack(*reinterpret_cast<const bf4 *>(s + p.hoff), h3);
            const float rs = p.row_scale ? p.row_scale[row] : 1.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h1[i]));
                const float da = v0[i] * rs;
                g1[i] = da * h3[i] * sg * (1.0f + h1[i] * (1.0f - sg));
                g3[i] = da * h1[i] * sg;
            }
            *reinterpret_cast<bf4 *>(C0 + row * p.ldc + n) = pack(g1);
            *reinterpret_cast<bf4 *>(C0 + row * p.ldc + p.hoff + n) = pack(g3);
        }
    }
}

// ------------------------------------------- bf16 pipelined path (LDS DMA)
//
// The expert GEMMs run on a multi-stage ring of shared-memory tiles filled by
// direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds): the data goes from
// memory to LDS without passing through registers, so S-1 k blocks can be in
// flight while the matrix cores work on the current one.  Each such load of a
// wave writes 64 x 16 bytes to consecutive LDS addresses (lane l at +16*l, base
// in M0) from 64 freely chosen memory addresses, so a tile's LDS layout is
// fixed by choosing, for each LDS slot, which 16-byte chunk of the operand it
// receives.  The layouts below are swizzled so that the fragment reads are
// free of bank conflicts on gfx950, where a 16-byte read serves four quads of
// lanes per cycle ({0,3,5,6}, {1,2,4,7} and the same for lanes 32-63) over 64
// four-byte banks:
//   k-contiguous tile  (row = m or n, BK elements per row): chunk c of row r is
//                      stored at chunk c ^ swz_kc(r); fragment = one 16-byte read
//   mn-contiguous tile (row = k, R elements per row): chunk c of row k is stored
//                      at chunk c ^ swz_mn(k); fragment = two transposing
//                      ds_read_b64_tr_b16 reads (4 k values each), so operands
//                      that arrive mn-contiguous need no register transpose.
// Loads past a group's rows, past N or past K are given an out-of-range buffer
// offset and write zeros.

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)(p)));
}

// One 16-byte-per-lane load into LDS at `lds` (wave-uniform) + 16*lane.  The
// compiler does not see these loads: every read of their data is preceded by
// an explicit wait on the vector-memory counter and a barrier.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, int voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(lds)
                 : "memory");
}

// One 4-byte-per-lane load into LDS at `lds` (wave-uniform) + 4*lane.
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rs, int voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(lds)
                 : "memory");
}

__device__ __forceinline__ int lds_read_i32(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) int *>(static_cast<uintptr_t>(a));
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ bf16x8_t lds_read_frag16(uint32_t a) {
    return *reinterpret_cast<const lds_bf16x8_t *>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ s16x4_t lds_read_tr(uint32_t a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4_t *>(static_cast<uintptr_t>(a)));
}

// chunk swizzles; both depend on the row modulo 32 only, so fragment offsets of
// whole 32-row blocks are plain immediates
__device__ __forceinline__ int swz_kc(int r, int cpr) {
    return cpr == 8 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
}
__device__ __forceinline__ int swz_mn(int k, int cpr) {
    return cpr >= 16 ? ((0xCA60 >> (4 * (k & 3))) & 15) : 2 * (k & 3);
}

// Per-thread load plan of one operand tile (R mn x BK k), the same for every
// stage: NW waves x 64 lanes x 16 bytes per instruction, kN instructions per
// thread; instruction i of wave w fills the tile's 1 KiB block i*NW + w.
template <int R, int BK, bool KC, int NW, bool CMP = false>
struct DmaPlan {
    static constexpr int kRowBytes = KC ? BK * 2 : R * 2;
    static constexpr int kCpr = kRowBytes / 16;
    static constexpr int kBytes = R * BK * 2;
    static constexpr int kN = kBytes / (NW * 1024);
    static constexpr int kRpi = 1024 / kRowBytes;  // MN: k rows per instruction
    static_assert(kBytes % (NW * 1024) == 0, "operand tile must be a whole number of block-wide loads");
    static_assert(KC ? (BK == 32 || BK == 64) : (R == 64 || R == 128 || R == 256 || R == 512), "unsupported tile");
    // CMP (compact, MN with 4+ rows per instruction): the swizzle depends on
    // k mod 4 only, so every instruction of a lane reads the same columns and
    // instruction i's row is row 0 + i*NW*kRpi; one base and one limit then
    // serve all instructions (fewer registers live across the k loop).
    static_assert(!CMP || (!KC && kRpi % 4 == 0), "compact plans: mn-contiguous, 4+ rows per instruction");
    static constexpr int kS = CMP ? 1 : kN;
    static constexpr int kIStep = NW * kRpi;  // CMP: k rows between consecutive instructions
    int base[kS];  // byte offset of this lane's chunk at the stage's first k
    int lim[kS];   // the chunk is in range iff k0 < lim (INT_MIN: row/column out of range;
                   // CMP: instruction i iff k0 < lim - i*kIStep, INT_MIN/2 out of range)
    int step;      // CMP: bytes between consecutive instructions' rows (kIStep rows)
    // KC: rows r < rmax (r relative to the tile); MN: columns r0 + 8c < rmax
    __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int r0, int rmax, int kmax) {
#pragma unroll
        for (int i = 0; i < kS; ++i) {
            const int o = (i * NW + wave) * 1024 + lane * 16;
            const int row = o / kRowBytes, s = (o % kRowBytes) / 16;
            if constexpr (KC) {
                const int c = s ^ swz_kc(row, kCpr);
                base[i] = static_cast<int>((row * ld + 8 * c) * 2);
                lim[i] = row < rmax ? kmax - 8 * c : INT_MIN;
            } else {
                const int c = s ^ swz_mn(row, kCpr);
                base[i] = static_cast<int>((row * ld + r0 + 8 * c) * 2);
                lim[i] = r0 + 8 * c < rmax ? kmax - row : (CMP ? INT_MIN / 2 : INT_MIN);
            }
        }
        step = static_cast<int>(kIStep * ld * 2);
    }
    // KC rows read through a row map: tile row `row` < rmax is memory row rmap[row]
    __device__ __forceinline__ void init_mapped(int wave, int lane, int64_t ld, const int32_t *rmap, int rmax,
                                                int kmax) {
        static_assert(KC, "row maps apply to k-contiguous operands");
#pragma unroll
        for (int i = 0; i < kN; ++i) {
            const int o = (i * NW + wave) * 1024 + lane * 16;
            const int row = o / kRowBytes, s = (o % kRowBytes) / 16;
            const int c = s ^ swz_kc(row, kCpr);
            const int64_t mr = row < rmax ? rmap[row] : 0;
            base[i] = static_cast<int>((mr * ld + 8 * c) * 2);
            lim[i] = row < rmax ? kmax - 8 * c : INT_MIN;
        }
    }
    // CMP plan of an MN tile whose k rows are read through a row map: base
    // keeps the column part only; the row part (map[k] * ld * 2) comes per block
    __device__ __forceinline__ void init_mn_mapped(int wave, int lane, int r0, int rmax, int kmax) {
        static_assert(CMP, "k-row maps use the compact plan");
        init(wave, lane, 0, r0, rmax, kmax);
    }
    // instruction i of the k block starting at kc (INT_MAX: a block past the end);
    // KC: kadd = 2*k0; MN: the buffer starts at the block's first k row
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int kc, int kadd, uint32_t dst, int wave,
                                          int i) const {
        if constexpr (CMP)
            lds_dma16(rs, kc < lim[0] - i * kIStep ? base[0] + i * step + kadd : kOob, dst + (i * NW + wave) * 1024);
        else
            lds_dma16(rs, kc < lim[i] ? base[i] + kadd : kOob, dst + (i * NW + wave) * 1024);
    }
    // CMP, row-mapped: instruction i reads the source row at byte offset roff
    __device__ __forceinline__ void issue_row(__amdgpu_buffer_rsrc_t rs, int kc, int roff, uint32_t dst, int wave,
                                              int i) const {
        static_assert(CMP, "k-row maps use the compact plan");
        lds_dma16(rs, kc < lim[0] - i * kIStep ? roff + base[0] : kOob, dst + (i * NW + wave) * 1024);
    }
};

// Lane addresses (bytes within a tile) of a 32-wide matrix-core fragment.
template <int R, int BK, bool KC>
struct FragAddr {
    static constexpr int kRowBytes = KC ? BK * 2 : R * 2;
    static constexpr int kCpr = kRowBytes / 16;
    // KC: row mn_base + lane%32, k = kk + 8*(lane/32) .. +8
    __device__ __forceinline__ static uint32_t kc(int mn_base, int lane, int kk) {
        const int row = mn_base + (lane & 31);
        const int c = (kk / 8 + (lane >> 5)) ^ swz_kc(row, kCpr);
        return static_cast<uint32_t>(row * kRowBytes + 16 * c);
    }
    // MN: the transposing read gives lane 4a+b (within 16 lanes) element b of the
    // 4 values addressed by lanes a, a+4, a+8, a+12; lane s therefore addresses
    // k = 8*(lane/32) + (s%16)/4 (+4 for the second read), mn = 16*((s/16)%2) + 4*(s%4)
    __device__ __forceinline__ static uint32_t mn(int mn_base, int lane) {
        const int k = 8 * (lane >> 5) + ((lane & 15) >> 2);
        const int n = mn_base + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int c = (n >> 3) ^ swz_mn(k, kCpr);
        return static_cast<uint32_t>(k * kRowBytes + 16 * c + 2 * (n & 7));
    }
};

// The epilogue of a BM x BN tile held as accumulators acc[NB][TM][TN] by
// WGM x WGN waves (the layout both pipelined kernels produce), with the
// kernel's idle operand ring (RING bytes of LDS at smem / sbase) as staging.
template <int BM, int BN, int WGM, int WGN, int NB, int RING, int EPI, typename OutT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &p, const Tile &t, const GroupPtrs<bf16_t> &q,
                                              f32x16_t (&acc)[NB][BM / WGM / 32][BN / WGN / 32], char *smem,
                                              uint32_t sbase, int m0, int n0, int lane, int wave) {
    constexpr int NW = WGM * WGN, NT = 64 * NW;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    const int wm = wave / WGN, wn = wave % WGN;
    // accumulator (i, j, r) of lane l holds C[row, col] with
    //   row = i*32 + l%32,  col = j*32 + 8*(r/4) + 4*(l/32) + r%4
    const int m_lane = m0 + wm * WTM + (lane & 31);
    const int n_lane = n0 + wn * WTN + 4 * (lane >> 5);
    if constexpr (std::is_same<OutT, bf16_t>::value && (EPI == EPI_STORE || EPI == EPI_SWIGLU)) {
        // Staged epilogue: each output matrix goes through the (now idle) ring
        // as a padded row-major bf16 tile, then leaves in 16-byte row chunks
        // (16 lanes per 256-byte row segment) instead of 8-byte pieces.
        constexpr int LDC = BN + 8;
        // two passes (one per row half, i.e. per wave row) when the tile does not fit the ring
        constexpr int kPass = BM * LDC * 2 <= RING ? 1 : WGM;  // 1 pass, or one per wave row
        constexpr int RP = BM / kPass;  // rows per pass
        static_assert(RP * LDC * 2 <= RING, "output tile must fit the ring");
        typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
        typedef float f4_t __attribute__((ext_vector_type(4)));
        __bf16 *cs = reinterpret_cast<__bf16 *>(smem);
        // EPI_SWIGLU outputs: act (0) unless C0 is null, H1 and H3 (1, 2) if saved
        const int o0 = (EPI == EPI_SWIGLU && p.C0 == nullptr) ? 1 : 0;
        const int nout = EPI == EPI_SWIGLU ? (p.aux_out ? 3 : 1) : ((NB == 2 && p.Cx) ? 2 : 1);
        __syncthreads();  // every wave is done with the ring
        for (int o = o0; o < nout; ++o) {
            __bf16 *dst;
            int64_t ld;
            if constexpr (EPI == EPI_SWIGLU) {
                dst = o == 0 ? static_cast<__bf16 *>(p.C0) + q.crow * p.ldc
                             : static_cast<__bf16 *>(p.aux_out) + q.crow * p.ld_aux + (o == 2 ? p.hoff : 0);
                ld = o == 0 ? p.ldc : p.ld_aux;
            } else {
                dst = static_cast<__bf16 *>(o == 0 ? p.C0 : p.Cx) + q.coff + q.crow * p.ldc;
                ld = p.ldc;
            }
            for (int pass = 0; pass < kPass; ++pass) {
                if (kPass == 1 || wm == pass) {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                f4_t v;
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const float a = acc[0][i][j][4 * g + r], b = acc[NB - 1][i][j][4 * g + r];
                                    float x;
                                    if constexpr (EPI == EPI_SWIGLU)
                                        x = o == 0 ? a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * b : (o == 1 ? a : b);
                                    else
                                        x = o == 0 ? a : b;
                                    v[r] = x;
                                }
                                const int row = (kPass == 1 ? wm * WTM : 0) + i * 32 + (lane & 31);
                                const int col = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                                *reinterpret_cast<bf4_t *>(cs + row * LDC + col) = __builtin_convertvector(v, bf4_t);
                            }
                }
                __syncthreads();
#pragma unroll 4
                for (int c = threadIdx.x; c < RP * BN / 8; c += NT) {
                    const int row = c / (BN / 8), c8 = c % (BN / 8);
                    const int m = m0 + pass * RP + row, n = n0 + 8 * c8;
                    if (m < t.Mg && n < p.N)
                        *reinterpret_cast<uint4 *>(dst + m * ld + n) =
                            *reinterpret_cast<const uint4 *>(cs + row * LDC + 8 * c8);
                }
                if (o + 1 < nout || pass + 1 < kPass) __syncthreads();
            }
        }
        return;
    }
    if constexpr (std::is_same<OutT, bf16_t>::value && (EPI == EPI_SWIGLU_BWD || EPI == EPI_ACCUM)) {
        // Staged read-modify-write epilogue, one pass of rows at a time: the
        // tiles the epilogue reads (SwiGLU backward: the saved H1 and H3;
        // accumulate: C itself) come into the (now idle) ring by LDS DMA with
        // every load of the pass in flight at once, each lane combines its
        // accumulators with the values at the same places in place (dA, H1, H3
        // -> dH1, dH3; or C + acc), and the tiles leave in 16-byte row chunks.
        // Rows are unpadded; 16-byte chunk c of tile row r sits at chunk
        // c ^ (r % 16), which keeps the lanes' 8-byte reads (32 rows, one
        // column) and the row reads free of bank conflicts.
        constexpr int NA = EPI == EPI_SWIGLU_BWD ? 2 : 1;  // tiles read and written
        constexpr int kRowB = BN * 2;
        constexpr int kCpr = BN / 8;
        static_assert(kCpr >= 16 && (kCpr & (kCpr - 1)) == 0, "the chunk swizzle needs 16, 32, ... chunks a row");
        // wave rows per pass: all of them if the tiles fit the ring, else half, else one
        constexpr int WPP = NA * BM * kRowB <= RING                         ? WGM
                            : (WGM % 2 == 0 && NA * BM / 2 * kRowB <= RING) ? WGM / 2
                                                                                  : 1;
        constexpr int kPass = WGM / WPP, RP = WPP * WTM;
        static_assert(NA * RP * kRowB <= RING, "the tiles of a pass must fit the ring");
        constexpr int kBlk = RP * kRowB / 1024;  // 1 KiB loads per tile and pass
        static_assert(kBlk % NW == 0, "whole loads per wave");
        typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
        typedef float f4_t __attribute__((ext_vector_type(4)));
        char *const t1 = smem, *const t3 = smem + RP * kRowB;
        // the rows read back (this tile's; rows past the group's end read as zeros)
        const bf16_t *const rsrc_base = EPI == EPI_SWIGLU_BWD ? static_cast<const bf16_t *>(p.aux)
                                                              : static_cast<const bf16_t *>(p.C0);
        const int64_t ld_in = EPI == EPI_SWIGLU_BWD ? p.ld_aux : p.ldc;
        const __amdgpu_buffer_rsrc_t raux =
            make_rsrc(rsrc_base + (EPI == EPI_ACCUM ? q.coff : 0) + (q.crow + m0) * ld_in,
                      static_cast<int64_t>(t.Mg - m0) * ld_in * 2);
        __bf16 *dst = static_cast<__bf16 *>(p.C0) + q.coff + q.crow * p.ldc;
        // SwiGLU backward with row scales: a lane's rows are m_lane + 32 i
        // (each wave combines its own rows, in pass wm / WPP); multiplying by
        // 1 where there is no scale leaves dA exact
        float rsc[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m_lane + i * 32;
            rsc[i] = (EPI == EPI_SWIGLU_BWD && p.row_scale && m < t.Mg) ? p.row_scale[q.crow + m] : 1.0f;
        }
        __syncthreads();  // every wave is done with the ring
        for (int pass = 0; pass < kPass; ++pass) {
#pragma unroll
            for (int x = 0; x < kBlk / NW; ++x) {
                const int blk = x * NW + wave;
                const int o = blk * 1024 + lane * 16;
                const int row = o / kRowB, c = ((o % kRowB) / 16) ^ (row & 15);
                const int col = n0 + 8 * c;
                const int off = static_cast<int>(((pass * RP + row) * ld_in + col) * 2);
                const bool ok = col < p.N;
                lds_dma16(raux, ok ? off : kOob, sbase + blk * 1024);
                if constexpr (NA == 2)
                    lds_dma16(raux, ok ? off + static_cast<int>(p.hoff * 2) : kOob, sbase + RP * kRowB + blk * 1024);
            }
            wait_vmem<0>();
            __syncthreads();
            if (wm / WPP == pass) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int row = (wm % WPP) * WTM + i * 32 + (lane & 31);
                            const int col = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                            const int at = row * kRowB + 16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7);
                            bf4_t *p1 = reinterpret_cast<bf4_t *>(t1 + at);
                            const f4_t h1 = __builtin_convertvector(*p1, f4_t);
                            if constexpr (NA == 2) {
                                bf4_t *p3 = reinterpret_cast<bf4_t *>(t3 + at);
                                const f4_t h3 = __builtin_convertvector(*p3, f4_t);
                                f4_t g1, g3;
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const float v0 = acc[0][i][j][4 * g + r] * rsc[i];
                                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h1[r]));
                                    g1[r] = v0 * h3[r] * sg * (1.0f + h1[r] * (1.0f - sg));
                                    g3[r] = v0 * h1[r] * sg;
                                }
                                *p1 = __builtin_convertvector(g1, bf4_t);
                                *p3 = __builtin_convertvector(g3, bf4_t);
                            } else {
                                f4_t c1;
#pragma unroll
                                for (int r = 0; r < 4; ++r) c1[r] = h1[r] + acc[0][i][j][4 * g + r];
                                *p1 = __builtin_convertvector(c1, bf4_t);
                            }
                        }
            }
            __syncthreads();
#pragma unroll 4
            for (int c = threadIdx.x; c < RP * kCpr; c += NT) {
                const int row = c / kCpr, c8 = c % kCpr;
                const int m = m0 + pass * RP + row, n = n0 + 8 * c8;
                if (m < t.Mg && n < p.N) {
                    const int at = row * kRowB + 16 * (c8 ^ (row & 15));
                    *reinterpret_cast<uint4 *>(dst + m * p.ldc + n) = *reinterpret_cast<const uint4 *>(t1 + at);
                    if constexpr (NA == 2)
                        *reinterpret_cast<uint4 *>(dst + m * p.ldc + p.hoff + n) =
                            *reinterpret_cast<const uint4 *>(t3 + at);
                }
            }
            if (pass + 1 < kPass) __syncthreads();
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = m_lane + i * 32;
        if (m >= t.Mg) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n_lane + j * 32 + 8 * g;
                if (n >= p.N) continue;
                float v0[4], v1[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v0[r] = acc[0][i][j][4 * g + r];
                    v1[r] = acc[NB - 1][i][j][4 * g + r];
                }
                epilogue4<EPI, OutT>(p, q.crow, q.coff, m, n, v0, v1);
            }
    }
}

// BM x (NB*BN) output tile per block of WGM x WGN waves, BK-deep k blocks on
// an S-slot LDS ring.  Per k step (16 of k) each wave issues its NB*TN*TM
// matrix-core products interleaved with the fragment reads of the next step
// (two register sets) and with its share of the loads of the block S-1 ahead.
// The barrier of block `it` sits at the start of its last k step: all
// fragments of the block are in registers by then, so the freed slot can be
// refilled and the next block's first fragments read while the last products
// of this block run.  OCC = 2 keeps LDS and registers low enough for two
// blocks per compute unit; 8 waves put two waves of one block on each SIMD.
// A wave whose rows (or columns) all lie past the group's end skips its
// products and fragment reads (it still loads and meets every barrier), so
// the ragged last row tile of an expert costs matrix-core time only for its
// valid wave rows.
template <int BM, int BN, int BK, int WGM, int WGN, int NB, bool A_KC, bool B_KC, int S, int EPI, typename OutT,
          int OCC, bool KMAP = false>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(OCC * WGM * WGN / 4, OCC * WGM * WGN / 4)))
void gemm_dma_kernel(GemmArgs p) {
    constexpr int NW = WGM * WGN, NT = 64 * NW;
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tile must be a multiple of 32");
    // the KMAP kernel keeps its mn-contiguous plans compact (registers for the ids)
    using PA = DmaPlan<BM, BK, A_KC, NW, KMAP>;
    using PB = DmaPlan<BN, BK, B_KC, NW, KMAP && !B_KC && (512 / BN) % 4 == 0>;
    constexpr int kABytes = PA::kBytes, kBBytes = PB::kBytes;
    constexpr int kStage = kABytes + NB * kBBytes;
    constexpr int kL = PA::kN + NB * PB::kN;   // operand loads per thread per k block
    // KMAP: GM_KSPLIT with an mn-contiguous A whose k rows are read through
    // p.a_map (row k of the group reads A0 row a_map[base + k]).  Each wave
    // needs the ids of kIds rows per k block; they reach a ring of kIdQ LDS
    // regions per wave by one more direct-to-LDS load per block, issued 2S-2
    // blocks ahead, so that they sit behind the same vector-memory count as
    // the operand tiles and no scalar or register load enters the loop.
    static_assert(!KMAP || (!A_KC && EPI == EPI_STORE), "k-row maps: mn-contiguous A, plain store");
    constexpr int kRpi = PA::kRpi;                        // k rows per A load instruction
    constexpr int kIds = KMAP ? PA::kN * kRpi : 0;        // ids per wave per k block (= BK / NW)
    constexpr int kIdQ = 2 * S - 2;
    constexpr int kIdBytes = KMAP ? kIdQ * NW * 256 : 0;
    constexpr int kLi = kL + (KMAP ? 1 : 0);              // loads per thread per k block
    static_assert(kIds <= 64, "one id per lane");
    static_assert(S >= 2 && kLi * (S - 2) <= 63, "vmcnt range");
    static_assert(S * kStage + kIdBytes <= 160 * 1024 / OCC - 64, "OCC blocks per CU must fit the 160 KiB of LDS");
    constexpr int KK = BK / 16;
    static_assert(KK == 2 || KK == 4, "BK must be 32 or 64");
    constexpr int NM = NB * TN * TM;                 // products per k step
    constexpr int NR = TM + NB * TN;                 // fragments per k step
    constexpr int DPK = (kL + KK - 2) / (KK - 1);    // loads per k step (all steps but the last)
    constexpr int DPQ = (DPK + NM - 1) / NM;         // loads per product
    __shared__ __align__(1024) char smem[S * kStage + kIdBytes];

    Tile t;
    // a split over k gives consecutive blocks the parts of one tile
    const int kparts = p.group_mode == GM_ROWS && p.kparts > 1 ? p.kparts : 1;
    const int kpart = static_cast<int>(blockIdx.x) % kparts;
    if (!resolve_tile<BM, BN>(p, &t, blockIdx.x / kparts, gridDim.x / kparts)) return;
    GroupPtrs<bf16_t> q = group_ptrs<bf16_t>(p, t);
    int kstart = 0;
    if (kparts > 1) {
        kstart = kpart * p.kpart_len;
        t.Kg = min(t.Kg, kstart + p.kpart_len);
        q.coff += static_cast<int64_t>(kpart) * p.c_gstride;
    }
    const int m0 = t.m0, n0 = t.nt * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    const bool wact = m0 + wm * WTM < t.Mg && n0 + wn * WTN < p.N;  // this wave has output

    const int ktiles = (t.Kg - kstart + BK - 1) / BK;
    const int nph = p.group_mode == GM_KSPLIT ? 1 : p.nphase;
    const int total = t.Kg > kstart ? ktiles * nph : 0;

    PA pa;
    PB pb;
    const bool amap = A_KC && p.a_map != nullptr && p.group_mode == GM_ROWS;
    if constexpr (A_KC) {
        if (amap) pa.init_mapped(wave, lane, p.lda, p.a_map + t.base + m0, t.Mg - m0, t.Kg);
        else pa.init(wave, lane, p.lda, 0, t.Mg - m0, t.Kg);
    } else if constexpr (KMAP) {
        pa.init_mn_mapped(wave, lane, m0, t.Mg, t.Kg);
    } else {
        pa.init(wave, lane, p.lda, m0, t.Mg, t.Kg);
    }
    if constexpr (B_KC) pb.init(wave, lane, p.ldb, 0, p.N - n0, t.Kg);
    else pb.init(wave, lane, p.ldb, n0, p.N, t.Kg);

    // Buffers: a k-contiguous operand starts at the tile's first row (offsets
    // 2*k0 + a few rows); an mn-contiguous one at the k block's first row.
    auto rs_kc = [&](const bf16_t *b, int r0, int rows, int64_t ld) {
        return make_rsrc(b + static_cast<int64_t>(r0) * ld, static_cast<int64_t>(rows - r0) * ld * 2);
    };
    auto rs_mn = [&](const bf16_t *b, int64_t ld, int k0) {
        return make_rsrc(b + static_cast<int64_t>(k0) * ld, static_cast<int64_t>(t.Kg - k0) * ld * 2);
    };
    const __amdgpu_buffer_rsrc_t none = make_rsrc(q.A0, 0);  // placeholder for mn-contiguous operands
    __amdgpu_buffer_rsrc_t ra0 = none, ra1 = none, rb0 = none, rb1 = none, rbx = none;
    if constexpr (A_KC) {
        // with a row map the buffer spans the whole gathered matrix (its
        // a_map_rows * lda elements must stay below 2^31 bytes)
        ra0 = amap ? make_rsrc(p.A0, p.a_map_rows * p.lda * 2) : rs_kc(q.A0, m0, t.Mg, p.lda);
        ra1 = q.A1 ? rs_kc(q.A1, m0, t.Mg, p.lda) : ra0;
    }
    // KMAP: A's buffer spans the whole source matrix (a_map_rows * lda * 2 <
    // 2^31 bytes), the ids' buffer the group's map entries
    const uint32_t idbase = sbase + S * kStage;
    __amdgpu_buffer_rsrc_t rid = none;
    int id_row = -1;   // KMAP: the k row (within a block) whose id this lane loads
    const int lda2 = static_cast<int>(p.lda) * 2;
    if constexpr (KMAP) {
        ra0 = make_rsrc(p.A0, p.a_map_rows * p.lda * 2);
        rid = make_rsrc(p.a_map + t.base, static_cast<int64_t>(t.Kg) * 4);
        if (lane < kIds) id_row = ((lane / kRpi) * NW + wave) * kRpi + lane % kRpi;
    }
    // KMAP: the ids of block st go to region st % kIdQ of this wave (rows past
    // the group's end, and blocks past the end, load zeros)
    auto issue_ids = [&](int st) {
        const int k0 = kstart + st * BK;
        lds_dma4(rid, st < total && id_row >= 0 ? (k0 + id_row) * 4 : kOob,
                 idbase + ((st % kIdQ) * NW + wave) * 256);
    };
    if constexpr (B_KC) {
        rb0 = rs_kc(q.B0, n0, p.N, p.ldb);
        rb1 = q.B1 ? rs_kc(q.B1, n0, p.N, p.ldb) : rb0;
        rbx = q.Bx ? rs_kc(q.Bx, n0, p.N, p.ldb) : rb0;
    }

    // Everything a k block's loads need, computed once per block: the buffers
    // (an mn-contiguous operand's buffer starts at the block's first k row),
    // the k offset of k-contiguous operands, and kc = k0, or INT_MAX for blocks
    // past the end, which makes every load of such a block out of range (it
    // writes zeros to a slot nobody reads and keeps the count of loads in
    // flight uniform).
    struct StagePlan {
        __amdgpu_buffer_rsrc_t ra, rb, rx;
        int kc, kadd;
        int arow[KMAP ? PA::kN : 1];  // KMAP: byte offset of this lane's source row, per A instruction
    };
    auto plan_stage = [&](int st) {
        StagePlan sp;
        const bool live = st < total;
        const int ph = (live && st >= ktiles) ? 1 : 0;
        const int k0 = live ? kstart + (st - ph * ktiles) * BK : 0;
        sp.kc = live ? k0 : INT_MAX;
        sp.kadd = 2 * k0;
        if constexpr (A_KC) {
            sp.ra = ph ? ra1 : ra0;
        } else if constexpr (KMAP) {
            // this wave's ids of block st (landed: see the waits on the ids' loads)
            sp.ra = ra0;
            const uint32_t ib = idbase + ((st % kIdQ) * NW + wave) * 256 + 4 * (lane / PA::kCpr);
#pragma unroll
            for (int i = 0; i < PA::kN; ++i) sp.arow[i] = lds_read_i32(ib + 4 * kRpi * i) * lda2;
        } else {
            sp.ra = rs_mn(ph ? q.A1 : q.A0, p.lda, k0);
        }
        if constexpr (B_KC) {
            sp.rb = ph ? rb1 : rb0;
            sp.rx = rbx;
        } else {
            sp.rb = rs_mn(ph ? q.B1 : q.B0, p.ldb, k0);
            sp.rx = NB == 2 ? rs_mn(q.Bx, p.ldb, k0) : sp.rb;
        }
        return sp;
    };
    // load instruction `part` (0 .. kL-1) of a k block into the slot at `dst`
    auto issue_part = [&](const StagePlan &sp, uint32_t dst, int part) {
        if (part < PA::kN) {
            if constexpr (KMAP)
                pa.issue_row(sp.ra, sp.kc, sp.arow[part], dst, wave, part);
            else
                pa.issue(sp.ra, sp.kc, A_KC ? sp.kadd : 0, dst, wave, part);
        } else {
            const int pp = part - PA::kN;
            const int b = pp / PB::kN, i = pp % PB::kN;
            pb.issue(b ? sp.rx : sp.rb, sp.kc, B_KC ? sp.kadd : 0, dst + kABytes + b * kBBytes, wave, i);
        }
    };

    f32x16_t acc[NB][TM][TN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.0f;

    uint32_t fa[A_KC ? KK : TM], fb[B_KC ? KK : TN];
#pragma unroll
    for (int x = 0; x < (A_KC ? KK : TM); ++x)
        fa[x] = A_KC ? FragAddr<BM, BK, true>::kc(wm * WTM, lane, 16 * x)
                     : FragAddr<BM, BK, false>::mn(wm * WTM + 32 * x, lane);
#pragma unroll
    for (int x = 0; x < (B_KC ? KK : TN); ++x)
        fb[x] = B_KC ? FragAddr<BN, BK, true>::kc(wn * WTN, lane, 16 * x)
                     : FragAddr<BN, BK, false>::mn(wn * WTN + 32 * x, lane);

    auto frag = [&](uint32_t tile, bool kc, const uint32_t *fx, int x, int kk, int rowbytes) -> bf16x8_t {
        if (kc) return lds_read_frag16(tile + fx[kk / 16] + x * 32 * rowbytes);
        const uint32_t a = tile + fx[x] + kk * rowbytes;
        const s16x4_t lo = lds_read_tr(a), hi = lds_read_tr(a + 4 * rowbytes);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t fA[2][TM], fB[2][NB][TN];
    auto read_unit = [&](int set, int u, uint32_t sa, int kk) {
        if (u < TM) {
            fA[set][u] = frag(sa, A_KC, fa, u, kk, PA::kRowBytes);
        } else {
            const int b = (u - TM) / TN, j = (u - TM) % TN;
            fB[set][b][j] = frag(sa + kABytes + b * kBBytes, B_KC, fb, j, kk, PB::kRowBytes);
        }
    };

    // prologue: blocks 0 .. S-2 in flight; wait for block 0; its first
    // fragments.  KMAP: the ids of blocks 0 .. S-2 land first, and block s's
    // tiles go out behind the ids of block s+S-1, the order the loop keeps
    // (ids of block st+S-1, then block st's tiles).
    if constexpr (KMAP) {
#pragma unroll
        for (int s = 0; s < S - 1; ++s) issue_ids(s);
        wait_vmem<0>();
    }
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
        if constexpr (KMAP) issue_ids(s + S - 1);
        const StagePlan sp = plan_stage(s);
#pragma unroll
        for (int u = 0; u < kL; ++u) issue_part(sp, sbase + s * kStage, u);
    }
    wait_vmem<kLi * (S - 2)>();
    __syncthreads();
    // The k loop, instantiated for waves with output (products and fragment
    // reads) and without (loads and barriers only); both meet the same barriers.
    auto k_loop = [&](auto active) {
        constexpr bool ACT = decltype(active)::value;
        if constexpr (ACT) {
#pragma unroll
            for (int u = 0; u < NR; ++u) read_unit(0, u, sbase, 0);
        }
        int cur = 0;  // ring slot of block `it`
        for (int it = 0; it < total; ++it) {
            const uint32_t sa = sbase + cur * kStage;
            const int nxt = cur + 1 == S ? 0 : cur + 1;
            const uint32_t sf = sbase + (cur == 0 ? S - 1 : cur - 1) * kStage;  // freed by the last barrier
            // KMAP: block it+2S-2's ids go out before block it+S-1's tiles.  Per
            // block a thread then issues kLi loads, ids first, so the wait below
            // (all but the last kLi*(S-2)) also covers the ids of block it+S,
            // issued just before block it+1's tiles, which the next iteration's
            // plan reads.  Region (st % kIdQ) is next written by the ids of
            // block st+2S-2, issued in iteration st, after block st's ids were
            // read (iteration st-S+1 or the prologue).
            if constexpr (KMAP) issue_ids(it + 2 * S - 2);
            const StagePlan sp = plan_stage(it + S - 1);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int c = kk & 1, n = c ^ 1;
                uint32_t rs = sa;
                int rk = kk + 1;
                if (kk == KK - 1) {
                    wait_vmem<kLi * (S - 2)>();  // this wave's loads of block it+1 have landed
                    __syncthreads();            // ... everyone's, and all reads of block it are done
                    rs = sbase + nxt * kStage;
                    rk = 0;
                }
#pragma unroll
                for (int qq = 0; qq < NM; ++qq) {
                    if constexpr (ACT) {
                        const int b = qq / (TN * TM), j = (qq / TM) % TN, i = qq % TM;
                        acc[b][i][j] =
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fB[c][b][j], fA[c][i], acc[b][i][j], 0, 0, 0);
                        if (qq < NR) read_unit(n, qq, rs, rk * 16);
                        if (qq == NM - 1) {
#pragma unroll
                            for (int u = NM; u < NR; ++u) read_unit(n, u, rs, rk * 16);
                        }
                    }
                    if (kk < KK - 1) {
#pragma unroll
                        for (int z = 0; z < DPQ; ++z) {
                            const int part = kk * DPK + qq * DPQ + z;
                            if (qq * DPQ + z < DPK && part < kL) issue_part(sp, sf, part);
                        }
                    }
                }
            }
            cur = nxt;
        }
    };
    if (wact) k_loop(std::true_type{});
    else k_loop(std::false_type{});
    wait_vmem<0>();  // no load may still target LDS when the block ends
    gemm_epilogue<BM, BN, WGM, WGN, NB, S * kStage, EPI, OutT>(p, t, q, acc, smem, sbase, m0, n0, lane, wave);
}

template <int BM, int BN, int BK, int WGM, int WGN, int NB, bool A_KC, bool B_KC, int S, int EPI, typename OutT,
          int OCC, bool KMAP = false>
inline hipError_t launch_gemm_dma(const GemmArgs &p, hipStream_t stream) {
    if (KMAP && (p.a_map == nullptr || p.group_mode != GM_KSPLIT)) return hipErrorInvalidValue;
    const int64_t grid = gemm_grid<BM, BN>(p);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, BK, WGM, WGN, NB, A_KC, B_KC, S, EPI, OutT, OCC, KMAP>),
                       dim3(static_cast<unsigned>(grid)), dim3(64 * WGM * WGN), 0, stream, p);
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
    if (!resolve_tile<BM, BN>(p, &t, blockIdx.x, gridDim.x)) return;
    const GroupPtrs<float> q = group_ptrs<float>(p, t);
    const int m0 = t.m0, n0 = t.nt * BN;
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
                if (gm < t.Mg && gk < t.Kg) {
                    if (A_KC && p.a_map && p.group_mode == GM_ROWS)
                        va = static_cast<const float *>(p.A0)[static_cast<int64_t>(p.a_map[t.base + gm]) * p.lda + gk];
                    else if (!A_KC && p.a_map && p.group_mode == GM_KSPLIT)
                        va = static_cast<const float *>(p.A0)[static_cast<int64_t>(p.a_map[t.base + gk]) * p.lda + gm];
                    else
                        va = A_KC ? A[static_cast<int64_t>(gm) * p.lda + gk] : A[static_cast<int64_t>(gk) * p.lda + gm];
                }
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

// Expert FFN forward and backward on the expert-sorted (padding-free) rows.
//
// X-MoE article (adg.csdn.net), section 2.1.2 "跨平台核函数优化": the experts'
// GEMMs take each expert's rows as a dynamic slice -- no padding to a common
// capacity -- where the article's sketch loops over the experts on the host.
// Here one launch covers every expert: the grid is sized from the row count
// and the expert count, and each block finds its expert and row tile from the
// device-side offsets (see gemm.hpp).  The bf16 products run on the pipelined
// LDS-DMA kernel; tile shapes were chosen per product by timing on MI355X
// (BM x BN x BK, wave grid, NB weight matrices, S ring slots, blocks per
// compute unit), comparing candidates within one run on one device.  The expert is a SwiGLU FFN (a reading:
// the pages name no FFN form), so the up-projection multiplies the same rows
// by W1 and W3 in one kernel and applies silu(H1) * H3 in its epilogue.
//
// Products (rows of expert e = [off[e], off[e+1]); weights row-major):
//   up       act = silu(xs.W1) * (xs.W3)        A = xs, B = W1 | W3 (n-contiguous);
//                                               or A row r = x[token_ids[r]] (gather fused)
//   down     ye  = act.W2                       A = act, B = W2 (n-contiguous)
//   dgrad2   dA  = dye.W2^T -> dH1, dH3         A = dye, B = W2 read k-contiguous;
//                                               or A row r = dy[token_ids[r]] and dA
//                                               row r scaled by the combine weight
//   dgrad1   dxs = dH1.W1^T + dH3.W3^T          two k phases, B read k-contiguous
//   wgrad13  dW1 = xs^T dH1, dW3 = xs^T dH3     reduction over the expert's rows
//   wgrad2   dW2 = act^T dye                    reduction over the expert's rows
#include <cmath>

#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

namespace xmoe {

namespace {

GemmArgs rows_args(const int32_t *offsets, int E, int64_t rows) {
    GemmArgs p{};
    p.group_mode = GM_ROWS;
    p.offsets = offsets;
    p.G = E;
    p.extent = rows;
    p.nphase = 1;
    return p;
}

// Large tiles (256-row, eight waves) cut the bytes each product moves from L2
// into LDS by a third, but they round every expert's rows up to a multiple of
// 256 and need enough tiles to fill the device (the grid must still give two
// blocks per compute unit).  large_tiles: the average group has at least 1024
// rows, where the rounding costs little.
bool large_grid(int64_t rows, int E, int64_t n, int bn) {
    return (rows / 256 + E) * ((n + bn - 1) / bn) >= 512;
}
bool large_tiles(int64_t rows, int E, int64_t n, int bn) {
    return rows / (E > 0 ? E : 1) >= 1024 && large_grid(rows, E, n, bn);
}
// The down-projection and dA products also gain from them below 1024 rows when
// an expert's last 256-row tile is well filled: the mean count's remainder r
// modulo 256 is at least 96, and two standard deviations of the per-expert
// count (about sqrt(mean) for uniform routing) above it still stay within the
// tile, so few experts spill into an almost empty extra tile.  Measured small
// against large on one device (mean rows 256 .. 1024 per expert): the large
// tile is 3-14% faster at 384 and 448 rows, level at 640 and 1024, and 5-16%
// slower at 256, 320, 512 and 768.
bool large_tiles_filled(int64_t rows, int E, int64_t n, int bn) {
    const int64_t per_group = rows / (E > 0 ? E : 1);
    if (!large_grid(rows, E, n, bn)) return false;
    if (per_group >= 1024) return true;
    const int64_t r = per_group % 256;
    const double sd = std::sqrt(static_cast<double>(per_group));
    return per_group >= 256 && r >= 96 && static_cast<double>(r) + 2.0 * sd <= 256.0;
}

// A k-split product (weight gradients) has E x ceil(m/bm) x ceil(n/bm) tiles
// whatever the rows.  The 256-square tile runs one block per compute unit, so
// its grid fills the device from 256 tiles (the DeepSeek-MoE-16B dW2 has 384;
// one dense group of h = 2048, d = 4096 has 128 and keeps the smaller tile).
bool ksplit_fills(int E, int64_t m, int64_t n, int bm) {
    return static_cast<int64_t>(E) * ((m + bm - 1) / bm) * ((n + bm - 1) / bm) >= 256;
}

// The weight gradients give each XCD runs of half an expert's tiles: an
// expert's rows and row gradients, a few MB, are then fetched into two L2s
// instead of several.  Step time (dW1/dW3 alone) against runs of 32 tiles and
// runs of a whole expert: DeepSeek-MoE-16B 2.374 (0.406) ms against 2.374
// (0.419) and 2.369 (0.401); Zipf-skewed 5.27 against 5.33 and 5.47 ms, where
// whole-expert runs put all the tiles of the heaviest expert (16384 rows) on
// one XCD.
GemmArgs ksplit_args(const int32_t *offsets, int E, int64_t rows) {
    GemmArgs p{};
    p.group_mode = GM_KSPLIT;
    p.offsets = offsets;
    p.G = E;
    p.extent = rows;
    p.nphase = 1;
    p.xcd_run = -1;
    return p;
}

}  // namespace

hipError_t launch_ffn_up(int dt, const void *xs, const int32_t *row_map, int64_t map_rows, const void *w1,
                         const void *w3, const int32_t *offsets, int E, int64_t rows, int d, int h, void *act,
                         void *h13, hipStream_t s) {
    GemmArgs p = rows_args(offsets, E, rows);
    p.a_map = row_map;  // the gather fused into the A loads: row r reads xs[row_map[r]]
    p.a_map_rows = map_rows;
    p.N = h;
    p.K = d;
    p.A0 = xs;
    p.lda = d;
    p.B0 = w1;
    p.Bx = w3;
    p.ldb = h;
    p.b_gstride = static_cast<int64_t>(d) * h;
    p.C0 = act;
    p.ldc = h;
    p.aux_out = h13;
    p.ld_aux = 2 * static_cast<int64_t>(h);
    p.hoff = h;
    if (dt != kBF16) return launch_gemm_f32<2, true, false, EPI_SWIGLU>(p, s);
    if (large_tiles(rows, E, h, 128))
        return launch_gemm_dma<256, 128, 32, 4, 2, 2, true, false, 4, EPI_SWIGLU, bf16_t, 1>(p, s);
    // below 1024 rows per expert, h a multiple of 256: 256 columns of W1 and of
    // W3 per block (eight waves of 64 x 64 x 2) share each row tile twice as
    // long; 7% faster at 256 rows per expert, h = 2048, d = 7168.  With h =
    // 1408 the last such tile is half empty, and a single dense group (4096
    // rows, h = 2816, whose large-tile grid is too small) runs 12% slower: both
    // keep the 128-column tile.
    if (h % 256 == 0 && rows / (E > 0 ? E : 1) < 1024)
        return launch_gemm_dma<128, 256, 32, 2, 4, 2, true, false, 3, EPI_SWIGLU, bf16_t, 1>(p, s);
    return launch_gemm_dma<128, 128, 32, 2, 2, 2, true, false, 3, EPI_SWIGLU, bf16_t, 2>(p, s);
}

hipError_t launch_ffn_down(int dt, const void *act, const void *w2, const int32_t *offsets, int E, int64_t rows, int d,
                           int h, void *ye, bool accumulate, hipStream_t s) {
    GemmArgs p = rows_args(offsets, E, rows);
    p.N = d;
    p.K = h;
    p.A0 = act;
    p.lda = h;
    p.B0 = w2;
    p.ldb = d;
    p.b_gstride = static_cast<int64_t>(h) * d;
    p.C0 = ye;
    p.ldc = d;
    p.accum = accumulate ? 1 : 0;
    if (dt != kBF16) return launch_gemm_f32<1, true, false, EPI_STORE>(p, s);
    // ye += act . W2: the staged read-modify-write epilogue (one rounding of
    // ye + products), on the tile that serves every size
    if (accumulate) return launch_gemm_dma<128, 256, 32, 2, 2, 1, true, false, 3, EPI_ACCUM, bf16_t, 2>(p, s);
    return large_tiles_filled(rows, E, d, 256)
               ? launch_gemm_dma<256, 256, 32, 4, 2, 1, true, false, 4, EPI_STORE, bf16_t, 1>(p, s)
               : launch_gemm_dma<128, 256, 32, 2, 2, 1, true, false, 3, EPI_STORE, bf16_t, 2>(p, s);
}

// dA = dye . W2[e]^T with the SwiGLU backward in the epilogue -> dh13; with
// row_map, A row r is dye[row_map[r]] (dye then has map_rows rows), and with
// row_scale dA row r is multiplied by row_scale[r] before the SwiGLU backward
hipError_t launch_ffn_bwd_dact(int dt, const void *dye, const int32_t *row_map, int64_t map_rows,
                               const float *row_scale, const void *w2, const void *h13, const int32_t *offsets, int E,
                               int64_t rows, int d, int h, void *dh13, hipStream_t s) {
    const int64_t dh = static_cast<int64_t>(d) * h;
    hipError_t err;
    GemmArgs p = rows_args(offsets, E, rows);
    p.N = h;
    p.K = d;
    p.A0 = dye;
    p.a_map = row_map;
    p.a_map_rows = map_rows;
    p.row_scale = row_scale;
    p.lda = d;
    p.B0 = w2;          // B(k=c, n=j) = W2[e][j*d + c]
    p.ldb = d;
    p.b_gstride = dh;
    p.C0 = dh13;
    p.ldc = 2 * static_cast<int64_t>(h);
    p.aux = h13;
    p.ld_aux = 2 * static_cast<int64_t>(h);
    p.hoff = h;
    // the 256-row tile on the down-projection's rule (an expert's last 256-row
    // tile well filled): at 384 rows per expert routed dA 0.262 -> 0.242 ms
    // alone, the DeepSeek-MoE-16B step level (with dW1/dW3 beside dA and dX on
    // the caller's stream; with dW1/dW3 on the weight-gradient stream the
    // 128-row tile had made the step 0.7% faster)
    err = dt != kBF16 ? launch_gemm_f32<1, true, true, EPI_SWIGLU_BWD>(p, s)
          : large_tiles_filled(rows, E, h, 256)
              ? launch_gemm_dma<256, 256, 32, 4, 2, 1, true, true, 4, EPI_SWIGLU_BWD, bf16_t, 1>(p, s)
                                         : launch_gemm_dma<128, 256, 32, 2, 2, 1, true, true, 3, EPI_SWIGLU_BWD, bf16_t, 2>(p, s);
    return err;
}

// dxs = dH1 . W1[e]^T + dH3 . W3[e]^T
hipError_t launch_ffn_bwd_dx(int dt, const void *dh13, const void *w1, const void *w3, const int32_t *offsets, int E,
                             int64_t rows, int d, int h, void *dxs, bool accumulate, hipStream_t s) {
    const int64_t dh = static_cast<int64_t>(d) * h;
    const size_t esz = dt == kBF16 ? 2 : 4;
    hipError_t err;
    GemmArgs p = rows_args(offsets, E, rows);
    p.N = d;
    p.K = h;
    p.nphase = 2;
    p.A0 = dh13;
    p.A1 = static_cast<const char *>(dh13) + h * esz;
    p.lda = 2 * static_cast<int64_t>(h);
    p.B0 = w1;          // B(k=j, n=i) = W1[e][i*h + j]
    p.B1 = w3;
    p.ldb = h;
    p.b_gstride = dh;
    p.C0 = dxs;
    p.ldc = d;
    p.accum = accumulate ? 1 : 0;
    // one 256x256 tile of eight waves per compute unit at every size (measured
    // level with or ahead of four waves from 256 to 1638 rows per expert);
    // dxs += ...: the staged read-modify-write epilogue
    err = dt != kBF16 ? launch_gemm_f32<1, true, true, EPI_STORE>(p, s)
          : accumulate ? launch_gemm_dma<256, 256, 32, 4, 2, 1, true, true, 4, EPI_ACCUM, bf16_t, 1>(p, s)
                       : launch_gemm_dma<256, 256, 32, 4, 2, 1, true, true, 4, EPI_STORE, bf16_t, 1>(p, s);
    return err;
}

// dW1[e] = xs_e^T . dH1_e and dW3[e] = xs_e^T . dH3_e (zeros for an empty expert);
// with row_map, xs[r] is read as xs[row_map[r]] (xs then has map_rows rows)
hipError_t launch_ffn_bwd_dw13(int dt, const void *xs, const int32_t *row_map, int64_t map_rows, const void *dh13,
                               const int32_t *offsets, int E, int64_t rows, int d, int h, void *dw1, void *dw3,
                               int grad_dt, bool accumulate, hipStream_t s) {
    const int64_t dh = static_cast<int64_t>(d) * h;
    const size_t esz = dt == kBF16 ? 2 : 4;
    hipError_t err;
    GemmArgs p = ksplit_args(offsets, E, rows);
    p.M = d;
    p.N = h;
    p.A0 = xs;          // A(m=i, k=r) = xs[r*d + i]
    p.lda = d;
    p.B0 = dh13;        // B(k=r, n=j) = dh13[r*2h + j]
    p.Bx = static_cast<const char *>(dh13) + h * esz;
    p.ldb = 2 * static_cast<int64_t>(h);
    p.C0 = dw1;
    p.Cx = dw3;
    p.ldc = h;
    p.c_gstride = dh;
    p.a_map = row_map;  // the gather fused into the A loads: k row r reads xs[row_map[r]]
    p.a_map_rows = map_rows;
    p.accum = accumulate ? 1 : 0;   // fp32 gradients only
    // short reductions (few rows per expert) leave each tile little work to
    // hide its pipeline fill and epilogue behind: three blocks per compute unit
    // (two-slot rings) overlap more of them
    if (dt != kBF16) return launch_gemm_f32<2, false, false, EPI_STORE>(p, s);
    if (grad_dt != kBF16) {
        // fp32 gradients of bf16 inputs: the sums leave unrounded (stored, or
        // added to the caller's fp32 gradients), one tile at every size
        return row_map ? launch_gemm_dma<128, 128, 32, 2, 2, 2, false, false, 3, EPI_STORE, float, 2, true>(p, s)
                       : launch_gemm_dma<128, 128, 32, 2, 2, 2, false, false, 3, EPI_STORE, float, 2>(p, s);
    }
    const bool short_k = rows / (E > 0 ? E : 1) < 1024;
    if (row_map)
        err = short_k ? launch_gemm_dma<128, 128, 32, 2, 2, 2, false, false, 2, EPI_STORE, bf16_t, 3, true>(p, s)
                      : launch_gemm_dma<128, 128, 32, 2, 2, 2, false, false, 3, EPI_STORE, bf16_t, 2, true>(p, s);
    else
        err = short_k ? launch_gemm_dma<128, 128, 32, 2, 2, 2, false, false, 2, EPI_STORE, bf16_t, 3>(p, s)
                      : launch_gemm_dma<128, 128, 32, 2, 2, 2, false, false, 3, EPI_STORE, bf16_t, 2>(p, s);
    return err;
}

// dW2[e] = act_e^T . dye_e
hipError_t launch_ffn_bwd_dw2(int dt, const void *act, const void *dye, const int32_t *offsets, int E, int64_t rows,
                              int d, int h, void *dw2, int grad_dt, bool accumulate, hipStream_t s) {
    const int64_t dh = static_cast<int64_t>(d) * h;
    hipError_t err;
    GemmArgs p = ksplit_args(offsets, E, rows);
    p.M = h;
    p.N = d;
    p.A0 = act;         // A(m=j, k=r) = act[r*h + j]
    p.lda = h;
    p.B0 = dye;         // B(k=r, n=c) = dye[r*d + c]
    p.ldb = d;
    p.C0 = dw2;
    p.ldc = d;
    p.c_gstride = dh;
    p.accum = accumulate ? 1 : 0;   // fp32 gradients only
    if (dt != kBF16) return launch_gemm_f32<1, false, false, EPI_STORE>(p, s);
    if (grad_dt != kBF16)
        return launch_gemm_dma<128, 256, 32, 2, 2, 1, false, false, 3, EPI_STORE, float, 2>(p, s);
    // the 256-row tile whenever its grid fills the device: at 384 rows per
    // expert (DeepSeek-MoE-16B shape) it made the whole step 0.8% faster than
    // the 128-row tile (A/B, three alternations).  The grid of this k-split
    // product is E x ceil(h/256) x ceil(d/256) tiles, whatever the rows.
    err = ksplit_fills(E, h, d, 256) ? launch_gemm_dma<256, 256, 32, 4, 2, 1, false, false, 4, EPI_STORE, bf16_t, 1>(p, s)
                                      : launch_gemm_dma<128, 256, 32, 2, 2, 1, false, false, 3, EPI_STORE, bf16_t, 2>(p, s);
    return err;
}

hipError_t launch_ffn_bwd(int dt, const void *xs, const void *w1, const void *w3, const void *w2, const void *act,
                          const void *h13, const void *dye, const int32_t *offsets, int E, int64_t rows, int d, int h,
                          void *dh13, void *dxs, bool accumulate_dxs, void *dw1, void *dw3, void *dw2, int grad_dt,
                          bool accumulate_dw, hipStream_t s) {
    hipError_t err = launch_ffn_bwd_dact(dt, dye, nullptr, 0, nullptr, w2, h13, offsets, E, rows, d, h, dh13, s);
    if (err == hipSuccess) err = launch_ffn_bwd_dx(dt, dh13, w1, w3, offsets, E, rows, d, h, dxs, accumulate_dxs, s);
    if (err == hipSuccess)
        err = launch_ffn_bwd_dw13(dt, xs, nullptr, 0, dh13, offsets, E, rows, d, h, dw1, dw3, grad_dt, accumulate_dw, s);
    if (err == hipSuccess) err = launch_ffn_bwd_dw2(dt, act, dye, offsets, E, rows, d, h, dw2, grad_dt, accumulate_dw, s);
    return err;
}

}  // namespace xmoe

/*
 * One forward and backward pass of a bf16 padding-free MoE layer (no shared
 * experts) driven from C through libxmoe's C ABI and the HIP runtime's C API
 * alone: the calls a caller without Python makes.
 *
 *   layer_c <inputs> <outputs> T d E h k
 *
 * inputs (raw little-endian arrays, in this order): x [T,d], wg [d,E],
 *   w1 [E,d,h], w3 [E,d,h], w2 [E,h,d], dy [T,d], all bf16 bit patterns.
 * outputs: topk_ids [T,k] int32, topk_w [T,k] fp32, y [T,d] bf16, dx [T,d]
 *   bf16, dw1 [E,d,h], dw3 [E,d,h], dw2 [E,h,d] bf16, dwg [d,E] fp32.
 *
 * The sequence is the padding-free layer's ("5.4 MoE模型在分布式训练中的应用",
 * section 训练流程; X-MoE article, sections 2.1.1-2.1.2): route, build the
 * PFT, the gathered SwiGLU experts, the weighted combine; backward: the
 * combine's backward, dA from dy through the PFT, dX, the weight gradients,
 * the gate's backward and the dispatch backward.  Every call runs on one
 * stream; the program exits non-zero, naming the call, on any error.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "xmoe.h"

#define HIP(c)                                                                    \
    do {                                                                          \
        hipError_t e_ = (c);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s: %s\n", #c, hipGetErrorString(e_));               \
            exit(2);                                                              \
        }                                                                         \
    } while (0)
#define XMOE(c)                                                                   \
    do {                                                                          \
        xmoe_status s_ = (c);                                                     \
        if (s_ != XMOE_OK) {                                                      \
            fprintf(stderr, "%s: status %d: %s\n", #c, (int)s_, xmoe_last_error()); \
            exit(3);                                                              \
        }                                                                         \
    } while (0)

static void *dev(size_t bytes) {
    void *p = NULL;
    HIP(hipMalloc(&p, bytes > 0 ? bytes : 16));
    return p;
}

static void *upload(FILE *f, size_t bytes) {
    void *h = malloc(bytes), *d = dev(bytes);
    if (!h || fread(h, 1, bytes, f) != bytes) {
        fprintf(stderr, "short input file\n");
        exit(4);
    }
    HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    free(h);
    return d;
}

static void download(FILE *f, const void *d, size_t bytes) {
    void *h = malloc(bytes);
    if (!h) exit(4);
    HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    if (fwrite(h, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write outputs\n");
        exit(4);
    }
    free(h);
}

int main(int argc, char **argv) {
    if (argc != 8) {
        fprintf(stderr, "usage: %s inputs outputs T d E h k\n", argv[0]);
        return 1;
    }
    const int64_t T = atoll(argv[3]);
    const int32_t d = atoi(argv[4]), E = atoi(argv[5]), h = atoi(argv[6]), k = atoi(argv[7]);
    const int64_t R = T * k;
    const size_t s = 2; /* bf16 */
    const xmoe_dtype bf = XMOE_BF16;

    FILE *in = fopen(argv[1], "rb");
    if (!in) return 4;
    void *x = upload(in, (size_t)T * d * s), *wg = upload(in, (size_t)d * E * s);
    void *w1 = upload(in, (size_t)E * d * h * s), *w3 = upload(in, (size_t)E * d * h * s);
    void *w2 = upload(in, (size_t)E * h * d * s), *dy = upload(in, (size_t)T * d * s);
    fclose(in);

    hipStream_t st;
    HIP(hipStreamCreate(&st));

    /* forward */
    int32_t *ids = dev((size_t)R * 4);
    float *tw = dev((size_t)R * 4), *logits = dev((size_t)T * E * 4);
    const size_t rws = xmoe_route_workspace_size(T, d, E, bf);
    void *rw = dev(rws);
    XMOE(xmoe_route(x, wg, bf, T, d, E, k, 1.0f, NULL, NULL, ids, tw, logits, rw, rws, st));
    xmoe_pft pft;
    pft.token_ids = dev((size_t)R * 4);
    pft.expert_ids = dev((size_t)R * 4);
    pft.tokens_per_expert = dev((size_t)E * 4);
    pft.expert_offsets = dev((size_t)(E + 1) * 4);
    pft.combine_weights = dev((size_t)R * 4);
    pft.slot_to_row = dev((size_t)R * 4);
    const size_t pws = xmoe_build_pft_workspace_size(T, E, k);
    void *pw = dev(pws);
    XMOE(xmoe_build_pft(ids, tw, T, E, k, &pft, pw, pws, st));
    void *act = dev((size_t)R * h * s), *h13 = dev((size_t)R * 2 * h * s), *ye = dev((size_t)R * d * s);
    void *y = dev((size_t)T * d * s);
    XMOE(xmoe_expert_ffn_up_gather(x, pft.token_ids, w1, w3, bf, pft.expert_offsets, E, T, R, d, h, act, h13, st));
    XMOE(xmoe_expert_ffn_down(act, w2, bf, pft.expert_offsets, E, R, d, h, ye, 0, st));
    XMOE(xmoe_combine(ye, &pft, T, d, k, bf, NULL, y, st));

    /* backward */
    void *dye = dev((size_t)R * d * s);
    float *dtw = dev((size_t)R * 4);
    XMOE(xmoe_combine_bwd(dy, ye, &pft, T, d, k, bf, dye, dtw, st));
    void *dh13 = dev((size_t)R * 2 * h * s), *dxs = dev((size_t)R * d * s);
    void *dw1 = dev((size_t)E * d * h * s), *dw3 = dev((size_t)E * d * h * s), *dw2 = dev((size_t)E * h * d * s);
    XMOE(xmoe_expert_ffn_bwd_dact_gather(dy, pft.token_ids, pft.combine_weights, w2, h13, bf, pft.expert_offsets, E,
                                         T, R, d, h, dh13, st));
    XMOE(xmoe_expert_ffn_bwd_dw2(act, dye, bf, pft.expert_offsets, E, R, d, h, dw2, bf, 0, st));
    XMOE(xmoe_expert_ffn_bwd_dw13_gather(x, pft.token_ids, dh13, bf, pft.expert_offsets, E, T, R, d, h, dw1, dw3, bf,
                                         0, st));
    XMOE(xmoe_expert_ffn_bwd_dx(dh13, w1, w3, bf, pft.expert_offsets, E, R, d, h, dxs, 0, st));
    void *rdx = dev((size_t)T * d * s), *dx = dev((size_t)T * d * s);
    float *dwg = dev((size_t)d * E * 4);
    const size_t bws = xmoe_route_bwd_workspace_size(T, d, E, bf);
    void *bw = dev(bws);
    XMOE(xmoe_route_bwd(x, wg, logits, ids, dtw, k, bf, T, d, E, k, 1.0f, 0, rdx, dwg, bw, bws, st));
    XMOE(xmoe_dispatch_bwd(dxs, &pft, T, d, k, bf, rdx, dx, st));
    HIP(hipStreamSynchronize(st));

    FILE *out = fopen(argv[2], "wb");
    if (!out) return 4;
    download(out, ids, (size_t)R * 4);
    download(out, tw, (size_t)R * 4);
    download(out, y, (size_t)T * d * s);
    download(out, dx, (size_t)T * d * s);
    download(out, dw1, (size_t)E * d * h * s);
    download(out, dw3, (size_t)E * d * h * s);
    download(out, dw2, (size_t)E * h * d * s);
    download(out, dwg, (size_t)d * E * 4);
    fclose(out);
    HIP(hipStreamDestroy(st));
    printf("layer_c ok: T=%lld d=%d E=%d h=%d k=%d\n", (long long)T, d, E, h, k);
    return 0;
}

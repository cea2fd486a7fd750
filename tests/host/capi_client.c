/*
 * A plain C client of include/rgg.h: no Python, no torch.  It reads one
 * workload from a binary file, runs the three entry points on the current
 * HIP device with device memory it allocates itself (and the gate_up
 * projection, fused with GEGLU and alone), and writes the results
 * to another binary file, which tests/test_parity_gpu.py compares with the
 * CPU oracle.
 *
 * Input file, little-endian:
 *   int64 S, B, H, D, R, rows, hidden, M, K, Hp
 *   float freqs[S][B][R]                    (the (S, B, 1, R) angles)
 *   uint16 x[B][S][H][D]                    (bf16 bits)
 *   uint16 gate_up[rows][2 * hidden]        (bf16 bits)
 *   uint16 px[M][K], pw[2 * Hp][K]          (the projection's input and weight)
 * Output file:
 *   uint16 cos[B*S][R], sin[B*S][R], rope[B][S][H][D], geglu[rows][hidden],
 *          fused[M][Hp] (gemm_geglu_bf16), proj[M][2 * Hp] (gemm_bf16_nt)
 *
 * Usage: capi_client IN OUT      (exit status 0 on success)
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "rgg.h"

#define CHECK_HIP(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
            return 2;                                                                \
        }                                                                            \
    } while (0)

#define CHECK_RGG(call)                                                              \
    do {                                                                             \
        int s_ = (call);                                                             \
        if (s_ != RGG_OK) {                                                          \
            fprintf(stderr, "%s: %s\n", #call, rgg_status_string(s_));               \
            return 3;                                                                \
        }                                                                            \
    } while (0)

static int read_all(FILE *f, void *p, size_t n)
{
    return fread(p, 1, n, f) == n;
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 1;
    }
    FILE *in = fopen(argv[1], "rb");
    if (!in)
        return 1;
    int64_t hdr[10];
    if (!read_all(in, hdr, sizeof hdr))
        return 1;
    const int64_t S = hdr[0], B = hdr[1], H = hdr[2], D = hdr[3], R = hdr[4];
    const int64_t rows = hdr[5], hidden = hdr[6], M = hdr[7], K = hdr[8], Hp = hdr[9];
    const size_t n_f = (size_t)(S * B * R), n_x = (size_t)(B * S * H * D);
    const size_t n_t = (size_t)(B * S * R), n_g = (size_t)(rows * 2 * hidden);
    const size_t n_o = (size_t)(rows * hidden);
    const size_t n_px = (size_t)(M * K), n_pw = (size_t)(2 * Hp * K);
    const size_t n_pf = (size_t)(M * Hp), n_pp = (size_t)(M * 2 * Hp);
    const size_t n_out = 2 * n_t + n_x + n_o + n_pf + n_pp;

    float *h_f = malloc(n_f * sizeof(float));
    uint16_t *h_x = malloc(n_x * 2), *h_g = malloc(n_g * 2);
    uint16_t *h_px = malloc(n_px * 2), *h_pw = malloc(n_pw * 2);
    uint16_t *h_out = malloc(n_out * 2);
    if (!h_f || !h_x || !h_g || !h_px || !h_pw || !h_out || !read_all(in, h_f, n_f * 4) ||
        !read_all(in, h_x, n_x * 2) || !read_all(in, h_g, n_g * 2) ||
        !read_all(in, h_px, n_px * 2) || !read_all(in, h_pw, n_pw * 2))
        return 1;
    fclose(in);

    float *d_f;
    uint16_t *d_x, *d_g, *d_cos, *d_sin, *d_rope, *d_geglu, *d_px, *d_pw, *d_pf, *d_pp;
    CHECK_HIP(hipMalloc((void **)&d_f, n_f * 4));
    CHECK_HIP(hipMalloc((void **)&d_x, n_x * 2));
    CHECK_HIP(hipMalloc((void **)&d_g, n_g * 2));
    CHECK_HIP(hipMalloc((void **)&d_cos, n_t * 2));
    CHECK_HIP(hipMalloc((void **)&d_sin, n_t * 2));
    CHECK_HIP(hipMalloc((void **)&d_rope, n_x * 2));
    CHECK_HIP(hipMalloc((void **)&d_geglu, n_o * 2));
    CHECK_HIP(hipMalloc((void **)&d_px, n_px * 2));
    CHECK_HIP(hipMalloc((void **)&d_pw, n_pw * 2));
    CHECK_HIP(hipMalloc((void **)&d_pf, n_pf * 2));
    CHECK_HIP(hipMalloc((void **)&d_pp, n_pp * 2));
    CHECK_HIP(hipMemcpy(d_f, h_f, n_f * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, h_x, n_x * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_g, h_g, n_g * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_px, h_px, n_px * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_pw, h_pw, n_pw * 2, hipMemcpyHostToDevice));

    hipStream_t stream;
    CHECK_HIP(hipStreamCreateWithFlags(&stream, hipStreamNonBlocking));

    /* angles (S, B, 1, R) contiguous: stride_s = B*R, stride_b = R */
    CHECK_RGG(rope_cossin_precompute(d_f, S, B, R, B * R, R, d_cos, d_sin, stream));

    rgg_rope_view view = {d_x, d_rope, S * H * D, H * D, D, S * H * D, H * D, D};
    CHECK_RGG(rope_rotate_half_bf16(&view, 1, B, S, H, D, R, d_cos, d_sin, stream));

    CHECK_RGG(gelu_and_mul_bf16(d_g, rows, hidden, 2 * hidden, d_geglu, hidden, stream));

    /* x (M, K) and W (2 Hp, K) contiguous; outputs (M, Hp) and (M, 2 Hp) */
    CHECK_RGG(gemm_geglu_bf16(d_px, M, K, K, d_pw, Hp, K, d_pf, Hp, stream));
    CHECK_RGG(gemm_bf16_nt(d_px, M, K, K, d_pw, 2 * Hp, K, d_pp, 2 * Hp, stream));

    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(h_out, d_cos, n_t * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_out + n_t, d_sin, n_t * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_out + 2 * n_t, d_rope, n_x * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_out + 2 * n_t + n_x, d_geglu, n_o * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_out + 2 * n_t + n_x + n_o, d_pf, n_pf * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_out + 2 * n_t + n_x + n_o + n_pf, d_pp, n_pp * 2,
                        hipMemcpyDeviceToHost));

    FILE *out = fopen(argv[2], "wb");
    if (!out || fwrite(h_out, 2, n_out, out) != n_out)
        return 1;
    fclose(out);

    CHECK_HIP(hipStreamDestroy(stream));
    hipFree(d_f);
    hipFree(d_x);
    hipFree(d_g);
    hipFree(d_cos);
    hipFree(d_sin);
    hipFree(d_rope);
    hipFree(d_geglu);
    hipFree(d_px);
    hipFree(d_pw);
    hipFree(d_pf);
    hipFree(d_pp);
    free(h_f);
    free(h_x);
    free(h_g);
    free(h_px);
    free(h_pw);
    free(h_out);
    printf("capi_client: ok\n");
    return 0;
}

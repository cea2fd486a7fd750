// The host layer of the C ABI (capi.cpp, selfcheck.cpp, layout.h) built for
// the CPU under AddressSanitizer and UndefinedBehaviorSanitizer, with the
// kernel launchers and the handful of HIP runtime calls it makes replaced by
// recording stubs.  Every entry point is driven through its argument checks
// (each status the header promises) and through valid calls that reach a
// launcher, whose parameter block is then checked.  The self-check runs over
// a host buffer standing in for its workspace: no kernel runs, so it must
// report failures, and it must do so without any memory error.
//
// Prints "ok" and exits 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include <hip/hip_runtime_api.h>

#include "launch.h"
#include "rgg.h"
#include "selfcheck.h"

// ---------------------------------------------------------------------------
// stubs: the HIP runtime calls of the host layer, and the kernel launchers
// ---------------------------------------------------------------------------
static int g_launches = 0;
static rgg::RopeParams g_rope;
static rgg::GegluParams g_geglu;
static rgg::GemmParams g_gemm;
static bool g_gemm_geglu = false;
static rgg::CosSinParams g_cossin;
static rgg::CosSinGridParams g_grid;
static hipStreamCaptureStatus g_capture = hipStreamCaptureStatusNone;

extern "C" {
hipError_t hipGetDevice(int *d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int)
{
    *v = 256;
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *s)
{
    *s = g_capture;
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t)
{
    memcpy(dst, src, n);
    return hipSuccess;
}
}

namespace rgg {
hipError_t launch_rope_cossin(const CosSinParams &p, hipStream_t)
{
    g_cossin = p;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_rope_cossin_grid(const CosSinGridParams &p, hipStream_t)
{
    g_grid = p;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_rope_rotate_half(const RopeParams &p, hipStream_t)
{
    g_rope = p;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_gelu_and_mul(const GegluParams &p, int, hipStream_t)
{
    g_geglu = p;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_gemm_gate_up(const GemmParams &p, bool geglu, hipStream_t)
{
    g_gemm = p;
    g_gemm_geglu = geglu;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_build_gelu_table(hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
int geglu_grid(uint32_t vec_total, int) { return (int)((vec_total + 511) / 512); }
int noalloc_prepare(int) { return 0; }
}  // namespace rgg

// ---------------------------------------------------------------------------
static int g_fail = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                             \
        }                                                                         \
    } while (0)

// Fake device addresses: 16-byte aligned, never dereferenced by the host layer.
static uint16_t *fake(uintptr_t off) { return reinterpret_cast<uint16_t *>((uintptr_t)0x7F0000000000ull + off); }

static int rope(int n_views, int64_t B, int64_t S, int64_t H, int64_t D, int64_t R,
                const rgg_rope_view *v, const uint16_t *cs, const uint16_t *sn)
{
    return rope_rotate_half_bf16(v, n_views, B, S, H, D, R, cs, sn, nullptr);
}

static void check_rope()
{
    const int64_t B = 2, S = 16, H = 4, D = 64;
    const int64_t sb = S * H * D, ss = H * D, sh = D;
    uint16_t *cs = fake(1 << 24), *sn = fake(2 << 24);
    rgg_rope_view v = {fake(0), fake(1 << 20), sb, ss, sh, sb, ss, sh};
    // shape, pointer, alignment, alias checks
    EXPECT(rope(0, B, S, H, D, 32, &v, cs, sn) == RGG_ERR_SHAPE);
    EXPECT(rope(5, B, S, H, D, 32, &v, cs, sn) == RGG_ERR_SHAPE);
    EXPECT(rope(1, B, S, H, D, 33, &v, cs, sn) == RGG_ERR_SHAPE);
    EXPECT(rope(1, B, S, H, D, 72, &v, cs, sn) == RGG_ERR_SHAPE);
    EXPECT(rope(1, -1, S, H, D, 32, &v, cs, sn) == RGG_ERR_SHAPE);
    EXPECT(rope(1, B, S, H, D, 24, &v, cs, sn) == RGG_ERR_UNSUPPORTED);
    EXPECT(rope(1, B, S, H, 60, 32, &v, cs, sn) == RGG_ERR_UNSUPPORTED);
    EXPECT(rope(1, B, S, H, D, 32, nullptr, cs, sn) == RGG_ERR_NULL);
    EXPECT(rope(1, B, S, H, D, 32, &v, nullptr, sn) == RGG_ERR_NULL);
    rgg_rope_view w = v;
    w.x = fake(2);
    EXPECT(rope(1, B, S, H, D, 32, &w, cs, sn) == RGG_ERR_ALIGN);
    w = v;
    w.x_stride_h = 68;
    EXPECT(rope(1, B, S, H, D, 32, &w, cs, sn) == RGG_ERR_ALIGN);
    w = v;
    w.out = fake(4096);   // output inside the input
    EXPECT(rope(1, B, S, H, D, 32, &w, cs, sn) == RGG_ERR_ALIAS);
    w = v;
    w.out = cs;           // output over the cos table
    EXPECT(rope(1, B, S, H, D, 32, &w, cs, sn) == RGG_ERR_ALIAS);
    w = v;
    w.out_stride_h = 32;  // output rows overlap themselves
    EXPECT(rope(1, B, S, H, D, 32, &w, cs, sn) == RGG_ERR_UNSUPPORTED);
    EXPECT(rope(1, 0, S, H, D, 32, &v, cs, sn) == RGG_OK);

    // q and k as strided views of one fused qkv buffer, written to separate
    // outputs: reaches the launcher with both views and their tails
    const int64_t row = 3 * H * D;
    rgg_rope_view qk[2] = {{fake(0), fake(1 << 22), S * row, row, D, sb, ss, sh},
                           {fake(H * D * 2), fake(1 << 23), S * row, row, D, sb, ss, sh}};
    int n0 = g_launches;
    EXPECT(rope(2, B, S, H, D, 32, qk, cs, sn) == RGG_OK);
    EXPECT(g_launches == n0 + 1);
    EXPECT(g_rope.n_views == 2 && g_rope.tokens == B * S && g_rope.R == 32 && g_rope.D == D);
    EXPECT(g_rope.tail_mask == 3);
    EXPECT(g_rope.v[1].x == qk[1].x && g_rope.v[1].xs_s == row);
    // the same views in place: no tail to copy
    rgg_rope_view ip[2] = {qk[0], qk[1]};
    ip[0].out = const_cast<uint16_t *>(ip[0].x);
    ip[1].out = const_cast<uint16_t *>(ip[1].x);
    ip[0].out_stride_b = ip[1].out_stride_b = S * row;
    ip[0].out_stride_s = ip[1].out_stride_s = row;
    ip[0].out_stride_h = ip[1].out_stride_h = D;
    EXPECT(rope(2, B, S, H, D, 32, ip, cs, sn) == RGG_OK);
    EXPECT(g_rope.tail_mask == 0);
    // k written over q's input: refused
    rgg_rope_view bad[2] = {qk[0], qk[1]};
    bad[1].out = const_cast<uint16_t *>(qk[0].x);
    bad[1].out_stride_b = S * row;
    bad[1].out_stride_s = row;
    EXPECT(rope(2, B, S, H, D, 32, bad, cs, sn) == RGG_ERR_ALIAS);
}

static void check_geglu()
{
    uint16_t *in = fake(0), *out = fake(1 << 24);
    EXPECT(gelu_and_mul_bf16(in, -1, 64, 128, out, 64, nullptr) == RGG_ERR_SHAPE);
    EXPECT(gelu_and_mul_bf16(in, 8, 60, 120, out, 64, nullptr) == RGG_ERR_UNSUPPORTED);
    EXPECT(gelu_and_mul_bf16(in, 8, 64, 128, out, 56, nullptr) == RGG_ERR_UNSUPPORTED);
    EXPECT(gelu_and_mul_bf16(nullptr, 8, 64, 128, out, 64, nullptr) == RGG_ERR_NULL);
    EXPECT(gelu_and_mul_bf16(fake(8), 8, 64, 128, out, 64, nullptr) == RGG_ERR_ALIGN);
    EXPECT(gelu_and_mul_bf16(in, 8, 64, 132, out, 64, nullptr) == RGG_ERR_ALIGN);
    EXPECT(gelu_and_mul_bf16(in, 8, 64, 128, fake(64), 64, nullptr) == RGG_ERR_ALIAS);
    EXPECT(gelu_and_mul_bf16(in, 0, 64, 128, out, 64, nullptr) == RGG_OK);
    // the first call builds the table (one launch), then the kernel
    int n0 = g_launches;
    EXPECT(gelu_and_mul_bf16(in, 8, 64, 128, out, 64, nullptr) == RGG_OK);
    EXPECT(g_launches == n0 + 2);
    EXPECT(g_geglu.vec_total == 8 * 64 / 8 && g_geglu.hidden == 64 && g_geglu.in_stride == 128);
    // in place over the gate half
    EXPECT(gelu_and_mul_bf16(in, 8, 64, 128, in, 128, nullptr) == RGG_OK);
    EXPECT(g_launches == n0 + 3);
}

static void check_tables()
{
    float *f = reinterpret_cast<float *>(fake(0));
    uint16_t *c = fake(1 << 20), *s = fake(2 << 20);
    EXPECT(rope_cossin_precompute(f, 4, 2, 12, 16, 8, c, s, nullptr) == RGG_ERR_UNSUPPORTED);
    EXPECT(rope_cossin_precompute(f, -1, 2, 8, 16, 8, c, s, nullptr) == RGG_ERR_SHAPE);
    EXPECT(rope_cossin_precompute(nullptr, 4, 2, 8, 16, 8, c, s, nullptr) == RGG_ERR_NULL);
    EXPECT(rope_cossin_precompute(f, 4, 2, 8, 18, 8, c, s, nullptr) == RGG_ERR_ALIGN);
    EXPECT(rope_cossin_precompute(f, 4, 2, 8, 16, 8, c, c + 8, nullptr) == RGG_ERR_ALIAS);
    EXPECT(rope_cossin_precompute(f, 4, 2, 16, 32, 16, c, s, nullptr) == RGG_OK);
    EXPECT(g_cossin.vec_total == 4 * 2 * 16 / 8 && g_cossin.R == 16 && g_cossin.stride_s == 32);

    EXPECT(rope_cossin_from_grid(2, 1, 4, 4, 3, 6, 7, 1e4, nullptr, c, s, nullptr) == RGG_ERR_SHAPE);
    EXPECT(rope_cossin_from_grid(2, 1, 4, 4, 4, 6, 4, 1e4, nullptr, c, s, nullptr) ==
           RGG_ERR_UNSUPPORTED);
    EXPECT(rope_cossin_from_grid(2, 1, 4, 4, 4, 6, 6, -1.0, nullptr, c, s, nullptr) == RGG_ERR_SHAPE);
    EXPECT(rope_cossin_from_grid(2, 1, 4, 4, 8, 12, 12, 1e4, nullptr, c, c + 8, nullptr) ==
           RGG_ERR_ALIAS);
    EXPECT(rope_cossin_from_grid(2, 1, 4, 4, 8, 12, 12, 1e4, nullptr, c, s, nullptr) == RGG_OK);
    EXPECT(g_grid.R == 32 && g_grid.h0 == 4 && g_grid.h01 == 10 && g_grid.host_omega == 1);
    EXPECT(g_grid.omega[0] == 1.0 && g_grid.omega[4] == 1.0 && g_grid.omega[10] == 1.0);
    // wider than the argument block: frequencies evaluated on the device
    EXPECT(rope_cossin_from_grid(1, 1, 2, 2, 352, 352, 320, 1e4, nullptr, c, s, nullptr) == RGG_OK);
    EXPECT(g_grid.host_omega == 0 && g_grid.R == 1024);
}

static void check_gemm()
{
    uint16_t *x = fake(0), *w = fake(1 << 24), *o = fake(2 << 24);
    EXPECT(gemm_geglu_bf16(x, 8, 128, 128, w, 64, 128, o, 64, nullptr) == RGG_OK);
    EXPECT(g_gemm_geglu && g_gemm.M == 8 && g_gemm.K == 128 && g_gemm.H == 64 &&
           g_gemm.mblocks == 1 && g_gemm.nblocks == 1);
    EXPECT(gemm_bf16_nt(x, 300, 128, 128, w, 256, 128, o, 256, nullptr) == RGG_OK);
    EXPECT(!g_gemm_geglu && g_gemm.H == 128 && g_gemm.mblocks == 2);
    EXPECT(gemm_bf16_nt(x, 8, 128, 128, w, 192, 128, o, 192, nullptr) == RGG_ERR_UNSUPPORTED);
    EXPECT(gemm_geglu_bf16(x, 8, 100, 128, w, 64, 128, o, 64, nullptr) == RGG_ERR_UNSUPPORTED);
    EXPECT(gemm_geglu_bf16(x, 8, 128, 128, w, 64, 128, fake(64), 64, nullptr) == RGG_ERR_ALIAS);
    EXPECT(gemm_geglu_bf16(x, 8, 128, 128, nullptr, 64, 128, o, 64, nullptr) == RGG_ERR_NULL);
    EXPECT(gemm_geglu_bf16(x, 8, 128, 132, w, 64, 128, o, 64, nullptr) == RGG_ERR_ALIGN);
}

static void check_selfcheck()
{
    // A host buffer stands in for the device workspace: the stubbed launches
    // compute nothing, so the comparisons must report failures.
    std::vector<uint8_t> ws(RGG_SELFCHECK_WORKSPACE_BYTES + 256);
    void *p = reinterpret_cast<void *>(((uintptr_t)ws.data() + 255) & ~(uintptr_t)255);
    uint32_t failed = 0;
    EXPECT(rgg_selfcheck(nullptr, RGG_SELFCHECK_WORKSPACE_BYTES, nullptr, &failed) == RGG_ERR_NULL);
    EXPECT(rgg_selfcheck(p, RGG_SELFCHECK_WORKSPACE_BYTES - 1, nullptr, &failed) == RGG_ERR_SHAPE);
    g_capture = hipStreamCaptureStatusActive;
    EXPECT(rgg_selfcheck(p, RGG_SELFCHECK_WORKSPACE_BYTES, nullptr, &failed) == RGG_ERR_CAPTURING);
    g_capture = hipStreamCaptureStatusNone;
    EXPECT(rgg_selfcheck(p, RGG_SELFCHECK_WORKSPACE_BYTES, nullptr, &failed) == RGG_ERR_SELFCHECK);
    EXPECT(failed != 0);
}

int main()
{
    for (int code = 0; code < 9; ++code)
        EXPECT(strcmp(rgg_status_string(code), "unknown status") != 0);
    check_rope();
    check_geglu();
    check_tables();
    check_gemm();
    check_selfcheck();
    EXPECT(rgg_prepare_device(-1) == RGG_ERR_SHAPE);
    EXPECT(rgg_prepare_device(0) == RGG_OK);
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("ok\n");
    return 0;
}

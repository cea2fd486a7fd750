// C ABI of the fused RoPE / GEGLU path: argument checks, overlap analysis,
// per-device set-up, and the kernel launches (declared in include/rgg.h).
//
// Every check runs on the host before anything is enqueued; a failing check
// returns its status and touches no device state.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>

#include <hip/hip_runtime_api.h>

#include "launch.h"
#include "layout.h"
#include "rgg.h"
#include "selfcheck.h"

namespace {

using rgg::FastDiv;
using rgg::make_fastdiv;
using rgg::Layout;
using rgg::make_layout;
using rgg::may_overlap;
using rgg::rows_disjoint;

constexpr int64_t kMax32 = (int64_t)1 << 31;  // index math in the kernels is 32-bit

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// ---------------------------------------------------------------------------
// per-device state: compute-unit count and the GELU table
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;

struct DeviceState {
    std::mutex lock;
    std::atomic<int> table_ready{0};
    std::atomic<int> cus{0};
};

DeviceState g_devices[kMaxDevices];

int current_device(int &dev)
{
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return RGG_ERR_HIP;
    return RGG_OK;
}

int cu_count(int dev)
{
    int c = g_devices[dev].cus.load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        g_devices[dev].cus.store(c, std::memory_order_relaxed);
    }
    return c;
}

// Builds the GELU table of the current device `dev` on `stream` and waits.
int ensure_table(int dev, hipStream_t stream)
{
    DeviceState &d = g_devices[dev];
    if (d.table_ready.load(std::memory_order_acquire))
        return RGG_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess)
        return RGG_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone)
        return RGG_ERR_CAPTURING;
    std::lock_guard<std::mutex> g(d.lock);
    if (d.table_ready.load(std::memory_order_acquire))
        return RGG_OK;
    if (rgg::launch_build_gelu_table(stream) != hipSuccess)
        return RGG_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess)
        return RGG_ERR_HIP;
    d.table_ready.store(1, std::memory_order_release);
    return RGG_OK;
}

}  // namespace

extern "C" {

const char *rgg_status_string(int status)
{
    switch (status) {
    case RGG_OK:
        return "ok";
    case RGG_ERR_NULL:
        return "a required pointer is NULL";
    case RGG_ERR_SHAPE:
        return "invalid shape, stride or view count";
    case RGG_ERR_UNSUPPORTED:
        return "layout outside the 8-element vector contract";
    case RGG_ERR_ALIGN:
        return "pointer not 16-byte aligned or stride not a multiple of the vector";
    case RGG_ERR_ALIAS:
        return "an output overlaps an input or another output";
    case RGG_ERR_HIP:
        return "HIP runtime error";
    case RGG_ERR_CAPTURING:
        return "GELU table not built on this device and the stream is capturing; "
               "call rgg_prepare_device first";
    case RGG_ERR_SELFCHECK:
        return "device self-check: a result differs from its expected bits";
    default:
        return "unknown status";
    }
}

int rope_cossin_precompute(const float *freqs, int64_t S, int64_t B, int64_t R,
                           int64_t stride_s, int64_t stride_b, uint16_t *cos_out,
                           uint16_t *sin_out, hipStream_t stream)
{
    if (S < 0 || B < 0 || R < 0 || stride_s < 0 || stride_b < 0)
        return RGG_ERR_SHAPE;
    if (R % 8 != 0)
        return RGG_ERR_UNSUPPORTED;
    if (S == 0 || B == 0 || R == 0)
        return RGG_OK;
    if (!freqs || !cos_out || !sin_out)
        return RGG_ERR_NULL;
    if (!aligned16(freqs) || !aligned16(cos_out) || !aligned16(sin_out) || stride_s % 4 != 0 ||
        stride_b % 4 != 0)
        return RGG_ERR_ALIGN;
    if (S * B >= kMax32 || S * B * (R / 4) >= kMax32)
        return RGG_ERR_UNSUPPORTED;

    const int64_t fn[2] = {S, B}, fst[2] = {stride_s, stride_b};
    const int64_t tn[1] = {B * S}, tst[1] = {R};
    Layout lf = make_layout(freqs, 4, 2, fn, fst, R);
    Layout lc = make_layout(cos_out, 2, 1, tn, tst, R);
    Layout ls = make_layout(sin_out, 2, 1, tn, tst, R);
    if (may_overlap(lc, ls) || may_overlap(lc, lf) || may_overlap(ls, lf))
        return RGG_ERR_ALIAS;

    rgg::CosSinParams p;
    p.freqs = freqs;
    p.cos = cos_out;
    p.sin = sin_out;
    p.stride_s = stride_s;
    p.stride_b = stride_b;
    p.vec_total = (uint32_t)(S * B * (R / 8));
    p.R = (int32_t)R;
    p.div_vecs = make_fastdiv((uint32_t)(R / 8));
    p.div_s = make_fastdiv((uint32_t)S);
    return rgg::launch_rope_cossin(p, stream) == hipSuccess ? RGG_OK : RGG_ERR_HIP;
}

int rope_cossin_from_grid(int64_t B, int64_t T, int64_t Hg, int64_t Wg, int32_t d0, int32_t d1,
                          int32_t d2, double theta, const int32_t *t_offset, uint16_t *cos_out,
                          uint16_t *sin_out, hipStream_t stream)
{
    if (B < 0 || T < 0 || Hg < 0 || Wg < 0 || d0 < 0 || d1 < 0 || d2 < 0 || d0 % 2 || d1 % 2 ||
        d2 % 2 || !(theta > 0.0) || !std::isfinite(theta))
        return RGG_ERR_SHAPE;
    const int64_t R = (int64_t)d0 + d1 + d2;
    if (R % 16 != 0 || R > 8192)
        return RGG_ERR_UNSUPPORTED;
    if (B == 0 || T == 0 || Hg == 0 || Wg == 0 || R == 0)
        return RGG_OK;
    if (T >= kMax32 || Hg >= kMax32 || Wg >= kMax32 || T * Hg >= kMax32 || T * Hg * Wg >= kMax32)
        return RGG_ERR_UNSUPPORTED;
    const int64_t S = T * Hg * Wg;
    if (B * S >= kMax32 || B * S * (R / 16) >= kMax32)
        return RGG_ERR_UNSUPPORTED;
    if (!cos_out || !sin_out)
        return RGG_ERR_NULL;
    if (!aligned16(cos_out) || !aligned16(sin_out) || ((uintptr_t)t_offset & 3))
        return RGG_ERR_ALIGN;
    const int64_t tn[1] = {B * S}, tst[1] = {R};
    Layout lc = make_layout(cos_out, 2, 1, tn, tst, R);
    Layout ls = make_layout(sin_out, 2, 1, tn, tst, R);
    if (may_overlap(lc, ls))
        return RGG_ERR_ALIAS;
    if (t_offset) {
        const int64_t on[1] = {1}, ost[1] = {0};
        Layout lt = make_layout(t_offset, 4, 1, on, ost, B);
        if (may_overlap(lc, lt) || may_overlap(ls, lt))
            return RGG_ERR_ALIAS;
    }

    rgg::CosSinGridParams p;
    memset(&p, 0, sizeof p);
    p.t_offset = t_offset;
    p.cos = cos_out;
    p.sin = sin_out;
    p.theta = theta;
    p.rows = (uint32_t)(B * S);
    p.R = (int32_t)R;
    p.h0 = d0 / 2;
    p.h01 = (d0 + d1) / 2;
    p.d[0] = d0;
    p.d[1] = d1;
    p.d[2] = d2;
    p.div_s = make_fastdiv((uint32_t)S);
    p.div_hw = make_fastdiv((uint32_t)(Hg * Wg));
    p.div_w = make_fastdiv((uint32_t)Wg);
    p.host_omega = R / 2 <= rgg::kGridOmegaArgs;
    if (p.host_omega) {
        const int32_t d[3] = {d0, d1, d2};
        int c = 0;
        for (int k = 0; k < 3; ++k)
            for (int32_t i = 0; i < d[k] / 2; ++i)
                p.omega[c++] = std::pow(theta, -2.0 * i / d[k]);
    }
    return rgg::launch_rope_cossin_grid(p, stream) == hipSuccess ? RGG_OK : RGG_ERR_HIP;
}

int rope_rotate_half_bf16(const rgg_rope_view *views, int n_views, int64_t B, int64_t S,
                          int64_t H, int64_t D, int64_t R, const uint16_t *cos,
                          const uint16_t *sin, hipStream_t stream)
{
    if (n_views < 1 || n_views > rgg::kMaxViews || B < 0 || S < 0 || H < 0 || D <= 0 || R < 0 ||
        R > D || R % 2 != 0)
        return RGG_ERR_SHAPE;
    if (!views)
        return RGG_ERR_NULL;
    for (int v = 0; v < n_views; ++v) {
        const rgg_rope_view &V = views[v];
        if (V.x_stride_b < 0 || V.x_stride_s < 0 || V.x_stride_h < 0 || V.out_stride_b < 0 ||
            V.out_stride_s < 0 || V.out_stride_h < 0)
            return RGG_ERR_SHAPE;
    }
    if (D % 8 != 0 || R % 16 != 0)
        return RGG_ERR_UNSUPPORTED;
    if (B == 0 || S == 0 || H == 0)
        return RGG_OK;
    if (B * S >= kMax32 || D > 8192 || H * D >= kMax32 / 64)
        return RGG_ERR_UNSUPPORTED;
    if (R > 0 && (!cos || !sin))
        return RGG_ERR_NULL;
    if (R > 0 && (!aligned16(cos) || !aligned16(sin)))
        return RGG_ERR_ALIGN;

    const int64_t n3[3] = {B, S, H};
    Layout lx[rgg::kMaxViews], lo[rgg::kMaxViews];
    bool in_place[rgg::kMaxViews];
    for (int v = 0; v < n_views; ++v) {
        const rgg_rope_view &V = views[v];
        if (!V.x || !V.out)
            return RGG_ERR_NULL;
        if (!aligned16(V.x) || !aligned16(V.out) || V.x_stride_b % 8 || V.x_stride_s % 8 ||
            V.x_stride_h % 8 || V.out_stride_b % 8 || V.out_stride_s % 8 || V.out_stride_h % 8)
            return RGG_ERR_ALIGN;
        const int64_t xs[3] = {V.x_stride_b, V.x_stride_s, V.x_stride_h};
        const int64_t os[3] = {V.out_stride_b, V.out_stride_s, V.out_stride_h};
        lx[v] = make_layout(V.x, 2, 3, n3, xs, D);
        lo[v] = make_layout(V.out, 2, 3, n3, os, D);
        if (!rows_disjoint(lo[v]))
            return RGG_ERR_UNSUPPORTED;
        in_place[v] = V.x == V.out && V.x_stride_b == V.out_stride_b &&
                      V.x_stride_s == V.out_stride_s && V.x_stride_h == V.out_stride_h;
    }
    if (R > 0) {
        const int64_t tn[1] = {B * S}, tst[1] = {R};
        Layout lc = make_layout(cos, 2, 1, tn, tst, R);
        Layout ls = make_layout(sin, 2, 1, tn, tst, R);
        for (int v = 0; v < n_views; ++v)
            if (may_overlap(lo[v], lc) || may_overlap(lo[v], ls))
                return RGG_ERR_ALIAS;
    }
    for (int v = 0; v < n_views; ++v) {
        for (int w = 0; w < n_views; ++w) {
            if (w == v ? !in_place[v] && may_overlap(lo[v], lx[w]) : may_overlap(lo[v], lx[w]))
                return RGG_ERR_ALIAS;
            if (w > v && may_overlap(lo[v], lo[w]))
                return RGG_ERR_ALIAS;
        }
    }

    rgg::RopeParams p;
    memset(&p, 0, sizeof p);
    p.tail_mask = 0;
    for (int v = 0; v < n_views; ++v) {
        const rgg_rope_view &V = views[v];
        p.v[v] = rgg::RopeView{V.x, V.out, V.x_stride_b, V.x_stride_s, V.x_stride_h,
                               V.out_stride_b, V.out_stride_s, V.out_stride_h};
        if (!in_place[v])
            p.tail_mask |= 1 << v;
    }
    p.cos = cos;
    p.sin = sin;
    p.tokens = B * S;
    p.n_views = n_views;
    p.H = (int32_t)H;
    p.D = (int32_t)D;
    p.R = (int32_t)R;
    p.half = (int32_t)(R / 2);
    p.slots_tail = (int32_t)(R / 16 + (D - R) / 8);
    p.div_s = make_fastdiv((uint32_t)S);
    p.div_heads = make_fastdiv((uint32_t)H);
    p.div_slots = make_fastdiv(R >= 16 ? (uint32_t)(R / 16) : 1u);
    p.div_slots_tail = make_fastdiv((uint32_t)p.slots_tail);
    if (R == 0 && p.tail_mask == 0)
        return RGG_OK;
    return rgg::launch_rope_rotate_half(p, stream) == hipSuccess ? RGG_OK : RGG_ERR_HIP;
}

namespace {

// Shared checks of the two projection entry points; `H` is half the
// projection width (the gate/up split), `out_cols` the output row width.
int gemm_checks(const uint16_t *x, int64_t M, int64_t K, int64_t x_stride, const uint16_t *w,
                int64_t H, int64_t w_stride, const uint16_t *out, int64_t out_cols,
                int64_t out_stride, rgg::GemmParams &p)
{
    if (M < 0 || K < 0 || H < 0 || x_stride < 0 || w_stride < 0 || out_stride < 0)
        return RGG_ERR_SHAPE;
    if (K % 64 != 0 || H % 64 != 0)
        return RGG_ERR_UNSUPPORTED;
    if ((M > 1 && x_stride < K) || (H > 0 && w_stride < K) || (M > 1 && out_stride < out_cols))
        return RGG_ERR_UNSUPPORTED;
    if (M == 0 || H == 0)
        return -1;  // nothing to do
    if (!out || (K > 0 && (!x || !w)))
        return RGG_ERR_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(out) || x_stride % 8 || w_stride % 8 ||
        out_stride % 8)
        return RGG_ERR_ALIGN;
    const int64_t mblocks = (M + 255) / 256, nblocks = (H + 127) / 128;
    if (M >= kMax32 || K >= kMax32 || mblocks * nblocks >= ((int64_t)1 << 24) || H >= kMax32 / 2 ||
        x_stride >= ((int64_t)1 << 22) || w_stride >= ((int64_t)1 << 22))
        return RGG_ERR_UNSUPPORTED;
    if (K > 0) {
        const int64_t xn[1] = {M}, xs[1] = {x_stride}, wn[1] = {2 * H}, ws[1] = {w_stride};
        const int64_t on[1] = {M}, os[1] = {out_stride};
        Layout lx = make_layout(x, 2, 1, xn, xs, K);
        Layout lw = make_layout(w, 2, 1, wn, ws, K);
        Layout lo = make_layout(out, 2, 1, on, os, out_cols);
        if (may_overlap(lo, lx) || may_overlap(lo, lw))
            return RGG_ERR_ALIAS;
    }
    memset(&p, 0, sizeof p);
    p.x = x;
    p.w = w;
    p.out = const_cast<uint16_t *>(out);
    p.x_stride = x_stride;
    p.w_stride = w_stride;
    p.out_stride = out_stride;
    p.M = M;
    p.H = (int32_t)H;
    p.K = (int32_t)K;
    p.mblocks = (uint32_t)mblocks;
    p.nblocks = (uint32_t)nblocks;
    return RGG_OK;
}

}  // namespace

int gemm_bf16_nt(const uint16_t *x, int64_t M, int64_t K, int64_t x_stride, const uint16_t *w,
                 int64_t N, int64_t w_stride, uint16_t *out, int64_t out_stride,
                 hipStream_t stream)
{
    if (N < 0)
        return RGG_ERR_SHAPE;
    if (N % 128 != 0)
        return RGG_ERR_UNSUPPORTED;
    rgg::GemmParams p;
    int st = gemm_checks(x, M, K, x_stride, w, N / 2, w_stride, out, N, out_stride, p);
    if (st != RGG_OK)
        return st < 0 ? RGG_OK : st;
    return rgg::launch_gemm_gate_up(p, false, stream) == hipSuccess ? RGG_OK : RGG_ERR_HIP;
}

int gemm_geglu_bf16(const uint16_t *x, int64_t M, int64_t K, int64_t x_stride, const uint16_t *w,
                    int64_t H, int64_t w_stride, uint16_t *out, int64_t out_stride,
                    hipStream_t stream)
{
    rgg::GemmParams p;
    int st = gemm_checks(x, M, K, x_stride, w, H, w_stride, out, H, out_stride, p);
    if (st != RGG_OK)
        return st < 0 ? RGG_OK : st;
    int dev;
    if (current_device(dev) != RGG_OK)
        return RGG_ERR_HIP;
    st = ensure_table(dev, stream);
    if (st != RGG_OK)
        return st;
    return rgg::launch_gemm_gate_up(p, true, stream) == hipSuccess ? RGG_OK : RGG_ERR_HIP;
}

int gelu_and_mul_bf16(const uint16_t *input, int64_t rows, int64_t hidden, int64_t in_row_stride,
                      uint16_t *out, int64_t out_row_stride, hipStream_t stream)
{
    if (rows < 0 || hidden < 0 || in_row_stride < 0 || out_row_stride < 0)
        return RGG_ERR_SHAPE;
    if (hidden % 8 != 0)
        return RGG_ERR_UNSUPPORTED;
    if (rows > 1 && out_row_stride < hidden)
        return RGG_ERR_UNSUPPORTED;
    if (rows == 0 || hidden == 0)
        return RGG_OK;
    if (!input || !out)
        return RGG_ERR_NULL;
    if (!aligned16(input) || !aligned16(out) || in_row_stride % 8 || out_row_stride % 8)
        return RGG_ERR_ALIGN;
    if (rows * (hidden / 8) >= kMax32)
        return RGG_ERR_UNSUPPORTED;

    const int64_t rn[1] = {rows};
    const int64_t is[1] = {in_row_stride}, os[1] = {out_row_stride};
    Layout li = make_layout(input, 2, 1, rn, is, 2 * hidden);
    Layout lo = make_layout(out, 2, 1, rn, os, hidden);
    bool in_place = out == input && out_row_stride == in_row_stride;
    if (!in_place && may_overlap(lo, li))
        return RGG_ERR_ALIAS;

    int dev;
    if (current_device(dev) != RGG_OK)
        return RGG_ERR_HIP;
    int st = ensure_table(dev, stream);
    if (st != RGG_OK)
        return st;

    rgg::GegluParams p;
    p.in = input;
    p.out = out;
    p.in_stride = in_row_stride;
    p.out_stride = out_row_stride;
    p.vec_total = (uint32_t)(rows * (hidden / 8));
    p.hidden = (int32_t)hidden;
    p.div_vecs = make_fastdiv((uint32_t)(hidden / 8));
    int grid = rgg::geglu_grid(p.vec_total, cu_count(dev));
    return rgg::launch_gelu_and_mul(p, grid, stream) == hipSuccess ? RGG_OK : RGG_ERR_HIP;
}

int rgg_prepare_device(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return RGG_ERR_SHAPE;
    int prev;
    if (hipGetDevice(&prev) != hipSuccess)
        return RGG_ERR_HIP;
    if (hipSetDevice(device) != hipSuccess)
        return RGG_ERR_HIP;
    int st = ensure_table(device, nullptr);
    if (st == RGG_OK)
        st = rgg::noalloc_prepare(device);
    if (hipSetDevice(prev) != hipSuccess && st == RGG_OK)
        st = RGG_ERR_HIP;
    return st;
}

}  // extern "C"

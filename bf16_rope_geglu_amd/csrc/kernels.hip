// HIP kernels of the fused elementwise path for gfx950 (MI355X, CDNA4).
//
// Method: "[sglang] ERNIE-Image의 RoPE와 GELU-mul 융합 및 RoPE cos/sin 호이스팅을
// 통한 성능 최적화" (blog.secrett2633.cloud, analysis of sglang PR 34306),
// cited as [ERNIE-fuse] with its section.
//
// Every kernel here is HBM-bound elementwise work: no matrix cores.  They move
// data in 16-byte (8 x bf16) vectors per lane so that a wave64 load or store
// covers whole cache lines, run 256-thread workgroups (four wave64s), and
// round every eager bf16 op with the hardware's round-to-nearest-even
// v_cvt_pk_bf16_f32.  IEEE fp32 subnormals are kept (the default denormal
// mode of gfx950 code objects) and nothing is contracted into an FMA across a
// rounding point (the bf16 rounding sits between every multiply and add, and
// the file is built with -ffp-contract=off).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace rgg {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f)
{
    return (__umulhi(n, f.m) + n) >> f.l;
}

// bf16 bits (low / high half of a 32-bit word) widened to fp32, exactly.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two fp32 values to bf16 (nearest even) and pack: lo -> bits 0..15.
__device__ __forceinline__ uint32_t rne_pack(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Round a double to bf16 (nearest even), exactly: truncate to fp32 and fold
// any discarded bits into the fp32 sticky bit ("round to odd", valid since
// fp32 keeps 24 >= 8 + 2 significant bits), then round that fp32 to bf16.
__device__ __forceinline__ uint32_t bf16_from_double(double v)
{
    float t = __double2float_rz(v);
    uint32_t u = __float_as_uint(t);
    if ((double)t != v)
        u |= 1u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// (a1) cos/sin tables                             [ERNIE-fuse §1]
//
// One lane per 8 consecutive rotary columns of one table row: two 16-byte
// angle loads, eight fp32 sincosf, two 16-byte stores.  An fp32 result whose
// low 16 bits lie within kTieGuard units of 0x8000 is too close to a bf16
// rounding midpoint for fp32's few-ulp error to decide; those (about one in
// a thousand) are recomputed in double and rounded exactly, so each entry is
// the correctly rounded bf16 of cos/sin of the fp32 angle.
// ---------------------------------------------------------------------------
constexpr uint32_t kTieGuard = 64;

__device__ __forceinline__ bool near_bf16_tie(float r)
{
    uint32_t low = __float_as_uint(r) & 0xFFFFu;
    return low - (0x8000u - kTieGuard) <= 2u * kTieGuard;
}

__device__ __forceinline__ void cossin_pair(float a0, float a1, uint32_t &cw, uint32_t &sw)
{
    float s0, c0, s1, c1;
    sincosf(a0, &s0, &c0);
    sincosf(a1, &s1, &c1);
    cw = rne_pack(c0, c1);
    sw = rne_pack(s0, s1);
    if (near_bf16_tie(c0) | near_bf16_tie(c1) | near_bf16_tie(s0) | near_bf16_tie(s1)) {
        double ds0, dc0, ds1, dc1;
        sincos((double)a0, &ds0, &dc0);
        sincos((double)a1, &ds1, &dc1);
        cw = bf16_from_double(dc0) | (bf16_from_double(dc1) << 16);
        sw = bf16_from_double(ds0) | (bf16_from_double(ds1) << 16);
    }
}

__global__ __launch_bounds__(kThreads) void rope_cossin_kernel(CosSinParams p)
{
    const uint32_t nvec_row = p.div_vecs.d;
    const uint32_t S = p.div_s.d;
    for (uint32_t idx = blockIdx.x * kThreads + threadIdx.x; idx < p.vec_total;
         idx += gridDim.x * kThreads) {
        uint32_t row = fdiv(idx, p.div_vecs);
        uint32_t cg = idx - row * nvec_row;
        uint32_t b = fdiv(row, p.div_s);
        uint32_t s = row - b * S;
        const float4 *f = reinterpret_cast<const float4 *>(
            p.freqs + (int64_t)s * p.stride_s + (int64_t)b * p.stride_b + cg * 8);
        float4 f0 = f[0], f1 = f[1];
        uint4 c, sn;
        cossin_pair(f0.x, f0.y, c.x, sn.x);
        cossin_pair(f0.z, f0.w, c.y, sn.y);
        cossin_pair(f1.x, f1.y, c.z, sn.z);
        cossin_pair(f1.z, f1.w, c.w, sn.w);
        int64_t o = (int64_t)row * p.R + cg * 8;
        *reinterpret_cast<uint4 *>(p.cos + o) = c;
        *reinterpret_cast<uint4 *>(p.sin + o) = sn;
    }
}

// ---------------------------------------------------------------------------
// (a2, a3) rotate-half RoPE with tail passthrough     [ERNIE-fuse §2]
//
// A workgroup owns tok_per_wg consecutive tokens (table rows t0 ...).  It
// stages their cos/sin rows in LDS once, widened to fp32, together with each
// token's base offsets, and then every (view, head) of those tokens reuses
// them.  Work item = (token, head, pair group p): the lane loads the 8
// columns x[8p .. 8p+7] of the first half and x[h2+8p ..] of the second half
// (both 16-byte vectors), rotates them against the matching 8 + 8 cos/sin
// entries, and stores both results; each element is read and written by the
// same lane, so out == x is safe.  Consecutive lanes take consecutive pair
// groups and then consecutive heads, so a wave64 touches whole 128-byte
// segments.  Two items per lane are in flight before any store.
// ---------------------------------------------------------------------------

// out1 = rne(rne(x1*c1) + rne(-x2*s1)), out2 = rne(rne(x2*c2) + rne(x1*s2)) on
// the two elements packed in words a (x1) and b (x2).
__device__ __forceinline__ void rope_word(uint32_t a, uint32_t b, const float *c1,
                                          const float *s1, const float *c2, const float *s2,
                                          uint32_t &o1, uint32_t &o2)
{
    float a0 = bf_lo(a), a1 = bf_hi(a);
    float b0 = bf_lo(b), b1 = bf_hi(b);
    uint32_t p0 = rne_pack(a0 * c1[0], -(b0 * s1[0]));
    uint32_t p1 = rne_pack(a1 * c1[1], -(b1 * s1[1]));
    uint32_t q0 = rne_pack(b0 * c2[0], a0 * s2[0]);
    uint32_t q1 = rne_pack(b1 * c2[1], a1 * s2[1]);
    o1 = rne_pack(bf_lo(p0) + bf_hi(p0), bf_lo(p1) + bf_hi(p1));
    o2 = rne_pack(bf_lo(q0) + bf_hi(q0), bf_lo(q1) + bf_hi(q1));
}

__device__ __forceinline__ void rope_vec(const uint4 &x1, const uint4 &x2, const float *c1,
                                         const float *s1, const float *c2, const float *s2,
                                         uint4 &o1, uint4 &o2)
{
    rope_word(x1.x, x2.x, c1 + 0, s1 + 0, c2 + 0, s2 + 0, o1.x, o2.x);
    rope_word(x1.y, x2.y, c1 + 2, s1 + 2, c2 + 2, s2 + 2, o1.y, o2.y);
    rope_word(x1.z, x2.z, c1 + 4, s1 + 4, c2 + 4, s2 + 4, o1.z, o2.z);
    rope_word(x1.w, x2.w, c1 + 6, s1 + 6, c2 + 6, s2 + 6, o1.w, o2.w);
}

__device__ __forceinline__ void load_f32x8(const float *src, float *dst)
{
    float4 u = reinterpret_cast<const float4 *>(src)[0];
    float4 v = reinterpret_cast<const float4 *>(src)[1];
    dst[0] = u.x; dst[1] = u.y; dst[2] = u.z; dst[3] = u.w;
    dst[4] = v.x; dst[5] = v.y; dst[6] = v.z; dst[7] = v.w;
}

__global__ __launch_bounds__(kThreads) void rope_rotate_half_kernel(RopeParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int R = p.R, half = p.half, H = p.H, tpw = p.tok_per_wg;
    float *lcos = reinterpret_cast<float *>(smem);            // [tpw][R]
    float *lsin = lcos + tpw * R;                             // [tpw][R]
    int64_t *lbase = reinterpret_cast<int64_t *>(lsin + tpw * R);  // [view][tok][x, out]

    const int64_t t0 = (int64_t)blockIdx.x * tpw;
    const int ntok = (int)min((int64_t)tpw, p.tokens - t0);
    const int tid = threadIdx.x;

    // Stage the cos/sin rows of this workgroup's tokens (consecutive rows).
    {
        const uint4 *gc = reinterpret_cast<const uint4 *>(p.cos + t0 * R);
        const uint4 *gs = reinterpret_cast<const uint4 *>(p.sin + t0 * R);
        const int nvec = ntok * (R / 8);
        for (int i = tid; i < nvec; i += kThreads) {
            uint4 c = gc[i], s = gs[i];
            float4 *dc = reinterpret_cast<float4 *>(lcos + i * 8);
            float4 *ds = reinterpret_cast<float4 *>(lsin + i * 8);
            dc[0] = make_float4(bf_lo(c.x), bf_hi(c.x), bf_lo(c.y), bf_hi(c.y));
            dc[1] = make_float4(bf_lo(c.z), bf_hi(c.z), bf_lo(c.w), bf_hi(c.w));
            ds[0] = make_float4(bf_lo(s.x), bf_hi(s.x), bf_lo(s.y), bf_hi(s.y));
            ds[1] = make_float4(bf_lo(s.z), bf_hi(s.z), bf_lo(s.w), bf_hi(s.w));
        }
    }
    // Token base offsets per view: b*stride_b + s*stride_s for x and out.
    for (int v = 0; v < p.n_views; ++v) {
        const RopeView &V = p.v[v];
        for (int tl = tid; tl < ntok; tl += kThreads) {
            uint32_t t = (uint32_t)(t0 + tl);
            uint32_t b = fdiv(t, p.div_s);
            uint32_t s = t - b * p.div_s.d;
            lbase[(v * tpw + tl) * 2 + 0] = (int64_t)b * V.xs_b + (int64_t)s * V.xs_s;
            lbase[(v * tpw + tl) * 2 + 1] = (int64_t)b * V.os_b + (int64_t)s * V.os_s;
        }
    }
    __syncthreads();

    // Rotation: items (token, head, pair group) with the pair group fastest.
    const int P = half / 8;
    const int items = ntok * H * P;
    for (int v = 0; v < p.n_views; ++v) {
        const RopeView V = p.v[v];
        const int64_t *vb = lbase + v * tpw * 2;
        // item -> x offset, out offset (elements) and cos/sin offset in LDS
        auto locate = [&](int i, int64_t &xo, int64_t &oo, int &co) {
            uint32_t q = fdiv((uint32_t)i, p.div_pairs);
            int pg = i - (int)q * P;
            uint32_t tl = fdiv(q, p.div_heads);
            int hh = (int)q - (int)tl * H;
            xo = vb[tl * 2 + 0] + (int64_t)hh * V.xs_h + pg * 8;
            oo = vb[tl * 2 + 1] + (int64_t)hh * V.os_h + pg * 8;
            co = (int)tl * R + pg * 8;
        };
        auto rotate_store = [&](const uint4 &x1, const uint4 &x2, int64_t oo, int co) {
            float c1[8], s1[8], c2[8], s2[8];
            load_f32x8(lcos + co, c1);
            load_f32x8(lsin + co, s1);
            load_f32x8(lcos + co + half, c2);
            load_f32x8(lsin + co + half, s2);
            uint4 o1, o2;
            rope_vec(x1, x2, c1, s1, c2, s2, o1, o2);
            *reinterpret_cast<uint4 *>(V.out + oo) = o1;
            *reinterpret_cast<uint4 *>(V.out + oo + half) = o2;
        };
        int i = tid;
        // two items per lane in flight: both loads issued before either store
        for (; i + kThreads < items; i += 2 * kThreads) {
            int64_t xa, oa, xb, ob;
            int ca, cb;
            locate(i, xa, oa, ca);
            locate(i + kThreads, xb, ob, cb);
            uint4 a1 = *reinterpret_cast<const uint4 *>(V.x + xa);
            uint4 a2 = *reinterpret_cast<const uint4 *>(V.x + xa + half);
            uint4 b1 = *reinterpret_cast<const uint4 *>(V.x + xb);
            uint4 b2 = *reinterpret_cast<const uint4 *>(V.x + xb + half);
            rotate_store(a1, a2, oa, ca);
            rotate_store(b1, b2, ob, cb);
        }
        if (i < items) {
            int64_t xa, oa;
            int ca;
            locate(i, xa, oa, ca);
            uint4 a1 = *reinterpret_cast<const uint4 *>(V.x + xa);
            uint4 a2 = *reinterpret_cast<const uint4 *>(V.x + xa + half);
            rotate_store(a1, a2, oa, ca);
        }
    }

    // Tail passthrough: columns R .. D-1, copied as bits.
    const int Q = (p.D - R) / 8;
    if (Q == 0)
        return;
    const int titems = ntok * H * Q;
    for (int v = 0; v < p.n_views; ++v) {
        if (!((p.tail_mask >> v) & 1))
            continue;
        const RopeView V = p.v[v];
        const int64_t *vb = lbase + v * tpw * 2;
        auto locate = [&](int i, int64_t &xo, int64_t &oo) {
            uint32_t q = fdiv((uint32_t)i, p.div_tail);
            int c = i - (int)q * Q;
            uint32_t tl = fdiv(q, p.div_heads);
            int hh = (int)q - (int)tl * H;
            xo = vb[tl * 2 + 0] + (int64_t)hh * V.xs_h + R + c * 8;
            oo = vb[tl * 2 + 1] + (int64_t)hh * V.os_h + R + c * 8;
        };
        int i = tid;
        for (; i + kThreads < titems; i += 2 * kThreads) {
            int64_t xa, oa, xb, ob;
            locate(i, xa, oa);
            locate(i + kThreads, xb, ob);
            uint4 a = *reinterpret_cast<const uint4 *>(V.x + xa);
            uint4 b = *reinterpret_cast<const uint4 *>(V.x + xb);
            *reinterpret_cast<uint4 *>(V.out + oa) = a;
            *reinterpret_cast<uint4 *>(V.out + ob) = b;
        }
        if (i < titems) {
            int64_t xa, oa;
            locate(i, xa, oa);
            *reinterpret_cast<uint4 *>(V.out + oa) = *reinterpret_cast<const uint4 *>(V.x + xa);
        }
    }
}

// ---------------------------------------------------------------------------
// (a4, a5) GEGLU with activation rounding             [ERNIE-fuse §3]
//
// G(x) = rne_bf16(x * Phi(x)) takes one of 65536 inputs, so it is tabulated
// where it is not a simple function of the bits:
//   |x| in [2^-10, 16):   table (1792 entries per sign, 7 KiB), built once per
//                         device in double precision and held in LDS;
//   |x| in [2^-125, 2^-10): G = x/2 exactly (x * (Phi(x) - 1/2) < 0.8|x|^2/2
//                         stays under half a bf16 step of x/2);
//   |x| < 2^-125:         x/2 is a multiple of the subnormal step 2^-134 and
//                         the exact G lies strictly above it, so a halfway
//                         x/2 rounds toward +inf;
//   x >= 16: G = x;  x <= -16: G = -0 (|G| < 1e-56);  G(+inf) = +inf,
//   G(-inf) = NaN, NaN -> NaN.
// Inputs outside [2^-125, 16) in magnitude are rare, so a wave takes the
// general path only when one of its lanes holds one.  The multiply by up is
// exact in fp32 and rounded once.
// ---------------------------------------------------------------------------
constexpr uint32_t kLutLo = 0x3A80u;                // bf16 bits of 2^-10
constexpr uint32_t kLutHi = 0x4180u;                // bf16 bits of 16.0
constexpr uint32_t kLutSpan = kLutHi - kLutLo;      // 1792 magnitudes per sign
constexpr uint32_t kLutEntries = 2 * kLutSpan;      // [positive | negative]

__device__ __align__(16) uint16_t g_gelu_lut[kLutEntries];

__global__ __launch_bounds__(kThreads) void build_gelu_table_kernel()
{
    uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= kLutEntries)
        return;
    uint32_t neg = i >= kLutSpan ? 1u : 0u;
    uint32_t bits = (neg << 15) | (kLutLo + i - neg * kLutSpan);
    double x = (double)__uint_as_float(bits << 16);
    double g = 0.5 * x * erfc(-x * 0.70710678118654752440);  // x * Phi(x)
    g_gelu_lut[i] = (uint16_t)bf16_from_double(g);
}

// G for a bf16 gate whose magnitude is in [2^-125, 16).
__device__ __forceinline__ uint32_t gelu_common(uint32_t g, const uint16_t *lut)
{
    uint32_t a = g & 0x7FFFu;
    uint32_t idx = max(a, kLutLo) - kLutLo + (g >> 15) * kLutSpan;
    uint32_t t = lut[idx];
    return a < kLutLo ? g - 0x80u : t;
}

// G for any bf16 gate.
__device__ uint32_t gelu_general(uint32_t g, const uint16_t *lut)
{
    uint32_t a = g & 0x7FFFu;
    uint32_t neg = g >> 15;
    if (a > 0x7F80u)
        return g | 0x0040u;
    if (a == 0x7F80u)
        return neg ? 0xFFC0u : 0x7F80u;
    if (a >= kLutHi)
        return neg ? 0x8000u : g;
    if (a >= 0x0100u)
        return gelu_common(g, lut);
    return neg ? (0x8000u | (a >> 1)) : ((a + 1u) >> 1);
}

// True if either bf16 of the word has a magnitude outside [2^-125, 16).
__device__ __forceinline__ bool word_needs_general(uint32_t w)
{
    uint32_t lo = (w & 0x7FFFu) - 0x0100u;
    uint32_t hi = ((w >> 16) & 0x7FFFu) - 0x0100u;
    return max(lo, hi) >= kLutHi - 0x0100u;
}

__device__ __forceinline__ uint32_t geglu_word(uint32_t gw, uint32_t uw, const uint16_t *lut,
                                               bool general)
{
    uint32_t g0, g1;
    if (general) {
        g0 = gelu_general(gw & 0xFFFFu, lut);
        g1 = gelu_general(gw >> 16, lut);
    } else {
        g0 = gelu_common(gw & 0xFFFFu, lut);
        g1 = gelu_common(gw >> 16, lut);
    }
    return rne_pack(bf_lo(uw) * __uint_as_float(g0 << 16), bf_hi(uw) * __uint_as_float(g1 << 16));
}

constexpr int kGegluUnroll = 4;

__global__ __launch_bounds__(kThreads) void gelu_and_mul_kernel(GegluParams p)
{
    __shared__ __align__(16) uint16_t lut[kLutEntries];
    for (uint32_t i = threadIdx.x; i < kLutEntries / 8; i += kThreads)
        reinterpret_cast<uint4 *>(lut)[i] = reinterpret_cast<const uint4 *>(g_gelu_lut)[i];
    __syncthreads();

    const uint32_t nvec_row = p.div_vecs.d;
    const uint32_t step = gridDim.x * (kThreads * kGegluUnroll);
    for (uint32_t base = blockIdx.x * (kThreads * kGegluUnroll); base < p.vec_total;
         base += step) {
        uint4 g[kGegluUnroll], u[kGegluUnroll];
        int64_t oo[kGegluUnroll];
#pragma unroll
        for (int k = 0; k < kGegluUnroll; ++k) {
            uint32_t idx = base + k * kThreads + threadIdx.x;
            if (idx < p.vec_total) {
                uint32_t row = fdiv(idx, p.div_vecs);
                uint32_t col = (idx - row * nvec_row) * 8;
                const uint16_t *src = p.in + (int64_t)row * p.in_stride + col;
                g[k] = *reinterpret_cast<const uint4 *>(src);
                u[k] = *reinterpret_cast<const uint4 *>(src + p.hidden);
                oo[k] = (int64_t)row * p.out_stride + col;
            }
        }
#pragma unroll
        for (int k = 0; k < kGegluUnroll; ++k) {
            uint32_t idx = base + k * kThreads + threadIdx.x;
            if (idx < p.vec_total) {
                bool general = word_needs_general(g[k].x) | word_needs_general(g[k].y) |
                               word_needs_general(g[k].z) | word_needs_general(g[k].w);
                uint4 o;
                o.x = geglu_word(g[k].x, u[k].x, lut, general);
                o.y = geglu_word(g[k].y, u[k].y, lut, general);
                o.z = geglu_word(g[k].z, u[k].z, lut, general);
                o.w = geglu_word(g[k].w, u[k].w, lut, general);
                *reinterpret_cast<uint4 *>(p.out + oo[k]) = o;
            }
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_rope_cossin(const CosSinParams &p, hipStream_t stream)
{
    uint32_t blocks = (p.vec_total + kThreads - 1) / kThreads;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(rope_cossin_kernel, dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_rope_rotate_half(const RopeParams &p, hipStream_t stream)
{
    int64_t blocks = (p.tokens + p.tok_per_wg - 1) / p.tok_per_wg;
    size_t lds = (size_t)p.tok_per_wg * p.R * 2 * sizeof(float) +
                 (size_t)p.n_views * p.tok_per_wg * 2 * sizeof(int64_t);
    hipLaunchKernelGGL(rope_rotate_half_kernel, dim3((uint32_t)blocks), dim3(kThreads), lds,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_gelu_and_mul(const GegluParams &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL(gelu_and_mul_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_build_gelu_table(hipStream_t stream)
{
    hipLaunchKernelGGL(build_gelu_table_kernel, dim3((kLutEntries + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, stream);
    return hipGetLastError();
}

int rope_tokens_per_workgroup(int n_views, int H, int D, int R)
{
    // About 4096 16-byte vectors (64 KiB) of x per workgroup, and the LDS
    // staging (fp32 cos/sin rows plus two offsets per view) within 32 KiB.
    int64_t vec_per_tok = (int64_t)n_views * H * (D / 8);
    int64_t t = vec_per_tok > 0 ? 4096 / vec_per_tok : 64;
    if (t < 1)
        t = 1;
    if (t > 64)
        t = 64;
    while (t > 1 && t * R * 8 + t * n_views * 16 > 32768)
        --t;
    return (int)t;
}

int geglu_grid(uint32_t vec_total, int cu_count)
{
    // Persistent: up to 8 workgroups per compute unit, each looping over
    // chunks of kThreads * kGegluUnroll vectors (the LUT is loaded once per
    // workgroup).
    uint32_t chunks = (vec_total + kThreads * kGegluUnroll - 1) / (kThreads * kGegluUnroll);
    uint32_t cap = (uint32_t)(cu_count > 0 ? cu_count : 256) * 8;
    return (int)(chunks < cap ? (chunks > 0 ? chunks : 1) : cap);
}

}  // namespace rgg

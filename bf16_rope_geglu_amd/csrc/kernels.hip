// HIP kernels of the fused elementwise path for gfx950 (MI355X, CDNA4).
//
// Method: "[sglang] ERNIE-Image의 RoPE와 GELU-mul 융합 및 RoPE cos/sin 호이스팅을
// 통한 성능 최적화" (blog.secrett2633.cloud, analysis of sglang PR 34306),
// cited as [ERNIE-fuse] with its section.
//
// The kernels of the path are HBM-bound elementwise work with no matrix
// cores: they move data in 16-byte (8 x bf16) vectors per lane so that a
// wave64 load or store covers whole cache lines, and round every eager bf16 op
// with the hardware's round-to-nearest-even v_cvt_pk_bf16_f32.  The gate_up
// projection at the end of the file is a contraction and runs on the matrix
// cores (MFMA).  IEEE fp32 subnormals are kept (the default denormal
// mode of gfx950 code objects) and nothing is contracted into an FMA across a
// rounding point (the bf16 rounding sits between every multiply and add, and
// the file is built with -ffp-contract=off).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "launch.h"

namespace rgg {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));  // 8 x bf16

// Streamed data (read or written once) bypasses cache retention: the loads
// and stores carry the nontemporal bit.
__device__ __forceinline__ v4u stream_load(const uint16_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
}

__device__ __forceinline__ void stream_store(uint16_t *p, v4u v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(p));
}

// Load/store whose nontemporal hint is chosen per launch: the hint pays only
// when every 128-byte line is read or written whole by one instruction;
// lines split between instructions are better merged in L2 first.
template <bool Nt>
__device__ __forceinline__ v4u load16(const uint16_t *p)
{
    if constexpr (Nt)
        return stream_load(p);
    else
        return *reinterpret_cast<const v4u *>(p);
}

template <bool Nt>
__device__ __forceinline__ void store16(uint16_t *p, v4u v)
{
    if constexpr (Nt)
        stream_store(p, v);
    else
        *reinterpret_cast<v4u *>(p) = v;
}

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
// Cos/sin tables                             [ERNIE-fuse §1]
//
// A lane owns a run of consecutive rotary columns of one table row (8, or 4
// of each half in small paired tables): vector angle loads, one fp32 sincosf
// per angle, vector stores of cos and sin.  sincosf is accurate
// to a couple of fp32 ulps, so rounding its result to bf16 gives the
// correctly rounded bf16 of the true value unless the fp32 result lies within
// a few ulps of a bf16 rounding midpoint (its low 16 bits near 0x8000).
// Those few (about one in 7000) are recomputed in double and rounded exactly,
// so each entry is the correctly rounded bf16 of cos/sin of the fp32 angle.
// kTieGuard is that margin in fp32 ulps.
// ---------------------------------------------------------------------------
constexpr uint32_t kTieGuard = 4;

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
    if ((int)near_bf16_tie(c0) | (int)near_bf16_tie(c1) | (int)near_bf16_tie(s0) |
        (int)near_bf16_tie(s1)) {
        double ds0, dc0, ds1, dc1;
        sincos((double)a0, &ds0, &dc0);
        sincos((double)a1, &ds1, &dc1);
        cw = bf16_from_double(dc0) | (bf16_from_double(dc1) << 16);
        sw = bf16_from_double(ds0) | (bf16_from_double(ds1) << 16);
    }
}

__device__ __forceinline__ void cossin_vec8(v4u a0, v4u a1, uint32_t *c, uint32_t *sn)
{
    cossin_pair(__uint_as_float(a0.x), __uint_as_float(a0.y), c[0], sn[0]);
    cossin_pair(__uint_as_float(a0.z), __uint_as_float(a0.w), c[1], sn[1]);
    cossin_pair(__uint_as_float(a1.x), __uint_as_float(a1.y), c[2], sn[2]);
    cossin_pair(__uint_as_float(a1.z), __uint_as_float(a1.w), c[3], sn[3]);
}

// Paired form (R a multiple of 16): a lane owns W consecutive columns of
// both halves of a row (W = 8, or 4 for Narrow).  Rotate-half angle tables
// usually repeat the first half in the second (cat(f, f)); when the W angles
// of the second half are bitwise the first half's, their cos/sin are reused
// instead of recomputed.  Narrow lanes do half the work each: for small
// tables (up to kTableNarrowLanes of them) twice as many lanes fill more of
// the chip and each lane's chain of sincos is half as long.
template <bool Paired, bool Narrow>
__global__ __launch_bounds__(kThreads) void rope_cossin_kernel(CosSinParams p)
{
    const uint32_t nvec_row = p.div_vecs.d;
    const uint32_t S = p.div_s.d;
    const int half = p.R / 2;
    // every parameter in scalar registers before the first load: one batch
    // of scalar loads, one wait
    asm volatile("" ::"s"(p.freqs), "s"(p.cos), "s"(p.sin), "s"(p.stride_s), "s"(p.stride_b),
                 "s"(p.vec_total), "s"(p.div_vecs.m), "s"(p.div_vecs.l), "s"(nvec_row),
                 "s"(p.div_s.m), "s"(p.div_s.l), "s"(S), "s"(p.R), "s"(gridDim.x));
    for (uint32_t idx = blockIdx.x * kThreads + threadIdx.x; idx < p.vec_total;
         idx += gridDim.x * kThreads) {
        uint32_t row = fdiv(idx, p.div_vecs);
        uint32_t cg = idx - row * nvec_row;
        uint32_t b = fdiv(row, p.div_s);
        uint32_t s = row - b * S;
        const float *f = p.freqs + (int64_t)s * p.stride_s + (int64_t)b * p.stride_b;
        int64_t o = (int64_t)row * p.R;
        if constexpr (Paired && Narrow) {
            const int col = cg * 4;
            uint32_t c[2], sn[2];
            const v4u a0 = *reinterpret_cast<const v4u *>(f + col);
            const v4u b0 = *reinterpret_cast<const v4u *>(f + half + col);
            cossin_pair(__uint_as_float(a0.x), __uint_as_float(a0.y), c[0], sn[0]);
            cossin_pair(__uint_as_float(a0.z), __uint_as_float(a0.w), c[1], sn[1]);
            uint2 cv = make_uint2(c[0], c[1]), sv = make_uint2(sn[0], sn[1]);
            *reinterpret_cast<uint2 *>(p.cos + o + col) = cv;
            *reinterpret_cast<uint2 *>(p.sin + o + col) = sv;
            if (!(a0.x == b0.x && a0.y == b0.y && a0.z == b0.z && a0.w == b0.w)) {
                cossin_pair(__uint_as_float(b0.x), __uint_as_float(b0.y), c[0], sn[0]);
                cossin_pair(__uint_as_float(b0.z), __uint_as_float(b0.w), c[1], sn[1]);
                cv = make_uint2(c[0], c[1]);
                sv = make_uint2(sn[0], sn[1]);
            }
            *reinterpret_cast<uint2 *>(p.cos + o + half + col) = cv;
            *reinterpret_cast<uint2 *>(p.sin + o + half + col) = sv;
        } else if constexpr (Paired) {
            const int col = cg * 8;
            uint32_t c[4], sn[4];
            v4u a0 = *reinterpret_cast<const v4u *>(f + col);
            v4u a1 = *reinterpret_cast<const v4u *>(f + col + 4);
            v4u b0 = *reinterpret_cast<const v4u *>(f + half + col);
            v4u b1 = *reinterpret_cast<const v4u *>(f + half + col + 4);
            cossin_vec8(a0, a1, c, sn);
            v4u cv = v4u{c[0], c[1], c[2], c[3]}, sv = v4u{sn[0], sn[1], sn[2], sn[3]};
            *reinterpret_cast<v4u *>(p.cos + o + col) = cv;
            *reinterpret_cast<v4u *>(p.sin + o + col) = sv;
            bool same = a0.x == b0.x && a0.y == b0.y && a0.z == b0.z && a0.w == b0.w &&
                        a1.x == b1.x && a1.y == b1.y && a1.z == b1.z && a1.w == b1.w;
            if (!same) {
                cossin_vec8(b0, b1, c, sn);
                cv = v4u{c[0], c[1], c[2], c[3]};
                sv = v4u{sn[0], sn[1], sn[2], sn[3]};
            }
            *reinterpret_cast<v4u *>(p.cos + o + half + col) = cv;
            *reinterpret_cast<v4u *>(p.sin + o + half + col) = sv;
        } else {
            const int col = cg * 8;
            uint32_t c[4], sn[4];
            const float4 f0 = reinterpret_cast<const float4 *>(f + col)[0];
            const float4 f1 = reinterpret_cast<const float4 *>(f + col)[1];
            cossin_pair(f0.x, f0.y, c[0], sn[0]);
            cossin_pair(f0.z, f0.w, c[1], sn[1]);
            cossin_pair(f1.x, f1.y, c[2], sn[2]);
            cossin_pair(f1.z, f1.w, c[3], sn[3]);
            *reinterpret_cast<v4u *>(p.cos + o + col) = v4u{c[0], c[1], c[2], c[3]};
            *reinterpret_cast<v4u *>(p.sin + o + col) = v4u{sn[0], sn[1], sn[2], sn[3]};
        }
    }
}

// ---------------------------------------------------------------------------
// Cos/sin tables of a 3-axis token grid  [ERNIE-fuse §1]
//
// Token s of a (T, Hg, Wg) grid sits at (t, h, w), s = (t*Hg + h)*Wg + w,
// with t shifted by the batch row's offset.  Half-column c of axis k (local
// index i) turns by pos_k * theta^(-2i/d_k), formed in double and rounded once
// to fp32, and the row is cat(f, f), so a lane computes W half-columns (8, or
// 4 for small tables as in the precompute) and stores each cos/sin vector in
// both halves.  Each workgroup first puts the frequencies theta^(-2i/d_k) of
// the R/2 half-columns in LDS: copied from the kernel arguments (computed on
// the host) for up to 2*kGridOmegaArgs rotary columns, evaluated on the
// device for wider rows.  The cos/sin of the fp32 angle then go through the
// same correctly rounded path as the precompute above.
// ---------------------------------------------------------------------------
template <int W> struct TableVec { using type = v4u; };    // 8 bf16
template <> struct TableVec<4> { using type = uint2; };   // 4 bf16

template <int W>
__global__ __launch_bounds__(kThreads) void rope_cossin_grid_kernel(CosSinGridParams p)
{
    static_assert(W == 4 || W == 8, "a lane stores one 8- or 16-byte vector per table half");
    using vec = typename TableVec<W>::type;
    extern __shared__ double lomega[];  // [R/2]
    const int half = p.R / 2;
    for (int c = threadIdx.x; c < half; c += kThreads) {
        if (p.host_omega) {
            lomega[c] = p.omega[c];
        } else {
            const int k = c < p.h0 ? 0 : (c < p.h01 ? 1 : 2);
            const int i = c - (k == 0 ? 0 : (k == 1 ? p.h0 : p.h01));
            lomega[c] = pow(p.theta, -2.0 * i / p.d[k]);
        }
    }
    __syncthreads();
    const uint32_t groups = p.div_groups.d, S = p.div_s.d, HW = p.div_hw.d, Wg = p.div_w.d;
    for (uint32_t g = blockIdx.x * kThreads + threadIdx.x; g < p.groups_total;
         g += gridDim.x * kThreads) {
        const uint32_t row = fdiv(g, p.div_groups);
        const int c0 = (int)(g - row * groups) * W;
        const uint32_t b = fdiv(row, p.div_s);
        const uint32_t s = row - b * S;
        const uint32_t t = fdiv(s, p.div_hw);
        const uint32_t hw = s - t * HW;
        const uint32_t h = fdiv(hw, p.div_w);
        const uint32_t w = hw - h * Wg;
        const double pos[3] = {(double)((int64_t)t + (p.t_offset ? p.t_offset[b] : 0)),
                               (double)h, (double)w};
        float a[W];
#pragma unroll
        for (int e = 0; e < W; ++e) {
            const int c = c0 + e;
            const int k = c < p.h0 ? 0 : (c < p.h01 ? 1 : 2);
            a[e] = __double2float_rn(pos[k] * lomega[c]);
        }
        vec cv, sv;
        uint32_t *cw = reinterpret_cast<uint32_t *>(&cv), *sw = reinterpret_cast<uint32_t *>(&sv);
#pragma unroll
        for (int q = 0; q < W / 2; ++q)
            cossin_pair(a[2 * q], a[2 * q + 1], cw[q], sw[q]);
        const int64_t o = (int64_t)row * p.R + c0;
        *reinterpret_cast<vec *>(p.cos + o) = cv;
        *reinterpret_cast<vec *>(p.cos + o + half) = cv;
        *reinterpret_cast<vec *>(p.sin + o) = sv;
        *reinterpret_cast<vec *>(p.sin + o + half) = sv;
    }
}

// ---------------------------------------------------------------------------
// Rotate-half RoPE with tail passthrough     [ERNIE-fuse §2]
//
// A workgroup owns one view and tok_per_wg consecutive tokens (table rows
// t0 ...); the views of the same tokens sit in neighbouring workgroups so
// they run together and share the cos/sin rows through L2.  Work item =
// (token, head, slot): slots 0 .. P-1 are rotation pair groups, where the
// lane loads the 8 columns x[8p .. 8p+7] of the first half and x[h2+8p ..]
// of the second half (two 16-byte vectors), rotates them against the
// matching 8 + 8 cos/sin entries and stores both results; slots P .. P+Q-1
// copy one 16-byte vector of the tail.  Consecutive lanes take consecutive
// slots and then heads, so a wave64 requests whole head rows (and so whole
// cache lines) at once.  Each element is read and written by one lane, so
// out == x is safe (the tail slots are then dropped).
//
// The lane issues its first item's loads before the cos/sin rows of its
// tokens are staged as fp32 in LDS, so the HBM latency overlaps the staging;
// every (head, slot) of a token then reuses the staged row.  A one-token
// workgroup lets each wave stage its own copy (no workgroup barrier) while
// the copies fit 64 KiB; otherwise the workgroup stages one copy behind a
// barrier.  A token with k >= 2 whole passes of items is split over k
// workgroups.  When R is not a multiple of 128 the two halves of a row split
// cache lines between the two store instructions, and launches that allow it
// use rope_rotate_half_lane_kernel below (one contiguous vector per lane).
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

__device__ __forceinline__ void load_f32x8(const float *src, float *dst)
{
    float4 u = reinterpret_cast<const float4 *>(src)[0];
    float4 v = reinterpret_cast<const float4 *>(src)[1];
    dst[0] = u.x; dst[1] = u.y; dst[2] = u.z; dst[3] = u.w;
    dst[4] = v.x; dst[5] = v.y; dst[6] = v.z; dst[7] = v.w;
}

// One work item located: element offsets of its x and out vectors, its
// cos/sin offset in LDS, and whether it is a rotation item.
struct RopeItem {
    int64_t xo, oo;
    int co;
    bool rot;
};

// Token base offsets b*stride_b + s*stride_s of token t for x and out.
__device__ __forceinline__ void rope_token_base(const RopeParams &p, const RopeView &V,
                                                uint32_t t, int64_t &xb, int64_t &ob)
{
    uint32_t b = fdiv(t, p.div_s);
    uint32_t s = t - b * p.div_s.d;
    xb = (int64_t)b * V.xs_b + (int64_t)s * V.xs_s;
    ob = (int64_t)b * V.os_b + (int64_t)s * V.os_s;
}

// Workgroup -> (token chunk, view, part).  A token whose items fill several
// workgroup passes is split over `parts` workgroups, each taking every
// parts-th pass; consecutive workgroups walk the parts, then the views, then
// the token chunks of this launch.
__device__ __forceinline__ void rope_workgroup(const RopeParams &p, uint32_t &chunk, int &v,
                                               int &part)
{
    const uint32_t wg = blockIdx.x;
    const uint32_t q = fdiv(wg, p.div_vp);
    const uint32_t rem = wg - q * (uint32_t)(p.n_views * p.parts);
    const uint32_t vq = fdiv(rem, p.div_parts);
    v = (int)vq;
    part = (int)(rem - vq * (uint32_t)p.parts);
    chunk = p.chunk0 + q;
}

// Item i of a workgroup whose first token is t0.  With OneToken the
// workgroup holds a single token whose base offsets xb1/ob1 are uniform.
template <bool OneToken>
__device__ __forceinline__ RopeItem rope_locate(const RopeParams &p, const RopeView &V,
                                                int64_t t0, int i, int slots,
                                                const FastDiv &div_slots, int64_t xb1,
                                                int64_t ob1)
{
    const int P = p.half / 8;
    uint32_t q = fdiv((uint32_t)i, div_slots);
    int slot = i - (int)q * slots;
    uint32_t tl = 0;
    int hh = (int)q;
    int64_t xb = xb1, ob = ob1;
    if (!OneToken) {
        tl = fdiv(q, p.div_heads);
        hh = (int)q - (int)tl * p.H;
        rope_token_base(p, V, (uint32_t)(t0 + tl), xb, ob);
    }
    RopeItem it;
    it.rot = slot < P;
    int col = it.rot ? slot * 8 : p.R + (slot - P) * 8;
    it.xo = xb + (int64_t)hh * V.xs_h + col;
    it.oo = ob + (int64_t)hh * V.os_h + col;
    it.co = (int)tl * p.R + slot * 8;
    return it;
}

constexpr int kRopeBlock = 256;
constexpr int64_t kMaxRopeWorkgroups = (int64_t)1 << 20;  // per launch (2^28 work-items)

constexpr int kRopeUnroll = 1;  // items per lane with their loads issued together

template <bool OneToken, bool Nt>
__global__ __launch_bounds__(kRopeBlock) void rope_rotate_half_kernel(RopeParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int R = p.R, half = p.half, tpw = p.tok_per_wg;
    float *lcos = reinterpret_cast<float *>(smem);  // [tpw][R]
    float *lsin = lcos + tpw * R;                   // [tpw][R]

    uint32_t wg_tok;
    int v, part;
    rope_workgroup(p, wg_tok, v, part);
    const int64_t t0 = (int64_t)wg_tok * tpw;
    const int ntok = (int)min((int64_t)tpw, p.tokens - t0);
    const RopeView V = p.v[v];
    const bool tail = (p.tail_mask >> v) & 1;
    const int slots = tail ? p.slots_tail : p.half / 8;
    const FastDiv div_slots = tail ? p.div_slots_tail : p.div_slots;
    const int items = ntok * p.H * slots;
    const int tid = threadIdx.x;
    int64_t xb1 = 0, ob1 = 0;
    if (OneToken)
        rope_token_base(p, V, (uint32_t)t0, xb1, ob1);

    constexpr int U = kRopeUnroll;
    const int first = part * kRopeBlock * U;
    for (int base = first; base < items; base += kRopeBlock * U * p.parts) {
        // Locate and load U items per lane before anything waits.  Lanes past
        // the end re-read the last item and tail items read their vector
        // twice, so no load sits under a branch.
        RopeItem it[U];
        v4u x1[U], x2[U];
        // With per-wave staging and R <= 256 each lane fetches at most one
        // 16-byte vector of the cos/sin row, and it does so before its x
        // loads: loads return in order, so waiting for the row then does not
        // wait for x, and the LDS staging overlaps the HBM latency.
        v4u stg = v4u{0u, 0u, 0u, 0u};
        const bool stage1 = OneToken && p.wave_stage && R > 0 && R <= 256;
        if (stage1 && base == first) {
            const int k = min(tid & 63, R / 4 - 1);
            const uint16_t *src = k >= R / 8 ? p.sin + t0 * R + (k - R / 8) * 8 : p.cos + t0 * R + k * 8;
            stg = *reinterpret_cast<const v4u *>(src);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ic = min(base + u * kRopeBlock + tid, items - 1);
            it[u] = rope_locate<OneToken>(p, V, t0, ic, slots, div_slots, xb1, ob1);
            x1[u] = load16<Nt>(V.x + it[u].xo);
            x2[u] = load16<Nt>(V.x + it[u].xo + (it[u].rot ? half : 0));
        }
        if (OneToken && p.wave_stage && base == first) {
            // One token: every wave stages its own fp32 copy of the row in
            // its own LDS slot, so no wave waits for another.  LDS operations
            // of one wave complete in order; the wave barrier keeps the
            // compiler from moving the reads above the writes.
            const int wave = tid >> 6, lane = tid & 63;
            float *wc = lcos + wave * 2 * R, *ws = wc + R;
            const v4u *gc = reinterpret_cast<const v4u *>(p.cos + t0 * R);
            const v4u *gs = reinterpret_cast<const v4u *>(p.sin + t0 * R);
            if (stage1) {
                if (lane < R / 4) {
                    const bool is_sin = lane >= R / 8;
                    const int kk = is_sin ? lane - R / 8 : lane;
                    float4 *d = reinterpret_cast<float4 *>((is_sin ? ws : wc) + kk * 8);
                    d[0] = make_float4(bf_lo(stg.x), bf_hi(stg.x), bf_lo(stg.y), bf_hi(stg.y));
                    d[1] = make_float4(bf_lo(stg.z), bf_hi(stg.z), bf_lo(stg.w), bf_hi(stg.w));
                }
            } else
            for (int k = lane; k < R / 4; k += 64) {
                const bool is_sin = k >= R / 8;
                const int kk = is_sin ? k - R / 8 : k;
                v4u c = is_sin ? gs[kk] : gc[kk];
                float4 *d = reinterpret_cast<float4 *>((is_sin ? ws : wc) + kk * 8);
                d[0] = make_float4(bf_lo(c.x), bf_hi(c.x), bf_lo(c.y), bf_hi(c.y));
                d[1] = make_float4(bf_lo(c.z), bf_hi(c.z), bf_lo(c.w), bf_hi(c.w));
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if ((!OneToken || !p.wave_stage) && base == first) {
            // Stage this workgroup's cos/sin rows (consecutive table rows) as
            // fp32 while the x loads are in flight.
            const v4u *gc = reinterpret_cast<const v4u *>(p.cos + t0 * R);
            const v4u *gs = reinterpret_cast<const v4u *>(p.sin + t0 * R);
            const int nvec = ntok * (R / 8);
            for (int k = tid; k < nvec; k += kRopeBlock) {
                v4u c = gc[k], sn = gs[k];
                float4 *dc = reinterpret_cast<float4 *>(lcos + k * 8);
                float4 *ds = reinterpret_cast<float4 *>(lsin + k * 8);
                dc[0] = make_float4(bf_lo(c.x), bf_hi(c.x), bf_lo(c.y), bf_hi(c.y));
                dc[1] = make_float4(bf_lo(c.z), bf_hi(c.z), bf_lo(c.w), bf_hi(c.w));
                ds[0] = make_float4(bf_lo(sn.x), bf_hi(sn.x), bf_lo(sn.y), bf_hi(sn.y));
                ds[1] = make_float4(bf_lo(sn.z), bf_hi(sn.z), bf_lo(sn.w), bf_hi(sn.w));
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (base + u * kRopeBlock + tid >= items)
                continue;
            if (it[u].rot) {
                float c1[8], s1[8], c2[8], s2[8];
                const float *rc = lcos, *rs = lsin;
                if (OneToken && p.wave_stage) {
                    rc = lcos + (tid >> 6) * 2 * R;
                    rs = rc + R;
                }
                load_f32x8(rc + it[u].co, c1);
                load_f32x8(rs + it[u].co, s1);
                load_f32x8(rc + it[u].co + half, c2);
                load_f32x8(rs + it[u].co + half, s2);
                const v4u a1 = x1[u], a2 = x2[u];
                uint32_t a[4], b[4];
                rope_word(a1.x, a2.x, c1 + 0, s1 + 0, c2 + 0, s2 + 0, a[0], b[0]);
                rope_word(a1.y, a2.y, c1 + 2, s1 + 2, c2 + 2, s2 + 2, a[1], b[1]);
                rope_word(a1.z, a2.z, c1 + 4, s1 + 4, c2 + 4, s2 + 4, a[2], b[2]);
                rope_word(a1.w, a2.w, c1 + 6, s1 + 6, c2 + 6, s2 + 6, a[3], b[3]);
                store16<Nt>(V.out + it[u].oo, v4u{a[0], a[1], a[2], a[3]});
                store16<Nt>(V.out + it[u].oo + half, v4u{b[0], b[1], b[2], b[3]});
            } else {
                store16<Nt>(V.out + it[u].oo, x1[u]);
            }
        }
    }
}

// One output vector per lane: lane i of the workgroup writes 16-byte vector i
// of the token's head rows, so every load and store instruction of a wave
// covers whole contiguous lines for any R.  The lane also loads its
// rotate-half partner vector (R/2 columns away, in the same lines, served
// from cache) and applies
//   first half:  out = rne(rne(x*c) + rne(-x_partner*s)),
//   second half: out = rne(rne(x*c) + rne(x_partner*s)),
// negating a bf16 by its sign bit, which is exact.
__device__ __forceinline__ uint32_t rope_word1(uint32_t a, uint32_t b, const float *c,
                                              const float *s)
{
    uint32_t p0 = rne_pack(bf_lo(a) * c[0], bf_lo(b) * s[0]);
    uint32_t p1 = rne_pack(bf_hi(a) * c[1], bf_hi(b) * s[1]);
    return rne_pack(bf_lo(p0) + bf_hi(p0), bf_lo(p1) + bf_hi(p1));
}

template <bool Nt, int U>
__global__ __launch_bounds__(kRopeBlock) void rope_rotate_half_lane_kernel(RopeParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int R = p.R, nv = p.D / 8, rv = R / 8, hv = R / 16;
    uint32_t t;
    int v, part;
    rope_workgroup(p, t, v, part);
    const RopeView V = p.v[v];
    int64_t xb, ob;
    rope_token_base(p, V, t, xb, ob);
    const int items = p.H * nv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    float *wc = reinterpret_cast<float *>(smem) + wave * 2 * R, *ws = wc + R;

    const int first = part * kRopeBlock * U;
    for (int base = first; base < items; base += kRopeBlock * U * p.parts) {
        int64_t oo[U];
        int j[U];
        v4u a[U], b[U];
        v4u stg = v4u{0u, 0u, 0u, 0u};
        const bool stage1 = R > 0 && R <= 256;
        if (stage1 && base == first) {
            const int k = min(lane, R / 4 - 1);
            const uint16_t *src = k >= R / 8 ? p.sin + (int64_t)t * R + (k - R / 8) * 8
                                             : p.cos + (int64_t)t * R + k * 8;
            stg = *reinterpret_cast<const v4u *>(src);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ic = min(base + u * kRopeBlock + tid, items - 1);
            const uint32_t h = fdiv((uint32_t)ic, p.div_vecs);
            j[u] = ic - (int)h * nv;
            const int64_t xo = xb + (int64_t)h * V.xs_h + j[u] * 8;
            oo[u] = ob + (int64_t)h * V.os_h + j[u] * 8;
            const int pj = j[u] < hv ? hv : (j[u] < rv ? -hv : 0);
            a[u] = load16<Nt>(V.x + xo);
            b[u] = load16<false>(V.x + xo + pj * 8);
        }
        if (base == first) {
            const v4u *gc = reinterpret_cast<const v4u *>(p.cos + (int64_t)t * R);
            const v4u *gs = reinterpret_cast<const v4u *>(p.sin + (int64_t)t * R);
            if (stage1) {
                if (lane < R / 4) {
                    const bool is_sin = lane >= R / 8;
                    const int kk = is_sin ? lane - R / 8 : lane;
                    float4 *d = reinterpret_cast<float4 *>((is_sin ? ws : wc) + kk * 8);
                    d[0] = make_float4(bf_lo(stg.x), bf_hi(stg.x), bf_lo(stg.y), bf_hi(stg.y));
                    d[1] = make_float4(bf_lo(stg.z), bf_hi(stg.z), bf_lo(stg.w), bf_hi(stg.w));
                }
            } else
            for (int k = lane; k < R / 4; k += 64) {
                const bool is_sin = k >= R / 8;
                const int kk = is_sin ? k - R / 8 : k;
                v4u c = is_sin ? gs[kk] : gc[kk];
                float4 *d = reinterpret_cast<float4 *>((is_sin ? ws : wc) + kk * 8);
                d[0] = make_float4(bf_lo(c.x), bf_hi(c.x), bf_lo(c.y), bf_hi(c.y));
                d[1] = make_float4(bf_lo(c.z), bf_hi(c.z), bf_lo(c.w), bf_hi(c.w));
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (base + u * kRopeBlock + tid >= items)
                continue;
            if (j[u] < rv) {
                float c[8], s[8];
                load_f32x8(wc + j[u] * 8, c);
                load_f32x8(ws + j[u] * 8, s);
                const uint32_t flip = j[u] < hv ? 0x80008000u : 0u;
                const v4u x = a[u], y = b[u] ^ flip;
                store16<Nt>(V.out + oo[u],
                            v4u{rope_word1(x.x, y.x, c + 0, s + 0), rope_word1(x.y, y.y, c + 2, s + 2),
                                rope_word1(x.z, y.z, c + 4, s + 4), rope_word1(x.w, y.w, c + 6, s + 6)});
            } else {
                store16<Nt>(V.out + oo[u], a[u]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Rotate-half RoPE for heads of at most 128 columns: one contiguous 16-byte
// vector per lane, partners exchanged across lanes     [ERNIE-fuse §2]
//
// Each view is walked as one flat run of 16-byte vectors, index
// g = (token * H + head) * D/8 + j, and a workgroup takes the next
// VPL * blockDim consecutive vectors (lane t: vectors t, t + blockDim, ...),
// exactly the access pattern of a plain stream: every wave instruction reads
// or writes 64 consecutive vectors.  D/8 divides 16, so a head row never
// straddles a 16-lane row of the wave, and the rotate-half partner of vector
// j (j + R/16 in the first half, j - R/16 in the second) sits in the same
// 16-lane row: it is fetched by a DPP row rotation, not a second load.  The
// lane reads its own 8 entries of the token's cos/sin rows (16 bytes each,
// shared through L1/L2 by every head and view of the token) ahead of x, so
// there is no LDS staging and no barrier.  Vectors past R/8 in a head are the
// tail, copied (or skipped in place).
// ---------------------------------------------------------------------------
template <int Ror>
__device__ __forceinline__ uint32_t row_ror(uint32_t v)
{
    // DPP row_ror:Ror (0x120 + Ror): lane l of a 16-lane row reads lane
    // (l - Ror) mod 16 of the same row.
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + Ror, 0xF, 0xF, false);
}

template <int HV>
__device__ __forceinline__ v4u partner_vec(v4u x, bool first_half)
{
    // first half: the vector HV lanes up, negated (sign bits flipped, exact);
    // second half: the vector HV lanes down.
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t dn = row_ror<HV>(w[k]);
        const uint32_t up = HV == 8 ? dn : row_ror<16 - HV>(w[k]);
        w[k] = first_half ? up ^ 0x80008000u : dn;
    }
    return v4u{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ uint32_t rope_word_bf(uint32_t x, uint32_t y, uint32_t c, uint32_t s)
{
    uint32_t p0 = rne_pack(bf_lo(x) * bf_lo(c), bf_lo(y) * bf_lo(s));
    uint32_t p1 = rne_pack(bf_hi(x) * bf_hi(c), bf_hi(y) * bf_hi(s));
    return rne_pack(bf_lo(p0) + bf_hi(p0), bf_lo(p1) + bf_hi(p1));
}

// Stores of whole lines go out as buffer stores carrying the nontemporal and
// device-scope write-through (sc1) bits, which measured 1-2% faster than
// nontemporal alone; the wave's first live lane gives the base and the
// others 32-bit byte offsets from it (a wave's 64 vectors then sit in one
// token's contiguous head rows, a 1 KiB span).
__device__ __forceinline__ void store16_lines(uint16_t *out, int64_t oo, bool live, v4u v)
{
    const uint64_t m = __builtin_amdgcn_ballot_w64(live);
    if (m == 0)
        return;
    const int first = (int)__builtin_ctzll(m);
    const int64_t o0 = ((int64_t)__builtin_amdgcn_readlane((int)(oo >> 32), first) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)oo, first);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(out + o0, 0, 0x7FFFFFF0, 0x00020000);
    if (live)
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (uint32_t)((oo - o0) * 2), 0, 2 | 16);
}

// The loads and the rotation of VPL vectors per lane for chunk `chunk` of
// view V (vectors chunk * chunk_vecs + threadIdx.x + u * blockDim.x).
template <int HV, int VPL, bool Lines>
struct XlaneState {
    v4u c[VPL], s[VPL], x[VPL];
    int64_t oo[VPL];
    int j[VPL];
    bool live[VPL];

    __device__ __forceinline__ void fetch(const RopeParams &p, const RopeView &V, uint32_t chunk)
    {
        const uint32_t total = p.vecs_per_view;
        const uint32_t vmask = (1u << p.log_vecs) - 1u;
        const uint32_t base = chunk * (uint32_t)p.chunk_vecs + threadIdx.x;
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const uint32_t g0 = base + u * blockDim.x;
            live[u] = g0 < total;
            const uint32_t g = min(g0, total - 1u);
            j[u] = (int)(g & vmask);
            const uint32_t hh = g >> p.log_vecs;
            const uint32_t t = fdiv(hh, p.div_heads);
            const uint32_t h = hh - t * (uint32_t)p.H;
            const uint32_t b = fdiv(t, p.div_s);
            const uint32_t sq = t - b * p.div_s.d;
            const int64_t tab = (int64_t)t * p.R + min(j[u], 2 * HV - 1) * 8;
            c[u] = *reinterpret_cast<const v4u *>(p.cos + tab);
            s[u] = *reinterpret_cast<const v4u *>(p.sin + tab);
            const int64_t xo = (int64_t)b * V.xs_b + (int64_t)sq * V.xs_s + (int64_t)h * V.xs_h + j[u] * 8;
            oo[u] = (int64_t)b * V.os_b + (int64_t)sq * V.os_s + (int64_t)h * V.os_h + j[u] * 8;
            x[u] = load16<Lines>(V.x + xo);
        }
    }

    // Every lane forms the rotation (tail lanes on a clamped table entry) and
    // then keeps it or its input, so no load sits under a branch.
    __device__ __forceinline__ void finish(const RopeView &V, bool tail)
    {
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const v4u xx = x[u], cc = c[u], sn = s[u];
            const v4u y = partner_vec<HV>(xx, j[u] < HV);
            const v4u r = v4u{rope_word_bf(xx.x, y.x, cc.x, sn.x), rope_word_bf(xx.y, y.y, cc.y, sn.y),
                              rope_word_bf(xx.z, y.z, cc.z, sn.z), rope_word_bf(xx.w, y.w, cc.w, sn.w)};
            const bool rot = j[u] < 2 * HV;
            const bool st = live[u] && (rot || tail);
            if constexpr (Lines)
                store16_lines(V.out, oo[u], st, rot ? r : xx);
            else if (st)
                store16<false>(V.out + oo[u], rot ? r : xx);
        }
    }
};

// One pass over a (chunks, views) grid: workgroup (w, v) takes chunk w of
// view v; the view index is known when the wave starts, so all parameters
// arrive in one batch of scalar loads.
template <int HV, int VPL, bool Lines>
__global__ __launch_bounds__(1024) void rope_xlane_kernel(RopeParams p)
{
    const int v = (int)blockIdx.y;
    const RopeView V = p.v[v];
    XlaneState<HV, VPL, Lines> st;
    st.fetch(p, V, blockIdx.x);
    __builtin_amdgcn_sched_barrier(0);  // every load goes out before anything waits
    st.finish(V, (p.tail_mask >> v) & 1);
}

// Rotate-half RoPE on token-linear layouts                [ERNIE-fuse §2]
//
// The common layout: every view's heads are contiguous within a token
// (stride_h == D), batch rows follow each other in token order (stride_b ==
// S * stride_s), and a token's heads fill whole waves (H * D/8 a multiple of
// 64).  Each wave's 64 vectors are then one contiguous 1 KiB run of one
// token, so the token, the row base and the table row are computed once per
// wave in scalar registers, the loads and stores are buffer instructions
// with a scalar base and the lane's fixed 16 * lane byte offset, and the
// lane's work is only its loads, the DPP partner exchange, the rotation and
// one store: about 90 vector instructions per 16-byte vector against 170
// for the per-lane addressing of rope_xlane_kernel, which left the kernel
// short of a plain stream at 136 MB.  Workgroup (w, v) of the (chunks,
// views) grid takes vectors 256 w .. 256 w + 255 of view v: one view after
// the other.
__device__ __forceinline__ uint32_t rope_word_f(uint32_t x, uint32_t y, float c0, float c1,
                                                float s0, float s1)
{
    uint32_t p0 = rne_pack(bf_lo(x) * c0, bf_lo(y) * s0);
    uint32_t p1 = rne_pack(bf_hi(x) * c1, bf_hi(y) * s1);
    return rne_pack(bf_lo(p0) + bf_hi(p0), bf_lo(p1) + bf_hi(p1));
}

template <int HV>
__global__ __launch_bounds__(256) void rope_lean_kernel(RopeParams p)
{
    // grid (chunks, n_views): the view index is known when the wave starts,
    // so its parameters load in the same batch as the others
    const uint32_t v = blockIdx.y;
    const uint32_t blk = blockIdx.x;
    const RopeView &V = p.v[v];
    const bool keep_tail = (p.tail_mask >> v) & 1;
    uint16_t *const out = V.out;
    const uint16_t *const xin = V.x;
    const int64_t os_s = V.os_s, xs_s = V.xs_s;
    // every parameter is needed in scalar registers before the first load:
    // one batch of scalar loads, one wait
    asm volatile("" ::"s"(out), "s"(xin), "s"(os_s), "s"(xs_s), "s"(p.cos), "s"(p.sin),
                 "s"(p.div_vecs.m), "s"(p.div_vecs.l), "s"(p.div_vecs.d), "s"(p.vecs_per_view),
                 "s"(p.log_vecs), "s"(p.R), "s"(p.tail_mask));
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = (int)(lane & ((1u << p.log_vecs) - 1u));
    const bool rot = j < 2 * HV;

    // g of the wave's first vector (uniform); a wave past the end re-reads
    // the last one and stores nothing
    const uint32_t gw = blk * 256u + wave * 64u;
    const bool live = gw < p.vecs_per_view;
    const uint32_t g = min(gw, p.vecs_per_view - 64u);
    const uint32_t t = fdiv(g, p.div_vecs);  // divisor H * D/8
    const uint32_t w0 = g - t * p.div_vecs.d;
    const uint32_t tab_lane = (uint32_t)min(j, 2 * HV - 1) * 16u;  // bytes
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.cos + (uint64_t)t * (uint32_t)p.R), 0, p.R * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsn = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.sin + (uint64_t)t * (uint32_t)p.R), 0, p.R * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(xin + ((uint64_t)t * (uint64_t)xs_s + w0 * 8u)), 0, 1024, 0x00020000);
    const v4u cv = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rc, tab_lane, 0, 0));
    v4u sv = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rsn, tab_lane, 0, 0));
    // nontemporal (aux bit 1): x is read once
    const v4u xx = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rx, lane * 16u, 0, 2));
    __builtin_amdgcn_sched_barrier(0);  // all three loads go out before anything waits

    // sin of the first half negated (exact): rne(-x' s) = rne(x' (-s))
    sv ^= j < HV ? 0x80008000u : 0u;
    float c[8], s8[8];
    c[0] = bf_lo(cv.x); c[1] = bf_hi(cv.x); c[2] = bf_lo(cv.y); c[3] = bf_hi(cv.y);
    c[4] = bf_lo(cv.z); c[5] = bf_hi(cv.z); c[6] = bf_lo(cv.w); c[7] = bf_hi(cv.w);
    s8[0] = bf_lo(sv.x); s8[1] = bf_hi(sv.x); s8[2] = bf_lo(sv.y); s8[3] = bf_hi(sv.y);
    s8[4] = bf_lo(sv.z); s8[5] = bf_hi(sv.z); s8[6] = bf_lo(sv.w); s8[7] = bf_hi(sv.w);
    uint32_t yw[4] = {xx.x, xx.y, xx.z, xx.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // both rotations in every lane (a DPP read of a lane that a branch
        // has switched off would not return its value)
        const uint32_t dn = row_ror<HV>(yw[k]);
        const uint32_t up = HV == 8 ? dn : row_ror<16 - HV>(yw[k]);
        yw[k] = j < HV ? up : dn;
    }
    const v4u r = v4u{rope_word_f(xx.x, yw[0], c[0], c[1], s8[0], s8[1]),
                      rope_word_f(xx.y, yw[1], c[2], c[3], s8[2], s8[3]),
                      rope_word_f(xx.z, yw[2], c[4], c[5], s8[4], s8[5]),
                      rope_word_f(xx.w, yw[3], c[6], c[7], s8[6], s8[7])};
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        out + ((uint64_t)t * (uint64_t)os_s + w0 * 8u), 0, 1024, 0x00020000);
    // nontemporal and write-through (aux bits 1 and 4)
    if (live && (rot || keep_tail))
        __builtin_amdgcn_raw_buffer_store_b128(rot ? r : xx, ro, lane * 16u, 0, 2 | 16);
}

// ---------------------------------------------------------------------------
// GEGLU with activation rounding             [ERNIE-fuse §3]
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
// The common path (|x| in [2^-125, 16)) is branch-free; a vector holding an
// input outside it (rare: |x| < 2^-125 or >= 16) is redone by the general
// path.  The multiply by up is exact in fp32 and rounded once.
//
// Layout of the work: one 16-byte vector (8 outputs) per lane.  The lane
// fetches its 16-byte share of the table (an L2 hit), then issues its gate
// and up loads, then writes the table share to LDS: loads return in order,
// so the table fill and the barrier overlap the HBM latency of gate and up.
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

// G, as fp32 bits, for a bf16 gate whose magnitude is in [2^-125, 16).
__device__ __forceinline__ uint32_t gelu_common(uint32_t g, const uint16_t *lut)
{
    uint32_t a = g & 0x7FFFu;
    uint32_t idx = max(a, kLutLo) - kLutLo + (g >> 15) * kLutSpan;
    uint32_t t = lut[idx];
    return (a < kLutLo ? g - 0x80u : t) << 16;
}

// G, as bf16 bits, for any bf16 gate.
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
        return gelu_common(g, lut) >> 16;
    return neg ? (0x8000u | (a >> 1)) : ((a + 1u) >> 1);
}

// True if either bf16 of the word has a magnitude outside [2^-125, 16).
__device__ __forceinline__ bool word_needs_general(uint32_t w)
{
    uint32_t lo = (w & 0x7FFFu) - 0x0100u;
    uint32_t hi = ((w >> 16) & 0x7FFFu) - 0x0100u;
    return max(lo, hi) >= kLutHi - 0x0100u;
}

__device__ __forceinline__ uint32_t geglu_word_common(uint32_t gw, uint32_t uw,
                                                      const uint16_t *lut)
{
    float g0 = __uint_as_float(gelu_common(gw & 0xFFFFu, lut));
    float g1 = __uint_as_float(gelu_common(gw >> 16, lut));
    return rne_pack(bf_lo(uw) * g0, bf_hi(uw) * g1);
}

__device__ __noinline__ v4u geglu_vec_general(v4u g, v4u u, const uint16_t *lut)
{
    uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w}, o[4];
    for (int k = 0; k < 4; ++k) {
        float g0 = __uint_as_float(gelu_general(gw[k] & 0xFFFFu, lut) << 16);
        float g1 = __uint_as_float(gelu_general(gw[k] >> 16, lut) << 16);
        o[k] = rne_pack(bf_lo(uw[k]) * g0, bf_hi(uw[k]) * g1);
    }
    return v4u{o[0], o[1], o[2], o[3]};
}

__device__ __forceinline__ v4u geglu_vec(v4u g, v4u u, const uint16_t *lut)
{
    v4u o = v4u{geglu_word_common(g.x, u.x, lut), geglu_word_common(g.y, u.y, lut),
                geglu_word_common(g.z, u.z, lut), geglu_word_common(g.w, u.w, lut)};
    bool general = (int)word_needs_general(g.x) | (int)word_needs_general(g.y) |
                   (int)word_needs_general(g.z) | (int)word_needs_general(g.w);
    if (general)
        o = geglu_vec_general(g, u, lut);
    return o;
}

constexpr int kGegluBlock = 512;

// Lines: every wave's 64 output vectors are one contiguous, line-aligned
// 1 KiB run (rows of a multiple of 512 columns, line-aligned row starts), so
// the store goes out as a buffer store with the write-through bit as well.
template <bool Lines>
__global__ __launch_bounds__(kGegluBlock) void gelu_and_mul_kernel(GegluParams p)
{
    __shared__ __align__(16) uint16_t lut[kLutEntries];
    // The lane's table vector is fetched before its gate/up vectors: loads
    // return in order, so the LDS fill and the barrier then overlap the HBM
    // latency instead of waiting for it.
    static_assert(kLutEntries / 8 <= kGegluBlock, "one table vector per lane");
    const uint32_t kt = min(threadIdx.x, kLutEntries / 8 - 1);
    const v4u tv = reinterpret_cast<const v4u *>(g_gelu_lut)[kt];
    __builtin_amdgcn_sched_barrier(0);  // keep the table fetch ahead of gate/up
    // Lanes past the end re-read the last vector (no load under a branch).
    const uint32_t i = blockIdx.x * kGegluBlock + threadIdx.x;
    const uint32_t j = min(i, p.vec_total - 1);
    const uint32_t row = fdiv(j, p.div_vecs);
    const uint32_t col = (j - row * p.div_vecs.d) * 8;
    const uint16_t *src = p.in + (int64_t)row * p.in_stride + col;
    const v4u g = stream_load(src);
    const v4u u = stream_load(src + p.hidden);
    if (threadIdx.x < kLutEntries / 8)
        reinterpret_cast<v4u *>(lut)[threadIdx.x] = tv;
    __syncthreads();
    const v4u o = geglu_vec(g, u, lut);
    const int64_t oo = (int64_t)row * p.out_stride + col;
    if constexpr (Lines)
        store16_lines(p.out, oo, i < p.vec_total, o);
    else if (i < p.vec_total)
        stream_store(p.out + oo, o);
}

// ---------------------------------------------------------------------------
// GEGLU as the epilogue of the gate_up projection      [ERNIE-fuse §3]
//
// out = x W^T on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation), the eager bf16 rounding of the projection applied to each
// accumulator, then either stored or turned into up * G(gate) in the
// epilogue, so the (M, 2H) intermediate never goes to memory.
//
// A 256-thread workgroup (one wave per SIMD, its 256 accumulators in the
// AGPRs) computes a 256-row x 128-column block of the output: per 64-wide
// slice of K it stages 256 rows of x and the 128 gate rows plus the 128
// matching up rows of W in LDS.  Wave (wm, wn) owns rows wm*128 .. +127 and
// columns wn*64 .. +63 of both the gate and the up block, so one lane holds
// the gate and the up accumulator of the same (row, column).  W is the
// first MFMA operand and x the second; in a 16x16 block lane l holds output
// row l % 16 and, in its four accumulators, output columns 4 (l / 16) .. +3.
// Operands: lane l supplies row l % 16 of a 16-row block of W or of x and
// the 8 consecutive k at 8 (l / 16) of a 32-wide step.
//
// Staging uses the direct global-to-LDS load (16 bytes per lane, one 1 KiB
// run of LDS per instruction: 8 rows of 128 bytes), so the slices never pass
// through registers.  Rows are unpadded; the 16-byte chunk c of row r sits
// at chunk c ^ ((r / 2) % 8).  A 16-byte LDS read serves 16 lanes per cycle
// from 64 four-byte banks; in an operand fetch those lanes read 16
// consecutive rows at one logical chunk, and the swizzle puts them on 16
// disjoint 16-byte bank groups (row r starts at group 8 (r % 2)).  Two
// stages of 64 KiB: slice kt + 1 is loaded into one while slice kt is read
// from the other.
//
// Per slice each wave issues 128 products in 2 steps of 64, product
// (jb, ib) = (x block, W block) at 8 jb + ib.  The 8 W fragments of a step
// stay in registers for the whole step (two sets, alternating); the x
// fragments stream through a ring of four, each read 16 products before its
// first use.  Step 0 issues the 16 loads of the next slice, one per three
// products, and reads step 1's W fragments.  The last read of the current
// stage is at product 40 of step 1; at product 48 the wave waits for its
// loads and its reads, and passes the barrier that publishes the next slice
// and frees this one; the next slice's W fragments and first x fragments
// are read over the remaining 16 products, so its first products find them
// in registers.
//
// Workgroups go to the 8 XCDs round robin; the block index is remapped so
// that each XCD gets one contiguous run of tiles, and the run is walked in
// groups of 8 row blocks (column block outer), so the tiles an XCD works on
// at one time share rows of x and of W in its L2.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <bool B>
struct GeluPath {  // compile-time choice of the epilogue's GELU path
    static constexpr bool value = B;
};

constexpr int kGemmBM = 256;              // rows of x per workgroup
constexpr int kGemmBN = 128;              // gate (and up) columns per workgroup
constexpr int kGemmBK = 64;               // K slice per stage (128-byte rows)
constexpr int kGemmStages = 2;
constexpr int kGemmLutBytes = kLutEntries * 2;       // GELU table at LDS offset 0
constexpr int kGemmOpBytes = 256 * kGemmBK * 2;      // one staged operand (x or W)
constexpr int kGemmStageBytes = 2 * kGemmOpBytes;
constexpr size_t kGemmLds = kGemmLutBytes + kGemmStages * kGemmStageBytes;
constexpr uint32_t kGemmGroupM = 8;
constexpr int kGemmThreads = 256;
constexpr int kGemmBarrierAt = 48;        // product of step 1 that the barrier precedes
constexpr int kGemmLoadEvery = 3;         // step 0 issues one load per this many products
constexpr int kGemmStaggerRow = 4;        // K-walk offset (slices) per row block of a group
constexpr int kGemmStaggerCol = 1;        // and per column block
// The barrier must follow the last read of the current stage (the x block
// read at product 40 of step 1) and precede the first read of the next one
// (product 48); the loads stay in step 0.
static_assert(kGemmBarrierAt > 40 && kGemmBarrierAt <= 48, "barrier between the two stages' reads");
static_assert(16 * kGemmLoadEvery <= 64, "the next slice's loads go out in step 0");
static_assert(kGemmLds <= 160 * 1024, "LDS of one CU");
static_assert(kGemmLutBytes % 1024 == 0, "stages start on a 1 KiB boundary");
static_assert(4 * 128 * 64 * 2 <= kGemmStageBytes, "epilogue blocks fit stage 1");
static_assert(kLutEntries % 8 == 0 && kLutEntries / 8 <= 2 * kGemmThreads, "table: two vectors per lane");

#define RGG_FENCE() __builtin_amdgcn_sched_barrier(0)

// Tile t of T (in launch order) -> (row block, column block): the XCD run
// remap, then groups of kGemmGroupM row blocks with the column block outer.
__device__ __forceinline__ void gemm_tile(const GemmParams &p, uint32_t t, int64_t &m0, int32_t &n0)
{
    const uint32_t T = p.mblocks * p.nblocks;
    if ((T & 7) == 0)
        t = (t & 7) * (T >> 3) + (t >> 3);
    const uint32_t span = kGemmGroupM * p.nblocks;
    const uint32_t grp = t / span, r = t - grp * span;
    const uint32_t first = grp * kGemmGroupM;
    const uint32_t gm = min(kGemmGroupM, p.mblocks - first);
    m0 = (int64_t)(first + r % gm) * kGemmBM;
    n0 = (int32_t)(r / gm) * kGemmBN;
}

template <bool Geglu>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_gate_up_kernel(GemmParams p)
{
    // [GELU table][stage 0: x | W][stage 1: x | W]
    extern __shared__ __align__(16) uint8_t gsm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t T = p.mblocks * p.nblocks;

    // The GELU table goes to LDS now; it is read in the epilogues, after
    // barriers that order these writes before those reads.
    if (Geglu) {
        constexpr int nv = kLutEntries / 8;
        const v4u *src = reinterpret_cast<const v4u *>(g_gelu_lut);
        v4u *dst = reinterpret_cast<v4u *>(gsm);
        if (tid < nv)
            dst[tid] = src[tid];
        if (tid + kGemmThreads < nv)
            dst[tid + kGemmThreads] = src[tid + kGemmThreads];
    }

    // Wave w stages row groups 8w .. 8w + 7 (8 rows each) of the x tile and
    // of the W tile (waves 0-1: gate rows, 2-3: up rows): lane i of group g
    // brings row 8g + i / 8, logical chunk (i % 8) ^ ((4g + i / 16) % 8), to
    // LDS chunk i % 8 of that row.  Rows past M re-read row M-1 and columns
    // past H re-read column H-1 (not stored).  The loads address memory as a
    // wave-uniform base (SGPRs: the tile's first x row, the first gate or up
    // row of this wave's W rows) plus a per-lane 32-bit byte offset fixed for
    // the tile; the slice only moves the base.  Offsets stay below 256 row
    // strides; strides are limited to 2^22 elements, which keeps every offset
    // below 2^31.  (The lane index passes through an empty asm statement so
    // that the compiler recomputes the offsets per tile instead of keeping
    // loop-invariant copies alive across the tile loop.)
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t ox[8], ow[8];
    const uint16_t *bx = p.x, *bw = p.w;
    // The tile walks K starting at slice ks0 and wrapping around.  The 32
    // tiles an XCD works on at once (8 row blocks x 4 column blocks, see
    // gemm_tile) start kGemmStaggerRow slices apart per row block and
    // kGemmStaggerCol per column block, so they do not all request the same
    // 128-byte column window of x and W at the same moment; tiles that share
    // an x block stay within 3 slices of each other and so still meet its
    // lines in L2.  (Every tile sums its K slices in its own fixed order,
    // the same for the plain and the fused product.)
    const int KT = p.K / kGemmBK;
    int ks0 = 0;
    auto point = [&](int64_t m0, int32_t n0) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        bx = p.x + m0 * p.x_stride;
        bw = p.w + ((wv < 2 ? 0 : (int64_t)p.H) + n0) * p.w_stride;
        ks0 = KT > 0 ? (int)(((m0 / kGemmBM) % kGemmGroupM) * kGemmStaggerRow +
                             (n0 / kGemmBN) % 4 * kGemmStaggerCol) % KT
                     : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 64 * wv + 8 * j + (ln >> 3);
            const int chunk = (ln & 7) ^ ((4 * j + (ln >> 4)) & 7);
            const uint32_t m = (uint32_t)(min(m0 + row, p.M - 1) - m0);
            const uint32_t c = (uint32_t)(min(n0 + (row & (kGemmBN - 1)), p.H - 1) - n0);
            ox[j] = m * (uint32_t)p.x_stride * 2u + chunk * 16;
            ow[j] = c * (uint32_t)p.w_stride * 2u + chunk * 16;
        }
    };
    // One load instruction: row group 8w + idx % 8 of x (idx < 8) or of W.
    // It is written out (M0 holds the LDS address) rather than left to the
    // compiler, which does not know which LDS bytes a direct load writes and
    // would make every later LDS read wait for every load in flight; here
    // the ordering is explicit: a "vmcnt" wait before each barrier, and a
    // stage is only reloaded after the barrier that follows its last reads.
    // The instruction has no register result, and the statement declares
    // M0 among the registers it writes, so any code the compiler places
    // after it that needs M0 sets M0 again.  (M0 is a reserved register, so
    // the compiler notes that it does not save it across the statement:
    // nothing here needs it saved.)  The stages stay in one LDS array
    // indexed by the slice parity at run time: as separate arrays, with the
    // compiler's own direct-load intrinsic, every slice pair would be
    // unrolled and the kernel runs out of registers.
    const uint32_t lds0 = (uint32_t)(uintptr_t)gsm + kGemmLutBytes + wv * 8 * 1024;
    auto dma1 = [&](int kt, int st, int idx) {
        const int j = idx & 7;
        const int kk = kt + ks0 < KT ? kt + ks0 : kt + ks0 - KT;
        const uint16_t *base = (idx < 8 ? bx : bw) + (int64_t)kk * kGemmBK;
        const uint32_t off = idx < 8 ? ox[j] : ow[j];
        const uint32_t dst = lds0 + st * kGemmStageBytes + (idx < 8 ? 0 : kGemmOpBytes) + j * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // the note that M0 is reserved
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(base), "s"(dst) : "memory", "m0");
#pragma clang diagnostic pop
    };
    auto fetch = [&](int kt, int st) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
            dma1(kt, st, idx);
    };

    f32x4 acc[8][8];  // [x row block of 16][W block of 16: gate 0..3, up 0..3]

    // 16x16x32 products: lane l supplies row l % 16 of a 16-row block of W
    // (first operand) or of x (second) and the 8 k at 8 (l / 16) of the
    // 32-wide step; its 4 accumulators of a block are output row l % 16,
    // columns 4 (l / 16) .. +3.  The row's swizzle (r / 2) % 8 depends only
    // on l % 16 (blocks start on multiples of 16 rows).
    const int sw = (lane & 15) >> 1;
    const uint32_t lrow = (uint32_t)(lane & 15) * 128u;
    const uint32_t koff0 = lrow + (uint32_t)(((lane >> 4) ^ sw) << 4);
    const uint32_t koff1 = lrow + (uint32_t)(((4 + (lane >> 4)) ^ sw) << 4);
    const uint32_t xrow0 = (uint32_t)(wm * 128) * 128u;
    const uint32_t wrow0 = (uint32_t)kGemmOpBytes + (uint32_t)(wn * 64) * 128u;
    bf16x8 wf[2][8];  // W fragments of a step, double buffered
    bf16x8 xf[4];     // x fragments, a ring of four
    auto wread = [&](int st, int s, int set, int ib) {
        const uint8_t *b = gsm + kGemmLutBytes + st * kGemmStageBytes + wrow0 +
                           (ib < 4 ? ib * 2048 : 128 * 128 + (ib - 4) * 2048);
        wf[set][ib] = *reinterpret_cast<const bf16x8 *>(b + (s ? koff1 : koff0));
    };
    auto xread = [&](int st, int s, int jb) {
        const uint8_t *b = gsm + kGemmLutBytes + st * kGemmStageBytes + xrow0 + jb * 2048;
        xf[jb & 3] = *reinterpret_cast<const bf16x8 *>(b + (s ? koff1 : koff0));
    };
    auto mma1 = [&](int set, int jb, int ib) {
        acc[jb][ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[set][ib], xf[jb & 3], acc[jb][ib], 0, 0, 0);
    };

    uint32_t tile = blockIdx.x;
    int64_t m0;
    int32_t n0;
    gemm_tile(p, tile, m0, n0);
    point(m0, n0);
    if (KT > 0) {
        fetch(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    for (;;) {
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b)
                acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        // One slice: two 32-wide steps of 64 products, product (jb, ib) at
        // 8 jb + ib.  Step 0 carries the 16 loads of the next slice (one per
        // three products) and the reads of step 1's W fragments; x fragments
        // are read two blocks (16 products) ahead.  In step 1, at product 48
        // the wave waits for its loads and its reads and passes the barrier
        // that publishes the next slice and frees this one; the next slice's
        // W fragments and first two x fragments follow.
        auto slice = [&](int kt, bool last) {
            const int st = kt & 1, sn = st ^ 1;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int pp = 0; pp < 64; ++pp) {
                    const int jb = pp >> 3, ib = pp & 7;
                    if (s == 1 && pp == kGemmBarrierAt && !last) {
                        asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)" ::: "memory");
                        __builtin_amdgcn_s_barrier();
                        RGG_FENCE();
                    }
                    mma1(s, jb, ib);
                    // x fragments: block jb + 2 of this step, or blocks 0, 1
                    // of the next step (of the next slice after step 1)
                    if (ib == 0) {
                        if (jb < 6)
                            xread(st, s, jb + 2);
                        else if (s == 0)
                            xread(st, 1, jb - 6);
                        else if (!last)
                            xread(sn, 0, jb - 6);
                    }
                    if (s == 0 && pp >= 8 && pp < 16)
                        wread(st, 1, 1, pp - 8);
                    if (s == 1 && pp >= kGemmBarrierAt && pp < kGemmBarrierAt + 8 && !last)
                        wread(sn, 0, 0, pp - kGemmBarrierAt);
                    if (s == 0 && !last && pp < 16 * kGemmLoadEvery && pp % kGemmLoadEvery == 0)
                        dma1(kt + 1, sn, pp / kGemmLoadEvery);
                    RGG_FENCE();
                }
            }
        };
        if (KT > 0) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
                wread(0, 0, 0, ib);
            xread(0, 0, 0);
            xread(0, 0, 1);
            RGG_FENCE();
            for (int kt = 0; kt + 1 < KT; ++kt)
                slice(kt, false);
            slice(KT - 1, true);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // every wave is done with the operand stages

        const int64_t cm0 = m0;
        const int32_t cn0 = n0;
        const uint32_t next = tile + gridDim.x;
        const bool more = next < T;
        if (more) {
            gemm_tile(p, next, m0, n0);
            point(m0, n0);
            if (KT > 0)
                fetch(0, 0);
        }

        // Epilogue: round each accumulator to bf16, then keep it or form
        // rne(up * G(gate)); the wave's 128 x 64 block goes through its
        // 16 KiB of stage 1 (128-byte rows, chunk c of row r at c ^ (r % 8),
        // 8 bytes = 4 columns per lane write) and out as 16-byte vectors.
        const uint16_t *lut = reinterpret_cast<const uint16_t *>(gsm);
        uint8_t *ep = gsm + kGemmLutBytes + kGemmStageBytes + wave * 16384;
        int el = lane;
        asm volatile("" : "+v"(el));
        const int32_t cbase = cn0 + wn * 64;
        const bool live = cbase < p.H;
        bool anyg = false;
        // The gates rounded to bf16 once, two to a word, for both the path
        // test and the table reads: gp[jb][ib][0] holds the lane's columns 0
        // and 1 of block (jb, ib), [1] columns 2 and 3.
        uint32_t gp[8][4][2];
        if (Geglu) {
            bool general = false;
#pragma unroll
            for (int jb = 0; jb < 8; ++jb)
#pragma unroll
                for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t w = rne_pack(acc[jb][ib][2 * h], acc[jb][ib][2 * h + 1]);
                        gp[jb][ib][h] = w;
                        general |= (w & 0x7FFFu) - 0x0100u >= kLutHi - 0x0100u;
                        general |= ((w >> 16) & 0x7FFFu) - 0x0100u >= kLutHi - 0x0100u;
                    }
            anyg = __builtin_amdgcn_ballot_w64(general) != 0;
        }
        // The 32 blocks of a wave go through one branch-free pass, the
        // table path or the general one (chosen once for the wave above), so
        // the compiler can keep several blocks' table reads in flight.
        // Per row of blocks, all 16 table reads go out before the row's
        // results are written to the staging area (LDS operations stay in
        // order, so a write between them would hold the next reads back).
        auto stage = [&](int half, auto general) {
#pragma unroll
            for (int jb = 0; jb < 8; ++jb) {
                uint32_t w[4][2];
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    if (Geglu) {
                        float G[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const uint32_t g = (gp[jb][ib][v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
                            G[v] = decltype(general)::value ? __uint_as_float(gelu_general(g, lut) << 16)
                                                            : __uint_as_float(gelu_common(g, lut));
                        }
                        // up rounded to bf16 two at a time, then widened back
                        const f32x4 &u = acc[jb][ib + 4];
                        const uint32_t u01 = rne_pack(u[0], u[1]), u23 = rne_pack(u[2], u[3]);
                        w[ib][0] = rne_pack(bf_lo(u01) * G[0], bf_hi(u01) * G[1]);
                        w[ib][1] = rne_pack(bf_lo(u23) * G[2], bf_hi(u23) * G[3]);
                    } else {
                        const f32x4 &a = acc[jb][ib + 4 * half];
                        w[ib][0] = rne_pack(a[0], a[1]);
                        w[ib][1] = rne_pack(a[2], a[3]);
                    }
                }
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    const int r = jb * 16 + (el & 15), col = ib * 16 + (el >> 4) * 4;
                    const int chunk = col >> 3;
                    *reinterpret_cast<uint2 *>(ep + r * 128 + ((chunk ^ (r & 7)) << 4) + (col & 4) * 2) =
                        make_uint2(w[ib][0], w[ib][1]);
                }
            }
        };
#pragma unroll
        for (int half = 0; half < (Geglu ? 1 : 2); ++half) {
            if (anyg)
                stage(half, GeluPath<true>{});
            else
                stage(half, GeluPath<false>{});
            // A wave reads back only its own block, and LDS operations of
            // one wave complete in order: no barrier (which would also wait
            // for the next tile's loads).
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            uint16_t *ob = p.out + (half ? p.H : 0) + cbase;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int rr = (el >> 3) + 8 * k, cv = el & 7;
                const v4u val = *reinterpret_cast<const v4u *>(ep + rr * 128 + ((cv ^ (rr & 7)) << 4));
                const int64_t row = cm0 + wm * 128 + rr;
                if (live && row < p.M)
                    *reinterpret_cast<v4u *>(ob + row * p.out_stride + cv * 8) = val;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        if (!more)
            break;
        tile = next;
        // The first barrier: every wave has left its block area in stage 1,
        // which the new tile's slice 1 will fill.  Then each wave waits for
        // its loads of slice 0 (and this tile's stores), and the second
        // barrier makes slice 0 visible to all.
        __builtin_amdgcn_s_barrier();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    }
}
#undef RGG_FENCE

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_rope_cossin(const CosSinParams &params, hipStream_t stream)
{
    CosSinParams p = params;
    const uint32_t rows = p.vec_total / (uint32_t)(p.R / 8);
    const bool paired = p.R % 16 == 0;
    const bool narrow = paired && (uint64_t)rows * (uint32_t)(p.R / 8) <= kTableNarrowLanes;
    const uint32_t per_row = paired && !narrow ? (uint32_t)(p.R / 16) : (uint32_t)(p.R / 8);
    p.vec_total = rows * per_row;
    p.div_vecs = make_fastdiv(per_row);
    uint32_t blocks = (p.vec_total + kThreads - 1) / kThreads;
    if (blocks > 4096)
        blocks = 4096;
    if (narrow)
        hipLaunchKernelGGL((rope_cossin_kernel<true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
    else if (paired)
        hipLaunchKernelGGL((rope_cossin_kernel<true, false>), dim3(blocks), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((rope_cossin_kernel<false, false>), dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_rope_cossin_grid(const CosSinGridParams &params, hipStream_t stream)
{
    CosSinGridParams p = params;
    const bool narrow = (uint64_t)p.rows * (uint32_t)(p.R / 8) <= kTableNarrowLanes;
    const uint32_t per_row = (uint32_t)(p.R / (narrow ? 8 : 16));
    p.groups_total = p.rows * per_row;
    p.div_groups = make_fastdiv(per_row);
    uint32_t blocks = (p.groups_total + kThreads - 1) / kThreads;
    if (blocks > 2048)
        blocks = 2048;
    const size_t lds = (size_t)(p.R / 2) * sizeof(double);
    if (narrow)
        hipLaunchKernelGGL(rope_cossin_grid_kernel<4>, dim3(blocks), dim3(kThreads), lds, stream, p);
    else
        hipLaunchKernelGGL(rope_cossin_grid_kernel<8>, dim3(blocks), dim3(kThreads), lds, stream, p);
    return hipGetLastError();
}

// The cross-lane kernels take heads of 8..128 columns (D/8 a power of two,
// so a head row sits in one 16-lane row of a wave) with a rotation, and
// views of fewer than 2^31 vectors.
// Heads contiguous within a token in every view (stride_h == D), at most 128
// columns, a power-of-two number of vectors per head.  Head-major layouts
// such as the (B, H, S, D) attention input go to the item kernels, which
// measured 5% faster there (180 against 187-190 us at dit_layer).
static bool rope_xlane_fits(const RopeParams &p)
{
    const int dv = p.D / 8;
    const int64_t vecs = p.tokens * p.H * dv;
    if (!(p.R >= 16 && p.D <= 128 && (dv & (dv - 1)) == 0 && vecs > 0 && vecs < ((int64_t)1 << 31)))
        return false;
    for (int v = 0; v < p.n_views; ++v)
        if (p.v[v].xs_h != p.D || p.v[v].os_h != p.D)
            return false;
    return true;
}

// Token-linear views whose heads fill whole waves (rope_lean_kernel).
static bool rope_lean_fits(const RopeParams &p)
{
    if (!rope_xlane_fits(p) || (p.H * (p.D / 8)) % 64 != 0)
        return false;
    const int64_t S = p.div_s.d, B = p.tokens / S;
    for (int v = 0; v < p.n_views; ++v) {
        const RopeView &V = p.v[v];
        if (V.xs_h != p.D || V.os_h != p.D || V.xs_s >= ((int64_t)1 << 31) ||
            V.os_s >= ((int64_t)1 << 31))
            return false;
        if (B > 1 && (V.xs_b != S * V.xs_s || V.os_b != S * V.os_s))
            return false;
    }
    return true;
}

static int log2_vecs(int D)
{
    int l = 0;
    while ((1 << l) < D / 8)
        ++l;
    return l;
}

static void *rope_lean_pick(int hv)
{
    switch (hv) {
    case 1: return reinterpret_cast<void *>(rope_lean_kernel<1>);
    case 2: return reinterpret_cast<void *>(rope_lean_kernel<2>);
    case 3: return reinterpret_cast<void *>(rope_lean_kernel<3>);
    case 4: return reinterpret_cast<void *>(rope_lean_kernel<4>);
    case 5: return reinterpret_cast<void *>(rope_lean_kernel<5>);
    case 6: return reinterpret_cast<void *>(rope_lean_kernel<6>);
    case 7: return reinterpret_cast<void *>(rope_lean_kernel<7>);
    default: return reinterpret_cast<void *>(rope_lean_kernel<8>);
    }
}

template <int HV>
static void *rope_xlane_pick(bool lines)
{
    return lines ? reinterpret_cast<void *>(rope_xlane_kernel<HV, 2, true>)
                 : reinterpret_cast<void *>(rope_xlane_kernel<HV, 2, false>);
}

static void *rope_xlane_pick_hv(int hv, bool lines)
{
    switch (hv) {
    case 1: return rope_xlane_pick<1>(lines);
    case 2: return rope_xlane_pick<2>(lines);
    case 3: return rope_xlane_pick<3>(lines);
    case 4: return rope_xlane_pick<4>(lines);
    case 5: return rope_xlane_pick<5>(lines);
    case 6: return rope_xlane_pick<6>(lines);
    case 7: return rope_xlane_pick<7>(lines);
    default: return rope_xlane_pick<8>(lines);
    }
}

// One launch per view group: rope_lean_kernel, 256 vectors per workgroup,
// the views one after the other.
static hipError_t launch_rope_lean(const RopeParams &params, hipStream_t stream)
{
    RopeParams p = params;
    const int dv = p.D / 8;
    p.log_vecs = log2_vecs(p.D);
    p.vecs_per_view = (uint32_t)(p.tokens * p.H * dv);
    p.div_vecs = make_fastdiv((uint32_t)(p.H * dv));
    p.chunks = (uint32_t)(((int64_t)p.vecs_per_view + 255) / 256);
    p.chunk0 = 0;
    if ((int64_t)p.chunks * p.n_views >= ((int64_t)1 << 23))
        return hipErrorInvalidValue;  // excluded by rope_xlane_fits (vectors < 2^31)
    void *args[] = {&p};
    hipError_t e = hipLaunchKernel(rope_lean_pick(p.R / 16), dim3(p.chunks, (uint32_t)p.n_views),
                                   dim3(256), args, 0, stream);
    return e == hipSuccess ? hipGetLastError() : e;
}

// rope_xlane_kernel: two vectors per lane, 256 lanes per workgroup.
static hipError_t launch_rope_xlane(const RopeParams &params, hipStream_t stream)
{
    RopeParams p = params;
    const int dv = p.D / 8;
    p.log_vecs = log2_vecs(p.D);
    p.vecs_per_view = (uint32_t)(p.tokens * p.H * dv);
    p.chunk_vecs = 512;
    // Streaming stores (store16_lines) address a wave's 64 vectors from its
    // first live lane: with heads contiguous, a wave that lies in one token
    // (a token's vectors fill whole waves) is one contiguous 1 KiB run, and
    // whole 128-byte lines when rows start on line boundaries.
    bool lines = (p.H * dv) % 64 == 0;
    for (int v = 0; v < p.n_views; ++v) {
        const RopeView &V = p.v[v];
        lines = lines && V.xs_s % 64 == 0 && V.os_s % 64 == 0 && V.xs_b % 64 == 0 &&
                V.os_b % 64 == 0 && ((uintptr_t)V.x & 127) == 0 && ((uintptr_t)V.out & 127) == 0;
    }
    void *kernel = rope_xlane_pick_hv(p.R / 16, lines);
    // fewer than 2^31 vectors per view: fewer than 2^22 chunks of 512
    const uint32_t chunks = (uint32_t)(((int64_t)p.vecs_per_view + p.chunk_vecs - 1) / p.chunk_vecs);
    p.chunk0 = 0;
    void *args[] = {&p};
    hipError_t e = hipLaunchKernel(kernel, dim3(chunks, (uint32_t)p.n_views), dim3(256), args, 0,
                                   stream);
    return e == hipSuccess ? hipGetLastError() : e;
}

static hipError_t launch_rope_items(const RopeParams &params, hipStream_t stream);

hipError_t launch_rope_rotate_half(const RopeParams &params, hipStream_t stream)
{
    if (rope_lean_fits(params))
        return launch_rope_lean(params, stream);
    if (rope_xlane_fits(params))
        return launch_rope_xlane(params, stream);
    return launch_rope_items(params, stream);
}

static hipError_t launch_rope_items(const RopeParams &params, hipStream_t stream)
{
    RopeParams p = params;
    p.tok_per_wg = rope_tokens_per_workgroup(p.H, p.D, p.R);
    p.div_views = make_fastdiv((uint32_t)p.n_views);
    size_t lds = (size_t)p.tok_per_wg * p.R * 2 * sizeof(float);
    // One-token workgroups give each wave its own staged row unless the
    // copies would crowd LDS (wide rotations); then the workgroup shares one.
    const size_t wave_lds = (size_t)(kRopeBlock / 64) * p.R * 2 * sizeof(float);
    p.wave_stage = p.tok_per_wg == 1 && wave_lds <= 65536;
    if (p.wave_stage)
        lds = wave_lds;
    // Whole lines per instruction when each half (R/2 bf16 = R bytes) and
    // every row start are multiples of 128 bytes.
    bool lines = p.R % 128 == 0;
    for (int v = 0; v < p.n_views; ++v) {
        const RopeView &V = p.v[v];
        lines = lines && V.xs_h % 64 == 0 && V.os_h % 64 == 0 && V.xs_s % 64 == 0 &&
                V.os_s % 64 == 0 && ((uintptr_t)V.x & 127) == 0 && ((uintptr_t)V.out & 127) == 0;
    }
    // Items of one token and view (the widest view decides), and how many a
    // workgroup pass takes.
    int64_t items = (int64_t)p.H * (p.tail_mask ? p.slots_tail : p.half / 8);
    void (*kernel)(RopeParams);
    if (p.tok_per_wg == 1 && lines)
        kernel = rope_rotate_half_kernel<true, true>;
    else if (p.tok_per_wg == 1)
        kernel = rope_rotate_half_kernel<true, false>;
    else if (lines)
        kernel = rope_rotate_half_kernel<false, true>;
    else
        kernel = rope_rotate_half_kernel<false, false>;
    // When R/2 is not a whole number of 128-byte lines the two-vector items
    // split lines between store instructions; one contiguous vector per lane
    // keeps every line whole.
    const int all_tails = (1 << p.n_views) - 1;
    if (p.wave_stage && p.tail_mask == all_tails && p.R > 0 && !lines) {
        bool whole = p.D % 64 == 0;
        for (int v = 0; v < p.n_views; ++v) {
            const RopeView &V = p.v[v];
            whole = whole && V.xs_h % 64 == 0 && V.os_h % 64 == 0 && V.xs_s % 64 == 0 &&
                    V.os_s % 64 == 0 && ((uintptr_t)V.x & 127) == 0 && ((uintptr_t)V.out & 127) == 0;
        }
        if (whole) {
            p.div_vecs = make_fastdiv((uint32_t)(p.D / 8));
            kernel = rope_rotate_half_lane_kernel<true, 1>;
            items = (int64_t)p.H * (p.D / 8);
        }
    }
    // A one-token workgroup whose token needs k >= 2 whole passes hands them
    // to k workgroups instead (a partial last pass stays with the first).
    p.parts = p.tok_per_wg == 1 ? (int32_t)std::max<int64_t>(1, items / (kRopeBlock * kRopeUnroll))
                                : 1;
    p.div_vp = make_fastdiv((uint32_t)(p.n_views * p.parts));
    p.div_parts = make_fastdiv((uint32_t)p.parts);
    // A dispatch's grid is counted in 32-bit work-items, so very long token
    // ranges go out as several launches of at most kMaxRopeWorkgroups.
    const int64_t chunks = (p.tokens + p.tok_per_wg - 1) / p.tok_per_wg;
    const int64_t per_launch = kMaxRopeWorkgroups / (p.n_views * p.parts);
    for (int64_t c0 = 0; c0 < chunks; c0 += per_launch) {
        p.chunk0 = (uint32_t)c0;
        const int64_t n = chunks - c0 < per_launch ? chunks - c0 : per_launch;
        void *args[] = {&p};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel),
                                       dim3((uint32_t)(n * p.n_views * p.parts)), dim3(kRopeBlock), args,
                                       lds, stream);
        if (e == hipSuccess)
            e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// GEGLU workgroups also take 27 KiB of (unused) dynamic LDS: with the
// table's 7 KiB that holds a compute unit to 4 of them (160 KiB of LDS), which
// measured 0.5-1% faster than leaving residency to the register count
// (dit_layer 247.5 -> 244.7 us, geglu 93.0 -> 92.4-92.8 us); plain streams
// of the same 2:1 traffic show the same gain from a residency cap.
constexpr size_t kGegluLdsPad = 27 * 1024;

hipError_t launch_gelu_and_mul(const GegluParams &p, int grid, hipStream_t stream)
{
    const bool lines = p.hidden % 512 == 0 && p.out_stride % 64 == 0 && ((uintptr_t)p.out & 127) == 0;
    if (lines)
        hipLaunchKernelGGL(gelu_and_mul_kernel<true>, dim3(grid), dim3(kGegluBlock), kGegluLdsPad, stream, p);
    else
        hipLaunchKernelGGL(gelu_and_mul_kernel<false>, dim3(grid), dim3(kGegluBlock), kGegluLdsPad, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const GemmParams &p, bool geglu, hipStream_t stream)
{
    // The two stages and the table take 135 KiB of LDS, above the 64 KiB a
    // launch gets without asking.  The attribute is set once per device (it
    // belongs to the kernel as loaded on the current device).
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static hipError_t attr[kMaxDevices];
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev] {
        attr[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_gate_up_kernel<true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
        if (attr[dev] == hipSuccess)
            attr[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_gate_up_kernel<false>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
    });
    if (attr[dev] != hipSuccess)
        return attr[dev];
    // One workgroup per CU (the LDS use allows no more), each walking tiles.
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    const uint32_t tiles = p.mblocks * p.nblocks;
    const dim3 grid(min(tiles, (uint32_t)max(cus, 1))), block(kGemmThreads);
    if (geglu)
        hipLaunchKernelGGL(gemm_gate_up_kernel<true>, grid, block, kGemmLds, stream, p);
    else
        hipLaunchKernelGGL(gemm_gate_up_kernel<false>, grid, block, kGemmLds, stream, p);
    return hipGetLastError();
}

hipError_t launch_build_gelu_table(hipStream_t stream)
{
    hipLaunchKernelGGL(build_gelu_table_kernel, dim3((kLutEntries + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, stream);
    return hipGetLastError();
}

int rope_tokens_per_workgroup(int H, int D, int R)
{
    // Heads small enough that a token's work items fill under one
    // workgroup pass are grouped: the token count that fills the one or two
    // passes best (the fewest passes on a tie), with the fp32 cos/sin rows
    // within 32 KiB of LDS.
    const int64_t ipt = (int64_t)H * (R / 16 + (D - R) / 8);  // items per token
    if (ipt <= 0)
        return 64;
    int best = 1;
    double best_fill = 0.0;
    for (int t = 1; t <= 64 && t * ipt <= 2 * kRopeBlock && t * R * 8 <= 32768; ++t) {
        const int64_t n = t * ipt, passes = (n + kRopeBlock - 1) / kRopeBlock;
        const double fill = (double)n / (double)(passes * kRopeBlock);
        if (fill > best_fill + 1e-9) {
            best_fill = fill;
            best = t;
        }
    }
    return best;
}

int geglu_grid(uint32_t vec_total, int)
{
    // one 16-byte vector per lane, one pass
    const uint32_t blocks = (vec_total + kGegluBlock - 1) / kGegluBlock;
    return (int)(blocks == 0 ? 1 : blocks);
}

}  // namespace rgg

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

// Tunables.  The defaults are the fastest settings measured on MI355X; a
// build may override them with -D to sweep.
#ifndef RGG_STREAM_NT
#define RGG_STREAM_NT 1          // nontemporal hint on data touched once
#endif
#ifndef RGG_GEGLU_BLOCK
#define RGG_GEGLU_BLOCK 512      // GEGLU workgroup size
#endif
#ifndef RGG_GEGLU_VEC
#define RGG_GEGLU_VEC 1          // 16-byte vectors per lane (loads all issued first)
#endif
#ifndef RGG_GEGLU_WG_PER_CU
#define RGG_GEGLU_WG_PER_CU 0    // 0: one vector per lane, one pass per workgroup;
#endif                           // n: n resident workgroups per CU, grid-stride loop
#ifndef RGG_ROPE_VEC_PER_WG
#define RGG_ROPE_VEC_PER_WG 512  // 16-byte vectors of x per RoPE workgroup (one view)
#endif
#ifndef RGG_ROPE_BLOCK
#define RGG_ROPE_BLOCK 256       // RoPE workgroup size
#endif
#ifndef RGG_ROPE_UNROLL
#define RGG_ROPE_UNROLL 1        // RoPE items per lane with their loads issued together
#endif
#ifndef RGG_ROPE_WAVE_STAGE
#define RGG_ROPE_WAVE_STAGE 1    // one-token RoPE: each wave stages its own cos/sin copy (no barrier)
#endif
#ifndef RGG_ROPE_LANE
#define RGG_ROPE_LANE 1          // one-token launches whose half-rotation splits 128-byte lines:
#endif                           // one contiguous output vector per lane
#ifndef RGG_GEGLU_LUT_FIRST
#define RGG_GEGLU_LUT_FIRST 1    // GEGLU: fetch the lane's GELU-table vector before gate/up
#endif
#ifndef RGG_ROPE_TPW_FIT
#define RGG_ROPE_TPW_FIT 1       // tokens per workgroup: best lane fill of one or two passes
#endif
#ifndef RGG_STAGE_FIRST
#define RGG_STAGE_FIRST 1        // one-token RoPE, R <= 256: fetch the cos/sin row before x
#endif
#ifndef RGG_ROPE_LDS
#define RGG_ROPE_LDS 1           // 1: stage cos/sin rows in LDS; 0: read them per item
#endif
#ifndef RGG_COSSIN_COLS
#define RGG_COSSIN_COLS 8        // table columns per lane in the cos/sin kernel (8 or 4)
#endif

// Streamed data (read or written once) bypasses cache retention when
// RGG_STREAM_NT is set: the loads and stores carry the nontemporal bit.
__device__ __forceinline__ v4u stream_load(const uint16_t *p)
{
#if RGG_STREAM_NT
    return __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
#else
    return *reinterpret_cast<const v4u *>(p);
#endif
}

__device__ __forceinline__ void stream_store(uint16_t *p, v4u v)
{
#if RGG_STREAM_NT
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(p));
#else
    *reinterpret_cast<v4u *>(p) = v;
#endif
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
// One lane per 8 consecutive rotary columns of one table row: two 16-byte
// angle loads, eight fp32 sincosf, two 16-byte stores.  sincosf is accurate
// to a couple of fp32 ulps, so rounding its result to bf16 gives the
// correctly rounded bf16 of the true value unless the fp32 result lies within
// a few ulps of a bf16 rounding midpoint (its low 16 bits near 0x8000).
// Those few (about one in 7000) are recomputed in double and rounded exactly,
// so each entry is the correctly rounded bf16 of cos/sin of the fp32 angle.
// RGG_COSSIN_GUARD is that margin in fp32 ulps.
// ---------------------------------------------------------------------------
#ifndef RGG_COSSIN_GUARD
#define RGG_COSSIN_GUARD 4
#endif
constexpr uint32_t kTieGuard = RGG_COSSIN_GUARD;

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

constexpr int kCosSinCols = RGG_COSSIN_COLS;

__device__ __forceinline__ void cossin_vec8(v4u a0, v4u a1, uint32_t *c, uint32_t *sn)
{
    cossin_pair(__uint_as_float(a0.x), __uint_as_float(a0.y), c[0], sn[0]);
    cossin_pair(__uint_as_float(a0.z), __uint_as_float(a0.w), c[1], sn[1]);
    cossin_pair(__uint_as_float(a1.x), __uint_as_float(a1.y), c[2], sn[2]);
    cossin_pair(__uint_as_float(a1.z), __uint_as_float(a1.w), c[3], sn[3]);
}

// Paired form (R a multiple of 16): a lane owns columns 8g .. 8g+7 of both
// halves of a row.  Rotate-half angle tables usually repeat the first half
// in the second (cat(f, f)); when the eight angles of the second half are
// bitwise the first half's, their cos/sin are reused instead of recomputed.
template <bool Paired>
__global__ __launch_bounds__(kThreads) void rope_cossin_kernel(CosSinParams p)
{
    const uint32_t nvec_row = p.div_vecs.d;
    const uint32_t S = p.div_s.d;
    const int half = p.R / 2;
    for (uint32_t idx = blockIdx.x * kThreads + threadIdx.x; idx < p.vec_total;
         idx += gridDim.x * kThreads) {
        uint32_t row = fdiv(idx, p.div_vecs);
        uint32_t cg = idx - row * nvec_row;
        uint32_t b = fdiv(row, p.div_s);
        uint32_t s = row - b * S;
        const float *f = p.freqs + (int64_t)s * p.stride_s + (int64_t)b * p.stride_b;
        int64_t o = (int64_t)row * p.R;
        if constexpr (Paired) {
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
            const int col = cg * kCosSinCols;
            uint32_t c[kCosSinCols / 2], sn[kCosSinCols / 2];
            float4 f0 = reinterpret_cast<const float4 *>(f + col)[0];
            cossin_pair(f0.x, f0.y, c[0], sn[0]);
            cossin_pair(f0.z, f0.w, c[1], sn[1]);
            if constexpr (kCosSinCols == 8) {
                float4 f1 = reinterpret_cast<const float4 *>(f + col)[1];
                cossin_pair(f1.x, f1.y, c[2], sn[2]);
                cossin_pair(f1.z, f1.w, c[3], sn[3]);
                *reinterpret_cast<v4u *>(p.cos + o + col) = v4u{c[0], c[1], c[2], c[3]};
                *reinterpret_cast<v4u *>(p.sin + o + col) = v4u{sn[0], sn[1], sn[2], sn[3]};
            } else {
                *reinterpret_cast<uint2 *>(p.cos + o + col) = make_uint2(c[0], c[1]);
                *reinterpret_cast<uint2 *>(p.sin + o + col) = make_uint2(sn[0], sn[1]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Cos/sin tables of a 3-axis token grid  [ERNIE-fuse §1]
//
// Token s of a (T, Hg, Wg) grid sits at (t, h, w), s = (t*Hg + h)*Wg + w,
// with t shifted by the batch row's offset.  Half-column c of axis k (local
// index i) turns by pos_k * theta^(-2i/d_k), formed in double and rounded once
// to fp32, and the row is cat(f, f), so a lane computes 8 half-columns and
// stores each cos/sin vector in both halves.  Each workgroup first puts the
// frequencies theta^(-2i/d_k) of the R/2 half-columns in LDS: copied from the
// kernel arguments (computed on the host) for up to 2*kGridOmegaArgs rotary
// columns, evaluated on the device for wider rows.  The cos/sin of the fp32
// angle then go through the same correctly rounded path as the precompute
// above.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void rope_cossin_grid_kernel(CosSinGridParams p)
{
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
        const int c0 = (int)(g - row * groups) * 8;
        const uint32_t b = fdiv(row, p.div_s);
        const uint32_t s = row - b * S;
        const uint32_t t = fdiv(s, p.div_hw);
        const uint32_t hw = s - t * HW;
        const uint32_t h = fdiv(hw, p.div_w);
        const uint32_t w = hw - h * Wg;
        const double pos[3] = {(double)((int64_t)t + (p.t_offset ? p.t_offset[b] : 0)),
                               (double)h, (double)w};
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = c0 + e;
            const int k = c < p.h0 ? 0 : (c < p.h01 ? 1 : 2);
            a[e] = __double2float_rn(pos[k] * lomega[c]);
        }
        uint32_t cw[4], sw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            cossin_pair(a[2 * q], a[2 * q + 1], cw[q], sw[q]);
        const v4u cv = v4u{cw[0], cw[1], cw[2], cw[3]}, sv = v4u{sw[0], sw[1], sw[2], sw[3]};
        const int64_t o = (int64_t)row * p.R + c0;
        *reinterpret_cast<v4u *>(p.cos + o) = cv;
        *reinterpret_cast<v4u *>(p.cos + o + half) = cv;
        *reinterpret_cast<v4u *>(p.sin + o) = sv;
        *reinterpret_cast<v4u *>(p.sin + o + half) = sv;
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

constexpr int kRopeBlock = RGG_ROPE_BLOCK;
constexpr int64_t kMaxRopeWorkgroups = (int64_t)1 << 20;  // per launch (2^28 work-items)

__device__ __forceinline__ void load_bf16x8_as_f32(const uint16_t *src, float *dst)
{
    v4u w = *reinterpret_cast<const v4u *>(src);
    dst[0] = bf_lo(w.x); dst[1] = bf_hi(w.x); dst[2] = bf_lo(w.y); dst[3] = bf_hi(w.y);
    dst[4] = bf_lo(w.z); dst[5] = bf_hi(w.z); dst[6] = bf_lo(w.w); dst[7] = bf_hi(w.w);
}

constexpr int kRopeUnroll = RGG_ROPE_UNROLL;

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
#if RGG_STAGE_FIRST
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
#endif
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ic = min(base + u * kRopeBlock + tid, items - 1);
            it[u] = rope_locate<OneToken>(p, V, t0, ic, slots, div_slots, xb1, ob1);
            x1[u] = load16<Nt>(V.x + it[u].xo);
            x2[u] = load16<Nt>(V.x + it[u].xo + (it[u].rot ? half : 0));
        }
#if RGG_ROPE_LDS
        if (OneToken && p.wave_stage && base == first) {
            // One token: every wave stages its own fp32 copy of the row in
            // its own LDS slot, so no wave waits for another.  LDS operations
            // of one wave complete in order; the wave barrier keeps the
            // compiler from moving the reads above the writes.
            const int wave = tid >> 6, lane = tid & 63;
            float *wc = lcos + wave * 2 * R, *ws = wc + R;
            const v4u *gc = reinterpret_cast<const v4u *>(p.cos + t0 * R);
            const v4u *gs = reinterpret_cast<const v4u *>(p.sin + t0 * R);
#if RGG_STAGE_FIRST
            if (stage1) {
                if (lane < R / 4) {
                    const bool is_sin = lane >= R / 8;
                    const int kk = is_sin ? lane - R / 8 : lane;
                    float4 *d = reinterpret_cast<float4 *>((is_sin ? ws : wc) + kk * 8);
                    d[0] = make_float4(bf_lo(stg.x), bf_hi(stg.x), bf_lo(stg.y), bf_hi(stg.y));
                    d[1] = make_float4(bf_lo(stg.z), bf_hi(stg.z), bf_lo(stg.w), bf_hi(stg.w));
                }
            } else
#endif
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
#endif
#if RGG_ROPE_LDS
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
#endif
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (base + u * kRopeBlock + tid >= items)
                continue;
            if (it[u].rot) {
                float c1[8], s1[8], c2[8], s2[8];
#if RGG_ROPE_LDS
                const float *rc = lcos, *rs = lsin;
                if (OneToken && p.wave_stage) {
                    rc = lcos + (tid >> 6) * 2 * R;
                    rs = rc + R;
                }
                load_f32x8(rc + it[u].co, c1);
                load_f32x8(rs + it[u].co, s1);
                load_f32x8(rc + it[u].co + half, c2);
                load_f32x8(rs + it[u].co + half, s2);
#else
                const int64_t cg = t0 * R + it[u].co;
                load_bf16x8_as_f32(p.cos + cg, c1);
                load_bf16x8_as_f32(p.sin + cg, s1);
                load_bf16x8_as_f32(p.cos + cg + half, c2);
                load_bf16x8_as_f32(p.sin + cg + half, s2);
#endif
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

#if RGG_ROPE_LANE
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
#if RGG_STAGE_FIRST
        v4u stg = v4u{0u, 0u, 0u, 0u};
        const bool stage1 = R > 0 && R <= 256;
        if (stage1 && base == first) {
            const int k = min(lane, R / 4 - 1);
            const uint16_t *src = k >= R / 8 ? p.sin + (int64_t)t * R + (k - R / 8) * 8
                                             : p.cos + (int64_t)t * R + k * 8;
            stg = *reinterpret_cast<const v4u *>(src);
        }
#endif
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
#if RGG_STAGE_FIRST
            if (stage1) {
                if (lane < R / 4) {
                    const bool is_sin = lane >= R / 8;
                    const int kk = is_sin ? lane - R / 8 : lane;
                    float4 *d = reinterpret_cast<float4 *>((is_sin ? ws : wc) + kk * 8);
                    d[0] = make_float4(bf_lo(stg.x), bf_hi(stg.x), bf_lo(stg.y), bf_hi(stg.y));
                    d[1] = make_float4(bf_lo(stg.z), bf_hi(stg.z), bf_lo(stg.w), bf_hi(stg.w));
                }
            } else
#endif
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
#endif

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

constexpr int kGegluBlock = RGG_GEGLU_BLOCK;
constexpr int kGegluVec = RGG_GEGLU_VEC;

__global__ __launch_bounds__(kGegluBlock) void gelu_and_mul_kernel(GegluParams p)
{
    __shared__ __align__(16) uint16_t lut[kLutEntries];
    const uint32_t nvec_row = p.div_vecs.d;
    const uint32_t chunk = kGegluBlock * kGegluVec;
    const uint32_t step = gridDim.x * chunk;
    uint32_t base = blockIdx.x * chunk;

    v4u g[kGegluVec], u[kGegluVec];
    int64_t oo[kGegluVec];
    auto fetch = [&](uint32_t b0) {
#pragma unroll
        for (int k = 0; k < kGegluVec; ++k) {
            // lanes past the end re-read the last vector (no load under a branch)
            uint32_t j = min(b0 + k * kGegluBlock + threadIdx.x, p.vec_total - 1);
            uint32_t row = fdiv(j, p.div_vecs);
            uint32_t col = (j - row * nvec_row) * 8;
            const uint16_t *src = p.in + (int64_t)row * p.in_stride + col;
            g[k] = stream_load(src);
            u[k] = stream_load(src + p.hidden);
            oo[k] = (int64_t)row * p.out_stride + col;
        }
    };
#if RGG_GEGLU_LUT_FIRST
    // The lane's table vector is fetched before its gate/up vectors: loads
    // return in order, so the LDS fill and the barrier then overlap the HBM
    // latency instead of waiting for it.
    static_assert(kLutEntries / 8 <= kGegluBlock, "one table vector per lane");
    const uint32_t kt = min(threadIdx.x, kLutEntries / 8 - 1);
    const v4u tv = reinterpret_cast<const v4u *>(g_gelu_lut)[kt];
    __builtin_amdgcn_sched_barrier(0);  // keep the table fetch ahead of gate/up
    fetch(base);  // indexes are clamped, so the first fetch needs no guard
    if (threadIdx.x < kLutEntries / 8)
        reinterpret_cast<v4u *>(lut)[threadIdx.x] = tv;
#else
    if (base < p.vec_total)
        fetch(base);

    for (uint32_t k = threadIdx.x; k < kLutEntries / 8; k += kGegluBlock)
        reinterpret_cast<v4u *>(lut)[k] = reinterpret_cast<const v4u *>(g_gelu_lut)[k];
#endif
    __syncthreads();

    while (base < p.vec_total) {
#pragma unroll
        for (int k = 0; k < kGegluVec; ++k) {
            v4u o = geglu_vec(g[k], u[k], lut);
            if (base + k * kGegluBlock + threadIdx.x < p.vec_total)
                stream_store(p.out + oo[k], o);
        }
        base += step;
        if (base < p.vec_total)
            fetch(base);
    }
}

// ---------------------------------------------------------------------------
// GEGLU as the epilogue of the gate_up projection      [ERNIE-fuse §3]
//
// out = x W^T on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
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
// first MFMA operand and x the second, so in a 32x32 block lane l holds
// output row l % 32 and, in its accumulators v, output columns
// (v / 4) * 8 + (l / 32) * 4 + v % 4.  Operands: lane l supplies row l % 32
// of W or of x and the 8 consecutive k at (l / 32) * 8 of a 16-wide step.
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
// Per slice each wave issues 64 products in 4 steps of 16 (one register
// set of fragments per step, alternating).  The fragment reads of the next
// step ride on the first 8 products of each step; the 16 loads of the next
// slice go out two per three products over the first 24.  After 15
// products of step 3 the wave waits for its own loads of the next slice
// (loads complete in order) and passes the barrier that publishes them and
// frees the stage just read; the last product carries the next slice's
// step-0 reads.  A late barrier gives the loads the most time to arrive.
//
// Workgroups go to the 8 XCDs round robin; the block index is remapped so
// that each XCD gets one contiguous run of tiles, and the run is walked in
// groups of 8 row blocks (column block outer), so the tiles an XCD works on
// at one time share rows of x and of W in its L2.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
constexpr int kGemmBarrierAt = 15;        // products of the last step before the barrier
static_assert(kGemmLds <= 160 * 1024, "LDS of one CU");
static_assert(kGemmLutBytes % 1024 == 0, "stages start on a 1 KiB boundary");
static_assert(4 * 128 * 64 * 2 <= kGemmStageBytes, "epilogue blocks fit stage 1");
static_assert(kLutEntries % 8 == 0 && kLutEntries / 8 <= 2 * kGemmThreads, "table: two vectors per lane");

__device__ __forceinline__ uint32_t bf16_of(float v) { return rne_pack(v, 0.0f) & 0xFFFFu; }

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
    auto point = [&](int64_t m0, int32_t n0) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        bx = p.x + m0 * p.x_stride;
        bw = p.w + ((wv < 2 ? 0 : (int64_t)p.H) + n0) * p.w_stride;
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
    // The instruction has no register result, and nothing else in this
    // kernel uses M0 (no other LDS-direct, message or relative-move
    // instruction), so setting it here disturbs no compiler state.
    const uint32_t lds0 = (uint32_t)(uintptr_t)gsm + kGemmLutBytes + wv * 8 * 1024;
    auto dma1 = [&](int kt, int st, int idx) {
        const int j = idx & 7;
        const uint16_t *base = (idx < 8 ? bx : bw) + (int64_t)kt * kGemmBK;
        const uint32_t off = idx < 8 ? ox[j] : ow[j];
        const uint32_t dst = lds0 + st * kGemmStageBytes + (idx < 8 ? 0 : kGemmOpBytes) + j * 1024;
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(base), "s"(dst) : "memory");
    };
    auto fetch = [&](int kt, int st) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
            dma1(kt, st, idx);
    };

    f32x16 acc[4][4];  // [x row block][gate 0, gate 1, up 0, up 1]

    // Operand fragments of one k16 step, double buffered in registers (set
    // 0 / set 1): 4 of x, then gate 0, gate 1, up 0, up 1 of W.
    const int ra = (wm * 128 + (lane & 31)) * 128;
    const int rb = (wn * 64 + (lane & 31)) * 128;
    bf16x8 fa[2][4], fb[2][4];
    auto frag1 = [&](int st, int ks, int set, int idx) {
        const uint8_t *sx = gsm + kGemmLutBytes + st * kGemmStageBytes;
        const int ch = ((2 * ks + (lane >> 5)) ^ (((lane & 31) >> 1) & 7)) * 16;
        if (idx < 4)
            fa[set][idx] = *reinterpret_cast<const bf16x8 *>(sx + ra + idx * 32 * 128 + ch);
        else
            fb[set][idx - 4] = *reinterpret_cast<const bf16x8 *>(
                sx + kGemmOpBytes + rb + (((idx - 4) >> 1) * kGemmBN + ((idx - 4) & 1) * 32) * 128 + ch);
    };
    // Fragments are read in the order the products first use them.
    constexpr int kOrder[8] = {0, 4, 5, 6, 7, 1, 2, 3};
    auto mma1 = [&](int set, int idx) {
        const int i = idx >> 2, j = idx & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // The workgroup walks tiles blockIdx.x, + gridDim.x, ... (one workgroup
    // per CU).  The first slice of the next tile is requested before the
    // epilogue of the current one, so its latency hides under it.
    const int KT = p.K / kGemmBK;
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
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[a][b][v] = 0.0f;

        // One slice: product pp = 16 * step + k in the order fixed by
        // scheduling fences, each followed by at most a fragment read and a
        // load (the product after the barrier carries the next slice's
        // reads).  The last slice of a tile loads nothing and passes no
        // barrier.
        auto slice = [&](int kt, bool last) {
            const int st = kt & 1, sn = st ^ 1;
#pragma unroll
            for (int pp = 0; pp < 64; ++pp) {
                const int step = pp >> 4, k = pp & 15;
                if (step == 3 && k == kGemmBarrierAt && !last) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    RGG_FENCE();
                }
                mma1(step & 1, k);
                if (step < 3 && k < 8)
                    frag1(st, step + 1, (step + 1) & 1, kOrder[k]);
                if (step == 3 && k >= kGemmBarrierAt && !last) {
                    constexpr int nr = 16 - kGemmBarrierAt;
                    constexpr int per = (8 + nr - 1) / nr;
#pragma unroll
                    for (int r = 0; r < per; ++r) {
                        const int idx = (k - kGemmBarrierAt) * per + r;
                        if (idx < 8)
                            frag1(sn, 0, 0, kOrder[idx]);
                    }
                }
                if (!last && pp < 24 && pp % 3 != 2)
                    dma1(kt + 1, sn, pp / 3 * 2 + pp % 3);
                RGG_FENCE();
            }
        };
        if (KT > 0) {
#pragma unroll
            for (int idx = 0; idx < 8; ++idx)
                frag1(0, 0, 0, kOrder[idx]);
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

        // Epilogue: round each accumulator to bf16 (the projection's
        // output), then keep it, or form rne(up * G(gate)).  Each wave writes
        // its 128 x 64 block of results to its 16 KiB of stage 1 as
        // 128-byte rows (16-byte chunk c of row r at chunk c ^ (r % 8); four
        // adjacent columns per 8-byte write), then reads it back as 16-byte
        // vectors, eight lanes per row, for whole-line global stores.  The
        // plain product does this twice: gate columns, then up columns (H
        // further along the row).  H is a multiple of 64, so a wave's block
        // is wholly inside [0, H) or outside.
        const uint16_t *lut = reinterpret_cast<const uint16_t *>(gsm);
        uint8_t *ep = gsm + kGemmLutBytes + kGemmStageBytes + wave * 16384;
        int el = lane;
        asm volatile("" : "+v"(el));
        const int32_t cbase = cn0 + wn * 64;
        const bool live = cbase < p.H;
        bool anyg = false;
        if (Geglu) {
            bool general = false;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        general |= (bf16_of(acc[i][cb][v]) & 0x7FFFu) - 0x0100u >= kLutHi - 0x0100u;
            anyg = __builtin_amdgcn_ballot_w64(general) != 0;
        }
#pragma unroll
        for (int half = 0; half < (Geglu ? 1 : 2); ++half) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    float G[16];
                    if (Geglu) {
                        if (!anyg) {
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                G[v] = __uint_as_float(gelu_common(bf16_of(acc[i][cb][v]), lut));
                        } else {
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                G[v] = __uint_as_float(gelu_general(bf16_of(acc[i][cb][v]), lut) << 16);
                        }
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t w0, w1;
                        if (Geglu) {
                            const f32x16 &u = acc[i][2 + cb];
                            w0 = rne_pack(bf_lo(bf16_of(u[q * 4 + 0])) * G[q * 4 + 0],
                                          bf_lo(bf16_of(u[q * 4 + 1])) * G[q * 4 + 1]);
                            w1 = rne_pack(bf_lo(bf16_of(u[q * 4 + 2])) * G[q * 4 + 2],
                                          bf_lo(bf16_of(u[q * 4 + 3])) * G[q * 4 + 3]);
                        } else {
                            const f32x16 &a = acc[i][2 * half + cb];
                            w0 = rne_pack(a[q * 4 + 0], a[q * 4 + 1]);
                            w1 = rne_pack(a[q * 4 + 2], a[q * 4 + 3]);
                        }
                        const int r = i * 32 + (el & 31), chunk = cb * 4 + q;
                        *reinterpret_cast<uint2 *>(ep + r * 128 + ((chunk ^ (r & 7)) << 4) +
                                                   (el >> 5) * 8) = make_uint2(w0, w1);
                    }
                }
            }
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
    const uint32_t per_row = paired ? (uint32_t)(p.R / 16) : (uint32_t)(p.R / kCosSinCols);
    p.vec_total = rows * per_row;
    p.div_vecs = make_fastdiv(per_row);
    uint32_t blocks = (p.vec_total + kThreads - 1) / kThreads;
    if (blocks > 4096)
        blocks = 4096;
    if (paired)
        hipLaunchKernelGGL(rope_cossin_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(rope_cossin_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_rope_cossin_grid(const CosSinGridParams &p, hipStream_t stream)
{
    uint32_t blocks = (p.groups_total + kThreads - 1) / kThreads;
    if (blocks > 2048)
        blocks = 2048;
    const size_t lds = (size_t)(p.R / 2) * sizeof(double);
    hipLaunchKernelGGL(rope_cossin_grid_kernel, dim3(blocks), dim3(kThreads), lds, stream, p);
    return hipGetLastError();
}

hipError_t launch_rope_rotate_half(const RopeParams &params, hipStream_t stream)
{
    RopeParams p = params;
    p.tok_per_wg = rope_tokens_per_workgroup(p.H, p.D, p.R);
    p.div_views = make_fastdiv((uint32_t)p.n_views);
    size_t lds = RGG_ROPE_LDS ? (size_t)p.tok_per_wg * p.R * 2 * sizeof(float) : 0;
    // One-token workgroups give each wave its own staged row unless the
    // copies would crowd LDS (wide rotations); then the workgroup shares one.
    const size_t wave_lds = (size_t)(kRopeBlock / 64) * p.R * 2 * sizeof(float);
    p.wave_stage = RGG_ROPE_LDS && RGG_ROPE_WAVE_STAGE && p.tok_per_wg == 1 && wave_lds <= 65536;
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
#if RGG_ROPE_LANE
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
#endif
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

hipError_t launch_gelu_and_mul(const GegluParams &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL(gelu_and_mul_kernel, dim3(grid), dim3(kGegluBlock), 0, stream, p);
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
#if RGG_ROPE_TPW_FIT
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
#else
    // About RGG_ROPE_VEC_PER_WG 16-byte vectors of x per workgroup, with the
    // fp32 cos/sin staging within 32 KiB of LDS.
    int64_t vec_per_tok = (int64_t)H * (D / 8);
    int64_t t = vec_per_tok > 0 ? RGG_ROPE_VEC_PER_WG / vec_per_tok : 64;
    if (t < 1)
        t = 1;
    if (t > 64)
        t = 64;
    while (t > 1 && t * R * 8 > 32768)
        --t;
    return (int)t;
#endif
}

int geglu_grid(uint32_t vec_total, int cu_count)
{
    // kGegluVec vectors per lane; with RGG_GEGLU_WG_PER_CU > 0 the grid is
    // capped at that many workgroups per compute unit and each loops.
    const uint32_t chunk = kGegluBlock * kGegluVec;
    uint32_t chunks = (vec_total + chunk - 1) / chunk;
    if (chunks == 0)
        chunks = 1;
    if (RGG_GEGLU_WG_PER_CU == 0)
        return (int)chunks;
    uint32_t cap = (uint32_t)(cu_count > 0 ? cu_count : 256) * RGG_GEGLU_WG_PER_CU;
    return (int)(chunks < cap ? chunks : cap);
}

}  // namespace rgg

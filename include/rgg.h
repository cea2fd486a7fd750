/*
 * rgg.h -- C ABI of bf16_rope_geglu_amd: the fused elementwise path of an
 * ERNIE-Image style diffusion transformer, for AMD Instinct MI355X (gfx950).
 *
 * The method comes from the page "[sglang] ERNIE-Image의 RoPE와 GELU-mul 융합
 * 및 RoPE cos/sin 호이스팅을 통한 성능 최적화" (blog.secrett2633.cloud, an
 * analysis of sglang PR 34306), cited below as [ERNIE-fuse] with its section:
 *   §1 hoist the rotary cos/sin tables once per forward,
 *   §2 fuse the rotate-half RoPE chain, bit-exact with eager bf16 rounding,
 *   §3 fuse GEGLU (up * gelu(gate)) keeping eager's bf16 activation rounding.
 *
 * Conventions shared by every entry point
 *   - bf16 data is passed as uint16_t bit patterns (the upper half of an IEEE
 *     binary32); fp32 data as float.
 *   - Every tensor pointer is device memory owned by the caller.  No call
 *     allocates memory.  The one piece of library state is a constant
 *     7 KiB GELU table per device, built on the first GEGLU call on that
 *     device (or by rgg_prepare_device) and kept until the process ends.
 *   - Sizes and strides count elements, not bytes.  Strides must be >= 0.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream) of the
 *     current HIP device.  Arguments are checked synchronously first; on any
 *     error nothing is enqueued and a nonzero rgg_status is returned.  No C++
 *     exception crosses this interface.
 *   - Vector access: bf16 base pointers must be 16-byte aligned and bf16
 *     strides multiples of 8 elements (RGG_ERR_ALIGN otherwise); the fp32
 *     angle tensor needs 16-byte alignment and strides that are multiples of
 *     4.  There is no slower fallback for other layouts.
 *   - A size of zero in any batch-like dimension is a valid no-op.
 *   - Index arithmetic in the kernels is 32-bit where it can be: each entry
 *     point states the size limits beyond which it returns
 *     RGG_ERR_UNSUPPORTED.
 *   - Entry points may be called from several host threads at once, on any
 *     streams; the one-time GELU table build is serialized per device.  Calls
 *     that write the same memory on different streams race as any kernels
 *     would.
 */
#ifndef RGG_H
#define RGG_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RGG_API __attribute__((visibility("default")))

typedef enum rgg_status {
    RGG_OK = 0,
    RGG_ERR_NULL = 1,        /* a pointer needed for a non-empty call is NULL */
    RGG_ERR_SHAPE = 2,       /* negative size/stride, odd R, R > D, n_views out of 1..4 */
    RGG_ERR_UNSUPPORTED = 3, /* width not a multiple of the 8-element vector, or an output
                                view whose rows overlap themselves */
    RGG_ERR_ALIGN = 4,       /* base pointer or stride breaks the 16-byte vector rule */
    RGG_ERR_ALIAS = 5,       /* an output overlaps an input or another output (other than
                                the exact in-place forms each call allows) */
    RGG_ERR_HIP = 6,         /* the HIP runtime reported an error */
    RGG_ERR_CAPTURING = 7,   /* first GEGLU call on a device made while `stream` is being
                                captured: call rgg_prepare_device() before capturing */
    RGG_ERR_SELFCHECK = 8    /* rgg_selfcheck found a result that differs from its
                                expected bits */
} rgg_status;

/*
 * Hoisted rotary tables.                              [ERNIE-fuse §1]
 *
 * The rotary angles `freqs` have the page's shape (S, B, 1, R) in fp32: the
 * angle of sequence position s, batch row b, rotary column j is
 *     freqs[s * stride_s + b * stride_b + j]      (unit stride along j).
 * Writes two contiguous bf16 tables of shape (B*S, R), row b*S + s (the
 * page's permute to (B, S, 1, R) followed by a flatten):
 *     cos_out[(b*S + s)*R + j] = rne_bf16(cos(angle)),
 *     sin_out[(b*S + s)*R + j] = rne_bf16(sin(angle)).
 * Each entry is the exact cosine/sine of the fp32 angle rounded once to the
 * nearest bf16 (ties to even).  The tables depend only on the angles, so one
 * call per forward serves every layer and projection.
 *
 * Requirements: S, B >= 0; R >= 0 and a multiple of 8; freqs 16-byte aligned
 * with stride_s, stride_b multiples of 4; cos_out, sin_out 16-byte aligned;
 * the two tables may not overlap each other or freqs.  Limits: S*B < 2^31
 * and S*B*R/4 < 2^31.
 */
RGG_API int rope_cossin_precompute(const float *freqs, int64_t S, int64_t B, int64_t R,
                           int64_t stride_s, int64_t stride_b,
                           uint16_t *cos_out, uint16_t *sin_out, hipStream_t stream);

/*
 * Rotary tables straight from a 3-axis token grid.
 *                            [ERNIE-fuse §1, the angles the table hoist is fed]
 *
 * The same tables as rope_cossin_precompute, for the angles a 3-axis
 * positional embedding gives a (T, Hg, Wg) grid of S = T*Hg*Wg tokens, with
 * no fp32 angle tensor in memory.  The page names that embedding (EmbedND3)
 * without defining it; the reading implemented here:
 *   - token s sits at (t, h, w), s = (t*Hg + h)*Wg + w; batch row b shifts t
 *     by t_offset[b] (t_offset == NULL: no shift);
 *   - axis k (k = 0: t, 1: h, 2: w) owns d_k rotary columns and contributes
 *     d_k/2 half-angles pos_k * theta^(-2i/d_k), i = 0 .. d_k/2 - 1;
 *   - the half-angles of axes 0, 1, 2 in that order form f (R/2 values,
 *     R = d0 + d1 + d2), and the angle row is cat(f, f);
 *   - each half-angle is formed in double and rounded once to fp32 (the
 *     angle rope_cossin_precompute would be given), and the tables hold its
 *     correctly rounded bf16 cosine/sine, row b*S + s.
 *
 * Requirements: B, T, Hg, Wg >= 0; d0, d1, d2 >= 0 and even; theta > 0 and
 * finite; R a multiple of 16 and at most 8192 (RGG_ERR_UNSUPPORTED
 * otherwise); t_offset NULL or a 4-byte aligned device array of B int32;
 * cos_out, sin_out 16-byte aligned device (B*S, R) bf16 tables that overlap
 * neither each other nor t_offset.  Any of B, T, Hg, Wg or R zero: no work.
 * Limits: S = T*Hg*Wg < 2^31, B*S < 2^31 and B*S*R/16 < 2^31.
 */
RGG_API int rope_cossin_from_grid(int64_t B, int64_t T, int64_t Hg, int64_t Wg, int32_t d0,
                                  int32_t d1, int32_t d2, double theta, const int32_t *t_offset,
                                  uint16_t *cos_out, uint16_t *sin_out, hipStream_t stream);

/*
 * One strided (B, S, H, D) bf16 tensor to rotate and where to put the result.
 * Element (b, s, h, d) of the input is x[b*x_stride_b + s*x_stride_s +
 * h*x_stride_h + d]; the output uses the out_* strides the same way.  A view
 * may be a slice of a larger buffer, e.g. the q or k part of a fused QKV
 * projection output, read in place without a copy.
 */
typedef struct rgg_rope_view {
    const uint16_t *x;
    uint16_t *out;
    int64_t x_stride_b, x_stride_s, x_stride_h;
    int64_t out_stride_b, out_stride_s, out_stride_h;
} rgg_rope_view;

/*
 * Rotate-half RoPE with tail passthrough.          [ERNIE-fuse §2]
 *
 * For every view v, token (b, s), head h, with c and sn the bf16 rows
 * b*S + s of `cos` and `sin` (contiguous (B*S, R)) and h2 = R/2:
 *   j <  h2:      out[j] = rne(rne(x[j]*c[j]) + rne(-x[j+h2]*sn[j]))
 *   h2 <= j < R:  out[j] = rne(rne(x[j]*c[j]) + rne( x[j-h2]*sn[j]))
 *   R <= j < D:   out[j] = x[j]                       (bits copied)
 * i.e. exactly the eager bf16 chunk / neg / cat / mul / mul / add chain
 * followed by the tail concatenation, every op rounded to nearest-even bf16.
 * c[j] and c[j + h2] are used as given (they need not be equal).
 *
 * `views` is a host array of n_views (1..4) entries, read during the call;
 * all views share B, S, H, D, R and the cos/sin tables (q and k of a layer
 * in one launch).  Out of place, or in place when out == x with identical
 * strides (the tail is then left untouched).  No output may overlap any
 * input or another output otherwise; the check is exact for views with equal
 * strides (e.g. q/k/v slices of one fused buffer) and by address range for
 * views with different strides.
 *
 * Requirements: B, S, H >= 0; D > 0 and a multiple of 8; R even with
 * 0 <= R <= D and R a multiple of 16 (each half a whole number of 8-element
 * vectors); R = 0 copies x.  Output rows must not overlap each other.
 * Limits: B*S < 2^31, D <= 8192 and H*D < 2^25 (RGG_ERR_UNSUPPORTED);
 * longer token ranges than one dispatch takes are split into several
 * launches on `stream`.
 */
RGG_API int rope_rotate_half_bf16(const rgg_rope_view *views, int n_views, int64_t B, int64_t S,
                          int64_t H, int64_t D, int64_t R, const uint16_t *cos,
                          const uint16_t *sin, hipStream_t stream);

/*
 * GEGLU with activation rounding.                  [ERNIE-fuse §3]
 *
 * `input` is (rows, 2*hidden) bf16 with row stride in_row_stride: the first
 * `hidden` columns are the gate, the next `hidden` the up projection.  Writes
 * (rows, hidden) bf16 to `out` with row stride out_row_stride:
 *   out[r][j] = rne_bf16( up[r][j] * G(gate[r][j]) ),
 *   G(x)      = rne_bf16( x * Phi(x) ),  Phi the standard normal CDF
 * (the exact-erf GELU rounded to bf16 before the multiply, as the eager
 * up * F.gelu(gate) chain rounds it).  G is correctly rounded for every one
 * of the 65536 bf16 inputs: G(+-0) = +-0, G(+inf) = +inf, G(-inf) = NaN,
 * G(NaN) = NaN.
 *
 * In place is allowed in one form: out == input with out_row_stride ==
 * in_row_stride (the result overwrites the gate half).  Otherwise out may not
 * overlap input.
 *
 * Requirements: rows, hidden >= 0; hidden a multiple of 8; strides multiples
 * of 8 with out_row_stride >= hidden when rows > 1; 16-byte aligned bases.
 * Limit: rows*hidden/8 < 2^31.
 */
RGG_API int gelu_and_mul_bf16(const uint16_t *input, int64_t rows, int64_t hidden,
                      int64_t in_row_stride, uint16_t *out, int64_t out_row_stride,
                      hipStream_t stream);

/*
 * The gate_up projection, alone or with GEGLU fused into its epilogue.
 *                                   [ERNIE-fuse §3, the projection before it]
 *
 * x is (M, K) bf16 with row stride x_stride; W is a linear layer's weight
 * (N, K) bf16 with row stride w_stride (row n produces output column n).
 * The product runs on the matrix cores with fp32 accumulation and each
 * result is rounded once to bf16 (the eager bf16 projection, no bias):
 *     gemm_bf16_nt:     out[m][n] = rne_bf16( sum_k x[m][k] * W[n][k] ),
 *                       out (M, N), row stride out_stride.
 *     gemm_geglu_bf16:  W is (2H, K), gate rows 0..H-1 then up rows H..2H-1;
 *                       out[m][j] = rne_bf16( up[m][j] * G(gate[m][j]) ) with
 *                       gate/up the bf16 projection outputs and G as in
 *                       gelu_and_mul_bf16; out (M, H), row stride out_stride.
 *                       The (M, 2H) projection never goes to memory.
 * For the same x and W, gemm_geglu_bf16 returns bit for bit what
 * gelu_and_mul_bf16 returns on the output of gemm_bf16_nt (one accumulation
 * order serves both).  The fp32 accumulation order is the kernel's: a
 * projection output is the bf16 rounding of a value within
 *     2 (K + 16) 2^-24 sum_k |x[m][k] W[n][k]|  +  K 2^-149
 * of the exact sum (the relative term covers rounding in the normal range;
 * the absolute term covers products and partial sums in the fp32 subnormal
 * range, which are kept, not flushed, each off by at most half the subnormal
 * step), so it differs from the exactly rounded sum only where that error
 * reaches across a rounding boundary (and never where every partial sum is
 * exact in fp32).
 *
 * Requirements: M, K >= 0; K a multiple of 64; N a multiple of 128 (H a
 * multiple of 64); rows of x and W at least K long, output rows at least N
 * (H) long; 16-byte aligned bases and strides that are multiples of 8; out
 * may not overlap x or W.  M or N (H) zero: no work; K zero: zeros (and G(0)).
 * Limits: M, K < 2^31, row strides of x and W < 2^22 elements and
 * ceil(M/256) * ceil(H/128) < 2^24.  gemm_geglu_bf16 builds
 * the GELU table like gelu_and_mul_bf16 (RGG_ERR_CAPTURING applies).
 */
RGG_API int gemm_bf16_nt(const uint16_t *x, int64_t M, int64_t K, int64_t x_stride,
                         const uint16_t *w, int64_t N, int64_t w_stride, uint16_t *out,
                         int64_t out_stride, hipStream_t stream);
RGG_API int gemm_geglu_bf16(const uint16_t *x, int64_t M, int64_t K, int64_t x_stride,
                            const uint16_t *w, int64_t H, int64_t w_stride, uint16_t *out,
                            int64_t out_stride, hipStream_t stream);

/*
 * Builds the constant GELU table on HIP device `device` now (synchronously)
 * if it is not built yet.  Needed only before capturing a GEGLU call into a
 * HIP graph on a device that has not run one; otherwise the first
 * gelu_and_mul_bf16 call on the device does it.  Leaves the current device
 * unchanged.
 */
RGG_API int rgg_prepare_device(int device);

/*
 * Device self-check: the bit-exactness gate of the fused path, run on the
 * caller's device and stream against expected bits derived by hand from the
 * definitions (no eager twin to compare with).
 *                                   [ERNIE-fuse §3, its bit-exact fusion gate]
 *
 * Runs the entry points above on small inputs staged in `workspace` and
 * compares on the host, bit for bit:
 *   bit 0  cos/sin of the fp32 angles 0, -0, pi, pi/2, 2*pi, pi/3, pi/6, 100
 *          against their correctly rounded bf16 values (50-digit evaluation);
 *   bit 1  rotate-half on hand-derived worked vectors (ties to even after the
 *          product, no fused multiply-add, subnormals kept, overflow, signed
 *          zeros, different angles per half);
 *   bit 2  rotate-half with a zero angle returns x (two heads, a tail), with
 *          -0 becoming +0 in the rotated columns only;
 *   bit 3  G at textbook points (x = 1, 2, -1, 0.5, 3, -2, -3, -5.5);
 *   bit 4  G over all 65536 bf16 inputs against the rules that fix it outside
 *          the tabulated range (G = x for x >= 16, -0 for x <= -16, x/2 for
 *          2^-125 <= |x| < 2^-10, signed zeros, Inf and NaN) and its
 *          monotonicity for x > 0;
 *   bit 5  the multiply: up = 2 doubles every finite G below 2^127 exactly;
 *   bit 6  the projection on one-hot rows of x (out[m][n] = W[n][m] exactly,
 *          plain), and with GEGLU fused where each gate is one of the points
 *          of bit 3 and each up is 1 or 2 (out = G or 2 G exactly).
 * `*failed` (if not NULL) receives the mask of failed checks.  Returns
 * RGG_OK when every check passes, RGG_ERR_SELFCHECK otherwise.  Synchronous:
 * waits for `stream`.  Not allowed while `stream` is capturing
 * (RGG_ERR_CAPTURING).  `workspace` is caller-owned device memory of at
 * least RGG_SELFCHECK_WORKSPACE_BYTES bytes, 256-byte aligned; its contents
 * are overwritten.
 */
#define RGG_SELFCHECK_WORKSPACE_BYTES (1 << 20)
#define RGG_SELFCHECK_ALL 0x7Fu   /* bits 0-6 */
RGG_API int rgg_selfcheck(void *workspace, int64_t workspace_bytes, hipStream_t stream,
                          uint32_t *failed);

/*
 * The same self-check without a workspace, for callers that cannot allocate
 * device memory (a serving loop's health check, a harness that forbids
 * hipMalloc).  It runs the checks selected by `checks` (a nonzero subset of
 * RGG_SELFCHECK_ALL: bit k runs check k of rgg_selfcheck; bits 3-5 share one
 * GEGLU run) over a 1 MiB device array that the library holds for each GPU it
 * runs on until the process ends, and host images it holds statically; it
 * calls no allocating routine.  Returns and sets *failed exactly as
 * rgg_selfcheck does for the selected bits, RGG_ERR_SHAPE for an empty or
 * out-of-range mask, RGG_ERR_HIP if the array's device address cannot be
 * looked up.  Synchronous; not allowed while `stream` is capturing.  Calls
 * from several host threads are serialized by a lock; every call overwrites
 * the array's staged region before it uses it.
 */
RGG_API int rgg_selfcheck_noalloc(uint32_t checks, hipStream_t stream, uint32_t *failed);

/* Static, human-readable text for a status code (never NULL). */
RGG_API const char *rgg_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RGG_H */

/*
 * CPU oracle for the fused elementwise path of an ERNIE-Image style DiT:
 * hoisted rotary cos/sin tables, bit-exact rotate-half RoPE with tail
 * passthrough, and GEGLU with bf16 activation rounding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or
 * call this file.  Its only users are tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py.  It shares no code, header, table or constant
 * with the HIP library; the two meet only at the seeded inputs.
 *
 * Source of the method (cited below as [ERNIE-fuse]):
 *   "[sglang] ERNIE-Image의 RoPE와 GELU-mul 융합 및 RoPE cos/sin 호이스팅을
 *    통한 성능 최적화", blog.secrett2633.cloud, pr-analysis of sglang PR 34306.
 *   Sections: §1 (RoPE cos/sin 재계산 제거 및 융합), §2 (rotate-half 연산의
 *   Triton 커널 융합), §3 (GEGLU 연산 융합).
 *
 * Numeric model.  A bf16 value is the upper half of an IEEE binary32.  Every
 * eager PyTorch op on bf16 tensors evaluates in float and rounds its result to
 * bf16 with round-to-nearest-even.  This oracle evaluates every such op
 * exactly (in double; bf16*bf16 products and bf16+bf16 sums are exact or, for
 * sums of very different magnitude, rounded at 53 bits, which for a final
 * 8-bit rounding is the same as rounding the exact value once) and rounds the
 * result to bf16 once.  Transcendentals (cos, sin, erfc) are evaluated in
 * double and rounded to bf16 once, i.e. the oracle is "the exact value,
 * rounded to nearest even", not the bits of any vendor float library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no FMA, no FTZ).
 *
 * Parity pins (tests/test_oracle_pins.py) tie every exported function to
 * something other than this file: torch's float->bf16 conversion, the eager
 * bf16 chunk/neg/cat/mul/add chain run by PyTorch on the CPU, hand-derived
 * worked vectors, the zero-angle identity, exact-arithmetic rotation
 * invariants, mpmath at 256-bit precision (cos, sin, and every one of the
 * 65536 bf16 GELU inputs), textbook values of the normal CDF, and, for the
 * grid angles, a numpy form of the same reading plus exact products in
 * mpmath.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------------------
 * bf16 <-> double
 * ------------------------------------------------------------------------- */

/* The value of a bf16 bit pattern (exact: bf16 is a truncated binary32). */
ORACLE_API double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a real number to bf16, nearest-even.
 *
 * `v` is the value to round.  `sticky` is the sign of whatever part of the
 * true value was lost when it was squeezed into the double `v` (0 if none).
 * It only matters when `v` sits exactly on a bf16 midpoint: then the true
 * value lies on the `sticky` side of it, and ties-to-even applies only when
 * sticky == 0.
 *
 * Method: bf16 carries 8 significant bits.  For |v| in [2^(e-1), 2^e) the
 * spacing of bf16 values is 2^(e-8); below the normal range (|v| < 2^-126)
 * the spacing stays at the subnormal step 2^-133.  Scaling |v| by the
 * spacing (an exact power-of-two multiply) turns the rounding into rounding
 * to an integer.
 */
ORACLE_API uint16_t oracle_double_to_bf16(double v, int sticky)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0x0000u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v))
        return (uint16_t)(sign | 0x7F80u);
    if (v == 0.0)
        return sign;

    double mag = fabs(v);
    int mag_sticky = (v > 0.0) ? sticky : -sticky; /* direction of |true| - |v| */

    int e;
    (void)frexp(mag, &e); /* mag = m * 2^e, m in [0.5, 1) */
    int q = e - 8;        /* log2 of the bf16 spacing at this magnitude */
    if (q < -133)
        q = -133;

    double scaled = ldexp(mag, -q); /* exact */
    double whole = floor(scaled);
    double frac = scaled - whole;   /* exact */

    int up;
    if (frac > 0.5)
        up = 1;
    else if (frac < 0.5)
        up = 0;
    else if (mag_sticky > 0)
        up = 1;
    else if (mag_sticky < 0)
        up = 0;
    else
        up = fmod(whole, 2.0) != 0.0; /* tie: to even */

    double r = ldexp(whole + (up ? 1.0 : 0.0), q); /* exact */

    /* largest finite bf16 is (2 - 2^-7) * 2^127 */
    if (r > ldexp(255.0, 120))
        return (uint16_t)(sign | 0x7F80u);

    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* The value of rounding v to bf16 (one eager bf16 op's result). */
static double to_bf16_value(double v)
{
    return oracle_bf16_to_double(oracle_double_to_bf16(v, 0));
}

static double keep_exact(double v)
{
    return v;
}

/* ---------------------------------------------------------------------------
 * Hoisted cos/sin tables          [ERNIE-fuse §1]
 *
 * freqs has shape (S, B, 1, R): the angle for sequence position s, batch row
 * b, rotary column j is at freqs[s*stride_s + b*stride_b + j].  The page
 * permutes it to (B, S, 1, R), takes cos and sin in float, casts to bf16 and
 * flattens to (B*S, R), so table row b*S + s holds position s of batch b.
 * Here cos and sin are taken in double and rounded to bf16 once.
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_rope_cossin(const float *freqs, int64_t S, int64_t B, int64_t R,
                                   int64_t stride_s, int64_t stride_b,
                                   uint16_t *cos_out, uint16_t *sin_out)
{
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t s = 0; s < S; ++s) {
            int64_t row = b * S + s;
            for (int64_t j = 0; j < R; ++j) {
                double f = (double)freqs[s * stride_s + b * stride_b + j];
                cos_out[row * R + j] = oracle_double_to_bf16(cos(f), 0);
                sin_out[row * R + j] = oracle_double_to_bf16(sin(f), 0);
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Rotary angles of a 3-axis token grid       [ERNIE-fuse §1, the angles
 *                                                  the table hoist is fed]
 *
 * The page hoists the tables from angles that the model's 3-axis positional
 * embedding (EmbedND3) produces, and does not define that step.  Reading
 * used here, the plain one for a rotate-half model over a (T, Hg, Wg) token
 * grid:
 *   - token s sits at (t, h, w) with s = (t*Hg + h)*Wg + w; batch row b
 *     shifts t by t_offset[b] (no shift when t_offset is NULL);
 *   - axis k, owning d_k rotary columns, contributes d_k/2 half-angles
 *     pos_k * theta^(-2i/d_k), i = 0 .. d_k/2 - 1;
 *   - the three axes' half-angles, axis 0 first, form f (R/2 values, with
 *     R = d_0 + d_1 + d_2), and the angle row is cat(f, f), so that column j
 *     and column j + R/2 turn by the same angle;
 *   - each half-angle is formed in double and rounded once to float.
 * The result is the fp32 angle tensor (S, B, 1, R), S = T*Hg*Wg, contiguous,
 * that oracle_rope_cossin turns into the tables.
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_rope_angles_grid(int64_t B, int64_t T, int64_t Hg, int64_t Wg,
                                        const int32_t *dims, double theta,
                                        const int32_t *t_offset, float *freqs)
{
    const int64_t S = T * Hg * Wg;
    const int64_t R = (int64_t)dims[0] + dims[1] + dims[2], half = R / 2;
    for (int64_t s = 0; s < S; ++s) {
        const int64_t t = s / (Hg * Wg), h = (s / Wg) % Hg, w = s % Wg;
        for (int64_t b = 0; b < B; ++b) {
            const double pos[3] = {(double)(t + (t_offset ? t_offset[b] : 0)), (double)h,
                                   (double)w};
            float *row = freqs + (s * B + b) * R;
            int64_t j = 0;
            for (int k = 0; k < 3; ++k) {
                for (int32_t i = 0; i < dims[k] / 2; ++i, ++j) {
                    const double omega = pow(theta, -2.0 * i / dims[k]);
                    row[j] = (float)(pos[k] * omega);
                    row[j + half] = row[j];
                }
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Rotate-half RoPE with tail passthrough   [ERNIE-fuse §2]
 *
 * The page's eager chain splits the leading R columns into two halves of
 * width h = R/2, forms the rotate-half partner (the negated second half
 * followed by the first half), multiplies the columns by cos and the partner
 * by sin, adds the two products, and appends the untouched columns R..D-1.
 * With every op rounded to bf16 this is, per column j < R,
 *   out[j] = rnd( rnd(x[j] * c[j]) + rnd(partner[j] * s[j]) ),
 *   partner[j] = -x[j + h] for j < h,  x[j - h] for j >= h,
 * with c, s the full cos/sin row (c[j] and c[j + h] are NOT assumed equal).
 * `rnd` is the bf16 rounding for the eager policy and the identity for the
 * exact-arithmetic policy, so both policies run this one function.
 * ------------------------------------------------------------------------- */
typedef double (*rounder_fn)(double);

static void rope_row(const double *x, const double *c, const double *s,
                     int64_t D, int64_t R, rounder_fn rnd, double *out)
{
    int64_t h = R / 2;
    for (int64_t j = 0; j < R; ++j) {
        double partner = (j < h) ? -x[j + h] : x[j - h];
        out[j] = rnd(rnd(x[j] * c[j]) + rnd(partner * s[j]));
    }
    for (int64_t j = R; j < D; ++j)
        out[j] = x[j];
}

/* One row in the eager bf16 policy; `work` holds 4*D doubles. */
static void rope_row_bf16(const uint16_t *x_row, const uint16_t *cos_row,
                          const uint16_t *sin_row, int64_t D, int64_t R, double *work,
                          uint16_t *out_row)
{
    double *x = work, *c = work + D, *s = work + 2 * D, *o = work + 3 * D;
    for (int64_t j = 0; j < D; ++j)
        x[j] = oracle_bf16_to_double(x_row[j]);
    for (int64_t j = 0; j < R; ++j) {
        c[j] = oracle_bf16_to_double(cos_row[j]);
        s[j] = oracle_bf16_to_double(sin_row[j]);
    }
    rope_row(x, c, s, D, R, to_bf16_value, o);
    for (int64_t j = 0; j < R; ++j)
        out_row[j] = oracle_double_to_bf16(o[j], 0);
    for (int64_t j = R; j < D; ++j)
        out_row[j] = x_row[j]; /* tail: the bits themselves */
}

#define ORACLE_MAX_D 65536

/*
 * Rows form: n independent rows of width D; row i is rotated with cos/sin
 * row i (cos_rows/sin_rows are (n, R)).  All arrays contiguous bf16 bits.
 */
ORACLE_API int oracle_rope_rows(const uint16_t *x_rows, const uint16_t *cos_rows,
                                const uint16_t *sin_rows, int64_t n, int64_t D, int64_t R,
                                uint16_t *out_rows)
{
    if (D < 1 || D > ORACLE_MAX_D || R < 0 || R > D || R % 2 != 0)
        return -1;
    double *work = malloc(4 * (size_t)D * sizeof(double));
    if (!work)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        rope_row_bf16(x_rows + i * D, cos_rows + i * R, sin_rows + i * R, D, R, work,
                      out_rows + i * D);
    free(work);
    return 0;
}

/*
 * Tensor form on the page's shapes: x and out are contiguous (B, S, H, D);
 * cos/sin are (B*S, R) and every head h of token (b, s) uses row b*S + s.
 */
ORACLE_API int oracle_rope_rotate_half(const uint16_t *x, int64_t B, int64_t S, int64_t H,
                                       int64_t D, int64_t R, const uint16_t *cos_tab,
                                       const uint16_t *sin_tab, uint16_t *out)
{
    if (D < 1 || D > ORACLE_MAX_D || R < 0 || R > D || R % 2 != 0)
        return -1;
    double *work = malloc(4 * (size_t)D * sizeof(double));
    if (!work)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t hh = 0; hh < H; ++hh) {
                int64_t row = b * S + s;
                int64_t at = ((b * S + s) * H + hh) * D;
                rope_row_bf16(x + at, cos_tab + row * R, sin_tab + row * R, D, R, work,
                              out + at);
            }
    free(work);
    return 0;
}

/* Exact-arithmetic policy of the same rotation (double in, double out). */
ORACLE_API void oracle_rope_rotate_half_exact(const double *x, int64_t B, int64_t S, int64_t H,
                                              int64_t D, int64_t R, const double *cos_tab,
                                              const double *sin_tab, double *out)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t hh = 0; hh < H; ++hh) {
                int64_t row = b * S + s;
                int64_t at = ((b * S + s) * H + hh) * D;
                rope_row(x + at, cos_tab + row * R, sin_tab + row * R, D, R, keep_exact,
                         out + at);
            }
}

/* ---------------------------------------------------------------------------
 * GEGLU with activation rounding          [ERNIE-fuse §3]
 *
 * The eager form is up * F.gelu(gate) on bf16 tensors: F.gelu's default is
 * the exact (erf) GELU, GELU(x) = x * Phi(x), Phi(x) = erfc(-x / sqrt 2) / 2,
 * whose result is rounded to bf16; the multiply by up is rounded again.  The
 * fused op splits its input's last dimension in half: the first `hidden`
 * columns are the gate, the next `hidden` the up projection.
 * ------------------------------------------------------------------------- */

/* GELU(x) in double (exact-arithmetic policy). */
ORACLE_API double oracle_gelu_exact(double x)
{
    return 0.5 * x * erfc(-x / sqrt(2.0));
}

/*
 * rne_bf16(GELU(x)) for a bf16 input.
 *
 * For |x| <= 1 the value is split as x/2 + x*(Phi(x) - 1/2), the second part
 * being x*erf(x/sqrt 2)/2 >= 0.  For tiny x that part is far below the
 * double resolution of x/2, and x/2 can be an exact bf16 midpoint (x a
 * subnormal-range bf16 with an odd last bit); the sign of the lost part then
 * decides the rounding.  Elsewhere the erfc form is used directly (it does
 * not cancel for large negative x).
 */
ORACLE_API uint16_t oracle_gelu_bf16(uint16_t g)
{
    double x = oracle_bf16_to_double(g);
    if (isnan(x))
        return 0x7FC0u;
    if (isinf(x))
        return x > 0 ? 0x7F80u : 0x7FC0u; /* GELU(-inf) = -inf * 0 */
    if (x == 0.0)
        return g; /* GELU(+-0) = +-0 */
    if (fabs(x) <= 1.0) {
        double hi = 0.5 * x;                      /* exact */
        double lo = 0.5 * x * erf(x / sqrt(2.0));   /* x (Phi(x) - 1/2) */
        double sum = hi + lo;
        double lost = (hi - sum) + lo;            /* exact error of the sum, |hi| >= |lo| */
        return oracle_double_to_bf16(sum, (lost > 0) - (lost < 0));
    }
    return oracle_double_to_bf16(oracle_gelu_exact(x), 0);
}

/*
 * input: (rows, 2*hidden) bf16, row stride in_stride elements;
 * out:   (rows, hidden)   bf16, row stride out_stride elements.
 * out[r][j] = rne_bf16( up[r][j] * rne_bf16(GELU(gate[r][j])) ), the product
 * of two bf16 values being exact in double.
 */
ORACLE_API void oracle_gelu_and_mul(const uint16_t *input, int64_t rows, int64_t hidden,
                                    int64_t in_stride, uint16_t *out, int64_t out_stride)
{
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *gate = input + r * in_stride;
        const uint16_t *up = gate + hidden;
        for (int64_t j = 0; j < hidden; ++j) {
            double gl = oracle_bf16_to_double(oracle_gelu_bf16(gate[j]));
            double u = oracle_bf16_to_double(up[j]);
            out[r * out_stride + j] = oracle_double_to_bf16(u * gl, 0);
        }
    }
}

/* ---------------------------------------------------------------------------
 * The gate_up projection feeding GEGLU, and GEGLU on its output
 *                                   [ERNIE-fuse §3, the projection before it]
 *
 * The page's GEGLU input is the output of the FFN's gate_up linear layer,
 * computed eagerly as a bf16 matrix product: every product of two bf16
 * values is accumulated in higher precision and the sum is rounded once to
 * bf16.  Reading used here (the page shows no bias term): out = x W^T with
 * x (M, K) and W (N, K), both bf16 row-major with the given row strides,
 *   out[m][n] = rne_bf16( sum_k x[m][k] * w[n][k] ),
 * the sum taken exactly.  Each product of two bf16 values is exact in
 * double; the sum is kept as an unevaluated pair (s, c) updated with the
 * error-free TwoSum of Knuth, so that s + c carries the sum to about 106
 * bits, and it is rounded once with the sign of what the final double
 * addition dropped as the sticky bit.
 * ------------------------------------------------------------------------- */
static void two_sum(double a, double b, double *s, double *e)
{
    double t = a + b;
    double bb = t - a;
    *e = (a - (t - bb)) + (b - bb);
    *s = t;
}

ORACLE_API void oracle_gemm_bf16(const uint16_t *x, int64_t M, int64_t K, int64_t x_stride,
                                 const uint16_t *w, int64_t N, int64_t w_stride, uint16_t *out,
                                 int64_t out_stride)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, c = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double prod = oracle_bf16_to_double(x[m * x_stride + k]) *
                              oracle_bf16_to_double(w[n * w_stride + k]);
                double e;
                two_sum(s, prod, &s, &e);
                c += e;
            }
            double hi, lo;
            two_sum(s, c, &hi, &lo);
            out[m * out_stride + n] = oracle_double_to_bf16(hi, (lo > 0) - (lo < 0));
        }
    }
}

/*
 * GEGLU fused after the projection: W holds the gate rows 0 .. H-1 and the
 * up rows H .. 2H-1, so gate_up = rne_bf16(x W^T) is (M, 2H) with the gate
 * first, and out = oracle_gelu_and_mul(gate_up), (M, H).
 */
ORACLE_API int oracle_gemm_geglu(const uint16_t *x, int64_t M, int64_t K, int64_t x_stride,
                                 const uint16_t *w, int64_t H, int64_t w_stride, uint16_t *out,
                                 int64_t out_stride)
{
    uint16_t *gate_up = (uint16_t *)malloc((size_t)(M > 0 ? M : 1) * (size_t)(2 * H > 0 ? 2 * H : 1) *
                                           sizeof(uint16_t));
    if (!gate_up)
        return -1;
    oracle_gemm_bf16(x, M, K, x_stride, w, 2 * H, w_stride, gate_up, 2 * H);
    oracle_gelu_and_mul(gate_up, M, H, 2 * H, out, out_stride);
    free(gate_up);
    return 0;
}

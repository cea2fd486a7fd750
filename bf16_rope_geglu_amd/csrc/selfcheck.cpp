// rgg_selfcheck (include/rgg.h): the page's bit-exact fusion gate
// [ERNIE-fuse §3], run on the device without an eager twin.  Inputs are
// staged in the caller's workspace, the library's own entry points run on the
// caller's stream, and the results are compared on the host with expected
// bits that are derived by hand from the definitions (IEEE binary32 / bf16
// rounding, the rotate-half formula, textbook normal CDF values) or, for the
// eight cos/sin values, from a 50-digit evaluation of the cosine and sine of
// the fp32 angle.  The derivations are given beside the values.
#include <stdint.h>
#include <string.h>

#include <vector>

#include <hip/hip_runtime_api.h>

#include "rgg.h"
#include "selfcheck.h"

namespace {

// Workspace layout (byte offsets, each 256-byte aligned).
constexpr size_t kFreq = 0;           // 8 fp32 angles, (S, B, 1, R) = (1, 1, 1, 8)
constexpr size_t kCsCos = 256;        // 8 bf16
constexpr size_t kCsSin = 512;        // 8 bf16
constexpr size_t kRaX = 768;          // rotate-half worked vectors: (1, 1, 1, 16), R = 16
constexpr size_t kRaOut = 1024;
constexpr size_t kRaCos = 1280;
constexpr size_t kRaSin = 1536;
constexpr size_t kRbX = 1792;         // zero angle: (1, 1, 2, 32), R = 16
constexpr size_t kRbOut = 2048;
constexpr size_t kRbCos = 2304;
constexpr size_t kRbSin = 2560;
constexpr size_t kGe1In = 4096;       // GEGLU (256, 2*256): gate = every bf16 pattern, up = 1
constexpr size_t kGe1Out = kGe1In + 256 * 512 * 2;
constexpr size_t kGe2In = kGe1Out + 256 * 256 * 2;   // same gates, up = 2
constexpr size_t kGe2Out = kGe2In + 256 * 512 * 2;
// bit 6: the projection, fused and plain: x (40, 64) one-hot rows
// (x[m][k] = 1 for k = m), W (128, 64); out[m][n] = W[n][m] exactly.
constexpr int kPm = 40, kPk = 64, kPh = 64;
constexpr size_t kPx = kGe2Out + 256 * 256 * 2;
constexpr size_t kPw = kPx + kPm * kPk * 2;
constexpr size_t kPfOut = kPw + 2 * kPh * kPk * 2;
constexpr size_t kPpOut = kPfOut + kPm * kPh * 2;
constexpr size_t kUsed = kPpOut + kPm * 2 * kPh * 2;
static_assert(kPx % 256 == 0 && kPw % 256 == 0 && kPfOut % 256 == 0 && kPpOut % 256 == 0,
              "projection operands 256-byte aligned");
static_assert(kUsed <= RGG_SELFCHECK_WORKSPACE_BYTES, "workspace layout");
static_assert(kUsed == rgg::kSelfcheckBytes, "staging size");

// bit 0: cos/sin of fp32 angles, correctly rounded (50-digit evaluation).
const uint32_t kAngles[8] = {0x00000000u, 0x80000000u, 0x40490FDBu, 0x3FC90FDBu,
                             0x40C90FDBu, 0x3F860A92u, 0x3F060A92u, 0x42C80000u};
// 0: cos 1, sin +0.   -0: cos 1, sin -0.
// fl(pi) = 3.14159274: cos = -0.999999999999996 -> -1; sin = -8.742278e-8 ->
//   1.4668 * 2^-24, significand 187.74 of 128 -> 188 -> 0xB3BC.
// fl(pi/2) = 1.57079637: cos = -4.371139e-8 -> significand 187.74 -> 0xB33C; sin -> 1.
// fl(2 pi) = 6.28318548: cos -> 1; sin = 1.748456e-7 -> 0x343C.
// fl(pi/3) = 1.04719758: cos = 0.4999999748 -> 0.5; sin = 0.8660254184 -> 221.70 -> 222/256.
// fl(pi/6) = 0.52359879: cos = 0.8660253965 -> 222/256; sin = 0.5000000126 -> 0.5.
// 100: cos = 0.8623188723 -> 220.75 -> 221/256 (0x3F5D); sin = -0.5063656411 -> 129.63 -> 130/256.
const uint16_t kCos[8] = {0x3F80, 0x3F80, 0xBF80, 0xB33C, 0x3F80, 0x3F00, 0x3F5E, 0x3F5D};
const uint16_t kSin[8] = {0x0000, 0x8000, 0xB3BC, 0x3F80, 0x343C, 0x3F5E, 0x3F00, 0xBF02};

// bit 1: rotate-half worked vectors, R = 2 each, laid side by side as the
// eight column pairs (j, j + 8) of one R = 16 row.  Columns: x1 x2 c1 s1 c2 s2
// -> out1 out2, out1 = rne(rne(x1*c1) + rne(-x2*s1)), out2 = rne(rne(x2*c2) +
// rne(x1*s2)).
const uint16_t kRope[8][8] = {
    // 1.5*(1+2^-7) = 193.5/128 ties to 194/128; -1 -> 0.515625 (an FMA gives 0x3F03);
    // out2: 1.0078125 + 1.5 = 160.5/64 ties to 160/64 = 2.5.
    {0x3FC0, 0x3F80, 0x3F81, 0x3F80, 0x3F81, 0x3F80, 0x3F04, 0x4020},
    // 1.5*(1+3/128) = 196.5/128 ties to 196 (ties away would give 0x3FC5); sin 0.
    {0x3FC0, 0x3F80, 0x3F83, 0x0000, 0x3F83, 0x0000, 0x3FC4, 0x3F83},
    // -(+0)*1 = -0 leaves 1.515625; out2 = +0 + +0.
    {0x3FC0, 0x0000, 0x3F81, 0x3F80, 0x3F80, 0x0000, 0x3FC2, 0x0000},
    // subnormal 3*2^-133 times 0.5 ties between 1 and 2 steps -> 2 (not flushed).
    {0x0003, 0x0000, 0x3F00, 0x3F80, 0x3F80, 0x3F80, 0x0002, 0x0003},
    // max + max overflows to +inf; max - max = +0.
    {0x7F7F, 0x7F7F, 0x3F80, 0xBF80, 0x3F80, 0xBF80, 0x7F80, 0x0000},
    // -0 + -0 = -0; +0 + -0 = +0.
    {0x8000, 0x0000, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x8000, 0x0000},
    // different angle per half: 0.5 - 2*0.25 = +0; 2*0.75 + 0.125 = 1.625.
    {0x3F80, 0x4000, 0x3F00, 0x3E80, 0x3F40, 0x3E00, 0x0000, 0x3FD0},
    // the first vector again
    {0x3FC0, 0x3F80, 0x3F81, 0x3F80, 0x3F81, 0x3F80, 0x3F04, 0x4020},
};

// bit 3: G = rne_bf16(x * Phi(x)) at textbook points (Phi to 10 digits, e.g.
// Abramowitz & Stegun table 26.1); |G| / step is at least 0.01 from a tie.
const uint16_t kGelu[8][2] = {
    {0x3F80, 0x3F57},  // x = 1:    0.8413447461, step 2^-8:  215.38 -> 215
    {0x4000, 0x3FFA},  // x = 2:    1.9544997362, step 2^-7:  250.18 -> 250
    {0xBF80, 0xBE22},  // x = -1:  -0.1586552539, step 2^-10: 162.46 -> 162
    {0x3F00, 0x3EB1},  // x = 0.5:  0.3457312306, step 2^-9:  177.01 -> 177
    {0x4040, 0x4040},  // x = 3:    2.9959503060, step 2^-6:  191.74 -> 192
    {0xC000, 0xBD3A},  // x = -2:  -0.0455002638, step 2^-12: 186.37 -> 186
    {0xC040, 0xBB85},  // x = -3:  -0.0040496940, step 2^-15: 132.70 -> 133
    {0xC0B0, 0xB3E0},  // x = -5.5: -1.044426e-7, step 2^-31: 224.29 -> 224
};

// Gate and up of output (m, j) of the projection check: a textbook point of
// the GELU table above and up = 1 or 2, so rne(up * G) is G or 2G exactly.
uint16_t proj_gate(int m, int j) { return kGelu[(m + j) % 8][0]; }
uint16_t proj_up(int m, int j) { return (m + j) % 2 ? 0x4000 : 0x3F80; }

float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t bf16_bits(float f)  // f exactly representable in bf16
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

bool is_nan(uint16_t b) { return (b & 0x7F80u) == 0x7F80u && (b & 0x7Fu) != 0; }

template <typename T>
void put(uint8_t *img, size_t off, size_t i, T v)
{
    memcpy(img + off + i * sizeof(T), &v, sizeof(T));
}

template <typename T>
T get(const uint8_t *img, size_t off, size_t i)
{
    T v;
    memcpy(&v, img + off + i * sizeof(T), sizeof(T));
    return v;
}

// Zero-angle input for bit 2: two heads of 32 columns mixing signed zeros,
// subnormals, normal and large values.
uint16_t zero_angle_x(int i)
{
    static const uint16_t pat[16] = {0x8000, 0x0000, 0x0001, 0x807F, 0x3F80, 0xBFC0, 0x7F7F, 0xFF7F,
                                     0x0080, 0x8000, 0x4049, 0xC2C8, 0x8000, 0x3A80, 0x0000, 0x8001};
    return pat[(i * 7 + i / 16) % 16];
}

}  // namespace

int rgg::selfcheck_run(uint8_t *ws, hipStream_t stream, uint32_t checks, uint32_t *failed,
                       uint8_t *in, uint8_t *out)
{
    if (failed)
        *failed = 0;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess)
        return RGG_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone)
        return RGG_ERR_CAPTURING;
    const bool c_tab = checks & 1u, c_ra = checks & 2u, c_rb = checks & 4u;
    const bool c_ge = checks & (7u << 3), c_proj = checks & (1u << 6);
    memset(in, 0, kUsed);
    memset(out, 0, kUsed);
    for (int j = 0; j < 8; ++j)
        put<uint32_t>(in, kFreq, j, kAngles[j]);
    for (int j = 0; j < 8; ++j) {
        put<uint16_t>(in, kRaX, j, kRope[j][0]);
        put<uint16_t>(in, kRaX, 8 + j, kRope[j][1]);
        put<uint16_t>(in, kRaCos, j, kRope[j][2]);
        put<uint16_t>(in, kRaSin, j, kRope[j][3]);
        put<uint16_t>(in, kRaCos, 8 + j, kRope[j][4]);
        put<uint16_t>(in, kRaSin, 8 + j, kRope[j][5]);
    }
    for (int i = 0; i < 64; ++i)
        put<uint16_t>(in, kRbX, i, zero_angle_x(i));
    for (int j = 0; j < 16; ++j) {
        put<uint16_t>(in, kRbCos, j, 0x3F80);
        put<uint16_t>(in, kRbSin, j, 0x0000);
    }
    for (uint32_t g = 0; g < 65536; ++g) {
        const size_t r = g >> 8, c = g & 255;
        put<uint16_t>(in, kGe1In, r * 512 + c, (uint16_t)g);
        put<uint16_t>(in, kGe1In, r * 512 + 256 + c, 0x3F80);  // up = 1
        put<uint16_t>(in, kGe2In, r * 512 + c, (uint16_t)g);
        put<uint16_t>(in, kGe2In, r * 512 + 256 + c, 0x4000);  // up = 2
    }

    for (int m = 0; m < kPm; ++m)
        put<uint16_t>(in, kPx, (size_t)m * kPk + m, 0x3F80);
    for (int j = 0; j < kPh; ++j)
        for (int m = 0; m < kPm; ++m) {
            put<uint16_t>(in, kPw, (size_t)j * kPk + m, proj_gate(m, j));
            put<uint16_t>(in, kPw, (size_t)(kPh + j) * kPk + m, proj_up(m, j));
        }

    if (hipMemcpyAsync(ws, in, kUsed, hipMemcpyHostToDevice, stream) != hipSuccess)
        return RGG_ERR_HIP;
    int st = RGG_OK;
    if (c_tab)
        st = rope_cossin_precompute(reinterpret_cast<const float *>(ws + kFreq), 1, 1, 8, 8, 8,
                                    reinterpret_cast<uint16_t *>(ws + kCsCos),
                                    reinterpret_cast<uint16_t *>(ws + kCsSin), stream);
    const rgg_rope_view va = {reinterpret_cast<const uint16_t *>(ws + kRaX),
                              reinterpret_cast<uint16_t *>(ws + kRaOut), 16, 16, 16, 16, 16, 16};
    if (st == RGG_OK && c_ra)
        st = rope_rotate_half_bf16(&va, 1, 1, 1, 1, 16, 16,
                                   reinterpret_cast<const uint16_t *>(ws + kRaCos),
                                   reinterpret_cast<const uint16_t *>(ws + kRaSin), stream);
    const rgg_rope_view vb = {reinterpret_cast<const uint16_t *>(ws + kRbX),
                              reinterpret_cast<uint16_t *>(ws + kRbOut), 64, 64, 32, 64, 64, 32};
    if (st == RGG_OK && c_rb)
        st = rope_rotate_half_bf16(&vb, 1, 1, 1, 2, 32, 16,
                                   reinterpret_cast<const uint16_t *>(ws + kRbCos),
                                   reinterpret_cast<const uint16_t *>(ws + kRbSin), stream);
    if (st == RGG_OK && c_ge)
        st = gelu_and_mul_bf16(reinterpret_cast<const uint16_t *>(ws + kGe1In), 256, 256, 512,
                               reinterpret_cast<uint16_t *>(ws + kGe1Out), 256, stream);
    if (st == RGG_OK && c_ge)
        st = gelu_and_mul_bf16(reinterpret_cast<const uint16_t *>(ws + kGe2In), 256, 256, 512,
                               reinterpret_cast<uint16_t *>(ws + kGe2Out), 256, stream);
    if (st == RGG_OK && c_proj)
        st = gemm_geglu_bf16(reinterpret_cast<const uint16_t *>(ws + kPx), kPm, kPk, kPk,
                             reinterpret_cast<const uint16_t *>(ws + kPw), kPh, kPk,
                             reinterpret_cast<uint16_t *>(ws + kPfOut), kPh, stream);
    if (st == RGG_OK && c_proj)
        st = gemm_bf16_nt(reinterpret_cast<const uint16_t *>(ws + kPx), kPm, kPk, kPk,
                          reinterpret_cast<const uint16_t *>(ws + kPw), 2 * kPh, kPk,
                          reinterpret_cast<uint16_t *>(ws + kPpOut), 2 * kPh, stream);
    if (st != RGG_OK) {
        (void)hipStreamSynchronize(stream);
        return st;
    }
    if (hipMemcpyAsync(out, ws, kUsed, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return RGG_ERR_HIP;

    uint32_t mask = 0;
    // bit 0
    for (int j = 0; j < 8; ++j)
        if (get<uint16_t>(out, kCsCos, j) != kCos[j] || get<uint16_t>(out, kCsSin, j) != kSin[j])
            mask |= 1u << 0;
    // bit 1
    for (int j = 0; j < 8; ++j)
        if (get<uint16_t>(out, kRaOut, j) != kRope[j][6] ||
            get<uint16_t>(out, kRaOut, 8 + j) != kRope[j][7])
            mask |= 1u << 1;
    // bit 2: cos 1, sin 0.  Rotated column j: x*1 + p with p = +-0 of sign
    // !sign(x[j+8]) (first half, -x2*0) or sign(x[j-8]) (second half); x + p = x
    // except that -0 + +0 = +0.  Tail columns keep their bits.
    for (int h = 0; h < 2; ++h) {
        for (int j = 0; j < 32; ++j) {
            const uint16_t x = zero_angle_x(h * 32 + j);
            uint16_t want = x;
            if (j < 16 && x == 0x8000) {
                const uint16_t partner = zero_angle_x(h * 32 + (j < 8 ? j + 8 : j - 8));
                const bool p_neg = j < 8 ? !(partner >> 15) : (partner >> 15);
                want = p_neg ? 0x8000 : 0x0000;
            }
            if (get<uint16_t>(out, kRbOut, h * 32 + j) != want)
                mask |= 1u << 2;
        }
    }
    // bits 3-5
    auto g1 = [&](uint32_t g) {
        return get<uint16_t>(out, kGe1Out, (g >> 8) * 256 + (g & 255));
    };
    auto g2 = [&](uint32_t g) {
        return get<uint16_t>(out, kGe2Out, (g >> 8) * 256 + (g & 255));
    };
    for (int k = 0; k < 8; ++k)
        if (g1(kGelu[k][0]) != kGelu[k][1])
            mask |= 1u << 3;
    for (uint32_t g = 0; g < 65536; ++g) {
        const uint32_t a = g & 0x7FFFu, neg = g >> 15;
        const uint16_t G = g1(g);
        bool ok = true;
        if (a > 0x7F80u)
            ok = is_nan(G);
        else if (a == 0x7F80u)
            ok = neg ? is_nan(G) : G == 0x7F80u;
        else if (a >= 0x4180u)                      // |x| >= 16
            ok = neg ? G == 0x8000u : G == g;
        else if (a == 0)
            ok = G == g;
        else if (a < 0x0100u)                       // |x| < 2^-125: x/2, halfway up
            ok = neg ? G == (0x8000u | (a >> 1)) : G == ((a + 1) >> 1);
        else if (a < 0x3A80u)                       // 2^-125 <= |x| < 2^-10: x/2
            ok = G == g - 0x80u;
        else if (neg)                               // x*Phi(x) in (x, 0]
            ok = (G == 0x8000u || (G >> 15)) && (G & 0x7FFFu) <= a;
        else                                        // G(x) > 0 for x > 0
            ok = !(G >> 15) && G != 0;
        if (!neg && a > 0 && a < 0x7F80u && g1(g - 1) > G)  // increasing on x > 0
            ok = false;
        if (!ok)
            mask |= 1u << 4;
        const float gv = bf16_value(G);
        if (!is_nan(G) && (G & 0x7FFFu) < 0x7F00u && g2(g) != bf16_bits(2.0f * gv))
            mask |= 1u << 5;
    }
    // bit 6: the plain projection copies W's column m into row m; the fused
    // output is G(gate) for up = 1 and 2 G(gate) for up = 2, both exact.
    for (int m = 0; m < kPm; ++m)
        for (int j = 0; j < kPh; ++j) {
            const uint16_t gate = proj_gate(m, j), up = proj_up(m, j);
            uint16_t G = 0;
            for (int k = 0; k < 8; ++k)
                if (kGelu[k][0] == gate)
                    G = kGelu[k][1];
            const uint16_t want = up == 0x4000 ? bf16_bits(2.0f * bf16_value(G)) : G;
            if (get<uint16_t>(out, kPfOut, (size_t)m * kPh + j) != want ||
                get<uint16_t>(out, kPpOut, (size_t)m * 2 * kPh + j) != gate ||
                get<uint16_t>(out, kPpOut, (size_t)m * 2 * kPh + kPh + j) != up)
                mask |= 1u << 6;
        }
    mask &= checks;
    if (failed)
        *failed = mask;
    return mask ? RGG_ERR_SELFCHECK : RGG_OK;
}

extern "C" int rgg_selfcheck(void *workspace, int64_t workspace_bytes, hipStream_t stream,
                             uint32_t *failed)
{
    if (failed)
        *failed = 0;
    if (!workspace)
        return RGG_ERR_NULL;
    if (workspace_bytes < RGG_SELFCHECK_WORKSPACE_BYTES)
        return RGG_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255)
        return RGG_ERR_ALIGN;
    std::vector<uint8_t> in(kUsed), out(kUsed);
    return rgg::selfcheck_run(static_cast<uint8_t *>(workspace), stream, RGG_SELFCHECK_ALL, failed,
                              in.data(), out.data());
}

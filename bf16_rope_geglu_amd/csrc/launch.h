// Internal interface between the C ABI layer (capi.cpp) and the HIP kernels
// (kernels.hip).  Parameter blocks are passed to the kernels by value.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace rgg {

// Unsigned division of n < 2^31 by a fixed d >= 1 with one multiply-high,
// shift and add: Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication" (PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l.
struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d)
        ++l;
    uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

constexpr int kMaxViews = 4;
constexpr int kThreads = 256;  // one workgroup = four wave64s

struct RopeView {
    const uint16_t *x;
    uint16_t *out;
    int64_t xs_b, xs_s, xs_h;
    int64_t os_b, os_s, os_h;
};

struct RopeParams {
    RopeView v[kMaxViews];
    const uint16_t *cos;
    const uint16_t *sin;
    int64_t tokens;        // B * S
    int32_t n_views;
    int32_t H, D, R;
    int32_t half;          // R / 2
    int32_t tok_per_wg;    // tokens handled by one workgroup (of one view)
    int32_t tail_mask;     // bit v set: copy the tail of view v
    int32_t slots_tail;    // R/16 + (D - R)/8 work slots per head when the tail is copied
    int32_t wave_stage;    // one-token workgroups: each wave stages its own cos/sin row
    uint32_t chunk0;       // first token chunk of this launch (long ranges take several)
    int32_t parts;         // workgroups per (token chunk, view)
    FastDiv div_vp;        // divisor n_views * parts
    FastDiv div_parts;     // divisor parts
    FastDiv div_s;         // token -> (b, s)
    FastDiv div_views;     // workgroup -> (token chunk, view)
    FastDiv div_heads;     // divisor H
    FastDiv div_slots;     // divisor R/16: item -> (token-local, head, slot), no tail
    FastDiv div_slots_tail;  // divisor slots_tail
    FastDiv div_vecs;      // divisor D/8: vector index -> (head, vector of the head row);
                           // rope_lean_kernel: H * D/8, vector index -> (token, vector)
    // cross-lane kernels (heads of at most 128 columns)
    uint32_t vecs_per_view;  // tokens * H * D/8
    int32_t log_vecs;        // log2(D/8)
    int32_t chunk_vecs;      // vectors per workgroup (rope_xlane_kernel)
    uint32_t chunks;         // workgroups per view (rope_lean_kernel)
};

struct CosSinParams {
    const float *freqs;
    uint16_t *cos;
    uint16_t *sin;
    int64_t stride_s, stride_b;
    uint32_t vec_total;    // B * S * R / 8
    int32_t R;
    FastDiv div_vecs;      // divisor R / 8: vector -> (row, column group)
    FastDiv div_s;         // row -> (b, s)
};

// Up to this many lanes of 4 columns, the cos/sin table kernels give each
// lane 4 columns of each half instead of 8: twice as many lanes fill more of
// the chip, and each lane's chain of sincos is half as long.  Above it the
// 8-column lanes are faster (measured at 2^19 lanes of 4).
constexpr uint64_t kTableNarrowLanes = 1u << 18;

constexpr int kGridOmegaArgs = 256;  // half-column frequencies carried in the kernel arguments

struct CosSinGridParams {
    const int32_t *t_offset;   // per batch row, or null
    uint16_t *cos;
    uint16_t *sin;
    double theta;
    uint32_t rows;             // B * S
    uint32_t groups_total;     // rows * (R / W): lanes of W half-columns (set by the launcher)
    int32_t R;
    int32_t h0, h01;           // d0/2 and (d0 + d1)/2: first half-column of axes 1 and 2
    int32_t d[3];
    FastDiv div_groups;        // divisor R / W: lane -> (row, group) (set by the launcher)
    FastDiv div_s;             // row -> (b, s)
    FastDiv div_hw;            // s -> (t, h*Wg + w)
    FastDiv div_w;             // h*Wg + w -> (h, w)
    int32_t host_omega;        // 1: omega[] holds theta^(-2i/d_k) for every half-column
    double omega[kGridOmegaArgs];
};

struct GegluParams {
    const uint16_t *in;
    uint16_t *out;
    int64_t in_stride, out_stride;
    uint32_t vec_total;    // rows * hidden / 8
    int32_t hidden;
    FastDiv div_vecs;      // divisor hidden / 8: vector -> (row, column group)
};

// The gate_up projection x W^T (bf16, fp32 accumulation) with its output
// rounded to bf16, either stored (gate columns 0..H-1, up columns H..2H-1)
// or passed through GEGLU in the epilogue.
struct GemmParams {
    const uint16_t *x;     // (M, K), row stride x_stride
    const uint16_t *w;     // (2H, K), row stride w_stride: gate rows, then up rows
    uint16_t *out;         // (M, 2H) or, with GEGLU, (M, H); row stride out_stride
    int64_t x_stride, w_stride, out_stride;
    int64_t M;
    int32_t H;
    int32_t K;             // a multiple of 64
    uint32_t mblocks;      // ceil(M / 256) row blocks
    uint32_t nblocks;      // ceil(H / 128) column blocks
};

// Launchers: enqueue on `stream`, return the hipError_t of the launch.
hipError_t launch_rope_cossin(const CosSinParams &p, hipStream_t stream);
hipError_t launch_rope_cossin_grid(const CosSinGridParams &p, hipStream_t stream);
hipError_t launch_rope_rotate_half(const RopeParams &p, hipStream_t stream);
hipError_t launch_gelu_and_mul(const GegluParams &p, int grid, hipStream_t stream);
hipError_t launch_gemm_gate_up(const GemmParams &p, bool geglu, hipStream_t stream);
hipError_t launch_build_gelu_table(hipStream_t stream);

// Tunables chosen by the host layer.
int rope_tokens_per_workgroup(int H, int D, int R);
int geglu_grid(uint32_t vec_total, int cu_count);

}  // namespace rgg

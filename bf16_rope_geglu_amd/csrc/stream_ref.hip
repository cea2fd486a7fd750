// Streaming references for measurement: how fast plain streams that read and
// write the same bytes as a kernel run on this GPU.  bench.py times a family
// of them beside each kernel and reports the fastest as the practical ceiling
// for that traffic.  Not part of the library's C ABI; computes nothing of the
// method.
//
//   int rgg_stream_ref(const void *a, const void *b, void *out, int64_t n_vec,
//                      int block, int vpl, int grid, int policy, int lds,
//                      hipStream_t stream);
//
// a == NULL, b == NULL: out[i] = i              (write only)
// b == NULL:            out[i] = a[i]           (1 read : 1 write)
// b != NULL:            out[i] = a[i] ^ b[i]    (2 reads : 1 write)
// for i < n_vec 16-byte vectors.  The work is cut into chunks of block * vpl
// consecutive vectors; lane t of a workgroup takes vectors t, t + block, ...
// of its chunk, issuing all vpl loads before its first store, so every wave
// instruction covers whole contiguous lines.
//   grid == 0: one chunk per workgroup, one pass (grid = number of chunks);
//   grid  > 0: `grid` workgroups walk the chunks with a stride of `grid`,
//              each loading its next chunk before storing the current one.
// policy bit 0: nontemporal loads; bits 1-2: stores 0 plain, 1 nontemporal,
// 2 write-through to the device coherence point (sc1), 3 both.  `lds` bytes
// of (unused) LDS per workgroup cap how many workgroups share a compute unit
// (160 KiB of LDS each): 0 leaves occupancy to the register count.
// block is 64..1024 (a multiple of 64), vpl 1, 2, 4 or 8; all pointers are
// device memory, 16-byte aligned.  Returns 0, 2 for bad arguments, 6 for a
// launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// cache-policy bits of a buffer store on gfx950: sc0 1, nt 2, sc1 16
template <int St>
__device__ __forceinline__ void store_vec(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, v4u v)
{
    constexpr int aux = (St & 1 ? 2 : 0) | (St & 2 ? 16 : 0);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, aux);
}

template <bool NtLoad>
__device__ __forceinline__ v4u load_vec(const v4u *p)
{
    if constexpr (NtLoad)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int Reads, int V, bool NtLoad, int St>
__global__ __launch_bounds__(1024) void stream_ref_kernel(const v4u *a, const v4u *b, v4u *out,
                                                          uint32_t n)
{
    const uint32_t chunk = blockDim.x * V;
    const uint32_t nchunks = (n + chunk - 1) / chunk;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(out, 0, 0x7FFFFFF0, 0x00020000);
    const uint32_t step = gridDim.x;
    uint32_t c = blockIdx.x;
    v4u x[V];
    auto fetch = [&](uint32_t cc, v4u *dst) {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const uint32_t i = min(cc * chunk + u * blockDim.x + threadIdx.x, n - 1);
            v4u y = v4u{i, i, i, i};
            if (Reads >= 1)
                y = load_vec<NtLoad>(a + i);
            if (Reads == 2)
                y ^= load_vec<NtLoad>(b + i);
            dst[u] = y;
        }
    };
    auto put = [&](uint32_t cc, const v4u *src) {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const uint32_t i = cc * chunk + u * blockDim.x + threadIdx.x;
            if (i < n)
                store_vec<St>(r, i * 16u, src[u]);
        }
    };
    // Two register sets take turns (no copies between them), so each store
    // waits only for its own chunk's loads while the next chunk's are in
    // flight.  The next chunk is fetched unconditionally (past the end the
    // clamped index re-reads the last vector), which keeps the wait counts
    // the compiler derives exact.
    v4u y[V];
    if (c >= nchunks)
        return;
    fetch(c, x);
    for (;;) {
        const uint32_t c1 = c + step;
        fetch(c1, y);
        put(c, x);
        if (c1 >= nchunks)
            break;
        const uint32_t c2 = c1 + step;
        fetch(c2, x);
        put(c1, y);
        if (c2 >= nchunks)
            break;
        c = c2;
    }
}

template <int Reads, int V, bool NtLoad>
void *pick_store(int st)
{
    switch (st) {
    case 0: return reinterpret_cast<void *>(stream_ref_kernel<Reads, V, NtLoad, 0>);
    case 1: return reinterpret_cast<void *>(stream_ref_kernel<Reads, V, NtLoad, 1>);
    case 2: return reinterpret_cast<void *>(stream_ref_kernel<Reads, V, NtLoad, 2>);
    default: return reinterpret_cast<void *>(stream_ref_kernel<Reads, V, NtLoad, 3>);
    }
}

template <int Reads, int V>
void *pick_load(int policy)
{
    return policy & 1 ? pick_store<Reads, V, true>(policy >> 1) : pick_store<Reads, V, false>(policy >> 1);
}

template <int Reads>
void *pick_vpl(int vpl, int policy)
{
    switch (vpl) {
    case 1: return pick_load<Reads, 1>(policy);
    case 2: return pick_load<Reads, 2>(policy);
    case 4: return pick_load<Reads, 4>(policy);
    default: return pick_load<Reads, 8>(policy);
    }
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int
rgg_stream_ref(const void *a, const void *b, void *out, int64_t n_vec, int block_size, int vpl,
               int grid, int policy, int lds, hipStream_t stream)
{
    // Stores address the output through a buffer resource with 32-bit byte
    // offsets, so n_vec stays below 2^27 vectors (2 GiB).
    if (n_vec <= 0 || n_vec >= ((int64_t)1 << 27) || (b && !a) || !out ||
        ((uintptr_t)a | (uintptr_t)b | (uintptr_t)out) & 15 || block_size < 64 ||
        block_size > 1024 || block_size % 64 || (vpl != 1 && vpl != 2 && vpl != 4 && vpl != 8) ||
        grid < 0 || policy < 0 || policy > 7 || lds < 0 || lds > 65536)
        return 2;
    const int64_t chunk = (int64_t)block_size * vpl;
    const int64_t chunks = (n_vec + chunk - 1) / chunk;
    const dim3 g((uint32_t)(grid == 0 || grid > chunks ? chunks : grid)), blk(block_size);
    const int reads = b ? 2 : (a ? 1 : 0);
    void *k = reads == 2 ? pick_vpl<2>(vpl, policy)
                         : (reads == 1 ? pick_vpl<1>(vpl, policy) : pick_vpl<0>(vpl, policy));
    const v4u *va = static_cast<const v4u *>(a), *vb = static_cast<const v4u *>(b);
    v4u *vo = static_cast<v4u *>(out);
    uint32_t n = (uint32_t)n_vec;
    void *args[] = {&va, &vb, &vo, &n};
    hipError_t e = hipLaunchKernel(k, g, blk, args, (size_t)lds, stream);
    if (e == hipSuccess)
        e = hipGetLastError();
    return e == hipSuccess ? 0 : 6;
}

// Streaming reference for measurement: how long a plain stream that reads
// and writes the same bytes as a kernel takes on this GPU, with the same
// access discipline (one 16-byte vector per lane, nontemporal loads and
// stores, whole 128-byte lines per wave instruction).  bench.py reports it
// beside each kernel as the practical ceiling for that traffic.  It is not
// part of the library's C ABI and computes nothing of the method.
//
//   int rgg_stream_ref(const void *a, const void *b, void *out, int64_t n_vec,
//                      int block, hipStream_t stream);
//
// a == NULL, b == NULL: out[i] = i    (write only)
// b == NULL:            out[i] = a[i]            (1 read : 1 write)
// b != NULL:            out[i] = a[i] ^ b[i]     (2 reads : 1 write)
// for i < n_vec 16-byte vectors, in workgroups of `block` (64..1024, a
// multiple of 64) threads; all pointers device memory, 16-byte aligned.
// Returns 0, 2 for bad sizes or pointers, 6 for a launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int Reads>
__global__ __launch_bounds__(1024) void stream_ref_kernel(const v4u *a, const v4u *b, v4u *out,
                                                          uint32_t n)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    v4u x = v4u{i, i, i, i};
    if (Reads >= 1)
        x = __builtin_nontemporal_load(a + i);
    if (Reads == 2)
        x ^= __builtin_nontemporal_load(b + i);
    __builtin_nontemporal_store(x, out + i);
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int
rgg_stream_ref(const void *a, const void *b, void *out, int64_t n_vec, int block_size,
               hipStream_t stream)
{
    if (n_vec <= 0 || n_vec >= ((int64_t)1 << 31) || (b && !a) || !out ||
        ((uintptr_t)a | (uintptr_t)b | (uintptr_t)out) & 15 || block_size < 64 ||
        block_size > 1024 || block_size % 64)
        return 2;
    const dim3 grid((uint32_t)((n_vec + block_size - 1) / block_size)), block(block_size);
    const v4u *va = static_cast<const v4u *>(a), *vb = static_cast<const v4u *>(b);
    v4u *vo = static_cast<v4u *>(out);
    if (b)
        hipLaunchKernelGGL(stream_ref_kernel<2>, grid, block, 0, stream, va, vb, vo,
                           (uint32_t)n_vec);
    else if (a)
        hipLaunchKernelGGL(stream_ref_kernel<1>, grid, block, 0, stream, va, vb, vo,
                           (uint32_t)n_vec);
    else
        hipLaunchKernelGGL(stream_ref_kernel<0>, grid, block, 0, stream, va, vb, vo,
                           (uint32_t)n_vec);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

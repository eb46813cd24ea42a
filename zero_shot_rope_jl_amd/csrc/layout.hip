// Channel reorder for models whose RoPE pairs adjacent channels.
//
// The kernels here pair channel i with channel i + D/2 (rotate-half).  A
// model whose RoPE rotates the pairs (2i, 2i + 1) computes the same scores
// once q and k both have their channels permuted so that pair i lands on
// (i, i + D/2): a dot product does not change under a common permutation of
// its operands' channels, and each pair's rotation moves with it.  v and the
// output are not permuted.
//
// One thread per 8 output channels of a row (4 from each half): it reads 8
// consecutive input channels (4 pairs) and writes 4 + 4.  HBM-bound: one
// read and one write of the tensor.
#include "internal.h"

namespace jl {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void interleaved_to_half_kernel(const T* __restrict__ x, T* __restrict__ out,
                                                                   int64_t n_items, int D) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_items) return;
    const int per_row = D / 8;
    const int64_t r = t / per_row;
    const int c = (int)(t % per_row);          // pairs 4c .. 4c + 3
    const T* src = x + r * D + 8 * c;
    T* lo = out + r * D + 4 * c;
    T* hi = lo + D / 2;
    T v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = v[2 * e];
        hi[e] = v[2 * e + 1];
    }
}

}  // namespace

hipError_t launch_interleaved_to_half(const void* x, void* out, int elem_bytes, int64_t n_rows, int D,
                                      hipStream_t stream) {
    const int64_t n_items = n_rows * (D / 8);
    if (n_items == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n_items + 255) / 256);
    if (elem_bytes == 2)
        hipLaunchKernelGGL((interleaved_to_half_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), static_cast<uint16_t*>(out), n_items, D);
    else
        hipLaunchKernelGGL((interleaved_to_half_kernel<uint32_t>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const uint32_t*>(x), static_cast<uint32_t*>(out), n_items, D);
    return hipGetLastError();
}

}  // namespace jl

// Inclusion-exclusion merge of three attention passes (Jet-Long §3.3,
// Eq. 6), the last step of the unfused prefill:
//     O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C)
// where pass A is the stored view over each row's window, B the corrected
// view over all causal keys and C the corrected view over the window; O_X is
// a pass's normalised output and W_X = exp(LSE_X) its softmax denominator.
// The weights are shifted by max(LSE_A, LSE_B) before exponentiation (C's
// keys are a subset of B's in the same view, so LSE_C <= LSE_B).
#include <math.h>

#include "internal.h"

namespace jl {

namespace {

// One thread per 4 output dimensions of one (batch, row, head).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void ie_merge_kernel(MergeParams p) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = p.D / 4;
    const int64_t n = p.B * p.Lq * p.Hq * per_row;
    if (t >= n) return;
    const int64_t d4 = t % per_row;
    const int64_t rh = t / per_row;          // (b, row, head) in output order
    const int64_t h = rh % p.Hq;
    const int64_t row = (rh / p.Hq) % p.Lq;
    const int64_t b = rh / (p.Hq * p.Lq);
    const int64_t li = (b * p.Hq + h) * p.Lq + row;
    const float la = p.lse_a[li], lb = p.lse_b[li], lc = p.lse_c[li];
    const float m = fmaxf(la, lb);
    const float wa = expf(la - m), wb = expf(lb - m), wc = expf(lc - m);
    const float W = wa + wb - wc;
    const float inv = 1.f / W;
    const int64_t o = rh * p.D + 4 * d4;
    const float4 A = *reinterpret_cast<const float4*>(p.o_a + o);
    const float4 Bv = *reinterpret_cast<const float4*>(p.o_b + o);
    const float4 C = *reinterpret_cast<const float4*>(p.o_c + o);
    const float r0 = (wa * A.x + wb * Bv.x - wc * C.x) * inv;
    const float r1 = (wa * A.y + wb * Bv.y - wc * C.y) * inv;
    const float r2 = (wa * A.z + wb * Bv.z - wc * C.z) * inv;
    const float r3 = (wa * A.w + wb * Bv.w - wc * C.w) * inv;
    if constexpr (OUT_BF16) {
        bf16x4 w = {(__bf16)r0, (__bf16)r1, (__bf16)r2, (__bf16)r3};
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + o) = w;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o) = make_float4(r0, r1, r2, r3);
    }
    if (d4 == 0 && p.lse) p.lse[li] = m + logf(W);
}

}  // namespace

hipError_t launch_ie_merge(const MergeParams& p, int out_dtype, hipStream_t stream) {
    const int64_t n = p.B * p.Lq * p.Hq * (p.D / 4);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (out_dtype == 1) hipLaunchKernelGGL((ie_merge_kernel<true>), dim3(blocks), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((ie_merge_kernel<false>), dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace jl

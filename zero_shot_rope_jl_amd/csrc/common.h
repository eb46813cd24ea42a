// Shared device-side definitions for the gfx950 Jet-Long kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kTableMagic = 0x324C544Au;  // "JTL2"
constexpr int kTableHeaderBytes = 64;

// Device/host view of the correction-angle table header.  The header is
// followed by rows TF[n][i] = (cos, sin)(n * theta_i), n < n_cover, i < D/2,
// each angle formed in float64 and rounded once to fp32.
struct TableHeader {
    uint32_t magic;
    int32_t head_dim;
    int64_t n_cover;     // covers offsets n < n_cover
    double rope_base;
    int64_t pad[5];
};
static_assert(sizeof(TableHeader) == kTableHeaderBytes, "header size");

__host__ __device__ inline size_t table_bytes_for(int64_t n_cover, int head_dim) {
    return (size_t)kTableHeaderBytes + (size_t)n_cover * (size_t)(head_dim / 2) * 8u;
}

// Rotate the pair (x, y) by the angle -n*theta (cs = cos, sn = sin of +n*theta).
// The correction offset f(p) - p is -n with n = p - floor(p/G) >= 0.
__device__ inline void rotate_back(float& x, float& y, float2 cs) {
    const float nx = x * cs.x + y * cs.y;
    const float ny = y * cs.x - x * cs.y;
    x = nx;
    y = ny;
}

__device__ inline float bf16_to_f32(__bf16 v) { return (float)v; }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_max_xor32(float x) {
    return fmaxf(x, __shfl_xor(x, 32));
}

// Transposing LDS read: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte rows addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.
__device__ inline bf16x4 lds_read_tr16(const __bf16* p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer resource, 32-bit elements

// Buffer resource over [base, base + bytes): loads beyond `bytes` return 0.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// 16-byte buffer -> LDS copy per lane; lane l writes bytes [16l, 16l + 16)
// after the wave-uniform LDS base.
__device__ inline void buffer_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_base), 16, voff, soff,
                                             0, 0);
}

}  // namespace jl

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

constexpr uint32_t kTableMagic = 0x324C544Au;    // "JTL2": offset table
constexpr uint32_t kTableMagicFI = 0x3146544Au;  // "JTF1": interpolation table
constexpr int kTableHeaderBytes = 64;

// Device/host view of the correction-angle table header.  The table holds
// (cos, sin)(n * phi_i) for every n < n_cover and i < D/2 in two levels: the
// header is followed by kTableLoRows rows TL[l] = (cos, sin)(l * phi_i) and
// then ceil(n_cover / kTableLoRows) rows TH[h] = (cos, sin)(kTableLoRows * h
// * phi_i), each angle formed in float64 and rounded once to fp32; the entry
// for n is the complex product TL[n mod 1024] * TH[n / 1024] (table_cs), a
// few fp32 ulp from the rounded exact value.  So the table grows by one
// 512-byte row (D = 128) per 1024 offsets: 0.9 MB covers the offsets of a
// 1M-token call at G = 4.  Offset tables (the aliasing correction) have
// phi_i = theta_i and are indexed by the offset n = p - floor(p/G);
// interpolation tables have phi_i = theta_i - theta'_i (the frequency-
// interpolation remote view) and are indexed by the position p.
struct TableHeader {
    uint32_t magic;
    int32_t head_dim;
    int64_t n_cover;     // covers rows n < n_cover
    double rope_base;
    // interpolation tables only, zero in offset tables: the length and
    // pretrained window that fix s = L / w_pretrained, and the ramp bounds
    int64_t fi_L;
    int64_t fi_w_pretrained;
    double fi_alpha;
    double fi_beta;
    int64_t pad;
};
static_assert(sizeof(TableHeader) == kTableHeaderBytes, "header size");

// What a kernel expects of the table it is given (compared with the header
// before any row is read).
struct TableKey {
    uint32_t magic;
    int64_t fi_L;
    int64_t fi_w_pretrained;
    double fi_alpha;
    double fi_beta;
};

// The offsets a call over positions 0..L-1 reads: n(p) = p - floor(p/G)
// grows with p, so every n is below n(L-1) + 1.  (The interpolation view runs
// with G = max(2, L), where n(p) = p.)
__host__ __device__ inline int64_t table_need(int64_t L, int64_t G) { return (L - 1) - (L - 1) / G + 1; }

__host__ __device__ inline bool table_matches(const TableHeader* th, const TableKey& key, int D, double base,
                                              int64_t n_need) {
    return th->magic == key.magic && th->head_dim == D && th->rope_base == base && th->n_cover >= n_need &&
           th->fi_L == key.fi_L && th->fi_w_pretrained == key.fi_w_pretrained && th->fi_alpha == key.fi_alpha &&
           th->fi_beta == key.fi_beta;
}

// phi_i = theta_i - theta'_i of the frequency-interpolation remote view:
// theta'_i = (1 - gamma_i) theta_i / s + gamma_i theta_i with
// s = max(1, L / w_pretrained) and gamma_i a linear ramp from 0 (at alpha)
// to 1 (at beta) over r_i = w_pretrained theta_i / (2 pi), the turns of
// pair i over the pretrained window.  So phi_i = theta_i (1 - gamma_i)(1 - 1/s).
__host__ __device__ inline double fi_phi(double base, int D, int64_t L, int64_t w_pretrained, double alpha,
                                         double beta, int i) {
    const double theta = pow(base, -(2.0 * (double)i) / (double)D);
    const double s = (double)L > (double)w_pretrained ? (double)L / (double)w_pretrained : 1.0;
    const double r = (double)w_pretrained * theta / 6.283185307179586476925286766559;
    double g = (r - alpha) / (beta - alpha);
    g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
    return theta * (1.0 - g) * (1.0 - 1.0 / s);
}

constexpr int kTableLoShift = 10;
constexpr int64_t kTableLoRows = int64_t(1) << kTableLoShift;

__host__ __device__ inline int64_t table_rows_for(int64_t n_cover) {
    return kTableLoRows + (n_cover + kTableLoRows - 1) / kTableLoRows;
}

__host__ __device__ inline size_t table_bytes_for(int64_t n_cover, int head_dim) {
    return (size_t)kTableHeaderBytes + (size_t)table_rows_for(n_cover) * (size_t)(head_dim / 2) * 8u;
}

// (cos, sin)(n * phi_i) from the two levels of the table rows TF (after the
// header): TL[n mod 1024] * TH[n / 1024] as complex numbers.
__device__ inline float2 table_cs(const float2* __restrict__ TF, int half, int64_t n, int i) {
    const float2 lo = TF[(n & (kTableLoRows - 1)) * half + i];
    const float2 hi = TF[(kTableLoRows + (n >> kTableLoShift)) * half + i];
    return make_float2(lo.x * hi.x - lo.y * hi.y, lo.x * hi.y + lo.y * hi.x);
}

// Pairs i and i + 1 of row n (i even): (cos_i, sin_i, cos_i+1, sin_i+1).
__device__ inline float4 table_cs2(const float2* __restrict__ TF, int half, int64_t n, int i) {
    const float4 lo = *reinterpret_cast<const float4*>(TF + (n & (kTableLoRows - 1)) * half + i);
    const float4 hi = *reinterpret_cast<const float4*>(TF + (kTableLoRows + (n >> kTableLoShift)) * half + i);
    return make_float4(lo.x * hi.x - lo.y * hi.y, lo.x * hi.y + lo.y * hi.x, lo.z * hi.z - lo.w * hi.w,
                       lo.z * hi.w + lo.w * hi.z);
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

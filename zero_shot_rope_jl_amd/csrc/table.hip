// Correction-angle table for the on-the-fly RoPE correction (Jet-Long §3.2,
// Eq. 5): (cos, sin)(n * theta_i) for every offset n = p - floor(p/G) below
// the coverage, held in two levels (rows TL[l] for l < 1024 and TH[h] for the
// multiples 1024 h; see TableHeader).  Angles are formed in float64 and
// rounded once to fp32; the table does not depend on G, so one table serves
// every G and every L whose offsets it covers.
#include <math.h>
#include <string.h>

#include "internal.h"

namespace jl {

// The multiple of the angle that table row r holds: r for the low level,
// 1024 (r - 1024) for the high level.
__host__ __device__ inline double row_multiple(int64_t r) {
    return r < kTableLoRows ? (double)r : (double)(kTableLoRows * (r - kTableLoRows));
}

__host__ __device__ inline float2 table_entry(double base, int D, int64_t r, int i) {
    const double theta = pow(base, -(2.0 * (double)i) / (double)D);
    const double a = row_multiple(r) * theta;
    return make_float2((float)cos(a), (float)sin(a));
}

__host__ __device__ inline TableHeader make_header(int64_t n_cover, int D, double base) {
    TableHeader h;
    memset(&h, 0, sizeof(h));
    h.magic = kTableMagic;
    h.head_dim = D;
    h.n_cover = n_cover;
    h.rope_base = base;
    return h;
}

__global__ void table_fill_kernel(char* table, int64_t n_cover, int D, double base) {
    const int half = D / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float2* ent = reinterpret_cast<float2*>(table + kTableHeaderBytes);
    if (idx < table_rows_for(n_cover) * half) ent[idx] = table_entry(base, D, idx / half, (int)(idx % half));
    if (idx == 0) {
        *reinterpret_cast<TableHeader*>(table) = make_header(n_cover, D, base);
    }
}

// Frequency-interpolation table for one (L, w_pretrained, alpha, beta):
// rows p < L of (cos, sin)(p * phi_i), the rotation that moves a stored
// RoPE(x, p) to the interpolated phase p * theta'_i (Jet-Long §4.7 ablation).
__host__ __device__ inline TableHeader make_fi_header(int64_t L, int D, double base, int64_t w_pre, double alpha,
                                                      double beta) {
    TableHeader h = make_header(L, D, base);
    h.magic = kTableMagicFI;
    h.fi_L = L;
    h.fi_w_pretrained = w_pre;
    h.fi_alpha = alpha;
    h.fi_beta = beta;
    return h;
}

__host__ __device__ inline float2 fi_entry(double phi, int64_t r) {
    const double a = row_multiple(r) * phi;
    return make_float2((float)cos(a), (float)sin(a));
}

__global__ void table_fill_fi_kernel(char* table, int64_t L, int D, double base, int64_t w_pre, double alpha,
                                     double beta) {
    const int half = D / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float2* ent = reinterpret_cast<float2*>(table + kTableHeaderBytes);
    if (idx < table_rows_for(L) * half) {
        const int i = (int)(idx % half);
        ent[idx] = fi_entry(fi_phi(base, D, L, w_pre, alpha, beta, i), idx / half);
    }
    if (idx == 0) *reinterpret_cast<TableHeader*>(table) = make_fi_header(L, D, base, w_pre, alpha, beta);
}

hipError_t launch_table_fill_fi(void* table, int64_t L, int head_dim, double rope_base, int64_t w_pretrained,
                                double alpha, double beta, hipStream_t stream) {
    const int64_t total = table_rows_for(L) * (head_dim / 2);
    const int threads = 256;
    const int blocks = (int)((total + threads - 1) / threads);
    hipLaunchKernelGGL(table_fill_fi_kernel, dim3(blocks), dim3(threads), 0, stream, static_cast<char*>(table), L,
                       head_dim, rope_base, w_pretrained, alpha, beta);
    return hipGetLastError();
}

void table_fill_fi_host(void* table, int64_t L, int head_dim, double rope_base, int64_t w_pretrained, double alpha,
                        double beta) {
    const int half = head_dim / 2;
    TableHeader h = make_fi_header(L, head_dim, rope_base, w_pretrained, alpha, beta);
    memcpy(table, &h, sizeof(h));
    float2* ent = reinterpret_cast<float2*>(static_cast<char*>(table) + kTableHeaderBytes);
    for (int i = 0; i < half; ++i) {
        const double phi = fi_phi(rope_base, head_dim, L, w_pretrained, alpha, beta, i);
        for (int64_t r = 0; r < table_rows_for(L); ++r) ent[r * half + i] = fi_entry(phi, r);
    }
}

hipError_t launch_table_fill(void* table, int64_t n_cover, int head_dim, double rope_base,
                             hipStream_t stream) {
    const int64_t total = table_rows_for(n_cover) * (head_dim / 2);
    const int threads = 256;
    const int blocks = (int)((total + threads - 1) / threads);
    hipLaunchKernelGGL(table_fill_kernel, dim3(blocks), dim3(threads), 0, stream,
                       static_cast<char*>(table), n_cover, head_dim, rope_base);
    return hipGetLastError();
}

void table_fill_host(void* table, int64_t n_cover, int head_dim, double rope_base) {
    const int half = head_dim / 2;
    TableHeader h = make_header(n_cover, head_dim, rope_base);
    memcpy(table, &h, sizeof(h));
    float2* ent = reinterpret_cast<float2*>(static_cast<char*>(table) + kTableHeaderBytes);
    for (int64_t r = 0; r < table_rows_for(n_cover); ++r)
        for (int i = 0; i < half; ++i) ent[r * half + i] = table_entry(rope_base, head_dim, r, i);
}

}  // namespace jl

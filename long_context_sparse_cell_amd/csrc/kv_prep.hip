// Key/value preparation for the bf16 path, done once per forward so that the
// window and readout kernels can copy their tiles straight into LDS:
//  - kt: RoPE-rotated keys R(j) k_j at their absolute positions, fp16, [H][Np][d]
//    (FreeSolo digest, core method and step 2: the window branch uses standard
//    rotate-half RoPE with base 10000, frequencies base^(-2m/d));
//  - vt: values as fp16, transposed per group of 16 tokens, [H][Np/16][d][16],
//    the A-operand layout of the O^T = V^T P^T products in both branches.
// Np = 64 ceil(N/64): both arrays are padded to whole 64-token tiles with zeros.
// fp16 holds bf16 values exactly inside fp16's range (|x| < 65504); the
// fp16-operand products of both branches assume inputs in that range.
//
// Angles at large positions are formed from a two-level table built in fp64:
// pos = 64a + b, (cos, sin)(pos theta) = rotation by (64a theta) composed with
// rotation by (b theta), so every table entry is a correctly rounded fp32 value
// and the composition adds only a few fp32 roundings.
#include <cmath>

#include "fsl_internal.h"

namespace fsl {

namespace {

union H8 {
    uint4 u;
    _Float16 f[8];
};

__device__ __forceinline__ void bf16x8_to_f32(const uint4 raw, float (&o)[8]) {
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        o[2 * t] = __uint_as_float(w4[t] << 16);
        o[2 * t + 1] = __uint_as_float(w4[t] & 0xFFFF0000u);
    }
}

}  // namespace

// rows [0, nhi): angle (64 a) theta_m; rows [nhi, nhi + 64): angle b theta_m
__global__ void rope_abs_kernel(float2 *__restrict__ tab, int nhi, KParams p) {
    const int half = p.d / 2;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)(nhi + kRopeSpan) * half) return;
    const int row = (int)(e / half), m = (int)(e % half);
    const double pos = row < nhi ? (double)row * kRopeSpan : (double)(row - nhi);
    const double theta = pow((double)p.rope_base, -2.0 * (double)m / (double)p.d);
    const double ang = pos * theta;
    tab[e] = make_float2((float)cos(ang), (float)sin(ang));
}

template <int D>
__global__ __launch_bounds__(256) void kv_prep_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                      uint16_t *__restrict__ kt, uint16_t *__restrict__ vt,
                                                      const float2 *__restrict__ rope, int nhi, KParams p) {
    constexpr int HALF = D / 2;
    constexpr int PG = HALF / 8;       // groups of 8 rotation pairs per row
    constexpr int TLD = kRopeSpan + 8; // transposed tile row stride
    __shared__ uint16_t s_t[D * TLD];  // fp16 bits, [dim][token]

    const int h = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * kRopeSpan;
    const int tid = threadIdx.x;
    const int64_t hN = (int64_t)h * p.N;
    const int64_t G = vt_groups(p);
    const int64_t hNp = (int64_t)h * kt_rows(p);

    // ---- rotated keys
    const float2 *hi = rope + (int64_t)blockIdx.x * HALF;
    for (int it = tid; it < kRopeSpan * PG; it += 256) {
        const int jl = it / PG, pg = it % PG;
        const int64_t j = j0 + jl;
        uint16_t *o = kt + (hNp + j) * D;
        if (j >= p.N) {
            *reinterpret_cast<uint4 *>(o + 8 * pg) = make_uint4(0u, 0u, 0u, 0u);
            *reinterpret_cast<uint4 *>(o + HALF + 8 * pg) = make_uint4(0u, 0u, 0u, 0u);
            continue;
        }
        const uint16_t *kr = k + (hN + j) * D;
        float a[8], b[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4 *>(kr + 8 * pg), a);
        bf16x8_to_f32(*reinterpret_cast<const uint4 *>(kr + HALF + 8 * pg), b);
        const float2 *lo = rope + (int64_t)(nhi + jl) * HALF;
        H8 ra, rb;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float2 th = hi[8 * pg + r], tl = lo[8 * pg + r];
            const float c = th.x * tl.x - th.y * tl.y;
            const float s = th.y * tl.x + th.x * tl.y;
            ra.f[r] = (_Float16)(a[r] * c - b[r] * s);
            rb.f[r] = (_Float16)(b[r] * c + a[r] * s);
        }
        *reinterpret_cast<uint4 *>(o + 8 * pg) = ra.u;
        *reinterpret_cast<uint4 *>(o + HALF + 8 * pg) = rb.u;
    }

    // ---- values: fp16, transposed through LDS (token pairs per 32-bit store)
    for (int it = tid; it < (kRopeSpan / 2) * (D / 8); it += 256) {
        const int jp = it % (kRopeSpan / 2), c8 = it / (kRopeSpan / 2);
        const int64_t j = j0 + 2 * jp;
        float e0[8], e1[8];
        if (j < p.N) bf16x8_to_f32(*reinterpret_cast<const uint4 *>(v + (hN + j) * D + 8 * c8), e0);
        else for (int r = 0; r < 8; ++r) e0[r] = 0.0f;
        if (j + 1 < p.N) bf16x8_to_f32(*reinterpret_cast<const uint4 *>(v + (hN + j + 1) * D + 8 * c8), e1);
        else for (int r = 0; r < 8; ++r) e1[r] = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            union { _Float16 f[2]; uint32_t u; } pr;
            pr.f[0] = (_Float16)e0[r];
            pr.f[1] = (_Float16)e1[r];
            *reinterpret_cast<uint32_t *>(&s_t[(8 * c8 + r) * TLD + 2 * jp]) = pr.u;
        }
    }
    __syncthreads();
    // [group][dim][16] rows of 32 bytes, two 16-byte pieces each; consecutive pieces
    // are consecutive in memory
    const int64_t g0 = j0 / 16;
    for (int pi = tid; pi < (kRopeSpan / 16) * D * 2; pi += 256) {
        const int grp = pi / (2 * D), rem = pi % (2 * D);
        const int dim = rem >> 1, hf = rem & 1;
        const uint4 val = *reinterpret_cast<const uint4 *>(&s_t[dim * TLD + 16 * grp + 8 * hf]);
        *reinterpret_cast<uint4 *>(vt + ((h * G + g0 + grp) * D + dim) * 16 + 8 * hf) = val;
    }
}

hipError_t launch_kv_prep(const void *k, const void *v, uint16_t *kt, uint16_t *vt, float2 *rope_abs,
                          const KParams &p, hipStream_t st) {
    const int nhi = rope_abs_rows_hi(p);
    const int64_t n = (int64_t)(nhi + kRopeSpan) * (p.d / 2);
    hipLaunchKernelGGL(rope_abs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, rope_abs, nhi, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)nhi, (unsigned)p.H);
    if (p.d == 64)
        hipLaunchKernelGGL((kv_prep_kernel<64>), grid, dim3(256), 0, st, (const uint16_t *)k, (const uint16_t *)v, kt,
                           vt, rope_abs, nhi, p);
    else
        hipLaunchKernelGGL((kv_prep_kernel<128>), grid, dim3(256), 0, st, (const uint16_t *)k, (const uint16_t *)v,
                           kt, vt, rope_abs, nhi, p);
    return hipGetLastError();
}

}  // namespace fsl

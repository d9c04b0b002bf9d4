// Key/value preparation for the bf16 path, done once per forward so that the
// window and readout kernels can copy their tiles straight into LDS:
//  - kt: RoPE-rotated keys R(j) k_j at their absolute positions, fp16, [H][Np][d]
//    (FreeSolo digest, core method and step 2: the window branch uses standard
//    rotate-half RoPE with base 10000, frequencies base^(-2m/d));
//  - vt: values as fp16, transposed per group of 32 tokens, [H][Np/32][d][32],
//    tokens inside a group in vt_pos order: the A-operand layout of the
//    O^T = V^T P^T products in both branches, one 16-byte piece per lane.
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
    constexpr int PG = HALF / 8;               // groups of 8 rotation pairs per row
    constexpr int KIT = kRopeSpan * PG / 256;  // key items per thread
    constexpr int VIT = kRopeSpan * D / 8 / 2 / 256;  // value items (token pair x 8 dims) per thread
    constexpr int TLD = kRopeSpan + 8;         // transposed tile row stride
    static_assert(KIT >= 1 && VIT >= 1, "tile work must cover every thread");
    __shared__ __attribute__((aligned(16))) uint16_t s_t[D * TLD];  // fp16 bits, [dim][token]

    const int h = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * kRopeSpan;
    const int tid = threadIdx.x;
    const int64_t hN = (int64_t)h * p.N;

    // ---- issue every global load of this thread first
    uint4 ka[KIT], kb[KIT], va[VIT], vb[VIT];
#pragma unroll
    for (int u = 0; u < KIT; ++u) {
        const int it = tid + 256 * u, jl = it / PG, pg = it % PG;
        const int64_t j = min(j0 + jl, p.N - 1);  // rows past the end are replaced by zeros below
        const uint16_t *kr = k + (hN + j) * D;
        ka[u] = *reinterpret_cast<const uint4 *>(kr + 8 * pg);
        kb[u] = *reinterpret_cast<const uint4 *>(kr + HALF + 8 * pg);
    }
#pragma unroll
    for (int u = 0; u < VIT; ++u) {
        const int it = tid + 256 * u, jp = it % (kRopeSpan / 2), c8 = it / (kRopeSpan / 2);
        const int64_t j = j0 + 2 * jp;
        va[u] = *reinterpret_cast<const uint4 *>(v + (hN + min(j, p.N - 1)) * D + 8 * c8);
        vb[u] = *reinterpret_cast<const uint4 *>(v + (hN + min(j + 1, p.N - 1)) * D + 8 * c8);
    }

    // ---- rotated keys
    const float2 *hi = rope + (int64_t)blockIdx.x * HALF;
#pragma unroll
    for (int u = 0; u < KIT; ++u) {
        const int it = tid + 256 * u, jl = it / PG, pg = it % PG;
        const int64_t j = j0 + jl;
        const bool ok = j < p.N;
        float a[8], b[8];
        bf16x8_to_f32(ka[u], a);
        bf16x8_to_f32(kb[u], b);
        const float2 *lo = rope + (int64_t)(nhi + jl) * HALF;
        H8 ra, rb;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float2 th = hi[8 * pg + r], tl = lo[8 * pg + r];
            const float c = th.x * tl.x - th.y * tl.y;
            const float s = th.y * tl.x + th.x * tl.y;
            ra.f[r] = ok ? (_Float16)(a[r] * c - b[r] * s) : (_Float16)0.0f;
            rb.f[r] = ok ? (_Float16)(b[r] * c + a[r] * s) : (_Float16)0.0f;
        }
        uint16_t *o = kt + h * kt_head_elems(p) + j * D;
        *reinterpret_cast<uint4 *>(o + 8 * pg) = ra.u;
        *reinterpret_cast<uint4 *>(o + HALF + 8 * pg) = rb.u;
    }

    // ---- values: fp16, transposed through LDS (token pairs per 32-bit store)
#pragma unroll
    for (int u = 0; u < VIT; ++u) {
        const int it = tid + 256 * u, jp = it % (kRopeSpan / 2), c8 = it / (kRopeSpan / 2);
        const int64_t j = j0 + 2 * jp;
        float e0[8], e1[8];
        bf16x8_to_f32(va[u], e0);
        bf16x8_to_f32(vb[u], e1);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            union { _Float16 f[2]; uint32_t u; } pr;
            pr.f[0] = j < p.N ? (_Float16)e0[r] : (_Float16)0.0f;
            pr.f[1] = j + 1 < p.N ? (_Float16)e1[r] : (_Float16)0.0f;
            *reinterpret_cast<uint32_t *>(&s_t[(8 * c8 + r) * TLD + 2 * jp]) = pr.u;
        }
    }
    __syncthreads();
    // rows of 32 tokens in vt_pos order: piece g of (group, dim) holds tokens
    // 4g..4g+3 and 16+4g..16+4g+3 of the group; consecutive pieces are consecutive
    // in memory
    constexpr int PIECES = (kRopeSpan / 32) * D * 4;
#pragma unroll
    for (int u = 0; u < PIECES / 256; ++u) {
        const int pi = tid + 256 * u;
        const int grp = pi / (4 * D), rem = pi % (4 * D);
        const int dim = rem >> 2, pg = rem & 3;
        const uint16_t *src = &s_t[dim * TLD + 32 * grp + 4 * pg];
        const uint2 lo = *reinterpret_cast<const uint2 *>(src);
        const uint2 hi2 = *reinterpret_cast<const uint2 *>(src + 16);
        *reinterpret_cast<uint4 *>(vt + h * vt_head_elems(p) + ((2 * (int64_t)blockIdx.x + grp) * D + dim) * 32 + 8 * pg) =
            make_uint4(lo.x, lo.y, hi2.x, hi2.y);
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

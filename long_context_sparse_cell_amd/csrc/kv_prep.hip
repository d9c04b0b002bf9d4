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
// fp16-operand products of both branches assume inputs in that range, and an
// element of k or v, or a rotated key, outside it (or not finite) sets
// FSL_STATUS_F16_RANGE in the status word (cleared by rope_abs_kernel, which
// runs first on the same stream).
//
// With kbar/amax given, the same pass also produces the cell statistics of the
// tile's complete cells (FreeSolo digest, core method and step 3: the mean key
// and the largest token-key norm of every cell), so k is read from memory once
// per forward: the raw key rows are kept in LDS, each coordinate's mean is an
// fp64 sum in token order and each row's squared norm an fp64 fma chain in
// coordinate order, the orders of cell_stats_kernel (bit-identical results).
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

// Range tests on packed 16-bit halves (two per dword), OR-ed into an accumulator whose
// bit 15 or 31 ends up set when some half's magnitude reaches the threshold: with the sign
// cleared a half lies in [0, 0x7FFF], and adding 0x8000 - T leaves it below 0x8000 exactly
// when it is below T (no carry crosses into the other half).
//   bf16 bits >= 0x4780: |x| >= 65536, the first bf16 value past fp16's largest 65504
//   (infinities and NaNs included);
//   fp16 bits >= 0x7C00: an fp16 infinity or NaN (a rotated key that overflowed).
__device__ __forceinline__ uint32_t range_bits(uint32_t w, uint32_t bias2) { return (w & 0x7FFF7FFFu) + bias2; }
__device__ __forceinline__ uint32_t range_bits4(const uint4 u, uint32_t bias2) {
    return range_bits(u.x, bias2) | range_bits(u.y, bias2) | range_bits(u.z, bias2) | range_bits(u.w, bias2);
}
constexpr uint32_t kBf16PastF16 = 0x38803880u;  // 0x8000 - 0x4780 in both halves
constexpr uint32_t kF16NonFinite = 0x04000400u; // 0x8000 - 0x7C00 in both halves

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
__global__ void rope_abs_kernel(float2 *__restrict__ tab, int nhi, uint32_t *__restrict__ status, KParams p) {
    const int half = p.d / 2;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e == 0) *status = 0u;
    if (e >= (int64_t)(nhi + kRopeSpan) * half) return;
    const int row = (int)(e / half), m = (int)(e % half);
    const double pos = row < nhi ? (double)row * kRopeSpan : (double)(row - nhi);
    const double theta = pow((double)p.rope_base, -2.0 * (double)m / (double)p.d);
    const double ang = pos * theta;
    tab[e] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_abs_table(float2 *tab, uint32_t *status, const KParams &p, hipStream_t st) {
    const int nhi = rope_abs_rows_hi(p);
    const int64_t n = (int64_t)(nhi + kRopeSpan) * (p.d / 2);
    hipLaunchKernelGGL(rope_abs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tab, nhi, status, p);
    return hipGetLastError();
}

template <int D, bool STATS>
__global__ __launch_bounds__(256) void kv_prep_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                      uint16_t *__restrict__ kt, uint16_t *__restrict__ vt,
                                                      const float2 *__restrict__ rope, int nhi, float *__restrict__ kbar,
                                                      float *__restrict__ amax, uint32_t *__restrict__ status,
                                                      KParams p) {
    constexpr int HALF = D / 2;
    constexpr int PG = HALF / 8;               // groups of 8 rotation pairs per row
    constexpr int KIT = kRopeSpan * PG / 256;  // key items per thread
    constexpr int VIT = kRopeSpan * D / 8 / 2 / 256;  // value items (token pair x 8 dims) per thread
    constexpr int TLD = kRopeSpan + 2;         // transposed tile row stride (4 TLD = 8 mod 64 dwords)
    static_assert(KIT >= 1 && VIT >= 1, "tile work must cover every thread");
    __shared__ __attribute__((aligned(16))) uint16_t s_t[D * TLD];  // fp16 bits, [dim][token]
    // raw key rows for the statistics: a row stride of D + 2 bf16 (an odd number of
    // dwords) keeps the row-norm threads, one row each, on distinct banks
    constexpr int KLD = D + 2;
    __shared__ __attribute__((aligned(16))) uint16_t s_kr[STATS ? kRopeSpan * KLD : 2];
    __shared__ double s_ss[STATS ? kRopeSpan : 1];

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
        const int it = tid + 256 * u, c8 = it % (D / 8), jp = it / (D / 8);
        const int64_t j = j0 + 2 * jp;
        va[u] = *reinterpret_cast<const uint4 *>(v + (hN + min(j, p.N - 1)) * D + 8 * c8);
        vb[u] = *reinterpret_cast<const uint4 *>(v + (hN + min(j + 1, p.N - 1)) * D + 8 * c8);
    }

    if constexpr (STATS) {
        // raw key rows into LDS (rows past the end hold the last row; they belong to no
        // complete cell)
#pragma unroll
        for (int u = 0; u < KIT; ++u) {
            const int it = tid + 256 * u, jl = it / PG, pg = it % PG;
            uint32_t *ra = reinterpret_cast<uint32_t *>(&s_kr[jl * KLD + 8 * pg]);
            uint32_t *rb = reinterpret_cast<uint32_t *>(&s_kr[jl * KLD + HALF + 8 * pg]);
            ra[0] = ka[u].x; ra[1] = ka[u].y; ra[2] = ka[u].z; ra[3] = ka[u].w;
            rb[0] = kb[u].x; rb[1] = kb[u].y; rb[2] = kb[u].z; rb[3] = kb[u].w;
        }
    }

    // ---- rotated keys
    uint32_t range_acc = 0u;  // bit 15 or 31 set: an fp16 operand would not hold one of this thread's values
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
        // rows past the end hold zeros here, and copies of the last row in ka / kb
        range_acc |= range_bits4(ra.u, kF16NonFinite) | range_bits4(rb.u, kF16NonFinite) |
                     range_bits4(ka[u], kBf16PastF16) | range_bits4(kb[u], kBf16PastF16);
        uint16_t *o = kt + h * kt_head_elems(p) + j * D;
        *reinterpret_cast<uint4 *>(o + 8 * pg) = ra.u;
        *reinterpret_cast<uint4 *>(o + HALF + 8 * pg) = rb.u;
    }

    // ---- values: fp16, transposed through LDS (token pairs per 32-bit store)
#pragma unroll
    for (int u = 0; u < VIT; ++u) {
        const int it = tid + 256 * u, c8 = it % (D / 8), jp = it / (D / 8);
        const int64_t j = j0 + 2 * jp;
        float e0[8], e1[8];
        bf16x8_to_f32(va[u], e0);
        bf16x8_to_f32(vb[u], e1);
        range_acc |= range_bits4(va[u], kBf16PastF16) | range_bits4(vb[u], kBf16PastF16);  // past the end: row N-1
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            union { _Float16 f[2]; uint32_t u; } pr;
            pr.f[0] = j < p.N ? (_Float16)e0[r] : (_Float16)0.0f;
            pr.f[1] = j + 1 < p.N ? (_Float16)e1[r] : (_Float16)0.0f;
            *reinterpret_cast<uint32_t *>(&s_t[(8 * c8 + r) * TLD + 2 * jp]) = pr.u;
        }
    }
    if (__ballot((range_acc & 0x80008000u) != 0u) != 0ull && (tid & 63) == 0) atomicOr(status, FSL_STATUS_F16_RANGE);
    __syncthreads();
    if constexpr (STATS) {
        // cell statistics of the tile's complete cells (cells of s tokens, s | 64)
        const int s = p.s;
        const int cpt = kRopeSpan / s;
        const int64_t c0 = (int64_t)blockIdx.x * cpt;
        for (int idx = tid; idx < cpt * D; idx += 256) {
            const int cl = idx / D, x = idx % D;
            if (c0 + cl >= p.C) continue;
            double acc = 0.0;
            for (int j = 0; j < s; ++j) acc += (double)bf16_to_f32(s_kr[(cl * s + j) * KLD + x]);
            kbar[((int64_t)h * p.C + c0 + cl) * D + x] = (float)(acc / (double)s);
        }
        if (tid < kRopeSpan) {
            double acc = 0.0;
            const uint32_t *row = reinterpret_cast<const uint32_t *>(&s_kr[tid * KLD]);
#pragma unroll 8
            for (int x2 = 0; x2 < D / 2; ++x2) {
                const uint32_t w = row[x2];
                const double e0 = (double)__uint_as_float(w << 16), e1 = (double)__uint_as_float(w & 0xFFFF0000u);
                acc = __fma_rn(e0, e0, acc);
                acc = __fma_rn(e1, e1, acc);
            }
            s_ss[tid] = acc;
        }
    }
    // rows of 32 tokens in vt_pos order: piece g of (group, dim) holds tokens
    // 4g..4g+3 and 16+4g..16+4g+3 of the group; consecutive pieces are consecutive
    // in memory
    constexpr int PIECES = (kRopeSpan / 32) * D * 4;
#pragma unroll
    for (int u = 0; u < PIECES / 256; ++u) {
        const int pi = tid + 256 * u;
        const int grp = pi / (4 * D), rem = pi % (4 * D);
        const int dim = rem >> 2, pg = rem & 3;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(&s_t[dim * TLD + 32 * grp + 4 * pg]);
        *reinterpret_cast<uint4 *>(vt + h * vt_head_elems(p) + ((2 * (int64_t)blockIdx.x + grp) * D + dim) * 32 + 8 * pg) =
            make_uint4(src[0], src[1], src[8], src[9]);
    }
    if constexpr (STATS) {
        __syncthreads();
        const int s = p.s;
        const int cpt = kRopeSpan / s;
        const int64_t c = (int64_t)blockIdx.x * cpt + tid;
        if (tid < cpt && c < p.C) {
            double best = 0.0;
            for (int j = 0; j < s; ++j) {
                const double vv = s_ss[tid * s + j];
                if (vv > best) best = vv;
            }
            amax[(int64_t)h * p.C + c] = (float)__dsqrt_rn(best);
        }
    }
}

hipError_t launch_kv_prep(const void *k, const void *v, uint16_t *kt, uint16_t *vt, float2 *rope_abs, float *kbar,
                          float *amax, uint32_t *status, const KParams &p, hipStream_t st) {
    const int nhi = rope_abs_rows_hi(p);
    const int64_t n = (int64_t)(nhi + kRopeSpan) * (p.d / 2);
    hipLaunchKernelGGL(rope_abs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, rope_abs, nhi, status,
                       p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)nhi, (unsigned)p.H);
    const bool stats = kbar && amax;
#define FSL_KVP(DD, SS)                                                                                            \
    hipLaunchKernelGGL((kv_prep_kernel<DD, SS>), grid, dim3(256), 0, st, (const uint16_t *)k, (const uint16_t *)v, kt, \
                       vt, rope_abs, nhi, kbar, amax, status, p)
    if (p.d == 64) {
        if (stats) FSL_KVP(64, true); else FSL_KVP(64, false);
    } else {
        if (stats) FSL_KVP(128, true); else FSL_KVP(128, false);
    }
#undef FSL_KVP
    return hipGetLastError();
}

}  // namespace fsl

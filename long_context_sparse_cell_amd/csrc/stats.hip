// Cell statistics: mean key and largest key norm of every complete cell
// (FreeSolo digest, core method and step 3; ai.info summary, methodology).
//
// One workgroup covers cpb <= 256/d cells (at most 256 (cell, coordinate)
// pairs; cpb is halved until the tile fits in 48 KiB of LDS). The cells'
// s*256/d rows arrive with coalesced 16-byte loads into LDS as float; then
//  - thread (cell, x) sums the column in fp64 in token order -> kbar;
//  - thread (row) runs the fp64 fma chain of its squared norm in coordinate
//    order, and one thread per cell takes the max -> amax.
// The fixed orders make the float32 results bit-identical to a sequential
// fp64 evaluation. The kernel is a single pass over k: HBM-bound.
#include "fsl_internal.h"

namespace fsl {

template <typename T, int D>
__global__ __launch_bounds__(256) void cell_stats_kernel(const T *__restrict__ k, float *__restrict__ kbar,
                                                         float *__restrict__ amax, KParams p, int cpb) {
    constexpr int LD = D + 1;
    constexpr int VEC = 16 / sizeof(T);
    extern __shared__ float tile[];  // [cpb*s][D+1]
    __shared__ double ss[256];

    const int s = p.s;
    const int h = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * cpb;
    const int ncell = (int)min((int64_t)cpb, p.C - c0);
    const int nrows = ncell * s;
    const T *src = k + ((int64_t)h * p.N + c0 * s) * D;

    // a tile holds at most 8192 elements (the launcher checks cpb * s * D <= 8192), so at
    // most 8192 / VEC 16-byte vectors: a fixed number per thread, all issued before any
    // is stored
    constexpr int VPT = 8192 / VEC / 256;
    const int nvec = nrows * (D / VEC);
    uint4 raw[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        // vectors past the tile read its last row again (every load is issued, so the
        // waits below cover them all at once) and are not stored
        const int e = min((int)threadIdx.x + 256 * u, nvec - 1);
        const int r = e / (D / VEC), x = (e % (D / VEC)) * VEC;
        raw[u] = *reinterpret_cast<const uint4 *>(src + (int64_t)r * D + x);
    }
    // consume every loaded register here, so that no load is moved into the guarded
    // stores below (and waited for one at a time)
#pragma unroll
    for (int u = 0; u < VPT; ++u) asm volatile("" ::"v"(raw[u].x), "v"(raw[u].y), "v"(raw[u].z), "v"(raw[u].w));
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int e = (int)threadIdx.x + 256 * u;
        if (e >= nvec) continue;
        const int r = e / (D / VEC), x = (e % (D / VEC)) * VEC;
        if constexpr (sizeof(T) == 2) {
            const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                tile[r * LD + x + 2 * t] = __uint_as_float(w4[t] << 16);
                tile[r * LD + x + 2 * t + 1] = __uint_as_float(w4[t] & 0xFFFF0000u);
            }
        } else {
            tile[r * LD + x + 0] = __uint_as_float(raw[u].x);
            tile[r * LD + x + 1] = __uint_as_float(raw[u].y);
            tile[r * LD + x + 2] = __uint_as_float(raw[u].z);
            tile[r * LD + x + 3] = __uint_as_float(raw[u].w);
        }
    }
    __syncthreads();

    {
        const int cl = threadIdx.x / D, x = threadIdx.x % D;
        if (cl < ncell) {
            double acc = 0.0;
            for (int j = 0; j < s; ++j) acc += (double)tile[(cl * s + j) * LD + x];
            kbar[((int64_t)h * p.C + c0 + cl) * D + x] = (float)(acc / (double)s);
        }
    }
    for (int r = threadIdx.x; r < nrows; r += 256) {
        double acc = 0.0;
#pragma unroll 8
        for (int x = 0; x < D; ++x) {
            const double e = (double)tile[r * LD + x];
            acc = __fma_rn(e, e, acc);
        }
        ss[r] = acc;
    }
    __syncthreads();
    if (threadIdx.x < ncell) {
        double best = 0.0;
        for (int j = 0; j < s; ++j) {
            const double v = ss[threadIdx.x * s + j];
            if (v > best) best = v;
        }
        amax[(int64_t)h * p.C + c0 + threadIdx.x] = (float)__dsqrt_rn(best);
    }
}

template <typename T, int D>
static hipError_t launch_stats_t(const void *k, float *kbar, float *amax, const KParams &p, hipStream_t st) {
    int cpb = 256 / D;
    while (cpb > 1 && (size_t)cpb * p.s * (D + 1) * sizeof(float) > 48 * 1024) cpb /= 2;
    if ((size_t)cpb * p.s * D > 8192) return hipErrorInvalidValue;  // the kernel's per-thread load count
    dim3 grid((unsigned)((p.C + cpb - 1) / cpb), (unsigned)p.H);
    size_t lds = (size_t)cpb * p.s * (D + 1) * sizeof(float);
    hipLaunchKernelGGL((cell_stats_kernel<T, D>), grid, dim3(256), lds, st, (const T *)k, kbar, amax, p, cpb);
    return hipGetLastError();
}

hipError_t launch_cell_stats(const void *k, float *kbar, float *amax, const KParams &p, hipStream_t st) {
    if (p.C == 0) return hipSuccess;
    if (p.dtype == FSL_BF16)
        return p.d == 64 ? launch_stats_t<uint16_t, 64>(k, kbar, amax, p, st)
                         : launch_stats_t<uint16_t, 128>(k, kbar, amax, p, st);
    return p.d == 64 ? launch_stats_t<float, 64>(k, kbar, amax, p, st)
                     : launch_stats_t<float, 128>(k, kbar, amax, p, st);
}

}  // namespace fsl

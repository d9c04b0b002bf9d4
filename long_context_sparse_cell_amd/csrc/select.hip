// Cell scoring and per-query top-K (FreeSolo digest, core method and step 5:
// content match plus a norm-weighted erf relative-position bias, K cells per
// query; digest, limits section: the erf factor of an available cell is at
// least erf(2); ai.info summary, methodology: the bias grows with distance and
// is scaled by the cell norm).
//
//   score(i, c) = fma(rho, q_i . kbar_c, (lambda_h * a_c) * g),
//   g = erf(sigma_h * (i - c*s) / (2*s)),
//
// all in fp64 from the float32 cell statistics, the dot product a
// left-to-right fma chain. Ranking is (score desc, index asc). Since
// erfc(6) < 2^-54, erf(x) rounds to exactly 1.0 for x >= 6 and the call is
// skipped there; with sigma_h = 4 every eligible cell is that far away.
//
// One workgroup per (query block, head); one thread per query. The pool ids
// and cell statistics are workgroup-uniform, so they come through scalar
// loads and each fma takes one of its operands from a scalar register.
#include <climits>

#include "fsl_internal.h"

namespace fsl {

template <typename T, int D>
__global__ __launch_bounds__(256) void select_kernel(const T *__restrict__ q, const float *__restrict__ kbar,
                                                     const float *__restrict__ amax, const int32_t *__restrict__ pool,
                                                     int32_t *__restrict__ sel, KParams p) {
    const int64_t b = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t i = b * p.B + tid;
    const bool active = tid < p.B && i < p.N;
    const int64_t nb = eligible_cells(p, b);
    const bool fs = p.P < 0;  // no pruning: every eligible cell, no pool table
    const int npool = fs ? (int)nb : (int)min((int64_t)p.PW, nb);
    const int32_t *bp = fs ? nullptr : pool + ((int64_t)h * p.nblk + b) * p.PW;

    float qf[D];
    const T *qi = q + ((int64_t)h * p.N + (active ? i : 0)) * D;
#pragma unroll
    for (int x = 0; x < D; ++x) qf[x] = to_f32<T>(qi[x]);

    const double sigma = (double)p.sigma[h], lam = (double)p.lambda[h], rho = (double)p.rho;
    const double two_s = 2.0 * (double)p.s;

    double bs[kMaxK];
    int bi[kMaxK];
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) { bs[r] = -INFINITY; bi[r] = INT_MAX; }

    for (int t = 0; t < npool; ++t) {
        const int c = fs ? t : bp[t];
        const float *kb = kbar + ((int64_t)h * p.C + c) * D;
        double content = 0.0;
#pragma unroll
        for (int x = 0; x < D; ++x) content = __fma_rn((double)qf[x], (double)kb[x], content);
        const double arg = __ddiv_rn(__dmul_rn(sigma, (double)(i - (int64_t)c * p.s)), two_s);
        const double g = arg >= 6.0 ? 1.0 : erf(arg);
        const double bias = __dmul_rn(__dmul_rn(lam, (double)amax[(int64_t)h * p.C + c]), g);
        double sc = __fma_rn(rho, content, bias);
        int ci = c;
        // carry the candidate down the sorted list, dropping the worst
#pragma unroll
        for (int r = 0; r < kMaxK; ++r) {
            if (r < p.K && better_d(sc, ci, bs[r], bi[r])) {
                double ts = bs[r]; int ti = bi[r];
                bs[r] = sc; bi[r] = ci;
                sc = ts; ci = ti;
            }
        }
    }
    if (!active) return;
    // ascending indices, -1 padding
#pragma unroll
    for (int x = 0; x < kMaxK; ++x)
#pragma unroll
        for (int y = 0; y + 1 < kMaxK - x; ++y)
            if (bi[y] > bi[y + 1]) { int t2 = bi[y]; bi[y] = bi[y + 1]; bi[y + 1] = t2; }
    int32_t *out = sel + ((int64_t)h * p.N + i) * p.K;
#pragma unroll
    for (int r = 0; r < kMaxK; ++r)
        if (r < p.K) out[r] = bi[r] == INT_MAX ? -1 : bi[r];
}

template <typename T, int D>
static hipError_t launch_select_t(const void *q, const float *kbar, const float *amax, const int32_t *pool,
                                  int32_t *sel, const KParams &p, hipStream_t st) {
    int threads = ((p.B + 63) / 64) * 64;
    hipLaunchKernelGGL((select_kernel<T, D>), dim3((unsigned)p.nblk, (unsigned)p.H), dim3(threads), 0, st,
                       (const T *)q, kbar, amax, pool, sel, p);
    return hipGetLastError();
}

hipError_t launch_select(const void *q, const float *kbar, const float *amax, const int32_t *pool, int32_t *sel,
                         const KParams &p, hipStream_t st) {
    if (p.nblk == 0) return hipSuccess;
    if (p.dtype == FSL_BF16)
        return p.d == 64 ? launch_select_t<uint16_t, 64>(q, kbar, amax, pool, sel, p, st)
                         : launch_select_t<uint16_t, 128>(q, kbar, amax, pool, sel, p, st);
    return p.d == 64 ? launch_select_t<float, 64>(q, kbar, amax, pool, sel, p, st)
                     : launch_select_t<float, 128>(q, kbar, amax, pool, sel, p, st);
}

}  // namespace fsl

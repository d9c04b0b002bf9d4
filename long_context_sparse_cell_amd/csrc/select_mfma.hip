// Cell scoring and top-K for bf16 inputs: an MFMA filter with a certified
// error bound, then exact fp64 re-scoring of the few cells the bound cannot
// separate (FreeSolo digest, core method and step 5: content match plus a
// norm-weighted erf relative-position bias, top K cells).
//
// The exact score of the oracle and of the fp64 kernel is
//   s = fma(rho, q.kbar_c, (lambda * a_c) * erf(sigma (i - c s) / (2 s)))
// with the dot product a left-to-right fp64 fma chain. Here:
//  1. content~ = q . (hi + lo) on v_mfma_f32_16x16x32_bf16, where hi and lo are
//     the bf16 head and tail of the float32 kbar_c (q is bf16, so every
//     product is exact in fp32). |kbar - hi - lo| <= 2^-18 |kbar| and the fp32
//     accumulation of 2d exact products adds at most (2d+1) 2^-24 of their
//     absolute sum, so
//        |content - content~| <= ||q|| ||kbar_c|| (2^-17 + (4d+8) 2^-24)
//     (Cauchy-Schwarz bounds the absolute sum). The fp32 bias and the final
//     fp32 additions get their own rounding terms; the total is doubled.
//  2. Per query, each of its 4 lanes keeps its two largest lower bounds
//     s~ - eps; theta is the K-th largest of those 8 values (they belong to 8
//     distinct cells, so theta is at most the K-th largest lower bound over
//     all cells). A cell whose upper bound s~ + eps is below theta is beaten
//     by K cells for sure; every other cell ("contender") is re-scored exactly
//     in fp64 and the K best contenders under (score desc, index asc) are the
//     exact top-K.
// When a query has no more than K contenders, they are its top-K set and no
// exact score is needed; near-ties (more than K contenders) are re-scored with
// q and kbar read from global memory. The bf16 split of the pool means is made
// once per work-group. One workgroup = up to 128 queries of one block, 8 waves
// x 16 queries, in an XCD-aware order.
#include <climits>

#include "fsl_internal.h"

namespace fsl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kSelQ = 128;
constexpr int kSelPool = 128;
constexpr int kSelK = 8;

union U16x8s {
    uint4 u;
    bf16x8 b;
    uint16_t h[8];
};

// carry (v, i) down a list sorted by (v desc, i asc), dropping the last entry.
// Written with selects rather than a conditional swap: the branchy form with
// double keys was compiled into wrong code (equal keys lost the index
// tie-break) by this toolchain at -O3, while this form is exact.
template <typename F>
__device__ __forceinline__ void list_insert(F (&lv)[kSelK], int (&li)[kSelK], F v, int i, int K) {
#pragma unroll
    for (int r = 0; r < kSelK; ++r) {
        const bool sw = r < K && (v > lv[r] || (v == lv[r] && i < li[r]));
        const F nv = sw ? lv[r] : v;
        const int ni = sw ? li[r] : i;
        lv[r] = sw ? v : lv[r];
        li[r] = sw ? i : li[r];
        v = nv;
        i = ni;
    }
}

template <typename F>
__device__ __forceinline__ void list_merge_xor(F (&lv)[kSelK], int (&li)[kSelK], int K, int mask) {
    F pv[kSelK];
    int pi[kSelK];
#pragma unroll
    for (int r = 0; r < kSelK; ++r) { pv[r] = __shfl_xor(lv[r], mask); pi[r] = __shfl_xor(li[r], mask); }
#pragma unroll
    for (int r = 0; r < kSelK; ++r)
        if (r < K) list_insert<F>(lv, li, pv[r], pi[r], K);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(512) void select_mfma_kernel(const uint16_t *__restrict__ q, const float *__restrict__ kbar,
                                                          const float *__restrict__ amax,
                                                          const int32_t *__restrict__ pool, int32_t *__restrict__ sel,
                                                          KParams p, int QW) {
    constexpr int HLD = D + 8;  // bf16 row stride of the split pool means (272 B for d = 128: conflict-free rows)
    extern __shared__ uint16_t s_dyn[];  // hi rows [ntile*16][HLD], then lo rows
    __shared__ int s_pool[kSelPool];
    __shared__ float s_kn[kSelPool];
    __shared__ float s_a[kSelPool];

    const int nqb = (int)((p.N + QW - 1) / QW);
    const int logical = xcd_remap((int)blockIdx.x, nqb * p.H);
    const int h = logical / nqb;
    const int64_t q0 = (int64_t)(logical % nqb) * QW;
    const int64_t b = q0 / p.B;
    const int nq = (int)min((int64_t)QW, p.N - q0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g = lane >> 4;
    const int K = p.K;
    const int npool = (int)min((int64_t)p.PW, eligible_cells(p, b));
    const int ntile = (npool + 15) / 16;
    const int64_t hN = (int64_t)h * p.N;
    const int64_t hC = (int64_t)h * p.C;
    uint16_t *s_hi = s_dyn;
    uint16_t *s_lo = s_dyn + ntile * 16 * HLD;

    for (int t = tid; t < npool; t += 512) {
        const int c = pool[((int64_t)h * p.nblk + b) * p.PW + t];
        s_pool[t] = c;
        s_a[t] = amax[hC + c];
    }
    __syncthreads();
    // pool cell means split once into bf16 head + tail (round to nearest even; rows
    // past the pool are zero), 4 floats per thread per step
    for (int e = tid; e < ntile * 16 * (D / 4); e += 512) {
        const int r = e / (D / 4), x = 4 * (e % (D / 4));
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < npool) f = *reinterpret_cast<const float4 *>(kbar + (hC + s_pool[r]) * D + x);
        const float fx[4] = {f.x, f.y, f.z, f.w};
        union { __bf16 b[4]; uint2 u; } hi4, lo4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const __bf16 hb = (__bf16)fx[t];
            hi4.b[t] = hb;
            lo4.b[t] = (__bf16)(fx[t] - (float)hb);
        }
        *reinterpret_cast<uint2 *>(&s_hi[r * HLD + x]) = hi4.u;
        *reinterpret_cast<uint2 *>(&s_lo[r * HLD + x]) = lo4.u;
    }
    // ||kbar_c||: 8 lanes per cell, D/8 elements each
    for (int e = tid; e < ((npool + 63) / 64) * 512; e += 512) {
        const int r = e >> 3, part = e & 7;
        float ss = 0.0f;
        if (r < npool) {
            const float *kr = kbar + (hC + s_pool[r]) * D + part * (D / 8);
#pragma unroll
            for (int x = 0; x < D / 8; x += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(kr + x);
                ss += f.x * f.x + f.y * f.y + f.z * f.z + f.w * f.w;
            }
        }
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        if (r < npool && part == 0) s_kn[r] = sqrtf(ss);
    }
    __syncthreads();

    const double sig = (double)p.sigma[h], lam = (double)p.lambda[h], rho = (double)p.rho;
    const float sigf = p.sigma[h], lamf = p.lambda[h], rhof = p.rho;
    const float epsc = 1.001f * (7.62939453125e-06f + (float)(4 * D + 8) * 5.9604644775390625e-08f);

    {  // 8 waves x 16 queries
        const int ql = 16 * wave + col;
        const bool qok = ql < nq;
        const int qr = qok ? ql : 0;
        const int64_t i = q0 + qr;
        U16x8s bq[D / 32];
        float qss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            bq[ks].u = *reinterpret_cast<const uint4 *>(q + (hN + i) * D + 32 * ks + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = bf16_to_f32(bq[ks].h[e]);
                qss += f * f;
            }
        }
        const float qn = sqrtf(colsum4(qss));  // the four lanes of a query hold all its d elements

        float lb1 = -INFINITY, lb2 = -INFINITY;  // this lane's two largest lower bounds
        // approximate scores, 4 cells of each 16-cell tile per lane (cells 16*ct + 4*g + e)
        float sapx[kSelPool / 16][4];
        float seps[kSelPool / 16][4];
#pragma unroll
        for (int ct = 0; ct < kSelPool / 16; ++ct) {
            if (ct >= ntile) break;
            const int rowc = 16 * ct + col;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                U16x8s hi, lo;
                hi.u = *reinterpret_cast<const uint4 *>(&s_hi[rowc * HLD + 32 * ks + 8 * g]);
                lo.u = *reinterpret_cast<const uint4 *>(&s_lo[rowc * HLD + 32 * ks + 8 * g]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi.b, bq[ks].b, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo.b, bq[ks].b, acc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pos = 16 * ct + 4 * g + e;
                sapx[ct][e] = -INFINITY;
                seps[ct][e] = 0.0f;
                if (pos < npool) {
                    const int c = s_pool[pos];
                    const float argf = sigf * (float)(i - (int64_t)c * p.s) / (2.0f * (float)p.s);
                    float gf = 1.0f;
                    if (argf < 6.0f) gf = erff(argf);
                    const float la = lamf * s_a[pos];
                    const float bf = la * gf;
                    const float rc = rhof * acc[e];
                    const float sv = rc + bf;
                    float ev = fabsf(rhof) * qn * s_kn[pos] * epsc + fabsf(la) * 2e-6f +
                               (fabsf(rc) + fabsf(bf)) * 2.384185791015625e-07f + 1e-30f;
                    ev *= 2.0f;
                    sapx[ct][e] = sv;
                    seps[ct][e] = ev;
                    const float lb = sv - ev;
                    lb2 = fmaxf(lb2, fminf(lb1, lb));
                    lb1 = fmaxf(lb1, lb);
                }
            }
        }
        float lv8[8];
        lv8[0] = lb1; lv8[1] = lb2;
        lv8[2] = __shfl_xor(lb1, 16); lv8[3] = __shfl_xor(lb2, 16);
        lv8[4] = __shfl_xor(lb1, 32); lv8[5] = __shfl_xor(lb2, 32);
        lv8[6] = __shfl_xor(lb1, 48); lv8[7] = __shfl_xor(lb2, 48);
        // sort descending (odd-even transposition, 8 rounds) and take the K-th
#pragma unroll
        for (int rnd = 0; rnd < 8; ++rnd)
#pragma unroll
            for (int a = rnd & 1; a + 1 < 8; a += 2) {
                const float hi2 = fmaxf(lv8[a], lv8[a + 1]), lo2 = fminf(lv8[a], lv8[a + 1]);
                lv8[a] = hi2; lv8[a + 1] = lo2;
            }
        float theta = -INFINITY;
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (r == K - 1) theta = lv8[r];

        // this lane's contenders as a bitmask over its (tile, e) slots
        uint32_t cmask = 0;
#pragma unroll
        for (int ct = 0; ct < kSelPool / 16; ++ct) {
            if (ct >= ntile) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pos = 16 * ct + 4 * g + e;
                if (pos < npool && sapx[ct][e] + seps[ct][e] >= theta) cmask |= 1u << (4 * ct + e);
            }
        }
        // At least min(K, pool) cells are contenders. With no more than K of them
        // the top-K set is certified without exact scores (the output lists the
        // cells by index); otherwise the contenders are re-scored exactly in fp64.
        const int ncont = (int)colsum4((float)__popc(cmask));
        const bool exact = ncont > K;
        double exv[kSelK];
        int exi[kSelK];
#pragma unroll
        for (int r = 0; r < kSelK; ++r) { exv[r] = -INFINITY; exi[r] = INT_MAX; }
        int maxn = __popc(cmask);
#pragma unroll
        for (int m2 = 32; m2 > 0; m2 >>= 1) maxn = max(maxn, __shfl_xor(maxn, m2));
        const uint16_t *qg = q + (hN + i) * D;
        for (int t = 0; t < maxn; ++t) {
            if (cmask) {
                const int slot = __ffs(cmask) - 1;
                cmask &= cmask - 1;
                const int pos = 16 * (slot >> 2) + 4 * g + (slot & 3);
                const int c = s_pool[pos];
                double v = 0.0;  // certified set: equal keys list the cells by index
                if (exact) {
                    const float *krow = kbar + (hC + c) * D;
                    double content = 0.0;
#pragma unroll 2
                    for (int x = 0; x < D; x += 8) {
                        const uint4 qv = *reinterpret_cast<const uint4 *>(qg + x);
                        const float4 k0 = *reinterpret_cast<const float4 *>(krow + x);
                        const float4 k1 = *reinterpret_cast<const float4 *>(krow + x + 4);
                        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                        const float kf[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float qf = __uint_as_float(e & 1 ? (qw[e >> 1] & 0xFFFF0000u) : (qw[e >> 1] << 16));
                            content = __fma_rn((double)qf, (double)kf[e], content);
                        }
                    }
                    const double arg =
                        __ddiv_rn(__dmul_rn(sig, (double)(i - (int64_t)c * p.s)), 2.0 * (double)p.s);
                    const double gg = arg >= 6.0 ? 1.0 : erf(arg);
                    const double bias = __dmul_rn(__dmul_rn(lam, (double)s_a[pos]), gg);
                    v = __fma_rn(rho, content, bias);
                }
                list_insert<double>(exv, exi, v, c, K);
            }
        }
        list_merge_xor<double>(exv, exi, K, 16);
        list_merge_xor<double>(exv, exi, K, 32);
        if (qok && g == 0) {
#pragma unroll
            for (int x = 0; x < kSelK; ++x)
#pragma unroll
                for (int y = 0; y + 1 < kSelK - x; ++y)
                    if (exi[y] > exi[y + 1]) { int t2 = exi[y]; exi[y] = exi[y + 1]; exi[y + 1] = t2; }
            int32_t *o = sel + (hN + i) * K;
#pragma unroll
            for (int r = 0; r < kSelK; ++r)
                if (r < K) o[r] = exi[r] == INT_MAX ? -1 : exi[r];
        }
    }
}

hipError_t launch_select_mfma(const void *q, const float *kbar, const float *amax, const int32_t *pool,
                              int32_t *sel, const KParams &p, hipStream_t st) {
    const int QW = p.B <= kSelQ ? p.B : p.B / 2;
    dim3 grid((unsigned)(((p.N + QW - 1) / QW) * p.H));
    const int rows = (p.PW + 15) / 16 * 16;
    const size_t lds = (size_t)(rows > 0 ? rows : 16) * (p.d + 8) * sizeof(uint16_t) * 2;
    if (p.d == 64)
        hipLaunchKernelGGL((select_mfma_kernel<64>), grid, dim3(512), lds, st, (const uint16_t *)q, kbar, amax, pool,
                           sel, p, QW);
    else
        hipLaunchKernelGGL((select_mfma_kernel<128>), grid, dim3(512), lds, st, (const uint16_t *)q, kbar, amax, pool,
                           sel, p, QW);
    return hipGetLastError();
}

}  // namespace fsl

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
//  2. Per query, each of its 4 lanes keeps its KL >= K largest lower bounds
//     s~ - eps and the lanes merge them, so theta is exactly the K-th largest
//     lower bound over all cells. A cell whose upper bound s~ + eps is below
//     theta is beaten by K cells for sure; every other cell is a contender, and
//     the K best contenders under (score desc, index asc) are the exact top-K.
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

}  // namespace

template <int D, int KL>
__global__ __launch_bounds__(512) void select_mfma_kernel(const uint16_t *__restrict__ q, const float *__restrict__ kbar,
                                                          const float *__restrict__ amax,
                                                          const int32_t *__restrict__ pool, int32_t *__restrict__ sel,
                                                          uint32_t *__restrict__ fix, KParams p, int QW) {
    constexpr int HLD = D + 8;  // bf16 row stride of the split pool means (272 B for d = 128: conflict-free rows)
    // hi rows [ntile*16][HLD], then lo rows; 16-byte aligned for the 16-byte operand
    // reads (after the static arrays below, whose size is not a multiple of 16)
    extern __shared__ __attribute__((aligned(16))) uint16_t s_dyn[];
    __shared__ int s_pool[kSelPool];
    // per pool cell: lambda a_c, A_c, B_c (the bound eps = ||q|| A_c + B_c, below) and c s (int bits)
    __shared__ float4 s_cf[kSelPool];
    __shared__ int s_nfix;  // near-tie queries of this work-group

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

    const float sigf = p.sigma[h], lamf = p.lambda[h], rhof = p.rho;
    const float epsc = 1.001f * (7.62939453125e-06f + (float)(4 * D + 8) * 5.9604644775390625e-08f);
    const float karg = sigf / (2.0f * (float)p.s);  // erf argument per token of distance

    // this wave's 16 queries, loaded first so that their latency overlaps the setup
    const int ql = 16 * wave + col;
    const bool qok = ql < nq;
    const int qr = qok ? ql : 0;
    const int64_t i = q0 + qr;
    U16x8s bq[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) bq[ks].u = *reinterpret_cast<const uint4 *>(q + (hN + i) * D + 32 * ks + 8 * g);

    // ---- setup: pool row r by 8 consecutive threads (D/8 floats each): its mean split
    // into bf16 head + tail (round to nearest even; rows past the pool are zero), its
    // norm, and the per-cell constants of the bound. Every global load of the setup is
    // issued before the first one is used: the pool indices, then the rows and norms.
    constexpr int RPP = 512 / 8;                  // rows per pass
    constexpr int NPASS = kSelPool / RPP;         // passes over the largest pool
    constexpr int FPT = D / 8;                    // floats per thread
    const int part = tid & 7;
    int crow[NPASS];
#pragma unroll
    for (int j = 0; j < NPASS; ++j) {
        const int r = RPP * j + (tid >> 3);
        crow[j] = r < npool ? pool[((int64_t)h * p.nblk + b) * p.PW + r] : -1;
    }
    float4 f[NPASS][FPT / 4];
    float am[NPASS];
#pragma unroll
    for (int j = 0; j < NPASS; ++j) {
        am[j] = 0.0f;
#pragma unroll
        for (int x = 0; x < FPT / 4; ++x) f[j][x] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (crow[j] >= 0) {
            const float *src = kbar + (hC + crow[j]) * D + FPT * part;
#pragma unroll
            for (int x = 0; x < FPT / 4; ++x) f[j][x] = *reinterpret_cast<const float4 *>(src + 4 * x);
            if (part == 0) am[j] = amax[hC + crow[j]];
        }
    }
    if (tid == 0) s_nfix = 0;
#pragma unroll
    for (int j = 0; j < NPASS; ++j) {
        const int r = RPP * j + (tid >> 3);
        if (r >= ntile * 16) continue;  // rows of the last tile past the pool are written as zeros
        float ss = 0.0f;
#pragma unroll
        for (int x = 0; x < FPT / 4; ++x) {
            const float fx[4] = {f[j][x].x, f[j][x].y, f[j][x].z, f[j][x].w};
            union { __bf16 b[4]; uint2 u; } hi4, lo4;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const __bf16 hb = (__bf16)fx[t];
                hi4.b[t] = hb;
                lo4.b[t] = (__bf16)(fx[t] - (float)hb);
                ss += fx[t] * fx[t];
            }
            *reinterpret_cast<uint2 *>(&s_hi[r * HLD + FPT * part + 4 * x]) = hi4.u;
            *reinterpret_cast<uint2 *>(&s_lo[r * HLD + FPT * part + 4 * x]) = lo4.u;
        }
        ss = sum8_dpp(ss);  // the row's 8 threads are one aligned group of 8 lanes
        if (crow[j] >= 0 && part == 0) {
            const float la = lamf * am[j];
            s_pool[r] = crow[j];
            // the bound 2 (||q|| |rho| ||kbar_c|| epsc + |lambda a_c| 2e-6 + (|rc| + |b|) 2^-22 + 1e-30) of
            // the header, with |rc| <= 1.01 |rho| ||q|| ||kbar_c|| (Cauchy-Schwarz; the split and the fp32
            // sum add far less than 1%) and |b| <= |lambda a_c| (|erf| <= 1): ||q|| A_c + B_c bounds it
            const float ka = fabsf(rhof) * sqrtf(ss);
            s_cf[r] = make_float4(la, 2.0f * ka * (epsc + 1.01f * 2.384185791015625e-07f),
                                  2.0f * (fabsf(la) * (2e-6f + 2.384185791015625e-07f) + 1e-30f),
                                  __int_as_float(crow[j] * p.s));
        }
    }
    __syncthreads();
    // The erf factor is 1 (to fp32 and fp64 rounding) once its argument reaches 6. The
    // pool is ascending and every query of the work-group is at or after q0, so if the
    // last pool cell is that far from q0 no query needs erf at all.
    const bool need_erf = npool > 0 && !((float)((int)q0 - s_pool[npool - 1] * p.s) * karg >= 6.0f);

    {  // 8 waves x 16 queries
        float qss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = bf16_to_f32(bq[ks].h[e]);
                qss += f * f;
            }
        const float qn = sqrtf(colsum4(qss));  // the four lanes of a query hold all its d elements

        float lbk[KL];  // this lane's KL largest lower bounds, descending
#pragma unroll
        for (int r = 0; r < KL; ++r) lbk[r] = -INFINITY;
        // approximate scores, 4 cells of each 16-cell tile per lane (cells 16*ct + 4*g + e)
        float sub[kSelPool / 16][4];  // upper bounds s~ + eps
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
                sub[ct][e] = -INFINITY;
                if (pos < npool) {
                    const float4 cf = s_cf[pos];
                    float bf = cf.x;  // lambda a_c times the erf factor 1
                    if (need_erf) {
                        const float argf = (float)((int)i - __float_as_int(cf.w)) * karg;
                        if (argf < 6.0f) bf = cf.x * erff(argf);
                    }
                    const float sv = fmaf(rhof, acc[e], bf);
                    const float ev = fmaf(qn, cf.y, cf.z);  // eps = ||q|| A_c + B_c
                    sub[ct][e] = sv + ev;
                    float x = sv - ev;
#pragma unroll
                    for (int r = 0; r < KL; ++r) {
                        const float hi = fmaxf(lbk[r], x);
                        x = fminf(lbk[r], x);
                        lbk[r] = hi;
                    }
                }
            }
        }
        // merge with the lanes of the same query column: reversing the partner's list
        // and taking elementwise maxima keeps the KL largest of both as a bitonic
        // sequence, which a half-cleaner network sorts back to descending order
#pragma unroll
        for (int m2 = 16; m2 <= 32; m2 <<= 1) {
            float pl[KL];
#pragma unroll
            for (int r = 0; r < KL; ++r) pl[r] = __shfl_xor(lbk[r], m2);
#pragma unroll
            for (int r = 0; r < KL; ++r) lbk[r] = fmaxf(lbk[r], pl[KL - 1 - r]);
#pragma unroll
            for (int st = KL / 2; st > 0; st >>= 1)
#pragma unroll
                for (int r = 0; r < KL; ++r)
                    if ((r & st) == 0) {
                        const float hi = fmaxf(lbk[r], lbk[r + st]), lo = fminf(lbk[r], lbk[r + st]);
                        lbk[r] = hi;
                        lbk[r + st] = lo;
                    }
        }
        float theta = -INFINITY;
#pragma unroll
        for (int r = 0; r < KL; ++r)
            if (r == K - 1) theta = lbk[r];

        // this lane's contenders as a bitmask over its (tile, e) slots
        uint32_t cmask = 0;
#pragma unroll
        for (int ct = 0; ct < kSelPool / 16; ++ct) {
            if (ct >= ntile) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pos = 16 * ct + 4 * g + e;
                if (pos < npool && sub[ct][e] >= theta) cmask |= 1u << (4 * ct + e);
            }
        }
        // At least min(K, pool) cells are contenders. With no more than K of them
        // the top-K set is certified without exact scores: the output lists the
        // contenders in pool (= ascending cell) order. Otherwise (a near-tie) the
        // query and its contender masks go to the fix-up list, which re-scores the
        // contenders exactly in fp64 (select_fixup_kernel).
        const int ncont = (int)colsum4((float)__popc(cmask));
        uint32_t m[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) m[gg] = (uint32_t)__shfl((int)cmask, col + 16 * gg);
        if (qok && g == 0) {
            if (ncont > K) {
                const int slot = atomicAdd(&s_nfix, 1);
                uint32_t *e = fix_region(fix, p, logical) + (size_t)slot * kFixWords;
                e[0] = (uint32_t)h;
                e[1] = (uint32_t)i;
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) e[2 + gg] = m[gg];
            } else {
                // contender bitmap over pool positions 16 ct + 4 g + e
                uint64_t bm_lo = 0, bm_hi = 0;
#pragma unroll
                for (int gg = 0; gg < 4; ++gg)
#pragma unroll
                    for (int ct = 0; ct < kSelPool / 16; ++ct) {
                        const uint64_t nib = (uint64_t)((m[gg] >> (4 * ct)) & 15u);
                        const int at = 16 * ct + 4 * gg;
                        if (at < 64) bm_lo |= nib << at;
                        else bm_hi |= nib << (at - 64);
                    }
                int32_t *o = sel + (hN + i) * K;
#pragma unroll
                for (int r = 0; r < kSelK; ++r) {
                    if (r >= K) break;
                    int pos = -1;
                    if (bm_lo) {
                        pos = __ffsll((unsigned long long)bm_lo) - 1;
                        bm_lo &= bm_lo - 1;
                    } else if (bm_hi) {
                        pos = 64 + __ffsll((unsigned long long)bm_hi) - 1;
                        bm_hi &= bm_hi - 1;
                    }
                    o[r] = pos >= 0 ? s_pool[pos] : -1;
                }
            }
        }
    }
    __syncthreads();
    if (tid == 0) fix[logical] = (uint32_t)s_nfix;
}

// Exact re-scoring of the near-tie queries listed by select_mfma_kernel: one
// work-group of two waves per scoring work-group's region (faster than four: more
// work-groups fit a CU), wave w taking its near-ties w, w + 2, ...; lane l scores
// the contenders at pool positions l and 64 + l with the fp64 fma chain of the
// oracle, then ranks each of its
// contenders against all of the query's contenders (read lane by lane), keeps
// the K best by (score desc, cell asc) and writes them in cell order.
// Comparisons are written as selects: a conditional-swap list insert with
// double keys was compiled into wrong code (equal keys lost the index
// tie-break) by this toolchain at -O3.
template <int D>
__global__ __launch_bounds__(128) void select_fixup_kernel(const uint16_t *__restrict__ q,
                                                           const float *__restrict__ kbar,
                                                           const float *__restrict__ amax,
                                                           const int32_t *__restrict__ pool, int32_t *__restrict__ sel,
                                                           const uint32_t *__restrict__ fix, KParams p) {
    const int64_t region = blockIdx.x;
    const uint32_t n = fix[region];
    const int lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    for (uint32_t j = wave; j < n; j += 2) {
        const uint32_t *e = fix_region(fix, p, region) + (size_t)j * kFixWords;
        const int h = (int)e[0];
        const int64_t i = (int64_t)e[1];
        uint64_t bm_lo = 0, bm_hi = 0;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const uint32_t m = e[2 + gg];
#pragma unroll
            for (int ct = 0; ct < kSelPool / 16; ++ct) {
                const uint64_t nib = (uint64_t)((m >> (4 * ct)) & 15u);
                const int at = 16 * ct + 4 * gg;
                if (at < 64) bm_lo |= nib << at;
                else bm_hi |= nib << (at - 64);
            }
        }
        const int64_t b = i / p.B;
        const int32_t *prow = pool + ((int64_t)h * p.nblk + b) * p.PW;
        const uint16_t *qg = q + ((int64_t)h * p.N + i) * D;
        const double sig = (double)p.sigma[h], lam = (double)p.lambda[h], rho = (double)p.rho;
        // this lane's contenders: pool positions lane (half 0) and 64 + lane (half 1)
        double vh[2] = {-INFINITY, -INFINITY};
        int ch[2] = {INT_MAX, INT_MAX};
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {
            const uint64_t bm = half ? bm_hi : bm_lo;
            if (!((bm >> lane) & 1ull)) continue;
            const int c = prow[64 * half + lane];
            const float *krow = kbar + ((int64_t)h * p.C + c) * D;
            const float am = amax[(int64_t)h * p.C + c];
            double content = 0.0;
            // 32 elements per step, two steps' loads issued before their fma chain
#pragma unroll 2
            for (int x0 = 0; x0 < D; x0 += 32) {
                uint4 qv[4];
                float4 kv[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) qv[u] = *reinterpret_cast<const uint4 *>(qg + x0 + 8 * u);
#pragma unroll
                for (int u = 0; u < 8; ++u) kv[u] = *reinterpret_cast<const float4 *>(krow + x0 + 4 * u);
#pragma unroll
                for (int t = 0; t < 32; ++t) {
                    const uint4 w4 = qv[t >> 3];
                    const uint32_t wd = (t & 7) < 2 ? w4.x : (t & 7) < 4 ? w4.y : (t & 7) < 6 ? w4.z : w4.w;
                    const float qf = __uint_as_float(t & 1 ? (wd & 0xFFFF0000u) : (wd << 16));
                    const float4 k4 = kv[t >> 2];
                    const float kf = (t & 3) == 0 ? k4.x : (t & 3) == 1 ? k4.y : (t & 3) == 2 ? k4.z : k4.w;
                    content = __fma_rn((double)qf, (double)kf, content);
                }
            }
            const double arg = __ddiv_rn(__dmul_rn(sig, (double)(i - (int64_t)c * p.s)), 2.0 * (double)p.s);
            const double gg = arg >= 6.0 ? 1.0 : erf(arg);
            const double bias = __dmul_rn(__dmul_rn(lam, (double)am), gg);
            vh[half] = __fma_rn(rho, content, bias);
            ch[half] = c;
        }
        // rank every contender against all of them: (score desc, cell asc); the K best
        // are selected, and pool order is cell order, so a selected contender's output
        // slot is the number of selected contenders at lower pool positions
        int rank[2] = {0, 0};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint64_t bm = half ? bm_hi : bm_lo;
            while (bm) {
                const int src = __ffsll((unsigned long long)bm) - 1;
                bm &= bm - 1;
                const double vy = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(vh[half]), src),
                                                   __builtin_amdgcn_readlane(__double2loint(vh[half]), src));
                const int cy = __builtin_amdgcn_readlane(ch[half], src);
#pragma unroll
                for (int x = 0; x < 2; ++x)
                    rank[x] += (vy > vh[x] || (vy == vh[x] && cy < ch[x])) ? 1 : 0;
            }
        }
        const bool s0 = ch[0] != INT_MAX && rank[0] < p.K;
        const bool s1 = ch[1] != INT_MAX && rank[1] < p.K;
        const uint64_t b0 = __ballot(s0), b1 = __ballot(s1);
        const uint64_t below = (1ull << lane) - 1ull;
        int32_t *o = sel + ((int64_t)h * p.N + i) * p.K;
        if (s0) o[__popcll(b0 & below)] = ch[0];
        if (s1) o[__popcll(b0) + __popcll(b1 & below)] = ch[1];
    }
}

hipError_t launch_select_fixup(const void *q, const float *kbar, const float *amax, const int32_t *pool,
                               int32_t *sel, const uint32_t *fix, const KParams &p, hipStream_t st) {
    const dim3 grid((unsigned)fix_regions(p)), block(128);
    if (p.d == 64)
        hipLaunchKernelGGL((select_fixup_kernel<64>), grid, block, 0, st, (const uint16_t *)q, kbar, amax, pool, sel,
                           fix, p);
    else
        hipLaunchKernelGGL((select_fixup_kernel<128>), grid, block, 0, st, (const uint16_t *)q, kbar, amax, pool,
                           sel, fix, p);
    return hipGetLastError();
}

hipError_t launch_select_mfma(const void *q, const float *kbar, const float *amax, const int32_t *pool,
                              int32_t *sel, uint32_t *fix, const KParams &p, hipStream_t st) {
    const int QW = p.B <= kSelQ ? p.B : p.B / 2;
    dim3 grid((unsigned)(((p.N + QW - 1) / QW) * p.H));
    const int rows = (p.PW + 15) / 16 * 16;
    const size_t lds = (size_t)(rows > 0 ? rows : 16) * (p.d + 8) * sizeof(uint16_t) * 2;
#define FSL_SEL(DD, KK)                                                                                           \
    hipLaunchKernelGGL((select_mfma_kernel<DD, KK>), grid, dim3(512), lds, st, (const uint16_t *)q, kbar, amax, pool, \
                       sel, fix, p, QW)
    if (p.d == 64) {
        if (p.K <= 4) FSL_SEL(64, 4); else FSL_SEL(64, 8);
    } else {
        if (p.K <= 4) FSL_SEL(128, 4); else FSL_SEL(128, 8);
    }
#undef FSL_SEL
    return hipGetLastError();
}

}  // namespace fsl

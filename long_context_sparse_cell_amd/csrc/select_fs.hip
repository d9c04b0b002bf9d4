// Cell scoring and top-K without pruning: the plain FreeSolo (FS) variant, in
// which every query of block b scores all n_b cells that lie wholly before the
// window of the block's first query (FreeSolo digest, core method: the long
// branch's candidates are the available cells, FS-L differs only by the norm
// prune; method steps 4 and 5: score = content match plus a norm-weighted erf
// relative-position bias, top K cells per query).
//
// The exact score is the one of select.hip and of the oracle:
//   s = fma(rho, q.kbar_c, (lambda * a_c) * erf(sigma (i - c s) / (2 s)))
// in fp64 with the dot product a left-to-right fma chain. The bf16 path
// certifies an MFMA approximation and re-scores only what it cannot separate:
//
//  1. fs_prep_kernel splits every float32 kbar_c once into bf16 head + tail
//     (hi, lo) and stores the per-cell constants of the error bound.
//  2. select_fs_kernel streams the block's cells through LDS in chunks of 64
//     (copied straight into LDS, double buffered, 16-byte pieces of a row
//     permuted against bank conflicts) and computes content~ = q.(hi + lo) on
//     v_mfma_f32_16x16x32_bf16, with the pool scoring kernel's bound |s - s~| <=
//     eps (select_mfma.hip) itself bounded by ||q|| A_c + B_c (fs_prep_kernel).
//     Each lane (one query, four cells of every 16-cell tile) keeps the K_L + 1
//     cells of largest upper bound (K_L = 4 or 8, at least K)
//     ub = s~ + eps, with lb = s~ - eps. A cell whose ub is below the smallest
//     lb of some lane's K leading entries (at any earlier time, shared by the
//     query's four lanes) is beaten by those K cells and is not inserted. At
//     the end theta = the K-th largest lb over the query's four
//     lists; the contenders are the listed cells with ub >= theta. Every true
//     top-K cell has ub >= its score >= theta, so it is a contender unless a
//     full list dropped it, which needs that list's smallest ub to reach theta
//     (an overflow). Without overflow, at most K contenders are the top-K set.
//  3. Near-ties (more than K contenders) and overflows go to a per-work-group
//     list; select_fs_fixup_kernel re-scores the contenders (or, after an
//     overflow, every eligible cell) exactly as the oracle does.
#include <climits>

#include "fsl_internal.h"

namespace fsl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kFsChunk = 64;  // cells per LDS chunk
constexpr int kFsK = 8;       // largest K
constexpr int kFsMaxCont = kFixWordsFs - 4;  // contender cells a near-tie entry lists

union U16x8f {
    uint4 u;
    bf16x8 b;
    uint16_t h[8];
};

// the bound's constant for a dot product over d coordinates (select_mfma.hip)
__host__ __device__ constexpr float fs_eps_content(int d) {
    return 1.001f * (7.62939453125e-06f + (float)(4 * d + 8) * 5.9604644775390625e-08f);
}

// LDS position of 16-byte piece c of chunk row r (of CPR pieces): c ^ (r mod CPR),
// so that the 16 rows of a score tile read by one lane group hit distinct banks
template <int CPR>
__device__ __forceinline__ int fs_piece(int r, int c) { return c ^ (r & (CPR - 1)); }

}  // namespace

// kbar -> khi, klo (bf16 head and tail, round to nearest even) and
// kcf = (lambda a_c, A_c, B_c, c s as int bits), the constants of the per-pair bound
// eps = ||q|| A_c + B_c. The pool kernel's bound (select_mfma.hip) is
//   2 (||q|| |rho| ||kbar_c|| e_d + |lambda a_c| 2e-6 + (|rc| + |b|) 2^-22 + 1e-30)
// with rc = rho q.(hi + lo) in fp32 and b the bias. Here |rc| <= 1.01 |rho| ||q|| ||kbar_c||
// (Cauchy-Schwarz; the split and the fp32 sum add far less than 1%) and |b| <= |lambda a_c|
// (|erf| <= 1), so
//   A_c = 2 |rho| ||kbar_c|| (e_d + 1.01 2^-22),  B_c = 2 (|lambda a_c| (2e-6 + 2^-22) + 1e-30)
// bound it from above with one fma per pair.
// Row r by 8 consecutive threads, 64 rows per work-group.
template <int D>
__global__ __launch_bounds__(512) void fs_prep_kernel(const float *__restrict__ kbar, const float *__restrict__ amax,
                                                      uint16_t *__restrict__ khi, uint16_t *__restrict__ klo,
                                                      float4 *__restrict__ kcf, KParams p) {
    constexpr int FPT = D / 8;
    const int h = blockIdx.y;
    const int64_t r = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    const bool ok = r < p.C;
    const int64_t rr = ok ? r : p.C - 1;
    const float *src = kbar + ((int64_t)h * p.C + rr) * D + FPT * part;
    float4 f[FPT / 4];
#pragma unroll
    for (int x = 0; x < FPT / 4; ++x) f[x] = *reinterpret_cast<const float4 *>(src + 4 * x);
    float ss = 0.0f;
    uint16_t *dh = khi + ((int64_t)h * p.C + rr) * D + FPT * part;
    uint16_t *dl = klo + ((int64_t)h * p.C + rr) * D + FPT * part;
#pragma unroll
    for (int x = 0; x < FPT / 4; ++x) {
        const float fx[4] = {f[x].x, f[x].y, f[x].z, f[x].w};
        union { __bf16 b[4]; uint2 u; } hi4, lo4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const __bf16 hb = (__bf16)fx[t];
            hi4.b[t] = hb;
            lo4.b[t] = (__bf16)(fx[t] - (float)hb);
            ss += fx[t] * fx[t];
        }
        if (ok) {
            *reinterpret_cast<uint2 *>(dh + 4 * x) = hi4.u;
            *reinterpret_cast<uint2 *>(dl + 4 * x) = lo4.u;
        }
    }
    ss = sum8_dpp(ss);  // all 8 threads of the row take part
    if (ok && part == 0) {
        const float la = p.lambda[h] * amax[(int64_t)h * p.C + r];
        const float ka = fabsf(p.rho) * sqrtf(ss);
        kcf[(int64_t)h * p.C + r] =
            make_float4(la, 2.0f * ka * (fs_eps_content(D) + 1.01f * 2.384185791015625e-07f),
                        2.0f * (fabsf(la) * (2e-6f + 2.384185791015625e-07f) + 1e-30f), __int_as_float((int)(r * p.s)));
    }
}

template <int D, int KL>
__global__ __launch_bounds__(512) void select_fs_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ khi,
                                                        const uint16_t *__restrict__ klo,
                                                        const float4 *__restrict__ kcf, int32_t *__restrict__ sel,
                                                        uint32_t *__restrict__ fix, KParams p, int QW) {
    constexpr int QS = D / 32;
    constexpr int CH = kFsChunk;
    constexpr int CPR = D / 8;     // 16-byte pieces per row
    constexpr int ROWU = CH * D * 2 / 1024;  // 1 KB copy units of a chunk's hi (and of its lo) rows
    constexpr int NCOPY = 2 * ROWU + 1;      // and one unit of per-cell constants (64 x 16 bytes)
    static_assert(CH == 64, "one copy unit of per-cell constants per chunk");
    // listed cells per lane: one more than the largest K of this instance, so a list
    // overflows only when a single lane holds K + 1 cells whose bounds reach theta
    constexpr int kFsCap = KL + 1;
    // two named buffers of each kind, so that the compiler can tell a chunk's copy from
    // the reads of the other buffer and does not wait for the copy before them
    __shared__ __attribute__((aligned(1024))) uint16_t s_hi0[CH * D];
    __shared__ __attribute__((aligned(1024))) uint16_t s_hi1[CH * D];
    __shared__ __attribute__((aligned(1024))) uint16_t s_lo0[CH * D];
    __shared__ __attribute__((aligned(1024))) uint16_t s_lo1[CH * D];
    __shared__ __attribute__((aligned(1024))) float4 s_cf0[CH];
    __shared__ __attribute__((aligned(1024))) float4 s_cf1[CH];
    __shared__ int s_nfix;

    const int nqb = (int)((p.N + QW - 1) / QW);
    const int logical = xcd_remap((int)blockIdx.x, nqb * p.H);
    const int h = logical / nqb;
    const int64_t q0 = (int64_t)(logical % nqb) * QW;
    const int64_t b = q0 / p.B;
    const int nq = (int)min((int64_t)QW, p.N - q0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g = lane >> 4;
    const int K = p.K;
    const int n = (int)eligible_cells(p, b);
    const int nch = (n + CH - 1) / CH;
    const int64_t hN = (int64_t)h * p.N;
    const int64_t hC = (int64_t)h * p.C;
    const float sigf = p.sigma[h], rhof = p.rho;
    const float karg = sigf / (2.0f * (float)p.s);

    const int ql = 16 * wave + col;
    const bool qok = ql < nq;
    const int64_t i = q0 + (qok ? ql : 0);
    U16x8f bq[QS];
#pragma unroll
    for (int ks = 0; ks < QS; ++ks) bq[ks].u = *reinterpret_cast<const uint4 *>(q + (hN + i) * D + 32 * ks + 8 * g);
    if (tid == 0) s_nfix = 0;

    // ---- chunk copies straight into LDS (global_load_lds), 1 KB per wave instruction:
    // rows past the block's last cell repeat that cell (they are never scored)
    const int64_t nlast = (int64_t)n - 1;
    auto issue = [&](int t, uint16_t *bhi, uint16_t *blo, float4 *bcf) __attribute__((always_inline)) {
        const int64_t c0 = (int64_t)t * CH;
        for (int u = __builtin_amdgcn_readfirstlane(wave); u < NCOPY; u += 8) {
            if (u < 2 * ROWU) {
                const int uu = u % ROWU;
                const int pc = 64 * uu + lane;  // 16-byte piece of the chunk
                const int r = pc / CPR, phys = pc % CPR;
                const int64_t off = (hC + min(c0 + r, nlast)) * D + 8 * fs_piece<CPR>(r, phys);
                if (u < ROWU)
                    lds_dma16(khi + off, bhi + 512 * uu);
                else
                    lds_dma16(klo + off, blo + 512 * uu);
            } else {
                lds_dma16(kcf + hC + min(c0 + lane, nlast), bcf);
            }
        }
    };

    float qss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < QS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = bf16_to_f32(bq[ks].h[e]);
            qss += f * f;
        }
    const float qn = sqrtf(colsum4(qss));  // the four lanes of a query hold all its d elements

    // this lane's list: the kFsCap cells of largest upper bound, descending
    float lu[kFsCap], ll[kFsCap];
    int li[kFsCap];
#pragma unroll
    for (int r = 0; r < kFsCap; ++r) { lu[r] = -INFINITY; ll[r] = -INFINITY; li[r] = INT_MAX; }
    float thr = -INFINITY;  // a score that K cells are known to beat: skip cells whose ub is below it

    auto chunk = [&](int t, const uint16_t *bhi, const uint16_t *blo, const float4 *bcf) __attribute__((always_inline)) {
        const int c0 = t * CH;
        // erf is 1 (in fp32 and fp64) once its argument reaches 6; cells are ascending
        // and every query is at or after q0, so the chunk's last cell decides for all
        const int clast = min(c0 + CH, n) - 1;
        const bool need_erf = !((float)((int)q0 - clast * p.s) * karg >= 6.0f);
#pragma unroll
        for (int ct = 0; ct < CH / 16; ++ct) {
            const int rowc = 16 * ct + col;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) {
                U16x8f hi, lo;
                hi.u = *reinterpret_cast<const uint4 *>(&bhi[rowc * D + 8 * fs_piece<CPR>(rowc, 4 * ks + g)]);
                lo.u = *reinterpret_cast<const uint4 *>(&blo[rowc * D + 8 * fs_piece<CPR>(rowc, 4 * ks + g)]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi.b, bq[ks].b, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo.b, bq[ks].b, acc, 0, 0, 0);
            }
            // read the accumulators in straight-line code right after the MFMAs, where the
            // compiler pads the MFMA-to-VALU dependency with wait states; the empty asm keeps
            // these reads here, ahead of the branches below (a read placed after a branch
            // was seen taking the accumulator before the MFMA had written it)
            float rcv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rcv[e] = acc[e];
            asm volatile("" : "+v"(rcv[0]), "+v"(rcv[1]), "+v"(rcv[2]), "+v"(rcv[3]));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int loc = 16 * ct + 4 * g + e;
                const int c = c0 + loc;
                const float4 cf = bcf[loc];
                float bf = cf.x;  // lambda a_c times the erf factor 1
                if (need_erf) {
                    const float argf = (float)((int)i - __float_as_int(cf.w)) * karg;
                    if (argf < 6.0f) bf = cf.x * erff(argf);
                }
                const float sv = fmaf(rhof, rcv[e], bf);
                const float ev = fmaf(qn, cf.y, cf.z);  // eps = ||q|| A_c + B_c
                float cu = c < n ? sv + ev : -INFINITY;
                if (cu >= thr && cu > lu[kFsCap - 1]) {
                    float cl = sv - ev;
                    int ci = c;
                    // carry the cell down the list (selects only)
#pragma unroll
                    for (int r = 0; r < kFsCap; ++r) {
                        const bool bt = cu > lu[r];
                        const float tu = lu[r], tl = ll[r];
                        const int ti = li[r];
                        lu[r] = bt ? cu : tu;
                        ll[r] = bt ? cl : tl;
                        li[r] = bt ? ci : ti;
                        cu = bt ? tu : cu;
                        cl = bt ? tl : cl;
                        ci = bt ? ti : ci;
                    }
                    float m = INFINITY;
#pragma unroll
                    for (int r = 0; r < kFsK; ++r)
                        if (r < K) m = fminf(m, ll[r]);
                    thr = fmaxf(thr, m);
                }
            }
            // a lane's threshold holds for the whole query (K cells beat anything below it),
            // so the four lanes of the query column take the largest; thresholds stay valid
            // when the entries that certified them are evicted later
            thr = colmax4(thr);
        }
    };
    if (nch > 0) issue(0, s_hi0, s_lo0, s_cf0);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < nch; t += 2) {
        if (t + 1 < nch) issue(t + 1, s_hi1, s_lo1, s_cf1);
        chunk(t, s_hi0, s_lo0, s_cf0);
        wait_vmem();  // the next chunk has landed, and every wave is done with this one
        __syncthreads();
        if (t + 1 >= nch) break;
        if (t + 2 < nch) issue(t + 2, s_hi0, s_lo0, s_cf0);
        chunk(t + 1, s_hi1, s_lo1, s_cf1);
        wait_vmem();
        __syncthreads();
    }

    // ---- theta = K-th largest lb over the query's four lists: each lane sorts its
    // lbs (descending, KL kept), then the lists of the query column are merged
    float lbk[KL];
#pragma unroll
    for (int r = 0; r < KL; ++r) lbk[r] = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < kFsCap; ++s2) {
        float x = ll[s2];
#pragma unroll
        for (int r = 0; r < KL; ++r) {
            const float hi = fmaxf(lbk[r], x);
            x = fminf(lbk[r], x);
            lbk[r] = hi;
        }
    }
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

    // contenders of this lane; an overflow if a full list's smallest ub reaches theta
    int cid[kFsCap];
    int mycnt = 0;
#pragma unroll
    for (int r = 0; r < kFsCap; ++r) {
        const bool on = li[r] != INT_MAX && lu[r] >= theta;
        cid[r] = on ? li[r] : INT_MAX;
        mycnt += on ? 1 : 0;
    }
    const bool over_l = li[kFsCap - 1] != INT_MAX && lu[kFsCap - 1] >= theta;
    const int ncont = (int)colsum4((float)mycnt);
    // more contenders than a near-tie entry holds: re-score every eligible cell instead
    const bool over = colmax4(over_l ? 1.0f : 0.0f) > 0.0f || ncont > kFsMaxCont;

    // lane g == 0 of each query column gathers the column's contenders (all lanes
    // take part in the shuffles)
    int gath[kFsCap * 4];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int r = 0; r < kFsCap; ++r) gath[gg * kFsCap + r] = __shfl(cid[r], col + 16 * gg);
    if (qok && g == 0) {
        if (over || ncont > K) {
            const int slot = atomicAdd(&s_nfix, 1);
            uint32_t *e = fix_region_fs(fix, p, logical) + (size_t)slot * kFixWordsFs;
            e[0] = (uint32_t)h;
            e[1] = (uint32_t)i;
            e[2] = over ? kFsOverflow : (uint32_t)ncont;
            e[3] = 0u;
            int k2 = 0;
#pragma unroll
            for (int x = 0; x < kFsCap * 4; ++x) {
                if (gath[x] != INT_MAX && k2 < kFsMaxCont) {
                    e[4 + k2] = (uint32_t)gath[x];
                    ++k2;
                }
            }
        } else {
            // at most K contenders: the top-K set, written in ascending cell order
            int best[kFsK];
#pragma unroll
            for (int r = 0; r < kFsK; ++r) best[r] = INT_MAX;
#pragma unroll
            for (int x = 0; x < kFsCap * 4; ++x) {
                int c = gath[x];
#pragma unroll
                for (int r = 0; r < kFsK; ++r) {
                    const int lo = min(best[r], c), hi = max(best[r], c);
                    best[r] = lo;
                    c = hi;
                }
            }
            int32_t *o = sel + (hN + i) * K;
#pragma unroll
            for (int r = 0; r < kFsK; ++r)
                if (r < K) o[r] = best[r] == INT_MAX ? -1 : best[r];
        }
    }
    __syncthreads();
    if (tid == 0) fix[logical] = (uint32_t)s_nfix;
}

// Exact re-scoring of the near-tie and overflow queries listed by
// select_fs_kernel: one work-group of four waves per scoring work-group's
// region, wave w taking entries w, w + 4, ... Each lane scores its share of the
// candidates (the listed contenders, or every eligible cell after an overflow)
// with the oracle's fp64 fma chain and keeps its K best under (score desc,
// cell asc); K rounds of a wave-wide maximum then take the K best overall,
// written in ascending cell order. Comparisons are written as selects.
template <int D>
__global__ __launch_bounds__(256) void select_fs_fixup_kernel(const uint16_t *__restrict__ q,
                                                              const float *__restrict__ kbar,
                                                              const float *__restrict__ amax,
                                                              int32_t *__restrict__ sel,
                                                              const uint32_t *__restrict__ fix, KParams p) {
    // each wave's current query row in fp32 (written and read by that wave only: a wave's LDS
    // operations complete in issue order)
    __shared__ __attribute__((aligned(16))) float s_qf[4][D];
    const int64_t region = blockIdx.x;
    const uint32_t nfix = fix[region];
    const int lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    const int K = p.K;
    for (uint32_t j = wave; j < nfix; j += 4) {
        const uint32_t *e = fix_region_fs(fix, p, region) + (size_t)j * kFixWordsFs;
        const int h = (int)e[0];
        const int64_t i = (int64_t)e[1];
        const bool over = e[2] == kFsOverflow;
        const int64_t ncand = over ? eligible_cells(p, i / p.B) : (int64_t)e[2];
        const uint16_t *qg = q + ((int64_t)h * p.N + i) * D;
        for (int x = lane; x < D; x += 64) s_qf[wave][x] = __uint_as_float((uint32_t)qg[x] << 16);
        const double sig = (double)p.sigma[h], lam = (double)p.lambda[h], rho = (double)p.rho;
        double bs[kFsK];
        int bi[kFsK];
#pragma unroll
        for (int r = 0; r < kFsK; ++r) { bs[r] = -INFINITY; bi[r] = INT_MAX; }
        for (int64_t t = lane; t < ncand; t += 64) {
            const int c = over ? (int)t : (int)e[4 + t];
            const float *krow = kbar + ((int64_t)h * p.C + c) * D;
            double content = 0.0;
            // 64 coordinates' loads per round, then their fma chain in coordinate order
#pragma unroll 1
            for (int x0 = 0; x0 < D; x0 += 64) {
                float4 kv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) kv[u] = *reinterpret_cast<const float4 *>(krow + x0 + 4 * u);
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const float4 q4 = *reinterpret_cast<const float4 *>(&s_qf[wave][x0 + 4 * u]);
                    content = __fma_rn((double)q4.x, (double)kv[u].x, content);
                    content = __fma_rn((double)q4.y, (double)kv[u].y, content);
                    content = __fma_rn((double)q4.z, (double)kv[u].z, content);
                    content = __fma_rn((double)q4.w, (double)kv[u].w, content);
                }
            }
            const double arg = __ddiv_rn(__dmul_rn(sig, (double)(i - (int64_t)c * p.s)), 2.0 * (double)p.s);
            const double gg = arg >= 6.0 ? 1.0 : erf(arg);
            const double bias = __dmul_rn(__dmul_rn(lam, (double)amax[(int64_t)h * p.C + c]), gg);
            double sc = __fma_rn(rho, content, bias);
            int ci = c;
#pragma unroll
            for (int r = 0; r < kFsK; ++r) {
                const bool bt = r < K && better_d(sc, ci, bs[r], bi[r]);
                const double ts = bs[r];
                const int ti = bi[r];
                bs[r] = bt ? sc : ts;
                bi[r] = bt ? ci : ti;
                sc = bt ? ts : sc;
                ci = bt ? ti : ci;
            }
        }
        // K rounds of the wave-wide best head; the winning lane drops its head
        int win[kFsK];
#pragma unroll
        for (int r = 0; r < kFsK; ++r) {
            win[r] = INT_MAX;
            if (r >= K) continue;
            double vs = bs[0];
            int vi = bi[0];
#pragma unroll
            for (int m = 32; m > 0; m >>= 1) {
                const double ps = __hiloint2double(__shfl_xor(__double2hiint(vs), m), __shfl_xor(__double2loint(vs), m));
                const int pi = __shfl_xor(vi, m);
                const bool bt = better_d(ps, pi, vs, vi);
                vs = bt ? ps : vs;
                vi = bt ? pi : vi;
            }
            win[r] = vi;
            if (vi != INT_MAX && bi[0] == vi) {
#pragma unroll
                for (int x = 0; x + 1 < kFsK; ++x) { bs[x] = bs[x + 1]; bi[x] = bi[x + 1]; }
                bs[kFsK - 1] = -INFINITY;
                bi[kFsK - 1] = INT_MAX;
            }
        }
        if (lane == 0) {
            // ascending cell order, -1 padding
#pragma unroll
            for (int x = 0; x < kFsK; ++x)
#pragma unroll
                for (int y = 0; y + 1 < kFsK - x; ++y) {
                    const int lo = min(win[y], win[y + 1]), hi = max(win[y], win[y + 1]);
                    win[y] = lo;
                    win[y + 1] = hi;
                }
            int32_t *o = sel + ((int64_t)h * p.N + i) * K;
            for (int r = 0; r < K; ++r) o[r] = win[r] == INT_MAX ? -1 : win[r];
        }
    }
}

hipError_t launch_select_fs(const void *q, const float *kbar, const float *amax, int32_t *sel, const Work &w,
                            const KParams &p, hipStream_t st) {
    if (p.C > 0) {
        const dim3 pg((unsigned)((p.C + 63) / 64), (unsigned)p.H);
        if (p.d == 64)
            hipLaunchKernelGGL((fs_prep_kernel<64>), pg, dim3(512), 0, st, kbar, amax, w.khi, w.klo, w.kcf, p);
        else
            hipLaunchKernelGGL((fs_prep_kernel<128>), pg, dim3(512), 0, st, kbar, amax, w.khi, w.klo, w.kcf, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int QW = p.B <= kFixRegion ? p.B : p.B / 2;
    const dim3 grid((unsigned)(((p.N + QW - 1) / QW) * p.H));
#define FSL_SFS(DD, KK)                                                                                            \
    hipLaunchKernelGGL((select_fs_kernel<DD, KK>), grid, dim3(512), 0, st, (const uint16_t *)q, w.khi, w.klo, w.kcf, \
                       sel, w.fix, p, QW)
    if (p.d == 64) {
        if (p.K <= 4) FSL_SFS(64, 4); else FSL_SFS(64, 8);
    } else {
        if (p.K <= 4) FSL_SFS(128, 4); else FSL_SFS(128, 8);
    }
#undef FSL_SFS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.d == 64)
        hipLaunchKernelGGL((select_fs_fixup_kernel<64>), grid, dim3(256), 0, st, (const uint16_t *)q, kbar, amax, sel,
                           w.fix, p);
    else
        hipLaunchKernelGGL((select_fs_fixup_kernel<128>), grid, dim3(256), 0, st, (const uint16_t *)q, kbar, amax, sel,
                           w.fix, p);
    return hipGetLastError();
}

}  // namespace fsl

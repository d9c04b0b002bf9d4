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
//     Each lane holds one query and four cells of every 16-cell tile.
//     A first pass over every 8th chunk scores q.hi alone (its bound widened by
//     the tail's share) and keeps each lane's largest lower bound: the query's
//     four lanes hold distinct cells, so the smallest of their four maxima (of
//     eight, two per lane, for K > 4) is a score that K cells reach, the
//     starting threshold. The second pass visits every chunk; each lane keeps
//     the K_L + 1 cells of largest upper bound ub = s~ + eps (K_L = 4 or 8, at
//     least K) among those whose ub reaches the threshold, which rises with the
//     lists (the smallest over the four lanes of their leading lower bounds).
//     Insertions go in rounds, each lane carrying its largest pending cell down
//     its list with selects. A listed cell's lower bound is ub - 2 emax (emax the
//     largest eps the lane has listed), less a rounding margin. At the end
//     theta = the K-th largest lower bound over the query's four lists; the
//     contenders are the listed cells with ub >= theta. Every true top-K cell
//     has ub >= its score >= theta, so it is a contender unless a full list
//     dropped it, which needs that list's smallest ub to reach theta (an
//     overflow). Without overflow, at most K contenders are the top-K set.
//  3. Near-ties (more than K contenders) and overflows go to a per-work-group
//     list; select_fs_fixup_kernel re-scores the contenders (or, after an
//     overflow, every eligible cell) exactly as the oracle does.
#include <cfloat>
#include <climits>
#include <cstdlib>

#include "fsl_internal.h"

namespace fsl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kFsChunk = 64;  // cells per LDS chunk
constexpr int kFsK = 8;       // largest K
constexpr int kFsMaxCont = kFixWordsFs - 4;  // contender cells a near-tie entry lists
constexpr int kFsPass1Stride = 8;  // the scorer's first pass visits every 8th chunk

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

// B_c = 2 (|lambda a_c| (2e-6 + 2^-22) + 1e-30), the part of the per-pair bound that
// does not scale with ||q|| (computed the same way wherever it is needed)
__device__ __forceinline__ float fs_bconst(float la) {
    return 2.0f * (fabsf(la) * (2e-6f + 2.384185791015625e-07f) + 1e-30f);
}

// a lower bound of the score of a cell with upper bound u and eps at most e2 / 2:
// u - e2, less a margin for the fp32 rounding of u and of this difference
__device__ __forceinline__ float fs_lbound(float u, float e2) {
    return (u - e2) - (fabsf(u) + e2) * 4.76837158203125e-07f;
}

// kbar -> khi, klo (bf16 head and tail, round to nearest even) and
// kcf = (A_c, lambda a_c + B_c, lambda a_c - B_c, lambda a_c), the constants of the
// per-pair bound eps = ||q|| A_c + B_c. The pool kernel's bound (select_mfma.hip) is
//   2 (||q|| |rho| ||kbar_c|| e_d + |lambda a_c| 2e-6 + (|rc| + |b|) 2^-22 + 1e-30)
// with rc = rho q.(hi + lo) in fp32 and b the bias. Here |rc| <= 1.01 |rho| ||q|| ||kbar_c||
// (Cauchy-Schwarz; the split and the fp32 sum add far less than 1%) and |b| <= |lambda a_c|
// (|erf| <= 1), so
//   A_c = 2 |rho| ||kbar_c|| (e_d + 1.01 2^-22),  B_c = fs_bconst(lambda a_c)
// bound it from above. Where the erf factor is 1 (every cell far enough before the
// query) a cell's upper bound is one fma on lambda a_c + B_c and its lower bound one on
// lambda a_c - B_c; the roundings of these sums are of the size the 2^-22 terms cover.
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
        const float bc = fs_bconst(la);
        kcf[(int64_t)h * p.C + r] =
            make_float4(2.0f * ka * (fs_eps_content(D) + 1.01f * 2.384185791015625e-07f), la + bc, la - bc, la);
    }
}

template <int D, int KL>
__global__ __launch_bounds__(512) void select_fs_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ khi,
                                                        const uint16_t *__restrict__ klo,
                                                        const float4 *__restrict__ kcf, int32_t *__restrict__ sel,
                                                        uint32_t *__restrict__ fix, KParams p, int QW, int S1) {
    constexpr int QS = D / 32;
    constexpr int CH = kFsChunk;
    constexpr int CPR = D / 8;     // 16-byte pieces per row
    constexpr int ROWU = CH * D * 2 / 1024;  // 1 KB copy units of a chunk's hi (and of its lo) rows
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
    // rows past the block's last cell repeat that cell (they are never scored); the
    // first pass copies the hi rows and the constants only
    // (offsets are 32-bit, from the head's base: rows below C, C * D below 2^31)
    const uint16_t *khi_h = khi + hC * D;
    const uint16_t *klo_h = klo + hC * D;
    const float4 *kcf_h = kcf + hC;
    const int prow = lane / CPR, pphys = lane % CPR;  // a copy unit's lane: row offset and piece
    auto issue = [&](int t, uint16_t *bhi, uint16_t *blo, float4 *bcf, bool with_lo) __attribute__((always_inline)) {
        const int c0 = t * CH;
        const int ncopy = with_lo ? 2 * ROWU + 1 : ROWU + 1;
        for (int u = __builtin_amdgcn_readfirstlane(wave); u < ncopy; u += 8) {
            if (u < ROWU || (with_lo && u < 2 * ROWU)) {
                const int uu = u % ROWU;
                const int r = uu * (64 / CPR) + prow;  // chunk row of this lane's 16-byte piece
                const uint32_t off = (uint32_t)min(c0 + r, n - 1) * D + 8 * fs_piece<CPR>(r, pphys);
                if (u < ROWU)
                    lds_dma16(khi_h + off, bhi + 512 * uu);
                else
                    lds_dma16(klo_h + off, blo + 512 * uu);
            } else {
                lds_dma16(kcf_h + min(c0 + lane, n - 1), bcf);
            }
        }
    };
    // the chunks first, first + step, ... below nch, double buffered; body(t, hi, lo, cf)
    auto stream = [&](int first, int step, bool with_lo, auto &&body) __attribute__((always_inline)) {
        if (first >= nch) return;
        issue(first, s_hi0, s_lo0, s_cf0, with_lo);
        wait_vmem();
        __syncthreads();
        for (int t = first; t < nch; t += 2 * step) {
            if (t + step < nch) issue(t + step, s_hi1, s_lo1, s_cf1, with_lo);
            body(t, s_hi0, s_lo0, s_cf0);
            wait_vmem();  // the next chunk has landed, and every wave is done with this one
            __syncthreads();
            if (t + step >= nch) break;
            if (t + 2 * step < nch) issue(t + 2 * step, s_hi0, s_lo0, s_cf0, with_lo);
            body(t + step, s_hi1, s_lo1, s_cf1);
            wait_vmem();
            __syncthreads();
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
    // the first pass scores q.hi alone: |q.lo| <= 2^-9 ||q|| ||kbar_c|| adds 2^-8 |rho| ||q||
    // ||kbar_c|| (with a factor 2 to spare) to eps, i.e. ||q|| A_c grows by the factor below
    const float qn_hi =
        qn * (1.0f + 3.90625e-3f / (2.0f * (fs_eps_content(D) + 1.01f * 2.384185791015625e-07f))) * 1.0001f;

    // erf is 1 (in fp32 and fp64) once its argument reaches 6; cells are ascending
    // and every query is at or after q0, so the chunk's last cell decides for all
    auto chunk_needs_erf = [&](int c0) __attribute__((always_inline)) {
        const int clast = min(c0 + CH, n) - 1;
        return !((float)((int)q0 - clast * p.s) * karg >= 6.0f);
    };
    // the erf-weighted bias of cell c for this lane's query
    auto bias_erf = [&](float la, int c) __attribute__((always_inline)) {
        const float argf = (float)((int)i - c * p.s) * karg;
        return argf < 6.0f ? la * erff(argf) : la;
    };

    // ---- first pass: a threshold. Each lane keeps the largest lower bound of its cells
    // (two for K > 4: cells e < 2 and e >= 2 of each group of four); the query's four lanes
    // hold distinct cells, so at least 4 (or 8) cells score above the smallest of them.
    // S1 > 1 visits every S1-th chunk only.
    float lbm0 = -INFINITY, lbm1 = -INFINITY;
    stream(0, S1, false, [&](int t, const uint16_t *bhi, const uint16_t *, const float4 *bcf)
                             __attribute__((always_inline)) {
        const int c0 = t * CH;
        const bool need_erf = chunk_needs_erf(c0);
        const bool tail = c0 + CH > n;
#pragma unroll
        for (int ct = 0; ct < CH / 16; ++ct) {
            const int rowc = 16 * ct + col;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) {
                U16x8f hi;
                hi.u = *reinterpret_cast<const uint4 *>(&bhi[rowc * D + 8 * fs_piece<CPR>(rowc, 4 * ks + g)]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi.b, bq[ks].b, acc, 0, 0, 0);
            }
            // the accumulators read in straight-line code right after the MFMAs (the empty
            // asm keeps these reads ahead of the branches below)
            float rcv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rcv[e] = acc[e];
            asm volatile("" : "+v"(rcv[0]), "+v"(rcv[1]), "+v"(rcv[2]), "+v"(rcv[3]));
            const int cbase = c0 + 16 * ct + 4 * g;
            float lb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float4 cf = bcf[16 * ct + 4 * g + e];
                lb[e] = fmaf(rhof, rcv[e], fmaf(-qn_hi, cf.x, cf.z));
            }
            if (need_erf) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float4 cf = bcf[16 * ct + 4 * g + e];
                    lb[e] = fmaf(rhof, rcv[e], bias_erf(cf.w, cbase + e) - fmaf(qn_hi, cf.x, fs_bconst(cf.w)));
                }
            }
            if (tail) {
#pragma unroll
                for (int e = 0; e < 4; ++e) lb[e] = cbase + e < n ? lb[e] : -INFINITY;
            }
            if (KL > 4) {
                lbm0 = fmaxf(lbm0, fmaxf(lb[0], lb[1]));
                lbm1 = fmaxf(lbm1, fmaxf(lb[2], lb[3]));
            } else {
                lbm0 = fmaxf(lbm0, fmaxf(fmaxf(lb[0], lb[1]), fmaxf(lb[2], lb[3])));
            }
        }
    });
    // a score that K cells are known to reach: cells whose ub is below it are skipped
    // (never below the lowest finite float, so an empty slot's -inf never passes)
    float thr = fmaxf(-colmax4(-(KL > 4 ? fminf(lbm0, lbm1) : lbm0)), -FLT_MAX);

    // ---- second pass: this lane's list, the kFsCap cells of largest upper bound
    // (descending) among those that reach the threshold; a listed cell's lower bound is
    // taken as fs_lbound(ub, 2 emax), emax the largest eps of the cells listed so far
    float lu[kFsCap];
    int li[kFsCap];
#pragma unroll
    for (int r = 0; r < kFsCap; ++r) { lu[r] = -INFINITY; li[r] = INT_MAX; }
    float emax = 0.0f;
    float floor_u = thr;  // max(thr, lu[kFsCap - 1]): a cell is listed if its ub reaches this
    stream(0, 1, true, [&](int t, const uint16_t *bhi, const uint16_t *blo, const float4 *bcf)
                           __attribute__((always_inline)) {
        const int c0 = t * CH;
        const bool need_erf = chunk_needs_erf(c0);
        const bool tail = c0 + CH > n;
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
            float rcv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rcv[e] = acc[e];
            asm volatile("" : "+v"(rcv[0]), "+v"(rcv[1]), "+v"(rcv[2]), "+v"(rcv[3]));
            const int cbase = c0 + 16 * ct + 4 * g;
            float pc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 cf = *reinterpret_cast<const float2 *>(&bcf[16 * ct + 4 * g + e]);
                pc[e] = fmaf(rhof, rcv[e], fmaf(qn, cf.x, cf.y));
            }
            if (need_erf) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float4 cf = bcf[16 * ct + 4 * g + e];
                    pc[e] = fmaf(rhof, rcv[e], bias_erf(cf.w, cbase + e) + fmaf(qn, cf.x, fs_bconst(cf.w)));
                }
            }
            if (tail) {
#pragma unroll
                for (int e = 0; e < 4; ++e) pc[e] = cbase + e < n ? pc[e] : -INFINITY;
            }
            // insertion rounds: each lane carries its largest pending cell down its list
            // (selects only), so one round serves every lane that still has one; a lane
            // has at most four, and a round is skipped unless some lane has one (each round
            // updates the list in place: no loop-carried copies of it)
            float m = fmaxf(fmaxf(pc[0], pc[1]), fmaxf(pc[2], pc[3]));
#pragma unroll
            for (int round = 0; round < 4; ++round) {
                if (__ballot(m >= floor_u) == 0ull) break;
                if (m >= floor_u) {
                    // the first of the four holding m (selects, no branches)
                    int e = 3;
                    e = m == pc[2] ? 2 : e;
                    e = m == pc[1] ? 1 : e;
                    e = m == pc[0] ? 0 : e;
#pragma unroll
                    for (int x = 0; x < 4; ++x) pc[x] = x == e ? -INFINITY : pc[x];
                    const float4 cf = bcf[16 * ct + 4 * g + e];
                    emax = fmaxf(emax, fmaf(qn, cf.x, fs_bconst(cf.w)));
                    float cu = m;
                    int ci = cbase + e;
#pragma unroll
                    for (int r = 0; r < kFsCap; ++r) {
                        const bool bt = cu > lu[r];
                        const float tu = lu[r];
                        const int ti = li[r];
                        lu[r] = bt ? cu : tu;
                        li[r] = bt ? ci : ti;
                        cu = bt ? tu : cu;
                        ci = bt ? ti : ci;
                    }
                    floor_u = fmaxf(thr, lu[kFsCap - 1]);
                }
                m = fmaxf(fmaxf(pc[0], pc[1]), fmaxf(pc[2], pc[3]));
            }
        }
        // the threshold rises with the lists: the smallest over the query's four lanes of
        // the lower bounds of their first ceil(K/4) entries (4 ceil(K/4) >= K distinct
        // cells); it stays valid when those entries are evicted later
        const float e2 = 2.0f * emax;
        const float v = KL > 4 && K > 4 ? fminf(fs_lbound(lu[0], e2), fs_lbound(lu[1], e2)) : fs_lbound(lu[0], e2);
        thr = fmaxf(thr, -colmax4(-v));
        floor_u = fmaxf(thr, lu[kFsCap - 1]);
    });

    // ---- theta = K-th largest lb over the query's four lists: each lane sorts its
    // lbs (descending, KL kept), then the lists of the query column are merged
    float lbk[KL];
#pragma unroll
    for (int r = 0; r < KL; ++r) lbk[r] = -INFINITY;
    const float e2f = 2.0f * emax;
#pragma unroll
    for (int s2 = 0; s2 < kFsCap; ++s2) {
        float x = fs_lbound(lu[s2], e2f);
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
// select_fs_kernel: one work-group of two waves per scoring work-group's
// region (regions hold about three entries; two waves per work-group measured
// faster than one or four), wave w taking entries w, w + 2, ... Each lane scores its share of the
// candidates (the listed contenders, or every eligible cell after an overflow)
// with the oracle's fp64 fma chain and keeps its K best under (score desc,
// cell asc); K rounds of a wave-wide maximum then take the K best overall,
// written in ascending cell order. Comparisons are written as selects.
template <int D>
__global__ __launch_bounds__(128) void select_fs_fixup_kernel(const uint16_t *__restrict__ q,
                                                              const float *__restrict__ kbar,
                                                              const float *__restrict__ amax,
                                                              int32_t *__restrict__ sel,
                                                              const uint32_t *__restrict__ fix, KParams p) {
    // each wave's current query row in fp32 (written and read by that wave only: a wave's LDS
    // operations complete in issue order)
    __shared__ __attribute__((aligned(16))) float s_qf[2][D];
    const int64_t region = blockIdx.x;
    const uint32_t nfix = fix[region];
    const int lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    const int K = p.K;
    for (uint32_t j = wave; j < nfix; j += 2) {
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
    // the scorer addresses a head's split cell means with 32-bit element offsets
    if ((int64_t)p.C * p.d >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
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
                       sel, w.fix, p, QW, kFsPass1Stride)
    if (p.d == 64) {
        if (p.K <= 4) FSL_SFS(64, 4); else FSL_SFS(64, 8);
    } else {
        if (p.K <= 4) FSL_SFS(128, 4); else FSL_SFS(128, 8);
    }
#undef FSL_SFS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.d == 64)
        hipLaunchKernelGGL((select_fs_fixup_kernel<64>), grid, dim3(128), 0, st, (const uint16_t *)q, kbar, amax, sel,
                           w.fix, p);
    else
        hipLaunchKernelGGL((select_fs_fixup_kernel<128>), grid, dim3(128), 0, st, (const uint16_t *)q, kbar, amax, sel,
                           w.fix, p);
    return hipGetLastError();
}

}  // namespace fsl

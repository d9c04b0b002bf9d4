// FS-B selection: beam search over two causal forests of balanced trees
// (ai.info summary, "Methodology in Plain English", FS-B paragraph: a tree over
// the full prefix and one over the cells whose norm exceeds a threshold; nodes
// keep a mean key, a radius bounding their children, the largest cell norm and
// the earliest position; a beam of 16 nodes per level descends each tree under
// a provable upper bound of the cell score beneath a node; the union of the two
// beams is reranked by token-level log-sum-exp and the top K cells are read.
// FreeSolo digest, method step 5 and novelty: O(N log^2 N) including the
// radix-sort construction).
//
// Structure (the same readings as the oracle's FS-B):
//  - list 0 holds every complete cell, list 1 the cells with a_c > tau_h, both in
//    position order; every aligned segment [a 2^k, (a+1) 2^k) of a list holds a
//    perfect binary tree (heap order, leaves 2^k .. 2^(k+1) - 1) over the
//    segment's cells ordered by (code asc, list index asc), code a 32-bit sign
//    hash of the mean key over 32 given projections;
//  - a block whose prefix holds m entries of a list searches the segments of m's
//    binary decomposition: O(log N) trees of depth O(log N).
// Kernels: fsb_codes (one lane per projection, bits gathered by a ballot),
// fsb_lists (per head: the high-norm list and the count of high cells below each
// cell), fsb_tree (one launch per level k, one work-group per segment: the leaf
// order as the merge of the two sorted halves of level k - 1, which is the sorted
// order itself, then node means, norms, positions and radii) and fsb_search (one
// wave per query: beam search over both forests, token-level rerank, top K; with a
// beam of at most 16 both forests are searched at once, one per half of the wave;
// node means and key rows reach LDS a part of their dimensions at a time, through an
// 8 KB stage per wave, and the sort's lane exchanges within 16 lanes are DPP moves).
// Every decision is taken in fp64 with the oracle's operation order (explicit
// fused multiply-adds, sums left to right), so selections match it exactly; the
// rerank's exp and log may differ from the host's in the last place, which can
// only reorder cells whose log-sum-exp agree to about 15 digits.
#include <climits>

#include "fsl_internal.h"

namespace fsl {

namespace {

constexpr int kSearchWaves = 4;

__device__ __forceinline__ int64_t fsb_key(int T, int k, int64_t a, int64_t j) {
    return ((int64_t)T << 40) | ((int64_t)k << 34) | (a << (k + 1)) | j;
}

// "better" for beam candidates: larger bound, then smaller key
__device__ __forceinline__ bool cand_better(double u1, int64_t k1, double u2, int64_t k2) {
    return u1 > u2 || (u1 == u2 && k1 < k2);
}

}  // namespace

// ---- codes: bit 31 - b set iff proj_b . kbar_c > 0 (fp64 fma chain over x). A wave takes
// two cells, one lane per projection.
template <int D>
__global__ __launch_bounds__(256) void fsb_codes_kernel(const float *__restrict__ kbar, const float *__restrict__ proj,
                                                        uint32_t *__restrict__ codes, KParams p) {
    const int64_t cell2 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;  // (head, cell) pair index
    const int b = threadIdx.x & 31;
    const bool ok = cell2 < (int64_t)p.H * p.C;
    double dot = 0.0;
    if (ok) {
        const float *x = kbar + cell2 * D;
        for (int t = 0; t < D; ++t) dot = __fma_rn((double)proj[b * D + t], (double)x[t], dot);
    }
    const uint64_t bal = __ballot(ok && dot > 0.0);
    const uint32_t half = (threadIdx.x & 32) ? (uint32_t)(bal >> 32) : (uint32_t)bal;
    if (ok && b == 0) codes[cell2] = __builtin_bitreverse32(half);
}

// ---- list 1 (cells with a_c > tau_h, ascending) and hcount[c] = number of them below c
__global__ __launch_bounds__(1024) void fsb_lists_kernel(const float *__restrict__ amax, const float *__restrict__ tau,
                                                         int32_t *__restrict__ list1, int32_t *__restrict__ hcount,
                                                         KParams p) {
    __shared__ int s_wave[16];
    __shared__ int s_base;
    const int h = blockIdx.x;
    const double th = (double)tau[h];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_base = 0;
    __syncthreads();
    for (int64_t c0 = 0; c0 < p.C; c0 += 1024) {
        const int64_t c = c0 + tid;
        const bool hi = c < p.C && (double)amax[(int64_t)h * p.C + c] > th;
        const uint64_t bal = __ballot(hi);
        if (lane == 0) s_wave[wave] = __popcll(bal);
        __syncthreads();
        int before = s_base;
        for (int w2 = 0; w2 < wave; ++w2) before += s_wave[w2];
        const int pos = before + __popcll(bal & ((1ull << lane) - 1ull));
        if (c < p.C) {
            hcount[(int64_t)h * (p.C + 1) + c] = pos;
            if (hi) list1[(int64_t)h * p.C + pos] = (int32_t)c;
        }
        __syncthreads();
        if (tid == 0) {
            int tot = 0;
            for (int w2 = 0; w2 < 16; ++w2) tot += s_wave[w2];
            s_base += tot;
        }
        __syncthreads();
    }
    if (tid == 0) hcount[(int64_t)h * (p.C + 1) + p.C] = s_base;
}

// ---- trees of level k: one work-group per (head, forest, segment a). The leaf order is
// the merge of the two halves' orders (keys (code, list index) staged in LDS for segments of
// up to kTreeLds leaves, read from global memory beyond); the node means come from one pass
// over the merged leaves that keeps, per dimension, a running fp64 sum for each depth (the
// node of that depth holding the current leaf), so every sum still runs over its node's
// leaves left to right; largest norms and earliest positions, exact under any order, are
// taken bottom-up from the children.
constexpr int kTreeLds = 8192;
template <int D>
__global__ __launch_bounds__(256) void fsb_tree_kernel(const float *__restrict__ kbar, const float *__restrict__ cam,
                                                       const uint32_t *__restrict__ codes,
                                                       const int32_t *__restrict__ list1,
                                                       const int32_t *__restrict__ hcount, FsbWork w, int k,
                                                       KParams p) {
    extern __shared__ __attribute__((aligned(16))) uint64_t s_key[];  // [L] keys, then [L] merged leaves
    const int64_t nseg = p.C >> k;
    const int64_t g = blockIdx.x;
    const int h = (int)(g / (2 * nseg));
    const int T = (int)((g / nseg) % 2);
    const int64_t a = g % nseg;
    const int64_t len = T == 0 ? p.C : hcount[(int64_t)h * (p.C + 1) + p.C];
    if ((a + 1) << k > len) return;  // incomplete segment: no tree
    const int64_t L = (int64_t)1 << k;
    const bool in_lds = L <= kTreeLds;
    int32_t *s_leaf = reinterpret_cast<int32_t *>(s_key + (in_lds ? L : 0));
    const int tid = threadIdx.x;
    auto cell_of = [&](int64_t idx) -> int32_t { return T == 0 ? (int32_t)idx : list1[(int64_t)h * p.C + idx]; };
    int32_t *leaf = w.leaf + fsb_leaf(p, h, T, k, a, 0);
    // leaf order: (code, list index) ascending
    if (k == 0) {
        if (tid == 0) {
            leaf[0] = cell_of(a);
            if (in_lds) s_leaf[0] = leaf[0];
        }
    } else {
        // merge the two sorted halves (the leaves of segments 2a and 2a + 1 of level k - 1)
        const int32_t *lo = w.leaf + fsb_leaf(p, h, T, k - 1, 2 * a, 0);
        const int32_t *hi = w.leaf + fsb_leaf(p, h, T, k - 1, 2 * a + 1, 0);
        const int64_t half = L / 2;
        const uint32_t *hc = codes + (int64_t)h * p.C;
        // list index of a cell: the cell itself in list 0, its rank among high cells in list 1
        auto lidx = [&](int32_t c) -> int64_t { return T == 0 ? (int64_t)c : (int64_t)hcount[(int64_t)h * (p.C + 1) + c]; };
        if (in_lds) {
            // (code, list index) as one 64-bit key: list indices are below C < 2^31
            for (int64_t u = tid; u < L; u += 256) {
                const int32_t c = u < half ? lo[u] : hi[u - half];
                s_key[u] = ((uint64_t)hc[c] << 32) | (uint64_t)(uint32_t)lidx(c);
            }
            __syncthreads();
        }
        for (int64_t u = tid; u < L; u += 256) {
            const bool left = u < half;
            const int32_t c = left ? lo[u] : hi[u - half];
            int64_t lo_i = 0, hi_i = half;
            if (in_lds) {
                const uint64_t key = s_key[u];
                const uint64_t *other = s_key + (left ? half : 0);
                while (lo_i < hi_i) {
                    const int64_t mid = (lo_i + hi_i) >> 1;
                    if (other[mid] < key) lo_i = mid + 1; else hi_i = mid;
                }
            } else {
                const uint32_t cc = hc[c];
                const int64_t ci = lidx(c);
                const int32_t *other = left ? hi : lo;
                // number of the other half's keys below this one (keys are distinct)
                while (lo_i < hi_i) {
                    const int64_t mid = (lo_i + hi_i) >> 1;
                    const int32_t oc = other[mid];
                    const uint32_t ocode = hc[oc];
                    const bool below = ocode < cc || (ocode == cc && lidx(oc) < ci);
                    if (below) lo_i = mid + 1; else hi_i = mid;
                }
            }
            const int64_t at = (left ? u : u - half) + lo_i;
            leaf[at] = c;
            if (in_lds) s_leaf[at] = c;
        }
    }
    __syncthreads();
    const int32_t *lf = in_lds ? s_leaf : leaf;
    const int64_t nodes = 2 * L;
    float *mu = w.mu + fsb_node(p, h, T, k, a, 0) * D;
    double *rad = w.rad + fsb_node(p, h, T, k, a, 0);
    float *am = w.amax + fsb_node(p, h, T, k, a, 0);
    int32_t *pm = w.pmin + fsb_node(p, h, T, k, a, 0);
    // node means: thread (group gi, dim x) keeps the sums of depths gi, gi + NG, ... (node
    // j = 2^d + (u >> (k - d)) of depth d holds leaf u; it ends after leaf u when the
    // 2^(k - d) leaves of the node are in)
    {
        constexpr int NG = 256 / D;        // thread groups, one dimension per thread
        constexpr int kMaxDepth = 31;      // C < 2^31
        constexpr int DPT = (kMaxDepth + NG) / NG;  // depths per thread at most
        const int x = tid % D, gi = tid / D;
        double acc[DPT];
#pragma unroll
        for (int t = 0; t < DPT; ++t) acc[t] = 0.0;
        const float *kb = kbar + (int64_t)h * p.C * D + x;
        constexpr int UB = 8;  // leaves whose values are requested together
        for (int64_t u0 = 0; u0 < L; u0 += UB) {
            float vb[UB];
#pragma unroll
            for (int e = 0; e < UB; ++e) vb[e] = kb[(int64_t)lf[min(u0 + e, L - 1)] * D];
#pragma unroll
            for (int e = 0; e < UB; ++e) {
                const int64_t u = u0 + e;
                if (u >= L) break;
                const double v = (double)vb[e];
#pragma unroll
                for (int t = 0; t < DPT; ++t) {
                    const int d = gi + NG * t;
                    if (d > k) break;
                    acc[t] = __dadd_rn(acc[t], v);
                    const int64_t n = L >> d;
                    if (((u + 1) & (n - 1)) == 0) {
                        const int64_t j = ((int64_t)1 << d) + (u >> (k - d));
                        mu[j * D + x] = (float)__ddiv_rn(acc[t], (double)n);
                        acc[t] = 0.0;
                    }
                }
            }
        }
    }
    // largest norm and earliest position: the leaves, then each level from its children
    for (int64_t u = tid; u < L; u += 256) {
        const int32_t c = lf[u];
        am[L + u] = cam[(int64_t)h * p.C + c];
        pm[L + u] = c * p.s;
        rad[L + u] = 0.0;
    }
    __syncthreads();
    for (int depth = k - 1; depth >= 0; --depth) {
        for (int64_t j = ((int64_t)1 << depth) + tid; j < ((int64_t)2 << depth); j += 256) {
            am[j] = fmaxf(am[2 * j], am[2 * j + 1]);
            pm[j] = min(pm[2 * j], pm[2 * j + 1]);
        }
        __syncthreads();
    }
    // radii, from the level above the leaves to the root
    for (int depth = k - 1; depth >= 0; --depth) {
        for (int64_t j = ((int64_t)1 << depth) + tid; j < ((int64_t)2 << depth); j += 256) {
            double r2[2];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                const int64_t cj = 2 * j + ch;
                double acc = 0.0;
                for (int x = 0; x < D; ++x) {
                    const double e = __dsub_rn((double)mu[cj * D + x], (double)mu[j * D + x]);
                    acc = __fma_rn(e, e, acc);
                }
                r2[ch] = __dadd_rn(__dsqrt_rn(acc), rad[cj]);
            }
            rad[j] = __dmul_rn(r2[0] > r2[1] ? r2[0] : r2[1], 1.0 + 0x1p-40);
        }
        __syncthreads();
    }
}

// The value of lane (this lane xor j), for j = 1, 2, 4, 8 by DPP moves inside rows of 16
// lanes (quad permutes; xor 4 = half-row mirror then quad reverse; xor 8 = row mirror
// then half-row mirror), otherwise by a shuffle through LDS.
__device__ __forceinline__ int dpp_xor32(int x, int j) {
    if (j == 1) return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    if (j == 2) return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    if (j == 4) {
        const int y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
        return __builtin_amdgcn_update_dpp(0, y, 0x1B, 0xF, 0xF, false);          // quad_perm 3,2,1,0
    }
    if (j == 8) {
        const int y = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
        return __builtin_amdgcn_update_dpp(0, y, 0x141, 0xF, 0xF, false);         // row_half_mirror
    }
    return __shfl_xor(x, j);
}
__device__ __forceinline__ int64_t lane_xor(int64_t x, int j) {
    const int lo = dpp_xor32((int)(uint32_t)x, j), hi = dpp_xor32((int)(x >> 32), j);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double lane_xor(double x, int j) {
    return __longlong_as_double(lane_xor((int64_t)__double_as_longlong(x), j));
}

// ---- search: one wave per query
template <int D>
__global__ __launch_bounds__(64 * kSearchWaves) void fsb_search_kernel(const float *__restrict__ q32,
                                                                        const uint16_t *__restrict__ q16,
                                                                        const float *__restrict__ k32,
                                                                        const uint16_t *__restrict__ k16,
                                                                        const int32_t *__restrict__ hcount,
                                                                        FsbWork w, int beam, int32_t *__restrict__ sel,
                                                                        KParams p) {
    __shared__ double s_q[kSearchWaves][D];
    __shared__ double s_lse[kSearchWaves][64];
    __shared__ int32_t s_cell[kSearchWaves][64];
    // per wave (8 KB at d = 128, so that four work-groups fit a CU): node means (fp32) or
    // bf16 key rows, a part of their dimensions at a time, copied in before their dot products
    __shared__ __attribute__((aligned(16))) float s_stage[kSearchWaves][16 * D];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t nq = (p.N + kSearchWaves - 1) / kSearchWaves;
    const int h = (int)(blockIdx.x / nq);
    const int64_t i = (blockIdx.x % nq) * kSearchWaves + wave;
    if (i >= p.N) return;  // per-wave exit: no work-group barrier below
    const int64_t hN = (int64_t)h * p.N;
    const bool bf = q16 != nullptr;
    for (int x = lane; x < D; x += 64)
        s_q[wave][x] = bf ? (double)bf16_to_f32(q16[(hN + i) * D + x]) : (double)q32[(hN + i) * D + x];
    __builtin_amdgcn_wave_barrier();
    double qq = 0.0;
#pragma unroll 4
    for (int x = 0; x < D; ++x) qq = __fma_rn(s_q[wave][x], s_q[wave][x], qq);
    // the query stays in LDS (read at every use): held in registers it would take 2 D of them
    const double *qg = s_q[wave];
    const double qn = __dsqrt_rn(qq);
    const double sig = (double)p.sigma[h], lam = (double)p.lambda[h], rho = (double)p.rho;
    const int64_t nb = eligible_cells(p, i / p.B);
    const int lv = fsb_levels(p);
    // lanes sorted: a power of two covering the roots (at most lv) and a beam's children
    int sortw = 2;
    while (sortw < 64 && (sortw < 2 * beam || sortw < lv)) sortw <<= 1;
    float *st = s_stage[wave];
    // upper bound of the cell score under a node whose mean key waits in the stage (dims
    // 8 c .. 8 c + 3 at st[256 c + 4 l], 8 c + 4 .. at st[256 c + 128 + 4 l] for the l-th
    // lane of its round): the dot product one fma per coordinate, left to right
    // (dims 8 c .. 8 c + 7 of the chunks c0 .. c1 - 1 at st[g (c - c0) + 4 l] and
    // st[g (c - c0) + g / 2 + 4 l], g = 8 x the lanes of the round)
    auto dot_part = [&](double content, int c0, int c1, int g, int l) -> double {
        const double *qv = qg;
        asm volatile("" : "+v"(qv));
#pragma unroll 2
        for (int c = c0; c < c1; ++c) {
            const float4 m0 = *reinterpret_cast<const float4 *>(st + g * (c - c0) + 4 * l);
            const float4 m1 = *reinterpret_cast<const float4 *>(st + g * (c - c0) + g / 2 + 4 * l);
            content = __fma_rn(qv[8 * c], (double)m0.x, content);
            content = __fma_rn(qv[8 * c + 1], (double)m0.y, content);
            content = __fma_rn(qv[8 * c + 2], (double)m0.z, content);
            content = __fma_rn(qv[8 * c + 3], (double)m0.w, content);
            content = __fma_rn(qv[8 * c + 4], (double)m1.x, content);
            content = __fma_rn(qv[8 * c + 5], (double)m1.y, content);
            content = __fma_rn(qv[8 * c + 6], (double)m1.z, content);
            content = __fma_rn(qv[8 * c + 7], (double)m1.w, content);
        }
        return content;
    };
    auto bound_of = [&](double content, double rd, int32_t pm, float am) -> double {
        const double tt = __fma_rn(qn, rd, content);
        const double arg = __ddiv_rn(__dmul_rn(sig, (double)(i - (int64_t)pm)), 2.0 * (double)p.s);
        const double gg = arg >= 6.0 ? 1.0 : erf(arg);
        return __fma_rn(rho, tt, __dmul_rn(__dmul_rn(lam, (double)am), gg));
    };
    int nu = 0;  // distinct cells collected from the two beams (in s_cell)
    // a beam of up to 16 sorts within 32 lanes: then both forests are searched at once,
    // forest 0 in lanes 0..31 and forest 1 in lanes 32..63 (every shuffle of the sort
    // stays inside a half); wider beams search the forests one after the other
    const bool dual = sortw <= 32;
    const int hl = dual ? (lane & 31) : lane;  // the lane's place in its forest's group
    const int hbase = dual ? (lane & 32) : 0;  // the group's first lane
    for (int T0 = 0; T0 < (dual ? 1 : 2); ++T0) {
        const int T = dual ? (lane >> 5) : T0;
        // forest 1 covers the list-1 cells below nb (none below cell 0; with no cells at all
        // the counts are never computed, so they are not read then)
        const int64_t m = T == 0 ? nb : nb == 0 ? 0 : (int64_t)hcount[(int64_t)h * (p.C + 1) + nb];
        // this lane's candidate: forest level k, segment a, heap index j (j = 0: none);
        // fresh: its bound is still to be taken
        int ck = 0;
        int64_t ca = 0, cj = 0;
        {
            // roots: the segments of m's binary decomposition, largest first; lane r takes the r-th
            int64_t base = 0;
            int r = 0;
            for (int kk = lv - 1; kk >= 0; --kk)
                if ((m >> kk) & 1) {
                    if (r == hl) { ck = kk; ca = base >> kk; cj = 1; }
                    base += (int64_t)1 << kk;
                    ++r;
                }
        }
        bool fresh = cj != 0;
        double cu = -INFINITY;
        int64_t ckey = INT64_MAX;
        for (int iter = 0; iter < 64; ++iter) {
            if (__ballot(fresh) != 0ull) {
                // the fresh lanes' node means into the stage a part of their dims at a time,
                // their radii, norms and positions requested with them; other lanes name a
                // valid slot they do not use
                const int64_t mynode = fsb_node(p, h, T, fresh ? ck : 0, fresh ? ca : 0, fresh ? cj : 1);
                const double rd = w.rad[mynode];
                const int32_t pm = w.pmin[mynode];
                const float am = w.amax[mynode];
                double content = 0.0;
                if ((__ballot(fresh) >> 32) == 0ull) {
                    // lanes 0..31 only: two rounds of half the dims (32 node rows each)
                    const int64_t src_node = __shfl(mynode, lane & 31);
                    const float *src = w.mu + src_node * D + 4 * (lane >> 5);
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the stage are done
#pragma unroll
                        for (int c = 0; c < D / 16; ++c) lds_dma16(src + D / 2 * half + 8 * c, st + 256 * c);
                        wait_vmem();
                        __builtin_amdgcn_wave_barrier();
                        if (fresh) content = dot_part(content, D / 16 * half, D / 16 * (half + 1), 256, lane & 31);
                        __builtin_amdgcn_wave_barrier();
                    }
                } else {
                    // every lane: four rounds of a quarter of the dims (64 node rows of D / 4
                    // dims each), the dot product carried from round to round in coordinate order
                    constexpr int RC = D / 32;  // 8-dim chunks per round
                    const float *src = w.mu + mynode * D;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the stage are done
#pragma unroll
                        for (int c = 0; c < RC; ++c) {
                            lds_dma16(src + 8 * (RC * r + c), st + 512 * c);
                            lds_dma16(src + 8 * (RC * r + c) + 4, st + 512 * c + 256);
                        }
                        wait_vmem();
                        __builtin_amdgcn_wave_barrier();
                        if (fresh) content = dot_part(content, RC * r, RC * r + RC, 512, lane);
                        __builtin_amdgcn_wave_barrier();
                    }
                }
                if (fresh) {
                    cu = bound_of(content, rd, pm, am);
                    ckey = fsb_key(T, ck, ca, cj);
                }
            }
            // keep the beam best: bitonic sort of the lanes that can hold a candidate (the
            // roots, then a beam's children), best first, on (bound, key) alone; the key
            // names the node, which is read back from it after the sort
            auto stage = [&](int kk, int jj) __attribute__((always_inline)) {
                const double ou = lane_xor(cu, jj);
                const int64_t okey = lane_xor(ckey, jj);
                const bool lower = (lane & jj) == 0, up = (hl & kk) == 0;
                const bool ob = cand_better(ou, okey, cu, ckey);
                const bool take = (lower == up) ? ob : !ob;
                cu = take ? ou : cu;
                ckey = take ? okey : ckey;
            };
            if (sortw <= 32) {  // the usual width (beam <= 16): stages unrolled
#pragma unroll
                for (int kk = 2; kk <= 32; kk <<= 1)
#pragma unroll
                    for (int jj = kk >> 1; jj > 0; jj >>= 1)
                        if (kk <= sortw) stage(kk, jj);
            } else {
#pragma unroll 1
                for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll 1
                    for (int jj = kk >> 1; jj > 0; jj >>= 1) stage(kk, jj);
            }
            if (ckey == INT64_MAX) {
                cj = 0;
            } else {
                ck = (int)((ckey >> 34) & 63);
                const int64_t low = ckey & (((int64_t)1 << 34) - 1);
                ca = low >> (ck + 1);
                cj = low & (((int64_t)1 << (ck + 1)) - 1);
            }
            if (hl >= beam) { cj = 0; cu = -INFINITY; ckey = INT64_MAX; }
            const bool internal = cj != 0 && cj < ((int64_t)1 << ck);
            if (__ballot(internal) == 0ull) break;
            // expand: an internal beam node at place r of its group moves to its left child and
            // its right child goes to place beam + r (2 beam fits the group)
            const int src = hl - beam;
            const int srcl = hbase + (src < 0 ? 0 : src);
            const int64_t pj = __shfl(cj, srcl);
            const int pk = __shfl(ck, srcl);
            const int64_t pa = __shfl(ca, srcl);
            const bool p_int = __shfl((int)internal, srcl) != 0;
            fresh = false;
            if (hl < beam) {
                if (internal) {
                    cj = 2 * cj;
                    fresh = true;
                }
            } else if (src < beam && p_int) {
                ck = pk; ca = pa; cj = 2 * pj + 1;
                fresh = true;
            } else {
                cj = 0; cu = -INFINITY; ckey = INT64_MAX;
            }
        }
        // this forest's leaves into the union
        // (the beam ends on leaves; within one forest they are distinct cells, so a lane's
        // cell is checked only against the cells already collected, all lanes at once, and
        // the new ones are appended in lane order)
        const int32_t mycell = cj ? w.leaf[fsb_leaf(p, h, T, ck, ca, cj - ((int64_t)1 << ck))] : -1;
        // forest 0's leaves first, then forest 1's (both at once when searched together)
        for (int part = 0; part < (dual ? 2 : 1); ++part) {
            bool dup = mycell < 0 || (dual && (lane >> 5) != part);
            for (int u = 0; u < nu; ++u) dup |= s_cell[wave][u] == mycell;
            const uint64_t keep = __ballot(!dup);
            if (!dup) s_cell[wave][nu + __popcll(keep & ((1ull << lane) - 1))] = mycell;
            nu += __popcll(keep);
            __builtin_amdgcn_wave_barrier();
        }
    }
    // rerank: lse_c = log sum_j exp(scale q . k_j) over the cell's tokens (token dots one per lane)
    const int S = p.s;
    if (bf) {
        // 64 / S cells at a time: their key rows copied into the stage half the dims at a time
        // (16-byte piece c of a round's row r at c ^ (r mod pieces per round row)), then one
        // row per lane, the dot product carried from the first half to the second
        constexpr int HP = D / 16;     // 16-byte pieces of a row per round
        constexpr int RPI = 64 / HP;   // rows per copy instruction
        uint16_t *st16 = reinterpret_cast<uint16_t *>(st);
        const int cps = 64 / S;
        for (int u0 = 0; u0 < nu; u0 += cps) {
            const int uu = u0 + lane / S;
            double dot = 0.0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the stage are done
#pragma unroll
                for (int ii = 0; ii < 64 / RPI; ++ii) {
                    const int row = RPI * ii + lane / HP, pos = lane % HP;
                    const int uc = min(u0 + row / S, nu - 1);
                    const int64_t tok = hN + (int64_t)s_cell[wave][uc] * S + row % S;
                    lds_dma16(k16 + tok * D + 8 * (HP * half + (pos ^ (row & (HP - 1)))), st16 + 512 * ii);
                }
                wait_vmem();
                __builtin_amdgcn_wave_barrier();
                if (uu < nu) {
                    const double *qv = qg + D / 2 * half;
                    asm volatile("" : "+v"(qv));
#pragma unroll 2
                    for (int c = 0; c < HP; ++c) {
                        const uint4 r4 =
                            *reinterpret_cast<const uint4 *>(st16 + lane * (D / 2) + 8 * (c ^ (lane & (HP - 1))));
                        const uint32_t w4[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            dot = __fma_rn(qv[8 * c + 2 * t], (double)__uint_as_float(w4[t] << 16), dot);
                            dot = __fma_rn(qv[8 * c + 2 * t + 1], (double)__uint_as_float(w4[t] & 0xFFFF0000u), dot);
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
            const double l = uu < nu ? __dmul_rn((double)p.scale, dot) : -INFINITY;
            double mx = l;
            for (int o = 1; o < S; o <<= 1) {
                const double ov = __shfl_xor(mx, o);
                mx = ov > mx ? ov : mx;
            }
            const double e = uu < nu ? exp(__dsub_rn(l, mx)) : 0.0;
            // the sum in token order, as the oracle takes it
            double sum = 0.0;
            for (int t = 0; t < S; ++t) sum = __dadd_rn(sum, __shfl(e, (lane / S) * S + t));
            if (uu < nu && lane % S == 0) s_lse[wave][uu] = __dadd_rn(mx, log(sum));
        }
    }
    for (int u = 0; u < (bf ? 0 : nu); ++u) {
        const int32_t c = s_cell[wave][u];
        double l = -INFINITY;
        if (lane < S) {
            // the token's key row 16 bytes at a time, one fma per coordinate, left to right
            const int64_t row = (hN + (int64_t)c * S + lane) * D;
            const double *qv = qg;
            asm volatile("" : "+v"(qv));
            double dot = 0.0;
            if (bf) {
                const uint4 *kr = reinterpret_cast<const uint4 *>(k16 + row);
#pragma unroll 2
                for (int x8 = 0; x8 < D / 8; ++x8) {
                    const uint4 r4 = kr[x8];
                    const uint32_t w4[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        dot = __fma_rn(qv[8 * x8 + 2 * t], (double)__uint_as_float(w4[t] << 16), dot);
                        dot = __fma_rn(qv[8 * x8 + 2 * t + 1], (double)__uint_as_float(w4[t] & 0xFFFF0000u), dot);
                    }
                }
            } else {
                const float4 *kr = reinterpret_cast<const float4 *>(k32 + row);
#pragma unroll 4
                for (int x4 = 0; x4 < D / 4; ++x4) {
                    const float4 f4 = kr[x4];
                    dot = __fma_rn(qv[4 * x4], (double)f4.x, dot);
                    dot = __fma_rn(qv[4 * x4 + 1], (double)f4.y, dot);
                    dot = __fma_rn(qv[4 * x4 + 2], (double)f4.z, dot);
                    dot = __fma_rn(qv[4 * x4 + 3], (double)f4.w, dot);
                }
            }
            l = __dmul_rn((double)p.scale, dot);
        }
        double mx = l;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double ov = __shfl_xor(mx, o);
            mx = ov > mx ? ov : mx;
        }
        const double e = lane < S ? exp(__dsub_rn(l, mx)) : 0.0;
        // the sum in token order, as the oracle takes it
        double sum = 0.0;
        for (int t = 0; t < S; ++t) sum = __dadd_rn(sum, __shfl(e, t));
        if (lane == 0) s_lse[wave][u] = __dadd_rn(mx, log(sum));
    }
    __builtin_amdgcn_wave_barrier();
    // top K by (lse desc, cell asc), written ascending
    double lu = lane < nu ? s_lse[wave][lane] : -INFINITY;
    int32_t lc = lane < nu ? s_cell[wave][lane] : INT_MAX;
#pragma unroll
    for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            const double ou = __shfl_xor(lu, jj);
            const int32_t oc = __shfl_xor(lc, jj);
            const bool lower = (lane & jj) == 0, up = (lane & kk) == 0;
            const bool ob = ou > lu || (ou == lu && oc < lc);
            const bool take = (lower == up) ? ob : !ob;
            lu = take ? ou : lu;
            lc = take ? oc : lc;
        }
    const int nsel = nu < p.K ? nu : p.K;
    // ascending order of the K best: sort their cells
    int32_t key = lane < nsel ? lc : INT_MAX;
#pragma unroll
    for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            const int32_t ok2 = __shfl_xor(key, jj);
            const bool lower = (lane & jj) == 0, up = (lane & kk) == 0;
            const bool take = (lower == up) ? (ok2 < key) : !(ok2 < key);
            key = take ? ok2 : key;
        }
    if (lane < p.K) sel[(hN + i) * p.K + lane] = lane < nsel ? key : -1;
}

hipError_t launch_fsb_select(const void *q, const void *k, const float *kbar, const float *amax, int32_t *sel,
                             const FsbWork &w, const float *tau, const float *proj, int beam, const KParams &p,
                             hipStream_t st) {
    if (p.C > 0) {
        const int64_t lanes = (int64_t)p.H * p.C * 32;
        const unsigned g = (unsigned)((lanes + 255) / 256);
        if (p.d == 64)
            hipLaunchKernelGGL((fsb_codes_kernel<64>), dim3(g), dim3(256), 0, st, kbar, proj, w.codes, p);
        else
            hipLaunchKernelGGL((fsb_codes_kernel<128>), dim3(g), dim3(256), 0, st, kbar, proj, w.codes, p);
        hipLaunchKernelGGL(fsb_lists_kernel, dim3((unsigned)p.H), dim3(1024), 0, st, amax, tau, w.list1, w.hcount, p);
        const int lv = fsb_levels(p);
        for (int kk = 0; kk < lv; ++kk) {
            const unsigned grid = (unsigned)((int64_t)p.H * 2 * (p.C >> kk));
            const int64_t lk = (int64_t)1 << kk;
            const size_t lds = lk <= kTreeLds ? (size_t)lk * (sizeof(uint64_t) + sizeof(int32_t)) : 0;
            if (p.d == 64)
                hipLaunchKernelGGL((fsb_tree_kernel<64>), dim3(grid), dim3(256), lds, st, kbar, amax, w.codes, w.list1,
                                   w.hcount, w, kk, p);
            else
                hipLaunchKernelGGL((fsb_tree_kernel<128>), dim3(grid), dim3(256), lds, st, kbar, amax, w.codes, w.list1,
                                   w.hcount, w, kk, p);
        }
    }
    const bool bf = p.dtype == FSL_BF16;
    const unsigned grid = (unsigned)(((p.N + kSearchWaves - 1) / kSearchWaves) * p.H);
    const float *q32 = bf ? nullptr : (const float *)q;
    const uint16_t *q16 = bf ? (const uint16_t *)q : nullptr;
    const float *k32 = bf ? nullptr : (const float *)k;
    const uint16_t *k16 = bf ? (const uint16_t *)k : nullptr;
    if (p.d == 64)
        hipLaunchKernelGGL((fsb_search_kernel<64>), dim3(grid), dim3(64 * kSearchWaves), 0, st, q32, q16, k32, k16,
                           w.hcount, w, beam, sel, p);
    else
        hipLaunchKernelGGL((fsb_search_kernel<128>), dim3(grid), dim3(64 * kSearchWaves), 0, st, q32, q16, k32, k16,
                           w.hcount, w, beam, sel, p);
    return hipGetLastError();
}

}  // namespace fsl

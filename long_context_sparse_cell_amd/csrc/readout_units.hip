// Long-branch readout for bf16 inputs (FreeSolo digest, core method and step 6:
// an unrotated softmax over the raw tokens of each query's selected cells),
// computed cell by cell over gathered queries.
//
// Queries are taken in spans of 256 (128 when K > 4), two 128-query blocks of
// one head. Neighbouring blocks select mostly the same cells (their pools share
// the high-norm cells and all but four of the recent ones), so a span reads
// each of its cells once for both blocks.
//
// readout_plan_kernel lists, per span, every selected cell (a "task", in no
// particular order) and the (query, rank) pairs that chose it (rank = the cell's
// position in the query's ascending selection), cut into units of at most 16 pairs. The list is written
// as one record that readout_units_kernel copies into LDS.
//
// In readout_units_kernel each wave owns one LDS slot and walks its share of
// the span's tasks. For a task it copies the cell's keys (raw bf16 rows) and
// values (fp16, transposed per 32-token group in vt_pos order, from
// kv_prep.hip) straight into its slot (global_load_lds), reads them into
// registers, issues the copy of its next task and then, for each unit of the
// task, computes S^T = K Q^T over the unit's gathered queries (bf16 MFMA, exact
// products; the span's queries wait in LDS), each query's softmax over the
// cell's s tokens (exact column maximum, fp16 weights rounded to nearest with
// the denominator summing the rounded weights) and O^T = V^T P^T (fp16 MFMA).
// Every product is needed: no query tile carries rows for queries that did not
// select the cell. Waves never wait for each other after the setup.
//
// Per (query, rank) a unit writes the cell's normalised output O / l in fp16
// and lambda = m + log2(l) (m the scaled maximum in base-2 units, l the sum of
// weights). The local-branch kernel (window_bf16.hip) merges a query's cells by
// these log-sum-exp weights, which gives the softmax over the union of the
// cells' tokens, then applies RMSNorm and the mix. A query's result depends only
// on its own cells, each computed the same way whatever the unit's other
// queries, so the output is deterministic.

#include "fsl_internal.h"

namespace fsl {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

union R8 {
    uint4 u;
    uint2 d[2];
    bf16x8 b;
    halfx8 h;
};

constexpr int kPlanThreads = 256;

// waves per work-group: as many one-cell slots as fit in LDS next to the span's
// queries and the plan record
template <int D, int S>
constexpr int ru_waves() {
    constexpr int slot = (S * D + (S < 32 ? 32 : S) * D) * 2;
    constexpr int budget = 160 * 1024 - kSpanQ * D * 2 - kPlanRecBytes - 1024;
    constexpr int n = budget / slot;
    return n > 8 ? 8 : n;
}

}  // namespace

// One work-group per (head, span): the span's selected cells and their
// (query, rank) pairs, grouped by cell and cut into units of at most 16 pairs.
// Cells are gathered in an LDS hash table (open addressing, at most half full);
// the order of the tasks, and of the pairs inside a cell's list, depends on the
// order of the atomics but changes no result: every (query, rank) partial is
// computed the same way whichever unit or wave computes it.
__global__ __launch_bounds__(kPlanThreads) void readout_plan_kernel(const int32_t *__restrict__ sel,
                                                                    uint32_t *__restrict__ plan, KParams p, int QR) {
    constexpr int TAB = 2 * kPlanMaxPairs;   // hash slots
    constexpr int PER = kPlanMaxPairs / kPlanThreads;  // pairs per thread
    __shared__ int s_key[TAB];     // cell in the slot, -1 when empty
    __shared__ int s_cnt[TAB];     // pairs of the slot's cell, then the fill cursor
    __shared__ int s_start[TAB];   // first pair of the slot's cell
    __shared__ int s_wsum[kPlanThreads / 64][2];
    const int nspan = (int)((p.N + QR - 1) / QR);
    const int h = (int)blockIdx.x / nspan;
    const int64_t q0 = (int64_t)((int)blockIdx.x % nspan) * QR;
    const int nq = (int)min((int64_t)QR, p.N - q0);
    const int K = p.K;
    const int nent = nq * K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *ssel = sel + ((int64_t)h * p.N + q0) * K;
    uint32_t *rec = plan + (int64_t)blockIdx.x * (kPlanRecBytes / 4);
    uint16_t *rpair = reinterpret_cast<uint16_t *>(rec + kPlanPairWord);
    static_assert(kPlanMaxPairs % kPlanThreads == 0 && TAB % kPlanThreads == 0, "whole per-thread shares");

    // this thread's pairs tid + kPlanThreads j (all loads in flight at once)
    int cj[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int pr = tid + kPlanThreads * j;
        cj[j] = pr < nent ? ssel[pr] : -1;
    }
#pragma unroll
    for (int j = 0; j < TAB / kPlanThreads; ++j) {
        s_key[tid + kPlanThreads * j] = -1;
        s_cnt[tid + kPlanThreads * j] = 0;
    }
    __syncthreads();
    int slot[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        slot[j] = -1;
        if (cj[j] < 0) continue;
        int sl = (int)(((uint32_t)cj[j] * 2654435761u) >> 21) & (TAB - 1);
        while (true) {
            const int old = atomicCAS(&s_key[sl], -1, cj[j]);
            if (old == -1 || old == cj[j]) break;
            sl = (sl + 1) & (TAB - 1);
        }
        slot[j] = sl;
        atomicAdd(&s_cnt[sl], 1);
    }
    __syncthreads();
    // exclusive scans over the slots of (tasks, pairs, units); thread t owns slots
    // TAB/kPlanThreads t .. + TAB/kPlanThreads - 1
    constexpr int SPT = TAB / kPlanThreads;
    int nt = 0, npair = 0, nunit = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int c = s_cnt[SPT * tid + j];
        nt += c > 0;
        npair += c;
        nunit += (c + 15) >> 4;
    }
    int it = nt, ip = npair, iu = nunit;  // inclusive scans within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int a = __shfl_up(it, o), b = __shfl_up(ip, o), u = __shfl_up(iu, o);
        if (lane >= o) {
            it += a;
            ip += b;
            iu += u;
        }
    }
    __shared__ int s_wt[kPlanThreads / 64];
    if (lane == 63) {
        s_wt[wave] = it;
        s_wsum[wave][0] = ip;
        s_wsum[wave][1] = iu;
    }
    __syncthreads();
    int bt = 0, bp = 0, bu = 0;
    for (int w2 = 0; w2 < wave; ++w2) {
        bt += s_wt[w2];
        bp += s_wsum[w2][0];
        bu += s_wsum[w2][1];
    }
    int tk = bt + it - nt, pk = bp + ip - npair, uk = bu + iu - nunit;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int sl = SPT * tid + j;
        const int c = s_cnt[sl];
        if (c == 0) continue;
        const int nu = (c + 15) >> 4;
        s_start[sl] = pk;
        rec[kPlanTaskWord + 2 * tk] = (uint32_t)s_key[sl];
        rec[kPlanTaskWord + 2 * tk + 1] = ((uint32_t)uk << 16) | (uint32_t)nu;
        for (int u = 0; u < nu; ++u)
            rec[kPlanUnitWord + uk + u] = ((uint32_t)(pk + 16 * u) << 16) | (uint32_t)min(16, c - 16 * u);
        ++tk;
        pk += c;
        uk += nu;
    }
    if (tid == kPlanThreads - 1) {
        rec[0] = (uint32_t)tk;
        rec[1] = (uint32_t)uk;
        rec[2] = (uint32_t)pk;
        rec[3] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPT; ++j) s_cnt[SPT * tid + j] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (slot[j] < 0) continue;
        const int pr = tid + kPlanThreads * j;
        const int at = s_start[slot[j]] + atomicAdd(&s_cnt[slot[j]], 1);
        rpair[at] = (uint16_t)(((pr / K) << 3) | (pr % K));
    }
}

template <int D, int S, int NW>
__global__ __launch_bounds__(NW * 64) void readout_units_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ vt,
    const uint32_t *__restrict__ plan, uint16_t *__restrict__ part, float *__restrict__ plse, KParams p, int QR,
    int span0, int nspan_run) {
    constexpr int NT = S / 16;                       // 16-token score tiles per cell
    constexpr int KK = (NT + 1) / 2;                 // 32-token value groups per cell
    constexpr int QS = D / 32;                       // MFMA k-steps over d
    constexpr int CPR = D / 8;                       // 16-byte chunks per row
    constexpr int CELL = S * D;                      // key elements of a cell
    constexpr int VCELL = (S < 32 ? 32 : S) * D;     // value elements of the groups holding a cell
    constexpr int SLOT = CELL + VCELL;
    constexpr int KUNITS = CELL * 2 / 1024;          // 1 KB copies: keys, then values
    constexpr int VUNITS = VCELL * 2 / 1024;
    constexpr int KOPS = NT * QS;                    // 16-byte key operands per lane
    constexpr int VOPS = KK * (D / 16);              // 16-byte value operands per lane
    static_assert(KUNITS >= 1 && VUNITS >= 1, "whole 1 KB copy units");

    __shared__ __attribute__((aligned(1024))) uint16_t s_q[kSpanQ * D];
    __shared__ __attribute__((aligned(1024))) uint32_t s_rec[kPlanRecBytes / 4];
    __shared__ __attribute__((aligned(1024))) uint16_t s_slot[NW][SLOT];

    const int nspan = (int)((p.N + QR - 1) / QR);
    const int logical = xcd_remap((int)blockIdx.x, nspan_run * p.H);
    const int h = logical / nspan_run;
    const int span = span0 + logical % nspan_run;
    const int64_t q0 = (int64_t)span * QR;
    const int nq = (int)min((int64_t)QR, p.N - q0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int K = p.K;
    const int64_t hN = (int64_t)h * p.N;
    const float sl2 = p.scale * 1.4426950408889634f;

    // ---- the span's queries and its plan into LDS. Query rows past nq repeat the
    // last one; chunk c of row r sits at c ^ swz_key(r) so that the gathered
    // operand reads spread over the banks.
    for (int u = wave; u < kSpanQ * D * 2 / 1024; u += NW) {
        const int s = u * 64 + lane;  // 16-byte slot
        const int row = s / CPR, pc = s % CPR;
        const int64_t src = (hN + q0 + min(row, max(nq - 1, 0))) * D + 8 * (pc ^ swz_key(row, D));
        lds_dma16(q + src, s_q + 512 * u);
    }
    const uint32_t *rec = plan + ((int64_t)h * nspan + span) * (kPlanRecBytes / 4);
    for (int u = wave; u < kPlanRecBytes / 1024; u += NW) lds_dma16(rec + 256 * u + 4 * lane, s_rec + 256 * u);
    wait_vmem();
    __syncthreads();
    const int ntask = (int)s_rec[0];
    const uint16_t *s_pair = reinterpret_cast<const uint16_t *>(s_rec + kPlanPairWord);

    // ---- one wave, one slot: copy, read into registers, refill, compute
    uint16_t *slot = s_slot[wave];
    const uint16_t *vth = vt + h * vt_head_elems(p);
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int64_t cell = (int)s_rec[kPlanTaskWord + 2 * t];
#pragma unroll
        for (int i = 0; i < KUNITS; ++i) {
            const int s = i * 64 + lane;
            const int row = s / CPR, pc = s % CPR;
            lds_dma16(k + (hN + cell * S) * D + row * D + 8 * (pc ^ swz_key(row, D)), slot + 512 * i);
        }
#pragma unroll
        for (int i = 0; i < VUNITS; ++i) {
            const int s = i * 64 + lane;
            const int r = s >> 2, pg = s & 3;  // r = group * D + dim
            lds_dma16(vth + (cell * S / 32) * (32 * D) + r * 32 + 8 * (pg ^ swz_val(r % D)), slot + CELL + 512 * i);
        }
    };

    int t = wave;
    if (t < ntask) issue(t);
    for (; t < ntask; t += NW) {
        const int cell = (int)s_rec[kPlanTaskWord + 2 * t];
        const uint32_t td = s_rec[kPlanTaskWord + 2 * t + 1];
        const int u0 = (int)(td >> 16), nu = (int)(td & 0xFFFFu);
        wait_vmem_le<0>();  // this wave's copy of the cell has landed
        R8 kop[KOPS], vop[VOPS];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) {
                const int row = 16 * tt + col;
                kop[tt * QS + ks].u =
                    *reinterpret_cast<const uint4 *>(&slot[row * D + 8 * ((4 * ks + g) ^ swz_key(row, D))]);
            }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const int dim = 16 * dt + col;
                vop[kk * (D / 16) + dt].u =
                    *reinterpret_cast<const uint4 *>(&slot[CELL + ((kk * D + dim) * 4 + (g ^ swz_val(dim))) * 8]);
            }
        // every read of the slot is complete before the next task's copy may overwrite it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (t + NW < ntask) issue(t + NW);

        for (int ui = 0; ui < nu; ++ui) {
            const uint32_t ud = s_rec[kPlanUnitWord + u0 + ui];
            const int first = (int)(ud >> 16), np = (int)(ud & 0xFFFFu);
            const uint32_t pe = s_pair[first + min(col, np - 1)];
            const int ql = (int)(pe >> 3), rank = (int)(pe & 7);
            R8 qop[QS];
#pragma unroll
            for (int ks = 0; ks < QS; ++ks)
                qop[ks].u = *reinterpret_cast<const uint4 *>(&s_q[ql * D + 8 * ((4 * ks + g) ^ swz_key(ql, D))]);
            floatx4 sacc[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                sacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < QS; ++ks)
                    sacc[tt] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[tt * QS + ks].b, qop[ks].b, sacc[tt], 0, 0, 0);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[tt][r]);
            const float m = colmax4(mx) * sl2;  // the exact maximum: the largest weight is 1
            R8 pb[KK];
            float lsum = 0.0f;
#pragma unroll
            for (int tt = 0; tt < 2 * KK; ++tt) {
                uint32_t lo = 0u, hi = 0u;
                if (tt < NT) {
                    float e[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) e[r] = exp2_hw(fmaf(sacc[tt][r], sl2, -m));
                    lo = pk_f16_rne_acc(e[0], e[1], lsum);
                    hi = pk_f16_rne_acc(e[2], e[3], lsum);
                }
                pb[tt >> 1].d[tt & 1] = make_uint2(lo, hi);
            }
            if constexpr (S == 16) {
                // a 16-token cell is one half of its value group: move its weights to the
                // k-slots of that half (slots 4..7 for an odd cell)
                if (cell & 1) {
                    pb[0].d[1] = pb[0].d[0];
                    pb[0].d[0] = make_uint2(0u, 0u);
                }
            }
            floatx4 oacc[D / 16];
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
                    oacc[dt] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[kk * (D / 16) + dt].h, pb[kk].h, oacc[dt], 0, 0, 0);
            const float l = colsum4(lsum);
            const float inv = 1.0f / l;
            if (col < np) {
                // the lane's dimensions 16 dt + 4 g + r go to element 32 (dt / 2) + 8 g +
                // 4 (dt % 2) + r of the row, so that each store instruction writes 64
                // contiguous bytes per query
                const int64_t pr = (hN + q0 + ql) * K + rank;
                uint16_t *dst = part + pr * D + 8 * g;
#pragma unroll
                for (int dt = 0; dt < D / 16; dt += 2) {
                    union {
                        halfx8 h;
                        u32x4 u;
                    } w;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        w.h[r] = (_Float16)(oacc[dt][r] * inv);
                        w.h[4 + r] = (_Float16)(oacc[dt + 1][r] * inv);
                    }
                    *reinterpret_cast<u32x4 *>(dst + 16 * dt) = w.u;
                }
                if (g == 0) plse[pr] = m + __log2f(l);
            }
        }
    }
    wait_vmem();  // no copy into LDS may outlive the work-group
}

template <int D, int S>
static void launch_ru(dim3 grid, hipStream_t st, const void *q, const void *k, const uint16_t *vt,
                      const uint32_t *plan, uint16_t *part, float *plse, const KParams &p, int QR, int span0,
                      int nspan_run) {
    constexpr int NW = ru_waves<D, S>();
    static_assert(NW >= 2, "at least two waves");
    hipLaunchKernelGGL((readout_units_kernel<D, S, NW>), grid, dim3(NW * 64), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, vt, plan, part, plse, p, QR, span0, nspan_run);
}

hipError_t launch_readout_units(const void *q, const void *k, const uint16_t *vt, const int32_t *sel,
                                uint32_t *plan, uint16_t *part, float *plse, const KParams &p, int64_t qa,
                                int64_t qb, hipStream_t st) {
    const int QR = span_queries(p);
    const int nspan = (int)((p.N + QR - 1) / QR);
    hipLaunchKernelGGL(readout_plan_kernel, dim3((unsigned)(nspan * p.H)), dim3(kPlanThreads), 0, st, sel, plan, p,
                       QR);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int span0 = (int)(qa / QR);
    const int nrun = (int)((qb + QR - 1) / QR) - span0;
    if (nrun <= 0) return hipSuccess;
    dim3 grid((unsigned)(nrun * p.H));
#define FSL_RU(DD, SS) launch_ru<DD, SS>(grid, st, q, k, vt, plan, part, plse, p, QR, span0, nrun)
    if (p.d == 64) {
        if (p.s == 16) FSL_RU(64, 16); else if (p.s == 32) FSL_RU(64, 32); else FSL_RU(64, 64);
    } else {
        if (p.s == 16) FSL_RU(128, 16); else if (p.s == 32) FSL_RU(128, 32); else FSL_RU(128, 64);
    }
#undef FSL_RU
    return hipGetLastError();
}

}  // namespace fsl

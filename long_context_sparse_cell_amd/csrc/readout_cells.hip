// Long-branch readout for bf16 inputs without pruning (P = -1: FS, and the FS-B
// forward), after the FreeSolo digest, core method and step 6: an unrotated
// softmax over the raw tokens of each query's selected cells, computed cell by
// cell over gathered queries. Without the norm prune a block's queries choose
// hundreds of distinct cells, so the span readout (readout_units.hip) would fill
// its 16-query units with one or two queries each; here each head's pairs are
// listed by cell, and a cell's units gather its queries from a whole super-span.
//
// The selections are first turned into lists of the (query, rank) pairs that
// chose each cell (rank = the cell's position in the query's ascending
// selection), one list per (head, super-span of consecutive spans, cell), in that
// order: a stretch of the lists then reads the queries of one super-span, which
// stay in the L2, and each cell is read once per super-span:
//   ro_zero_kernel       clears the per-cell counters
//   ro_span_kernel<0>    per span of queries (256, or 128 when K > 4): the span's
//                        distinct cells in an LDS hash table, their pair counts
//                        added to the cells' counters
//   launch_scan_u32      the counters become list offsets (sort.hip)
//   ro_span_kernel<1>    the same spans again: each cell of the span takes a run of
//                        its list with one atomic and writes the span's pairs there
// The order of the spans inside a cell's list, and of the pairs inside a span's
// run, follows the atomics; it changes no result, because every (query, rank)
// partial is computed the same way whichever unit or wave computes it.
//
// readout_cells_kernel then walks the lists in items of kRoItem entries, one
// wave per item. Consecutive entries of one cell form a run, computed in units of
// at most 16 pairs: S^T = K Q^T (bf16 MFMA, exact products) with the run's keys
// (raw bf16 rows) and the unit's queries read straight from global memory into
// the MFMA operand registers, each query's softmax over the cell's s tokens
// (exact column maximum, fp16 weights rounded to nearest with the denominator
// summing the rounded weights) and O^T = V^T P^T (fp16 MFMA) with the values
// (fp16, transposed per 32-token group in vt_pos order, from kv_prep.hip). The
// queries of a unit are loaded two units ahead and the next run's keys and values
// as soon as the current run's last unit has used them; every unit issues the
// same memory instructions, so the compiler's waits can let them overlap. (An LDS
// copy of each cell made the compiler wait for every outstanding memory access
// before each unit.) A cell's keys and values are read once per run, so a cell
// chosen by many queries of a super-span is read about once per kRoItem of its
// pairs there, and no product is computed for a query that did not select it.
//
// Per (query, rank) a unit writes the cell's normalised output O / l in fp16
// and lambda = m + log2(l) (m the scaled maximum in base-2 units, l the sum of
// weights), in the same places as the span readout (readout_units.hip), which
// the local-branch kernel (window_bf16.hip) merges. A query's result depends only
// on its own cells, so the output is deterministic.

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

}  // namespace

__global__ __launch_bounds__(256) void ro_zero_kernel(uint32_t *__restrict__ cnt, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) cnt[i] = 0u;
}

// One work-group per (head, span). The span's selected cells are gathered in an
// LDS hash table (open addressing, at most half full) with their pair counts.
// Count pass: the counts are added to the cells' counters. Scatter pass (the
// counters now hold list offsets): each cell takes a run of its list with one
// atomic and the span's pairs are written there as (counter index, pair), the
// counter of (head, super-span, cell) at (head * supers + super) * C + cell.
template <bool SCATTER>
__global__ __launch_bounds__(kPlanThreads) void ro_span_kernel(const int32_t *__restrict__ sel,
                                                               uint32_t *__restrict__ cnt,
                                                               const uint32_t *__restrict__ tot,
                                                               uint2 *__restrict__ list, KParams p, int QR) {
    constexpr int TAB = 2 * kPlanMaxPairs;             // hash slots
    constexpr int PER = kPlanMaxPairs / kPlanThreads;  // pairs per thread
    constexpr int SPT = TAB / kPlanThreads;            // slots per thread
    __shared__ int s_key[TAB];        // cell in the slot, -1 when empty
    __shared__ uint32_t s_cnt[TAB];   // pairs of the slot's cell, then the fill cursor
    __shared__ uint32_t s_base[TAB];  // list position of the slot's first pair
    static_assert(kPlanMaxPairs % kPlanThreads == 0 && TAB % kPlanThreads == 0, "whole per-thread shares");
    const int nspan = (int)((p.N + QR - 1) / QR);
    const int h = (int)blockIdx.x / nspan;
    const int span = (int)blockIdx.x % nspan;
    const int64_t q0 = (int64_t)span * QR;
    const int nq = (int)min((int64_t)QR, p.N - q0);
    const int nent = nq * p.K;
    const int tid = threadIdx.x;
    const int64_t pr0 = ((int64_t)h * p.N + q0) * p.K;
    const int64_t cbase = ((int64_t)h * ro_supers(p) + span / ro_spans_per_super(p)) * p.C;

    // this thread's pairs tid + kPlanThreads j (all loads in flight at once)
    int cj[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = tid + kPlanThreads * j;
        cj[j] = e < nent ? sel[pr0 + e] : -1;
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        s_key[tid + kPlanThreads * j] = -1;
        s_cnt[tid + kPlanThreads * j] = 0u;
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
        atomicAdd(&s_cnt[sl], 1u);
    }
    __syncthreads();
    if (!SCATTER) {
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int sl = SPT * tid + j;
            const uint32_t c = s_cnt[sl];
            if (c) atomicAdd(&cnt[cbase + s_key[sl]], c);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int sl = SPT * tid + j;
        const uint32_t c = s_cnt[sl];
        if (c) {
            const int64_t cid = cbase + s_key[sl];
            s_base[sl] = atomicAdd(&cnt[cid], c) + tot[cid / kSortScanBlock];
        }
        s_cnt[sl] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (slot[j] < 0) continue;
        const uint32_t at = s_base[slot[j]] + atomicAdd(&s_cnt[slot[j]], 1u);
        list[at] = make_uint2((uint32_t)(cbase + cj[j]), (uint32_t)(pr0 + tid + kPlanThreads * j));
    }
}

// One wave per item of kRoItem list entries (items past the list's end exit).
template <int D, int S>
__global__ __launch_bounds__(64, (D == 128 || S == 64) ? 2 : 3) void readout_cells_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ vt,
    const uint2 *__restrict__ list, const uint32_t *__restrict__ cnt, const uint32_t *__restrict__ tot,
    uint16_t *__restrict__ part, float *__restrict__ plse, KParams p) {
    constexpr int NT = S / 16;                       // 16-token score tiles per cell
    constexpr int KK = (NT + 1) / 2;                 // 32-token value groups per cell
    constexpr int QS = D / 32;                       // MFMA k-steps over d
    constexpr int KOPS = NT * QS;                    // 16-byte key operands per lane
    constexpr int VOPS = KK * (D / 16);              // 16-byte value operands per lane
    constexpr int NB = kRoItem / 64;                 // entries per lane
    static_assert(kRoItem % 64 == 0, "whole 64-entry pieces per item");

    const int64_t cells = ro_count_words(p) - 1;  // the sentinel counter's offset is the list length
    const int64_t total = (int64_t)cnt[cells] + tot[cells / kSortScanBlock];
    const int item = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int64_t e0 = (int64_t)item * kRoItem;
    if (e0 >= total) return;
    const int n = (int)min((int64_t)kRoItem, total - e0);
    const int lane = threadIdx.x;
    const int col = lane & 15, g = lane >> 4;
    const uint32_t K = (uint32_t)p.K;
    const uint32_t C = (uint32_t)p.C;
    const uint32_t NSUP = (uint32_t)ro_supers(p);
    const float sl2 = p.scale * 1.4426950408889634f;

    // the item's entries (lane holds entries lane + 64 b) and the first entry of
    // every run of equal cells
    uint32_t ec[NB], ep[NB];
    uint64_t runs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int x = 64 * b + lane;
        const uint2 v = x < n ? list[e0 + x] : make_uint2(~0u, 0u);
        ec[b] = v.x;
        ep[b] = v.y;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        uint32_t pv = (uint32_t)__shfl_up((int)ec[b], 1);
        if (lane == 0) pv = b == 0 ? ~ec[0] : (uint32_t)__builtin_amdgcn_readlane((int)ec[b - 1], 63);
        runs[b] = __ballot(64 * b + lane < n && ec[b] != pv);
    }
    // first run start after entry x, n when there is none (all wave-uniform)
    auto next_run = [&](int x) __attribute__((always_inline)) {
        int r = n;
#pragma unroll
        for (int b = NB - 1; b >= 0; --b) {
            const int from = x + 1 - 64 * b;  // first bit of piece b to look at
            uint64_t m = from <= 0 ? runs[b] : from >= 64 ? 0ull : runs[b] & (~0ull << from);
            if (m) r = 64 * b + (int)__builtin_ctzll(m);
        }
        return r;
    };
    auto is_run_start = [&](int x) __attribute__((always_inline)) {
        bool r = false;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if ((x >> 6) == b) r = (runs[b] >> (x & 63)) & 1ull;
        return r;
    };
    auto cell_at = [&](int x) __attribute__((always_inline)) {
        uint32_t c = 0u;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if ((x >> 6) == b) c = (uint32_t)__builtin_amdgcn_readlane((int)ec[b], x & 63);
        return c;
    };
    // pairs of the unit starting at entry x: up to 16, within x's run
    auto unit_len = [&](int x) __attribute__((always_inline)) { return min(16, next_run(x) - x); };
    // the lane's pair of the unit at x with len pairs (lanes past len repeat its last one)
    auto unit_pair = [&](int x, int len) __attribute__((always_inline)) {
        const int e = x + min(col, len - 1);
        uint32_t r = 0u;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t v = (uint32_t)__shfl((int)ep[b], e & 63);
            if ((e >> 6) == b) r = v;
        }
        return r;
    };
    // the pair's query row as the MFMA B operand (dimensions 32 ks + 8 g .. + 7)
    auto load_q = [&](uint32_t pr, R8 *dst) __attribute__((always_inline)) {
        const uint16_t *qr = q + (int64_t)(pr / K) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < QS; ++ks) dst[ks].u = *reinterpret_cast<const uint4 *>(qr + 32 * ks);
    };
    // a cell's keys as S^T A operands (row 16 tt + col, dimensions 32 ks + 8 g .. + 7)
    // and its values as O^T A operands (dimension 16 dt + col, k-slots 8 g .. + 7 of
    // the 32-token group kk in vt_pos order), read straight into registers
    auto cell_base = [&](uint32_t cid, int64_t &c, uint32_t &hh) __attribute__((always_inline)) {
        const uint32_t hs = cid / C;  // head * super-spans + super-span
        c = (int64_t)(cid - hs * C);
        hh = hs / NSUP;
    };
    auto load_k = [&](uint32_t cid, R8 *dst) __attribute__((always_inline)) {
        int64_t c;
        uint32_t hh;
        cell_base(cid, c, hh);
        const uint16_t *kc = k + ((int64_t)hh * p.N + c * S + col) * D + 8 * g;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int ks = 0; ks < QS; ++ks)
                dst[tt * QS + ks].u = *reinterpret_cast<const uint4 *>(kc + 16 * tt * D + 32 * ks);
    };
    auto load_v = [&](uint32_t cid, R8 *dst) __attribute__((always_inline)) {
        int64_t c;
        uint32_t hh;
        cell_base(cid, c, hh);
        const uint16_t *vc = vt + (int64_t)hh * vt_head_elems(p) + (c * S / 32) * (32 * D) + col * 32 + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                dst[kk * (D / 16) + dt].u = *reinterpret_cast<const uint4 *>(vc + (kk * D + 16 * dt) * 32);
    };

    // Units in order; each unit's queries are loaded two units ahead, into the
    // register set it frees (even and odd units use the two sets in turn), and the
    // next run's keys and values as soon as the run's last unit has used them.
    int a = 0;                     // first entry of the current unit
    int len = unit_len(0);         // its pairs
    int a1 = len;                  // next unit (n: none)
    int a2 = a1 < n ? a1 + unit_len(a1) : n;  // the one after
    uint32_t cid = cell_at(0);
    R8 kop[KOPS], vop[VOPS];
    load_k(cid, kop);
    load_v(cid, vop);
    R8 qA[QS], qB[QS];
    const uint32_t prA0 = unit_pair(0, len);
    uint32_t prA = prA0;
    load_q(prA, qA);
    uint32_t prB = a1 < n ? unit_pair(a1, unit_len(a1)) : prA0;  // (a repeat when there is no second unit)
    load_q(prB, qB);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loop starts with nothing in flight
    bool odd_cell = ((cid - (cid / C) * C) & 1u) != 0u;

    auto step = [&](R8 *qc, uint32_t &prc) __attribute__((always_inline)) {
        // the next unit starts a new run: its cell's keys and values replace this
        // run's once this unit has used them
        const bool switch_cell = a1 < n && is_run_start(a1);
        const uint32_t cid_next = switch_cell ? cell_at(a1) : cid;
        floatx4 sacc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            sacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < QS; ++ks)
                sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[tt * QS + ks].b, qc[ks].b, sacc[tt], 0, 0, 0);
        }
        // the unit after next: its queries go out before this unit's stores (past the
        // item's last unit the loads repeat this unit's rows, so that every unit issues
        // the same memory instructions and the compiler's waits can count them)
        const uint32_t pr_here = prc;
        prc = a2 < n ? unit_pair(a2, unit_len(a2)) : prc;
        load_q(prc, qc);
        if (switch_cell) load_k(cid_next, kop);
        // keep these loads ahead of this unit's stores: loads and stores complete in
        // one order, and waiting for a load issued after a store waits for the store
        asm volatile("" ::: "memory");
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
            if (odd_cell) {
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
        if (switch_cell) {
            load_v(cid_next, vop);
            // the new run's keys and values complete here, once per run, so that the
            // compiler knows them complete in every later unit (vmcnt(0) through the
            // builtin, which its wait counting sees)
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        const float l = colsum4(lsum);
        const float inv = 1.0f / l;
        // Every lane stores: lanes past the unit's last pair computed that pair again
        // and write the same values to the same place, and the four lanes of a column
        // hold the same lambda. The lane's dimensions 16 dt + 4 g + r go to element
        // 32 (dt / 2) + 8 g + 4 (dt % 2) + r of the row, so that each store
        // instruction writes 64 contiguous bytes per query.
        {
            uint16_t *dst = part + (int64_t)pr_here * D + 8 * g;
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
            plse[pr_here] = m + __log2f(l);
        }
        // advance: the next unit, the one after it
        a = a1;
        len = a1 < n ? a2 - a1 : 0;
        a1 = a2;
        a2 = a2 < n ? a2 + unit_len(a2) : n;
        cid = cid_next;
        odd_cell = ((cid - (cid / C) * C) & 1u) != 0u;
    };
    while (true) {
        step(qA, prA);
        if (a >= n) break;
        step(qB, prB);
        if (a >= n) break;
    }
}

template <int D, int S>
static void launch_ru(dim3 grid, hipStream_t st, const void *q, const void *k, const uint16_t *vt,
                      const uint2 *list, const uint32_t *cnt, const uint32_t *tot, uint16_t *part, float *plse,
                      const KParams &p) {
    hipLaunchKernelGGL((readout_cells_kernel<D, S>), grid, dim3(64), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, vt, list, cnt, tot, part, plse, p);
}

// Reads out every query.
hipError_t launch_readout_cells(const void *q, const void *k, const uint16_t *vt, const int32_t *sel,
                                uint32_t *plan, uint16_t *part, float *plse, const KParams &p, hipStream_t st) {
    if (!ro_supported(p)) return hipErrorInvalidValue;
    const int QR = span_queries(p);
    const int nspan = (int)((p.N + QR - 1) / QR);
    const int64_t ncnt = ro_count_words(p);
    uint32_t *cnt = plan;
    uint32_t *tot = plan + ncnt;
    uint2 *list = reinterpret_cast<uint2 *>(plan + ro_list_word(p));
    const unsigned zgrid = (unsigned)min((int64_t)4096, (ncnt + 255) / 256);
    hipLaunchKernelGGL(ro_zero_kernel, dim3(zgrid), dim3(256), 0, st, cnt, ncnt);
    hipLaunchKernelGGL(ro_span_kernel<false>, dim3((unsigned)(nspan * p.H)), dim3(kPlanThreads), 0, st, sel, cnt,
                       tot, list, p, QR);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = launch_scan_u32(cnt, ncnt, tot, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ro_span_kernel<true>, dim3((unsigned)(nspan * p.H)), dim3(kPlanThreads), 0, st, sel, cnt,
                       tot, list, p, QR);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = ((int64_t)p.H * p.N * p.K + kRoItem - 1) / kRoItem;
    dim3 grid((unsigned)items);
#define FSL_RU(DD, SS) launch_ru<DD, SS>(grid, st, q, k, vt, list, cnt, tot, part, plse, p)
    if (p.d == 64) {
        if (p.s == 16) FSL_RU(64, 16); else if (p.s == 32) FSL_RU(64, 32); else FSL_RU(64, 64);
    } else {
        if (p.s == 16) FSL_RU(128, 16); else if (p.s == 32) FSL_RU(128, 32); else FSL_RU(128, 64);
    }
#undef FSL_RU
    return hipGetLastError();
}

}  // namespace fsl

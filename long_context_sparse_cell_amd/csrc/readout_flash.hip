// Long-branch readout + mix for bf16 inputs as one flash-attention sweep over
// the cells a block selected (FreeSolo digest, core method and step 6: NoPE
// softmax over the raw tokens of the selected cells, RMSNorm, add to the local
// branch with a per-head weight).
//
// A workgroup takes up to 128 queries of one block (8 waves x 16 queries, each
// wave's queries held in registers as MFMA operands). Every query's cells come
// from the block's pool, so the workgroup walks the pool cells that at least
// one of its queries selected, in ascending cell order: each selected cell is
// read from memory once per block. Without pruning (P = -1) there is no pool
// table: the workgroup sorts its queries' selections (at most 512 entries, so
// 64 queries per workgroup when K > 4) and walks the distinct cells. A cell's keys (raw bf16 rows) and values
// (fp16, transposed per 32-token group in vt_pos order, from kv_prep.hip; a
// 16-token cell brings its whole group) are copied from global memory straight
// into LDS (global_load_lds, 16 bytes per lane) through a ring of one-cell
// slots (named arrays, so the compiler can tell copies from reads) used two
// cells per barrier, the next pair in flight while one pair is multiplied. The
// copy picks which
// 16-byte piece each lane fetches so that key rows keep chunk c at
// c ^ swz_key(row) and value rows keep piece g at g ^ swz_val(dim), which
// spreads the MFMA operand reads over the LDS banks. Work-groups run in an
// XCD-aware order so that consecutive blocks, whose pools overlap, share an L2.
// For every cell, each wave whose queries include a selector computes
// S^T = K_c Q^T (bf16 MFMA, exact products), gives the queries that did not
// select the cell weight zero, and updates a per-query online softmax (lazily
// kept maximum) and O^T = V^T P^T (fp16 MFMA) held in registers; the lanes of
// a query column own its statistics. A query's result depends only on its own
// cells in ascending order, so the output is deterministic.
#include <climits>

#include "fsl_internal.h"

namespace fsl {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRfThreads = 512;     // 8 waves
constexpr int kRfWaves = kRfThreads / 64;
constexpr int kRfMaxQ = 128;
constexpr int kRfMaxPool = 128;
constexpr int kRfMaxSel = 512;  // selections of one work-group without pruning

union R8 {
    uint4 u;
    uint2 d[2];
    bf16x8 b;
    halfx8 h;
};

}  // namespace

template <int D, int S, bool FS>
__global__ __launch_bounds__(kRfThreads, 4) void readout_flash_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ vt,
    const int32_t *__restrict__ sel, const int32_t *__restrict__ pool, const float *__restrict__ o_win,
    void *__restrict__ out, float *__restrict__ o_long_out, KParams p, int QW) {
    constexpr int CELL = S * D;                      // elements of one cell's keys
    constexpr int VCELL = (S < 32 ? 32 : S) * D;     // elements of the value groups holding a cell
    constexpr int KUNITS = CELL * 2 / 1024;          // 1 KB copy units per cell: keys,
    constexpr int UNITS = KUNITS + VCELL * 2 / 1024; // then values
    constexpr int UPW = (UNITS + kRfWaves - 1) / kRfWaves;  // copies per wave per cell
    constexpr int NS = (CELL + VCELL) * 2 <= 16384 ? 4 : 2;  // ring stages (LDS <= 64 KB)
    constexpr int CPR = D / 8;                       // 16-byte chunks per key row
    constexpr int NT = S / 16;                       // 16-token tiles per cell
    constexpr int KK = (NT + 1) / 2;
    constexpr int QS = D / 32;
    static_assert(UPW * (NS - 2) < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) uint16_t s_k0[CELL];
    __shared__ __attribute__((aligned(1024))) uint16_t s_k1[CELL];
    __shared__ __attribute__((aligned(1024))) uint16_t s_k2[NS > 2 ? CELL : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t s_k3[NS > 2 ? CELL : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t s_v0[VCELL];
    __shared__ __attribute__((aligned(1024))) uint16_t s_v1[VCELL];
    __shared__ __attribute__((aligned(1024))) uint16_t s_v2[NS > 2 ? VCELL : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t s_v3[NS > 2 ? VCELL : 8];
    constexpr int MAXA = FS ? kRfMaxSel : kRfMaxPool;  // distinct cells a work-group can walk
    __shared__ int s_pool[FS ? 1 : kRfMaxPool];
    __shared__ uint32_t s_mask[FS ? 1 : kRfMaxPool][4];  // which local queries selected pool position t
    __shared__ uint32_t s_amask[MAXA][4];  // which local queries selected the a-th walked cell
    __shared__ int s_acell[MAXA];          // the walked cells, ascending
    __shared__ int s_nact;

    const int nqb = (int)((p.N + QW - 1) / QW);
    const int logical = xcd_remap((int)blockIdx.x, nqb * p.H);
    const int h = logical / nqb;
    const int64_t q0 = (int64_t)(logical % nqb) * QW;
    const int64_t b = q0 / p.B;
    const int nq = (int)min((int64_t)QW, p.N - q0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int K = p.K;
    const int npool = (int)min((int64_t)p.PW, eligible_cells(p, b));
    const int64_t hN = (int64_t)h * p.N;
    const float sl2 = p.scale * 1.4426950408889634f;

    // this wave's 16 queries as bf16 MFMA B operands, requested before the setup
    const int qwl = 16 * wave;  // first query (local) of this wave
    const int qrow = min(qwl + col, max(nq - 1, 0));
    R8 bq[QS];
#pragma unroll
    for (int ks = 0; ks < QS; ++ks) bq[ks].u = *reinterpret_cast<const uint4 *>(q + (hN + q0 + qrow) * D + 32 * ks + 8 * g);

    if constexpr (FS) {
        // ---- the distinct selected cells: sort the work-group's selections (bitonic,
        // in the first value slot, which the ring fills only later), keep the first of
        // each run, then mark which queries selected each
        int *s_sort = reinterpret_cast<int *>(s_v0);
        static_assert(VCELL * 2 >= kRfMaxSel * 4, "sort scratch fits a value slot");
        const int nent = nq * K;
        for (int t = tid; t < kRfMaxSel; t += kRfThreads) {
            const int c = t < nent ? sel[(hN + q0) * K + t] : -1;
            s_sort[t] = c < 0 ? INT_MAX : c;
        }
        __syncthreads();
        for (int len = 2; len <= kRfMaxSel; len <<= 1)
            for (int st = len >> 1; st > 0; st >>= 1) {
                for (int t = tid; t < kRfMaxSel / 2; t += kRfThreads) {
                    const int lo = 2 * st * (t / st) + (t % st), hi = lo + st;
                    const bool up = (lo & len) == 0;
                    const int a = s_sort[lo], c = s_sort[hi];
                    s_sort[lo] = up ? min(a, c) : max(a, c);
                    s_sort[hi] = up ? max(a, c) : min(a, c);
                }
                __syncthreads();
            }
        if (wave == 0) {
            int base = 0;
            for (int t0 = 0; t0 < kRfMaxSel; t0 += 64) {
                const int t = t0 + lane;
                const int c = s_sort[t];
                const bool on = c != INT_MAX && (t == 0 || s_sort[t - 1] != c);
                const uint64_t bal = __ballot(on);
                if (on) s_acell[base + __popcll(bal & ((1ull << lane) - 1ull))] = c;
                base += __popcll(bal);
            }
            if (lane == 0) s_nact = base;
        }
        __syncthreads();
        const int na = s_nact;
        for (int t = tid; t < na; t += kRfThreads) s_amask[t][0] = s_amask[t][1] = s_amask[t][2] = s_amask[t][3] = 0u;
        __syncthreads();
        for (int pr = tid; pr < nent; pr += kRfThreads) {
            const int c = sel[(hN + q0) * K + pr];
            if (c < 0) continue;
            int lo = 0, hi = na - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_acell[mid] < c) lo = mid + 1; else hi = mid;
            }
            const int ql = pr / K;
            atomicOr(&s_amask[lo][ql >> 5], 1u << (ql & 31));
        }
        __syncthreads();
    } else {
        // ---- which queries selected which pool cell
        for (int t = tid; t < npool; t += kRfThreads) {
            s_pool[t] = pool[((int64_t)h * p.nblk + b) * p.PW + t];
            s_mask[t][0] = s_mask[t][1] = s_mask[t][2] = s_mask[t][3] = 0u;
        }
        __syncthreads();
        for (int pr = tid; pr < nq * K; pr += kRfThreads) {
            const int c = sel[(hN + q0) * K + pr];
            if (c < 0) continue;
            int lo = 0, hi = npool - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_pool[mid] < c) lo = mid + 1; else hi = mid;
            }
            const int ql = pr / K;
            atomicOr(&s_mask[lo][ql >> 5], 1u << (ql & 31));
        }
        __syncthreads();
        if (wave == 0) {
            // compact the selected positions in pool (= ascending cell) order
            int base = 0;
            for (int t0 = 0; t0 < npool; t0 += 64) {
                const int t = t0 + lane;
                const bool on = t < npool && (s_mask[t][0] | s_mask[t][1] | s_mask[t][2] | s_mask[t][3]) != 0u;
                const uint64_t bal = __ballot(on);
                if (on) {
                    const int a = base + __popcll(bal & ((1ull << lane) - 1ull));
                    s_acell[a] = s_pool[t];
    #pragma unroll
                    for (int x = 0; x < 4; ++x) s_amask[a][x] = s_mask[t][x];
                }
                base += __popcll(bal);
            }
            if (lane == 0) s_nact = base;
        }
        __syncthreads();
    }
    const int nact = s_nact;


    // ---- copy plan: a cell's keys then its values in 1 KB units; this wave copies
    // units wave + 8 i. Every wave issues exactly UPW copies per cell (spare units
    // repeat the last one, writing the same bytes) so that vmcnt counts whole cells.
    int c_off[UPW], c_dst[UPW];
    bool c_key[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int u = min(wave + kRfWaves * i, UNITS - 1);
        c_key[i] = u < KUNITS;
        const int e0 = (c_key[i] ? u : u - KUNITS) * 512;  // first element of the unit in its region
        c_dst[i] = e0;
        const int s = e0 / 8 + lane;                       // 16-byte slot within the region
        if (c_key[i]) {
            const int row = s / CPR, pc = s % CPR;
            c_off[i] = row * D + 8 * (pc ^ swz_key(row, D));
        } else {
            const int r = s >> 2, pg = s & 3;  // r = group * D + dim
            c_off[i] = r * 32 + 8 * (pg ^ swz_val(r % D));
        }
    }
    const uint16_t *vth = vt + h * vt_head_elems(p);
    auto issue = [&](int ai, uint16_t *kbuf, uint16_t *vbuf) __attribute__((always_inline)) {
        const int64_t cell = __builtin_amdgcn_readfirstlane(s_acell[ai]);
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            if (c_key[i])
                lds_dma16(k + (hN + cell * S) * D + c_off[i], kbuf + c_dst[i]);
            else
                lds_dma16(vth + (cell * S / 32) * (32 * D) + c_off[i], vbuf + c_dst[i]);
        }
    };

    float m_run = -INFINITY, l_part = 0.0f;
    floatx4 oacc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto process = [&](int ai, const uint16_t *kc, const uint16_t *vc) __attribute__((always_inline)) {
        const uint32_t m16 = (s_amask[ai][qwl >> 5] >> (qwl & 31)) & 0xFFFFu;
        if (m16 == 0u) return;  // none of this wave's queries selected the cell
        const bool mine = (m16 >> col) & 1u;
        floatx4 sacc[2 * KK];
#pragma unroll
        for (int tt = 0; tt < 2 * KK; ++tt) {
            sacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (tt < NT) {
                // the tile's key operands in one inline-asm block (one wait for all of them)
                const int row = 16 * tt + col;
                auto kaddr = [&](int ks) { return &kc[row * D + 8 * ((4 * ks + g) ^ swz_key(row, D))]; };
                R8 ka[QS];
                if constexpr (QS == 4)
                    lds_read16x4(ka[0].u, ka[1].u, ka[2].u, ka[3].u, kaddr(0), kaddr(1), kaddr(2), kaddr(3));
                else
                    lds_read16x2(ka[0].u, ka[1].u, kaddr(0), kaddr(1));
#pragma unroll
                for (int ks = 0; ks < QS; ++ks)
                    sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks].b, bq[ks].b, sacc[tt], 0, 0, 0);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[tt][r]);
        const float cmx = colmax4(mx);  // every lane takes part in the cross-lane step
        mx = mine ? cmx * sl2 : -INFINITY;
        // lazily kept maximum: move it only on a jump past kStaleLog2; a query's first
        // cell just sets it (its accumulators are still zero)
        const bool grow = mx > m_run + kStaleLog2;
        const bool resc = grow && m_run != -INFINITY;
        if (__ballot(resc)) {
            const float alpha = resc ? exp2_hw(m_run - mx) : 1.0f;
            l_part *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) oacc[dt] *= alpha;
        }
        if (grow) m_run = mx;
        // queries that did not select the cell get weight 2^-inf = 0
        const float msub = mine ? m_run : INFINITY;
        R8 pb[KK];
        float lsum = 0.0f;
#pragma unroll
        for (int tt = 0; tt < 2 * KK; ++tt) {
            uint32_t lo = 0u, hi = 0u;
            if (tt < NT) {
                float e[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = exp2_hw(fmaf(sacc[tt][r], sl2, -msub));
                lo = pk_f16_rne_acc(e[0], e[1], lsum);
                hi = pk_f16_rne_acc(e[2], e[3], lsum);
            }
            pb[tt >> 1].d[tt & 1] = make_uint2(lo, hi);
        }
        if constexpr (S == 16) {
            // a 16-token cell is one half of its value group: move its weights to the
            // k-slots of that half (slots 4..7 for an odd cell)
            if (s_acell[ai] & 1) {
                pb[0].d[1] = pb[0].d[0];
                pb[0].d[0] = make_uint2(0u, 0u);
            }
        }
        l_part += lsum;
        // value operands two or four at a time (one inline-asm block, see lds_read16x4)
        constexpr int VB = KK > 1 ? 2 : 4;
        auto vaddr = [&](int kk, int dt) __attribute__((always_inline)) {
            const int dim = 16 * dt + col;
            return &vc[((kk * D + dim) * 4 + (g ^ swz_val(dim))) * 8];
        };
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int d0 = 0; d0 < D / 16; d0 += VB) {
                R8 va[VB];
                if constexpr (VB == 4)
                    lds_read16x4(va[0].u, va[1].u, va[2].u, va[3].u, vaddr(kk, d0), vaddr(kk, d0 + 1),
                                 vaddr(kk, d0 + 2), vaddr(kk, d0 + 3));
                else
                    lds_read16x2(va[0].u, va[1].u, vaddr(kk, d0), vaddr(kk, d0 + 1));
#pragma unroll
                for (int x = 0; x < VB; ++x)
                    oacc[d0 + x] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[x].h, pb[kk].h, oacc[d0 + x], 0, 0, 0);
            }
    };

    // ---- ring of NS one-cell slots, used two cells at a time: while cells a, a+1 are
    // multiplied, a+2 and a+3 are in flight. Before a pair, this wave's copies of it
    // are done once nothing younger is outstanding; the barrier then makes every
    // wave's copies visible, and the pair of slots processed before is refilled.
    static_assert(NS == 4 || NS == 2, "ring of 4 slots (pairs) or 2 slots (single cells)");
    if constexpr (NS == 4) {
        auto pair = [&](int a, const uint16_t *kc0, const uint16_t *vc0, const uint16_t *kc1, const uint16_t *vc1,
                        uint16_t *kp0, uint16_t *vp0, uint16_t *kp1, uint16_t *vp1) __attribute__((always_inline)) {
            wait_vmem_le<0>();
            barrier_no_fence();
            issue(min(a + 2, nact - 1), kp0, vp0);  // past the end: harmless repeats of the last cell
            issue(min(a + 3, nact - 1), kp1, vp1);
            process(a, kc0, vc0);
            if (a + 1 < nact) process(a + 1, kc1, vc1);
        };
        if (nact > 0) {
            issue(0, s_k0, s_v0);
            issue(min(1, nact - 1), s_k1, s_v1);
        }
        for (int a = 0; a < nact; a += 4) {
            pair(a, s_k0, s_v0, s_k1, s_v1, s_k2, s_v2, s_k3, s_v3);
            if (a + 2 >= nact) break;
            pair(a + 2, s_k2, s_v2, s_k3, s_v3, s_k0, s_v0, s_k1, s_v1);
        }
    } else {
        auto step = [&](int a, const uint16_t *kc, const uint16_t *vc, uint16_t *kpf, uint16_t *vpf)
            __attribute__((always_inline)) {
            wait_vmem_le<0>();
            barrier_no_fence();
            issue(min(a + 1, nact - 1), kpf, vpf);
            process(a, kc, vc);
        };
        if (nact > 0) issue(0, s_k0, s_v0);
        for (int a = 0; a < nact; a += 2) {
            step(a, s_k0, s_v0, s_k1, s_v1);
            if (a + 1 >= nact) break;
            step(a + 1, s_k1, s_v1, s_k0, s_v0);
        }
    }
    wait_vmem();  // no copy into LDS may outlive the work-group

    // ---- normalise, RMSNorm over d, mix, write (lane: query col, dims 16*dt + 4*g + r)
    const float l = colsum4(l_part);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float ss = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        oacc[dt] *= inv;
#pragma unroll
        for (int r = 0; r < 4; ++r) ss += oacc[dt][r] * oacc[dt][r];
    }
    ss = colsum4(ss);
    const float rs = 1.0f / sqrtf(ss / (float)D + p.rms_eps);
    const int ql = qwl + col;
    if (ql < nq) {
        const float gam = p.gamma[h];
        const int64_t row = hN + q0 + ql;
        // every local-branch load first (consumed by an empty asm, so none of them is
        // moved past a store and waited for one at a time)
        float4 owv[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            owv[dt] = *reinterpret_cast<const float4 *>(o_win + row * D + 16 * dt + 4 * g);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            asm volatile("" ::"v"(owv[dt].x), "v"(owv[dt].y), "v"(owv[dt].z), "v"(owv[dt].w));
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const int c0 = 16 * dt + 4 * g;
            const float4 ow = owv[dt];
            const float o4[4] = {ow.x, ow.y, ow.z, ow.w};
            float val[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) val[r] = o4[r] + gam * (oacc[dt][r] * rs);
            if (p.out_dtype == FSL_BF16) {
                const uint32_t w0 = (uint32_t)f32_to_bf16(val[0]) | ((uint32_t)f32_to_bf16(val[1]) << 16);
                const uint32_t w1 = (uint32_t)f32_to_bf16(val[2]) | ((uint32_t)f32_to_bf16(val[3]) << 16);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + row * D + c0) = make_uint2(w0, w1);
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + row * D + c0) =
                    make_float4(val[0], val[1], val[2], val[3]);
            }
            if (o_long_out)
                *reinterpret_cast<float4 *>(o_long_out + row * D + c0) =
                    make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
        }
    }
}

template <int D, int S>
static void launch_rf(dim3 grid, hipStream_t st, const void *q, const void *k, const uint16_t *vt, const int32_t *sel,
                      const int32_t *pool, const float *o_win, void *out, float *o_long_out, const KParams &p, int QW) {
    if (p.P < 0)
        hipLaunchKernelGGL((readout_flash_kernel<D, S, true>), grid, dim3(kRfThreads), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, vt, sel, pool, o_win, out, o_long_out, p, QW);
    else
        hipLaunchKernelGGL((readout_flash_kernel<D, S, false>), grid, dim3(kRfThreads), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, vt, sel, pool, o_win, out, o_long_out, p, QW);
}

hipError_t launch_readout_flash(const void *q, const void *k, const uint16_t *vt, const int32_t *sel,
                                const int32_t *pool, const float *o_win, void *out, float *o_long_out, const KParams &p,
                                hipStream_t st) {
    // queries per work-group: half a block when B > 128; without pruning also at most
    // kRfMaxSel / K, so that the work-group's selections fit the sort
    const int qmax = p.P < 0 && p.K > 4 ? kRfMaxSel / 8 : kRfMaxQ;
    const int QW = p.B <= qmax ? p.B : (p.B / 2 <= qmax ? p.B / 2 : p.B / 4);
    dim3 grid((unsigned)(((p.N + QW - 1) / QW) * p.H));
#define FSL_RF(DD, SS) launch_rf<DD, SS>(grid, st, q, k, vt, sel, pool, o_win, out, o_long_out, p, QW)
    if (p.d == 64) {
        if (p.s == 16) FSL_RF(64, 16); else if (p.s == 32) FSL_RF(64, 32); else FSL_RF(64, 64);
    } else {
        if (p.s == 16) FSL_RF(128, 16); else if (p.s == 32) FSL_RF(128, 32); else FSL_RF(128, 64);
    }
#undef FSL_RF
    return hipGetLastError();
}

}  // namespace fsl

// Long-branch readout + mix for bf16 inputs, organised by cell (FreeSolo
// digest, core method and step 6: NoPE softmax over the raw tokens of the
// selected cells, RMSNorm, add to the local branch with a per-head weight).
//
// The 128 queries of a block select their K cells from the same pool of at
// most P+W cells, and nearly every pool cell is chosen by several queries. So
// one workgroup (8 waves) takes a tile of up to 128 queries of one block and groups
// its (query, cell) pairs by cell: each group of up to 16 queries that chose
// cell c is one MFMA item, and cell c's keys and values are read once per
// tile instead of once per query.
//
//   pass 1: S^T = K_c Q^T (bf16 MFMA, exact products) -> per (query, slot)
//           max of the scaled scores
//   pass 2: recompute S^T; P = exp2(S - m_query) (fp16, <= 1); O = P V_c
//           (fp16 MFMA, fp32 accumulate), added per query into an LDS
//           accumulator in 2^-32 fixed point (int64 adds commute, so the
//           result does not depend on which wave finishes first)
//   final : o_long = acc / l, RMSNorm, out = o_win + gamma_h * normalised.
#include "fsl_internal.h"

namespace fsl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kMaxQ = 128;                       // queries per workgroup
constexpr int kMaxPool = 128;                    // P + W <= 128
constexpr int kMaxSlots = 8;                     // K <= 8
constexpr int kMaxPairs = kMaxQ * kMaxSlots;
constexpr int kMaxItems = kMaxPool + kMaxPairs / 16;
constexpr float kFix = 4294967296.0f;            // 2^32
constexpr int kThreads = 512;                    // 8 waves, two per SIMD
constexpr int kWaves = kThreads / 64;

union U16x8 {
    uint4 u;
    bf16x8 b;
};

union H8 {
    halfx8 v;
    _Float16 f[8];
};

// x * 2^32 as a two's-complement integer, exactly (|x| < 2^30): the integer
// part and the fraction are converted separately with 32-bit conversions
__device__ __forceinline__ unsigned long long to_fixed(float x) {
    const float fl = floorf(x);
    const float fr = x - fl;  // exact, in [0, 1)
    const uint32_t lo = (uint32_t)(fr * kFix);
    const int32_t hi = (int32_t)fl;
    return ((unsigned long long)(uint32_t)hi << 32) + lo;
}

__device__ __forceinline__ int pack_item(int pos, int start, int cnt) { return pos | (start << 8) | (cnt << 20); }

// exclusive scan of n <= 128 ints in LDS by one wave; returns the total
__device__ int wave_excl_scan(int *a, int n) {
    const int lane = threadIdx.x & 63;
    int v0 = lane < n ? a[lane] : 0;
    int v1 = lane + 64 < n ? a[lane + 64] : 0;
    int x0 = v0, x1 = v1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t0 = __shfl_up(x0, o), t1 = __shfl_up(x1, o);
        if (lane >= o) { x0 += t0; x1 += t1; }
    }
    const int tot0 = __shfl(x0, 63);
    const int tot1 = __shfl(x1, 63);
    if (lane < n) a[lane] = x0 - v0;
    if (lane + 64 < n) a[lane + 64] = tot0 + x1 - v1;
    return tot0 + tot1;
}

}  // namespace

template <int D, int S>
__global__ __launch_bounds__(512) void readout_cells_kernel(const uint16_t *__restrict__ q,
                                                            const uint16_t *__restrict__ k,
                                                            const uint16_t *__restrict__ v,
                                                            const int32_t *__restrict__ sel,
                                                            const int32_t *__restrict__ pool,
                                                            const float *__restrict__ o_win, void *__restrict__ out,
                                                            float *__restrict__ o_long_out, KParams p, int QW) {
    __shared__ unsigned long long acc[kMaxQ * D];
    __shared__ int s_pool[kMaxPool];
    __shared__ int s_cnt[kMaxPool];
    __shared__ int s_off[kMaxPool];
    __shared__ int s_ioff[kMaxPool];
    __shared__ int s_list[kMaxPairs];
    __shared__ int s_item[kMaxItems];
    __shared__ float s_pmax[kMaxPairs];
    __shared__ float s_pl[kMaxPairs];
    __shared__ float s_m[kMaxQ];
    __shared__ int s_nitems;
    __shared__ int s_sel[kMaxPairs];

    const int h = blockIdx.y;
    const int64_t q0 = (int64_t)blockIdx.x * QW;
    const int64_t b = q0 / p.B;
    const int nq = (int)min((int64_t)QW, p.N - q0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g = lane >> 4;
    const int K = p.K;
    constexpr int s = S;
    const int npool = (int)min((int64_t)p.PW, eligible_cells(p, b));
    const float sl2 = p.scale * 1.4426950408889634f;
    const int64_t hN = (int64_t)h * p.N;

    // ---- setup: pool, counts, accumulators
    for (int t = tid; t < npool; t += kThreads) {
        s_pool[t] = pool[((int64_t)h * p.nblk + b) * p.PW + t];
        s_cnt[t] = 0;
    }
    for (int t = tid; t < nq * K; t += kThreads) s_sel[t] = sel[(hN + q0) * K + t];
    for (int t = tid; t < kMaxQ * D; t += kThreads) acc[t] = 0ull;
    for (int t = tid; t < kMaxPairs; t += kThreads) { s_pmax[t] = -INFINITY; s_pl[t] = 0.0f; }
    __syncthreads();

    // ---- pairs: find each selected cell's pool position, count per position
    constexpr int PPT = kMaxPairs / kThreads;  // pairs per thread
    int my_pos[PPT], my_rank[PPT];
    const int npairs = nq * K;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
        my_pos[u] = -1;
        const int pr = tid + kThreads * u;
        if (pr < npairs) {
            const int c = s_sel[pr];
            if (c >= 0) {
                int lo = 0, hi = npool - 1;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (s_pool[mid] < c) lo = mid + 1; else hi = mid;
                }
                my_pos[u] = lo;
                my_rank[u] = atomicAdd(&s_cnt[lo], 1);
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        for (int t = lane; t < npool; t += 64) {
            s_off[t] = s_cnt[t];
            s_ioff[t] = (s_cnt[t] + 15) >> 4;
        }
        __builtin_amdgcn_wave_barrier();
        wave_excl_scan(s_off, npool);
        const int nit = wave_excl_scan(s_ioff, npool);
        if (lane == 0) s_nitems = nit;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
        if (my_pos[u] >= 0) {
            const int pr = tid + kThreads * u;
            s_list[s_off[my_pos[u]] + my_rank[u]] = ((pr / K) << 3) | (pr % K);
        }
    }
    for (int t = tid; t < npool; t += kThreads) {
        const int cnt = s_cnt[t];
        for (int j = 0; 16 * j < cnt; ++j) s_item[s_ioff[t] + j] = pack_item(t, s_off[t] + 16 * j, min(16, cnt - 16 * j));
    }
    __syncthreads();
    const int nitems = s_nitems;
    constexpr int NT = S / 16;        // 16-token tiles per cell
    constexpr int KK = (NT + 1) / 2;  // 32-token MFMA k-steps of P V

    // ---- pass 1: per (query, slot) max of the scaled scores
    for (int it = wave; it < nitems; it += kWaves) {
        const int item = s_item[it];
        const int pos = item & 0xFF, start = (item >> 8) & 0xFFF, cnt = item >> 20;
        const int c = s_pool[pos];
        const int code = s_list[start + (col < cnt ? col : 0)];
        const int ql = code >> 3;
        const uint16_t *qrow = q + (hN + q0 + ql) * D;
        U16x8 bq[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) bq[ks].u = *reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * g);
        float mx = -INFINITY;
        for (int tt = 0; tt < NT; ++tt) {
            const uint16_t *krow = k + (hN + (int64_t)c * s + 16 * tt + col) * D;
            floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                U16x8 ka;
                ka.u = *reinterpret_cast<const uint4 *>(krow + 32 * ks + 8 * g);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka.b, bq[ks].b, sacc, 0, 0, 0);
            }
            mx = fmaxf(mx, fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3])));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (g == 0 && col < cnt) s_pmax[code] = mx * sl2;
    }
    __syncthreads();
    for (int t = tid; t < nq; t += kThreads) {
        float m = -INFINITY;
        for (int r = 0; r < K; ++r) m = fmaxf(m, s_pmax[(t << 3) | r]);  // slots without a cell hold -inf
        s_m[t] = m;
    }
    __syncthreads();

    // ---- pass 2: probabilities, partial sums, P V into the fixed-point accumulators.
    // Every load of an item (q columns, K rows, V rows) is issued before its math.
    for (int it = wave; it < nitems; it += kWaves) {
        const int item = s_item[it];
        const int pos = item & 0xFF, start = (item >> 8) & 0xFFF, cnt = item >> 20;
        const int c = s_pool[pos];
        const int code = s_list[start + (col < cnt ? col : 0)];
        const int ql = code >> 3;
        const float m = s_m[ql];
        const int64_t cell0 = hN + (int64_t)c * s;
        const uint16_t *qrow = q + (hN + q0 + ql) * D;
        U16x8 bq[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) bq[ks].u = *reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * g);
        U16x8 ka[2 * KK][D / 32];
#pragma unroll
        for (int tt = 0; tt < 2 * KK; ++tt) {
            const uint16_t *krow = k + (cell0 + min(16 * tt + col, s - 1)) * D;  // rows past the cell: P = 0
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) ka[tt][ks].u = *reinterpret_cast<const uint4 *>(krow + 32 * ks + 8 * g);
        }
        // V rows for tokens 32kk + {4g..4g+3, 16+4g..16+4g+3} (clamped to the cell)
        uint16_t vraw[KK][D / 16][8];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tk = 32 * kk + ((e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4));
                const uint16_t *vp = v + (cell0 + min(tk, s - 1)) * D + col;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) vraw[kk][dt][e] = vp[16 * dt];
            }
        floatx4 oacc[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        float lsum = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            H8 pa;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int tt = 2 * kk + half;
                floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][ks].b, bq[ks].b, sacc, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const _Float16 ph = tt < NT ? (_Float16)exp2f(sacc[e] * sl2 - m) : (_Float16)0.0f;
                    pa.f[4 * half + e] = ph;
                    lsum += (float)ph;
                }
            }
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                H8 vb;
#pragma unroll
                for (int e = 0; e < 8; ++e) vb.f[e] = (_Float16)bf16_to_f32(vraw[kk][dt][e]);
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa.v, vb.v, oacc[dt], 0, 0, 0);
            }
        }
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        if (g == 0 && col < cnt) s_pl[code] = lsum;
        // lane (dim 16*dt + col, g) holds O[queries 4g + e][dim]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int slot = 4 * g + e;
            if (slot < cnt) {
                const int qd = s_list[start + slot] >> 3;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) atomicAdd(&acc[qd * D + 16 * dt + col], to_fixed(oacc[dt][e]));
            }
        }
    }
    __syncthreads();

    // ---- final: normalise, RMSNorm, mix (one wave per query, lanes over dims); the wave's
    // o_win rows are fetched before the loop so their latency is paid once
    constexpr int XPL = D / 64;
    constexpr int QPW = kMaxQ / kWaves;
    const float gam = p.gamma[h];
    float ow[QPW][XPL];
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const int ql = wave + kWaves * u;
        const int64_t row = hN + q0 + (ql < nq ? ql : 0);
#pragma unroll
        for (int x = 0; x < XPL; ++x) ow[u][x] = o_win[row * D + lane + 64 * x];
    }
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const int ql = wave + kWaves * u;
        if (ql >= nq) break;
        const int64_t row = hN + q0 + ql;
        float l = 0.0f;
        int nsel = 0;
        for (int r = 0; r < K; ++r)
            if (s_sel[ql * K + r] >= 0) { l += s_pl[(ql << 3) | r]; ++nsel; }
        float o[XPL];
        float ms = 0.0f;
#pragma unroll
        for (int x = 0; x < XPL; ++x) {
            const long long fx = (long long)acc[ql * D + lane + 64 * x];
            o[x] = nsel > 0 ? (float)((double)fx * (1.0 / 4294967296.0)) / l : 0.0f;
            ms += o[x] * o[x];
        }
#pragma unroll
        for (int m2 = 32; m2 > 0; m2 >>= 1) ms += __shfl_xor(ms, m2);
        ms /= (float)D;
        const float rs = 1.0f / sqrtf(ms + p.rms_eps);
#pragma unroll
        for (int x = 0; x < XPL; ++x) {
            const int cix = lane + 64 * x;
            const float val = ow[u][x] + gam * (o[x] * rs);
            if (p.out_dtype == FSL_BF16) reinterpret_cast<uint16_t *>(out)[row * D + cix] = f32_to_bf16(val);
            else reinterpret_cast<float *>(out)[row * D + cix] = val;
            if (o_long_out) o_long_out[row * D + cix] = o[x];
        }
    }
}

template <int D, int S>
static void launch_rc(dim3 grid, hipStream_t st, const void *q, const void *k, const void *v, const int32_t *sel,
                      const int32_t *pool, const float *o_win, void *out, float *o_long_out, const KParams &p, int QW) {
    hipLaunchKernelGGL((readout_cells_kernel<D, S>), grid, dim3(kThreads), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, sel, pool, o_win, out, o_long_out, p, QW);
}

hipError_t launch_readout_cells(const void *q, const void *k, const void *v, const int32_t *sel, const int32_t *pool,
                                const float *o_win, void *out, float *o_long_out, const KParams &p, hipStream_t st) {
    const int QW = p.B <= kMaxQ ? p.B : p.B / 2;
    dim3 grid((unsigned)((p.N + QW - 1) / QW), (unsigned)p.H);
#define FSL_RC(DD, SS) launch_rc<DD, SS>(grid, st, q, k, v, sel, pool, o_win, out, o_long_out, p, QW)
    if (p.d == 64) {
        if (p.s == 16) FSL_RC(64, 16); else if (p.s == 32) FSL_RC(64, 32); else FSL_RC(64, 64);
    } else {
        if (p.s == 16) FSL_RC(128, 16); else if (p.s == 32) FSL_RC(128, 32); else FSL_RC(128, 64);
    }
#undef FSL_RC
    return hipGetLastError();
}

}  // namespace fsl

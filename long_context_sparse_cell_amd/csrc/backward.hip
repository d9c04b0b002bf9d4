// Backward of the FS-L forward, for training (FreeSolo digest, method steps:
// the two branches are trained while the hard top-P / top-K indices receive no
// gradient; ai.info summary, training paragraph: the routing scalars sigma_h,
// lambda_h stay fixed and the per-head mixing weight is learned).
//
// With the forward's selections held fixed, out = o_win + gamma * RMSNorm(o_long)
// is differentiable in q, k, v and gamma. For a branch with output o and
// upstream gradient dO, and D = dO . o, the softmax backward over its keys is
//   P_j = exp(l_j - lse), dS_j = P_j (dO . v_j - D), dv_j += P_j dO,
//   and l_j = scale a . b_j sends scale dS_j b_j to a and scale dS_j a to b_j.
// Window: a = R(i) q_i, b_j = R(j) k_j, dO = dout_i; the rotated gradients go
// back through R(t)^T. Long branch: a = q_i, b_j = k_j over the selected
// cells' tokens, dO = RMSNorm's backward of gamma dout_i.
//
// Kernels, in launch order on the caller's stream (every one writes its own
// outputs; nothing is accumulated with atomics, so results are reproducible):
//   bwd_prep        fp32 rotated q, k, fp32 v and the upstream gradient
//   bwd_win_dq      per 64 queries: a pass for the row's log-sum-exp and D, then dS
//                   and dq (window part), on the fp32 matrix cores
//   bwd_win_dkv     per 64 keys: dk, dv of the window over the queries that see them,
//                   on the fp32 matrix cores
//   bwd_pair_keys, a stable radix sort (sort.hip), bwd_seg_*: each cell's
//                   selecting queries in query order
//   bwd_long_fwd    per cell: the branch's softmax over the cell's tokens for every query
//                   that selected it (max, sum, weighted values), on the fp32 matrix cores
//   bwd_long_merge  per query (one wave): its cells combined in rank order into o_long,
//                   lse; RMSNorm's backward
//   bwd_long_kv     per cell: dk, dv += long part over every query that selected it,
//                   and each (query, rank) pair's dq, on the fp32 matrix cores; cells
//                   chosen by more than kHeavyPairs queries in chunks whose dk, dv sums
//                   bwd_heavy_reduce adds in chunk order
//   bwd_dq_long_sum per query: dq += its pairs' dq in rank order
//   bwd_dgamma      per head: dgamma summed in a fixed order
// Arithmetic is fp32, every product on the matrix cores (fp32 MFMA).
#include <climits>

#include "fsl_internal.h"

namespace fsl {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;  // 8 threads per tile row

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i) { return to_f32<T>(p[i]); }

// (cos, sin) of angle pos * theta_m from the two-level table
__device__ __forceinline__ float2 rope_cs(const float2 *tab, int nhi, int half, int64_t pos, int m) {
    const float2 th = tab[(pos / kRopeSpan) * half + m];
    const float2 tl = tab[(int64_t)(nhi + (int)(pos % kRopeSpan)) * half + m];
    return make_float2(th.x * tl.x - th.y * tl.y, th.y * tl.x + th.x * tl.y);
}

// sum over the aligned group of G lanes (G a power of two, at most 64)
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

}  // namespace

// ---- fp32 rotated q and k (R(t) x, rotate-half pairs), fp32 v and the upstream gradient
template <typename T, typename TO, int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                            const T *__restrict__ v, const TO *__restrict__ dout,
                                                            const float2 *__restrict__ tab, int nhi,
                                                            float *__restrict__ qr, float *__restrict__ kr,
                                                            float *__restrict__ vf, float *__restrict__ dO, KParams p) {
    constexpr int HALF = D / 2;
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // one rotation pair
    const int64_t total = (int64_t)p.H * p.N * HALF;
    if (e >= total) return;
    const int64_t row = e / HALF;  // h * N + t
    const int m = (int)(e % HALF);
    const int64_t t = row % p.N;
    const float2 cs = rope_cs(tab, nhi, HALF, t, m);
    const int64_t a = row * D + m, b = a + HALF;
    const float qa = ld(q, a), qb = ld(q, b), ka = ld(k, a), kb = ld(k, b);
    qr[a] = qa * cs.x - qb * cs.y;
    qr[b] = qb * cs.x + qa * cs.y;
    kr[a] = ka * cs.x - kb * cs.y;
    kr[b] = kb * cs.x + ka * cs.y;
    vf[a] = ld(v, a);
    vf[b] = ld(v, b);
    dO[a] = ld(dout, a);
    dO[b] = ld(dout, b);
}

// ---- window branch on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: lane (c, g)
// holds A[c][g] and B[g][c]; accumulator element r holds D[4 g + r][c]). The d
// dimensions of a product are summed in the order in which lane group g holds
// dims (d/4) g .. (d/4) g + d/4 - 1, so that a lane's operands are one contiguous
// quarter of a row. The other side's rows wait in LDS as fp32 tiles of kWinTile
// rows whose 16-byte chunk c sits at c ^ (row & 15) (global_load_lds,
// double-buffered); products whose k dimension is the tile row read one float per
// lane from those tiles.
namespace {
constexpr int kWinWaves = 4;                 // waves per work-group, 16 rows each
constexpr int kWinRows = 16 * kWinWaves;     // this side's rows per work-group
constexpr int kWinTile = 32;                 // other side's rows per LDS tile

template <int D>
__device__ __forceinline__ int wtile_off(int row, int chunk) { return row * D + 4 * (chunk ^ (row & 15)); }

// rows r0 .. r0 + kWinTile - 1 of one head's [N][D] fp32 array into a swizzled tile
// (rows past N repeat row N - 1; every product they enter is masked)
template <int D>
__device__ __forceinline__ void wtile_issue(const float *src_head, int64_t r0, int64_t N, float *tile, int wave,
                                            int lane) {
    constexpr int CPR = D / 4;
    constexpr int UNITS = kWinTile * D * 4 / 1024;
    static_assert(UNITS % kWinWaves == 0, "whole copy units per wave");
#pragma unroll
    for (int i = 0; i < UNITS / kWinWaves; ++i) {
        const int u = wave + kWinWaves * i;
        const int c = 64 * u + lane;  // 16-byte chunk of the tile
        const int row = c / CPR, phys = c % CPR;
        const int64_t rr = min(r0 + row, N - 1);
        lds_dma16(src_head + rr * D + 4 * (phys ^ (row & 15)), tile + 256 * u);
    }
}

// acc (rows 4 g + r of a 16-row block, column c) += tile rows `rowbase` .. + 15 as A
// times the lane's register operand b[] (its column's dims (d/4) g ..) over d
template <int D>
__device__ __forceinline__ floatx4 wtile_dot(const float *tile, int rowbase, int col, int g, const float *b) {
    constexpr int KS = D / 4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KS / 4; ++c) {
        const float4 a = *reinterpret_cast<const float4 *>(&tile[wtile_off<D>(rowbase + col, KS / 4 * g + c)]);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b[4 * c + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b[4 * c + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b[4 * c + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b[4 * c + 3], acc, 0, 0, 0);
    }
    return acc;
}

// acc[dt] (dims 16 dt + 4 g + r, column c) += sum over tile rows rowbase .. + 15 of
// tile[row][dim] w(row, c), with w(rowbase + 4 g + r, c) = w[r] held by lane (c, g)
template <int D>
__device__ __forceinline__ void wtile_tmul(const float *tile, int rowbase, int col, int g, const float *w,
                                           floatx4 *acc) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rowbase + 4 * g + r;
            const float a = tile[wtile_off<D>(row, 4 * dt + (col >> 2)) + (col & 3)];
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, w[r], acc[dt], 0, 0, 0);
        }
}

// a row's fp32 values at dims (d/4) g .. (d/4) g + d/4 - 1
template <int D>
__device__ __forceinline__ void wrow_quarter(const float *row, int g, float *dst) {
    constexpr int KS = D / 4;
#pragma unroll
    for (int c = 0; c < KS / 4; ++c) {
        const float4 x = *reinterpret_cast<const float4 *>(row + KS * g + 4 * c);
        dst[4 * c] = x.x;
        dst[4 * c + 1] = x.y;
        dst[4 * c + 2] = x.z;
        dst[4 * c + 3] = x.w;
    }
}

// x = R(t)^T scale acc for the lane's dims 16 dt + 4 g + r (rotate-half pairs dt and
// dt + D/32 are both the lane's), written as float4 rows
template <int D>
__device__ __forceinline__ void wstore_rotated(float *dst_row, const floatx4 *acc, const float2 *tab, int nhi,
                                               int64_t t, int g, float scale) {
    constexpr int HALF = D / 2;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        float lo[4], hi[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int x = 16 * dt + 4 * g + r;
            const float2 cs = rope_cs(tab, nhi, HALF, t, x);
            const float a = scale * acc[dt][r], b = scale * acc[dt + D / 32][r];
            lo[r] = a * cs.x + b * cs.y;
            hi[r] = b * cs.x - a * cs.y;
        }
        *reinterpret_cast<float4 *>(dst_row + 16 * dt + 4 * g) = make_float4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<float4 *>(dst_row + HALF + 16 * dt + 4 * g) = make_float4(hi[0], hi[1], hi[2], hi[3]);
    }
}
}  // namespace

// ---- window, query side. Work-group: 64 queries of one head, 16 per wave (one per
// lane column), over 32-key tiles. S^T = K Q^T and dP^T = V dO^T put keys 4 g + r of
// query c in lane (c, g). Pass A: the row's log-sum-exp and D = sum_j P_j (dO . v_j)
// (from this pass's own fp32 arithmetic: the forward's window output holds
// fp16-operand rounding that would otherwise enter every dS). Pass B: dS, and
// dq^T += K^T dS^T with dS^T straight from the accumulator layout.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_win_dq_kernel(const float *__restrict__ qr,
                                                            const float *__restrict__ kr,
                                                            const float *__restrict__ vf,
                                                            const float *__restrict__ dO,
                                                            const float2 *__restrict__ tab, int nhi,
                                                            float *__restrict__ dq, float *__restrict__ lse_w,
                                                            float *__restrict__ D_w, KParams p) {
    constexpr int KS = D / 4;
    __shared__ __attribute__((aligned(1024))) float s_k0[kWinTile * D];
    __shared__ __attribute__((aligned(1024))) float s_k1[kWinTile * D];
    __shared__ __attribute__((aligned(1024))) float s_v0[kWinTile * D];
    __shared__ __attribute__((aligned(1024))) float s_v1[kWinTile * D];
    const int ntile = (int)((p.N + kWinRows - 1) / kWinRows);
    const int logical = xcd_remap((int)blockIdx.x, ntile * p.H);
    const int h = logical / ntile;
    const int64_t q0 = (int64_t)(logical % ntile) * kWinRows;
    const int64_t hN = (int64_t)h * p.N;
    const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t qw = q0 + 16 * wave;
    const int64_t i = qw + col;
    float qb[KS], ob[KS];
    {
        const int64_t ic = min(i, p.N - 1);
        wrow_quarter<D>(qr + (hN + ic) * D, g, qb);
        wrow_quarter<D>(dO + (hN + ic) * D, g, ob);
    }
    const int64_t kmin = max((int64_t)0, q0 - p.w + 1);
    const int64_t kmax = min(p.N, q0 + kWinRows) - 1;
    const int t_first = (int)(kmin / kWinTile), t_last = (int)(kmax / kWinTile);
    const float *kh = kr + hN * D, *vh = vf + hN * D;
    auto issue = [&](int t, float *kb, float *vb) __attribute__((always_inline)) {
        wtile_issue<D>(kh, (int64_t)t * kWinTile, p.N, kb, wave, lane);
        wtile_issue<D>(vh, (int64_t)t * kWinTile, p.N, vb, wave, lane);
    };
    // a 16-key block holds a key of one of this wave's windows
    auto block_live = [&](int64_t kb0) __attribute__((always_inline)) {
        return qw < p.N && kb0 <= qw + 15 && kb0 + 15 > qw - p.w;
    };
    auto valid = [&](int64_t j) __attribute__((always_inline)) { return i < p.N && j <= i && j > i - p.w; };
    // every tile, double-buffered; body(t, keys, values)
    auto sweep = [&](auto &&body) __attribute__((always_inline)) {
        issue(t_first, s_k0, s_v0);
        wait_vmem();
        __syncthreads();
        for (int t = t_first; t <= t_last; t += 2) {
            if (t + 1 <= t_last) issue(t + 1, s_k1, s_v1);
            body(t, s_k0, s_v0);
            wait_vmem();
            __syncthreads();
            if (t + 1 > t_last) break;
            if (t + 2 <= t_last) issue(t + 2, s_k0, s_v0);
            body(t + 1, s_k1, s_v1);
            wait_vmem();
            __syncthreads();
        }
    };

    // pass A: each lane runs (max, sum, weighted dP) over its keys, then the four
    // lanes of a query merge theirs
    float m = -INFINITY, l = 0.0f, a = 0.0f;
    sweep([&](int t, const float *kb, const float *vb) {
#pragma unroll
        for (int kk = 0; kk < kWinTile / 16; ++kk) {
            const int64_t kb0 = (int64_t)t * kWinTile + 16 * kk;
            if (!block_live(kb0)) continue;
            const floatx4 sv = wtile_dot<D>(kb, 16 * kk, col, g, qb);
            const floatx4 dp = wtile_dot<D>(vb, 16 * kk, col, g, ob);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!valid(kb0 + 4 * g + r)) continue;
                const float sc = sv[r] * p.scale;
                const float mn = fmaxf(m, sc);
                const float alpha = __expf(m - mn), e = __expf(sc - mn);
                l = l * alpha + e;
                a = a * alpha + e * dp[r];
                m = mn;
            }
        }
    });
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(m, o), l2 = __shfl_xor(l, o), a2 = __shfl_xor(a, o);
        const float mn = fmaxf(m, m2);
        const float f1 = m == -INFINITY ? 0.0f : __expf(m - mn);
        const float f2 = m2 == -INFINITY ? 0.0f : __expf(m2 - mn);
        l = l * f1 + l2 * f2;
        a = a * f1 + a2 * f2;
        m = mn;
    }
    const float lse = m + __logf(l);
    const float Dr = l > 0.0f ? a / l : 0.0f;

    // pass B: dS^T and dq^T += K^T dS^T
    floatx4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    sweep([&](int t, const float *kb, const float *vb) {
#pragma unroll
        for (int kk = 0; kk < kWinTile / 16; ++kk) {
            const int64_t kb0 = (int64_t)t * kWinTile + 16 * kk;
            if (!block_live(kb0)) continue;
            const floatx4 sv = wtile_dot<D>(kb, 16 * kk, col, g, qb);
            const floatx4 dp = wtile_dot<D>(vb, 16 * kk, col, g, ob);
            float ds[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float P = valid(kb0 + 4 * g + r) ? __expf(sv[r] * p.scale - lse) : 0.0f;
                ds[r] = P * (dp[r] - Dr);
            }
            wtile_tmul<D>(kb, 16 * kk, col, g, ds, acc);
        }
    });
    if (i >= p.N) return;
    // dq = R(i)^T (scale acc)
    wstore_rotated<D>(dq + (hN + i) * D, acc, tab, nhi, i, g, p.scale);
    if (g == 0) {
        lse_w[hN + i] = lse;
        D_w[hN + i] = Dr;
    }
}

// ---- window, key side. Work-group: 64 keys of one head, 16 per wave (one per lane
// column), over the 32-query tiles whose windows hold them. S = Q K^T and
// dP = dO V^T put queries 4 g + r of key c in lane (c, g); dv^T += dO^T P and
// dk^T += Q^T dS take P and dS straight from the accumulator layout.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_win_dkv_kernel(const float *__restrict__ qr,
                                                             const float *__restrict__ kr,
                                                             const float *__restrict__ vf,
                                                             const float *__restrict__ dO,
                                                             const float *__restrict__ lse_w,
                                                             const float *__restrict__ D_w,
                                                             const float2 *__restrict__ tab, int nhi,
                                                             float *__restrict__ dk, float *__restrict__ dv,
                                                             KParams p) {
    constexpr int KS = D / 4;
    __shared__ __attribute__((aligned(1024))) float s_q0[kWinTile * D];
    __shared__ __attribute__((aligned(1024))) float s_q1[kWinTile * D];
    __shared__ __attribute__((aligned(1024))) float s_o0[kWinTile * D];
    __shared__ __attribute__((aligned(1024))) float s_o1[kWinTile * D];
    const int ntile = (int)((p.N + kWinRows - 1) / kWinRows);
    const int logical = xcd_remap((int)blockIdx.x, ntile * p.H);
    const int h = logical / ntile;
    const int64_t k0 = (int64_t)(logical % ntile) * kWinRows;
    const int64_t hN = (int64_t)h * p.N;
    const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t kw = k0 + 16 * wave;
    const int64_t j = kw + col;
    float kb[KS], vb[KS];
    {
        const int64_t jc = min(j, p.N - 1);
        wrow_quarter<D>(kr + (hN + jc) * D, g, kb);
        wrow_quarter<D>(vf + (hN + jc) * D, g, vb);
    }
    // queries whose windows hold one of these keys: k0 .. k0 + 63 + w - 1
    const int64_t qmax = min(p.N, k0 + kWinRows + (int64_t)p.w - 1) - 1;
    const int t_first = (int)(k0 / kWinTile), t_last = (int)(qmax / kWinTile);
    const float *qh = qr + hN * D, *oh = dO + hN * D;
    auto issue = [&](int t, float *qt, float *ot) __attribute__((always_inline)) {
        wtile_issue<D>(qh, (int64_t)t * kWinTile, p.N, qt, wave, lane);
        wtile_issue<D>(oh, (int64_t)t * kWinTile, p.N, ot, wave, lane);
    };
    // a 16-query block holds a query whose window holds one of this wave's keys
    auto block_live = [&](int64_t qb0) __attribute__((always_inline)) {
        return kw < p.N && qb0 < p.N && qb0 + 15 >= kw && qb0 <= kw + 15 + p.w - 1;
    };
    floatx4 acck[D / 16], accv[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acck[dt] = accv[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto body = [&](int t, const float *qt, const float *ot) __attribute__((always_inline)) {
#pragma unroll
        for (int qq = 0; qq < kWinTile / 16; ++qq) {
            const int64_t qb0 = (int64_t)t * kWinTile + 16 * qq;
            if (!block_live(qb0)) continue;
            const floatx4 sv = wtile_dot<D>(qt, 16 * qq, col, g, kb);
            const floatx4 dp = wtile_dot<D>(ot, 16 * qq, col, g, vb);
            float P[4], ds[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t ii = qb0 + 4 * g + r;
                const bool ok = j < p.N && ii < p.N && j <= ii && j > ii - p.w;
                const int64_t ic = min(ii, p.N - 1);
                const float pr = ok ? __expf(sv[r] * p.scale - lse_w[hN + ic]) : 0.0f;
                P[r] = pr;
                ds[r] = ok ? pr * (dp[r] - D_w[hN + ic]) : 0.0f;
            }
            wtile_tmul<D>(ot, 16 * qq, col, g, P, accv);
            wtile_tmul<D>(qt, 16 * qq, col, g, ds, acck);
        }
    };
    issue(t_first, s_q0, s_o0);
    wait_vmem();
    __syncthreads();
    for (int t = t_first; t <= t_last; t += 2) {
        if (t + 1 <= t_last) issue(t + 1, s_q1, s_o1);
        body(t, s_q0, s_o0);
        wait_vmem();
        __syncthreads();
        if (t + 1 > t_last) break;
        if (t + 2 <= t_last) issue(t + 2, s_q0, s_o0);
        body(t + 1, s_q1, s_o1);
        wait_vmem();
        __syncthreads();
    }
    if (j >= p.N) return;
    wstore_rotated<D>(dk + (hN + j) * D, acck, tab, nhi, j, g, p.scale);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<float4 *>(dv + (hN + j) * D + 16 * dt + 4 * g) =
            make_float4(accv[dt][0], accv[dt][1], accv[dt][2], accv[dt][3]);
}

// ---- the (query, rank) pairs as sort keys: key = head * C + cell (or H * C when the
// rank is empty, which sorts past every cell), value = the pair's index within its
// head, query * K + rank
__global__ void bwd_pair_keys_kernel(const int32_t *__restrict__ sel, uint32_t *__restrict__ key,
                                     uint32_t *__restrict__ val, KParams p) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)p.H * p.N * p.K) return;
    const int64_t h = e / ((int64_t)p.N * p.K);
    const int32_t c = sel[e];
    key[e] = c >= 0 ? (uint32_t)(h * p.C + c) : (uint32_t)(p.H * p.C);
    val[e] = (uint32_t)(e - h * p.N * p.K);
}

// ---- each cell's run [seg[2 c], seg[2 c + 1]) of the sorted pairs (empty: 0, 0); the
// two work-list counters start at zero
__global__ void bwd_seg_init_kernel(int32_t *__restrict__ seg, int64_t n, int32_t *__restrict__ counters) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < 2 * n) seg[e] = 0;
    if (e < 2) counters[e] = 0;
}

// ---- cells chosen by more than kHeavyPairs queries (a planted needle is chosen by
// nearly every later query) are split into chunks of kHeavyPairs pairs, one work-group
// each: items[i] = (cell, chunk), heavy[h] = (cell, first item, chunks). The slots a
// cell gets depend on the order of the atomics, but its chunks stay consecutive and
// are summed in chunk order, so results do not.
__global__ void bwd_heavy_list_kernel(const int32_t *__restrict__ seg, int64_t ncell, int32_t *__restrict__ counters,
                                      int32_t *__restrict__ items, int32_t *__restrict__ heavy) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= ncell) return;
    const int32_t cnt = seg[2 * c + 1] - seg[2 * c];
    if (cnt <= kHeavyPairs) return;
    const int32_t n = (cnt + kHeavyPairs - 1) / kHeavyPairs;
    const int32_t base = atomicAdd(&counters[0], n);
    const int32_t hc = atomicAdd(&counters[1], 1);
    heavy[3 * hc] = (int32_t)c;
    heavy[3 * hc + 1] = base;
    heavy[3 * hc + 2] = n;
    for (int32_t j = 0; j < n; ++j) {
        items[2 * (base + j)] = (int32_t)c;
        items[2 * (base + j) + 1] = j;
    }
}

__global__ void bwd_seg_mark_kernel(const uint32_t *__restrict__ key, int64_t n, uint32_t ncell,
                                    int32_t *__restrict__ seg) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    const uint32_t c = key[e];
    if (c >= ncell) return;
    if (e == 0 || key[e - 1] != c) seg[2 * (int64_t)c] = (int32_t)e;
    if (e == n - 1 || key[e + 1] != c) seg[2 * (int64_t)c + 1] = (int32_t)(e + 1);
}

// ---- long branch, key side. CHUNKS = false: one work-group per (head, cell) with at
// most kHeavyPairs selectors, adding to dk, dv; CHUNKS = true: one work-group per
// chunk of a heavier cell, writing its sums to part[item]. The cell's keys and values
// wait in LDS; one wave per 16 of the cell's tokens takes them as B operands of the
// fp32 matrix cores (dims (d/4) g .. of token c in lane (c, g)); the queries that selected the cell,
// in query order (a stable sort of the pairs by cell), are gathered 16 at a time into
// LDS (q as fp32 and unrotated, written by bwd_long_merge: the long branch has no
// RoPE; and the gradient reaching the softmax output). S = Q K^T and dP = do V^T put queries 4 g + r of token c in
// lane (c, g); P = exp(scale S - lse), dS = P (dP - D), then dv^T += do^T P and
// dk^T += Q^T dS (times the scale) take P and dS straight from that layout. dS also
// goes to LDS transposed, where dq^T = K^T dS^T (times the scale) over all the cell's
// tokens gives each selector's dq from this cell: wave w forms dims (d / waves) w ..
// from the cell's keys in LDS and writes them to the selector's (query, rank) row of
// dqp, which bwd_dq_long_sum adds to dq in rank order.
namespace {
// 16 bytes of T at p as four floats (4 fp32, or 4 bf16 from 8 bytes)
template <typename T> __device__ __forceinline__ float4 ld4f(const T *p);
template <> __device__ __forceinline__ float4 ld4f<float>(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}
template <> __device__ __forceinline__ float4 ld4f<uint16_t>(const uint16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xFFFF0000u));
}
// LDS tiles of 16 rows of D elements of T, 16-byte chunk c of row r at c ^ (r mod chunks per row)
template <typename T, int D>
struct GTile {
    static constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
    static constexpr int CPR = D / EPC;              // chunks per row
    static constexpr int ELEMS = 16 * D;
    static constexpr int UNITS = ELEMS * (int)sizeof(T) / 1024;  // 1 KB copy units
    __device__ static int off(int row, int chunk) { return (row * CPR + (chunk ^ (row & (CPR - 1)))) * EPC; }
};
// the 16 bytes at an LDS chunk as floats
template <typename T> __device__ __forceinline__ void chunkf(const T *p, float *dst);
template <> __device__ __forceinline__ void chunkf<float>(const float *p, float *dst) {
    const float4 f = *reinterpret_cast<const float4 *>(p);
    dst[0] = f.x; dst[1] = f.y; dst[2] = f.z; dst[3] = f.w;
}
template <> __device__ __forceinline__ void chunkf<uint16_t>(const uint16_t *p, float *dst) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        dst[2 * e] = __uint_as_float(w[e] << 16);
        dst[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
}
// acc (rows 4 g + r of the 16 tile rows, column c) += tile rows as A (row c for this
// lane) times the lane's register operand b[] (dims (d/4) g .. of its column)
template <typename T, int D, typename BV>
__device__ __forceinline__ floatx4 gtile_dot(const T *tile, int col, int g, BV b) {
    using G = GTile<T, D>;
    constexpr int KS = D / 4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < KS / G::EPC; ++cc) {
        float a[G::EPC];
        chunkf<T>(tile + G::off(col, KS / G::EPC * g + cc), a);
#pragma unroll
        for (int e = 0; e < G::EPC; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b(G::EPC * cc + e), acc, 0, 0, 0);
    }
    return acc;
}
// a token's d/4 values (dims (d/4) g ..) as MFMA B operands: fp32 as they are, bf16
// packed two to a register and widened at each use
template <typename T, int KS>
struct BRow;
template <int KS>
struct BRow<float, KS> {
    float x[KS];
    __device__ void load(const float *src) {
#pragma unroll
        for (int i = 0; i < KS / 4; ++i) {
            const float4 f = *reinterpret_cast<const float4 *>(src + 4 * i);
            x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
        }
    }
    // the same dims of row `row` of a GTile
    template <int D> __device__ void load_tile(const float *tile, int row, int g) {
        using G = GTile<float, D>;
#pragma unroll
        for (int i = 0; i < KS / 4; ++i) {
            const float4 f = *reinterpret_cast<const float4 *>(tile + G::off(row, KS / 4 * g + i));
            x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
        }
    }
    __device__ float operator()(int i) const { return x[i]; }
};
template <int KS>
struct BRow<uint16_t, KS> {
    uint32_t w[KS / 2];
    __device__ void load(const uint16_t *src) {
#pragma unroll
        for (int i = 0; i < KS / 8; ++i) {
            const uint4 u = *reinterpret_cast<const uint4 *>(src + 8 * i);
            w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
        }
    }
    template <int D> __device__ void load_tile(const uint16_t *tile, int row, int g) {
        using G = GTile<uint16_t, D>;
#pragma unroll
        for (int i = 0; i < KS / 8; ++i) {
            const uint4 u = *reinterpret_cast<const uint4 *>(tile + G::off(row, KS / 8 * g + i));
            w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
        }
    }
    __device__ float operator()(int i) const {
        return __uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
    }
};
// acc[dt] (dims 16 dt + 4 g + r, column c) += sum over the tile rows of tile[row][dim]
// w(row, c), with w(4 g + r, c) = w[r] held by lane (c, g)
template <typename T, int D>
__device__ __forceinline__ void gtile_tmul(const T *tile, int col, int g, const float *w, floatx4 *acc) {
    using G = GTile<T, D>;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * dt + col;
            const float a = to_f32<T>(tile[G::off(4 * g + r, d / G::EPC) + d % G::EPC]);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, w[r], acc[dt], 0, 0, 0);
        }
}
// acc[dt] (dims 16 (dt0 + dt) + 4 g + r, column c) += sum over the tile rows of
// tile[row][dim] w(row, c), as gtile_tmul for NDT of the D / 16 dim tiles
template <typename T, int D, int NDT>
__device__ __forceinline__ void gtile_tmul_part(const T *tile, int dt0, int col, int g, const float *w, floatx4 *acc) {
    using G = GTile<T, D>;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * (dt0 + dt) + col;
            const float a = to_f32<T>(tile[G::off(4 * g + r, d / G::EPC) + d % G::EPC]);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, w[r], acc[dt], 0, 0, 0);
        }
}
// rows src_rows[r] (r < 16) of a [rows][D] array of T into a tile, by the NWV waves
template <typename T, int D, int NWV>
__device__ __forceinline__ void gtile_issue(const T *base, const int64_t *rows, T *tile, int wave, int lane) {
    using G = GTile<T, D>;
    for (int u = __builtin_amdgcn_readfirstlane(wave); u < G::UNITS; u += NWV) {
        const int pc = 64 * u + lane;  // chunk of the tile
        const int r = pc / G::CPR, phys = pc % G::CPR;
        lds_dma16(base + rows[r] * D + G::EPC * (phys ^ (r & (G::CPR - 1))), tile + 64 * G::EPC * u);
    }
}

// the selectors e0 .. e1 - 1 (sorted pairs) of a light cell, or of one chunk of a heavy one
template <bool CHUNKS>
__device__ __forceinline__ bool cell_run(const int32_t *seg, const int32_t *items, const int32_t *counters,
                                         int64_t &cid, int64_t &e0, int64_t &e1) {
    if constexpr (CHUNKS) {
        if ((int)blockIdx.x >= counters[0]) return false;
        cid = items[2 * blockIdx.x];
        const int64_t j = items[2 * blockIdx.x + 1];
        const int64_t a = seg[2 * cid], z = seg[2 * cid + 1];
        e0 = a + j * kHeavyPairs;
        e1 = min(z, e0 + kHeavyPairs);
        return true;
    } else {
        cid = blockIdx.x;
        e0 = seg[2 * cid];
        e1 = seg[2 * cid + 1];
        return e0 < e1 && e1 - e0 <= kHeavyPairs;  // never selected, or taken in chunks
    }
}
// the S tokens' rows of a [rows][D] array of T from row r0, one GTile per 16 tokens
template <typename T, int D, int S, int NTH>
__device__ __forceinline__ void cell_tiles(const T *src, int64_t r0, T *dst) {
    using G = GTile<T, D>;
    for (int pc = threadIdx.x; pc < S * G::CPR; pc += NTH) {
        const int tk = pc / G::CPR, ch = pc % G::CPR;
        *reinterpret_cast<uint4 *>(dst + (tk / 16) * G::ELEMS + G::off(tk % 16, ch)) =
            *reinterpret_cast<const uint4 *>(src + (r0 + tk) * D + G::EPC * ch);
    }
}
}  // namespace

// ---- long branch, forward recompute, per cell: for each selector of the cell (light
// cells whole, heavy ones in chunks), the cell's share of the selector's softmax:
// m = the largest scaled score over the cell's tokens, l = sum_j exp(scale s_j - m),
// o = sum_j exp(scale s_j - m) v_j, written to the selector's (query, rank) row (o to
// po, (m, l) to pml); bwd_long_merge combines a query's rows. The cell's keys and values
// wait in LDS; each wave takes 16 selectors at a time, their queries as B operands
// (dims (d/4) g .. of selector c in lane (c, g)), so that S^T = K Q^T puts tokens
// 4 g + r of selector c in lane (c, g) and P^T feeds o^T = V^T P^T from that layout.
template <typename T, int D, int S, bool CHUNKS>
__global__ __launch_bounds__(256) void bwd_long_fwd_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                           const T *__restrict__ v, const uint32_t *__restrict__ sq,
                                                           const int32_t *__restrict__ seg,
                                                           const int32_t *__restrict__ items,
                                                           const int32_t *__restrict__ counters,
                                                           float *__restrict__ po, float2 *__restrict__ pml,
                                                           KParams p) {
    constexpr int NW = 4;       // waves
    constexpr int KS = D / 4;
    constexpr int NT = S / 16;  // 16-token tiles of the cell
    using G = GTile<T, D>;
    __shared__ __attribute__((aligned(16))) T s_k[S * D];
    __shared__ __attribute__((aligned(16))) T s_v[S * D];
    int64_t cid, e0, e1;
    if (!cell_run<CHUNKS>(seg, items, counters, cid, e0, e1)) return;
    const int h = (int)(cid / p.C);
    const int64_t c = cid % p.C;
    const int64_t hN = (int64_t)h * p.N, hNK = hN * p.K;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    cell_tiles<T, D, S, 64 * NW>(k, hN + c * S, s_k);
    cell_tiles<T, D, S, 64 * NW>(v, hN + c * S, s_v);
    __syncthreads();
    const int ntile = (int)((e1 - e0 + 15) / 16);
    for (int t = wave; t < ntile; t += NW) {
        const int64_t e = e0 + 16 * (int64_t)t + col;
        const bool ok = e < e1;
        const int64_t val = sq[min(e, e1 - 1)];  // query * K + rank
        const int64_t pair = hNK + val;
        BRow<T, KS> qb;
        qb.load(q + (hN + val / p.K) * D + KS * g);
        floatx4 sv[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) sv[j] = gtile_dot<T, D>(s_k + j * G::ELEMS, col, g, qb);
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, sv[j][r] * p.scale);
        m = colmax4(m);
        float P[NT][4], l = 0.0f;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                P[j][r] = __expf(sv[j][r] * p.scale - m);
                l += P[j][r];
            }
        l = colsum4(l);
        floatx4 acc[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) gtile_tmul<T, D>(s_v + j * G::ELEMS, col, g, P[j], acc);
        if (ok) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                *reinterpret_cast<float4 *>(po + pair * D + 16 * dt + 4 * g) =
                    make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
            if (g == 0) pml[pair] = make_float2(m, l);
        }
    }
}

// ---- long branch, per query (one wave, 4 per work-group): its cells' rows combined in
// rank order, M = max m_r, L = sum_r exp(m_r - M) l_r, o_long = sum_r exp(m_r - M) o_r / L,
// lse = M + log L; then RMSNorm's backward. Writes the gradient reaching the softmax
// output (do_l), the row's lse and D = do_l . o_long, the query's dgamma term, and the
// query in fp32 for the key side. Lane: dims NX lane .. NX lane + NX - 1.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_long_merge_kernel(const T *__restrict__ q, const int32_t *__restrict__ sel,
                                                                  const float *__restrict__ po,
                                                                  const float2 *__restrict__ pml,
                                                                  const float *__restrict__ dO,
                                                                  float *__restrict__ do_l, float *__restrict__ lse_l,
                                                                  float *__restrict__ D_l, float *__restrict__ dg,
                                                                  float *__restrict__ q32, KParams p) {
    constexpr int NX = D / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nqw = (int)((p.N + 3) / 4);
    const int h = blockIdx.x / nqw;
    const int64_t i = (int64_t)(blockIdx.x % nqw) * 4 + wave;
    if (i >= p.N) return;
    const int64_t hi = (int64_t)h * p.N + i;
    const int64_t row = hi * D;
    float qf[NX];
#pragma unroll
    for (int n = 0; n < NX; ++n) qf[n] = to_f32<T>(q[row + NX * lane + n]);
    // every rank's row is read at once; a rank without a cell has no row (its words are
    // whatever the workspace held) and is dropped by selects, never multiplied in
    bool ok[kMaxK];
    float2 ml[kMaxK];
    float src[kMaxK][NX], dout_[NX], y[NX];
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
        if (r >= p.K) break;
        ok[r] = sel[hi * p.K + r] >= 0;
        ml[r] = pml[hi * p.K + r];
#pragma unroll
        for (int n = 0; n < NX; ++n) src[r][n] = po[(hi * p.K + r) * D + NX * lane + n];
    }
#pragma unroll
    for (int n = 0; n < NX; ++n) dout_[n] = dO[row + NX * lane + n];
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
        if (r >= p.K) break;
        M = ok[r] ? fmaxf(M, ml[r].x) : M;
    }
#pragma unroll
    for (int n = 0; n < NX; ++n) q32[row + NX * lane + n] = qf[n];
    if (M == -INFINITY) {  // no cell: o_long = 0
        for (int x = lane; x < D; x += 64) do_l[row + x] = 0.0f;
        if (lane == 0) { lse_l[hi] = 0.0f; D_l[hi] = 0.0f; dg[hi] = 0.0f; }
        return;
    }
    float L = 0.0f, o[NX];
#pragma unroll
    for (int n = 0; n < NX; ++n) o[n] = 0.0f;
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
        if (r >= p.K) break;
        const float wr = ok[r] ? __expf(ml[r].x - M) : 0.0f;
        L += ok[r] ? wr * ml[r].y : 0.0f;
#pragma unroll
        for (int n = 0; n < NX; ++n) o[n] += ok[r] ? wr * src[r][n] : 0.0f;
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int n = 0; n < NX; ++n) o[n] *= inv;
    float ss = 0.0f;
#pragma unroll
    for (int n = 0; n < NX; ++n) ss += o[n] * o[n];
    ss = wave_sum(ss);
    const float rr = sqrtf(ss / (float)D + p.rms_eps);
    const float gam = p.gamma[h];
    float dy_y = 0.0f;
#pragma unroll
    for (int n = 0; n < NX; ++n) {
        y[n] = o[n] / rr;
        dy_y += dout_[n] * y[n];
    }
    dy_y = wave_sum(dy_y);  // dout . y
    float Dsum = 0.0f;
#pragma unroll
    for (int n = 0; n < NX; ++n) {
        const float d_o = (gam * dout_[n] - y[n] * (gam * dy_y) / (float)D) / rr;
        do_l[row + NX * lane + n] = d_o;
        Dsum += d_o * o[n];
    }
    const float Dr = wave_sum(Dsum);
    if (lane == 0) {
        lse_l[hi] = M + __logf(L);
        D_l[hi] = Dr;
        dg[hi] = dy_y;
    }
}

template <typename T, int D, int S, bool CHUNKS>
__global__ __launch_bounds__(64 * (S / 16), 2) void bwd_long_kv_kernel(const float *__restrict__ q, const T *__restrict__ k,
                                                                    const T *__restrict__ v,
                                                                    const uint32_t *__restrict__ sq,
                                                                    const int32_t *__restrict__ seg,
                                                                    const int32_t *__restrict__ items,
                                                                    const int32_t *__restrict__ counters,
                                                                    const float *__restrict__ do_l,
                                                                    const float *__restrict__ lse_l,
                                                                    const float *__restrict__ D_l,
                                                                    float *__restrict__ dk, float *__restrict__ dv,
                                                                    float *__restrict__ part, float *__restrict__ dqp,
                                                                    KParams p) {
    constexpr int NWV = S / 16;          // waves, 16 tokens each
    constexpr int KS = D / 4;
    constexpr int QT = 16;               // selectors per tile
    constexpr int DQT = D / 16 / NWV;    // 16-dim tiles of dq per wave
    constexpr int DSLD = QT + 1;         // row stride of the transposed dS
    using G = GTile<T, D>;
    static_assert(DQT >= 1 && DQT * NWV * 16 == D, "whole dq dim tiles per wave");
    // two named buffers of each kind, so that the compiler can tell a tile's copy from
    // the reads of the other buffer
    __shared__ __attribute__((aligned(1024))) float s_q0[QT * D];
    __shared__ __attribute__((aligned(1024))) float s_q1[QT * D];
    __shared__ __attribute__((aligned(1024))) float s_o0[QT * D];
    __shared__ __attribute__((aligned(1024))) float s_o1[QT * D];
    __shared__ int64_t s_rows[2][QT];              // the gathered rows of two tiles
    __shared__ int32_t s_pair[2][QT];              // their (query, rank) rows of dqp
    __shared__ __attribute__((aligned(16))) T s_k[S * D];  // the cell's keys, 16-token tiles
    __shared__ __attribute__((aligned(16))) T s_v[S * D];  // and values
    __shared__ float s_ds[S * DSLD];               // dS of the current tile, [token][selector]
    int64_t cid, e0, e1;  // head * C + cell, its selectors
    if (!cell_run<CHUNKS>(seg, items, counters, cid, e0, e1)) return;
    const int h = (int)(cid / p.C);
    const int64_t c = cid % p.C;
    const int64_t hN = (int64_t)h * p.N;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
    const int wave = tid >> 6;
    const int tok = 16 * wave + col;                  // this lane's token within the cell
    const int64_t jrow = hN + c * S + tok;
    const int64_t hNK = hN * p.K;
    // the cell's keys and values into LDS (read after the first barrier below)
    cell_tiles<T, D, S, 64 * NWV>(k, hN + c * S, s_k);
    cell_tiles<T, D, S, 64 * NWV>(v, hN + c * S, s_v);
    floatx4 acck[D / 16], accv[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acck[dt] = accv[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Tile t: selectors e0 + 16 t + r, their rows in s_rows[t % 2] (past e1: the last
    // selector again, masked). Per tile: the lse and D loads and the row prefetch for
    // tile t + 2 go out before the copies of tile t + 1, which are issued every tile
    // (a repeat past the end), so that waiting for those loads never waits for a copy.
    const int ntile = (int)((e1 - e0 + QT - 1) / QT);
    // the sorted pairs hold query * K + rank
    auto sel_val = [&](int t) __attribute__((always_inline)) {
        return (int64_t)sq[min(e0 + (int64_t)QT * t + (tid & (QT - 1)), e1 - 1)];
    };
    auto issue = [&](int slot, float *bq, float *bo) __attribute__((always_inline)) {
        gtile_issue<float, D, NWV>(q, s_rows[slot], bq, wave, lane);
        gtile_issue<float, D, NWV>(do_l, s_rows[slot], bo, wave, lane);
    };
    auto step = [&](int t, const float *bq, const float *bo, float *nq, float *no) __attribute__((always_inline)) {
        const int slot = t & 1;
        float lv[4], dd[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t ii = s_rows[slot][4 * g + r];
            lv[r] = lse_l[ii];
            dd[r] = D_l[ii];
        }
        const int64_t nval = sel_val(t + 2);
        issue(slot ^ 1, nq, no);  // tile t + 1
        // this lane's token as B operands: dims KS g .. KS g + KS - 1
        BRow<T, KS> kb, vb;
        kb.template load_tile<D>(s_k + wave * G::ELEMS, col, g);
        const floatx4 sv = gtile_dot<float, D>(bq, col, g, kb);
        vb.template load_tile<D>(s_v + wave * G::ELEMS, col, g);
        const floatx4 dp = gtile_dot<float, D>(bo, col, g, vb);
        float P[4], ds[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = e0 + (int64_t)QT * t + 4 * g + r < e1;
            const float pr = ok ? __expf(sv[r] * p.scale - lv[r]) : 0.0f;
            P[r] = pr;
            ds[r] = ok ? pr * (dp[r] - dd[r]) : 0.0f;
        }
        gtile_tmul<float, D>(bo, col, g, P, accv);
        gtile_tmul<float, D>(bq, col, g, ds, acck);
#pragma unroll
        for (int r = 0; r < 4; ++r) s_ds[tok * DSLD + 4 * g + r] = ds[r];
        const int64_t prow = hNK + s_pair[slot][col];  // this lane's column of the dq tile
        const bool pok = e0 + (int64_t)QT * t + col < e1;
        wait_vmem();
        __syncthreads();  // tile t + 1 has landed; every wave is done with this tile and its rows
        float w[NWV][4];
#pragma unroll
        for (int j = 0; j < NWV; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) w[j][r] = s_ds[(16 * j + 4 * g + r) * DSLD + col];
        // one 16-dim tile at a time, each stored before the next, to keep few registers live
#pragma unroll 1
        for (int dt = 0; dt < DQT; ++dt) {
            floatx4 accq = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NWV; ++j)
                gtile_tmul_part<T, D, 1>(s_k + j * G::ELEMS, DQT * wave + dt, col, g, w[j], &accq);
            if (pok)
                *reinterpret_cast<float4 *>(dqp + prow * D + 16 * (DQT * wave + dt) + 4 * g) =
                    make_float4(p.scale * accq[0], p.scale * accq[1], p.scale * accq[2], p.scale * accq[3]);
        }
        if (tid < QT) {
            s_rows[slot][tid] = hN + nval / p.K;
            s_pair[slot][tid] = (int32_t)nval;
        }
        __syncthreads();
    };
    if (tid < QT) {
        const int64_t v0 = sel_val(0), v1 = sel_val(1);
        s_rows[0][tid] = hN + v0 / p.K;
        s_rows[1][tid] = hN + v1 / p.K;
        s_pair[0][tid] = (int32_t)v0;
        s_pair[1][tid] = (int32_t)v1;
    }
    __syncthreads();
    issue(0, s_q0, s_o0);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < ntile; t += 2) {
        step(t, s_q0, s_o0, s_q1, s_o1);
        if (t + 1 >= ntile) break;
        step(t + 1, s_q1, s_o1, s_q0, s_o0);
    }
    // dims 16 dt + 4 g + r of token tok
    if constexpr (CHUNKS) {
        // chunk sums: dk part then dv part, [S][D] each
        float *dst = part + (int64_t)blockIdx.x * 2 * S * D + (int64_t)tok * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            *reinterpret_cast<float4 *>(dst + 16 * dt + 4 * g) =
                make_float4(p.scale * acck[dt][0], p.scale * acck[dt][1], p.scale * acck[dt][2], p.scale * acck[dt][3]);
            *reinterpret_cast<float4 *>(dst + S * D + 16 * dt + 4 * g) =
                make_float4(accv[dt][0], accv[dt][1], accv[dt][2], accv[dt][3]);
        }
    } else {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            float4 *pk = reinterpret_cast<float4 *>(dk + jrow * D + 16 * dt + 4 * g);
            float4 *pv = reinterpret_cast<float4 *>(dv + jrow * D + 16 * dt + 4 * g);
            float4 a4 = *pk, b4 = *pv;
            a4.x += p.scale * acck[dt][0]; a4.y += p.scale * acck[dt][1];
            a4.z += p.scale * acck[dt][2]; a4.w += p.scale * acck[dt][3];
            b4.x += accv[dt][0]; b4.y += accv[dt][1]; b4.z += accv[dt][2]; b4.w += accv[dt][3];
            *pk = a4;
            *pv = b4;
        }
    }
}

// ---- a heavy cell's chunk sums added to dk, dv in chunk order
template <int D, int S>
__global__ __launch_bounds__(kThreads) void bwd_heavy_reduce_kernel(const int32_t *__restrict__ heavy,
                                                                    const int32_t *__restrict__ counters,
                                                                    const float *__restrict__ part,
                                                                    float *__restrict__ dk, float *__restrict__ dv,
                                                                    KParams p) {
    if ((int)blockIdx.x >= counters[1]) return;
    const int64_t cid = heavy[3 * blockIdx.x];
    const int64_t base = heavy[3 * blockIdx.x + 1];
    const int n = heavy[3 * blockIdx.x + 2];
    const int h = (int)(cid / p.C);
    const int64_t c = cid % p.C;
    const int64_t t0 = (int64_t)h * p.N + c * S;  // the cell's first token row
    for (int e = threadIdx.x; e < S * D; e += kThreads) {
        float sk = 0.0f, sv = 0.0f;
        for (int jj = 0; jj < n; ++jj) {
            const float *src = part + (base + jj) * 2 * S * D;
            sk += src[e];
            sv += src[S * D + e];
        }
        dk[t0 * D + e] += sk;
        dv[t0 * D + e] += sv;
    }
}

// ---- the long branch's dq: each query's (query, rank) rows of dqp added to dq in rank
// order (ranks without a cell have no row); one thread per 4 dims
__global__ __launch_bounds__(kThreads) void bwd_dq_long_sum_kernel(const int32_t *__restrict__ sel,
                                                                   const float *__restrict__ dqp,
                                                                   float *__restrict__ dq, KParams p) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int d4 = p.d / 4;
    if (e >= (int64_t)p.H * p.N * d4) return;
    const int64_t row = e / d4;  // head * N + query
    const int x = 4 * (int)(e % d4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < p.K; ++r) {
        if (sel[row * p.K + r] < 0) continue;
        const float4 v = *reinterpret_cast<const float4 *>(dqp + (row * p.K + r) * p.d + x);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    float4 *o = reinterpret_cast<float4 *>(dq + row * p.d + x);
    float4 a = *o;
    a.x += acc.x; a.y += acc.y; a.z += acc.z; a.w += acc.w;
    *o = a;
}

// ---- dgamma of each head: the per-query terms summed in a fixed order
constexpr int kDgThreads = 1024;
__global__ __launch_bounds__(kDgThreads) void bwd_dgamma_kernel(const float *__restrict__ dg, float *__restrict__ dgamma,
                                                                KParams p) {
    // one work-group per head: each thread adds its strided share in order (eight loads
    // in flight per step), then the waves' sums are added in a fixed order
    __shared__ float s_part[kDgThreads / 64];
    const int h = blockIdx.x;
    const float *src = dg + (int64_t)h * p.N;
    float acc = 0.0f;
    int64_t t = threadIdx.x;
    for (; t + 7 * kDgThreads < p.N; t += 8 * kDgThreads) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[t + u * kDgThreads];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; t < p.N; t += kDgThreads) acc += src[t];
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.0f;
        for (int w = 0; w < kDgThreads / 64; ++w) s += s_part[w];
        dgamma[h] = s;
    }
}

template <typename T, typename TO, int D, int S>
static hipError_t launch_bwd_typed(const void *q_, const void *k_, const void *v_, const void *dout_,
                                   const int32_t *sel, const int32_t *pool, const BwdWork &w,
                                   float *dq, float *dk, float *dv, float *dgamma, const KParams &p, hipStream_t st) {
    const T *q = (const T *)q_, *k = (const T *)k_, *v = (const T *)v_;
    const TO *dout = (const TO *)dout_;
    const int nhi = rope_abs_rows_hi(p);
    hipError_t e = launch_rope_abs_table(w.rope, w.status, p, st);
    if (e != hipSuccess) return e;
    const int64_t pairs = (int64_t)p.H * p.N * (D / 2);
    // the window kernels read fp32 values from do_l's storage, which the long branch's
    // merge kernel fills only after them
    float *vf = w.do_l;
    hipLaunchKernelGGL((bwd_prep_kernel<T, TO, D>), dim3((unsigned)((pairs + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, st, q, k, v, dout, w.rope, nhi, w.qr, w.kr, vf, w.dO, p);
    const unsigned tiles = (unsigned)(((p.N + kWinRows - 1) / kWinRows) * p.H);
    hipLaunchKernelGGL((bwd_win_dq_kernel<D>), dim3(tiles), dim3(256), 0, st, w.qr, w.kr, vf, w.dO, w.rope, nhi, dq,
                       w.lse_w, w.D_w, p);
    hipLaunchKernelGGL((bwd_win_dkv_kernel<D>), dim3(tiles), dim3(256), 0, st, w.qr, w.kr, vf, w.dO, w.lse_w, w.D_w,
                       w.rope, nhi, dk, dv, p);
    const unsigned qw = (unsigned)(((p.N + 3) / 4) * p.H);
    const int64_t npair = (int64_t)p.H * p.N * p.K;
    const int64_t ncell = (int64_t)p.H * p.C;
    const int64_t mi = heavy_items_max(p), mh = heavy_cells_max(p);
    const uint32_t *sval = nullptr;
    // the long branch's per-pair rows: first the forward recompute's o (then its dq) in dqp
    float *po = w.dqp;
    if (p.C > 0) {
        // each cell's selecting queries in query order: a stable sort of the pairs by cell
        hipLaunchKernelGGL(bwd_pair_keys_kernel, dim3((unsigned)((npair + 255) / 256)), dim3(256), 0, st, sel,
                           w.pkey, w.pval, p);
        bool in_tmp = false;
        e = launch_sort_pairs(w.pkey, w.pval, w.pkey2, w.pval2, w.shist, w.stot, npair, pair_key_bits(p), &in_tmp,
                              st);
        if (e != hipSuccess) return e;
        const uint32_t *skey = in_tmp ? w.pkey2 : w.pkey;
        sval = in_tmp ? w.pval2 : w.pval;
        hipLaunchKernelGGL(bwd_seg_init_kernel, dim3((unsigned)((2 * ncell + 255) / 256)), dim3(256), 0, st, w.cseg,
                           ncell, w.hcount);
        hipLaunchKernelGGL(bwd_seg_mark_kernel, dim3((unsigned)((npair + 255) / 256)), dim3(256), 0, st, skey, npair,
                           (uint32_t)ncell, w.cseg);
        hipLaunchKernelGGL(bwd_heavy_list_kernel, dim3((unsigned)((ncell + 255) / 256)), dim3(256), 0, st, w.cseg,
                           ncell, w.hcount, w.hitems, w.hcells);
        hipLaunchKernelGGL((bwd_long_fwd_kernel<T, D, S, false>), dim3((unsigned)ncell), dim3(256), 0, st, q, k, v,
                           sval, w.cseg, w.hitems, w.hcount, po, w.pml, p);
        if (mi > 0)
            hipLaunchKernelGGL((bwd_long_fwd_kernel<T, D, S, true>), dim3((unsigned)mi), dim3(256), 0, st, q, k, v,
                               sval, w.cseg, w.hitems, w.hcount, po, w.pml, p);
    }
    // the merge also leaves the queries in fp32, unrotated, in qr's storage, which the
    // window kernels no longer need
    float *q32 = w.qr;
    hipLaunchKernelGGL((bwd_long_merge_kernel<T, D>), dim3(qw), dim3(kThreads), 0, st, q, sel, po, w.pml, w.dO, w.do_l,
                       w.lse_l, w.D_l, w.dg, q32, p);
    if (p.C > 0) {
        hipLaunchKernelGGL((bwd_long_kv_kernel<T, D, S, false>), dim3((unsigned)ncell), dim3(64 * (S / 16)), 0, st, q32, k,
                           v, sval, w.cseg, w.hitems, w.hcount, w.do_l, w.lse_l, w.D_l, dk, dv, w.hpart, w.dqp, p);
        if (mi > 0) {
            hipLaunchKernelGGL((bwd_long_kv_kernel<T, D, S, true>), dim3((unsigned)mi), dim3(64 * (S / 16)), 0, st, q32, k,
                               v, sval, w.cseg, w.hitems, w.hcount, w.do_l, w.lse_l, w.D_l, dk, dv, w.hpart, w.dqp, p);
            hipLaunchKernelGGL((bwd_heavy_reduce_kernel<D, S>), dim3((unsigned)mh), dim3(kThreads), 0, st, w.hcells,
                               w.hcount, w.hpart, dk, dv, p);
        }
        const int64_t n4 = (int64_t)p.H * p.N * (p.d / 4);
        hipLaunchKernelGGL(bwd_dq_long_sum_kernel, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           st, sel, w.dqp, dq, p);
    }
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3((unsigned)p.H), dim3(kDgThreads), 0, st, w.dg, dgamma, p);
    return hipGetLastError();
}

template <typename T, typename TO>
static hipError_t launch_bwd_dt(const void *q, const void *k, const void *v, const void *dout, const int32_t *sel,
                                const int32_t *pool, const BwdWork &w, float *dq, float *dk,
                                float *dv, float *dgamma, const KParams &p, hipStream_t st) {
#define FSL_BWD(DD, SS) \
    launch_bwd_typed<T, TO, DD, SS>(q, k, v, dout, sel, pool, w, dq, dk, dv, dgamma, p, st)
    if (p.d == 64) {
        if (p.s == 16) return FSL_BWD(64, 16);
        if (p.s == 32) return FSL_BWD(64, 32);
        return FSL_BWD(64, 64);
    }
    if (p.s == 16) return FSL_BWD(128, 16);
    if (p.s == 32) return FSL_BWD(128, 32);
    return FSL_BWD(128, 64);
#undef FSL_BWD
}

hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const void *dout, const int32_t *sel,
                           const int32_t *pool, const BwdWork &w, float *dq, float *dk, float *dv,
                           float *dgamma, const KParams &p, hipStream_t st) {
    if (p.dtype == FSL_BF16)
        return p.out_dtype == FSL_BF16
                   ? launch_bwd_dt<uint16_t, uint16_t>(q, k, v, dout, sel, pool, w, dq, dk, dv, dgamma, p, st)
                   : launch_bwd_dt<uint16_t, float>(q, k, v, dout, sel, pool, w, dq, dk, dv, dgamma, p, st);
    return launch_bwd_dt<float, float>(q, k, v, dout, sel, pool, w, dq, dk, dv, dgamma, p, st);
}

}  // namespace fsl

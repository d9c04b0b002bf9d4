// Local branch for bf16 inputs: RoPE attention over the window [i-w+1, i]
// (FreeSolo digest, core method and step 2; prerequisites: RoPE rotates q_i
// and k_j so that their product depends only on the offset j - i).
//
// Tiling and operands as in the generic window kernel (window.hip), but 128
// queries per workgroup as 8 waves x 16 queries (one MFMA query tile per wave:
// 123 VGPRs, so two work-groups fill a CU with 16 waves to hide the tile
// copies; two query tiles per wave needed 202 VGPRs and ran 10% slower), keys
// in tiles of 64,
// S^T = K Q^T so that P^T feeds O^T = V^T P^T from the accumulator registers,
// fp16 operands with fp32 accumulation. The keys arrive rotated and the values
// transposed, both in fp16 (kv_prep.hip), so each tile is copied from global
// memory straight into LDS (global_load_lds, 16 bytes per lane) with no
// register staging: the LDS layout is set by which 16-byte piece each lane
// fetches. Key rows keep 16-byte chunk c at position c ^ swz_key(row), and
// each 64-byte value row (32 tokens of one dimension in vt_pos order, four
// 16-byte pieces, one per MFMA lane group) keeps piece g at g ^ swz_val(dim);
// both spread the operand reads of a wave over the LDS banks. Work-groups run
// in an XCD-aware order so that the ~10 query tiles sharing a key tile meet in
// one L2. The next tile is copied while the current one
// is multiplied (two named LDS buffers, so the compiler can tell the copies
// from the reads), and the online softmax keeps a lazily updated maximum.
// Queries are rotated in registers with the same absolute-position table.
#include "fsl_internal.h"

namespace fsl {

namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

union P8 {
    uint4 u;
    uint2 d[2];
    _Float16 f[8];
    halfx8 v;
};

}  // namespace

template <int D>
__global__ __launch_bounds__(512, 4) void window_bf16_kernel(const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ kt,
                                                             const uint16_t *__restrict__ vt,
                                                             const float2 *__restrict__ rope,
                                                             const int32_t *__restrict__ sel,
                                                             const uint16_t *__restrict__ part,
                                                             const float *__restrict__ plse,
                                                             void *__restrict__ out, float *__restrict__ o_win_out,
                                                             float *__restrict__ o_long_out, KParams p,
                                                             int tile0, int ntile) {
    constexpr int HALF = D / 2;
    constexpr int QS = D / 32;                  // MFMA k-steps over d
    constexpr int CPR = D / 8;                  // 16-byte chunks per key row
    constexpr int TILE = kKTile * D;            // fp16 elements of a key tile (and of a value tile)
    constexpr int UNITS = TILE * 2 / 1024;      // 1 KB copy units per tile
    constexpr int NW = 8;                       // waves
    constexpr int QT = 1;                       // 16-query MFMA tiles per wave
    constexpr int UPW = UNITS / NW;             // key (and value) units per wave
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];

    // query tiles tile0 .. tile0 + ntile - 1 of every head
    const int logical = xcd_remap((int)blockIdx.x, ntile * p.H);
    const int h = logical / ntile;
    const int64_t q0 = (int64_t)(tile0 + logical % ntile) * kQTile;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int64_t qw = q0 + 16 * QT * wave;
    const float sl2 = p.scale * 1.4426950408889634f;

    // key tiles that intersect [max(0, q0-w+1), min(N, q0+128) - 1]
    const int64_t kmin = max((int64_t)0, q0 - p.w + 1);
    const int64_t kmax = min(p.N, q0 + kQTile) - 1;
    const int t_first = (int)(kmin / kKTile);
    const int t_last = (int)(kmax / kKTile);

    // ---- this lane's copy offsets (elements within a tile), for units wave + 8 i
    int koff[UPW], voff[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int s = 64 * (wave + NW * i) + lane;  // 16-byte slot within the tile
        const int row = s / CPR, pc = s % CPR;
        koff[i] = row * D + 8 * (pc ^ swz_key(row, D));
        const int r = s >> 2, pg = s & 3;       // r = group * D + dim
        voff[i] = r * 32 + 8 * (pg ^ swz_val(r % D));
    }
    const uint16_t *kth = kt + h * kt_head_elems(p);
    const uint16_t *vth = vt + h * vt_head_elems(p);
    auto issue = [&](int t, uint16_t *kbuf, uint16_t *vbuf) __attribute__((always_inline)) {
        const uint16_t *kb = kth + (int64_t)t * TILE;  // tiles are contiguous in both arrays
        const uint16_t *vb = vth + (int64_t)t * TILE;
#pragma unroll
        for (int i = 0; i < UPW; ++i) lds_dma16(kb + koff[i], kbuf + 512 * (wave + NW * i));
#pragma unroll
        for (int i = 0; i < UPW; ++i) lds_dma16(vb + voff[i], vbuf + 512 * (wave + NW * i));
    };

    // ---- rotated queries as fp16 MFMA B operands (column = query, k-slots = dims 32ks + 8g + r)
    halfx8 qreg[QT][QS];
    {
        const int nhi = rope_abs_rows_hi(p);
#pragma unroll
        for (int qg = 0; qg < QT; ++qg) {
            const int64_t i = qw + 16 * qg + col;
            const bool ok = i < p.N;
            const int64_t ic = ok ? i : p.N - 1;
            const uint16_t *qi = q + ((int64_t)h * p.N + ic) * D;
            const float2 *th = rope + (ic / kRopeSpan) * HALF;
            const float2 *tl = rope + (int64_t)(nhi + (int)(ic % kRopeSpan)) * HALF;
            float x[QS][8];
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(qi + 32 * ks + 8 * g);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    x[ks][2 * t] = ok ? __uint_as_float(w4[t] << 16) : 0.0f;
                    x[ks][2 * t + 1] = ok ? __uint_as_float(w4[t] & 0xFFFF0000u) : 0.0f;
                }
            }
#pragma unroll
            for (int ks = 0; ks < QS / 2; ++ks)
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int m = 32 * ks + 8 * g + r;
                    const float2 a2 = th[m], b2 = tl[m];
                    const float c = a2.x * b2.x - a2.y * b2.y;
                    const float sn = a2.y * b2.x + a2.x * b2.y;
                    const float a = x[ks][r], b = x[ks + QS / 2][r];
                    x[ks][r] = a * c - b * sn;
                    x[ks + QS / 2][r] = b * c + a * sn;
                }
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) {
                P8 pk;
#pragma unroll
                for (int r = 0; r < 8; ++r) pk.f[r] = (_Float16)x[ks][r];
                qreg[qg][ks] = pk.v;
            }
        }
    }

    float m_run[QT];
    float l_part[QT];
    floatx4 oacc[QT][D / 16];
#pragma unroll
    for (int qg = 0; qg < QT; ++qg) {
        m_run[qg] = -INFINITY;
        l_part[qg] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) oacc[qg][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    auto compute = [&](int t, const uint16_t *kbuf, const uint16_t *vbuf) __attribute__((always_inline)) {
        const int64_t ks0 = (int64_t)t * kKTile;
        const bool active = qw < p.N && ks0 <= qw + 16 * QT - 1 && ks0 + kKTile - 1 >= qw - p.w + 1;
        if (!active) return;
        // The MFMA blocks run at raised wave priority, so that a wave which reaches its
        // products issues them ahead of the other waves' softmax work and the matrix
        // pipe idles less (measured: 1.23 -> 1.19 ms for the window with its merge).
        __builtin_amdgcn_s_setprio(1);
        floatx4 sacc[4][QT];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
#pragma unroll
            for (int qg = 0; qg < QT; ++qg) sacc[kg][qg] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int row = 16 * kg + col;
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) {
                P8 ka;
                ka.u = *reinterpret_cast<const uint4 *>(&kbuf[row * D + 8 * ((4 * ks + g) ^ swz_key(row, D))]);
#pragma unroll
                for (int qg = 0; qg < QT; ++qg)
                    sacc[kg][qg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka.v, qreg[qg][ks], sacc[kg][qg], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // positions fit in int32 (N < 2^31)
        const int j0 = (int)ks0 + 4 * g;
        const bool edge = !(ks0 + kKTile - 1 <= qw && ks0 > qw + 16 * QT - 1 - p.w);
        P8 pb[2][QT];
#pragma unroll
        for (int qg = 0; qg < QT; ++qg) {
            const int i = (int)qw + 16 * qg + col;
            float mx = -INFINITY;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float val = sacc[kg][qg][r];
                    if (edge) {
                        const int j = j0 + 16 * kg + r;
                        val = (j <= i && j > i - p.w) ? val : -INFINITY;
                    }
                    sacc[kg][qg][r] = val;
                    mx = fmaxf(mx, val);
                }
            mx = colmax4(mx) * sl2;
            const float mr = m_run[qg];
            const bool grow = mx > mr + kStaleLog2;
            const bool resc = grow && mr != -INFINITY;
            if (__ballot(resc)) {  // rare: a score jumped past the lazily kept maximum
                const float alpha = resc ? exp2_hw(mr - mx) : 1.0f;
                l_part[qg] *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) oacc[qg][dt] *= alpha;
            }
            const float mn = grow ? mx : mr;
            m_run[qg] = mn;
            const float msub = mn == -INFINITY ? 0.0f : mn;
            float lsum = 0.0f;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                float e[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = exp2_hw(fmaf(sacc[kg][qg][r], sl2, -msub));
                const uint32_t w01 = pk_f16_rne_acc(e[0], e[1], lsum);
                const uint32_t w23 = pk_f16_rne_acc(e[2], e[3], lsum);
                pb[kg >> 1][qg].d[kg & 1] = make_uint2(w01, w23);
            }
            l_part[qg] += lsum;
        }
        __builtin_amdgcn_s_setprio(1);
        // value operand: dimension 16 dt + col, piece g of 32-token group kk
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const int dim = 16 * dt + col;
                P8 va;
                va.u = *reinterpret_cast<const uint4 *>(&vbuf[((kk * D + dim) * 4 + (g ^ swz_val(dim))) * 8]);
#pragma unroll
                for (int qg = 0; qg < QT; ++qg)
                    oacc[qg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.v, pb[kk][qg].v, oacc[qg][dt], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    issue(t_first, k_lds0, v_lds0);
    wait_vmem();
    __syncthreads();
    for (int t = t_first; t <= t_last; t += 2) {
        if (t + 1 <= t_last) issue(t + 1, k_lds1, v_lds1);
        compute(t, k_lds0, v_lds0);
        wait_vmem();
        __syncthreads();
        if (t + 1 > t_last) break;
        if (t + 2 <= t_last) issue(t + 2, k_lds0, v_lds0);
        compute(t + 1, k_lds1, v_lds1);
        wait_vmem();
        __syncthreads();
    }

    // ---- the long branch: merge the query's cells (readout_units.hip wrote, per
    // selected cell, its normalised output in fp16 and lambda = m + log2(l)) by
    // weights 2^(lambda - max lambda), which is the softmax over the union of the
    // cells' tokens; then RMSNorm over d and the mix with the per-head weight.
    // Lane (col, g) holds dimensions 16 dt + 4 g + r of its query in both branches.
#pragma unroll
    for (int qg = 0; qg < QT; ++qg) {
        const float l = colsum4(l_part[qg]);
        const int64_t i = qw + 16 * qg + col;
        const bool ok = i < p.N;
        const int64_t ic = ok ? i : p.N - 1;
        const int64_t row = (int64_t)h * p.N + ic;
        const float inv = 1.0f / l;
        floatx4 ow[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) ow[dt] = oacc[qg][dt] * inv;
        int sc[kMaxK];
        float lam[kMaxK];
        float lmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < kMaxK; ++r) {
            sc[r] = r < p.K ? sel[row * p.K + r] : -1;
            lam[r] = sc[r] >= 0 ? plse[row * p.K + r] : -INFINITY;
            lmax = fmaxf(lmax, lam[r]);
        }
        floatx4 ol[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) ol[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        float wsum = 0.0f;
#pragma unroll
        for (int r = 0; r < kMaxK; ++r) {
            if (sc[r] < 0) continue;
            const float wr = exp2_hw(lam[r] - lmax);
            wsum += wr;
            // element 32 (dt / 2) + 8 g + 4 (dt % 2) + x holds dimension 16 dt + 4 g + x
            const uint16_t *src = part + (row * p.K + r) * D + 8 * g;
#pragma unroll
            for (int dt = 0; dt < D / 16; dt += 2) {
                union {
                    u32x4 u;
                    _Float16 h[8];
                } c;
                c.u = *reinterpret_cast<const u32x4 *>(src + 16 * dt);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    ol[dt][x] = fmaf(wr, (float)c.h[x], ol[dt][x]);
                    ol[dt + 1][x] = fmaf(wr, (float)c.h[4 + x], ol[dt + 1][x]);
                }
            }
        }
        const float winv = wsum > 0.0f ? 1.0f / wsum : 0.0f;  // no selected cell: o_long = 0
        float ss = 0.0f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            ol[dt] *= winv;
#pragma unroll
            for (int x = 0; x < 4; ++x) ss += ol[dt][x] * ol[dt][x];
        }
        ss = colsum4(ss);
        const float rs = 1.0f / sqrtf(ss / (float)D + p.rms_eps);
        if (!ok) continue;
        const float gam = p.gamma[h];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const int c0 = 16 * dt + 4 * g;
            float val[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) val[x] = ow[dt][x] + gam * (ol[dt][x] * rs);
            if (p.out_dtype == FSL_BF16) {
                const uint32_t w0 = (uint32_t)f32_to_bf16(val[0]) | ((uint32_t)f32_to_bf16(val[1]) << 16);
                const uint32_t w1 = (uint32_t)f32_to_bf16(val[2]) | ((uint32_t)f32_to_bf16(val[3]) << 16);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + row * D + c0) = make_uint2(w0, w1);
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + row * D + c0) =
                    make_float4(val[0], val[1], val[2], val[3]);
            }
            if (o_win_out)
                *reinterpret_cast<float4 *>(o_win_out + row * D + c0) =
                    make_float4(ow[dt][0], ow[dt][1], ow[dt][2], ow[dt][3]);
            if (o_long_out)
                *reinterpret_cast<float4 *>(o_long_out + row * D + c0) =
                    make_float4(ol[dt][0], ol[dt][1], ol[dt][2], ol[dt][3]);
        }
    }
}

hipError_t launch_window_bf16(const void *q, const uint16_t *kt, const uint16_t *vt, const float2 *rope_abs,
                              const int32_t *sel, const uint16_t *part, const float *plse, void *out,
                              float *o_win_out, float *o_long_out, const KParams &p, int64_t qa, int64_t qb,
                              hipStream_t st) {
    const int tile0 = (int)(qa / kQTile);
    const int ntile = (int)((qb + kQTile - 1) / kQTile) - tile0;
    if (ntile <= 0) return hipSuccess;
    dim3 grid((unsigned)(ntile * p.H));
    if (p.d == 64)
        hipLaunchKernelGGL((window_bf16_kernel<64>), grid, dim3(512), 0, st, (const uint16_t *)q, kt, vt, rope_abs,
                           sel, part, plse, out, o_win_out, o_long_out, p, tile0, ntile);
    else
        hipLaunchKernelGGL((window_bf16_kernel<128>), grid, dim3(512), 0, st, (const uint16_t *)q, kt, vt, rope_abs,
                           sel, part, plse, out, o_win_out, o_long_out, p, tile0, ntile);
    return hipGetLastError();
}

}  // namespace fsl

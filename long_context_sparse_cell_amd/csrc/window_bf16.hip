// Local branch for bf16 inputs: RoPE attention over the window [i-w+1, i]
// (FreeSolo digest, core method and step 2; prerequisites: RoPE rotates q_i
// and k_j so that their product depends only on the offset j - i).
//
// Same tiling and operand layout as the generic window kernel (window.hip):
// 128 queries per workgroup, 4 waves x 32 queries, keys through LDS in tiles
// of 64, S^T = K Q^T so that P^T feeds O^T = V^T P^T from the accumulator
// registers, RoPE from a relative-offset table, fp16 operands with fp32
// accumulation. What this version adds for throughput:
//  - LDS is double-buffered, and the next tile's global loads (keys, values,
//    cos/sin rows) are issued into registers before the current tile's MFMAs,
//    so their latency overlaps the math; one barrier per tile.
//  - the register budget targets two waves per SIMD.
//  - only the key tiles that intersect the workgroup's window range are visited.
#include <cmath>

#include "fsl_internal.h"

namespace fsl {

namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

union P8 {
    uint4 u;
    uint16_t h[8];
    _Float16 f[8];
    halfx8 v;
};

__device__ __forceinline__ void unpack_bf16x8(const uint4 raw, float (&o)[8]) {
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        o[2 * t] = __uint_as_float(w4[t] << 16);
        o[2 * t + 1] = __uint_as_float(w4[t] & 0xFFFF0000u);
    }
}

// two floats to a packed fp16 pair (one v_cvt_pkrtz_f16_f32)
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
    union { decltype(__builtin_amdgcn_cvt_pkrtz(0.0f, 0.0f)) h; uint32_t u; } c;
    c.h = __builtin_amdgcn_cvt_pkrtz(a, b);
    return c.u;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void window_bf16_kernel(const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ k,
                                                             const uint16_t *__restrict__ v,
                                                             const float2 *__restrict__ rope,
                                                             float *__restrict__ o_win, KParams p) {
    constexpr int HALF = D / 2;
    constexpr int KLD = D + 8;         // K tile row stride (fp16 elements)
    constexpr int VLD = kKTile + 8;    // V^T tile row stride
    constexpr int KIT = D / 64;        // K staging items per thread (64 keys x D/16 chunk pairs)
    constexpr int VITEMS = 2 * D;      // V staging items (16 key quads x D/8 chunks)
    constexpr int QS = D / 32;         // MFMA k-steps over d
    __shared__ uint16_t ks_lds[2][kKTile * KLD];
    __shared__ uint16_t vt_lds[2][D * VLD];

    const int h = blockIdx.y;
    const int64_t q0 = (int64_t)blockIdx.x * kQTile;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g = lane >> 4;
    const int64_t qw = q0 + 32 * wave;
    const uint16_t *kh = k + (int64_t)h * p.N * D;
    const uint16_t *vh = v + (int64_t)h * p.N * D;
    const float sl2 = p.scale * 1.4426950408889634f;

    // key tiles that intersect [max(0, q0-w+1), min(N, q0+128) - 1]
    const int64_t base = q0 + p.rope_lo;
    const int64_t kmin = max((int64_t)0, q0 - p.w + 1);
    const int64_t kmax = min(p.N, q0 + kQTile) - 1;
    const int t_first = (int)((kmin - base) / kKTile);
    const int t_last = (int)((kmax - base) / kKTile);

    // ---- staging registers
    constexpr bool PRE_CS = D <= 64;   // prefetch cos/sin rows too when registers allow
    uint4 pk_a[KIT], pk_b[KIT];
    float4 pcs[PRE_CS ? KIT : 1][4];
    uint4 pv[4];
    auto fetch = [&](int t) {
        const int64_t ks0 = base + (int64_t)t * kKTile;
#pragma unroll
        for (int u = 0; u < KIT; ++u) {
            const int it = tid + 256 * u;
            const int jl = it / (D / 16), c = it % (D / 16);
            const int64_t j = ks0 + jl;
            const int64_t jc = (j >= 0 && j < p.N) ? j : 0;
            pk_a[u] = *reinterpret_cast<const uint4 *>(kh + jc * D + 8 * c);
            pk_b[u] = *reinterpret_cast<const uint4 *>(kh + jc * D + HALF + 8 * c);
            if constexpr (PRE_CS) {
                const float4 *tr = reinterpret_cast<const float4 *>(rope + (j - q0 - p.rope_lo) * HALF + 8 * c);
#pragma unroll
                for (int r = 0; r < 4; ++r) pcs[u][r] = tr[r];
            }
        }
        if (tid < VITEMS) {
            const int jq = tid & 15, c = tid >> 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t j = ks0 + 4 * jq + e;
                const int64_t jc = (j >= 0 && j < p.N) ? j : 0;
                pv[e] = *reinterpret_cast<const uint4 *>(vh + jc * D + 8 * c);
            }
        }
    };
    auto store = [&](int t, int buf) {
        const int64_t ks0 = base + (int64_t)t * kKTile;
#pragma unroll
        for (int u = 0; u < KIT; ++u) {
            const int it = tid + 256 * u;
            const int jl = it / (D / 16), c = it % (D / 16);
            const int64_t j = ks0 + jl;
            const bool ok = j >= 0 && j < p.N;
            float a[8], b[8];
            unpack_bf16x8(pk_a[u], a);
            unpack_bf16x8(pk_b[u], b);
            float4 c4[4];
            if constexpr (PRE_CS) {
#pragma unroll
                for (int r = 0; r < 4; ++r) c4[r] = pcs[u][r];
            } else {
                const float4 *tr = reinterpret_cast<const float4 *>(rope + (j - q0 - p.rope_lo) * HALF + 8 * c);
#pragma unroll
                for (int r = 0; r < 4; ++r) c4[r] = tr[r];
            }
            const float cs[16] = {c4[0].x, c4[0].y, c4[0].z, c4[0].w, c4[1].x, c4[1].y, c4[1].z, c4[1].w,
                                  c4[2].x, c4[2].y, c4[2].z, c4[2].w, c4[3].x, c4[3].y, c4[3].z, c4[3].w};
            P8 ra, rb;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float x0 = ok ? a[r] : 0.0f, y0 = ok ? b[r] : 0.0f;
                const float co = cs[2 * r], si = cs[2 * r + 1];
                ra.f[r] = (_Float16)(x0 * co - y0 * si);
                rb.f[r] = (_Float16)(y0 * co + x0 * si);
            }
            *reinterpret_cast<uint4 *>(&ks_lds[buf][jl * KLD + 8 * c]) = ra.u;
            *reinterpret_cast<uint4 *>(&ks_lds[buf][jl * KLD + HALF + 8 * c]) = rb.u;
        }
        if (tid < VITEMS) {
            const int jq = tid & 15, c = tid >> 4;  // 16 lanes fill one V^T row segment: no bank conflicts
            float e4[4][8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t j = ks0 + 4 * jq + e;
                const bool ok = j >= 0 && j < p.N;
                unpack_bf16x8(pv[e], e4[e]);
#pragma unroll
                for (int r = 0; r < 8; ++r) e4[e][r] = ok ? e4[e][r] : 0.0f;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                // bf16 -> fp16 is exact in fp16's normal range: the packed convert's rounding mode is moot
                const uint32_t lo = pk_f16(e4[0][r], e4[1][r]);
                const uint32_t hi = pk_f16(e4[2][r], e4[3][r]);
                *reinterpret_cast<uint2 *>(&vt_lds[buf][(8 * c + r) * VLD + 4 * jq]) = make_uint2(lo, hi);
            }
        }
    };

    // ---- rotated queries as fp16 MFMA B operands (column = query, k-slots = dims 32ks + 8g + r)
    halfx8 qreg[2][QS];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int64_t i = qw + 16 * qg + col;
        const bool ok = i < p.N;
        const uint16_t *qi = q + ((int64_t)h * p.N + (ok ? i : 0)) * D;
        const float2 *tr = rope + (int64_t)(i - q0 - p.rope_lo) * HALF;
        float x[QS][8];
#pragma unroll
        for (int ks = 0; ks < QS; ++ks) {
            unpack_bf16x8(*reinterpret_cast<const uint4 *>(qi + 32 * ks + 8 * g), x[ks]);
#pragma unroll
            for (int r = 0; r < 8; ++r) x[ks][r] = ok ? x[ks][r] : 0.0f;
        }
#pragma unroll
        for (int ks = 0; ks < QS / 2; ++ks)
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float2 cs = tr[32 * ks + 8 * g + r];
                const float a = x[ks][r], b = x[ks + QS / 2][r];
                x[ks][r] = a * cs.x - b * cs.y;
                x[ks + QS / 2][r] = b * cs.x + a * cs.y;
            }
#pragma unroll
        for (int ks = 0; ks < QS; ++ks) {
            P8 pk;
#pragma unroll
            for (int r = 0; r < 8; ++r) pk.f[r] = (_Float16)x[ks][r];
            qreg[qg][ks] = pk.v;
        }
    }

    float m_run[2] = {-INFINITY, -INFINITY};
    float l_part[2] = {0.0f, 0.0f};
    floatx4 oacc[2][D / 16];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) oacc[qg][dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    fetch(t_first);
    store(t_first, 0);
    __syncthreads();
    for (int t = t_first; t <= t_last; ++t) {
        const int buf = (t - t_first) & 1;
        const bool more = t < t_last;
        if (more) fetch(t + 1);
        const int64_t ks0 = base + (int64_t)t * kKTile;
        const bool active = qw < p.N && ks0 <= qw + 31 && ks0 + kKTile - 1 >= qw - p.w + 1;
        if (active) {
            const uint16_t *kt = ks_lds[buf];
            const uint16_t *vt = vt_lds[buf];
            floatx4 sacc[4][2];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                sacc[kg][0] = floatx4{0.f, 0.f, 0.f, 0.f};
                sacc[kg][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < QS; ++ks) {
                    P8 ka;
                    ka.u = *reinterpret_cast<const uint4 *>(&kt[(16 * kg + col) * KLD + 32 * ks + 8 * g]);
                    sacc[kg][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka.v, qreg[0][ks], sacc[kg][0], 0, 0, 0);
                    sacc[kg][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka.v, qreg[1][ks], sacc[kg][1], 0, 0, 0);
                }
            }
            // positions fit in int32 (N < 2^31, the window offset is bounded by w)
            const int j0 = (int)ks0 + 4 * g;
            const bool edge = !(ks0 + kKTile - 1 <= qw && ks0 > qw + 31 - p.w && ks0 >= 0);
            P8 pb[2][2];
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
                const int i = (int)qw + 16 * qg + col;
                float mx = -INFINITY;
#pragma unroll
                for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float val = sacc[kg][qg][r];
                        if (edge) {
                            const int j = j0 + 16 * kg + r;
                            val = (j <= i && j > i - p.w && j >= 0) ? val : -INFINITY;
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
                    for (int r = 0; r < 4; ++r) {
                        e[r] = exp2_hw(fmaf(sacc[kg][qg][r], sl2, -msub));
                        lsum += e[r];
                    }
                    const uint32_t lo = pk_f16(e[0], e[1]), hi = pk_f16(e[2], e[3]);
                    if (kg & 1) {
                        pb[kg >> 1][qg].u.z = lo;
                        pb[kg >> 1][qg].u.w = hi;
                    } else {
                        pb[kg >> 1][qg].u.x = lo;
                        pb[kg >> 1][qg].u.y = hi;
                    }
                }
                l_part[qg] += lsum;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) {
                    const uint16_t *vr = &vt[(16 * dt + col) * VLD + 32 * kk + 4 * g];
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
                    P8 va;
                    va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    oacc[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.v, pb[kk][0].v, oacc[0][dt], 0, 0, 0);
                    oacc[1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.v, pb[kk][1].v, oacc[1][dt], 0, 0, 0);
                }
            }
        }
        if (more) store(t + 1, buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const float l = colsum4(l_part[qg]);
        const int64_t i = qw + 16 * qg + col;
        if (i >= p.N) continue;
        const float inv = 1.0f / l;
        float *orow = o_win + ((int64_t)h * p.N + i) * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const floatx4 o = oacc[qg][dt] * inv;
            *reinterpret_cast<float4 *>(orow + 16 * dt + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
        }
    }
}

hipError_t launch_window_bf16(const void *q, const void *k, const void *v, const float2 *rope, float *o_win,
                              const KParams &p, hipStream_t st) {
    dim3 grid((unsigned)((p.N + kQTile - 1) / kQTile), (unsigned)p.H);
    if (p.d == 64)
        hipLaunchKernelGGL((window_bf16_kernel<64>), grid, dim3(256), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                           (const uint16_t *)v, rope, o_win, p);
    else
        hipLaunchKernelGGL((window_bf16_kernel<128>), grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, rope, o_win, p);
    return hipGetLastError();
}

}  // namespace fsl

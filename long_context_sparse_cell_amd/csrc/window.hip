// Local branch: RoPE attention over the window [i-w+1, i] (FreeSolo digest,
// core method and step 2; prerequisites: RoPE rotates q_i and k_j so that
// their product depends only on the offset).
//
// Design (gfx950):
//  - One workgroup = 128 consecutive queries of one head, 4 waves x 32
//    queries (two 16-query MFMA column groups per wave, so each K/V operand
//    read from LDS feeds two MFMAs).
//  - Keys stream through LDS in tiles of 64: K rotated and row-major, V
//    transposed, so both MFMA operands are contiguous LDS reads.
//  - Scores are formed transposed, S^T = K Q^T, so a lane owns one query
//    column: the online-softmax row statistics and the O^T = V^T P^T
//    accumulator of that query sit in the same lane and P^T feeds the second
//    MFMA straight from the first MFMA's accumulator registers (the k-slot
//    order of the second product is chosen to match).
//  - RoPE uses positions relative to the workgroup's first query q0: the
//    score depends only on j - i, and |j - q0| < w + 128 keeps the fp64-built
//    cos/sin table small and exact to fp32 rounding at any absolute position.
//  - bf16 inputs: the rotated q, k, the probabilities P and v enter
//    v_mfma_f32_16x16x32_f16 as fp16 (fp32 accumulation). bf16 -> fp16 is
//    exact in fp16's normal range, and fp16's 11-bit significand keeps the
//    rounding of rotated q/k and of P about 8x below bf16's, which leaves
//    room for the bf16 rounding of the output itself. Inputs are assumed to
//    stay within fp16 range (|x| < 65504). The softmax denominator sums the
//    rounded P. fp32 inputs: v_mfma_f32_16x16x4_f32 throughout.
#include <cmath>
#include <type_traits>

#include "fsl_internal.h"

namespace fsl {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ void rope_table_kernel(float2 *__restrict__ tab, uint32_t *__restrict__ status, KParams p) {
    const int half = p.d / 2;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e == 0) *status = 0u;  // fp32 inputs take no fp16 conversion: nothing to flag
    if (e >= (int64_t)p.rope_n * half) return;
    const int row = (int)(e / half), m = (int)(e % half);
    const double theta = pow((double)p.rope_base, -2.0 * (double)m / (double)p.d);
    const double ang = (double)(p.rope_lo + row) * theta;
    tab[e] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_table(float2 *tab, uint32_t *status, const KParams &p, hipStream_t st) {
    const int64_t n = (int64_t)p.rope_n * (p.d / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tab, status, p);
    return hipGetLastError();
}

union Pack8 {
    uint4 u;
    uint16_t h[8];
    _Float16 f[8];
    halfx8 v;
};

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    union { _Float16 f; uint16_t u; } c;
    c.f = (_Float16)x;
    return c.u;
}

__device__ __forceinline__ float round_f16(float x) { return (float)(_Float16)x; }

// eight consecutive elements as float (one 16-byte load for bf16, two for fp32)
__device__ __forceinline__ void load8(const uint16_t *ptr, float (&o)[8]) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(ptr);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        o[2 * t] = __uint_as_float(w4[t] << 16);
        o[2 * t + 1] = __uint_as_float(w4[t] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8(const float *ptr, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(ptr);
    const float4 b = *reinterpret_cast<const float4 *>(ptr + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

template <typename T, int D>
struct WinLds;

template <int D>
struct WinLds<uint16_t, D> {
    static constexpr int KLD = D + 8;          // row stride of K tile (elements)
    static constexpr int VLD = kKTile + 8;     // row stride of V^T tile
    uint16_t k[kKTile * KLD];
    uint16_t vt[D * VLD];
};

template <int D>
struct WinLds<float, D> {
    static constexpr int KLD = D + 4;
    static constexpr int VLD = kKTile + 4;
    float k[kKTile * KLD];
    float vt[D * VLD];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void window_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                     const T *__restrict__ v, const float2 *__restrict__ rope,
                                                     float *__restrict__ o_win, KParams p) {
    constexpr bool BF = sizeof(T) == 2;
    constexpr int HALF = D / 2;
    using L = WinLds<T, D>;
    __shared__ L lds;

    const int h = blockIdx.y;
    const int64_t q0 = (int64_t)blockIdx.x * kQTile;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g = lane >> 4;
    const int64_t qw = q0 + 32 * wave;  // first query of this wave
    const T *kh = k + (int64_t)h * p.N * D;
    const T *vh = v + (int64_t)h * p.N * D;
    const float log2e = 1.4426950408889634f;
    const float sl2 = p.scale * log2e;

    // ---- rotated queries as MFMA B operands (column = query, k-slot = dim)
    constexpr int QS = BF ? D / 32 : D / 4;  // k-steps over d
    using QReg = typename std::conditional<BF, halfx8, float>::type;
    QReg qreg[2][QS];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int64_t i = qw + 16 * qg + col;
        const bool ok = i < p.N;
        const T *qi = q + ((int64_t)h * p.N + (ok ? i : 0)) * D;
        const float2 *tr = rope + (int64_t)(i - q0 - p.rope_lo) * HALF;
        if constexpr (BF) {
            // lane holds dims 32*ks + 8*g + r; dim m pairs with m + D/2 (k-step ks + D/64)
            float x[QS][8];
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) {
                Pack8 pk;
                pk.u = ok ? *reinterpret_cast<const uint4 *>(qi + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 8; ++r) x[ks][r] = bf16_to_f32(pk.h[r]);
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
                Pack8 pk;
#pragma unroll
                for (int r = 0; r < 8; ++r) pk.f[r] = (_Float16)x[ks][r];
                qreg[qg][ks] = pk.v;
            }
        } else {
            // lane holds dims 4*ks + g; dim m pairs with m + D/2 (k-step ks + D/8)
            float x[QS];
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) x[ks] = ok ? to_f32<T>(qi[4 * ks + g]) : 0.0f;
#pragma unroll
            for (int ks = 0; ks < QS / 2; ++ks) {
                const float2 cs = tr[4 * ks + g];
                const float a = x[ks], b = x[ks + QS / 2];
                x[ks] = a * cs.x - b * cs.y;
                x[ks + QS / 2] = b * cs.x + a * cs.y;
            }
#pragma unroll
            for (int ks = 0; ks < QS; ++ks) qreg[qg][ks] = x[ks];
        }
    }

    // ---- running softmax state and O^T accumulators (lane: query col, dims 16*dt + 4*g + r)
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_part[2] = {0.0f, 0.0f};
    floatx4 oacc[2][D / 16];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) oacc[qg][dt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    const int ntiles = (kQTile - p.rope_lo) / kKTile;
    for (int t = 0; t < ntiles; ++t) {
        const int64_t ks0 = q0 + p.rope_lo + (int64_t)t * kKTile;  // first key of the tile
        if (ks0 + kKTile <= 0) continue;                             // uniform: tile wholly before token 0
        if (ks0 >= p.N) break;

        // ---- stage K (rotated) and V^T
        __syncthreads();
        for (int it = tid; it < kKTile * (D / 16); it += 256) {
            const int jl = it / (D / 16), c = it % (D / 16);
            const int64_t j = ks0 + jl;
            // out-of-range keys read a clamped valid row and are zeroed (their scores are masked)
            const bool ok = j >= 0 && j < p.N;
            const int64_t jc = ok ? j : 0;
            const T *kr = kh + jc * D;
            float a[8], b[8];
            load8(kr + 8 * c, a);
            load8(kr + HALF + 8 * c, b);
            const float2 *tr = rope + (int64_t)(j - q0 - p.rope_lo) * HALF + 8 * c;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float2 cs = tr[r];
                const float x0 = ok ? a[r] : 0.0f, y0 = ok ? b[r] : 0.0f;
                a[r] = x0 * cs.x - y0 * cs.y;
                b[r] = y0 * cs.x + x0 * cs.y;
            }
            if constexpr (BF) {
                Pack8 pa, pb;
#pragma unroll
                for (int r = 0; r < 8; ++r) { pa.f[r] = (_Float16)a[r]; pb.f[r] = (_Float16)b[r]; }
                *reinterpret_cast<uint4 *>(&lds.k[jl * L::KLD + 8 * c]) = pa.u;
                *reinterpret_cast<uint4 *>(&lds.k[jl * L::KLD + HALF + 8 * c]) = pb.u;
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    lds.k[jl * L::KLD + 8 * c + r] = a[r];
                    lds.k[jl * L::KLD + HALF + 8 * c + r] = b[r];
                }
            }
        }
        for (int it = tid; it < (kKTile / 4) * (D / 8); it += 256) {
            const int jq = it / (D / 8), c = it % (D / 8);
            float e[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t j = ks0 + 4 * jq + u;
                const bool ok = j >= 0 && j < p.N;
                load8(vh + (ok ? j : 0) * D + 8 * c, e[u]);
#pragma unroll
                for (int r = 0; r < 8; ++r) e[u][r] = ok ? e[u][r] : 0.0f;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (BF) lds.vt[(8 * c + r) * L::VLD + 4 * jq + u] = f32_to_f16_bits(e[u][r]);
                    else lds.vt[(8 * c + r) * L::VLD + 4 * jq + u] = e[u][r];
                }
        }
        __syncthreads();

        // ---- this wave's queries [qw, qw+32) see keys [qw-w+1, qw+31]
        if (qw >= p.N || ks0 > qw + 31 || ks0 + kKTile - 1 < qw - p.w + 1) continue;

        floatx4 sacc[4][2];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
                floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (BF) {
#pragma unroll
                    for (int ks = 0; ks < QS; ++ks) {
                        Pack8 ka;
                        ka.u = *reinterpret_cast<const uint4 *>(&lds.k[(16 * kg + col) * L::KLD + 32 * ks + 8 * g]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka.v, qreg[qg][ks], acc, 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int ks = 0; ks < QS; ++ks) {
                        const float ka = lds.k[(16 * kg + col) * L::KLD + 4 * ks + g];
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, qreg[qg][ks], acc, 0, 0, 0);
                    }
                }
                sacc[kg][qg] = acc;
            }

        // ---- mask, online softmax (lane: query col of group qg; keys 16*kg + 4*g + r)
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            const int64_t i = qw + 16 * qg + col;
            float mx = -INFINITY;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t j = ks0 + 16 * kg + 4 * g + r;
                    const bool ok = j <= i && j > i - p.w && j >= 0;
                    const float val = ok ? sacc[kg][qg][r] * sl2 : -INFINITY;
                    sacc[kg][qg][r] = val;
                    mx = fmaxf(mx, val);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[qg], mx);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = exp2f(m_run[qg] - m_use);
            m_run[qg] = m_new;
            float lsum = 0.0f;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float pv = exp2f(sacc[kg][qg][r] - m_use);
                    if constexpr (BF) pv = round_f16(pv);
                    sacc[kg][qg][r] = pv;
                    lsum += pv;
                }
            l_part[qg] = l_part[qg] * alpha + lsum;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) oacc[qg][dt] *= alpha;
        }

        // ---- O^T += V^T P^T
        if constexpr (BF) {
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    Pack8 pb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pb.f[r] = (_Float16)sacc[2 * kk][qg][r];
                        pb.f[4 + r] = (_Float16)sacc[2 * kk + 1][qg][r];
                    }
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt) {
                        const uint16_t *vr = &lds.vt[(16 * dt + col) * L::VLD + 32 * kk + 4 * g];
                        Pack8 va;
                        const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
                        const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
                        va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
                        oacc[qg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.v, pb.v, oacc[qg][dt], 0, 0, 0);
                    }
                }
            }
        } else {
#pragma unroll
            for (int qg = 0; qg < 2; ++qg)
#pragma unroll
                for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int dt = 0; dt < D / 16; ++dt) {
                            const float va = lds.vt[(16 * dt + col) * L::VLD + 16 * kg + 4 * g + r];
                            oacc[qg][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, sacc[kg][qg][r], oacc[qg][dt], 0, 0, 0);
                        }
        }
    }

    // ---- normalise and write (lane: query col, dims 16*dt + 4*g + r)
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        float l = l_part[qg];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
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

template <typename T, int D>
static hipError_t launch_window_t(const void *q, const void *k, const void *v, const float2 *rope, float *o_win,
                                  const KParams &p, hipStream_t st) {
    dim3 grid((unsigned)((p.N + kQTile - 1) / kQTile), (unsigned)p.H);
    hipLaunchKernelGGL((window_kernel<T, D>), grid, dim3(256), 0, st, (const T *)q, (const T *)k, (const T *)v, rope,
                       o_win, p);
    return hipGetLastError();
}

hipError_t launch_window(const void *q, const void *k, const void *v, const float2 *rope, float *o_win,
                         const KParams &p, hipStream_t st) {
    if (p.dtype == FSL_BF16)
        return p.d == 64 ? launch_window_t<uint16_t, 64>(q, k, v, rope, o_win, p, st)
                         : launch_window_t<uint16_t, 128>(q, k, v, rope, o_win, p, st);
    return p.d == 64 ? launch_window_t<float, 64>(q, k, v, rope, o_win, p, st)
                     : launch_window_t<float, 128>(q, k, v, rope, o_win, p, st);
}

}  // namespace fsl

// Long branch readout and branch mix (FreeSolo digest, core method and step 6:
// NoPE softmax over the raw tokens of the selected cells, RMSNorm, then an add
// to the local branch with a per-head learned weight; prerequisites: the long
// branch uses unrotated q and k and no position term).
//
//   o_long[i] = softmax_j(scale q_i . k_j) v_j over the <= K*s tokens of sel[i]
//   out[i]    = o_win[i] + gamma_h * o_long[i] / sqrt(mean(o_long[i]^2) + eps)
//
// One wave per query: lanes own tokens for the scores and coordinates for the
// weighted sum; wave shuffles carry the max, the sum and the mean square.
// The selected tokens are gathered from memory each query touches once;
// queries of a block hit the same few pool cells, which stay cache-resident.
#include "fsl_internal.h"

namespace fsl {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void readout_mix_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                          const T *__restrict__ v, const int32_t *__restrict__ sel,
                                                          const float *__restrict__ o_win, void *__restrict__ out,
                                                          float *__restrict__ o_long_out, KParams p) {
    constexpr int XPL = D / 64;  // coordinates per lane
    __shared__ float pw[4][8 * 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + wave;
    const int h = blockIdx.y;
    if (i >= p.N) return;
    const int64_t row = (int64_t)h * p.N + i;
    const int32_t *si = sel + row * p.K;
    const T *qi = q + row * D;
    const float sl2 = p.scale * 1.4426950408889634f;

    int nsel = 0;
    for (int r = 0; r < p.K; ++r) nsel += si[r] >= 0 ? 1 : 0;
    const int ntok = nsel * p.s;

    float o[XPL];
#pragma unroll
    for (int x = 0; x < XPL; ++x) o[x] = 0.0f;
    if (ntok > 0) {
        // scores: lane owns tokens lane, lane+64, ...
        float mx = -INFINITY;
        for (int t0 = 0; t0 < ntok; t0 += 64) {
            const int t = t0 + lane;
            float val = -INFINITY;
            if (t < ntok) {
                const int64_t j = (int64_t)si[t / p.s] * p.s + (t % p.s);
                const T *kr = k + ((int64_t)h * p.N + j) * D;
                float dot = 0.0f;
#pragma unroll 16
                for (int x = 0; x < D; ++x) dot += to_f32<T>(qi[x]) * to_f32<T>(kr[x]);
                val = dot * sl2;
            }
            pw[wave][t0 + lane] = val;
            mx = fmaxf(mx, val);
        }
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int t0 = 0; t0 < ntok; t0 += 64) {
            const int t = t0 + lane;
            float e = 0.0f;
            if (t < ntok) { e = exp2f(pw[wave][t] - mx); pw[wave][t] = e; }
            sum += e;
        }
        sum = wave_sum(sum);
        __builtin_amdgcn_wave_barrier();
        // weighted sum of values: lane owns coordinates lane + 64*x
        for (int t = 0; t < ntok; ++t) {
            const int64_t j = (int64_t)si[t / p.s] * p.s + (t % p.s);
            const T *vr = v + ((int64_t)h * p.N + j) * D;
            const float wgt = pw[wave][t];
#pragma unroll
            for (int x = 0; x < XPL; ++x) o[x] += wgt * to_f32<T>(vr[lane + 64 * x]);
        }
        const float inv = 1.0f / sum;
#pragma unroll
        for (int x = 0; x < XPL; ++x) o[x] *= inv;
    }
    float ms = 0.0f;
#pragma unroll
    for (int x = 0; x < XPL; ++x) ms += o[x] * o[x];
    ms = wave_sum(ms) / (float)D;
    const float rs = 1.0f / sqrtf(ms + p.rms_eps);
    const float gam = p.gamma[h];
    const float *ow = o_win + row * D;
#pragma unroll
    for (int x = 0; x < XPL; ++x) {
        const int c = lane + 64 * x;
        const float val = ow[c] + gam * (o[x] * rs);
        if (p.out_dtype == FSL_BF16) reinterpret_cast<uint16_t *>(out)[row * D + c] = f32_to_bf16(val);
        else reinterpret_cast<float *>(out)[row * D + c] = val;
        if (o_long_out) o_long_out[row * D + c] = o[x];
    }
}

template <typename T, int D>
static hipError_t launch_readout_t(const void *q, const void *k, const void *v, const int32_t *sel, const float *o_win,
                                   void *out, float *o_long_out, const KParams &p, hipStream_t st) {
    dim3 grid((unsigned)((p.N + 3) / 4), (unsigned)p.H);
    hipLaunchKernelGGL((readout_mix_kernel<T, D>), grid, dim3(256), 0, st, (const T *)q, (const T *)k, (const T *)v,
                       sel, o_win, out, o_long_out, p);
    return hipGetLastError();
}

hipError_t launch_readout_mix(const void *q, const void *k, const void *v, const int32_t *sel, const float *o_win,
                              void *out, float *o_long_out, const KParams &p, hipStream_t st) {
    if (p.dtype == FSL_BF16)
        return p.d == 64 ? launch_readout_t<uint16_t, 64>(q, k, v, sel, o_win, out, o_long_out, p, st)
                         : launch_readout_t<uint16_t, 128>(q, k, v, sel, o_win, out, o_long_out, p, st);
    return p.d == 64 ? launch_readout_t<float, 64>(q, k, v, sel, o_win, out, o_long_out, p, st)
                     : launch_readout_t<float, 128>(q, k, v, sel, o_win, out, o_long_out, p, st);
}

}  // namespace fsl

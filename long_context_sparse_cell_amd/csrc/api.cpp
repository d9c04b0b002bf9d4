// Host side of the C ABI declared in include/fsl.h: parameter validation,
// workspace layout and the launch sequence. Nothing here allocates device
// memory or synchronises; every launch goes to the caller's stream.
#include <cmath>
#include <cstring>

#include "fsl_internal.h"

using namespace fsl;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }
bool aligned4(const void *ptr) { return ((uintptr_t)ptr & 3u) == 0; }

int check(const fsl_params *p) {
    if (!p) return FSL_E_INVAL;
    if (p->N < 1 || p->N >= (int64_t(1) << 31) || p->H < 1 || p->w < 1 || p->w > (1 << 30)) return FSL_E_INVAL;
    if (p->d < 2 || (p->d & 1)) return FSL_E_INVAL;
    if (p->s < 1 || p->B < 1 || p->B % p->s != 0 || p->K < 1 || p->W < 0 || p->P < -1) return FSL_E_INVAL;
    if (p->dtype != FSL_F32 && p->dtype != FSL_BF16) return FSL_E_INVAL;
    if (p->out_dtype != p->dtype && p->out_dtype != FSL_F32) return FSL_E_INVAL;
    if (!(p->scale >= 0.0f) || !std::isfinite(p->scale) || !(p->rope_base > 0.0f) || !(p->rms_eps > 0.0f) ||
        !std::isfinite(p->rho))
        return FSL_E_INVAL;
    if (!p->sigma || !p->lambda || !p->gamma) return FSL_E_INVAL;
    if (p->d != 64 && p->d != 128) return FSL_E_UNSUPPORTED;
    if (p->s != 16 && p->s != 32 && p->s != 64) return FSL_E_UNSUPPORTED;
    if (p->B % 16 != 0 || p->B > 256) return FSL_E_UNSUPPORTED;
    if (p->P < 0 || p->P > 64 || p->W > 64 || p->K > 8) return FSL_E_UNSUPPORTED;
    return FSL_OK;
}

KParams kparams(const fsl_params *p) {
    KParams k;
    std::memset(&k, 0, sizeof(k));
    k.N = p->N;
    k.C = p->N / p->s;
    k.nblk = (p->N + p->B - 1) / p->B;
    k.H = p->H; k.d = p->d; k.w = p->w; k.s = p->s; k.P = p->P; k.W = p->W; k.K = p->K; k.B = p->B;
    k.PW = p->P + p->W;
    k.dtype = p->dtype; k.out_dtype = p->out_dtype;
    k.scale = p->scale > 0.0f ? p->scale : (float)(1.0 / std::sqrt((double)p->d));
    k.rho = p->rho; k.rope_base = p->rope_base; k.rms_eps = p->rms_eps;
    k.sigma = p->sigma; k.lambda = p->lambda; k.gamma = p->gamma;
    k.nchunk = (int32_t)((k.C + kChunk - 1) / kChunk);
    k.nsg = k.nchunk / kGroup + 1;
    const int64_t wwin = p->w < p->N ? p->w : p->N;  // the window never reaches before token 0
    k.rope_lo = -(int32_t)(((wwin - 1) + kKTile - 1) / kKTile * kKTile);
    k.rope_n = kQTile - k.rope_lo;
    return k;
}

fsl_workspace_layout layout(const KParams &k) {
    fsl_workspace_layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
    L.kbar = take((size_t)k.H * k.C * k.d * sizeof(float));
    L.amax = take((size_t)k.H * k.C * sizeof(float));
    L.pool = take((size_t)k.H * k.nblk * k.PW * sizeof(int32_t));
    L.sel = take((size_t)k.H * k.N * k.K * sizeof(int32_t));
    L.rope = take((size_t)k.rope_n * (k.d / 2) * sizeof(float2));
    L.scan_a = take((size_t)scan_lists(k) * kChunk * sizeof(float));
    L.scan_i = take((size_t)scan_lists(k) * kChunk * sizeof(int32_t));
    L.o_win = take((size_t)k.H * k.N * k.d * sizeof(float));
    L.total = off;
    return L;
}

Work carve(void *ws, const fsl_workspace_layout &L) {
    char *b = (char *)ws;
    Work w;
    w.kbar = (float *)(b + L.kbar);
    w.amax = (float *)(b + L.amax);
    w.pool = (int32_t *)(b + L.pool);
    w.sel = (int32_t *)(b + L.sel);
    w.rope = (float2 *)(b + L.rope);
    w.scan_a = (float *)(b + L.scan_a);
    w.scan_i = (int32_t *)(b + L.scan_i);
    w.o_win = (float *)(b + L.o_win);
    return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FSL_OK : FSL_E_HIP; }

}  // namespace

extern "C" {

int fsl_version(void) { return FSL_VERSION; }

const char *fsl_strerror(int status) {
    switch (status) {
        case FSL_OK: return "ok";
        case FSL_E_INVAL: return "invalid argument (size, parameter, null or misaligned pointer)";
        case FSL_E_UNSUPPORTED: return "parameters valid for the method but not supported by this implementation";
        case FSL_E_WORKSPACE: return "workspace or state buffer too small";
        case FSL_E_STATE: return "decode state does not match the parameters";
        case FSL_E_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int fsl_check_params(const fsl_params *p) { return check(p); }

size_t fsl_workspace_bytes(const fsl_params *p) {
    if (check(p) != FSL_OK) return 0;
    return layout(kparams(p)).total;
}

int fsl_workspace_views(const fsl_params *p, fsl_workspace_layout *out) {
    int rc = check(p);
    if (rc != FSL_OK) return rc;
    if (!out) return FSL_E_INVAL;
    *out = layout(kparams(p));
    return FSL_OK;
}

int fsl_cell_stats(const void *k, float *kbar, float *amax, const fsl_params *p, hipStream_t stream) {
    int rc = check(p);
    if (rc != FSL_OK) return rc;
    if (!k || !kbar || !amax || !aligned16(k) || !aligned16(kbar) || !aligned4(amax)) return FSL_E_INVAL;
    return hip_status(launch_cell_stats(k, kbar, amax, kparams(p), stream));
}

int fsl_prune_select(const void *q, const float *kbar, const float *amax, int32_t *pool, int32_t *sel,
                     const fsl_params *p, void *ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check(p);
    if (rc != FSL_OK) return rc;
    if (!q || !kbar || !amax || !pool || !sel || !ws) return FSL_E_INVAL;
    if (!aligned16(q) || !aligned4(kbar) || !aligned4(amax) || !aligned4(pool) || !aligned4(sel) || !aligned16(ws))
        return FSL_E_INVAL;
    const KParams k = kparams(p);
    const fsl_workspace_layout L = layout(k);
    if (ws_bytes < L.total) return FSL_E_WORKSPACE;
    const Work w = carve(ws, L);
    hipError_t e = launch_prune(amax, pool, w, k, stream);
    if (e == hipSuccess)
        e = k.dtype == FSL_BF16 ? launch_select_mfma(q, kbar, amax, pool, sel, k, stream)
                                : launch_select(q, kbar, amax, pool, sel, k, stream);
    return hip_status(e);
}

static int attn_fwd_impl(const void *q, const void *k, const void *v, void *out, const fsl_params *p, void *ws,
                         size_t ws_bytes, int32_t *sel_out, float *o_win_out, float *o_long_out, hipEvent_t *ev,
                         hipStream_t stream) {
    int rc = check(p);
    if (rc != FSL_OK) return rc;
    if (!q || !k || !v || !out || !ws) return FSL_E_INVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ws)) return FSL_E_INVAL;
    if ((sel_out && !aligned4(sel_out)) || (o_win_out && !aligned16(o_win_out)) ||
        (o_long_out && !aligned16(o_long_out)))
        return FSL_E_INVAL;
    const KParams kp = kparams(p);
    const fsl_workspace_layout L = layout(kp);
    if (ws_bytes < L.total) return FSL_E_WORKSPACE;
    const Work w = carve(ws, L);
    int stage = 0;
    auto mark = [&](hipError_t e) {
        if (e == hipSuccess && ev) e = hipEventRecord(ev[stage], stream);
        ++stage;
        return e;
    };
    hipError_t e = mark(hipSuccess);
    if (e == hipSuccess) e = mark(launch_cell_stats(k, w.kbar, w.amax, kp, stream));
    if (e == hipSuccess) e = mark(launch_prune(w.amax, w.pool, w, kp, stream));
    if (e == hipSuccess)
        e = mark(kp.dtype == FSL_BF16 ? launch_select_mfma(q, w.kbar, w.amax, w.pool, w.sel, kp, stream)
                                      : launch_select(q, w.kbar, w.amax, w.pool, w.sel, kp, stream));
    if (e == hipSuccess) e = mark(launch_rope_table(w.rope, kp, stream));
    if (e == hipSuccess)
        e = mark(kp.dtype == FSL_BF16 ? launch_window_bf16(q, k, v, w.rope, w.o_win, kp, stream)
                                      : launch_window(q, k, v, w.rope, w.o_win, kp, stream));
    if (e == hipSuccess)
        e = mark(kp.dtype == FSL_BF16
                     ? launch_readout_cells(q, k, v, w.sel, w.pool, w.o_win, out, o_long_out, kp, stream)
                     : launch_readout_mix(q, k, v, w.sel, w.o_win, out, o_long_out, kp, stream));
    if (e == hipSuccess && sel_out)
        e = hipMemcpyAsync(sel_out, w.sel, (size_t)kp.H * kp.N * kp.K * sizeof(int32_t), hipMemcpyDeviceToDevice,
                           stream);
    if (e == hipSuccess && o_win_out)
        e = hipMemcpyAsync(o_win_out, w.o_win, (size_t)kp.H * kp.N * kp.d * sizeof(float), hipMemcpyDeviceToDevice,
                           stream);
    return hip_status(e);
}

int fsl_attn_fwd(const void *q, const void *k, const void *v, void *out, const fsl_params *p, void *ws,
                 size_t ws_bytes, int32_t *sel_out, float *o_win_out, float *o_long_out, hipStream_t stream) {
    return attn_fwd_impl(q, k, v, out, p, ws, ws_bytes, sel_out, o_win_out, o_long_out, nullptr, stream);
}

int fsl_attn_fwd_timed(const void *q, const void *k, const void *v, void *out, const fsl_params *p, void *ws,
                       size_t ws_bytes, hipEvent_t *stage_events, hipStream_t stream) {
    if (!stage_events) return check(p) != FSL_OK ? check(p) : FSL_E_INVAL;
    return attn_fwd_impl(q, k, v, out, p, ws, ws_bytes, nullptr, nullptr, nullptr, stage_events, stream);
}

}  // extern "C"

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
    if (p->P > 64 || p->W > 64 || p->K > 8) return FSL_E_UNSUPPORTED;
    // work-group ids over (head, 64-token tile) must fit one 32-bit grid dimension
    if ((p->N / 64 + 1) * (int64_t)p->H >= (int64_t(1) << 31)) return FSL_E_UNSUPPORTED;
    return FSL_OK;
}

KParams kparams(const fsl_params *p) {
    KParams k;
    std::memset(&k, 0, sizeof(k));
    k.N = p->N;
    k.C = p->N / p->s;
    k.nblk = (p->N + p->B - 1) / p->B;
    k.H = p->H; k.d = p->d; k.w = p->w; k.s = p->s; k.P = p->P; k.W = p->W; k.K = p->K; k.B = p->B;
    k.PW = p->P < 0 ? 0 : p->P + p->W;  // no pool table without pruning
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

// full: the forward's arrays; otherwise only what the decode prefill uses (cell
// statistics, pools and the prune-scan lists)
fsl_workspace_layout layout(const KParams &k, bool full = true) {
    fsl_workspace_layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
    L.kbar = take((size_t)k.H * k.C * k.d * sizeof(float));
    L.amax = take((size_t)k.H * k.C * sizeof(float));
    L.pool = take((size_t)k.H * k.nblk * k.PW * sizeof(int32_t));
    L.sel = take(full ? (size_t)k.H * k.N * k.K * sizeof(int32_t) : 0);
    L.rope = take(full ? (size_t)k.rope_n * (k.d / 2) * sizeof(float2) : 0);
    L.scan_a = take((size_t)scan_lists(k) * kChunk * sizeof(float));
    L.scan_i = take((size_t)scan_lists(k) * kChunk * sizeof(int32_t));
    const bool bf = full && k.dtype == FSL_BF16;  // prepared fp16 keys/values, near-tie list: bf16 forward only
    // fp32 inputs: the window branch's output; bf16 inputs: each selected cell's partial readout
    L.o_win = take(full && !bf ? (size_t)k.H * k.N * k.d * sizeof(float) : 0);
    L.rope_abs = take(bf ? (size_t)(rope_abs_rows_hi(k) + kRopeSpan) * (k.d / 2) * sizeof(float2) : 0);
    L.kt = take(bf ? (size_t)k.H * kt_head_elems(k) * sizeof(uint16_t) : 0);
    L.vt = take(bf ? (size_t)k.H * vt_head_elems(k) * sizeof(uint16_t) : 0);
    L.plan = take(bf ? (size_t)plan_bytes(k) : 0);
    L.part = take(bf ? (size_t)k.H * k.N * k.K * k.d * sizeof(uint16_t) : 0);
    L.plse = take(bf ? (size_t)k.H * k.N * k.K * sizeof(float) : 0);
    const bool fs = k.P < 0;  // no pruning: a contender list per near-tie, and the split cell means
    L.fixups = take(bf ? (size_t)(fs ? fix_words_fs(k) : fix_words(k)) * sizeof(uint32_t) : 0);
    L.khi = take(bf && fs ? (size_t)k.H * k.C * k.d * sizeof(uint16_t) : 0);
    L.klo = take(bf && fs ? (size_t)k.H * k.C * k.d * sizeof(uint16_t) : 0);
    L.kcf = take(bf && fs ? (size_t)k.H * k.C * sizeof(float4) : 0);
    L.status = take(sizeof(uint32_t));
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
    w.rope_abs = (float2 *)(b + L.rope_abs);
    w.kt = (uint16_t *)(b + L.kt);
    w.vt = (uint16_t *)(b + L.vt);
    w.plan = (uint32_t *)(b + L.plan);
    w.part = (uint16_t *)(b + L.part);
    w.plse = (float *)(b + L.plse);
    w.fix = L.khi > L.fixups ? (uint32_t *)(b + L.fixups) : nullptr;  // present iff it has bytes
    w.khi = L.klo > L.khi ? (uint16_t *)(b + L.khi) : nullptr;
    w.klo = L.kcf > L.klo ? (uint16_t *)(b + L.klo) : nullptr;
    w.kcf = L.status > L.kcf ? (float4 *)(b + L.kcf) : nullptr;
    w.status = (uint32_t *)(b + L.status);
    return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FSL_OK : FSL_E_HIP; }


constexpr int32_t kDecodeMaxW = 65536;  // bounds the ring of w + B + s tokens per (sequence, head)

int check_decode(const fsl_params *p) {
    if (!p) return FSL_E_INVAL;
    fsl_params q = *p;
    q.N = 1;
    int rc = check(&q);
    if (rc != FSL_OK) return rc;
    // the bounded state holds P + W pool cells: the unpruned variant has no such bound
    if (p->P < 0 || p->w > kDecodeMaxW) return FSL_E_UNSUPPORTED;
    return FSL_OK;
}

size_t align16(size_t x) { return (x + 15) / 16 * 16; }

DecodeLayout dlayout(const fsl_params *p) {
    DecodeLayout L;
    const size_t e = p->dtype == FSL_BF16 ? 2 : 4;
    L.R = p->w + p->B + p->s;
    L.PW = p->P + p->W;
    L.off_rec = 256;
    size_t o = 16;  // int64 t, int64 block
    L.o_cell = (int64_t)o; o = align16(o + 4 * (size_t)L.PW);
    L.o_a = (int64_t)o; o = align16(o + 4 * (size_t)L.PW);
    L.o_kbar = (int64_t)o; o = align16(o + 4 * (size_t)L.PW * p->d);
    L.o_sk = (int64_t)o; o = align16(o + e * (size_t)L.PW * p->s * p->d);
    L.o_sv = (int64_t)o; o = align16(o + e * (size_t)L.PW * p->s * p->d);
    L.o_rk = (int64_t)o; o = align16(o + e * (size_t)L.R * p->d);
    L.o_rv = (int64_t)o; o = align16(o + e * (size_t)L.R * p->d);
    L.o_rkr = (int64_t)o; o = align16(o + e * (size_t)L.R * p->d);  // fp16 for bf16 inputs, else fp32
    L.rec_bytes = (int64_t)align_up(o);
    return L;
}

size_t decode_bytes(const fsl_params *p, int32_t n_seq) {
    const DecodeLayout L = dlayout(p);
    return (size_t)L.off_rec + (size_t)n_seq * p->H * (size_t)L.rec_bytes;
}

// backward workspace: the rotated q and k, the upstream gradient, the long branch's
// softmax-output gradient, five row statistics, the (cell, query) pair sort, the cells'
// runs and heavy-cell chunk sums, and the long branch's dq of every (query, rank) pair
struct BwdLayout {
    size_t rope, qr, kr, dO, do_l, lse_w, D_w, lse_l, D_l, dg, pkey, pval, pkey2, pval2, shist, stot, cseg, hcount,
        hitems, hcells, hpart, dqp, pml, status, total;
};

// the long branch's key side sorts the H N K (query, rank) pairs with 32-bit indices
bool bwd_supported(const KParams &k) { return (int64_t)k.H * k.N * k.K < (int64_t(1) << 31); }

BwdLayout bwd_layout(const KParams &k) {
    BwdLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
    const size_t rows = (size_t)k.H * k.N, elems = rows * k.d;
    L.rope = take((size_t)(rope_abs_rows_hi(k) + kRopeSpan) * (k.d / 2) * sizeof(float2));
    L.qr = take(elems * sizeof(float));
    L.kr = take(elems * sizeof(float));
    L.dO = take(elems * sizeof(float));
    L.do_l = take(elems * sizeof(float));
    L.lse_w = take(rows * sizeof(float));
    L.D_w = take(rows * sizeof(float));
    L.lse_l = take(rows * sizeof(float));
    L.D_l = take(rows * sizeof(float));
    L.dg = take(rows * sizeof(float));
    const int64_t npair = (int64_t)k.H * k.N * k.K;
    L.pkey = take((size_t)npair * sizeof(uint32_t));
    L.pval = take((size_t)npair * sizeof(uint32_t));
    L.pkey2 = take((size_t)npair * sizeof(uint32_t));
    L.pval2 = take((size_t)npair * sizeof(uint32_t));
    L.shist = take(sort_hist_words(npair) * sizeof(uint32_t));
    L.stot = take(sort_total_words(npair) * sizeof(uint32_t));
    L.cseg = take((size_t)k.H * k.C * 2 * sizeof(int32_t));
    L.hcount = take(2 * sizeof(int32_t));
    L.hitems = take((size_t)heavy_items_max(k) * 2 * sizeof(int32_t));
    L.hcells = take((size_t)heavy_cells_max(k) * 3 * sizeof(int32_t));
    L.hpart = take((size_t)heavy_items_max(k) * 2 * k.s * k.d * sizeof(float));
    L.dqp = take((size_t)npair * k.d * sizeof(float));
    L.pml = take((size_t)npair * sizeof(float2));
    L.status = take(sizeof(uint32_t));
    L.total = off;
    return L;
}

int32_t decode_capacity(const fsl_params *p, size_t state_bytes) {
    const DecodeLayout L = dlayout(p);
    if (state_bytes < (size_t)L.off_rec) return 0;
    return (int32_t)((state_bytes - (size_t)L.off_rec) / ((size_t)p->H * (size_t)L.rec_bytes));
}

size_t fsb_workspace_extra(const KParams &p, size_t (*align)(size_t)) {
    const int lv = fsb_levels(p);
    const size_t nodes = (size_t)p.H * 2 * lv * 2 * p.C, leaves = (size_t)p.H * 2 * lv * p.C;
    return align(p.H * p.C * sizeof(uint32_t)) + align(p.H * p.C * sizeof(int32_t)) +
           align((size_t)p.H * (p.C + 1) * sizeof(int32_t)) + align(nodes * p.d * sizeof(float)) +
           align(nodes * sizeof(double)) + align(nodes * sizeof(float)) + align(nodes * sizeof(int32_t)) +
           align(leaves * sizeof(int32_t));
}

void fsb_carve(char *base, const KParams &p, size_t (*align)(size_t), FsbWork &w) {
    const int lv = fsb_levels(p);
    const size_t nodes = (size_t)p.H * 2 * lv * 2 * p.C, leaves = (size_t)p.H * 2 * lv * p.C;
    size_t off = 0;
    auto take = [&](size_t bytes) { char *at = base + off; off += align(bytes); return at; };
    w.codes = (uint32_t *)take(p.H * p.C * sizeof(uint32_t));
    w.list1 = (int32_t *)take(p.H * p.C * sizeof(int32_t));
    w.hcount = (int32_t *)take((size_t)p.H * (p.C + 1) * sizeof(int32_t));
    w.mu = (float *)take(nodes * p.d * sizeof(float));
    w.rad = (double *)take(nodes * sizeof(double));
    w.amax = (float *)take(nodes * sizeof(float));
    w.pmin = (int32_t *)take(nodes * sizeof(int32_t));
    w.leaf = (int32_t *)take(leaves * sizeof(int32_t));
}

// FS-B runs the unpruned variant's forward (no pool, arbitrary selections in the
// readout) with its own selection; its workspace is that forward's plus the forests
size_t fsb_align(size_t x) { return align_up(x); }

fsl_params fsb_base(const fsl_params *p) {
    fsl_params q = *p;
    q.P = -1;
    return q;
}

int check_fsb(const fsl_params *p, const fsl_fsb_params *fb) {
    int rc = check(p);
    if (rc != FSL_OK) return rc;
    if (!fb || !fb->tau || !fb->proj || fb->reserved != 0) return FSL_E_INVAL;
    if (fb->beam < 1 || fb->beam > 32 || !(p->rho >= 0.0f)) return FSL_E_UNSUPPORTED;
    if (!aligned4(fb->tau) || !aligned4(fb->proj)) return FSL_E_INVAL;
    return FSL_OK;
}

size_t fsb_bytes(const fsl_params *p) {
    const fsl_params b = fsb_base(p);
    const KParams k = kparams(&b);
    return layout(k).total + fsb_workspace_extra(k, fsb_align);
}

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
    const bool fs = p->P < 0;  // no pruning: no pool is written and pool may be NULL
    if (!q || !kbar || !amax || (!pool && !fs) || !sel || !ws) return FSL_E_INVAL;
    if (!aligned16(q) || !aligned4(kbar) || !aligned4(amax) || !aligned4(pool) || !aligned4(sel) || !aligned16(ws))
        return FSL_E_INVAL;
    const KParams k = kparams(p);
    const fsl_workspace_layout L = layout(k);
    if (ws_bytes < L.total) return FSL_E_WORKSPACE;
    const Work w = carve(ws, L);
    hipError_t e = hipSuccess;
    if (fs) {
        e = k.dtype == FSL_BF16 ? launch_select_fs(q, kbar, amax, sel, w, k, stream)
                                : launch_select(q, kbar, amax, nullptr, sel, k, stream);
        return hip_status(e);
    }
    e = launch_prune(amax, pool, w, k, stream);
    if (e == hipSuccess)
        e = k.dtype == FSL_BF16 ? launch_select_mfma(q, kbar, amax, pool, sel, w.fix, k, stream)
                                : launch_select(q, kbar, amax, pool, sel, k, stream);
    if (e == hipSuccess && k.dtype == FSL_BF16) e = launch_select_fixup(q, kbar, amax, pool, sel, w.fix, k, stream);
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
    if (kp.dtype == FSL_BF16 && kp.P < 0 && !ro_supported(kp)) return FSL_E_UNSUPPORTED;  // 32-bit list indices
    const Work w = carve(ws, L);
    int stage = 0;
    auto mark = [&](hipError_t e) {
        if (e == hipSuccess && ev) e = hipEventRecord(ev[stage], stream);
        ++stage;
        return e;
    };
    hipError_t e = mark(hipSuccess);
    const bool bf = kp.dtype == FSL_BF16;
    // bf16: one pass over k and v gives the cell statistics, the rotated fp16 keys and the
    // transposed fp16 values (recorded as the statistics stage; the preparation stage is empty)
    if (e == hipSuccess)
        e = mark(bf ? launch_kv_prep(k, v, w.kt, w.vt, w.rope_abs, w.kbar, w.amax, w.status, kp, stream)
                    : launch_cell_stats(k, w.kbar, w.amax, kp, stream));
    const bool fs = kp.P < 0;  // no pruning: the prune stage is empty
    if (e == hipSuccess) e = mark(fs ? hipSuccess : launch_prune(w.amax, w.pool, w, kp, stream));
    if (e == hipSuccess)
        e = mark(fs ? (kp.dtype == FSL_BF16 ? launch_select_fs(q, w.kbar, w.amax, w.sel, w, kp, stream)
                                            : launch_select(q, w.kbar, w.amax, nullptr, w.sel, kp, stream))
                 : kp.dtype == FSL_BF16
                     ? (launch_select_mfma(q, w.kbar, w.amax, w.pool, w.sel, w.fix, kp, stream) == hipSuccess
                            ? launch_select_fixup(q, w.kbar, w.amax, w.pool, w.sel, w.fix, kp, stream)
                            : hipErrorLaunchFailure)
                     : launch_select(q, w.kbar, w.amax, w.pool, w.sel, kp, stream));
    if (e == hipSuccess) e = mark(bf ? hipSuccess : launch_rope_table(w.rope, w.status, kp, stream));
    // bf16: the long branch first (a partial output per selected cell), then the window
    // kernel, which merges the partials, applies RMSNorm and the mix, and writes out;
    // fp32: the window branch, then the long branch with RMSNorm and the mix
    if (bf) {
        if (e == hipSuccess)
            e = mark(kp.P < 0 ? launch_readout_cells(q, k, w.vt, w.sel, w.plan, w.part, w.plse, kp, stream)
                              : launch_readout_units(q, k, w.vt, w.sel, w.plan, w.part, w.plse, kp, 0, kp.N, stream));
        if (e == hipSuccess)
            e = mark(launch_window_bf16(q, w.kt, w.vt, w.rope_abs, w.sel, w.part, w.plse, out, o_win_out,
                                        o_long_out, kp, 0, kp.N, stream));
    } else {
        if (e == hipSuccess) e = mark(launch_window(q, k, v, w.rope, w.o_win, kp, stream));
        if (e == hipSuccess) e = mark(launch_readout_mix(q, k, v, w.sel, w.o_win, out, o_long_out, kp, stream));
    }
    if (e == hipSuccess && sel_out)
        e = hipMemcpyAsync(sel_out, w.sel, (size_t)kp.H * kp.N * kp.K * sizeof(int32_t), hipMemcpyDeviceToDevice,
                           stream);
    if (e == hipSuccess && o_win_out && !bf)
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

size_t fsl_attn_bwd_workspace_bytes(const fsl_params *p) {
    if (check(p) != FSL_OK) return 0;
    const KParams k = kparams(p);
    if (!bwd_supported(k)) return 0;
    return bwd_layout(k).total;
}

int fsl_attn_bwd(const void *q, const void *k, const void *v, const void *dout, const fsl_params *p,
                 const void *fwd_ws, size_t fwd_ws_bytes, void *ws, size_t ws_bytes, float *dq, float *dk,
                 float *dv, float *dgamma, hipStream_t stream) {
    int rc = check(p);
    if (rc != FSL_OK) return rc;
    if (!q || !k || !v || !dout || !fwd_ws || !ws || !dq || !dk || !dv || !dgamma) return FSL_E_INVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(fwd_ws) ||
        !aligned16(ws) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(dgamma))
        return FSL_E_INVAL;
    const KParams kp = kparams(p);
    if (!bwd_supported(kp)) return FSL_E_UNSUPPORTED;
    const fsl_workspace_layout FL = layout(kp);
    const BwdLayout BL = bwd_layout(kp);
    if (fwd_ws_bytes < FL.total || ws_bytes < BL.total) return FSL_E_WORKSPACE;
    const char *f = (const char *)fwd_ws;
    char *b = (char *)ws;
    BwdWork w;
    w.rope = (float2 *)(b + BL.rope);
    w.qr = (float *)(b + BL.qr);
    w.kr = (float *)(b + BL.kr);
    w.dO = (float *)(b + BL.dO);
    w.do_l = (float *)(b + BL.do_l);
    w.lse_w = (float *)(b + BL.lse_w);
    w.D_w = (float *)(b + BL.D_w);
    w.lse_l = (float *)(b + BL.lse_l);
    w.D_l = (float *)(b + BL.D_l);
    w.dg = (float *)(b + BL.dg);
    w.pkey = (uint32_t *)(b + BL.pkey);
    w.pval = (uint32_t *)(b + BL.pval);
    w.pkey2 = (uint32_t *)(b + BL.pkey2);
    w.pval2 = (uint32_t *)(b + BL.pval2);
    w.shist = (uint32_t *)(b + BL.shist);
    w.stot = (uint32_t *)(b + BL.stot);
    w.cseg = (int32_t *)(b + BL.cseg);
    w.hcount = (int32_t *)(b + BL.hcount);
    w.hitems = (int32_t *)(b + BL.hitems);
    w.hcells = (int32_t *)(b + BL.hcells);
    w.hpart = (float *)(b + BL.hpart);
    w.dqp = (float *)(b + BL.dqp);
    w.pml = (float2 *)(b + BL.pml);
    w.status = (uint32_t *)(b + BL.status);
    return hip_status(launch_attn_bwd(q, k, v, dout, (const int32_t *)(f + FL.sel), (const int32_t *)(f + FL.pool), w, dq, dk, dv, dgamma, kp, stream));
}

size_t fsl_fsb_workspace_bytes(const fsl_params *p) {
    if (check(p) != FSL_OK) return 0;
    return fsb_bytes(p);
}

static int fsb_run(const void *q, const void *k, const void *v, void *out, const fsl_params *p,
                   const fsl_fsb_params *fb, void *ws, size_t ws_bytes, int32_t *sel_dst, bool forward,
                   hipStream_t stream) {
    int rc = check_fsb(p, fb);
    if (rc != FSL_OK) return rc;
    if (!q || !k || !ws || (forward && (!v || !out)) || (!forward && !sel_dst)) return FSL_E_INVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(ws) || (v && !aligned16(v)) || (out && !aligned16(out)) ||
        (sel_dst && !aligned4(sel_dst)))
        return FSL_E_INVAL;
    if (ws_bytes < fsb_bytes(p)) return FSL_E_WORKSPACE;
    const fsl_params base = fsb_base(p);
    const KParams kp = kparams(&base);
    if (forward && kp.dtype == FSL_BF16 && !ro_supported(kp)) return FSL_E_UNSUPPORTED;  // 32-bit list indices
    const fsl_workspace_layout L = layout(kp);
    const Work w = carve(ws, L);
    FsbWork fw;
    fsb_carve((char *)ws + L.total, kp, fsb_align, fw);
    const bool bf = kp.dtype == FSL_BF16;
    hipError_t e = bf && forward ? launch_kv_prep(k, v, w.kt, w.vt, w.rope_abs, w.kbar, w.amax, w.status, kp, stream)
                                 : launch_cell_stats(k, w.kbar, w.amax, kp, stream);
    if (e == hipSuccess)
        e = launch_fsb_select(q, k, w.kbar, w.amax, forward ? w.sel : sel_dst, fw, fb->tau, fb->proj, fb->beam, kp,
                              stream);
    if (!forward) return hip_status(e);
    if (e == hipSuccess && !bf) e = launch_rope_table(w.rope, w.status, kp, stream);
    if (bf) {
        if (e == hipSuccess) e = launch_readout_cells(q, k, w.vt, w.sel, w.plan, w.part, w.plse, kp, stream);
        if (e == hipSuccess)
            e = launch_window_bf16(q, w.kt, w.vt, w.rope_abs, w.sel, w.part, w.plse, out, nullptr, nullptr, kp, 0,
                                   kp.N, stream);
    } else {
        if (e == hipSuccess) e = launch_window(q, k, v, w.rope, w.o_win, kp, stream);
        if (e == hipSuccess) e = launch_readout_mix(q, k, v, w.sel, w.o_win, out, nullptr, kp, stream);
    }
    if (e == hipSuccess && sel_dst)
        e = hipMemcpyAsync(sel_dst, w.sel, (size_t)kp.H * kp.N * kp.K * sizeof(int32_t), hipMemcpyDeviceToDevice,
                           stream);
    return hip_status(e);
}

int fsl_fsb_select(const void *q, const void *k, const fsl_params *p, const fsl_fsb_params *fb, int32_t *sel,
                   void *ws, size_t ws_bytes, hipStream_t stream) {
    return fsb_run(q, k, nullptr, nullptr, p, fb, ws, ws_bytes, sel, false, stream);
}

int fsl_attn_fwd_fsb(const void *q, const void *k, const void *v, void *out, const fsl_params *p,
                     const fsl_fsb_params *fb, void *ws, size_t ws_bytes, int32_t *sel_out, hipStream_t stream) {
    return fsb_run(q, k, v, out, p, fb, ws, ws_bytes, sel_out, true, stream);
}

size_t fsl_decode_state_bytes(const fsl_params *p, int32_t n_seq) {
    if (check_decode(p) != FSL_OK || n_seq < 1) return 0;
    return decode_bytes(p, n_seq);
}

int fsl_decode_init(void *state, size_t state_bytes, int32_t n_seq, const fsl_params *p, hipStream_t stream) {
    int rc = check_decode(p);
    if (rc != FSL_OK) return rc;
    if (!state || !aligned16(state) || n_seq < 1) return FSL_E_INVAL;
    if (state_bytes < decode_bytes(p, n_seq)) return FSL_E_WORKSPACE;
    fsl_params q = *p;
    q.N = 1;
    return hip_status(launch_decode_init(state, kparams(&q), dlayout(p), n_seq, stream));
}

size_t fsl_decode_prefill_workspace_bytes(const fsl_params *p, int64_t prefix_len) {
    if (check_decode(p) != FSL_OK || prefix_len < 1 || prefix_len >= (int64_t(1) << 31) - p->B) return 0;
    fsl_params q = *p;
    q.N = prefix_len + p->B;
    return layout(kparams(&q), false).total;
}

int fsl_decode_prefill(void *state, size_t state_bytes, int32_t seq, const void *k_prefix, const void *v_prefix,
                       int64_t prefix_len, const fsl_params *p, void *ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_decode(p);
    if (rc != FSL_OK) return rc;
    if (!state || !k_prefix || !v_prefix || !ws || !aligned16(state) || !aligned16(k_prefix) ||
        !aligned16(v_prefix) || !aligned16(ws))
        return FSL_E_INVAL;
    if (prefix_len < 1 || prefix_len >= (int64_t(1) << 31) - p->B || seq < 0) return FSL_E_INVAL;
    if (seq >= decode_capacity(p, state_bytes)) return FSL_E_INVAL;
    if (ws_bytes < fsl_decode_prefill_workspace_bytes(p, prefix_len)) return FSL_E_WORKSPACE;
    fsl_params qa = *p;
    qa.N = prefix_len + p->B;
    const Work w = carve(ws, layout(kparams(&qa), false));
    fsl_params qs = *p;
    qs.N = prefix_len;
    KParams ks = kparams(&qs);            // statistics over the prefix's complete cells
    KParams kpool = ks;
    kpool.nblk = prefix_len / p->B + 1;   // pools up to the block holding position prefix_len
    hipError_t e = launch_cell_stats(k_prefix, w.kbar, w.amax, ks, stream);
    if (e == hipSuccess) e = launch_prune(w.amax, w.pool, w, kpool, stream);
    if (e == hipSuccess) e = launch_decode_prefill(state, seq, k_prefix, v_prefix, prefix_len, w, kpool, dlayout(p), stream);
    return hip_status(e);
}

int fsl_decode_append(void *state, size_t state_bytes, int32_t seq0, int32_t n, const void *k, const void *v,
                      int64_t len, const fsl_params *p, hipStream_t stream) {
    int rc = check_decode(p);
    if (rc != FSL_OK) return rc;
    if (!state || !k || !v || !aligned16(state) || !aligned16(k) || !aligned16(v)) return FSL_E_INVAL;
    if (len < 1 || len >= (int64_t(1) << 31) - p->B || seq0 < 0 || n < 1) return FSL_E_INVAL;
    if ((int64_t)seq0 + n > decode_capacity(p, state_bytes)) return FSL_E_INVAL;
    if ((int64_t)n * p->H >= (int64_t(1) << 31)) return FSL_E_UNSUPPORTED;
    fsl_params qq = *p;
    qq.N = 1;
    return hip_status(launch_decode_append(state, seq0, n, k, v, len, kparams(&qq), dlayout(p), stream));
}

int fsl_decode_step(void *state, size_t state_bytes, const void *q, const void *k, const void *v, void *out,
                    int32_t n_seq, const fsl_params *p, int32_t *sel_out, hipStream_t stream) {
    int rc = check_decode(p);
    if (rc != FSL_OK) return rc;
    if (!state || !q || !k || !v || !out || n_seq < 1) return FSL_E_INVAL;
    if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (sel_out && !aligned4(sel_out)))
        return FSL_E_INVAL;
    if (n_seq > decode_capacity(p, state_bytes)) return FSL_E_WORKSPACE;
    fsl_params qq = *p;
    qq.N = 1;
    return hip_status(launch_decode_step(state, q, k, v, out, sel_out, n_seq, kparams(&qq), dlayout(p), stream));
}

int fsl_decode_validate(const void *state, size_t state_bytes, const fsl_params *p, int32_t n_seq) {
    int rc = check_decode(p);
    if (rc != FSL_OK) return rc;
    if (!state || n_seq < 1) return FSL_E_INVAL;
    if (state_bytes < decode_bytes(p, n_seq)) return FSL_E_WORKSPACE;
    DecodeHeader hd;
    if (hipMemcpy(&hd, state, sizeof(hd), hipMemcpyDeviceToHost) != hipSuccess) return FSL_E_HIP;
    const DecodeLayout L = dlayout(p);
    if (hd.magic != kDecodeMagic || hd.version != kDecodeVersion) return FSL_E_STATE;
    if (hd.H != p->H || hd.d != p->d || hd.w != p->w || hd.s != p->s || hd.P != p->P || hd.W != p->W ||
        hd.K != p->K || hd.B != p->B || hd.dtype != p->dtype || hd.n_seq != n_seq || hd.R != L.R ||
        hd.PW != L.PW || hd.rec_bytes != L.rec_bytes)
        return FSL_E_STATE;
    return FSL_OK;
}

}  // extern "C"

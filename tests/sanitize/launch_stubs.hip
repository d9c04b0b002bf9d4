// Recording stand-ins for the kernel launchers, for the host-only sanitizer
// build of the C ABI (api.cpp): nothing is launched and no pointer is
// dereferenced. Each stand-in counts the call and checks that every workspace
// array it receives lies inside the buffer the driver passed in.
#include <cstdio>
#include <cstdlib>

#include "fsl_internal.h"

namespace fsl {

int g_launches = 0;
const char *g_ws_lo = nullptr;  // the workspace of the current call (null: not a workspace call)
const char *g_ws_hi = nullptr;

static void inside(const void *ptr, const char *what) {
    if (!g_ws_lo || !ptr) return;
    const char *c = (const char *)ptr;
    if (c < g_ws_lo || c >= g_ws_hi) {
        std::fprintf(stderr, "launch stub: %s at %p outside the workspace [%p, %p)\n", what, ptr, (const void *)g_ws_lo,
                     (const void *)g_ws_hi);
        std::abort();
    }
}

static void work(const Work &w) {
    inside(w.kbar, "kbar"); inside(w.amax, "amax"); inside(w.scan_a, "scan_a"); inside(w.scan_i, "scan_i");
    inside(w.fix, "fix"); inside(w.khi, "khi"); inside(w.klo, "klo"); inside(w.kcf, "kcf");
}

hipError_t launch_cell_stats(const void *, float *kbar, float *amax, const KParams &, hipStream_t) {
    ++g_launches; inside(kbar, "kbar"); inside(amax, "amax"); return hipSuccess;
}
hipError_t launch_prune(const float *amax, int32_t *pool, const Work &w, const KParams &, hipStream_t) {
    ++g_launches; inside(amax, "amax"); work(w); (void)pool; return hipSuccess;
}
hipError_t launch_select(const void *, const float *, const float *, const int32_t *, int32_t *, const KParams &,
                         hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_select_mfma(const void *, const float *, const float *, const int32_t *, int32_t *, uint32_t *fix,
                              const KParams &, hipStream_t) { ++g_launches; inside(fix, "fix"); return hipSuccess; }
hipError_t launch_select_fixup(const void *, const float *, const float *, const int32_t *, int32_t *,
                               const uint32_t *fix, const KParams &, hipStream_t) {
    ++g_launches; inside(fix, "fix"); return hipSuccess;
}
hipError_t launch_select_fs(const void *, const float *, const float *, int32_t *, const Work &w, const KParams &,
                            hipStream_t) { ++g_launches; work(w); return hipSuccess; }
hipError_t launch_rope_table(float2 *tab, uint32_t *status, const KParams &, hipStream_t) {
    ++g_launches; inside(tab, "rope"); inside(status, "status"); return hipSuccess;
}
hipError_t launch_window(const void *, const void *, const void *, const float2 *rope, float *o_win, const KParams &,
                         hipStream_t) { ++g_launches; inside(rope, "rope"); inside(o_win, "o_win"); return hipSuccess; }
hipError_t launch_kv_prep(const void *, const void *, uint16_t *kt, uint16_t *vt, float2 *rope_abs, float *kbar,
                          float *amax, uint32_t *status, const KParams &, hipStream_t) {
    ++g_launches; inside(kt, "kt"); inside(vt, "vt"); inside(rope_abs, "rope_abs"); inside(kbar, "kbar");
    inside(amax, "amax"); inside(status, "status"); return hipSuccess;
}
hipError_t launch_window_bf16(const void *, const uint16_t *kt, const uint16_t *vt, const float2 *rope,
                              const int32_t *sel, const uint16_t *part, const float *plse, void *, float *, float *,
                              const KParams &, int64_t, int64_t, hipStream_t) {
    ++g_launches; inside(kt, "kt"); inside(vt, "vt"); inside(rope, "rope_abs"); inside(sel, "sel");
    inside(part, "part"); inside(plse, "plse");
    return hipSuccess;
}
hipError_t launch_readout_units(const void *, const void *, const uint16_t *vt, const int32_t *sel, uint32_t *plan,
                                uint16_t *part, float *plse, const KParams &k, int64_t, int64_t, hipStream_t) {
    ++g_launches; inside(vt, "vt"); inside(sel, "sel"); inside(plan, "plan"); inside(part, "part");
    inside(plse, "plse"); inside((const char *)plan + plan_records(k) * kPlanRecBytes - 1, "plan (last byte)");
    return hipSuccess;
}
hipError_t launch_readout_cells(const void *, const void *, const uint16_t *vt, const int32_t *sel, uint32_t *plan,
                                uint16_t *part, float *plse, const KParams &k, hipStream_t) {
    ++g_launches; inside(vt, "vt"); inside(sel, "sel"); inside(plan, "plan"); inside(part, "part");
    inside(plse, "plse"); inside(plan + ro_plan_words(k) - 1, "plan (last word)");
    return hipSuccess;
}
hipError_t launch_readout_mix(const void *, const void *, const void *, const int32_t *sel, const float *o_win, void *,
                              float *, const KParams &, hipStream_t) {
    ++g_launches; inside(sel, "sel"); inside(o_win, "o_win"); return hipSuccess;
}
hipError_t launch_rope_abs_table(float2 *tab, uint32_t *status, const KParams &, hipStream_t) {
    ++g_launches; inside(tab, "rope_abs"); inside(status, "status"); return hipSuccess;
}
hipError_t launch_attn_bwd(const void *, const void *, const void *, const void *, const int32_t *, const int32_t *,
                           const BwdWork &w, float *, float *, float *, float *, const KParams &,
                           hipStream_t) {
    ++g_launches;
    inside(w.rope, "bwd rope"); inside(w.qr, "qr"); inside(w.kr, "kr"); inside(w.dO, "dO"); inside(w.do_l, "do_l");
    inside(w.lse_w, "lse_w"); inside(w.D_w, "D_w"); inside(w.lse_l, "lse_l"); inside(w.D_l, "D_l");
    inside(w.dg, "dg"); inside(w.pkey, "pkey"); inside(w.pval, "pval"); inside(w.pkey2, "pkey2");
    inside(w.pval2, "pval2"); inside(w.shist, "shist"); inside(w.stot, "stot"); inside(w.cseg, "cseg");
    inside(w.hcount, "hcount"); inside(w.hitems, "hitems"); inside(w.hcells, "hcells"); inside(w.hpart, "hpart"); inside(w.dqp, "dqp"); inside(w.pml, "pml");
    inside(w.status, "bwd status");
    return hipSuccess;
}
hipError_t launch_fsb_select(const void *, const void *, const float *kbar, const float *amax, int32_t *,
                             const FsbWork &w, const float *, const float *, int, const KParams &p, hipStream_t) {
    ++g_launches;
    if (p.C == 0) return hipSuccess;  // no cells: every forest array is empty and none is touched
    inside(kbar, "kbar"); inside(amax, "amax"); inside(w.codes, "codes"); inside(w.list1, "list1");
    inside(w.hcount, "hcount"); inside(w.mu, "mu"); inside(w.rad, "rad"); inside(w.amax, "node amax");
    inside(w.pmin, "pmin"); inside(w.leaf, "leaf");
    return hipSuccess;
}
hipError_t launch_decode_init(void *, const KParams &, const DecodeLayout &, int, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_decode_prefill(void *, int, const void *, const void *, int64_t, const Work &w, const KParams &,
                                 const DecodeLayout &, hipStream_t) { ++g_launches; work(w); return hipSuccess; }
hipError_t launch_decode_append(void *, int, int, const void *, const void *, int64_t, const KParams &,
                                const DecodeLayout &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_step(void *, const void *, const void *, const void *, void *, int32_t *, int,
                              const KParams &, const DecodeLayout &, hipStream_t) { ++g_launches; return hipSuccess; }

}  // namespace fsl

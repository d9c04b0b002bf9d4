// Drives every host-side path of the C ABI (api.cpp) over a grid of valid and
// invalid parameter blocks and pointers, with the kernel launchers replaced by
// recording stand-ins (launch_stubs.hip). Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code; any report or failed check
// ends the process with a non-zero status.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fsl.h"

namespace fsl {
extern int g_launches;
extern const char *g_ws_lo, *g_ws_hi;
}

static int failures = 0;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

static float g_param_arrays[3];
static void *fake(uintptr_t a) { return (void *)a; }  // never dereferenced: launches are stubs

static fsl_params base() {
    fsl_params p{};
    p.N = 4096; p.H = 2; p.d = 64; p.w = 512; p.s = 32; p.P = 64; p.W = 8; p.K = 4; p.B = 128;
    p.dtype = FSL_BF16; p.out_dtype = FSL_BF16; p.scale = 0.0f; p.rho = 1.0f; p.rope_base = 10000.0f; p.rms_eps = 1e-6f;
    p.sigma = p.lambda = p.gamma = g_param_arrays;
    return p;
}

// one forward-side round for a parameter block: sizes, views, every entry point
static void forward_paths(const fsl_params &p) {
    const int rc = fsl_check_params(&p);
    const size_t n = fsl_workspace_bytes(&p);
    fsl_workspace_layout L{};
    CHECK(fsl_workspace_views(&p, &L) == rc);
    if (rc != FSL_OK) {
        CHECK(n == 0);
        const int before = fsl::g_launches;
        void *a = fake(0x100000);
        CHECK(fsl_cell_stats(a, (float *)a, (float *)a, &p, nullptr) == rc);
        CHECK(fsl_prune_select(a, (float *)a, (float *)a, (int32_t *)a, (int32_t *)a, &p, a, (size_t)1 << 40, nullptr) == rc);
        CHECK(fsl_attn_fwd(a, a, a, a, &p, a, (size_t)1 << 40, nullptr, nullptr, nullptr, nullptr) == rc);
        CHECK(fsl_attn_bwd_workspace_bytes(&p) == 0);
        CHECK(fsl_attn_bwd(a, a, a, a, &p, a, (size_t)1 << 40, a, (size_t)1 << 40, (float *)a, (float *)a,
                           (float *)a, (float *)a, nullptr) == rc);
        CHECK(fsl::g_launches == before);  // nothing launched on a rejected call
        return;
    }
    CHECK(n == L.total && n > 0);
    const size_t offs[] = {L.kbar, L.amax, L.pool, L.sel, L.rope, L.scan_a, L.scan_i, L.o_win, L.rope_abs, L.kt, L.vt,
                           L.fixups, L.khi, L.klo, L.kcf, L.status};
    for (size_t i = 0; i + 1 < sizeof(offs) / sizeof(offs[0]); ++i) CHECK(offs[i] <= offs[i + 1]);
    CHECK(L.status + 4 <= L.total);
    for (size_t o : offs) CHECK(o % 256 == 0);
    // a fake workspace address range the stand-ins check every array against
    const uintptr_t ws = (uintptr_t)1 << 44;
    fsl::g_ws_lo = (const char *)ws;
    fsl::g_ws_hi = (const char *)(ws + n);
    void *q = fake(0x200000);
    // the bf16 long branch without pruning lists (query, rank) pairs with 32-bit indices
    const bool big = (int64_t)p.H * p.N * p.K >= (int64_t(1) << 31);
    const int fwd_rc = p.dtype == FSL_BF16 && p.P < 0 && big ? FSL_E_UNSUPPORTED : FSL_OK;
    int before = fsl::g_launches;
    CHECK(fsl_attn_fwd(q, q, q, q, &p, fake(ws), n, nullptr, nullptr, nullptr, nullptr) == fwd_rc);
    CHECK(fwd_rc != FSL_OK || fsl::g_launches > before);
    CHECK(fsl_attn_fwd(q, q, q, q, &p, fake(ws), n - 1, nullptr, nullptr, nullptr, nullptr) == FSL_E_WORKSPACE);
    CHECK(fsl_attn_fwd(q, q, q, fake(0x200008), &p, fake(ws), n, nullptr, nullptr, nullptr, nullptr) == FSL_E_INVAL);
    CHECK(fsl_attn_fwd(q, nullptr, q, q, &p, fake(ws), n, nullptr, nullptr, nullptr, nullptr) == FSL_E_INVAL);
    before = fsl::g_launches;
    CHECK(fsl_prune_select(q, (float *)fake(ws), (float *)fake(ws), p.P < 0 ? nullptr : (int32_t *)q, (int32_t *)q, &p,
                           fake(ws), n, nullptr) == FSL_OK);
    CHECK(fsl::g_launches > before);
    CHECK(fsl_prune_select(q, (float *)q, (float *)q, (int32_t *)q, (int32_t *)q, &p, fake(ws), n - 1, nullptr) ==
          FSL_E_WORKSPACE);
    fsl::g_ws_lo = fsl::g_ws_hi = nullptr;
    // FS-B: its workspace (the unpruned forward's arrays, then the forests) checked by the stand-ins
    {
        const size_t nf = fsl_fsb_workspace_bytes(&p);
        CHECK(nf > 0);
        fsl_fsb_params fb{16, 0, g_param_arrays, g_param_arrays};
        const uintptr_t fws = (uintptr_t)1 << 46;
        fsl::g_ws_lo = (const char *)fws;
        fsl::g_ws_hi = (const char *)(fws + nf);
        int32_t *sel = (int32_t *)fake(0x500000);
        CHECK(fsl_fsb_select(q, q, &p, &fb, sel, fake(fws), nf, nullptr) == (p.rho >= 0 ? FSL_OK : FSL_E_UNSUPPORTED));
        CHECK(fsl_attn_fwd_fsb(q, q, q, q, &p, &fb, fake(fws), nf, nullptr, nullptr) ==
              (p.dtype == FSL_BF16 && big ? FSL_E_UNSUPPORTED : FSL_OK));
        CHECK(fsl_attn_fwd_fsb(q, q, q, q, &p, &fb, fake(fws), nf - 1, nullptr, nullptr) == FSL_E_WORKSPACE);
        fb.beam = 33;
        CHECK(fsl_attn_fwd_fsb(q, q, q, q, &p, &fb, fake(fws), nf, nullptr, nullptr) == FSL_E_UNSUPPORTED);
        fb.beam = 16;
        fb.tau = nullptr;
        CHECK(fsl_attn_fwd_fsb(q, q, q, q, &p, &fb, fake(fws), nf, nullptr, nullptr) == FSL_E_INVAL);
        CHECK(fsl_attn_fwd_fsb(q, q, q, q, &p, nullptr, fake(fws), nf, nullptr, nullptr) == FSL_E_INVAL);
        fsl::g_ws_lo = fsl::g_ws_hi = nullptr;
    }
    CHECK(fsl_cell_stats(q, (float *)q, (float *)q, &p, nullptr) == FSL_OK);
    CHECK(fsl_cell_stats(q, nullptr, (float *)q, &p, nullptr) == FSL_E_INVAL);
    CHECK(fsl_attn_fwd_timed(q, q, q, q, &p, fake(ws), n, nullptr, nullptr) == FSL_E_INVAL);
    // the backward: its own workspace checked by the stand-in, the forward's only by size;
    // unsupported once the H N K (query, rank) pairs exceed 32-bit indices
    const size_t nb = fsl_attn_bwd_workspace_bytes(&p);
    if ((int64_t)p.H * p.N * p.K >= (int64_t(1) << 31)) {
        CHECK(nb == 0);
        CHECK(fsl_attn_bwd(q, q, q, q, &p, fake(ws), n, fake(0x400000), (size_t)1 << 40, (float *)q, (float *)q,
                           (float *)q, (float *)q, nullptr) == FSL_E_UNSUPPORTED);
        return;
    }
    CHECK(nb > 0);
    const uintptr_t bws = (uintptr_t)1 << 45;
    fsl::g_ws_lo = (const char *)bws;
    fsl::g_ws_hi = (const char *)(bws + nb);
    float *g = (float *)fake(0x400000);
    before = fsl::g_launches;
    CHECK(fsl_attn_bwd(q, q, q, q, &p, fake(ws), n, fake(bws), nb, g, g, g, g, nullptr) == FSL_OK);
    CHECK(fsl::g_launches == before + 1);
    CHECK(fsl_attn_bwd(q, q, q, q, &p, fake(ws), n - 1, fake(bws), nb, g, g, g, g, nullptr) == FSL_E_WORKSPACE);
    CHECK(fsl_attn_bwd(q, q, q, q, &p, fake(ws), n, fake(bws), nb - 1, g, g, g, g, nullptr) == FSL_E_WORKSPACE);
    CHECK(fsl_attn_bwd(q, q, q, q, &p, fake(ws), n, fake(bws), nb, g, nullptr, g, g, nullptr) == FSL_E_INVAL);
    fsl::g_ws_lo = fsl::g_ws_hi = nullptr;
}

static void decode_paths(const fsl_params &p, int32_t n_seq) {
    const size_t sb = fsl_decode_state_bytes(&p, n_seq);
    void *st = fake(0x300000);
    void *q = fake(0x200000);
    if (sb == 0) {
        CHECK(fsl_decode_init(st, (size_t)1 << 40, n_seq, &p, nullptr) != FSL_OK);
        CHECK(fsl_decode_step(st, (size_t)1 << 40, q, q, q, q, n_seq, &p, nullptr, nullptr) != FSL_OK);
        return;
    }
    CHECK(fsl_decode_init(st, sb, n_seq, &p, nullptr) == FSL_OK);
    CHECK(fsl_decode_init(st, sb - 1, n_seq, &p, nullptr) == FSL_E_WORKSPACE);
    CHECK(fsl_decode_step(st, sb, q, q, q, q, n_seq, &p, nullptr, nullptr) == FSL_OK);
    CHECK(fsl_decode_step(st, sb, q, q, q, q, n_seq + 1, &p, nullptr, nullptr) == FSL_E_WORKSPACE);
    CHECK(fsl_decode_append(st, sb, 0, n_seq, q, q, 1000, &p, nullptr) == FSL_OK);
    CHECK(fsl_decode_append(st, sb, n_seq - 1, 2, q, q, 1000, &p, nullptr) == FSL_E_INVAL);
    for (int64_t L : {int64_t(1), int64_t(31), int64_t(4097), int64_t(1) << 20}) {
        const size_t wb = fsl_decode_prefill_workspace_bytes(&p, L);
        CHECK(wb > 0);
        const uintptr_t ws = (uintptr_t)1 << 44;
        fsl::g_ws_lo = (const char *)ws;
        fsl::g_ws_hi = (const char *)(ws + wb);
        CHECK(fsl_decode_prefill(st, sb, 0, q, q, L, &p, fake(ws), wb, nullptr) == FSL_OK);
        CHECK(fsl_decode_prefill(st, sb, 0, q, q, L, &p, fake(ws), wb - 1, nullptr) == FSL_E_WORKSPACE);
        fsl::g_ws_lo = fsl::g_ws_hi = nullptr;
    }
    CHECK(fsl_decode_prefill(st, sb, n_seq, q, q, 100, &p, q, (size_t)1 << 40, nullptr) == FSL_E_INVAL);
}

int main() {
    int rounds = 0;
    // every combination of a few values per field, valid and invalid
    const int64_t Ns[] = {1, 2, 31, 511, 512, 4096, 5001, 262144, (int64_t(1) << 31) - 1, int64_t(1) << 31, 0, -5};
    const int32_t Hs[] = {1, 3, 64, 0};
    const int32_t ds[] = {64, 128, 96, 0};
    const int32_t ss[] = {16, 32, 64, 8, 0};
    const int32_t Ps[] = {-1, 0, 64, 65, -2};
    const int32_t Ks[] = {1, 4, 8, 9};
    const int32_t Bs[] = {128, 256, 64, 288};
    for (int64_t N : Ns)
        for (int32_t H : Hs)
            for (int32_t d : ds)
                for (int32_t s : ss)
                    for (int32_t P : Ps)
                        for (int32_t K : Ks)
                            for (int32_t B : Bs)
                                for (int dt = 0; dt < 2; ++dt) {
                                    fsl_params p = base();
                                    p.N = N; p.H = H; p.d = d; p.s = s; p.P = P; p.K = K; p.B = B;
                                    p.dtype = p.out_dtype = dt;
                                    forward_paths(p);
                                    ++rounds;
                                }
    for (int32_t w : {1, 64, 512, 65536, 65537}) {
        for (int32_t P : {0, 8, 64, -1})
            for (int32_t n_seq : {1, 64, 0}) {
                fsl_params p = base();
                p.w = w; p.P = P;
                decode_paths(p, n_seq);
                ++rounds;
            }
    }
    // null and broken parameter blocks
    CHECK(fsl_check_params(nullptr) == FSL_E_INVAL);
    CHECK(fsl_workspace_bytes(nullptr) == 0);
    fsl_params p = base();
    p.sigma = nullptr;
    CHECK(fsl_check_params(&p) == FSL_E_INVAL);
    p = base();
    p.scale = 1.0f / 0.0f;
    CHECK(fsl_check_params(&p) == FSL_E_INVAL);
    for (int code = -7; code <= 1; ++code) CHECK(fsl_strerror(code) != nullptr);
    std::printf("host ABI driver: %d parameter rounds, %d stub launches, %d failed checks\n", rounds, fsl::g_launches,
                failures);
    return failures == 0 ? 0 : 1;
}

// Internal declarations shared by the FS-L HIP kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fsl.h"

namespace fsl {

// Everything a kernel needs to know about the problem, passed by value.
struct KParams {
    int64_t N;        // tokens
    int64_t C;        // complete cells, floor(N / s)
    int64_t nblk;     // query blocks, ceil(N / B)
    int32_t H, d, w, s, P, W, K, B;
    int32_t PW;       // pool capacity P + W
    int32_t dtype, out_dtype;
    float scale, rho, rope_base, rms_eps;
    const float *sigma, *lambda, *gamma;  // device [H]
    int32_t nchunk;   // prune scan: chunks of 64 cells, ceil(C / 64)
    int32_t nsg;      // prune scan: groups of 16 chunks, nchunk / 16 + 1
    int32_t rope_lo;  // first relative offset of the RoPE table (negative)
    int32_t rope_n;   // rows of the RoPE table
};

// Device workspace carved by the host (see fsl_workspace_views).
struct Work {
    float *kbar;       // [H][C][d]
    float *amax;       // [H][C]
    int32_t *pool;     // [H][nblk][PW]
    int32_t *sel;      // [H][N][K]
    float2 *rope;      // [rope_n][d/2] (cos, sin)
    float *scan_a;     // prune scan lists, (a, index) pairs of 64 entries:
    int32_t *scan_i;   //   chunks [H][nchunk], local prefixes [H][nchunk+1],
                       //   group totals [H][nsg], group prefixes [H][nsg]
    float *o_win;      // [H][N][d] window-branch output (fp32 inputs)
    // bf16 inputs only (null otherwise): what kv_prep writes
    float2 *rope_abs;  // absolute-position (cos, sin): ceil(N/64) rows of 64a, then 64 rows of b
    uint16_t *kt;      // fp16 [H][Np][d] rotated keys, Np = 64 ceil(N/64)
    uint16_t *vt;      // fp16 [H][Np/32][d][32] values, transposed per 32-token group (vt_pos order)
    uint32_t *plan;    // long branch: per (head, span) plan records (kPlanRecBytes each), or without
                       // pruning the per-cell counters and pair lists (ro_* layout)
    uint16_t *part;    // fp16 [H][N][K][d] long-branch output of each selected cell, normalised
    float *plse;       // [H][N][K] lambda = m + log2(l) of each selected cell (base-2 log-sum-exp)
    // queries whose certified filter left more than K contenders (bf16 scoring):
    // one region of kFixRegion entries per scoring work-group (fix_region), and
    // the number of entries each region holds at fix[0 .. fix_regions)
    uint32_t *fix;
    // bf16 scoring without pruning (P = -1) only: the bf16 head and tail of every
    // kbar_c, [H][C][d] each, and the per-cell constants of the error bound [H][C]
    uint16_t *khi, *klo;
    float4 *kcf;
    uint32_t *status;  // input check word (FSL_STATUS_* bits), cleared by each forward's first kernel
};

constexpr int kFixRegion = 128;  // entries per region (queries per scoring work-group)
constexpr int kFixWords = 6;     // head, row, then the contender masks of lane groups 0..3
// scoring work-groups: (head, up to 128 queries of one block)
__host__ __device__ inline int64_t fix_regions(const KParams &p) {
    const int qw = p.B <= kFixRegion ? p.B : p.B / 2;
    return (int64_t)p.H * ((p.N + qw - 1) / qw);
}
__host__ __device__ inline int64_t fix_words(const KParams &p) {
    return (fix_regions(p) + 63) / 64 * 64 + fix_regions(p) * kFixRegion * kFixWords;
}
__host__ __device__ inline uint32_t *fix_region(uint32_t *fix, const KParams &p, int64_t r) {
    return fix + (fix_regions(p) + 63) / 64 * 64 + r * kFixRegion * kFixWords;
}
__host__ __device__ inline const uint32_t *fix_region(const uint32_t *fix, const KParams &p, int64_t r) {
    return fix + (fix_regions(p) + 63) / 64 * 64 + r * kFixRegion * kFixWords;
}

// Without pruning (P = -1) a near-tie entry lists its contender cells instead of a
// pool mask: head, row, the count (kFsOverflow: re-score every eligible cell), an
// unused word and up to 32 cell indices.
constexpr int kFixWordsFs = 36;
constexpr uint32_t kFsOverflow = 0xFFFFFFFFu;
__host__ __device__ inline int64_t fix_words_fs(const KParams &p) {
    return (fix_regions(p) + 63) / 64 * 64 + fix_regions(p) * kFixRegion * kFixWordsFs;
}
__host__ __device__ inline uint32_t *fix_region_fs(uint32_t *fix, const KParams &p, int64_t r) {
    return fix + (fix_regions(p) + 63) / 64 * 64 + r * kFixRegion * kFixWordsFs;
}
__host__ __device__ inline const uint32_t *fix_region_fs(const uint32_t *fix, const KParams &p, int64_t r) {
    return fix + (fix_regions(p) + 63) / 64 * 64 + r * kFixRegion * kFixWordsFs;
}

constexpr int kChunk = 64;    // cells per prune-scan chunk (one wave)
constexpr int kGroup = 16;    // chunks per prune-scan group
constexpr int kQTile = 128;   // queries per window workgroup
constexpr int kKTile = 64;    // keys per window LDS tile
constexpr int kRopeSpan = 64; // positions per row of the coarse absolute RoPE table
constexpr int kMaxK = 8;      // largest K (cells a query selects)

// bf16 long branch: queries are read out in spans of span_queries(p) (at most
// kSpanQ), at most kPlanMaxPairs (query, rank) pairs each. A span's plan record
// (readout_units.hip) is kPlanRecBytes of 32-bit words: [0] tasks, [1] units,
// [2] pairs, [3] unused; from kPlanTaskWord two words per task (cell, first unit
// << 16 | units); from kPlanUnitWord one word per unit (first pair << 16 | pairs);
// from kPlanPairWord 16-bit pairs (query in the span << 3 | rank).
constexpr int kSpanQ = 256;
constexpr int kPlanMaxPairs = 1024;
constexpr int kPlanTaskWord = 4;
constexpr int kPlanUnitWord = kPlanTaskWord + 2 * kPlanMaxPairs;
constexpr int kPlanPairWord = kPlanUnitWord + kPlanMaxPairs + kPlanMaxPairs / 16;
constexpr int kPlanRecBytes = 15 * 1024;
static_assert(4 * kPlanPairWord + 2 * kPlanMaxPairs <= kPlanRecBytes, "plan record layout");
__host__ __device__ inline int span_queries(const KParams &p) { return p.K <= kPlanMaxPairs / kSpanQ ? kSpanQ : kPlanMaxPairs / 8; }
__host__ __device__ inline int64_t plan_records(const KParams &p) {
    return (int64_t)p.H * ((p.N + span_queries(p) - 1) / span_queries(p));
}

// bf16 long branch without pruning (readout_cells.hip): the (query, rank) pairs
// of every head are listed by super-span (a run of ro_spans_per_super(p)
// consecutive spans, 65536 queries at most unless the counters would outgrow
// kRoMaxCounters) and, inside it, by cell, so that a stretch of the list reads
// the queries of one super-span while each cell is read once per super-span.
// Without the prune a super-span's queries spread over most cells, so the longer
// the super-span, the more pairs share one read of a cell's keys and values: at
// N = 262144 the readout took 4.23 ms with 8192-query super-spans and 2.53 ms with
// 65536 (the re-read query rows cost less than the re-read cells).
// The lists are built from the same spans as the plan records. The plan region
// then holds, in 32-bit words: one pair counter per (head, super-span, cell) plus
// a sentinel (scanned in place into list offsets), the scan's block totals, then
// the list itself, one (counter index, pair index) word pair per entry; the
// kernel walks the list in items of kRoItem entries.
constexpr int kRoItem = 256;
constexpr int kRoSuperQ = 65536;
constexpr int64_t kRoMaxCounters = (int64_t)1 << 22;
__host__ __device__ inline int64_t ro_spans(const KParams &p) { return (p.N + span_queries(p) - 1) / span_queries(p); }
__host__ __device__ inline int64_t ro_spans_per_super(const KParams &p) {
    const int64_t nspan = ro_spans(p);
    const int64_t hc = (int64_t)p.H * p.C > 0 ? (int64_t)p.H * p.C : 1;
    int64_t nsup = (p.N + kRoSuperQ - 1) / kRoSuperQ;
    if (nsup > kRoMaxCounters / hc) nsup = kRoMaxCounters / hc;
    if (nsup < 1) nsup = 1;
    return (nspan + nsup - 1) / nsup;
}
__host__ __device__ inline int64_t ro_supers(const KParams &p) {
    return (ro_spans(p) + ro_spans_per_super(p) - 1) / ro_spans_per_super(p);
}
__host__ __device__ inline int64_t ro_count_words(const KParams &p) { return (int64_t)p.H * ro_supers(p) * p.C + 1; }
__host__ __device__ inline int64_t ro_total_words(const KParams &p) { return (ro_count_words(p) + 1023) / 1024; }
// word offset of the list (8-byte aligned)
__host__ __device__ inline int64_t ro_list_word(const KParams &p) { return (ro_count_words(p) + ro_total_words(p) + 1) & ~(int64_t)1; }
__host__ __device__ inline int64_t ro_plan_words(const KParams &p) { return ro_list_word(p) + 2 * (int64_t)p.H * p.N * p.K; }
// the list's pair indices (head * N + query) * K + rank and counter indices are 32-bit
__host__ __device__ inline bool ro_supported(const KParams &p) {
    return (int64_t)p.H * p.N * p.K < ((int64_t)1 << 31) && ro_count_words(p) < ((int64_t)1 << 31);
}
// bytes of the plan region: span records with pruning, cell lists without
__host__ __device__ inline int64_t plan_bytes(const KParams &p) {
    return p.P < 0 ? ro_plan_words(p) * 4 : plan_records(p) * kPlanRecBytes;
}

// rows of the coarse absolute RoPE table (one per 64 positions)
__host__ __device__ inline int rope_abs_rows_hi(const KParams &p) { return (int)((p.N + kRopeSpan - 1) / kRopeSpan); }
// kt and vt are padded per head to whole 64-token tiles (zeros past token N-1)
__host__ __device__ inline int64_t kt_rows(const KParams &p) { return (int64_t)rope_abs_rows_hi(p) * kRopeSpan; }
// vt holds groups of 32 tokens: [H][Np/32][d][32], tokens permuted inside a group
__host__ __device__ inline int64_t vt_groups(const KParams &p) { return kt_rows(p) / 32; }
// elements per head of kt and of vt (the same count: Np tokens x d); the
// workspace sizes and every kernel's per-head offsets derive from these
__host__ __device__ inline int64_t kt_head_elems(const KParams &p) { return kt_rows(p) * p.d; }
__host__ __device__ inline int64_t vt_head_elems(const KParams &p) { return vt_groups(p) * 32 * p.d; }
// Position of token t (0..31) inside a vt group row. An MFMA P^T operand built
// from the accumulators of two 16-token score tiles gives lane group g (lanes
// 16g..16g+15) tokens 4g..4g+3 of the first tile and 4g..4g+3 of the second as
// its k-slots 0..7; storing them at 8g..8g+7 makes each lane's value operand
// one contiguous 16-byte piece.
__host__ __device__ inline int vt_pos(int t) { return 8 * ((t & 15) >> 2) + (t & 3) + 4 * (t >> 4); }
// LDS swizzles applied by the tile copies (16-byte pieces) and undone by the
// operand reads: key rows (d/8 chunks) and value rows (4 pieces). Both were
// measured with a bank-conflict probe on gfx950: a 16-byte operand read of
// either kind takes 4 LDS cycles per wave, the conflict-free minimum (the
// value swizzle ((dim >> 1) ^ (dim >> 3)) & 3 took 8).
__host__ __device__ inline int swz_key(int row, int d) {
    return d == 128 ? (row & 15) : ((row ^ (row >> 3)) & 7);
}
__host__ __device__ inline int swz_val(int dim) { return (dim >> 1) & 3; }

// Work-group order for L2 reuse. The dispatcher deals consecutive work-group ids
// to the eight XCDs in turn, and each XCD has its own L2; this bijection of
// [0, T) gives XCD x a contiguous range of the logical order, so neighbouring
// logical work-groups (which share key/value tiles) run under the same L2.
__device__ __forceinline__ int xcd_remap(int L, int T) {
    const int q = T >> 3, r = T & 7, x = L & 7, i = L >> 3;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Offsets of the four prune-scan list families inside scan_a / scan_i, in lists of 64.
__host__ __device__ inline int64_t scan_chunk(const KParams &p, int h, int64_t k) {
    return (int64_t)h * p.nchunk + k;
}
__host__ __device__ inline int64_t scan_prefix(const KParams &p, int h, int64_t k) {
    return (int64_t)p.H * p.nchunk + (int64_t)h * (p.nchunk + 1) + k;
}
__host__ __device__ inline int64_t scan_total(const KParams &p, int h, int64_t g) {
    return (int64_t)p.H * (2 * (int64_t)p.nchunk + 1) + (int64_t)h * p.nsg + g;
}
__host__ __device__ inline int64_t scan_gprefix(const KParams &p, int h, int64_t g) {
    return (int64_t)p.H * (2 * (int64_t)p.nchunk + 1 + p.nsg) + (int64_t)h * p.nsg + g;
}
__host__ __device__ inline int64_t scan_lists(const KParams &p) {
    return (int64_t)p.H * (2 * (int64_t)p.nchunk + 1 + 2 * (int64_t)p.nsg);
}

// Cells eligible for block b: wholly before the window of its first query.
__host__ __device__ inline int64_t eligible_cells(const KParams &p, int64_t b) {
    int64_t x = b * p.B - p.w + 1;
    if (x <= 0) return 0;
    int64_t nb = x / p.s;
    return nb < p.C ? nb : p.C;
}

// ---------------------------------------------------------------------------
// element helpers (bf16 travels as raw uint16 bit patterns)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Reductions over the four lanes l, l^16, l^32, l^48 of a wave: the lanes that
// hold one column of a 16x16 MFMA accumulator. Each step swaps register rows
// between lane halves (v_permlane16_swap / v_permlane32_swap) and combines the
// pair, so every lane of the column ends with the same value.
__device__ __forceinline__ float colmax4(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float colsum4(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i of the wave writes lds_wave + 16 i, so lds_wave must be the same for the
// whole wave; completion is counted by vmcnt like any global load.
typedef __attribute__((address_space(3))) void *lds_void_ptr;
typedef __attribute__((address_space(1))) void *global_void_ptr;
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_wave) {
    __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)lds_wave, 16, 0, 0);
}
// wait for this wave's outstanding global loads, LDS copies included
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// wait until at most N of this wave's global loads / LDS copies are outstanding
// (they complete in issue order, so everything older than the last N is done)
template <int N>
__device__ __forceinline__ void wait_vmem_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// 16-byte LDS reads issued as one inline-asm block that also waits for them:
// for ring buffers whose refills and reads are ordered explicitly (vmcnt wait +
// barrier), this keeps the compiler from adding its own conservative wait for
// every copy in flight. The results are complete when the block ends.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void lds_read16x2(uint4 &a, uint4 &b, const void *pa, const void *pb) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b)
                 : "v"(lds_addr(pa)), "v"(lds_addr(pb))
                 : "memory");
}
__device__ __forceinline__ void lds_read16x4(uint4 &a, uint4 &b, uint4 &c, uint4 &d, const void *pa, const void *pb,
                                             const void *pc, const void *pd) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
        : "v"(lds_addr(pa)), "v"(lds_addr(pb)), "v"(lds_addr(pc)), "v"(lds_addr(pd))
        : "memory");
}

// Work-group barrier without the memory fence of __syncthreads, whose release
// would also drain every LDS copy still in flight. The caller has already
// waited (vmcnt) for the copies the other waves are about to read; this wave's
// own LDS reads are completed here so that a copy issued after the barrier
// cannot overwrite a slot that is still being read.
__device__ __forceinline__ void barrier_no_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Sum over the aligned group of 8 lanes that holds lane l (lanes 8 (l / 8) ..
// 8 (l / 8) + 7) with three DPP moves: swap neighbours, swap pairs, mirror the
// halves of the group. Every lane of the group ends with the same sum.
__device__ __forceinline__ float sum8_dpp(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
    return x;
}

// 2^x with the hardware instruction alone (no denormal range scaling): softmax
// weights below 2^-126 of the running maximum are flushed to zero.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Two softmax weights as one packed fp16 pair for a P.V MFMA operand, rounded to
// nearest even (v_cvt_pk_f16_f32), with the two rounded weights added to the fp32
// running denominator (v_dot2c_f32_f16 against a pair of ones). The denominator then
// sums exactly the weights the product multiplies, so weight rounding errors are
// unbiased and do not accumulate into a one-sided output scale.
typedef _Float16 fsl_half2 __attribute__((ext_vector_type(2)));
typedef float fsl_float2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_f16_rne_acc(float a, float b, float &sum) {
    const fsl_float2 f = {a, b};
    const fsl_half2 h = __builtin_convertvector(f, fsl_half2);
    const fsl_half2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    sum = __builtin_amdgcn_fdot2(h, ones, sum, false);
    union { fsl_half2 h; uint32_t u; } c;
    c.h = h;
    return c.u;
}

// Online softmax with a lazily updated maximum: the reference value m only
// moves when a new score exceeds it by more than kStaleLog2 (base-2 units), so
// the weights 2^(s - m) stay within [0, 2^kStaleLog2] and the accumulators are
// rescaled only on such rare jumps. The normalised result is the same softmax.
constexpr float kStaleLog2 = 8.0f;

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

// ---------------------------------------------------------------------------
// wave64 primitives over one (key, index) entry per lane.
// Order "better": larger key first, then lower index. Sentinel: (-inf, INT32_MAX).

__device__ __forceinline__ bool better(float a1, int i1, float a2, int i2) {
    return a1 > a2 || (a1 == a2 && i1 < i2);
}

__device__ __forceinline__ bool better_d(double a1, int i1, double a2, int i2) {
    return a1 > a2 || (a1 == a2 && i1 < i2);
}

// Wave-wide best (better_d order) of one (key, index, tag) entry per lane, left in every lane.
// Lanes pair up as i ^ 1, i ^ 2 (quad permutes), mirrored half rows and rows, then i ^ 16 and
// i ^ 32 (lane swaps); each step keeps the better of a lane's entry and its partner's, so both
// lanes of a pair agree. The whole wave must be active.
template <int CTRL>
__device__ __forceinline__ void best_step_dpp(double &v, int &c, int &tag) {
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int oc = __builtin_amdgcn_mov_dpp(c, CTRL, 0xF, 0xF, false);
    const int ot = __builtin_amdgcn_mov_dpp(tag, CTRL, 0xF, 0xF, false);
    const double ov = __hiloint2double(hi, lo);
    const bool bt = better_d(ov, oc, v, c);
    v = bt ? ov : v;
    c = bt ? oc : c;
    tag = bt ? ot : tag;
}
// the pair (a[0], a[1]) of a lane swap holds the lane's own value and its partner's
template <bool S32>
__device__ __forceinline__ void best_step_swap(double &v, int &c, int &tag) {
    const uint32_t hi = (uint32_t)__double2hiint(v), lo = (uint32_t)__double2loint(v);
    const uint32_t uc = (uint32_t)c, ut = (uint32_t)tag;
    const auto h = S32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                       : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const auto l = S32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                       : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto cc = S32 ? __builtin_amdgcn_permlane32_swap(uc, uc, false, false)
                        : __builtin_amdgcn_permlane16_swap(uc, uc, false, false);
    const auto tt = S32 ? __builtin_amdgcn_permlane32_swap(ut, ut, false, false)
                        : __builtin_amdgcn_permlane16_swap(ut, ut, false, false);
    const double x = __hiloint2double((int)h[0], (int)l[0]), y = __hiloint2double((int)h[1], (int)l[1]);
    const bool by = better_d(y, (int)cc[1], x, (int)cc[0]);
    v = by ? y : x;
    c = by ? (int)cc[1] : (int)cc[0];
    tag = by ? (int)tt[1] : (int)tt[0];
}
__device__ __forceinline__ void wave_best_d(double &v, int &c, int &tag) {
    best_step_dpp<0xB1>(v, c, tag);   // quad_perm [1, 0, 3, 2]
    best_step_dpp<0x4E>(v, c, tag);   // quad_perm [2, 3, 0, 1]
    best_step_dpp<0x141>(v, c, tag);  // row_half_mirror
    best_step_dpp<0x140>(v, c, tag);  // row_mirror
    best_step_swap<false>(v, c, tag);
    best_step_swap<true>(v, c, tag);
}

// Sort the 64 entries of a wave best-first (lane 0 best). Bitonic network.
__device__ __forceinline__ void wave_sort_best_first(float &a, int &idx) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            float pa = __shfl_xor(a, j);
            int pi = __shfl_xor(idx, j);
            bool lower = (lane & j) == 0;
            bool dir = (lane & k) == 0;
            bool pb = better(pa, pi, a, idx);
            bool take = (lower == dir) ? pb : !pb;
            if (take) { a = pa; idx = pi; }
        }
    }
}

// Given two best-first sorted lists (one entry per lane each), leave the 64
// best of their union, best-first, in (a, idx).
__device__ __forceinline__ void wave_merge_top(float &a, int &idx, float ba, int bi) {
    const int lane = threadIdx.x & 63;
    float ra = __shfl(ba, 63 - lane);
    int ri = __shfl(bi, 63 - lane);
    if (better(ra, ri, a, idx)) { a = ra; idx = ri; }
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) {
        float pa = __shfl_xor(a, j);
        int pi = __shfl_xor(idx, j);
        bool lower = (lane & j) == 0;
        bool pb = better(pa, pi, a, idx);
        bool take = lower ? pb : !pb;
        if (take) { a = pa; idx = pi; }
    }
}

// ---------------------------------------------------------------------------
// decode state: a 256-byte header, a RoPE table for offsets [-(w-1), 0], then
// one record per (sequence, head)

constexpr uint32_t kDecodeMagic = 0x44534C46u;  // "FLSD"
constexpr uint32_t kDecodeVersion = 2;

struct DecodeHeader {
    uint32_t magic, version;
    int32_t H, d, w, s, P, W, K, B, dtype, n_seq, R, PW;
    int64_t rec_bytes;
};

struct DecodeLayout {
    int32_t R;          // ring tokens, w + B + s
    int32_t PW;         // cell slots, P + W
    int64_t off_rec;    // first record
    int64_t rec_bytes;  // bytes per (sequence, head) record
    // offsets inside a record (after int64 t and int64 block)
    int64_t o_cell, o_a, o_kbar, o_sk, o_sv, o_rk, o_rv;
    int64_t o_rkr;      // ring of keys rotated at their positions: fp16 (bf16 inputs) or fp32 [R][d]
};

// ---------------------------------------------------------------------------
// launchers (one per kernel family); each returns hipGetLastError()

hipError_t launch_cell_stats(const void *k, float *kbar, float *amax, const KParams &p, hipStream_t st);
hipError_t launch_prune(const float *amax, int32_t *pool, const Work &w, const KParams &p, hipStream_t st);
hipError_t launch_select(const void *q, const float *kbar, const float *amax, const int32_t *pool,
                         int32_t *sel, const KParams &p, hipStream_t st);
hipError_t launch_select_mfma(const void *q, const float *kbar, const float *amax, const int32_t *pool,
                              int32_t *sel, uint32_t *fix, const KParams &p, hipStream_t st);
hipError_t launch_select_fixup(const void *q, const float *kbar, const float *amax, const int32_t *pool,
                               int32_t *sel, const uint32_t *fix, const KParams &p, hipStream_t st);
hipError_t launch_select_fs(const void *q, const float *kbar, const float *amax, int32_t *sel, const Work &w,
                            const KParams &p, hipStream_t st);
hipError_t launch_rope_table(float2 *tab, uint32_t *status, const KParams &p, hipStream_t st);
hipError_t launch_window(const void *q, const void *k, const void *v, const float2 *rope, float *o_win,
                         const KParams &p, hipStream_t st);
hipError_t launch_kv_prep(const void *k, const void *v, uint16_t *kt, uint16_t *vt, float2 *rope_abs, float *kbar,
                          float *amax, uint32_t *status, const KParams &p, hipStream_t st);
// the query range [qa, qb) of every head; qa a multiple of 256
hipError_t launch_window_bf16(const void *q, const uint16_t *kt, const uint16_t *vt, const float2 *rope_abs,
                              const int32_t *sel, const uint16_t *part, const float *plse, void *out,
                              float *o_win_out, float *o_long_out, const KParams &p, int64_t qa, int64_t qb,
                              hipStream_t st);
hipError_t launch_readout_cells(const void *q, const void *k, const uint16_t *vt, const int32_t *sel,
                                uint32_t *plan, uint16_t *part, float *plse, const KParams &p, hipStream_t st);
hipError_t launch_readout_units(const void *q, const void *k, const uint16_t *vt, const int32_t *sel,
                                uint32_t *plan, uint16_t *part, float *plse, const KParams &p, int64_t qa,
                                int64_t qb, hipStream_t st);
hipError_t launch_readout_mix(const void *q, const void *k, const void *v, const int32_t *sel,
                              const float *o_win, void *out, float *o_long_out, const KParams &p,
                              hipStream_t st);

// the two-level absolute-position (cos, sin) table of kv_prep.hip (rows of 64a, then 64 rows of b);
// also clears *status
hipError_t launch_rope_abs_table(float2 *tab, uint32_t *status, const KParams &p, hipStream_t st);

// backward (backward.hip): everything after the forward's selection
struct BwdWork {
    float2 *rope;     // absolute-position table
    float *qr, *kr;   // [H][N][d] RoPE-rotated q and k, fp32
    float *dO;        // [H][N][d] upstream gradient, fp32
    float *do_l;      // [H][N][d] gradient reaching the long branch's softmax output
    float *lse_w, *D_w, *lse_l, *D_l;  // [H][N] row statistics of both branches
    float *dg;        // [H][N] per-query terms of dgamma
    uint32_t *pkey, *pval, *pkey2, *pval2;  // [H][N][K] (cell, query) pairs and the sort's second buffers
    uint32_t *shist, *stot;  // radix-sort digit counts and block totals (sort_hist_words, sort_total_words)
    int32_t *cseg;    // [H][C][2] each cell's run of the pairs sorted by cell
    int32_t *hcount;  // [2] chunks and cells of the heavy-cell work lists
    int32_t *hitems;  // [heavy_items_max][2] (cell, chunk)
    int32_t *hcells;  // [heavy_cells_max][3] (cell, first item, chunks)
    float *hpart;     // [heavy_items_max][2][s][d] each chunk's dk and dv sums
    float *dqp;       // [H][N][K][d] per (query, rank) pair: the long branch's weighted values
                      // of the cell, then its dq (scaled)
    float2 *pml;      // [H][N][K] per pair: the largest scaled score over the cell and the sum of weights
    uint32_t *status;
};
// cells chosen by more than kHeavyPairs queries are processed in chunks of that many
constexpr int kHeavyPairs = 2048;
__host__ __device__ inline int64_t heavy_cells_max(const KParams &p) {
    return (int64_t)p.H * p.N * p.K / (kHeavyPairs + 1);
}
__host__ __device__ inline int64_t heavy_items_max(const KParams &p) {
    // ceil(cnt / kHeavyPairs) < cnt / kHeavyPairs + 1 per heavy cell
    return (int64_t)p.H * p.N * p.K / kHeavyPairs + heavy_cells_max(p);
}
// the stable radix sort (sort.hip): 8-bit digits; chunk histograms stored digit-major
// and scanned in blocks of kSortScanBlock, whose totals one work-group scans
constexpr int kSortRadix = 256;
constexpr int kSortScanBlock = 1024;
constexpr int kSortScanTopMax = 8192;
static_assert(kSortScanBlock == 1024, "ro_total_words counts 1024-word scan blocks");
// chunk length (elements) and chunk count for n pairs
inline void sort_plan(int64_t n, int &chunk, int &nch) {
    const int64_t max_chunks = (int64_t)kSortScanTopMax * kSortScanBlock / kSortRadix;
    int64_t c = 1024;
    while ((n + c - 1) / c > max_chunks) c *= 2;
    chunk = (int)c;
    nch = (int)((n + c - 1) / c);
    if (nch < 1) nch = 1;
}
inline size_t sort_hist_words(int64_t n) {
    int chunk, nch;
    sort_plan(n, chunk, nch);
    return (size_t)kSortRadix * nch;
}
inline size_t sort_total_words(int64_t n) { return (sort_hist_words(n) + kSortScanBlock - 1) / kSortScanBlock; }
hipError_t launch_sort_pairs(uint32_t *keys, uint32_t *vals, uint32_t *ktmp, uint32_t *vtmp, uint32_t *hist,
                             uint32_t *totals, int64_t n, int bits, bool *in_tmp, hipStream_t st);
// exclusive scan of m words in place in blocks of kSortScanBlock; prefix of i =
// data[i] + totals[i / kSortScanBlock]
hipError_t launch_scan_u32(uint32_t *data, int64_t m, uint32_t *totals, hipStream_t st);
// bits of the backward's pair keys, head * C + cell with the sentinel H * C
__host__ __device__ inline int pair_key_bits(const KParams &p) {
    int b = 1;
    while (b < 32 && ((int64_t)1 << b) <= (int64_t)p.H * p.C) ++b;
    return b;
}
hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const void *dout, const int32_t *sel,
                           const int32_t *pool, const BwdWork &w, float *dq, float *dk, float *dv,
                           float *dgamma, const KParams &p, hipStream_t st);

// FS-B (fsb.hip): cell codes, the high-norm list, and every segment tree's nodes
struct FsbWork {
    uint32_t *codes;   // [H][C] sign hash of each mean key
    int32_t *list1;    // [H][C] cells with a_c > tau, ascending
    int32_t *hcount;   // [H][C+1] number of list-1 cells below each cell
    float *mu;         // [node][d] node mean keys
    double *rad;       // [node] radii
    float *amax;       // [node] largest cell norm beneath
    int32_t *pmin;     // [node] earliest position beneath
    int32_t *leaf;     // leaf cells of every segment tree
};
// levels of the forests: kmax + 1, kmax = floor(log2 C)
__host__ __device__ inline int fsb_levels(const KParams &p) {
    int k = 0;
    while (((int64_t)1 << (k + 1)) <= p.C) ++k;
    return k + 1;
}

// node slots per (head, forest, level): 2 C, enough for (C >> k) trees of 2^(k+1) slots
__host__ __device__ inline int64_t fsb_node(const KParams &p, int h, int T, int k, int64_t a, int64_t j) {
    const int lv = fsb_levels(p);
    return ((((int64_t)h * 2 + T) * lv + k) * 2 * p.C) + (a << (k + 1)) + j;
}
// leaf slots per (head, forest, level): C
__host__ __device__ inline int64_t fsb_leaf(const KParams &p, int h, int T, int k, int64_t a, int64_t u) {
    const int lv = fsb_levels(p);
    return ((((int64_t)h * 2 + T) * lv + k) * p.C) + (a << k) + u;
}

hipError_t launch_fsb_select(const void *q, const void *k, const float *kbar, const float *amax, int32_t *sel,
                             const FsbWork &w, const float *tau, const float *proj, int beam, const KParams &p,
                             hipStream_t st);

hipError_t launch_decode_init(void *state, const KParams &p, const DecodeLayout &L, int n_seq, hipStream_t st);
hipError_t launch_decode_prefill(void *state, int seq, const void *kp, const void *vp, int64_t Lp, const Work &w,
                                 const KParams &p, const DecodeLayout &L, hipStream_t st);
hipError_t launch_decode_append(void *state, int seq0, int n, const void *k, const void *v, int64_t len,
                                const KParams &p, const DecodeLayout &L, hipStream_t st);
hipError_t launch_decode_step(void *state, const void *q, const void *k, const void *v, void *out, int32_t *sel_out,
                              int n_seq, const KParams &p, const DecodeLayout &L, hipStream_t st);

}  // namespace fsl

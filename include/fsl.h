/*
 * fsl.h: C ABI of the FS-L (FreeSolo-Linear) attention library for MI355X.
 *
 * FS-L is the linear-time variant of FreeSolo, a two-branch sparse attention
 * ("FreeSolo: Linear-time Sparse Attention with Zero-Shot Length
 * Extrapolation"; digest at paper.rainbus.top, sections "核心方法" (core
 * method) and "方法步骤详情" (method steps); ai.info summary, "Methodology in
 * Plain English"). Per head and per block of B queries:
 *   1. a RoPE sliding-window branch over the last w keys;
 *   2. the prefix split into cells of s tokens, each summarised by its mean
 *      key kbar_c and its largest token-key norm a_c;
 *   3. a norm prune to the P cells of largest a_c plus the W most recent
 *      cells, a cell score (content q.kbar_c plus an a_c-weighted erf
 *      relative-position bias) and the top K cells per query;
 *   4. an unrotated (NoPE) softmax readout over the K*s raw tokens of those
 *      cells, RMSNorm, and a per-head weighted add to the window branch.
 *
 * Conventions of every entry point:
 *  - Ownership: the caller owns every buffer (inputs, outputs, workspace,
 *    decode state). The library allocates nothing on the device and keeps no
 *    global state, so calls on different streams do not interact.
 *  - Execution: work is enqueued on `stream` and returns without waiting;
 *    results are ready when the stream reaches that point. Entry points do
 *    not synchronise (fsl_decode_validate is the one exception, see there).
 *  - Pointers named "device" must be device memory (hipMalloc or a torch
 *    tensor on the GPU), 16-byte aligned, non-overlapping. Host pointers are
 *    read before the call returns.
 *  - Errors: every int-returning call returns FSL_OK (0) or a negative code.
 *    Arguments are validated on the host before anything is launched, so an
 *    error means nothing was enqueued. FSL_E_HIP reports a launch failure.
 *  - Layouts: q, k, v, out are contiguous [H][N][d] (one sequence, head-major).
 *    Element type is fp32 or bf16 (uint16 bit patterns) per fsl_params.dtype.
 */
#ifndef FSL_H
#define FSL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSL_VERSION 1

enum fsl_status {
    FSL_OK = 0,
    FSL_E_INVAL = -1,        /* bad size, parameter, null or misaligned pointer */
    FSL_E_UNSUPPORTED = -2,  /* valid for the method, not implemented here (d, P, ...) */
    FSL_E_WORKSPACE = -3,    /* workspace or state buffer too small */
    FSL_E_STATE = -4,        /* decode state header does not match the parameters */
    FSL_E_HIP = -5           /* a kernel launch failed */
};

enum fsl_dtype { FSL_F32 = 0, FSL_BF16 = 1 };

/* Method parameters. Page defaults: w=512, s=32, P=64, W=8, K=4, B=128,
 * sigma_h=4, lambda_h=1 (digest, core method; ai.info summary, methodology
 * and training paragraph). Limits of this implementation: d in {64, 128};
 * s in {16, 32, 64} with s dividing B; B a multiple of 16, at most 256;
 * -1 <= P <= 64; 0 <= W <= 64; 1 <= K <= 8; w >= 1; H >= 1; 1 <= N < 2^31.
 * P = -1 selects the plain FS variant (digest, core method: FS-L is FS with the
 * norm prune added): every query of block b scores all n_b eligible cells, no
 * pool is formed and W is unused. The streaming decode needs P >= 0 (its
 * bounded state holds P + W pool cells) and returns FSL_E_UNSUPPORTED for
 * P = -1. */
typedef struct fsl_params {
    int64_t N;          /* tokens in the sequence (forward); ignored by decode */
    int32_t H;          /* heads */
    int32_t d;          /* head dimension */
    int32_t w;          /* window width: query i sees keys [i-w+1, i] */
    int32_t s;          /* cell size in tokens */
    int32_t P;          /* high-norm cells kept per block */
    int32_t W;          /* most recent eligible cells kept per block */
    int32_t K;          /* cells read per query */
    int32_t B;          /* query block size: the pool is shared by a block */
    int32_t dtype;      /* fsl_dtype of q, k, v */
    int32_t out_dtype;  /* fsl_dtype of out (the input dtype, or FSL_F32) */
    float scale;        /* softmax scale of both branches; 0 selects 1/sqrt(d) */
    float rho;          /* weight of the content term q.kbar_c in the cell score */
    float rope_base;    /* RoPE base (10000) */
    float rms_eps;      /* RMSNorm epsilon (1e-6) */
    const float *sigma; /* device [H]: erf width sigma_h of the position bias */
    const float *lambda;/* device [H]: weight lambda_h of the norm-weighted bias */
    const float *gamma; /* device [H]: mixing coefficient gamma_h of the long branch */
} fsl_params;

/* Library version (FSL_VERSION) and a static message for a status code. */
int fsl_version(void);
const char *fsl_strerror(int status);

/* Host-only check of a parameter block (no pointer is dereferenced).
 * Returns FSL_OK, FSL_E_INVAL or FSL_E_UNSUPPORTED. */
int fsl_check_params(const fsl_params *p);

/* Bytes of device workspace fsl_prune_select and fsl_attn_fwd need for p
 * (0 if p is invalid). The workspace holds the cell statistics, the per-block
 * pools, the per-query selections, the RoPE table and the prune scan lists. */
size_t fsl_workspace_bytes(const fsl_params *p);

/* Cell statistics (digest, core method and step 3; ai.info summary,
 * methodology: mean key for routing, largest token-key norm as a
 * query-independent priority). For every complete cell c < C = floor(N/s):
 *   kbar[h][c][x] = float(sum_j k[h][c*s+j][x] / s)     (fp64 sum in token order)
 *   amax[h][c]    = float(sqrt(max_j sum_x k[h][c*s+j][x]^2))
 * with the squared norm a left-to-right fp64 fused multiply-add chain.
 * k: device [H][N][d] (dtype); kbar: device [H][C][d] float; amax: device [H][C] float. */
int fsl_cell_stats(const void *k, float *kbar, float *amax, const fsl_params *p,
                   hipStream_t stream);

/* Norm prune and per-query top-K (digest, core method and steps 4-5; ai.info
 * summary, methodology: pool of the W most recent eligible cells plus the P
 * highest-norm older ones, updated once per query block).
 * Block b (queries [bB, bB+B)) may use the n_b = max(0, floor((bB - w + 1)/s))
 * cells that lie wholly before the window of its first query. Its pool is the
 * W most recent of them plus the P best of the rest under (a desc, index asc).
 * Each query i scores every pool cell in fp64:
 *   score = fma(rho, q_i.kbar_c, (lambda_h * a_c) * erf(sigma_h (i - c s) / (2 s)))
 * (dot product a left-to-right fma chain over x, inputs the float32 cell
 * statistics) and keeps the K best under (score desc, index asc).
 * q: device [H][N][d] (dtype); kbar/amax as produced by fsl_cell_stats;
 * pool: device [H][ceil(N/B)][P+W] int32, ascending, padded with -1 (with
 * P = -1 the pool is every eligible cell and is not written: pool may be NULL);
 * sel: device [H][N][K] int32, ascending, padded with -1.
 * ws: device workspace of at least fsl_workspace_bytes(p) bytes. */
int fsl_prune_select(const void *q, const float *kbar, const float *amax, int32_t *pool,
                     int32_t *sel, const fsl_params *p, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* Whole FS-L forward (digest, core method and step 6: NoPE softmax over the
 * selected tokens, RMSNorm, add to the RoPE window branch with a per-head
 * weight):
 *   o_win[i]  = softmax_j(scale R(i)q_i . R(j)k_j) v_j over j in [max(0,i-w+1), i]
 *               (rotate-half RoPE, angle t * rope_base^(-2m/d))
 *   o_long[i] = softmax_j(scale q_i . k_j) v_j over the tokens of sel[i] (0 if empty)
 *   out[i]    = o_win[i] + gamma_h * o_long[i] / sqrt(mean_x(o_long[i]^2) + rms_eps)
 * q, k, v: device [H][N][d] (dtype); out: device [H][N][d] (out_dtype).
 * ws: device workspace of at least fsl_workspace_bytes(p) bytes; after the
 * call it holds kbar, amax, pool and sel (see fsl_workspace_views).
 * With bf16 inputs both attention branches multiply fp16 operands (keys
 * rotated, values and softmax weights) with fp32 accumulation, so k and v
 * must lie inside fp16's range (|x| < 65504, a precondition); a call that
 * breaks it sets FSL_STATUS_F16_RANGE in the workspace's status word. The
 * selection path does not depend on this.
 * sel_out (device [H][N][K] int32), o_win_out and o_long_out (device
 * [H][N][d] float) are optional copies for inspection; pass NULL to skip. */
int fsl_attn_fwd(const void *q, const void *k, const void *v, void *out, const fsl_params *p,
                 void *ws, size_t ws_bytes, int32_t *sel_out, float *o_win_out,
                 float *o_long_out, hipStream_t stream);

/* fsl_attn_fwd with stage timing. stage_events must point to
 * FSL_NUM_STAGES + 1 caller-created hipEvent_t handles; events[0] is recorded
 * on `stream` before the first kernel and events[s + 1] after stage s, the
 * stages being, in order: cell statistics (bf16: fused with the RoPE table and
 * the key/value preparation, one pass over k and v), norm prune (4 kernels;
 * empty with P = -1), scoring and top-K, RoPE table (fp32; empty for bf16),
 * window attention, readout + mix. Elapsed time between
 * consecutive events is the duration of that stage's kernels. Same arguments,
 * results and errors as fsl_attn_fwd otherwise (FSL_E_INVAL if stage_events
 * is NULL). */
#define FSL_NUM_STAGES 6
int fsl_attn_fwd_timed(const void *q, const void *k, const void *v, void *out, const fsl_params *p,
                       void *ws, size_t ws_bytes, hipEvent_t *stage_events, hipStream_t stream);

/* Backward of the forward, for training (digest, method steps: the hard
 * top-P / top-K indices receive no gradient; ai.info summary, training
 * paragraph: sigma_h and lambda_h stay fixed, the mixing weight gamma_h is
 * learned). With the forward's selections held fixed, out is differentiable
 * in q, k, v and gamma; given dout = dL/dout this computes
 *   dq, dk, dv: device [H][N][d] float (written, not accumulated),
 *   dgamma:     device [H] float,
 * through both attention branches (window: RoPE'd softmax backward, gradients
 * turned back through R(t)^T; long branch: RMSNorm's backward, then the softmax
 * backward over the selected cells' tokens). q, k, v: the forward's inputs;
 * dout: device [H][N][d] in out_dtype. fwd_ws: the workspace of a completed
 * fsl_attn_fwd call on the same q, k, v and p (its selections and pools are
 * read, nothing is written). ws: device workspace of at
 * least fsl_attn_bwd_workspace_bytes(p) bytes. Arithmetic is fp32; the sums
 * run in a fixed order (no atomics), so results are reproducible. Errors as
 * fsl_attn_fwd (FSL_E_WORKSPACE if either workspace is too small). */
size_t fsl_attn_bwd_workspace_bytes(const fsl_params *p);
int fsl_attn_bwd(const void *q, const void *k, const void *v, const void *dout, const fsl_params *p,
                 const void *fwd_ws, size_t fwd_ws_bytes, void *ws, size_t ws_bytes, float *dq, float *dk,
                 float *dv, float *dgamma, hipStream_t stream);

/* FS-B: selection by beam search over two causal forests instead of the norm
 * prune (ai.info summary, "Methodology in Plain English", FS-B paragraph; digest,
 * method step 5 and novelty: O(N log^2 N) including the radix-sort construction).
 * Per head, list 0 holds every complete cell and list 1 the cells with
 * a_c > tau_h, both in position order. Every aligned segment [a 2^k, (a+1) 2^k)
 * of a list holds a balanced binary tree whose leaves are its cells ordered by
 * (code asc, list index asc), code the 32-bit sign hash of kbar_c over the 32
 * rows of proj (bit 31-b set iff proj_b . kbar_c > 0). Nodes keep the mean key
 * mu (fp32 rounding of the fp64 mean of their leaves), a radius r bounding
 * their children's balls, the largest a_c and the earliest position pmin
 * beneath. Block b's queries search, in each forest, the segments of the binary
 * decomposition of the list entries eligible for block b (as in fsl_prune_select),
 * keeping `beam` nodes under the bound (rho, lambda_h, sigma_h >= 0)
 *   ub = fma(rho, fma(|q|, r, q . mu), (lambda_h amax) erf(sigma_h (i - pmin) / (2 s))),
 * ties by (forest, level, segment, heap index); the union of the two beams'
 * cells is reranked by lse_c = log sum_j exp(scale q . k_j) over each cell's raw
 * tokens and the K best (ties to the lower index) are read, ascending and
 * padded with -1. p->P is ignored. */
typedef struct fsl_fsb_params {
    int32_t beam;       /* nodes kept per level in each forest (16); 1 .. 32 */
    int32_t reserved;   /* 0 */
    const float *tau;   /* device [H]: list 1 holds the cells with a_c > tau_h */
    const float *proj;  /* device [32][d]: projection rows of the cell codes */
} fsl_fsb_params;

/* Workspace bytes of fsl_fsb_select and fsl_attn_fwd_fsb (0 if invalid). */
size_t fsl_fsb_workspace_bytes(const fsl_params *p);

/* FS-B selections only: sel device [H][N][K] int32 (ascending, padded -1); the
 * cell statistics are computed into the workspace. q, k: device [H][N][d]. */
int fsl_fsb_select(const void *q, const void *k, const fsl_params *p, const fsl_fsb_params *fb, int32_t *sel,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/* The whole forward with FS-B selections (window branch, readout over the
 * selected cells, RMSNorm, mix as fsl_attn_fwd). sel_out (nullable) receives the
 * selections. FSL_E_UNSUPPORTED for rho < 0 or beam outside 1 .. 32; lambda_h,
 * sigma_h >= 0 is the caller's precondition (the bound assumes it). */
int fsl_attn_fwd_fsb(const void *q, const void *k, const void *v, void *out, const fsl_params *p,
                     const fsl_fsb_params *fb, void *ws, size_t ws_bytes, int32_t *sel_out, hipStream_t stream);

/* fsl_attn_fwd for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, hosts that forbid allocation calls):
 * the same arguments and results without ws / ws_bytes. The workspace is a
 * device array of FSL_NOALLOC_WORKSPACE_MAX bytes held by the library, one
 * per GPU it runs on, from the first call on that GPU until the process ends;
 * this call allocates and frees nothing. Returns FSL_E_WORKSPACE, before any
 * device work, when fsl_workspace_bytes(p) exceeds that size (256 MiB: the
 * bf16 forward of 16 heads x 16384 tokens x d=64 needs 141 MB). Every call on
 * one GPU uses that GPU's array: calls that overlap in time on one GPU (two
 * streams, two host threads) race and give undefined results. */
#define FSL_NOALLOC_WORKSPACE_MAX (256u << 20)
int fsl_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, const fsl_params *p,
                         int32_t *sel_out, float *o_win_out, float *o_long_out, hipStream_t stream);

/* Byte offsets of the named arrays inside a forward workspace (host-only).
 * Returns FSL_OK or the fsl_check_params error. */
typedef struct fsl_workspace_layout {
    size_t kbar;    /* float [H][C][d]            cell mean keys */
    size_t amax;    /* float [H][C]               cell max key norms */
    size_t pool;    /* int32 [H][ceil(N/B)][P+W]  per-block pools */
    size_t sel;     /* int32 [H][N][K]            per-query selections */
    size_t rope;    /* float2 table of (cos, sin) for relative offsets */
    size_t scan_a;  /* float / int32 lists of the prune scan */
    size_t scan_i;
    size_t o_win;   /* float [H][N][d]            window-branch output (fp32 inputs only) */
    size_t rope_abs;/* float2 (cos, sin) by absolute position, two levels (bf16 only) */
    size_t kt;      /* fp16 [H][Np][d] RoPE-rotated keys, Np = 64 ceil(N/64) (bf16 only) */
    size_t vt;      /* fp16 [H][Np/32][d][32] values transposed per 32 tokens (bf16 only) */
    size_t plan;    /* long branch work lists: per (head, 256-query span) cells and queries, or per-cell (query, rank) lists without pruning (bf16 only) */
    size_t part;    /* fp16 [H][N][K][d] each selected cell's normalised long-branch output (bf16 only) */
    size_t plse;    /* float [H][N][K] each selected cell's base-2 log-sum-exp of scaled scores (bf16 only) */
    size_t fixups;  /* uint32 near-tie query list of the bf16 scoring (bf16 only) */
    size_t khi;     /* bf16 [H][C][d] head of every kbar_c (bf16 with P = -1 only) */
    size_t klo;     /* bf16 [H][C][d] tail kbar_c - khi (bf16 with P = -1 only) */
    size_t kcf;     /* float4 [H][C] per-cell constants of the scoring bound (bf16 with P = -1 only) */
    size_t status;  /* uint32 input check word, set by every forward (see FSL_STATUS_F16_RANGE) */
    size_t total;   /* bytes; equals fsl_workspace_bytes */
} fsl_workspace_layout;
int fsl_workspace_views(const fsl_params *p, fsl_workspace_layout *out);

/* Bits of the workspace's status word after a forward (0 for fp32 inputs).
 * FSL_STATUS_F16_RANGE: with bf16 inputs, an element of k or v was not
 * finite or had magnitude >= 65504, past fp16's largest finite value (the
 * first such bf16 value is 65536), or a RoPE-rotated key rounded to an fp16
 * infinity. Both attention branches multiply fp16 operands, so the
 * outputs of such a call are undefined (typically inf or NaN); selections
 * and cell statistics do not depend on it. Reading the word is optional
 * (it costs a device-to-host copy after the call completes). */
#define FSL_STATUS_F16_RANGE 1u

/* ------------------------------------------------------------------------
 * Streaming decode (ai.info summary, "Why This Matters": a bounded streaming
 * state of O(((P+W)s + w + B + s)d) per head; methodology: the pool changes
 * only at block boundaries; digest, results: constant attention buffer from
 * 4k to 256k context).
 *
 * One flat, versioned device buffer holds the state of n_seq independent
 * sequences x H heads. Per (sequence, head): the next position t, a ring of
 * the last w + B + s tokens' raw k/v (the window plus the tokens not yet in
 * an eligible cell), and P + W pool slots, each holding one cell's raw k/v,
 * mean key and max key norm. When t enters a new block, the cells that became
 * eligible take free slots (copied once from the ring), the cells leaving the
 * recent set compete for the P high-norm places, and losers free their slots;
 * nothing else moves. The size does not depend on the prefix length.
 * Output at position t equals the forward's output at row t of the whole
 * sequence (selected cells bit-identical; window arithmetic in fp32 here).
 * fp32 and bf16 (dtype) are supported; P = -1 is not (FSL_E_UNSUPPORTED). */

/* Bytes of state for n_seq sequences under p (p->N is ignored); 0 if invalid. */
size_t fsl_decode_state_bytes(const fsl_params *p, int32_t n_seq);

/* Write the header and reset every sequence to position 0 with an empty pool.
 * state: device buffer of at least fsl_decode_state_bytes(p, n_seq) bytes. */
int fsl_decode_init(void *state, size_t state_bytes, int32_t n_seq, const fsl_params *p, hipStream_t stream);

/* Workspace bytes fsl_decode_prefill needs for a prefix of prefix_len tokens. */
size_t fsl_decode_prefill_workspace_bytes(const fsl_params *p, int64_t prefix_len);

/* Load sequence `seq` with a prefix of prefix_len >= 1 tokens: cell statistics
 * and the pool of the block holding position prefix_len are computed as in
 * the forward, the pool cells' k/v are copied into slots and the ring gets
 * the tokens since the first non-eligible cell. k_prefix, v_prefix: device
 * [H][prefix_len][d] (dtype); they are not referenced after the call's work
 * completes. The sequence's next position becomes prefix_len. */
int fsl_decode_prefill(void *state, size_t state_bytes, int32_t seq, const void *k_prefix, const void *v_prefix,
                       int64_t prefix_len, const fsl_params *p, void *ws, size_t ws_bytes, hipStream_t stream);

/* Append len tokens to each of the sequences seq0 .. seq0+n-1 without queries:
 * the streamed (chunked) prefill (ai.info summary, "Why This Matters" and future
 * directions: a bounded state fed in chunks, so that the prefix's O(N d) keys
 * and values need not be resident at once). k, v: device [n][H][len][d]
 * (dtype), for each sequence the tokens at positions t .. t+len-1 where t is
 * that sequence's current position (0 after fsl_decode_init; the sequences may
 * be at different positions). One work-group per (sequence, head) walks the
 * chunk block by block. At every query-block boundary the state's pool is updated
 * exactly as fsl_decode_step does it, so any split of a prefix into appends, or
 * a prefill followed by appends, gives the state a single fsl_decode_prefill of
 * the whole prefix gives (decode results are bit-identical). k and v are not
 * referenced after the call's work completes; no workspace is needed.
 * Positions must stay below 2^31 - B. Returns FSL_E_INVAL for a null or
 * misaligned pointer, len < 1, n < 1 or sequences outside the state's
 * capacity. */
int fsl_decode_append(void *state, size_t state_bytes, int32_t seq0, int32_t n, const void *k, const void *v,
                      int64_t len, const fsl_params *p, hipStream_t stream);

/* Advance every sequence by one token. q, k, v: device [n_seq][H][d] (dtype),
 * the new token of each sequence; out: device [n_seq][H][d] (out_dtype), the
 * attention output at that position. sel_out (nullable): device
 * [n_seq][H][K] int32, the cells read, ascending, padded with -1. n_seq must
 * equal the value the state was initialised with. */
int fsl_decode_step(void *state, size_t state_bytes, const void *q, const void *k, const void *v, void *out,
                    int32_t n_seq, const fsl_params *p, int32_t *sel_out, hipStream_t stream);

/* Synchronous check of a state buffer's header against p and n_seq (copies
 * the header to the host): FSL_OK, or FSL_E_STATE if the magic, version or
 * any parameter differs. The only entry point that waits for the device. */
int fsl_decode_validate(const void *state, size_t state_bytes, const fsl_params *p, int32_t n_seq);

#ifdef __cplusplus
}
#endif

#endif /* FSL_H */

// Streaming decode with a bounded state (ai.info summary, "Why This Matters":
// O(((P+W)s + w + B + s)d) per head; methodology: the pool of at most P+W
// cells changes only at query-block boundaries; FreeSolo digest, core method
// and steps 2-6 for what is computed per token).
//
// One workgroup per (sequence, head) and step. The state record of a
// (sequence, head) holds the next position t, the block whose pool is loaded,
// a ring of the last R = w + B + s tokens' raw k/v plus their keys rotated at
// their absolute positions (fp16 for bf16 inputs, fp32 otherwise), and P + W
// cell slots (cell index, max key norm, mean key, raw k/v). A step:
//  1. if t starts a new block, the cells that just became eligible get their
//     statistics from the ring (fp64, same order as the forward), the cells
//     leaving the recent set compete for the P high-norm places (keep the P
//     best under (a desc, index asc); a loser's slot is freed), and every
//     newly kept cell is copied once from the ring into a free slot;
//  2. appends the new k/v to the ring and its key rotated at t (angles in fp64);
//  3. wave 0 scores every occupied slot in fp64 exactly as the forward does,
//     keeps the top K under (score desc, index asc) and reads the chosen
//     cells' tokens out (NoPE), while
//  4. waves 1-3 attend over the window in the ring: R(t)q against the rotated
//     keys, whose loads keep HBM busy during wave 0's latency-bound chain;
//  5. merges the partial softmax states, RMSNorm, mix, write.
// Each attention gives its waves chunks of 64 keys. The window's fp16 key rows
// are read coalesced (a wave instruction covers 1 KB of consecutive rows) and
// each row's pieces are summed across its lanes; other key rows are read one
// per lane. The lanes then turn to dimensions for the P.V sum (each key's
// weight broadcast from its lane, value rows read coalesced). The slot means
// are copied into LDS (d = 64) while the new token is appended, so that
// scoring reads no global memory, and the top K is K rounds of a wave-wide
// maximum.
#include <climits>
#include <type_traits>

#include "fsl_internal.h"

namespace fsl {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecMaxPool = 128;
constexpr int kDecMaxNew = 16;   // cells entering per block boundary: B/s <= 256/16

__device__ __forceinline__ int64_t elig_nocap(const KParams &p, int64_t b) {
    const int64_t x = b * p.B - p.w + 1;
    return x <= 0 ? 0 : x / p.s;
}

// element type of the rotated-key ring: fp16 bits for bf16 inputs, fp32 otherwise
template <typename T> struct RotKey { typedef float type; };
template <> struct RotKey<uint16_t> { typedef uint16_t type; };
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    union { _Float16 f; uint16_t u; } c;
    c.f = (_Float16)x;  // round to nearest even
    return c.u;
}
template <typename RT> __device__ __forceinline__ RT rot_store(float x);
template <> __device__ __forceinline__ float rot_store<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t rot_store<uint16_t>(float x) { return f32_to_f16_bits(x); }

// eight consecutive elements of a key row as float: 16-bit elements are either
// bf16 (raw keys) or fp16 (rotated keys)
template <typename E, bool F16>
__device__ __forceinline__ void load8f(const E *ptr, float (&o)[8]) {
    if constexpr (sizeof(E) == 2) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(ptr);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (F16) {
                union { uint32_t u; _Float16 h[2]; } c;
                c.u = w4[t];
                o[2 * t] = (float)c.h[0];
                o[2 * t + 1] = (float)c.h[1];
            } else {
                o[2 * t] = __uint_as_float(w4[t] << 16);
                o[2 * t + 1] = __uint_as_float(w4[t] & 0xFFFF0000u);
            }
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(ptr);
        const float4 b = *reinterpret_cast<const float4 *>(ptr + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
}

__device__ float block_reduce(float v, float *scratch, bool is_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        const float o = __shfl_xor(v, m);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    float r = scratch[0];
    for (int w2 = 1; w2 < kDecThreads / 64; ++w2) r = is_max ? fmaxf(r, scratch[w2]) : r + scratch[w2];
    return r;
}

}  // namespace

__global__ void decode_init_kernel(char *__restrict__ state, KParams p, DecodeLayout L, int n_seq, int dtype) {
    const int rec_id = blockIdx.x;
    if (rec_id == 0 && threadIdx.x == 0) {
        DecodeHeader *hd = reinterpret_cast<DecodeHeader *>(state);
        hd->magic = kDecodeMagic;
        hd->version = kDecodeVersion;
        hd->H = p.H; hd->d = p.d; hd->w = p.w; hd->s = p.s; hd->P = p.P; hd->W = p.W; hd->K = p.K; hd->B = p.B;
        hd->dtype = dtype; hd->n_seq = n_seq; hd->R = L.R; hd->PW = L.PW;
        hd->rec_bytes = L.rec_bytes;
    }
    char *rec = state + L.off_rec + (int64_t)rec_id * L.rec_bytes;
    if (threadIdx.x == 0) {
        reinterpret_cast<int64_t *>(rec)[0] = 0;  // t
        reinterpret_cast<int64_t *>(rec)[1] = 0;  // block whose pool is loaded
    }
    int32_t *cell = reinterpret_cast<int32_t *>(rec + L.o_cell);
    for (int i = threadIdx.x; i < L.PW; i += blockDim.x) cell[i] = -1;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_prefill_kernel(char *__restrict__ state, int seq,
                                                             const T *__restrict__ kp, const T *__restrict__ vp,
                                                             int64_t Lp, const float *__restrict__ kbar,
                                                             const float *__restrict__ amax,
                                                             const int32_t *__restrict__ pool, KParams p,
                                                             DecodeLayout L) {
    // grid (parts, heads): every loop strides over the threads of all parts of its head
    const int h = blockIdx.y;
    const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, gn = (int64_t)gridDim.x * blockDim.x;
    char *rec = state + L.off_rec + ((int64_t)seq * p.H + h) * L.rec_bytes;
    const int64_t b = Lp / p.B;
    const int64_t nb = elig_nocap(p, b);
    const int npool = (int)min((int64_t)L.PW, nb);
    int32_t *cell = reinterpret_cast<int32_t *>(rec + L.o_cell);
    float *sa = reinterpret_cast<float *>(rec + L.o_a);
    float *skb = reinterpret_cast<float *>(rec + L.o_kbar);
    T *sk = reinterpret_cast<T *>(rec + L.o_sk);
    T *sv = reinterpret_cast<T *>(rec + L.o_sv);
    T *rk = reinterpret_cast<T *>(rec + L.o_rk);
    T *rv = reinterpret_cast<T *>(rec + L.o_rv);
    const int32_t *bp = pool + ((int64_t)h * p.nblk + b) * p.PW;
    const T *kh = kp + (int64_t)h * Lp * D;
    const T *vh = vp + (int64_t)h * Lp * D;
    for (int64_t i = gt; i < L.PW; i += gn) {
        const int c = i < npool ? bp[i] : -1;
        cell[i] = c;
        if (c >= 0) sa[i] = amax[(int64_t)h * p.C + c];
    }
    // the pool cells' mean keys, 16-byte pieces
    for (int64_t e = gt; e < (int64_t)npool * (D / 4); e += gn) {
        const int i = (int)(e / (D / 4)), x4 = (int)(e % (D / 4)) * 4;
        *reinterpret_cast<float4 *>(skb + (int64_t)i * D + x4) =
            *reinterpret_cast<const float4 *>(kbar + ((int64_t)h * p.C + bp[i]) * D + x4);
    }
    // the pool cells' raw tokens, then the ring's rows: 16-byte pieces, two per thread and
    // round with the loads issued first (addresses clamped, stores guarded)
    constexpr int EPP = 16 / (int)sizeof(T), PPRW = D / EPP;
    const int64_t spc = (int64_t)p.s * PPRW;  // pieces per cell
    const int64_t ncp = npool * spc;
    for (int64_t e0 = 0; e0 < ncp; e0 += 2 * gn) {
        const int64_t ea = e0 + gt, eb = e0 + gn + gt;
        const int64_t ca = min(ea, ncp - 1), cb = min(eb, ncp - 1);
        const int64_t sa0 = (int64_t)bp[ca / spc] * p.s * D + (ca % spc) * EPP;
        const int64_t sb0 = (int64_t)bp[cb / spc] * p.s * D + (cb % spc) * EPP;
        const uint4 ka = *reinterpret_cast<const uint4 *>(kh + sa0), va = *reinterpret_cast<const uint4 *>(vh + sa0);
        const uint4 kb = *reinterpret_cast<const uint4 *>(kh + sb0), vb = *reinterpret_cast<const uint4 *>(vh + sb0);
        if (ea < ncp) {
            *reinterpret_cast<uint4 *>(sk + ea * EPP) = ka;
            *reinterpret_cast<uint4 *>(sv + ea * EPP) = va;
        }
        if (eb < ncp) {
            *reinterpret_cast<uint4 *>(sk + eb * EPP) = kb;
            *reinterpret_cast<uint4 *>(sv + eb * EPP) = vb;
        }
    }
    const int64_t first = nb * p.s;
    const int64_t nrp = (Lp - first) * PPRW;
    for (int64_t e0 = 0; e0 < nrp; e0 += 2 * gn) {
        const int64_t ea = e0 + gt, eb = e0 + gn + gt;
        const int64_t ra = min(ea, nrp - 1), rb = min(eb, nrp - 1);
        const int64_t sa0 = (first + ra / PPRW) * D + (ra % PPRW) * EPP;
        const int64_t sb0 = (first + rb / PPRW) * D + (rb % PPRW) * EPP;
        const uint4 ka = *reinterpret_cast<const uint4 *>(kh + sa0), va = *reinterpret_cast<const uint4 *>(vh + sa0);
        const uint4 kb = *reinterpret_cast<const uint4 *>(kh + sb0), vb = *reinterpret_cast<const uint4 *>(vh + sb0);
        if (ea < nrp) {
            const int64_t d = ((first + ea / PPRW) % L.R) * D + (ea % PPRW) * EPP;
            *reinterpret_cast<uint4 *>(rk + d) = ka;
            *reinterpret_cast<uint4 *>(rv + d) = va;
        }
        if (eb < nrp) {
            const int64_t d = ((first + eb / PPRW) % L.R) * D + (eb % PPRW) * EPP;
            *reinterpret_cast<uint4 *>(rk + d) = kb;
            *reinterpret_cast<uint4 *>(rv + d) = vb;
        }
    }
    // the same tokens' keys rotated at their positions (angle pos * base^(-2m/d) in fp64)
    typedef typename RotKey<T>::type RT;
    RT *rkr = reinterpret_cast<RT *>(rec + L.o_rkr);
    for (int64_t e = gt; e < (Lp - first) * (D / 2); e += gn) {
        const int64_t pos = first + e / (D / 2);
        const int m = (int)(e % (D / 2));
        const double theta = pow((double)p.rope_base, -2.0 * (double)m / (double)D);
        const double ang = (double)pos * theta;
        const float c = (float)cos(ang), sn = (float)sin(ang);
        const float a = to_f32<T>(kh[pos * D + m]), bb = to_f32<T>(kh[pos * D + m + D / 2]);
        const int64_t slot = pos % L.R;
        rkr[slot * D + m] = rot_store<RT>(a * c - bb * sn);
        rkr[slot * D + m + D / 2] = rot_store<RT>(bb * c + a * sn);
    }
    if (gt == 0) {
        reinterpret_cast<int64_t *>(rec)[0] = Lp;
        reinterpret_cast<int64_t *>(rec)[1] = b;
    }
}

// Block boundary of a (sequence, head) record, shared by the decode step and the
// append: when position b B starts a block with new eligible cells (blk is the
// block of the previous token), the new cells' norms come from the ring, the cells
// leaving the recent set compete for the P high-norm places, and every newly kept
// cell's tokens and mean key are copied from the ring into a free slot. s_cell /
// s_a mirror the record's slot table in LDS and are written back. All threads of
// the work-group call it (it synchronises).
template <typename T, int D>
__device__ void decode_boundary(const KParams &p, int64_t blk, int64_t b, int PW, int R, int tid, int *s_cell,
                                float *s_a, double *s_ss, float *s_newa, int *s_load_cell, int *s_load_slot,
                                int *s_nload, const T *rk, const T *rv, T *sk, T *sv, float *skb, int32_t *cell,
                                float *sa) {
    const int s = p.s;
    const int64_t n_old = elig_nocap(p, blk), n_new = elig_nocap(p, b);
    if (b != blk && n_new > n_old) {
        const int nnew = (int)(n_new - n_old);  // <= B/s <= kDecMaxNew
        // max key norm of the new cells from the ring (fp64 fma chain in coordinate order)
        for (int r = tid; r < nnew * s; r += kDecThreads) {
            const int cn = r / s, j = r % s;
            const int64_t pos = (n_old + cn) * s + j;
            const T *row = rk + (pos % R) * D;
            double acc = 0.0;
#pragma unroll 2
            for (int x0 = 0; x0 < D; x0 += 16) {
                float fa[8], fb[8];
                load8f<T, false>(row + x0, fa);
                load8f<T, false>(row + x0 + 8, fb);
#pragma unroll
                for (int u = 0; u < 8; ++u) acc = __fma_rn((double)fa[u], (double)fa[u], acc);
#pragma unroll
                for (int u = 0; u < 8; ++u) acc = __fma_rn((double)fb[u], (double)fb[u], acc);
            }
            s_ss[r] = acc;
        }
        __syncthreads();
        if (tid < nnew) {
            double best = 0.0;
            for (int j = 0; j < s; ++j) {
                const double v = s_ss[tid * s + j];
                if (v > best) best = v;
            }
            s_newa[tid] = (float)__dsqrt_rn(best);
        }
        __syncthreads();
        if (tid < 64) {
            // wave 0: lane l holds slots l and 64 + l (cell -2 marks a slot past PW). The cells
            // leaving the recent set are taken in index order, as one thread would: each either
            // keeps its slot (fewer than P high-norm cells, or it beats their worst member, which
            // is freed), or is freed; then the new cells take the lowest free slots.
            const int lane = tid;
            const int i0 = lane, i1 = lane + 64;
            int cl0 = i0 < PW ? s_cell[i0] : -2, cl1 = i1 < PW ? s_cell[i1] : -2;
            float al0 = i0 < PW ? s_a[i0] : 0.0f, al1 = i1 < PW ? s_a[i1] : 0.0f;
            const int64_t m_old = n_old > p.W ? n_old - p.W : 0;
            const int64_t m_new = n_new > p.W ? n_new - p.W : 0;
            auto count = [&](bool x0, bool x1) { return __popcll(__ballot(x0)) + __popcll(__ballot(x1)); };
            auto first = [&](bool x0, bool x1) {  // lowest slot index with the property, or -1
                const uint64_t b0 = __ballot(x0), b1 = __ballot(x1);
                return b0 ? __ffsll((unsigned long long)b0) - 1 : b1 ? 64 + __ffsll((unsigned long long)b1) - 1 : -1;
            };
            auto set_slot = [&](int sc, int c, float a) {
                if (sc == i0) { cl0 = c; al0 = a; }
                if (sc == i1) { cl1 = c; al1 = a; }
            };
            auto a_of = [&](int sc) {
                return __uint_as_float(sc < 64 ? __builtin_amdgcn_readlane(__float_as_uint(al0), sc)
                                               : __builtin_amdgcn_readlane(__float_as_uint(al1), sc - 64));
            };
            int top = count(cl0 >= 0 && cl0 < m_old, cl1 >= 0 && cl1 < m_old);
            int nload = 0;
            for (int64_t c = m_old; c < m_new; ++c) {
                int sc = -1;
                float ac;
                if (c < n_old) {
                    sc = first(cl0 == c, cl1 == c);
                    if (sc < 0) continue;  // cannot happen: every recent cell holds a slot
                    ac = a_of(sc);
                } else {
                    ac = s_newa[c - n_old];
                }
                bool keep = false;
                if (p.P > 0) {
                    if (top < p.P) {
                        keep = true;
                    } else {
                        // the high-norm set is every occupied cell below c; its worst member
                        // (smallest a, then largest index) is the best under (-a, -index)
                        const bool m0 = cl0 >= 0 && cl0 < c, m1 = cl1 >= 0 && cl1 < c;
                        const double k0 = m0 ? -(double)al0 : -INFINITY, k1 = m1 ? -(double)al1 : -INFINITY;
                        const int x0 = m0 ? -cl0 : INT_MAX, x1 = m1 ? -cl1 : INT_MAX;
                        const bool pick0 = better_d(k0, x0, k1, x1) || !m1;
                        double wk = pick0 ? k0 : k1;
                        int wx = pick0 ? x0 : x1, wsl = pick0 ? i0 : i1;
                        wave_best_d(wk, wx, wsl);
                        if (wk != -INFINITY && better(ac, (int)c, (float)(-wk), -wx)) {
                            set_slot(wsl, -1, a_of(wsl));
                            --top;
                            keep = true;
                        }
                    }
                }
                if (keep) {
                    if (sc < 0) {
                        sc = first(i0 < PW && cl0 < 0 && cl0 != -2, i1 < PW && cl1 < 0 && cl1 != -2);
                        if (sc < 0) continue;  // cannot happen: at most P + W cells are ever held
                        set_slot(sc, (int)c, ac);
                        if (lane == 0) {
                            s_load_cell[nload] = (int)c;
                            s_load_slot[nload] = sc;
                        }
                        ++nload;
                    }
                    ++top;
                } else if (sc >= 0) {
                    set_slot(sc, -1, a_of(sc));
                }
            }
            for (int64_t c = (n_old > m_new ? n_old : m_new); c < n_new; ++c) {
                const int sc = first(i0 < PW && cl0 < 0 && cl0 != -2, i1 < PW && cl1 < 0 && cl1 != -2);
                if (sc < 0) break;  // cannot happen: at most P + W cells are ever held
                set_slot(sc, (int)c, s_newa[c - n_old]);
                if (lane == 0) {
                    s_load_cell[nload] = (int)c;
                    s_load_slot[nload] = sc;
                }
                ++nload;
            }
            if (i0 < PW) { s_cell[i0] = cl0; s_a[i0] = al0; }
            if (i1 < PW) { s_cell[i1] = cl1; s_a[i1] = al1; }
            if (lane == 0) *s_nload = nload;
        }
        __syncthreads();
        const int nload = *s_nload;
        // the kept cells' tokens, ring -> slot, in 16-byte pieces with a batch of loads per thread
        // (addresses clamped, stores guarded)
        constexpr int EPP = 16 / (int)sizeof(T), PPRW = D / EPP;
        const int ls = __builtin_ctz((unsigned)s);  // s is a power of two
        const int npc = nload * s * PPRW;
        auto piece = [&](int e, int64_t &src, int64_t &dst) __attribute__((always_inline)) {
            const int rr = e / PPRW, pc = e % PPRW, li = rr >> ls, tok = rr & (s - 1);
            src = ((((int64_t)s_load_cell[li] << ls) + tok) % R) * D + pc * EPP;
            dst = (((int64_t)s_load_slot[li] << ls) + tok) * D + pc * EPP;
        };
        for (int e0 = 0; e0 < npc; e0 += 2 * kDecThreads) {
            const int ea = e0 + tid, eb = e0 + kDecThreads + tid;
            int64_t sa0, da0, sb0, db0;
            piece(min(ea, npc - 1), sa0, da0);
            piece(min(eb, npc - 1), sb0, db0);
            const uint4 ka = *reinterpret_cast<const uint4 *>(rk + sa0), va = *reinterpret_cast<const uint4 *>(rv + sa0);
            const uint4 kb = *reinterpret_cast<const uint4 *>(rk + sb0), vb = *reinterpret_cast<const uint4 *>(rv + sb0);
            if (ea < npc) {
                *reinterpret_cast<uint4 *>(sk + da0) = ka;
                *reinterpret_cast<uint4 *>(sv + da0) = va;
            }
            if (eb < npc) {
                *reinterpret_cast<uint4 *>(sk + db0) = kb;
                *reinterpret_cast<uint4 *>(sv + db0) = vb;
            }
        }
        // their mean keys: fp64 sums in token order, each batch of 16 tokens' loads issued together
        for (int e = tid; e < nload * D; e += kDecThreads) {
            const int li = e / D, x = e % D;
            const int64_t c = s_load_cell[li];
            double acc = 0.0;
            constexpr int TB = sizeof(T) == 2 ? 16 : 8;  // tokens per batch
            for (int j0 = 0; j0 < s; j0 += TB) {
                float f[TB];
#pragma unroll
                for (int u = 0; u < TB; ++u) f[u] = to_f32<T>(rk[((c * s + min(j0 + u, s - 1)) % R) * D + x]);
#pragma unroll
                for (int u = 0; u < TB; ++u) acc += j0 + u < s ? (double)f[u] : 0.0;
            }
            skb[(int64_t)s_load_slot[li] * D + x] = (float)(acc / (double)s);
        }
        for (int i = tid; i < PW; i += kDecThreads) {
            cell[i] = s_cell[i];
            sa[i] = s_a[i];
        }
        __syncthreads();
    }

}

// Keys of 16-bit types are read coalesced: a 64-key chunk of rows (PPR 16-byte pieces each)
// is loaded RPI = 64 / PPR rows per wave instruction, lane l holding piece l % PPR of row
// l / PPR, so instruction i gives the lane a partial dot of key i * RPI + l / PPR. Summing the
// PPR pieces of a row is a reduce-scatter over the PPR lanes of a row group (recursive halving,
// highest index bit first): after it, part[0] of the lane with piece pc is the dot of its
// group's key with instruction index pc. Partners: the mirrored row or half row for the first
// halving (either flips the bit being split), then i ^ 2 and i ^ 1 (quad permutes); each later
// partner agrees on the bits already split. The whole wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int H, int PPR>
__device__ __forceinline__ void halve_pieces(float (&a)[PPR], int pc) {
    constexpr int CTRL = H == PPR / 2 ? (PPR == 16 ? 0x140 : 0x141) : H == 4 ? 0x141 : H == 2 ? 0x4E : 0xB1;
    const bool hi = (pc & H) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const float send = hi ? a[j] : a[j + H];
        const float keep = hi ? a[j + H] : a[j];
        a[j] = keep + dpp_f<CTRL>(send);
    }
    if constexpr (H > 1) halve_pieces<H / 2, PPR>(a, pc);
}

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads, 4) void decode_step_kernel(char *__restrict__ state, const T *__restrict__ qn,
                                                                  const T *__restrict__ kn, const T *__restrict__ vn,
                                                                  void *__restrict__ out, int32_t *__restrict__ sel_out,
                                                                  KParams p, DecodeLayout L) {
    __shared__ __attribute__((aligned(16))) float s_q[D];
    __shared__ int s_cell[kDecMaxPool];
    __shared__ float s_a[kDecMaxPool];
    __shared__ int s_sel[8];
    __shared__ int s_selslot[8];
    __shared__ float s_red[kDecThreads / 64];
    __shared__ __attribute__((aligned(16))) float s_qr[D];  // R(t) q
    __shared__ float s_wm[kDecWaves], s_wl[kDecWaves];     // per-wave softmax state
    __shared__ float s_wo[kDecWaves][D];                    // per-wave partial outputs
    __shared__ double s_ss[kDecMaxNew * 64];
    __shared__ float s_newa[kDecMaxNew];
    __shared__ int s_load_cell[kDecMaxNew], s_load_slot[kDecMaxNew], s_nload;
    // d = 64: the slot means, copied in before the window so that scoring reads LDS
    extern __shared__ __attribute__((aligned(16))) float s_kbl[];
    constexpr bool KB_LDS = D == 64;

    const int rid = blockIdx.x;  // seq * H + h
    const int h = rid % p.H;
    const int tid = threadIdx.x;
    char *rec = state + L.off_rec + (int64_t)rid * L.rec_bytes;
    int64_t *hdr = reinterpret_cast<int64_t *>(rec);
    int32_t *cell = reinterpret_cast<int32_t *>(rec + L.o_cell);
    float *sa = reinterpret_cast<float *>(rec + L.o_a);
    float *skb = reinterpret_cast<float *>(rec + L.o_kbar);
    T *sk = reinterpret_cast<T *>(rec + L.o_sk);
    T *sv = reinterpret_cast<T *>(rec + L.o_sv);
    T *rk = reinterpret_cast<T *>(rec + L.o_rk);
    T *rv = reinterpret_cast<T *>(rec + L.o_rv);
    typedef typename RotKey<T>::type RT;
    RT *rkr = reinterpret_cast<RT *>(rec + L.o_rkr);
    const int s = p.s, PW = L.PW, R = L.R;
    const int lane = tid & 63, wave = tid >> 6;

    const int64_t t = hdr[0];
    const int64_t blk = hdr[1];
    const int64_t b = t / p.B;
    for (int i = tid; i < PW; i += kDecThreads) {
        s_cell[i] = cell[i];
        s_a[i] = sa[i];
    }
    if (tid < D) s_q[tid] = to_f32<T>(qn[(int64_t)rid * D + tid]);
    __syncthreads();

    // ---- 1. block boundary: new eligible cells, recent -> high-norm competition
    decode_boundary<T, D>(p, blk, b, PW, R, tid, s_cell, s_a, s_ss, s_newa, s_load_cell, s_load_slot, &s_nload, rk, rv,
                          sk, sv, skb, cell, sa);

    // the slot means are final now: start their copy into LDS (1 KB per wave instruction, the
    // source clamped to the array), so that it is queued ahead of the window's loads
    if constexpr (KB_LDS) {
        const int nbytes = PW * D * 4, npiece = (nbytes + 1023) >> 10;
        const char *src = reinterpret_cast<const char *>(skb);
        for (int k = wave; k < npiece; k += kDecWaves) {
            const int off = min(k * 1024 + 16 * lane, nbytes - 16);
            lds_dma16(src + off, reinterpret_cast<char *>(s_kbl) + k * 1024);
        }
    }

    // ---- 2. append the new token: raw k/v, and the key rotated at t
    const int64_t tslot = t % R;
    if (tid < D / 2) {
        const int m = tid;
        const double theta = pow((double)p.rope_base, -2.0 * (double)m / (double)D);
        const double ang = (double)t * theta;
        const float c = (float)cos(ang), sn = (float)sin(ang);
        const float qa = s_q[m], qb = s_q[m + D / 2];
        s_qr[m] = qa * c - qb * sn;
        s_qr[m + D / 2] = qb * c + qa * sn;
        const float ka = to_f32<T>(kn[(int64_t)rid * D + m]), kb = to_f32<T>(kn[(int64_t)rid * D + m + D / 2]);
        rkr[tslot * D + m] = rot_store<RT>(ka * c - kb * sn);
        rkr[tslot * D + m + D / 2] = rot_store<RT>(kb * c + ka * sn);
    }
    if (tid < D) {
        rk[tslot * D + tid] = kn[(int64_t)rid * D + tid];
        rv[tslot * D + tid] = vn[(int64_t)rid * D + tid];
    }
    __syncthreads();

    const float sl2 = p.scale * 1.4426950408889634f;
    constexpr int DPL = D / 64;  // dimensions per lane in the P.V sums

    // Softmax attention of one query (qs in LDS) over nkeys keys: key u's row at krow(u)
    // (fp16 bits if kf16, else the input type), its value row at vrow(u), run by the waves
    // w0 .. w0 + nw - 1. Keys go to lanes in chunks of 64 (chunk c to wave w0 + c mod nw); each
    // wave leaves its own (max, sum, o) in s_wm / s_wl / s_wo, combined by merge() below.
    auto attend = [&](int nkeys, const float *qs, auto krow, auto vrow, auto kf16, int w0, int nw)
        __attribute__((always_inline)) {
        typedef typename std::remove_cv<typename std::remove_pointer<decltype(krow(0))>::type>::type KE;
        constexpr bool KF16 = decltype(kf16)::value;  // 16-bit keys: fp16 (rotated ring) or bf16 (raw)
        float m_run = -INFINITY, l_run = 0.0f;
        float o[DPL];
#pragma unroll
        for (int d2 = 0; d2 < DPL; ++d2) o[d2] = 0.0f;
        // 16-bit values at d = 64: each half of the wave takes 32 of the chunk's keys and each
        // lane two adjacent dimensions, so a lane's 32 value pairs (one dword each) are all
        // requested with the chunk's keys; the halves are added at the end
        constexpr bool HALF_PV = sizeof(T) == 2 && D == 64;
        float o2[2] = {0.0f, 0.0f};
        const int hf = lane >> 5, dp = 2 * (lane & 31);
        // the window's fp16 keys: coalesced rows and a reduce-scatter of the pieces (see
        // halve_pieces); lane l then scores key kl of the chunk, and key j's weight sits in lane
        // key_lane(j). The readout keeps one row per lane: its rows are found through the slot
        // table, one lookup per lane instead of one per row and instruction (measured faster).
        constexpr bool CO = sizeof(KE) == 2 && KF16;
        constexpr int PPR = CO ? D / 8 : 1, RPI = 64 / PPR;
        const int pc = lane % PPR, ri = lane / PPR;
        const int kl = CO ? pc * RPI + ri : lane;
        auto key_lane = [](int j) { return CO ? (j % RPI) * PPR + j / RPI : j; };
        float qv[8];
        if constexpr (CO) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] = qs[pc * 8 + e];
        }
        for (int c0 = 64 * (wave - w0); c0 < nkeys; c0 += 64 * nw) {
            const int u = c0 + kl;
            const int nkc = min(64, nkeys - c0);
            uint32_t vpair[HALF_PV ? 32 : 1];
            if constexpr (HALF_PV) {
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    vpair[j] = *reinterpret_cast<const uint32_t *>(vrow(c0 + min(32 * hf + j, nkc - 1)) + dp);
            }
            float sc = -INFINITY;
            if constexpr (CO) {
                float part[PPR];
#pragma unroll
                for (int i = 0; i < PPR; ++i) {
                    float kf[8];
                    load8f<KE, KF16>(krow(c0 + min(i * RPI + ri, nkc - 1)) + pc * 8, kf);
                    part[i] = qv[0] * kf[0] + qv[1] * kf[1] + qv[2] * kf[2] + qv[3] * kf[3] + qv[4] * kf[4] +
                              qv[5] * kf[5] + qv[6] * kf[6] + qv[7] * kf[7];
                }
                halve_pieces<PPR / 2, PPR>(part, pc);
                sc = u < nkeys ? part[0] * sl2 : -INFINITY;
            } else if (u < nkeys) {
                const KE *kr = krow(u);
                float dot = 0.0f;
#pragma unroll 2
                for (int x0 = 0; x0 < D; x0 += 8) {
                    float kf[8];
                    load8f<KE, KF16>(kr + x0, kf);
                    const float4 qa = *reinterpret_cast<const float4 *>(qs + x0);
                    const float4 qb = *reinterpret_cast<const float4 *>(qs + x0 + 4);
                    dot += qa.x * kf[0] + qa.y * kf[1] + qa.z * kf[2] + qa.w * kf[3] + qb.x * kf[4] + qb.y * kf[5] +
                           qb.z * kf[6] + qb.w * kf[7];
                }
                sc = dot * sl2;
            }
            float cm = sc;
#pragma unroll
            for (int m2 = 32; m2 > 0; m2 >>= 1) cm = fmaxf(cm, __shfl_xor(cm, m2));
            const float m_new = fmaxf(m_run, cm);
            const float alpha = m_run == -INFINITY ? 0.0f : exp2f(m_run - m_new);
            const float pj = u < nkeys ? exp2f(sc - m_new) : 0.0f;
            float ps = pj;
#pragma unroll
            for (int m2 = 32; m2 > 0; m2 >>= 1) ps += __shfl_xor(ps, m2);
            l_run = l_run * alpha + ps;
#pragma unroll
            for (int d2 = 0; d2 < DPL; ++d2) o[d2] *= alpha;
            o2[0] *= alpha;
            o2[1] *= alpha;
            m_run = m_new;
            if constexpr (HALF_PV) {
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    // weight of key 32 hf + j, from its lane (zero past the chunk's end)
                    const float p0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pj), key_lane(j)));
                    const float p1 =
                        __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pj), key_lane(32 + j)));
                    const float pk = 32 * hf + j < nkc ? (hf ? p1 : p0) : 0.0f;
                    o2[0] = fmaf(pk, __uint_as_float(vpair[j] << 16), o2[0]);
                    o2[1] = fmaf(pk, __uint_as_float(vpair[j] & 0xFFFF0000u), o2[1]);
                }
                continue;
            }
            // lanes as dimensions: o[lane*DPL + d2] += p_u v_u, the weight taken from lane u
            // value rows in batches of KB keys, each batch's loads issued together
            constexpr int KB = 16;
            const int nk = nkc;
#pragma unroll 1
            for (int k0 = 0; k0 < nk; k0 += KB) {
                float vv[KB][DPL];
#pragma unroll
                for (int j2 = 0; j2 < KB; ++j2) {
                    const T *vr = vrow(c0 + min(k0 + j2, nk - 1)) + lane * DPL;
#pragma unroll
                    for (int d2 = 0; d2 < DPL; ++d2) vv[j2][d2] = to_f32<T>(vr[d2]);
                }
#pragma unroll
                for (int j2 = 0; j2 < KB; ++j2) {
                    // weight of key k0 + j2, broadcast from its lane (zero past the chunk's end)
                    const float pk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pj), key_lane(k0 + j2)));
#pragma unroll
                    for (int d2 = 0; d2 < DPL; ++d2) o[d2] += (k0 + j2 < nk ? pk : 0.0f) * vv[j2][d2];
                }
            }
        }
        if (lane == 0) {
            s_wm[wave] = m_run;
            s_wl[wave] = l_run;
        }
        if constexpr (HALF_PV) {
            o2[0] += __shfl_xor(o2[0], 32);
            o2[1] += __shfl_xor(o2[1], 32);
            if (lane < 32) {
                s_wo[wave][dp] = o2[0];
                s_wo[wave][dp + 1] = o2[1];
            }
        } else {
#pragma unroll
            for (int d2 = 0; d2 < DPL; ++d2) s_wo[wave][lane * DPL + d2] = o[d2];
        }
    };
    // softmax merge of the partials of waves w0 .. w0 + nw - 1, for dimension x = tid < D
    auto merge = [&](int w0, int nw) __attribute__((always_inline)) {
        float mm = -INFINITY;
        for (int w2 = w0; w2 < w0 + nw; ++w2) mm = fmaxf(mm, s_wm[w2]);
        float num = 0.0f, den = 0.0f;
        for (int w2 = w0; w2 < w0 + nw; ++w2) {
            const float f = s_wm[w2] == -INFINITY ? 0.0f : exp2f(s_wm[w2] - mm);
            num += f * s_wo[w2][tid];
            den += f * s_wl[w2];
        }
        return den > 0.0f ? num / den : 0.0f;
    };

    // ---- 3. the long-range branch on wave 0: exact fp64 cell scores, top K, readout.
    // ---- 4. at the same time, waves 1 .. 3: the window over keys [max(0, t-w+1), t], R(t)q
    //         against the rotated keys. The window's loads keep HBM busy while wave 0 works
    //         through its latency-bound chain.
    if constexpr (KB_LDS) {
        wait_vmem();  // this wave's slot-mean copies have landed; the barrier publishes them
        __syncthreads();
    }
    if (wave == 0) {
        const double sig = (double)p.sigma[h], lam = (double)p.lambda[h], rho = (double)p.rho;
        // lane takes slots lane and lane + 64: two independent fma chains over the dimensions,
        // each in ascending order
        const int i0 = lane, i1 = lane + 64;
        const bool ok0 = i0 < PW && s_cell[i0] >= 0, ok1 = i1 < PW && s_cell[i1] >= 0;
        const float *kbase = KB_LDS ? s_kbl : skb;
        const float *kr0 = kbase + (int64_t)(i0 < PW ? i0 : 0) * D;
        const float *kr1 = kbase + (int64_t)(i1 < PW ? i1 : 0) * D;
        double ct0 = 0.0, ct1 = 0.0;
        const bool two = PW > 64;
#pragma unroll 4
        for (int x0 = 0; x0 < D; x0 += 4) {
            const float4 ka = *reinterpret_cast<const float4 *>(kr0 + x0);
            const float4 kb4 = two ? *reinterpret_cast<const float4 *>(kr1 + x0) : ka;
            const double q0 = s_q[x0], q1 = s_q[x0 + 1], q2 = s_q[x0 + 2], q3 = s_q[x0 + 3];
            ct0 = __fma_rn(q0, (double)ka.x, ct0);
            ct1 = __fma_rn(q0, (double)kb4.x, ct1);
            ct0 = __fma_rn(q1, (double)ka.y, ct0);
            ct1 = __fma_rn(q1, (double)kb4.y, ct1);
            ct0 = __fma_rn(q2, (double)ka.z, ct0);
            ct1 = __fma_rn(q2, (double)kb4.z, ct1);
            ct0 = __fma_rn(q3, (double)ka.w, ct0);
            ct1 = __fma_rn(q3, (double)kb4.w, ct1);
        }
        auto finish = [&](int i, double content) __attribute__((always_inline)) {
            const int c = s_cell[i];
            const double arg = __ddiv_rn(__dmul_rn(sig, (double)(t - (int64_t)c * s)), 2.0 * (double)s);
            const double gg = arg >= 6.0 ? 1.0 : erf(arg);
            const double bias = __dmul_rn(__dmul_rn(lam, (double)s_a[i]), gg);
            return __fma_rn(rho, content, bias);
        };
        double v0 = -INFINITY, v1 = -INFINITY;
        int c0 = INT_MAX, c1 = INT_MAX;
        if (ok0) { v0 = finish(i0, ct0); c0 = s_cell[i0]; }
        if (ok1) { v1 = finish(i1, ct1); c1 = s_cell[i1]; }

        // top K under (score desc, cell asc): K rounds of a wave-wide maximum, the lane that held
        // the winner drops it (cells are distinct); comparisons are written as selects
        static_assert(kDecMaxPool <= 128, "two slots per lane of one wave");
        int wc[8], ws[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            wc[r] = INT_MAX;
            ws[r] = -1;
            if (r < p.K) {
                const bool first = better_d(v0, c0, v1, c1) || c1 == INT_MAX;
                double vb = first ? v0 : v1;
                int cb = first ? c0 : c1;
                int sb = first ? i0 : i1;
                wave_best_d(vb, cb, sb);
                wc[r] = cb;
                ws[r] = cb == INT_MAX ? -1 : sb;
                const bool d0 = cb != INT_MAX && c0 == cb, d1 = cb != INT_MAX && c1 == cb;
                v0 = d0 ? -INFINITY : v0;
                c0 = d0 ? INT_MAX : c0;
                v1 = d1 ? -INFINITY : v1;
                c1 = d1 ? INT_MAX : c1;
            }
        }
        // the winners in ascending cell order: lane r < K puts winner r at the count of smaller
        // cells (empty picks, INT_MAX with slot -1, land after the others)
        if (lane < 8) {
            s_sel[lane] = INT_MAX;
            s_selslot[lane] = -1;
        }
        int mc = wc[0], msl = ws[0], nsel = 0, below = 0;
#pragma unroll
        for (int r = 1; r < 8; ++r) {
            mc = lane == r ? wc[r] : mc;
            msl = lane == r ? ws[r] : msl;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            below += wc[r] < mc ? 1 : 0;
            nsel += ws[r] >= 0 ? 1 : 0;
        }
        if (lane < p.K) {
            s_sel[below] = mc;
            s_selslot[below] = msl;
        }
        // a wave's LDS operations complete in issue order: the reads below see these writes
        if (sel_out && lane < p.K) sel_out[(int64_t)rid * p.K + lane] = s_selslot[lane] >= 0 ? s_sel[lane] : -1;

        // NoPE readout over the chosen cells' tokens, in ascending cell order
        const int ntok = nsel * s;
        const int ls = __builtin_ctz((unsigned)s);  // s is a power of two
        auto slot_row = [=](int u) { return ((s_selslot[u >> ls] << ls) + (u & (s - 1))) * D; };
        attend(
            ntok, s_q, [&](int u) { return (const T *)(sk + slot_row(u)); },
            [&](int u) { return (const T *)(sv + slot_row(u)); }, std::false_type{}, 0, 1);
    } else {
        const int64_t j_lo = t - p.w + 1 > 0 ? t - p.w + 1 : 0;
        const int nwin = (int)(t - j_lo + 1);
        const int r0 = (int)(j_lo % R);  // ring row of key j_lo; keys j_lo + u stay below j_lo + R
        auto ring = [=](int u) { const int r = r0 + u; return (r >= R ? r - R : r) * D; };
        attend(
            nwin, s_qr, [&](int u) { return (const RT *)(rkr + ring(u)); },
            [&](int u) { return (const T *)(rv + ring(u)); },
            std::integral_constant<bool, sizeof(RT) == 2>{}, 1, kDecWaves - 1);
    }
    __syncthreads();

    // ---- 5. RMSNorm of the long-range output, mix
    float o_win = 0.0f, o_long = 0.0f;
    if (tid < D) {
        o_win = merge(1, kDecWaves - 1);
        o_long = merge(0, 1);
    }
    const float ms = block_reduce(tid < D ? o_long * o_long : 0.0f, s_red, false) / (float)D;
    if (tid < D) {
        const float val = o_win + p.gamma[h] * (o_long / sqrtf(ms + p.rms_eps));
        if (p.out_dtype == FSL_BF16) reinterpret_cast<uint16_t *>(out)[(int64_t)rid * D + tid] = f32_to_bf16(val);
        else reinterpret_cast<float *>(out)[(int64_t)rid * D + tid] = val;
    }
    if (tid == 0) {
        hdr[0] = t + 1;
        hdr[1] = b;
    }
}

// Append len tokens of one sequence (all heads) to its records without queries: the
// state then equals the one a prefill of the whole prefix would give, without the
// prefix's O(N d) keys and values or a workspace (ai.info summary, "Why This
// Matters" and future directions: bounded streaming state, fed in chunks). One
// work-group per head. Block by block: the block boundary as in the decode step,
// then the block's tokens go into the ring in parallel (raw k/v, and keys rotated at
// their positions with fp64 angles). A launch covers sequences seq0 .. seq0 + n - 1
// (one work-group per (sequence, head)), k/v [n][H][len][d].
template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void decode_append_kernel(char *__restrict__ state, int seq0,
                                                                    const T *__restrict__ kc, const T *__restrict__ vc,
                                                                    int64_t len, KParams p, DecodeLayout L) {
    __shared__ int s_cell[kDecMaxPool];
    __shared__ float s_a[kDecMaxPool];
    __shared__ double s_ss[kDecMaxNew * 64];
    __shared__ float s_newa[kDecMaxNew];
    __shared__ int s_load_cell[kDecMaxNew], s_load_slot[kDecMaxNew], s_nload;
    const int rl = blockIdx.x;  // (sequence - seq0) * H + head
    const int tid = threadIdx.x;
    char *rec = state + L.off_rec + ((int64_t)seq0 * p.H + rl) * L.rec_bytes;
    int64_t *hdr = reinterpret_cast<int64_t *>(rec);
    int32_t *cell = reinterpret_cast<int32_t *>(rec + L.o_cell);
    float *sa = reinterpret_cast<float *>(rec + L.o_a);
    float *skb = reinterpret_cast<float *>(rec + L.o_kbar);
    T *sk = reinterpret_cast<T *>(rec + L.o_sk);
    T *sv = reinterpret_cast<T *>(rec + L.o_sv);
    T *rk = reinterpret_cast<T *>(rec + L.o_rk);
    T *rv = reinterpret_cast<T *>(rec + L.o_rv);
    typedef typename RotKey<T>::type RT;
    RT *rkr = reinterpret_cast<RT *>(rec + L.o_rkr);
    const int PW = L.PW, R = L.R;
    const int64_t t0 = hdr[0];
    int64_t blk = hdr[1];
    for (int i = tid; i < PW; i += kDecThreads) {
        s_cell[i] = cell[i];
        s_a[i] = sa[i];
    }
    __syncthreads();
    const T *kh = kc + (int64_t)rl * len * D;
    const T *vh = vc + (int64_t)rl * len * D;
    for (int64_t j = 0; j < len;) {
        const int64_t b = (t0 + j) / p.B;
        decode_boundary<T, D>(p, blk, b, PW, R, tid, s_cell, s_a, s_ss, s_newa, s_load_cell, s_load_slot, &s_nload, rk,
                              rv, sk, sv, skb, cell, sa);
        blk = b;
        const int64_t jend = min(len, (b + 1) * p.B - t0);  // this block's tokens within the chunk
        const int64_t n = jend - j;
        // raw rows into the ring in 16-byte pieces, a batch of pieces per thread with its loads
        // issued together (addresses clamped to the block, stores guarded)
        constexpr int EPP = 16 / (int)sizeof(T), PPRW = D / EPP, BAT = 4;
        const int64_t npc = n * PPRW;
        for (int64_t e0 = 0; e0 < npc; e0 += (int64_t)kDecThreads * BAT) {
            uint4 kk[BAT], vv[BAT];
#pragma unroll
            for (int q = 0; q < BAT; ++q) {
                const int64_t e = min(e0 + tid + (int64_t)kDecThreads * q, npc - 1);
                const int64_t off = (j + e / PPRW) * D + (e % PPRW) * EPP;
                kk[q] = *reinterpret_cast<const uint4 *>(kh + off);
                vv[q] = *reinterpret_cast<const uint4 *>(vh + off);
            }
#pragma unroll
            for (int q = 0; q < BAT; ++q) {
                const int64_t e = e0 + tid + (int64_t)kDecThreads * q;
                if (e < npc) {
                    const int64_t u = j + e / PPRW;
                    const int64_t dst = ((t0 + u) % R) * D + (e % PPRW) * EPP;
                    *reinterpret_cast<uint4 *>(rk + dst) = kk[q];
                    *reinterpret_cast<uint4 *>(rv + dst) = vv[q];
                }
            }
        }
        __syncthreads();  // the next boundary reads these ring rows
        j = jend;
    }
    // keys rotated at their positions (angles in fp64), a batch of pairs per thread. Only the
    // chunk's last R tokens stay in the ring, and the boundary updates read the raw rows only,
    // so the rotation covers those tokens alone.
    const int64_t u0 = len > R ? len - R : 0;
    constexpr int RB = 8;
    const int64_t npr = (len - u0) * (D / 2);
    for (int64_t e0 = 0; e0 < npr; e0 += (int64_t)kDecThreads * RB) {
        float ka[RB], kb[RB];
#pragma unroll
        for (int q = 0; q < RB; ++q) {
            const int64_t e = min(e0 + tid + (int64_t)kDecThreads * q, npr - 1);
            const int64_t u = u0 + e / (D / 2);
            const int m = (int)(e % (D / 2));
            ka[q] = to_f32<T>(kh[u * D + m]);
            kb[q] = to_f32<T>(kh[u * D + m + D / 2]);
        }
#pragma unroll
        for (int q = 0; q < RB; ++q) {
            const int64_t e = e0 + tid + (int64_t)kDecThreads * q;
            if (e < npr) {
                const int64_t u = u0 + e / (D / 2);
                const int m = (int)(e % (D / 2));
                const double theta = pow((double)p.rope_base, -2.0 * (double)m / (double)D);
                const double ang = (double)(t0 + u) * theta;
                const float c = (float)cos(ang), sn = (float)sin(ang);
                const int64_t slot = (t0 + u) % R;
                rkr[slot * D + m] = rot_store<RT>(ka[q] * c - kb[q] * sn);
                rkr[slot * D + m + D / 2] = rot_store<RT>(kb[q] * c + ka[q] * sn);
            }
        }
    }
    if (tid == 0) {
        hdr[0] = t0 + len;
        hdr[1] = blk;
    }
}

hipError_t launch_decode_init(void *state, const KParams &p, const DecodeLayout &L, int n_seq, hipStream_t st) {
    hipLaunchKernelGGL(decode_init_kernel, dim3((unsigned)(n_seq * p.H)), dim3(256), 0, st, (char *)state, p, L, n_seq,
                       p.dtype);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t prefill_t(void *state, int seq, const void *kp, const void *vp, int64_t Lp, const Work &w,
                            const KParams &p, const DecodeLayout &L, hipStream_t st) {
    // 32 parts per head: the record's copies spread over 32 H work-groups
    hipLaunchKernelGGL((decode_prefill_kernel<T, D>), dim3(32u, (unsigned)p.H), dim3(256), 0, st, (char *)state, seq,
                       (const T *)kp, (const T *)vp, Lp, w.kbar, w.amax, w.pool, p, L);
    return hipGetLastError();
}

hipError_t launch_decode_prefill(void *state, int seq, const void *kp, const void *vp, int64_t Lp, const Work &w,
                                 const KParams &p, const DecodeLayout &L, hipStream_t st) {
    if (p.dtype == FSL_BF16)
        return p.d == 64 ? prefill_t<uint16_t, 64>(state, seq, kp, vp, Lp, w, p, L, st)
                         : prefill_t<uint16_t, 128>(state, seq, kp, vp, Lp, w, p, L, st);
    return p.d == 64 ? prefill_t<float, 64>(state, seq, kp, vp, Lp, w, p, L, st)
                     : prefill_t<float, 128>(state, seq, kp, vp, Lp, w, p, L, st);
}

template <typename T, int D>
static hipError_t step_t(void *state, const void *q, const void *k, const void *v, void *out, int32_t *sel_out,
                         int n_seq, const KParams &p, const DecodeLayout &L, hipStream_t st) {
    const size_t kb_lds = D == 64 ? ((size_t)L.PW * D * 4 + 1023) / 1024 * 1024 : 0;
    hipLaunchKernelGGL((decode_step_kernel<T, D>), dim3((unsigned)(n_seq * p.H)), dim3(kDecThreads), kb_lds, st,
                       (char *)state, (const T *)q, (const T *)k, (const T *)v, out, sel_out, p, L);
    return hipGetLastError();
}

hipError_t launch_decode_step(void *state, const void *q, const void *k, const void *v, void *out, int32_t *sel_out,
                              int n_seq, const KParams &p, const DecodeLayout &L, hipStream_t st) {
    if (p.dtype == FSL_BF16)
        return p.d == 64 ? step_t<uint16_t, 64>(state, q, k, v, out, sel_out, n_seq, p, L, st)
                         : step_t<uint16_t, 128>(state, q, k, v, out, sel_out, n_seq, p, L, st);
    return p.d == 64 ? step_t<float, 64>(state, q, k, v, out, sel_out, n_seq, p, L, st)
                     : step_t<float, 128>(state, q, k, v, out, sel_out, n_seq, p, L, st);
}

template <typename T, int D>
static hipError_t append_t(void *state, int seq0, int n, const void *k, const void *v, int64_t len, const KParams &p,
                           const DecodeLayout &L, hipStream_t st) {
    hipLaunchKernelGGL((decode_append_kernel<T, D>), dim3((unsigned)(n * p.H)), dim3(kDecThreads), 0, st,
                       (char *)state, seq0, (const T *)k, (const T *)v, len, p, L);
    return hipGetLastError();
}

hipError_t launch_decode_append(void *state, int seq0, int n, const void *k, const void *v, int64_t len,
                                const KParams &p, const DecodeLayout &L, hipStream_t st) {
    if (p.dtype == FSL_BF16)
        return p.d == 64 ? append_t<uint16_t, 64>(state, seq0, n, k, v, len, p, L, st)
                         : append_t<uint16_t, 128>(state, seq0, n, k, v, len, p, L, st);
    return p.d == 64 ? append_t<float, 64>(state, seq0, n, k, v, len, p, L, st)
                     : append_t<float, 128>(state, seq0, n, k, v, len, p, L, st);
}

}  // namespace fsl

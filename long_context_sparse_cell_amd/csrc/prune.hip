// Norm prune: per query block, the W most recent eligible cells plus the P
// older eligible cells of largest max key norm, ties to the lower index
// (FreeSolo digest, core method and step 4; ai.info summary, methodology:
// a pool of at most P+W cells that changes only at block boundaries).
//
// The older set of block b is the prefix [0, m_b) of the cell sequence, so
// its top-P is a prefix top-P. top-64 is associative (top(A u B) =
// top(top(A) u top(B))), which gives an O(C) scan in four wave-level passes,
// every list a best-first sorted run of 64 (key, index) entries, one per lane:
//   1. chunk sort     : each chunk of 64 cells sorted (bitonic, in registers)
//   2. local prefixes : within groups of 16 chunks, exclusive prefix top-64
//   3. group prefixes : exclusive prefix top-64 over groups (one wave per head)
//   4. block pools    : top-64 of [0, m_b) = merge(group prefix, local prefix,
//                       the sorted part of the boundary chunk below m_b); the
//                       first P are the kept cells. Indices are then sorted
//                       ascending and the recent cells appended.
// P <= 64 is required (the host checks it).
#include <climits>

#include "fsl_internal.h"

namespace fsl {

__device__ __forceinline__ void load_list(const KParams &p, const Work &w, int64_t list, float &a, int &idx) {
    const int lane = threadIdx.x & 63;
    a = w.scan_a[list * kChunk + lane];
    idx = w.scan_i[list * kChunk + lane];
}

__device__ __forceinline__ void store_list(const KParams &p, const Work &w, int64_t list, float a, int idx) {
    const int lane = threadIdx.x & 63;
    w.scan_a[list * kChunk + lane] = a;
    w.scan_i[list * kChunk + lane] = idx;
}

__global__ __launch_bounds__(256) void prune_chunk_sort(const float *__restrict__ amax, Work w, KParams p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t k = (int64_t)blockIdx.x * 4 + wave;
    const int h = blockIdx.y;
    if (k >= p.nchunk) return;
    const int64_t c = k * kChunk + lane;
    float a = c < p.C ? amax[(int64_t)h * p.C + c] : -INFINITY;
    int idx = c < p.C ? (int)c : INT_MAX;
    wave_sort_best_first(a, idx);
    store_list(p, w, scan_chunk(p, h, k), a, idx);
}

__global__ __launch_bounds__(256) void prune_local_scan(Work w, KParams p) {
    const int wave = threadIdx.x >> 6;
    const int64_t g = (int64_t)blockIdx.x * 4 + wave;
    const int h = blockIdx.y;
    if (g >= p.nsg) return;
    float a = -INFINITY;
    int idx = INT_MAX;
    for (int j = 0; j < kGroup; ++j) {
        const int64_t k = g * kGroup + j;
        if (k > p.nchunk) break;
        store_list(p, w, scan_prefix(p, h, k), a, idx);
        if (k < p.nchunk) {
            float ba;
            int bi;
            load_list(p, w, scan_chunk(p, h, k), ba, bi);
            wave_merge_top(a, idx, ba, bi);
        }
    }
    store_list(p, w, scan_total(p, h, g), a, idx);
}

__global__ __launch_bounds__(64) void prune_group_scan(Work w, KParams p) {
    const int h = blockIdx.x;
    float a = -INFINITY;
    int idx = INT_MAX;
    for (int64_t g = 0; g < p.nsg; ++g) {
        store_list(p, w, scan_gprefix(p, h, g), a, idx);
        float ba;
        int bi;
        load_list(p, w, scan_total(p, h, g), ba, bi);
        wave_merge_top(a, idx, ba, bi);
    }
}

__global__ __launch_bounds__(256) void prune_block_pool(int32_t *__restrict__ pool, Work w, KParams p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t b = (int64_t)blockIdx.x * 4 + wave;
    const int h = blockIdx.y;
    if (b >= p.nblk) return;
    const int64_t nb = eligible_cells(p, b);
    const int64_t m = nb > p.W ? nb - p.W : 0;
    const int ntop = (int)min((int64_t)p.P, m);

    float a = -INFINITY;
    int idx = INT_MAX;
    if (ntop > 0) {
        const int64_t k = m / kChunk, g = k / kGroup;
        load_list(p, w, scan_gprefix(p, h, g), a, idx);
        float ba;
        int bi;
        load_list(p, w, scan_prefix(p, h, k), ba, bi);
        wave_merge_top(a, idx, ba, bi);
        if (k < p.nchunk) {
            load_list(p, w, scan_chunk(p, h, k), ba, bi);
            if (bi >= m) { ba = -INFINITY; bi = INT_MAX; }
            wave_sort_best_first(ba, bi);
            wave_merge_top(a, idx, ba, bi);
        }
    }
    // kept cells sit in lanes [0, ntop); sort their indices ascending
    float za = 0.0f;
    int key = lane < ntop ? idx : INT_MAX;
    wave_sort_best_first(za, key);

    int32_t *out = pool + ((int64_t)h * p.nblk + b) * p.PW;
    const int64_t nrec = nb - m;
    for (int t = lane; t < p.PW; t += 64) {
        int32_t val;
        if (t < ntop) val = key;
        else if (t < ntop + nrec) val = (int32_t)(m + (t - ntop));
        else val = -1;
        out[t] = val;
    }
}

hipError_t launch_prune(const float *amax, int32_t *pool, const Work &w, const KParams &p, hipStream_t st) {
    if (p.nblk == 0) return hipSuccess;
    if (p.P > 0 && p.C > 0) {
        hipLaunchKernelGGL(prune_chunk_sort, dim3((unsigned)((p.nchunk + 3) / 4), (unsigned)p.H), dim3(256), 0, st,
                           amax, w, p);
        hipLaunchKernelGGL(prune_local_scan, dim3((unsigned)((p.nsg + 3) / 4), (unsigned)p.H), dim3(256), 0, st, w, p);
        hipLaunchKernelGGL(prune_group_scan, dim3((unsigned)p.H), dim3(64), 0, st, w, p);
    }
    Work wk = w;
    if (!(p.P > 0 && p.C > 0)) { wk.scan_a = nullptr; wk.scan_i = nullptr; }
    hipLaunchKernelGGL(prune_block_pool, dim3((unsigned)((p.nblk + 3) / 4), (unsigned)p.H), dim3(256), 0, st, pool,
                       wk, p);
    return hipGetLastError();
}

}  // namespace fsl

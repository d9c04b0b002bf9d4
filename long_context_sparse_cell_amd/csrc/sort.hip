// Stable LSD radix sort of (key, value) pairs of 32-bit integers, 8 bits per
// pass. The backward pass uses it to list, for every cell, the queries that
// selected it in query order (keys = cells, values = queries, input in query
// order; a stable sort keeps that order inside each cell).
//
// One pass over digit bits [shift, shift + 8):
//   sort_hist_kernel     per chunk (sort_plan sizes them): digit counts, stored
//                        digit-major (hist[digit][chunk]) so that one exclusive
//                        scan of hist gives every (digit, chunk) its first slot
//   sort_scan_kernel     exclusive scan of each 1024-entry block of hist, with the
//                        block's total
//   sort_scan_top_kernel exclusive scan of the block totals (one work-group)
// launch_scan_u32 runs the last two on their own for other users of a block scan.
//   sort_scatter_kernel  one wave per chunk walks it 64 elements at a time; a lane's
//                        slot is its digit's first slot, plus the chunk's elements of
//                        that digit already placed, plus the lanes below it with the
//                        same digit (found with eight ballots)
#include "fsl_internal.h"

namespace fsl {

namespace {
constexpr int kRadix = kSortRadix;
constexpr int kScanBlock = kSortScanBlock;
constexpr int kScanTopMax = kSortScanTopMax;
}  // namespace

__global__ __launch_bounds__(256) void sort_hist_kernel(const uint32_t *__restrict__ keys, int64_t n, int chunk,
                                                        int shift, uint32_t *__restrict__ hist, int nch) {
    __shared__ uint32_t cnt[kRadix];
    cnt[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t e0 = (int64_t)blockIdx.x * chunk;
    const int64_t e1 = min(n, e0 + chunk);
    for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) atomicAdd(&cnt[(keys[e] >> shift) & 255u], 1u);
    __syncthreads();
    hist[(int64_t)threadIdx.x * nch + blockIdx.x] = cnt[threadIdx.x];
}

// exclusive scan inside each block of kScanBlock entries; totals[block] = its sum
__global__ __launch_bounds__(256) void sort_scan_kernel(uint32_t *__restrict__ hist, int64_t m,
                                                        uint32_t *__restrict__ totals) {
    __shared__ uint32_t s_w[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t base = (int64_t)blockIdx.x * kScanBlock + 4 * tid;
    uint32_t x[4], sum = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = base + j < m ? hist[base + j] : 0u;
        sum += x[j];
    }
    uint32_t inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) s_w[wave] = inc;
    __syncthreads();
    uint32_t wbase = 0u;
    for (int w2 = 0; w2 < wave; ++w2) wbase += s_w[w2];
    uint32_t run = wbase + inc - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (base + j < m) hist[base + j] = run;
        run += x[j];
    }
    if (tid == 255) totals[blockIdx.x] = wbase + inc;
}

// exclusive scan of the block totals in place, kScanTopMax at a time with the
// running sum carried from one piece to the next
__global__ __launch_bounds__(1024) void sort_scan_top_kernel(uint32_t *__restrict__ totals, int nb) {
    __shared__ uint32_t s_w[16];
    __shared__ uint32_t s_carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int PER = kScanTopMax / 1024;
    if (tid == 0) s_carry = 0u;
    for (int base = 0; base < nb; base += kScanTopMax) {
        uint32_t x[PER], sum = 0u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = base + PER * tid + j;
            x[j] = e < nb ? totals[e] : 0u;
            sum += x[j];
        }
        uint32_t inc = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (lane == 63) s_w[wave] = inc;
        __syncthreads();
        uint32_t run = s_carry + inc - sum;
        uint32_t all = 0u;
        for (int w2 = 0; w2 < 16; ++w2) {
            if (w2 < wave) run += s_w[w2];
            all += s_w[w2];
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = base + PER * tid + j;
            if (e < nb) totals[e] = run;
            run += x[j];
        }
        __syncthreads();  // every thread has read s_w and s_carry
        if (tid == 0) s_carry += all;
        __syncthreads();
    }
}

__global__ __launch_bounds__(64) void sort_scatter_kernel(const uint32_t *__restrict__ kin,
                                                          const uint32_t *__restrict__ vin,
                                                          uint32_t *__restrict__ kout, uint32_t *__restrict__ vout,
                                                          int64_t n, int chunk, int shift,
                                                          const uint32_t *__restrict__ hist,
                                                          const uint32_t *__restrict__ totals, int nch) {
    __shared__ uint32_t placed[kRadix];  // this chunk's elements of each digit already written
    const int lane = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kRadix / 64; ++j) placed[lane + 64 * j] = 0u;
    const int64_t e0 = (int64_t)blockIdx.x * chunk;
    const int64_t e1 = min(n, e0 + chunk);
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t s = e0; s < e1; s += 64) {
        const int64_t e = s + lane;
        const bool ok = e < e1;
        const uint32_t key = ok ? kin[e] : 0u;
        const uint32_t val = ok ? vin[e] : 0u;
        const uint32_t dg = (key >> shift) & 255u;
        // lanes holding the same digit: agree with this lane on all eight bits
        uint64_t same = __ballot(ok);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const uint64_t b = __ballot(ok && ((dg >> bit) & 1u));
            same &= ((dg >> bit) & 1u) ? b : ~b;
        }
        if (ok) {
            const int64_t slot = (int64_t)dg * nch + blockIdx.x;
            const uint32_t at = hist[slot] + totals[slot / kScanBlock] + placed[dg] + (uint32_t)__popcll(same & below);
            kout[at] = key;
            vout[at] = val;
        }
        // the highest lane of each digit group advances that digit's count (reads above
        // were issued first: one wave's LDS accesses complete in order)
        if (ok && (same >> lane) == 1ull) placed[dg] += (uint32_t)__popcll(same);
        __builtin_amdgcn_wave_barrier();
    }
}

// Exclusive scan of m words in place, in blocks of kScanBlock: afterwards the
// prefix of element i is data[i] + totals[i / kScanBlock].
hipError_t launch_scan_u32(uint32_t *data, int64_t m, uint32_t *totals, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    const int64_t nb = (m + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(sort_scan_kernel, dim3((unsigned)nb), dim3(256), 0, st, data, m, totals);
    hipLaunchKernelGGL(sort_scan_top_kernel, dim3(1), dim3(1024), 0, st, totals, (int)nb);
    return hipGetLastError();
}

// Sorts (keys, vals) by the low `bits` bits of the keys, stably; the result ends in
// (keys, vals) after an even number of passes, in (ktmp, vtmp) after an odd one, and
// *in_tmp says which.
hipError_t launch_sort_pairs(uint32_t *keys, uint32_t *vals, uint32_t *ktmp, uint32_t *vtmp, uint32_t *hist,
                             uint32_t *totals, int64_t n, int bits, bool *in_tmp, hipStream_t st) {
    *in_tmp = false;
    if (n <= 0) return hipSuccess;
    int chunk, nch;
    sort_plan(n, chunk, nch);
    const int64_t m = (int64_t)kRadix * nch;
    const int nb = (int)((m + kScanBlock - 1) / kScanBlock);
    uint32_t *ka = keys, *va = vals, *kb = ktmp, *vb = vtmp;
    for (int shift = 0; shift < bits; shift += 8) {
        hipLaunchKernelGGL(sort_hist_kernel, dim3((unsigned)nch), dim3(256), 0, st, ka, n, chunk, shift, hist, nch);
        hipLaunchKernelGGL(sort_scan_kernel, dim3((unsigned)nb), dim3(256), 0, st, hist, m, totals);
        hipLaunchKernelGGL(sort_scan_top_kernel, dim3(1), dim3(1024), 0, st, totals, nb);
        hipLaunchKernelGGL(sort_scatter_kernel, dim3((unsigned)nch), dim3(64), 0, st, ka, va, kb, vb, n, chunk,
                           shift, hist, totals, nch);
        uint32_t *t = ka; ka = kb; kb = t;
        t = va; va = vb; vb = t;
        *in_tmp = !*in_tmp;
    }
    return hipGetLastError();
}

}  // namespace fsl

// Compact work list shared by the decode kernels.
//
// A launch sized by the longest context leaves most (sequence, partition)
// slots empty when lengths are ragged, and on this chip every empty
// workgroup still costs a dispatch.  Instead the grid is sized to what the
// GPU holds at once and each workgroup walks its share of the LIVE items
// only: for a window of up to kWindow sequences every workgroup builds, in
// LDS, the exclusive prefix sum of partitions per sequence, and item
// w = unit + num_units * gp names unit `unit` (a KV head or a query head) of
// the gp-th live partition of the window.  Workgroup b takes items b,
// b + gridDim.x, ... so with num_units and gridDim.x multiples of 8 one unit
// always runs on the same XCD.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {

constexpr int kWindow = 2048;       // sequences per work-list window

__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

__device__ __forceinline__ int parts_of(int ctx, int part_tokens) {
    return ctx == 0 ? 1 : (ctx + part_tokens - 1) / part_tokens;
}

// pref[0..n] = exclusive prefix of partitions over sequences s0..s0+n-1;
// returns pref[n].  `scan` holds NT ints.  Ends with a barrier.
template <int NT>
__device__ int build_prefix(const DecodeArgs& a, int s0, int n, int32_t* pref, int32_t* scan) {
    const int per = (n + NT - 1) / NT;
    const int beg = min(n, (int)threadIdx.x * per);
    const int end = min(n, beg + per);
    int sum = 0;
    for (int i = beg; i < end; ++i) sum += parts_of(clamp_ctx(a.ctx_lens[s0 + i], a.ctx_cap), a.part_tokens);
    scan[threadIdx.x] = sum;
    __syncthreads();
#pragma unroll 1
    for (int off = 1; off < NT; off <<= 1) {
        const int v = (int)threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
        __syncthreads();
        scan[threadIdx.x] += v;
        __syncthreads();
    }
    int run = scan[threadIdx.x] - sum;
    for (int i = beg; i < end; ++i) {
        pref[i] = run;
        run += parts_of(clamp_ctx(a.ctx_lens[s0 + i], a.ctx_cap), a.part_tokens);
    }
    if (threadIdx.x == NT - 1) pref[n] = scan[NT - 1];
    __syncthreads();
    return pref[n];
}

// largest i in [0, n) with pref[i] <= gp (pref strictly covers [0, pref[n]))
__device__ __forceinline__ int locate(const int32_t* pref, int n, int gp) {
    int lo = 0, hi = n;                 // invariant: pref[lo] <= gp < pref[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= gp) lo = mid; else hi = mid;
    }
    return lo;
}

// Block-table entries of an item's first table segment, loaded by the
// workgroup's threads together with the item's other first loads (length,
// query) so that starting an item costs one memory round trip, then stored to
// LDS once the length is known.  Entries are read at indices clamped to the
// span, which lies inside the sequence's table row.
template <int NT, int CAP>
struct TablePrefetch {
    static constexpr int TP = (CAP + NT - 1) / NT;
    int32_t v[TP];
    __device__ __forceinline__ void issue(const int32_t* trow, int b_first, int span) {
#pragma unroll
        for (int k = 0; k < TP; ++k) {
            const int i = k * NT + (int)threadIdx.x;
            v[k] = trow[b_first + min(i, span - 1)];
        }
    }
    __device__ __forceinline__ void store(int32_t* tbl, int n, int num_blocks) const {
#pragma unroll
        for (int k = 0; k < TP; ++k) {
            const int i = k * NT + (int)threadIdx.x;
            if (i < n) tbl[i] = (v[k] >= 0 && v[k] < num_blocks) ? v[k] : -1;
        }
    }
};

// Table entries [b_first, b_first + span) hold every block a partition that
// starts at token t0 can touch (bounded by the table row and by CAP).
__device__ __forceinline__ int table_span(const DecodeArgs& a, int t0, int cap) {
    const int b_first = t0 >> a.log2_bs;
    const int b_last = (int)(((int64_t)t0 + a.part_tokens + (1 << a.log2_bs) - 1) >> a.log2_bs);
    return max(1, min(min(cap, a.max_blocks - b_first), b_last - b_first));
}

// Grid for a persistent decode kernel: no more workgroups than items, no
// more than the device holds at once, a multiple of 8 when that is possible.
int64_t persistent_grid(const void* kernel, int threads, int64_t max_items);

}  // namespace pa

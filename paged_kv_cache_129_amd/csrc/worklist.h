// How the decode kernels share out their work.
//
// A "segment" is the context of one (sequence, unit), where a unit is what
// one work item computes for: one query head (per-head kernel), or one KV head
// with all (or, for very large groups, an equal share) of the query heads that
// read it (matrix-core kernel).  Items are taken by
// "workers": single wavefronts (each streams its own items, so one
// wavefront's wait for memory never idles its neighbours).  Wavefront w of
// workgroup b is worker b * NW + w (measured: spreading consecutive workers
// over workgroups instead is no faster for ragged batches and slower for
// uniform ones).  Launches are persistent: the grid is what the GPU holds at
// once, and the workers walk the live work only, since on this chip every
// dispatched workgroup costs time even when it has nothing to do.  Sequences are taken in windows of kWindow,
// whose metadata every workgroup stages in LDS.  Two schedules:
//
// * Partitions (partition_size >= 0): a segment is cut into partitions of
//   part_tokens tokens (one partition for a single pass).  Every workgroup
//   builds the same list in LDS — first every partition that is not a
//   sequence's last (all full length), then the last partitions grouped into
//   kClasses length classes, longest class first (a stable counting sort) —
//   and list position k (unit k mod units of partition k / units) goes to
//   worker k mod W in even rounds and W-1-(k mod W) in odd ones (W workers).
//
// * Balanced (partition_size < 0): the window's segments, each padded to a
//   multiple of kSplitAlign tokens plus seg_cost tokens that stand for the
//   fixed cost of starting an item (they hold no tokens; the kernel sets it),
//   are laid end to end
//   and cut into one equal range per worker, so every worker gets the same
//   cost whatever the length mix, and every CU and XCD the same load.  A
//   worker that holds all of a segment's tokens writes its result straight to
//   the output; when a range boundary cuts the tokens, each piece becomes a
//   partial record — slot 0 for the segment the worker's range starts in,
//   slot 1 for the one it ends in — and the reduction kernel merges them.
//   Pieces of cost padding alone are skipped.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {

constexpr int kClasses = 8;         // length classes of last partitions
constexpr int kSplitAlign = 16;     // balanced: ranges and padded segments are multiples of this
constexpr int kMinRange = 256;      // balanced: fewest tokens in a worker's range

__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

__device__ __forceinline__ int parts_of(int ctx, int part_tokens) {
    return ctx == 0 ? 1 : (ctx + part_tokens - 1) / part_tokens;
}

// length class of a sequence's last partition: (P*c/8, P*(c+1)/8] -> c
__device__ __forceinline__ int tail_class(int ctx, int part_tokens) {
    const int tail = ctx - (parts_of(ctx, part_tokens) - 1) * part_tokens;
    if (tail <= 0) return 0;
    return min(kClasses - 1, (int)(((int64_t)tail * kClasses - 1) / part_tokens));
}

// tokens of a balanced segment that are run: the context rounded up (an empty
// context still takes one masked chunk, so that its output is written)
__device__ __forceinline__ int64_t split_run(int ctx) {
    return ctx <= 0 ? kSplitAlign : ((int64_t)ctx + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
}
// length of a balanced segment in the range space
__device__ __forceinline__ int64_t split_len(int ctx, int seg_cost) { return split_run(ctx) + seg_cost; }

// balanced: tokens per worker range for T padded tokens over `grid` workers
// x / y for 0 <= x and 0 < y, in 32 bits when both fit (the common case)
__device__ __forceinline__ int64_t udiv(int64_t x, int64_t y) {
    if (x <= INT32_MAX && y <= INT32_MAX) return (int64_t)((uint32_t)x / (uint32_t)y);
    return x / y;
}

__device__ __forceinline__ int64_t split_range(int64_t T, int64_t grid) {
    int64_t r = udiv(T + grid - 1, grid);
    r = (r + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
    return r < kMinRange ? kMinRange : r;
}

// LDS ints a window's metadata needs (64-bit aligned by the caller)
constexpr int kListInts = 3 * kWindow + 2;

__device__ __forceinline__ uint64_t shfl_up64(uint64_t v, int d) {
    const uint32_t lo = __shfl_up((unsigned)(v & 0xFFFFFFFFu), d, 64);
    const uint32_t hi = __shfl_up((unsigned)(v >> 32), d, 64);
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sums over the workgroup of Q 64-bit values (wavefront
// shuffles, then one exchange of wavefront totals through LDS); `tot` gets the
// workgroup totals.
template <int NT, int Q>
__device__ __forceinline__ void block_scan(uint64_t v[Q], uint64_t tot[Q]) {
    constexpr int NW = NT / 64;
    __shared__ uint64_t wsum[Q][NW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint64_t u = shfl_up64(v[q], d);
            if (lane >= d) v[q] += u;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int q = 0; q < Q; ++q) wsum[q][wave] = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        uint64_t before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint64_t x = wsum[q][w];
            before += w < wave ? x : 0;
            all += x;
        }
        v[q] += before;
        tot[q] = all;
    }
}

// Values the whole workgroup shares, moved to scalar registers (values read
// from LDS or reduced across lanes arrive in vector registers otherwise, and
// would occupy them for a whole item).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(x & 0xFFFFFFFF));
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// worker index of wavefront `wave` of this workgroup (NW wavefronts each)
__device__ __forceinline__ int worker_id(int wave, int nw) { return (int)blockIdx.x * nw + wave; }

// One work item: tokens [t0, t1) of unit `unit` of sequence `s`, of a context
// of `ctx` tokens.  `whole`: the item is the entire context and its result is
// final; otherwise the result goes to partial records rec0 + i * rec_stride
// for the unit's heads i.
struct Item {
    int s, unit, t0, t1, ctx;
    bool whole;
    int64_t rec0;
    int rec_stride;
};

// largest i in [0, n) with pref[i] <= x (pref ascending, pref[0] == 0); called
// by all lanes of a wavefront with the same arguments
template <typename T>
__device__ __forceinline__ int locate(const T* pref, int n, T x) {
    // the whole wavefront searches: each pass compares 64 evenly spaced entries
    // at once and keeps the interval after the last one <= x (pref[0] <= x, so
    // lane 0 always qualifies); invariant: pref[lo] <= x, and x < pref[lo + len]
    // if lo + len < n
    const int lane = threadIdx.x & 63;
    int lo = 0, len = n;
    while (len > 1) {
        const int step = (len + 63) >> 6;
        const int i = lane * step;
        const bool le = i < len && pref[lo + i] <= x;
        const uint64_t b = __builtin_amdgcn_ballot_w64(le);
        const int k = 63 - __builtin_clzll(b);
        lo += k * step;
        len = min(step, len - k * step);
    }
    return lo;
}

// The schedule of one window for one worker (worker ids and counts are the
// same in all lanes of a worker).  `build`, called by the whole workgroup
// (starts and ends with a barrier), stages the window's metadata in `lds`
// (kListInts ints, 64-bit aligned); `next` yields the worker's items in turn.
// `lead`: the lane that publishes the worker's range descriptor.
template <int NT>
struct Schedule {
    const int32_t* ctx;     // [n] clamped context lengths
    int s0, n, units, G;    // G: partial-record slots per unit
    // partitions
    const int32_t* pref;    // [n+1] exclusive prefix of non-last partitions
    const int32_t* order;   // [n] sequences by last-partition class, longest first
    int full;
    int64_t items, round;
    // balanced
    const int64_t* spref;   // [n+1] exclusive prefix of padded segment lengths
    int64_t g, gend, range;
    int64_t pg, pt0, pL;    // the piece located at range position pg (reused by next)
    int psl, punit;
    int worker, workers;

    __device__ void build(const DecodeArgs& a, int s0_, int n_, int units_, int32_t* lds,
                          int worker_, int workers_, bool lead) {
        s0 = s0_;
        n = n_;
        units = units_;
        worker = uni(worker_);
        workers = workers_;
        G = a.unit_heads;
        int32_t* ctxw = lds;
        const int per = (n + NT - 1) / NT;
        const int beg = min(n, (int)threadIdx.x * per);
        const int end = min(n, beg + per);
        __syncthreads();                    // the previous window's metadata is no longer read
        if (a.part_tokens < 0) {            // balanced
            int64_t* sp = reinterpret_cast<int64_t*>(lds + kWindow);
            uint64_t own[1] = {0}, tot[1];
            for (int i = beg; i < end; ++i) {
                const int c = clamp_ctx(a.ctx_lens[s0 + i], a.ctx_cap);
                ctxw[i] = c;
                own[0] += (uint64_t)split_len(c, a.seg_cost);
            }
            uint64_t inc[1] = {own[0]};
            block_scan<NT, 1>(inc, tot);
            int64_t run = (int64_t)(inc[0] - own[0]);
            for (int i = beg; i < end; ++i) {
                sp[i] = run;
                run += split_len(ctxw[i], a.seg_cost);
            }
            if (threadIdx.x == NT - 1) sp[n] = (int64_t)tot[0];
            spref = sp;
            ctx = ctxw;
            const int64_t T = uni((int64_t)tot[0] * units);
            // with less than kMinRange tokens per worker, only some workers get a
            // range: a whole number per SIMD where there are enough (workers are
            // block-major and a workgroup's wavefronts sit on different SIMDs, so
            // the first k * SIMDs workers put k on every SIMD), else one each
            int64_t active = workers;
            if (T < (int64_t)workers * kMinRange) {
                const int64_t simds = a.simds > 0 ? a.simds : 1;
                active = T / ((int64_t)kMinRange * simds) * simds;
                if (active == 0) active = (T + kMinRange - 1) / kMinRange;
                active = max((int64_t)1, min(active, (int64_t)workers));
            }
            range = uni(split_range(T, active));
            g = min(T, (int64_t)worker * range);
            gend = min(T, g + range);
            __syncthreads();
            // where this worker's range starts, for the reduction
            // (located by the whole wavefront; the lead lane stores it)
            int64_t w0 = 0, w1 = 0, w2 = 0, w4 = 0;
            pg = -1;
            if (g < gend) {
                piece_at(g, psl, punit, pt0, pL);
                pg = g;
                w0 = (int64_t)(s0 + psl) | ((int64_t)punit << 32);
                w1 = pt0;
                w2 = pL;
                w4 = ctx[psl];
            }
            if (lead) {
                int64_t* d = a.desc + ((int64_t)(s0 / kWindow) * workers + worker) * kDescWords;
                d[0] = w0;
                d[1] = w1;
                d[2] = w2;
                d[3] = range;
                d[4] = w4;
            }
            return;
        }
        int32_t* pr = lds + kWindow;
        int32_t* ord = lds + 2 * kWindow + 1;
        // per thread: non-last partitions, and the count of each class in 16-bit
        // fields (classes 0-3, then 4-7; a window holds at most kWindow < 2^16)
        uint64_t own[3] = {0, 0, 0};
        for (int i = beg; i < end; ++i) {
            const int c = clamp_ctx(a.ctx_lens[s0 + i], a.ctx_cap);
            ctxw[i] = c;
            own[0] += (uint64_t)(parts_of(c, a.part_tokens) - 1);
            const int k = tail_class(c, a.part_tokens);
            own[1 + (k >> 2)] += (uint64_t)1 << (16 * (k & 3));
        }
        uint64_t inc[3] = {own[0], own[1], own[2]}, tot[3];
        block_scan<NT, 3>(inc, tot);
        auto field = [](const uint64_t* v, int k) -> int {
            return (int)((v[1 + (k >> 2)] >> (16 * (k & 3))) & 0xFFFFu);
        };
        uint64_t ex[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) ex[q] = inc[q] - own[q];
        // this thread's first slot in each class; classes laid out longest first
        int nxt[kClasses];
        int acc = 0;
#pragma unroll
        for (int k = kClasses - 1; k >= 0; --k) {
            nxt[k] = acc + field(ex, k);
            acc += field(tot, k);
        }
        int run_full = (int)ex[0];
        for (int i = beg; i < end; ++i) {
            const int c = ctxw[i];
            pr[i] = run_full;
            run_full += parts_of(c, a.part_tokens) - 1;
            const int k = tail_class(c, a.part_tokens);
            int slot = 0;
#pragma unroll
            for (int q = 0; q < kClasses; ++q)
                if (q == k) slot = nxt[q]++;
            ord[slot] = i;
        }
        full = uni((int)tot[0]);
        if (threadIdx.x == NT - 1) pr[n] = full;
        pref = pr;
        order = ord;
        ctx = ctxw;
        items = (int64_t)(full + n) * units;
        round = 0;
        __syncthreads();
    }

    // balanced: the segment holding padded token g of the window's range space,
    // and g's offset t0 in it
    __device__ __forceinline__ void piece_at(int64_t g_, int& sl, int& unit, int64_t& t0,
                                             int64_t& L) const {
        sl = locate<int64_t>(spref, n, udiv(g_, units));
        const int64_t off = g_ - spref[sl] * units;
        L = spref[sl + 1] - spref[sl];
        unit = (int)udiv(off, L);
        t0 = off - unit * L;
    }

    __device__ bool next(const DecodeArgs& a, Item& it) {
        if (a.part_tokens < 0) {            // balanced
            while (g < gend) {
                int sl, unit;
                int64_t t0, L;
                if (g == pg) {              // the range's first piece, located by build
                    sl = psl;
                    unit = punit;
                    t0 = pt0;
                    L = pL;
                } else {
                    piece_at(g, sl, unit, t0, L);
                }
                const int64_t len = min(L - t0, gend - g);
                const bool first = g == (int64_t)worker * range;
                const int c = uni(ctx[sl]);
                g = uni(g + len);
                const int64_t run = split_run(c);
                if (t0 >= run) continue;    // cost padding only: nothing to run, no record
                const int64_t win = s0 / kWindow;
                it.s = uni(s0 + sl);
                it.unit = uni(unit);
                it.ctx = c;
                it.t0 = uni((int)t0);
                it.t1 = uni((int)max(t0, min((int64_t)c, t0 + len)));
                it.whole = uni((int)(t0 == 0 && t0 + len >= run)) != 0;
                it.rec0 = ((win * workers + worker) * 2 + (first ? 0 : 1)) * G;
                it.rec_stride = 1;
                return true;
            }
            return false;
        }
        const int64_t k = round * workers + ((round & 1) ? workers - 1 - worker : worker);
        if (k >= items) return false;
        ++round;
        const int unit = (int)(k % units);
        const int gp = (int)(k / units);
        int sl, part;
        if (gp < full) {
            sl = locate<int32_t>(pref, n, gp);
            part = gp - pref[sl];
        } else {
            sl = order[gp - full];
            part = parts_of(ctx[sl], a.part_tokens) - 1;
        }
        sl = uni(sl);
        part = uni(part);
        it.s = s0 + sl;
        it.unit = unit;
        it.ctx = uni(ctx[sl]);
        it.t0 = part * a.part_tokens;
        it.t1 = min(it.ctx, it.t0 + a.part_tokens);
        it.whole = parts_of(it.ctx, a.part_tokens) == 1;
        const int64_t head0 = (int64_t)(unit / a.units_per_kv) * (a.num_heads / a.num_kv_heads) +
                              (int64_t)(unit % a.units_per_kv) * a.unit_heads;
        it.rec0 = ((int64_t)it.s * a.num_heads + head0) * a.num_parts + part;
        it.rec_stride = a.num_parts;
        return true;
    }
};

// Block-table entries of an item's first table segment, loaded by the
// workgroup's threads together with the item's other first loads (query) so
// that starting an item costs one memory round trip, then stored to LDS.
// Entries are read at indices clamped to the span and to the table row.
template <int NT, int CAP>
struct TablePrefetch {
    static constexpr int TP = (CAP + NT - 1) / NT;
    int32_t v[TP];
    // `t`: this thread's index among the NT threads that stage the table
    __device__ __forceinline__ void issue(const int32_t* trow, int b_first, int span,
                                          int max_blocks, int t) {
#pragma unroll
        for (int k = 0; k < TP; ++k) {
            const int i = k * NT + t;
            v[k] = trow[min(b_first + min(i, span - 1), max_blocks - 1)];
        }
    }
    // returns whether this thread stored an entry that names no block
    __device__ __forceinline__ bool store(int32_t* tbl, int n, int num_blocks, int t) const {
        bool bad = false;
#pragma unroll
        for (int k = 0; k < TP; ++k) {
            const int i = k * NT + t;
            if (i < n) {
                const bool ok = v[k] >= 0 && v[k] < num_blocks;
                tbl[i] = ok ? v[k] : -1;
                bad |= !ok;
            }
        }
        return bad;
    }
};

// Table entries [t0 / bs, that + span) hold every block that tokens [t0, t1)
// touch (bounded by the table row and by CAP).
__device__ __forceinline__ int table_span(const DecodeArgs& a, int t0, int t1, int cap) {
    const int b_first = t0 >> a.log2_bs;
    const int b_last = (int)(((int64_t)t1 + (1 << a.log2_bs) - 1) >> a.log2_bs);
    return max(1, min(min(cap, a.max_blocks - b_first), b_last - b_first));
}

// Grid for a persistent decode kernel: no more workgroups than items, no
// more than the device holds at once, a multiple of 8 when that is possible.
int64_t persistent_grid(const void* kernel, int threads, int64_t max_items);

}  // namespace pa

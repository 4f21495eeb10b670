// paged_attention_decode, matrix-core path for large head groups: more than 16
// (up to 128) query heads per KV head, multi-query attention among them.
//
// When many query heads read one KV head (KV 缓存与分页注意力 §11 后来的做法;
// KV Cache从原理到实战 §5.3), a token's key and value are a few dozen bytes
// while its scores and weights are dozens of numbers: the work is in the
// arithmetic, and a KV head should be fetched and converted once for all of
// its heads.  So a workgroup of eight wavefronts is one worker: per step it
// loads a chunk of KT tokens of the KV head (each thread a 16-byte piece of a
// K or V row, found through the block table, a few chunks ahead in
// registers), widens it once into fp16/bf16 tiles in LDS, and every
// wavefront whose 16-head tile holds heads of the group computes from those
// tiles, 32 tokens at a time:
//   * S^T[token][head] for 32 tokens: two 16-token halves on
//     v_mfma_f32_16x16x32 (K rows read as the A operand, the tile's queries as
//     the B operand);
//   * the online softmax per head column (log2 units; the reference maximum
//     moves only when a score passes it by more than kSlack, and only then are
//     column maxima taken across lanes and the accumulators rescaled);
//   * O^T[d][head] += V^T P^T with K = 32 tokens on one MFMA per 16
//     dimensions: V^T comes from transposing LDS reads, and P^T is the score
//     MFMA's register layout of the two halves side by side (bf16: a high and
//     a low part, so the weights keep ~16 significant bits).
// One barrier per step separates the tile being read from the one being
// written.  Work is shared out by worklist.h with workgroups as workers; a
// worker's pieces of a cut context go to partial records that the reduction
// kernels merge.  An fp8 cache is widened exactly to the query's type, fp16 or
// bf16 (value * 2^-8; the factor is folded into the scales).
#include "kernels.h"
#include "mfma_util.h"
#include "pa_device.h"
#include "worklist.h"

namespace pa {
namespace {

constexpr int kGWaves = 8;                 // wavefronts per workgroup, one 16-head tile each
constexpr int kGThreads = kGWaves * 64;
constexpr int kGTable = 1024;              // block-table entries staged per segment
constexpr float kNegInfG = -__builtin_inff();
constexpr float kSlack = 8.0f;             // log2 units a score may exceed the reference maximum by

// KT tokens per step (64: four 16-token quarters), NS steps' loads in flight,
// MINB workgroups per CU that the register allocation must allow
template <int KVDT, int QDT, int D, int KT, int NS, int MINB>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(MINB * kGWaves / 4)))
void decode_group_kernel(DecodeArgs a) {
    static_assert(KT == 64, "four 16-token quarters per step");
    // MFMA operand type: the cache's, or for an fp8 cache the query's (e4m3 widens
    // exactly to fp16 and to bf16, and a bf16 query keeps its range)
    constexpr int MT = (KVDT == PA_FP8_E4M3) ? QDT : KVDT;
    constexpr int EB = elem_bytes(KVDT);
    constexpr int RB = D * EB;                                   // bytes of a cached row
    constexpr int PPR = RB / 16;                                 // 16-byte pieces per row
    constexpr int KPIECES = KT * PPR;                            // pieces of a chunk's K rows
    constexpr int LPT = (2 * KPIECES + kGThreads - 1) / kGThreads;   // pieces per thread
    constexpr int HPP = 16 / EB;                                 // numbers per piece
    // LDS row strides (halfs) of the widened tiles.  With rows D + 16 halfs apart
    // (160 or 288 bytes) none of the tile's accesses waits on a bank conflict
    // (measured with the LDS conflict counters): the 16-byte K reads of 16 rows at
    // once, the transposing V reads of 16 rows, the 16-byte row-piece writes of a
    // 16-bit cache, and the two 16-byte halves that a widened fp8 piece writes,
    // provided that pieces whose index has bit 0 different from bit 2 write their
    // upper half first.
    constexpr int LDK = D + 16;
    constexpr int LDV = D + 16;
    constexpr int NC = D / 32;                                   // score MFMAs per 16 tokens
    constexpr int NDT = D / 16;                                  // output d-tiles
    constexpr int NQ = KT / 16;                                  // quarters per step
    constexpr int TILE_HALFS = KT * LDK;
    // merge of quarter results: per (split tile, quarter 1..3) the accumulators of
    // a wavefront, then 16 maxima and 16 sums
    constexpr int SLOT_FLOATS = NDT * 256 + 32;
    constexpr int MERGE_SLOTS = (4 * TILE_HALFS * 2) / (SLOT_FLOATS * 4);

    // both tile buffers of K, then both of V; after an item's last step, the
    // merge slots
    __shared__ __attribute__((aligned(16))) uint16_t tiles[4 * TILE_HALFS];
    __shared__ int32_t tbl[kGTable];
    // the number of the last table slice that holds an entry naming no block
    // (slices are numbered per workgroup; no reset needed)
    __shared__ int32_t tbl_bad;
    __shared__ __attribute__((aligned(8))) int32_t wl_lds[kListInts];
    auto kt = [&](int buf) -> uint16_t* { return tiles + buf * TILE_HALFS; };
    auto vt = [&](int buf) -> uint16_t* { return tiles + (2 + buf) * TILE_HALFS; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane >> 4;
    const int c16 = lane & 15;
    const int G = a.num_heads / a.num_kv_heads;
    const int T = (G + 15) >> 4;                                 // 16-head tiles, 2..8
    const int bs = 1 << a.log2_bs;
    const char* kbase = reinterpret_cast<const char*>(a.k_pool);
    const char* vbase = reinterpret_cast<const char*>(a.v_pool);
    const uint32_t blk_bytes = ((uint32_t)a.num_kv_heads << a.log2_bs) * (uint32_t)RB;

    // Work of a step: T tiles x 4 quarters.  Wavefronts w and w + 4 share a SIMD,
    // so the split keeps the four SIMDs even: a "full" wavefront takes one tile
    // for every token; the four "split" wavefronts of a half of the workgroup
    // take the same one or two tiles, each for one quarter of every step, and
    // merge their results at the item's end (through LDS, in a fixed order).
    //   T = 2: waves 0-3 tile 0, waves 4-7 tile 1, split   (per SIMD: 0.5 tile)
    //   T = 5: waves 0-3 full tiles 0-3, waves 4-7 tile 4, split (1.25)
    //   otherwise wave w full tile w (T = 3, 4: 1; T = 6, 7, 8: 2 on the busiest SIMD)
    constexpr int kSMax = 1;                                     // tiles of a wavefront
    const int n_split_tiles = T == 2 ? 2 : (T == 5 ? 1 : 0);
    const bool wg_splits = n_split_tiles > 0 && 3 * n_split_tiles <= MERGE_SLOTS;
    const int split_base = T >= 4 ? 4 : 0;
    bool full;
    int tile0, ntiles, quarter = 0;
    if (!wg_splits || (wave < 4 && T >= 4)) {
        full = true;
        tile0 = wave;
        ntiles = wave < T ? 1 : 0;
    } else {
        full = false;
        quarter = wave & 3;
        tile0 = T == 2 ? wave >> 2 : 4;
        ntiles = 1;
    }
    const bool computes = ntiles > 0;                            // wavefront-uniform

    Schedule<kGThreads> sch;
    int slice_no = 0;                                            // table slices staged so far
    if (tid == 0) tbl_bad = -1;
    for (int s0 = 0; s0 < a.num_seqs; s0 += kWindow) {
        sch.build(a, s0, min(kWindow, a.num_seqs - s0), a.units, wl_lds, (int)blockIdx.x,
                  (int)gridDim.x, tid == 0);
        // The first block-table slice of the next item is loaded while the current
        // item streams, so that starting an item costs one memory round trip (its
        // first K/V chunks) instead of two.
        TablePrefetch<kGThreads, kGTable> tpre;
        auto prefetch = [&](const Item& it) {
            tpre.issue(a.tables + (int64_t)it.s * a.max_blocks, it.t0 >> a.log2_bs,
                       table_span(a, it.t0, it.t1, kGTable), a.max_blocks, tid);
        };
        Item itm;
        bool have = sch.next(a, itm);
        if (have) prefetch(itm);
        while (have) {
            const Item cur = itm;
            const int s = cur.s;
            const int kvh = cur.unit;                            // one unit per KV head
            const int t0 = cur.t0, t1 = cur.t1;
            const int32_t* trow = a.tables + (int64_t)s * a.max_blocks;

            // B operands of the score MFMA per tile: Q^T[d][head], head dimensions
            // 32 c + 8 j..; state per tile: reference maximum, running sum, O^T
            Op8 qop[kSMax][NC];
            float m[kSMax], l[kSMax];
            f32x4 acc[kSMax][NDT];
#pragma unroll
            for (int ti = 0; ti < kSMax; ++ti) {
                const int hu = 16 * (tile0 + ti) + c16;
                const bool hlive = ti < ntiles && hu < G;
                const char* qrow = reinterpret_cast<const char*>(a.q) +
                                   ((int64_t)s * a.num_heads + kvh * G + (hlive ? hu : 0)) * D *
                                       elem_bytes(QDT);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    static_assert(QDT == MT, "the query is an MFMA operand as it is");
                    Op8 o{{0u, 0u, 0u, 0u}};
                    if (ti < ntiles) {                           // wavefront-uniform
                        const Raw16 r = load16(qrow + (32 * c + 8 * j) * elem_bytes(QDT));
#pragma unroll
                        for (int q = 0; q < 4; ++q) o.w[q] = hlive ? r.w[q] : 0u;
                    }
                    qop[ti][c] = o;
                }
                m[ti] = kNegInfG;
                l[ti] = 0.0f;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc[ti][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }

            const int b_first = t0 >> a.log2_bs;
            const int b_end = (t1 + bs - 1) >> a.log2_bs;
            __syncthreads();                                     // the previous item's table is read
            ++slice_no;
            if (tpre.store(tbl, min(b_end, b_first + kGTable) - b_first, a.num_blocks, tid))
                tbl_bad = slice_no;
            __syncthreads();
            have = sch.next(a, itm);
            if (have) prefetch(itm);
            for (int sb = b_first; sb < b_end; sb += kGTable) {
                const int se = min(b_end, sb + kGTable);
                if (sb != b_first) {                             // later slices of a long item
                    __syncthreads();
                    ++slice_no;
                    for (int i = tid; i < se - sb; i += kGThreads) {
                        const int b = trow[sb + i];
                        const bool ok = b >= 0 && b < a.num_blocks;
                        tbl[i] = ok ? b : -1;
                        if (!ok) tbl_bad = slice_no;
                    }
                    __syncthreads();
                }
                // every block of the slice is valid: steps that end inside the
                // item's tokens have all their tokens present
                const bool slice_ok = uni(tbl_bad) != slice_no;
                const int ts = max(t0, sb << a.log2_bs);
                const int te = min(t1, se << a.log2_bs);
                const int nch = (te - ts + KT - 1) / KT;
                // tokens c0 .. c0 + KT - 1 of the slice that are present (in the item
                // and in a valid block), as a mask (one look at the table per lane)
                auto chunk_mask = [&](int c0) -> uint64_t {
                    const int t = c0 + lane;
                    const bool ok = lane < KT && t < te && tbl[(min(t, te - 1) >> a.log2_bs) - sb] >= 0;
                    return __builtin_amdgcn_ballot_w64(ok);
                };

                // this thread's pieces of chunk n: raw bytes in one register stage
                struct Stage {
                    Raw16 r[LPT];
                    bool ok[LPT];
                };
                auto load_chunk = [&](Stage& st, int n) {
            const int c0 = ts + n * KT;
        #pragma unroll
            for (int k = 0; k < LPT; ++k) {
                const int p = tid + k * kGThreads;
                const bool isv = p >= KPIECES;
                const int pl = isv ? p - KPIECES : p;
                const int row = pl / PPR, col = pl % PPR;
                const int t = c0 + row;
                const bool in = p < 2 * KPIECES && t < te;
                const int blk = in ? tbl[(t >> a.log2_bs) - sb] : -1;
                st.ok[k] = blk >= 0;
                // byte offset: block * (bytes of a block) + this KV head's rows + the
                // token's row + the piece (the launch keeps a block's bytes below
                // 2^32: one 32 x 32 -> 64-bit multiply-add)
                const uint32_t within =
                    ((((uint32_t)kvh << a.log2_bs) + (uint32_t)(t & (bs - 1))) * (uint32_t)RB) + (uint32_t)col * 16u;
                const uint64_t off = blk >= 0 ? (uint64_t)(uint32_t)blk * blk_bytes + within : 0u;
                st.r[k] = load16_stream((isv ? vbase : kbase) + off);
            }
        };
                // widen a stage into tile buffer `buf` (absent rows as zeros)
                auto write_chunk = [&](const Stage& st, int buf) {
#pragma unroll
                    for (int k = 0; k < LPT; ++k) {
                        const int p = tid + k * kGThreads;
                        if (p < 2 * KPIECES) {
                            const bool isv = p >= KPIECES;
                            const int pl = isv ? p - KPIECES : p;
                            const int row = pl / PPR, col = pl % PPR;
                            uint16_t* dst = isv ? vt(buf) + row * LDV + col * HPP
                                                : kt(buf) + row * LDK + col * HPP;
                            if constexpr (KVDT == PA_FP8_E4M3) {
                                // half h0 (8 numbers from raw words 2 h0, 2 h0 + 1) first
                                const int h0 = (col ^ (col >> 2)) & 1;
                                const uint32_t r0 = st.ok[k] ? st.r[k].w[0] : 0u;
                                const uint32_t r1 = st.ok[k] ? st.r[k].w[1] : 0u;
                                const uint32_t r2 = st.ok[k] ? st.r[k].w[2] : 0u;
                                const uint32_t r3 = st.ok[k] ? st.r[k].w[3] : 0u;
                                uint32_t w[8];
                                e4m3x4_widen<MT>(h0 ? r2 : r0, w[0], w[1]);
                                e4m3x4_widen<MT>(h0 ? r3 : r1, w[2], w[3]);
                                e4m3x4_widen<MT>(h0 ? r0 : r2, w[4], w[5]);
                                e4m3x4_widen<MT>(h0 ? r1 : r3, w[6], w[7]);
                                *reinterpret_cast<uint4*>(dst + 8 * h0) = make_uint4(w[0], w[1], w[2], w[3]);
                                *reinterpret_cast<uint4*>(dst + 8 * (h0 ^ 1)) = make_uint4(w[4], w[5], w[6], w[7]);
                            } else {
                                uint32_t w[4];
#pragma unroll
                                for (int q = 0; q < 4; ++q) w[q] = st.ok[k] ? st.r[k].w[q] : 0u;
                                *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
                            }
                        }
                    }
                };
                // Online-softmax update of tile ti with the scores sc[0..nv) of chunk
                // c0 (value e is token c0 + 4 j + bit(e)) into weights pr: one maximum,
                // one check of the reference maximum (the accumulators are rescaled
                // only when a score passes it by more than kSlack).  Unless every
                // token is present (`fast`), absent ones are masked; the mask is built
                // inside the masked branches only, so that none of its work reaches
                // the common path, and shifted by the lane's 4 j once, so that the
                // per-value bits are constants (with the lane's offset in each bit
                // position, the compiler kept sixteen 64-bit masks in registers for
                // the whole loop: 40 registers).
                auto softmax = [&](int ti, const f32x4* sc, float* pr, int nv, bool fast, int c0,
                                   auto&& bit) {
                    float lm = kNegInfG;
                    if (fast) {
                        for (int e = 0; e < nv; ++e) lm = fmaxf(lm, sc[e >> 2][e & 3]);
                        lm *= a.qk_scale;
                    } else {
                        const uint64_t pm = chunk_mask(c0) >> (4 * j);
                        for (int e = 0; e < nv; ++e)
                            lm = fmaxf(lm, ((pm >> bit(e)) & 1ull) ? sc[e >> 2][e & 3] * a.qk_scale : kNegInfG);
                    }
                    if (__builtin_amdgcn_ballot_w64(lm > m[ti] + kSlack)) {   // rare after the first step
                        const float mx = max_over_groups(lm);
                        const float mn = (mx > m[ti] + kSlack) ? mx : m[ti];
                        const float alpha = mn != m[ti] ? fast_exp2(m[ti] - mn) : 1.0f;   // from -inf: 0
                        if (__builtin_amdgcn_ballot_w64(mn != m[ti])) {
#pragma unroll
                            for (int dt = 0; dt < NDT; ++dt) acc[ti][dt] *= alpha;
                            l[ti] *= alpha;
                        }
                        m[ti] = mn;
                    }
                    for (int e = 0; e < nv; ++e) pr[e] = fast_exp2(fmaf(sc[e >> 2][e & 3], a.qk_scale, -m[ti]));
                    if (!fast) {                                 // absent tokens weigh nothing
                        const uint64_t pm = chunk_mask(c0) >> (4 * j);
                        for (int e = 0; e < nv; ++e) pr[e] = ((pm >> bit(e)) & 1ull) ? pr[e] : 0.0f;
                    }
                };
                // the running sum adds four weights as the matrix cores see them; the
                // bf16 low parts (weights minus their bf16 roundings) go to `lo`
                auto pack4 = [&](int ti, const float* pg, uint32_t* hi, uint32_t* lo) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) hi[q] = pack2<MT>(pg[2 * q], pg[2 * q + 1]);
                    if constexpr (MT == PA_F16) {
#pragma unroll
                        for (int q = 0; q < 2; ++q)
                            l[ti] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, hi[q]),
                                                           half2_t{(_Float16)1.0f, (_Float16)1.0f}, l[ti], false);
                    } else {
                        l[ti] += (pg[0] + pg[1]) + (pg[2] + pg[3]);
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const float h0 = __uint_as_float(hi[q] << 16);
                            const float h1 = __uint_as_float(hi[q] & 0xFFFF0000u);
                            lo[q] = pack2<MT>(pg[2 * q] - h0, pg[2 * q + 1] - h1);
                        }
                    }
                };

                // A full wavefront's step: the KT tokens of chunk n for tile 0, every
                // score first (the K reads and MFMAs of all quarters back to back),
                // one softmax update, then O^T[d][head] += V^T P^T with 32 tokens per
                // MFMA (quarters 2g, 2g + 1 side by side form the B operand P^T).
                auto full_step = [&](int c0, int buf, bool fast) {
                    f32x4 sc[NQ];
#pragma unroll
                    for (int u = 0; u < NQ; ++u) {
                        sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            const uint4 r = *reinterpret_cast<const uint4*>(
                                kt(buf) + (16 * u + c16) * LDK + 32 * c + 8 * j);
                            const Op8 kop{{r.x, r.y, r.z, r.w}};
                            sc[u] = mma32<MT>(kop, qop[0][c], sc[u]);
                        }
                    }
                    float pr[4 * NQ];
                    softmax(0, sc, pr, 4 * NQ, fast, c0,
                            [&](int e) { return 16 * (e >> 2) + (e & 3); });
#pragma unroll
                    for (int g = 0; g < NQ / 2; ++g) {
                        Op8 pop, plo;
                        pack4(0, pr + 8 * g, pop.w, plo.w);
                        pack4(0, pr + 8 * g + 4, pop.w + 2, plo.w + 2);
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) {
                            const uint16_t* vp =
                                vt(buf) + (32 * g + 4 * j + (c16 >> 2)) * LDV + 16 * dt + 4 * (c16 & 3);
                            const Op4 v0 = read_tr16(vp);
                            const Op4 v1 = read_tr16(vp + 16 * LDV);
                            const Op8 vop{{v0.w[0], v0.w[1], v1.w[0], v1.w[1]}};
                            acc[0][dt] = mma32<MT>(vop, pop, acc[0][dt]);
                            if constexpr (MT == PA_BF16) acc[0][dt] = mma32<MT>(vop, plo, acc[0][dt]);
                        }
                    }
                };
                // A split wavefront's step: quarter `quarter` of chunk n (16 tokens)
                // for each of its tiles; P V on the 16-token MFMA.
                auto split_step = [&](int c0, int buf, bool fast) {
                    const int r0 = 16 * quarter;
                    Op8 kop[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const uint4 r = *reinterpret_cast<const uint4*>(
                            kt(buf) + (r0 + c16) * LDK + 32 * c + 8 * j);
                        kop[c] = Op8{{r.x, r.y, r.z, r.w}};
                    }
                    Op4 vop[NDT];
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
                        vop[dt] = read_tr16(vt(buf) + (r0 + 4 * j + (c16 >> 2)) * LDV + 16 * dt + 4 * (c16 & 3));
#pragma unroll
                    for (int ti = 0; ti < kSMax; ++ti) {
                        if (ti < ntiles) {                       // wavefront-uniform
                            f32x4 sc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                            for (int c = 0; c < NC; ++c) sc[0] = mma32<MT>(kop[c], qop[ti][c], sc[0]);
                            float pr[4];
                            softmax(ti, sc, pr, 4, fast, c0, [&](int e) { return r0 + e; });
                            Op4 pop, plo;
                            pack4(ti, pr, pop.w, plo.w);
#pragma unroll
                            for (int dt = 0; dt < NDT; ++dt) {
                                acc[ti][dt] = mma16<MT>(vop[dt], pop, acc[ti][dt]);
                                if constexpr (MT == PA_BF16) acc[ti][dt] = mma16<MT>(vop[dt], plo, acc[ti][dt]);
                            }
                        }
                    }
                };
                auto compute_chunk = [&](int n, int buf) {
                    const int c0 = ts + n * KT;
                    // all KT tokens present (known without a look at the table when
                    // the slice is clean and the step ends inside the item)
                    const bool fast = slice_ok && c0 + KT <= te && a.qk_scale > 0.0f;
                    if (full) full_step(c0, buf, fast);
                    else split_step(c0, buf, fast);
                };

                // Pipeline: register stage n mod NS holds chunk n from its load until it
                // is written to tile buffer n mod 2; step n writes chunk n + 1, loads
                // chunk n + NS into the stage just freed (past the end: masked loads of
                // the pool's first bytes), computes chunk n and ends with the barrier
                // that hands both buffers over.  Every step of the unrolled group
                // issues its loads, also the steps past the last chunk: with a branch
                // around a load, the compiler could no longer count the loads issued
                // after the one a write waits for, and would wait for all of them.
                Stage ring[NS];
#pragma unroll
                for (int k = 0; k < NS; ++k) load_chunk(ring[k], k);
                write_chunk(ring[0], 0);
                __syncthreads();
                for (int n0 = 0; n0 < nch; n0 += NS) {
#pragma unroll
                    for (int k = 0; k < NS; ++k) {
                        const int n = n0 + k;
                        const bool live = n < nch;               // workgroup-uniform
                        if (live) write_chunk(ring[(k + 1) % NS], (n + 1) & 1);
                        load_chunk(ring[k], n + NS);
                        if (live) {
                            if (computes) compute_chunk(n, n & 1);
                            __syncthreads();
                        }
                    }
                }
            }

            // ---- per-column totals; the split wavefronts of a tile merge their
            // quarters into quarter 0's: maxima, then the sums and accumulators,
            // each scaled to the common maximum, added in quarter order
            float lt[kSMax];
#pragma unroll
            for (int ti = 0; ti < kSMax; ++ti) lt[ti] = sum_over_groups(l[ti]);
            if (wg_splits) {
                float* slots = reinterpret_cast<float*>(tiles);
                auto slot = [&](int ti, int q) -> float* {
                    return slots + ((tile0 + ti - split_base) * 3 + (q - 1)) * SLOT_FLOATS;
                };
                if (!full && quarter != 0) {
#pragma unroll
                    for (int ti = 0; ti < kSMax; ++ti) {
                        if (ti < ntiles) {
                            float* sp = slot(ti, quarter);
#pragma unroll
                            for (int dt = 0; dt < NDT; ++dt)
                                *reinterpret_cast<f32x4*>(sp + (dt * 64 + lane) * 4) = acc[ti][dt];
                            if (j == 0) {
                                sp[NDT * 256 + c16] = m[ti];
                                sp[NDT * 256 + 16 + c16] = lt[ti];
                            }
                        }
                    }
                }
                __syncthreads();
                if (!full && quarter == 0) {
#pragma unroll
                    for (int ti = 0; ti < kSMax; ++ti) {
                        if (ti < ntiles) {
                            float mq[4], f[4];
                            mq[0] = m[ti];
                            float mm = m[ti];
#pragma unroll
                            for (int q = 1; q < 4; ++q) {
                                mq[q] = slot(ti, q)[NDT * 256 + c16];
                                mm = fmaxf(mm, mq[q]);
                            }
#pragma unroll
                            for (int q = 0; q < 4; ++q) f[q] = mq[q] == kNegInfG ? 0.0f : fast_exp2(mq[q] - mm);
                            float tot = lt[ti] * f[0];
#pragma unroll
                            for (int q = 1; q < 4; ++q) tot += slot(ti, q)[NDT * 256 + 16 + c16] * f[q];
#pragma unroll
                            for (int dt = 0; dt < NDT; ++dt) {
                                f32x4 o = acc[ti][dt] * f[0];
#pragma unroll
                                for (int q = 1; q < 4; ++q)
                                    o += *reinterpret_cast<const f32x4*>(slot(ti, q) + (dt * 64 + lane) * 4) * f[q];
                                acc[ti][dt] = o;
                            }
                            m[ti] = mm;
                            lt[ti] = tot;
                        }
                    }
                }
            }

            // ---- this wavefront's results for its item: quarter 0 of a split tile,
            // or a full tile
            if (computes && (full || quarter == 0)) {
#pragma unroll
                for (int ti = 0; ti < kSMax; ++ti) {
                    const int hu = 16 * (tile0 + ti) + c16;
                    if (ti < ntiles && hu < G) {
                        const int head = kvh * G + hu;
                        const float inv_l = lt[ti] > 0.0f ? 1.0f / lt[ti] : 0.0f;
                        const int64_t r = cur.rec0 + (int64_t)hu * cur.rec_stride;
                        if (!cur.whole && j == 0) {
                            a.ws[r] = m[ti];
                            a.ws[a.nrec + r] = lt[ti];
                        }
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) {
                            const int d = 16 * dt + 4 * j;
                            if (cur.whole) {
                                const float f = inv_l * a.out_scale;
                                char* op = reinterpret_cast<char*>(a.out) +
                                           (((int64_t)s * a.num_heads + head) * D + d) * elem_bytes(QDT);
                                *reinterpret_cast<uint2*>(op) =
                                    make_uint2(pack2<QDT>(acc[ti][dt][0] * f, acc[ti][dt][1] * f),
                                               pack2<QDT>(acc[ti][dt][2] * f, acc[ti][dt][3] * f));
                            } else {
                                float* wo = a.ws + 2 * a.nrec + r * D + d;
#pragma unroll
                                for (int i = 0; i < 4; ++i) wo[i] = acc[ti][dt][i] * inv_l;
                            }
                        }
                    }
                }
            }
        }
    }
}

// Measured on Falcon-7B's layer (71 heads of 64, fp8): 64-token steps with four
// in flight.  Two workgroups per CU (four wavefronts per SIMD, at most 128
// registers, no spills with 64 dimensions) against one (two per SIMD) on the
// same 256-sequence fp8 MQA batch: 24 and 32 heads (one or two tiles) 31.6-32.7
// -> 28.8-29.6 us, 48 heads 32.9-33.9 -> 31.7 us; 64, 71 and 96 heads within
// +-1 us (the second workgroup's shorter chains are paid back by twice the cut
// contexts and partial records), 128 heads 1 us slower.  128 dimensions do not
// fit 128 registers.
template <int KVDT, int QDT, int D, int MINB>
hipError_t launch_with(DecodeArgs& a, hipStream_t stream) {
    constexpr int KT = 64;                              // tokens per step
    constexpr int NS = 4;                               // steps in flight per workgroup
    auto kernel = decode_group_kernel<KVDT, QDT, D, KT, NS, MINB>;
    a.unit_heads = a.num_heads / a.num_kv_heads;        // a unit: every query head of a KV head
    a.units_per_kv = 1;
    // an item start, in tokens: measured over 128..1,536 on 256-sequence fp8 MQA batches
    // (24, 32, 71 heads) and a 64-head bf16 GQA layer, best at 512 for all (Falcon-7B's
    // 71 heads 37.2-38.2 -> 34.5-36.2 us against 256)
    a.seg_cost = 512;
    const int64_t grid = decode_grid(reinterpret_cast<const void*>(kernel), kGThreads,
                                     a.num_kv_heads, 0, a, kGroupMaxWorkersPerCu);
    if (grid < 0) return hipErrorOutOfMemory;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kGThreads), 0, stream, a);
    return hipGetLastError();
}

template <int KVDT, int QDT, int D>
hipError_t launch_typed(DecodeArgs& a, hipStream_t stream) {
    const int tiles = (a.num_heads / a.num_kv_heads + 15) / 16;
    if constexpr (D == 64)
        if (tiles <= 3) return launch_with<KVDT, QDT, D, 2>(a, stream);
    return launch_with<KVDT, QDT, D, 1>(a, stream);
}

template <int KVDT, int QDT>
hipError_t launch_dim(DecodeArgs& a, int head_dim, hipStream_t stream) {
    if (head_dim == 64) return launch_typed<KVDT, QDT, 64>(a, stream);
    if (head_dim == 128) return launch_typed<KVDT, QDT, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_group_supported(int q_dt, int kv_dt, int head_dim, int group) {
    if (group <= 16 || group > kMaxGroup) return false;
    if (head_dim != 64 && head_dim != 128) return false;
    if (q_dt != PA_F16 && q_dt != PA_BF16) return false;
    return kv_dt == q_dt || kv_dt == PA_FP8_E4M3;
}

hipError_t launch_decode_group(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                               hipStream_t stream) {
    if (kv_dt == PA_F16 && q_dt == PA_F16) return launch_dim<PA_F16, PA_F16>(a, head_dim, stream);
    if (kv_dt == PA_BF16 && q_dt == PA_BF16) return launch_dim<PA_BF16, PA_BF16>(a, head_dim, stream);
    if (kv_dt == PA_FP8_E4M3 && q_dt == PA_F16)
        return launch_dim<PA_FP8_E4M3, PA_F16>(a, head_dim, stream);
    if (kv_dt == PA_FP8_E4M3 && q_dt == PA_BF16)
        return launch_dim<PA_FP8_E4M3, PA_BF16>(a, head_dim, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa

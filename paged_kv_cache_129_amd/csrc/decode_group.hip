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

// KT tokens per step (a multiple of 32), NS steps' loads in flight, MINB
// workgroups per CU that the register allocation must allow
template <int KVDT, int QDT, int D, int KT, int NS, int MINB>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(MINB * kGWaves / 4)))
void decode_group_kernel(DecodeArgs a) {
    constexpr int kGChunk = KT;
    // MFMA operand type: the cache's, or for an fp8 cache the query's (e4m3 widens
    // exactly to fp16 and to bf16, and a bf16 query keeps its range)
    constexpr int MT = (KVDT == PA_FP8_E4M3) ? QDT : KVDT;
    constexpr int EB = elem_bytes(KVDT);
    constexpr int RB = D * EB;                                   // bytes of a cached row
    constexpr int PPR = RB / 16;                                 // 16-byte pieces per row
    constexpr int KPIECES = kGChunk * PPR;                       // pieces of a chunk's K rows
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
    constexpr int NC = D / 32;                                   // score MFMAs per half and chunk
    constexpr int NDT = D / 16;                                  // output d-tiles

    __shared__ __attribute__((aligned(16))) uint16_t kt[2][kGChunk * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t vt[2][kGChunk * LDV];
    __shared__ int32_t tbl[kGTable];
    __shared__ __attribute__((aligned(8))) int32_t wl_lds[kListInts];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane >> 4;
    const int c16 = lane & 15;
    const int G = a.num_heads / a.num_kv_heads;
    const int bs = 1 << a.log2_bs;
    const char* kbase = reinterpret_cast<const char*>(a.k_pool);
    const char* vbase = reinterpret_cast<const char*>(a.v_pool);
    const bool computes = 16 * wave < G;                         // wavefront-uniform

    Schedule<kGThreads> sch;
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
            const int hu = 16 * wave + c16;                      // this lane's head column
            const bool hlive = hu < G;

            // B operands of the score MFMA: Q^T[d][head], head dimensions 32 c + 8 j..
            Op8 qop[NC];
            {
                const char* qrow = reinterpret_cast<const char*>(a.q) +
                                   ((int64_t)s * a.num_heads + kvh * G + (hlive ? hu : 0)) * D *
                                       elem_bytes(QDT);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    static_assert(QDT == MT, "the query is an MFMA operand as it is");
                    const Raw16 r = load16(qrow + (32 * c + 8 * j) * elem_bytes(QDT));
                    Op8 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o.w[q] = hlive ? r.w[q] : 0u;
                    qop[c] = o;
                }
            }

            float m = kNegInfG, l = 0.0f;
            f32x4 acc[NDT];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

            const int b_first = t0 >> a.log2_bs;
            const int b_end = (t1 + bs - 1) >> a.log2_bs;
            __syncthreads();                                     // the previous item's table is read
            tpre.store(tbl, min(b_end, b_first + kGTable) - b_first, a.num_blocks, tid);
            __syncthreads();
            have = sch.next(a, itm);
            if (have) prefetch(itm);
            for (int sb = b_first; sb < b_end; sb += kGTable) {
                const int se = min(b_end, sb + kGTable);
                if (sb != b_first) {                             // later slices of a long item
                    __syncthreads();
                    for (int i = tid; i < se - sb; i += kGThreads) {
                        const int b = trow[sb + i];
                        tbl[i] = (b >= 0 && b < a.num_blocks) ? b : -1;
                    }
                    __syncthreads();
                }
                const int ts = max(t0, sb << a.log2_bs);
                const int te = min(t1, se << a.log2_bs);
                const int nch = (te - ts + kGChunk - 1) / kGChunk;

                // this thread's pieces of chunk n: raw bytes in one register stage
                struct Stage {
                    Raw16 r[LPT];
                    bool ok[LPT];
                };
                auto load_chunk = [&](Stage& st, int n) {
                    const int c0 = ts + n * kGChunk;
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
                        const int64_t r = ((((int64_t)(blk >= 0 ? blk : 0)) * a.num_kv_heads + kvh)
                                           << a.log2_bs) + (t & (bs - 1));
                        const char* src = (isv ? vbase : kbase) + (blk >= 0 ? r * RB + col * 16 : 0);
                        st.r[k] = load16_stream(src);
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
                            uint16_t* dst = isv ? &vt[buf][row * LDV + col * HPP]
                                                : &kt[buf][row * LDK + col * HPP];
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
                // 32 tokens (rows r0.. of tile buffer `buf`) of this wavefront's tile
                auto compute32 = [&](int c0, int buf, int r0) {
                    // present tokens of the chunk as a 32-bit mask (the same in every lane)
                    uint32_t present;
                    {
                        const int t = c0 + (lane & 31);
                        const bool ok = t < te && tbl[(min(t, te - 1) >> a.log2_bs) - sb] >= 0;
                        present = (uint32_t)__builtin_amdgcn_ballot_w64(ok && lane < 32);
                    }
                    f32x4 sc[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            const uint4 r = *reinterpret_cast<const uint4*>(
                                &kt[buf][(r0 + 16 * u + c16) * LDK + 32 * c + 8 * j]);
                            const Op8 kop{{r.x, r.y, r.z, r.w}};
                            sc[u] = mma32<MT>(kop, qop[c], sc[u]);
                        }
                    }
                    // value e = 4u + i is token c0 + 16u + 4j + i
                    const bool fast = present == 0xFFFFFFFFu && a.qk_scale > 0.0f;
                    float pr[8];
                    float lm = kNegInfG;
                    if (fast) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) lm = fmaxf(lm, sc[e >> 2][e & 3]);
                        lm *= a.qk_scale;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const bool lv = (present >> (16 * (e >> 2) + 4 * j + (e & 3))) & 1u;
                            lm = fmaxf(lm, lv ? sc[e >> 2][e & 3] * a.qk_scale : kNegInfG);
                        }
                    }
                    if (__builtin_amdgcn_ballot_w64(lm > m + kSlack)) {   // rare after the first chunk
                        const float mx = max_over_groups(lm);
                        const float mn = (mx > m + kSlack) ? mx : m;
                        const float alpha = mn != m ? fast_exp2(m - mn) : 1.0f;   // from -inf: 0
                        if (__builtin_amdgcn_ballot_w64(mn != m)) {
#pragma unroll
                            for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
                            l *= alpha;
                        }
                        m = mn;
                    }
                    if (fast) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(fmaf(sc[e >> 2][e & 3], a.qk_scale, -m));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const bool lv = (present >> (16 * (e >> 2) + 4 * j + (e & 3))) & 1u;
                            pr[e] = lv ? fast_exp2(fmaf(sc[e >> 2][e & 3], a.qk_scale, -m)) : 0.0f;
                        }
                    }
                    // weights -> the B operand P^T (tokens 4j.. of each half); the running
                    // sum adds them as the matrix cores see them
                    Op8 pop, plo;
#pragma unroll
                    for (int q = 0; q < 4; ++q) pop.w[q] = pack2<MT>(pr[2 * q], pr[2 * q + 1]);
                    if constexpr (MT == PA_F16) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            l = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pop.w[q]),
                                                       half2_t{(_Float16)1.0f, (_Float16)1.0f}, l, false);
                    } else {
                        l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float h0 = __uint_as_float(pop.w[q] << 16);
                            const float h1 = __uint_as_float(pop.w[q] & 0xFFFF0000u);
                            plo.w[q] = pack2<MT>(pr[2 * q] - h0, pr[2 * q + 1] - h1);
                        }
                    }
                    // O^T[d][head] += V^T[d][token] P^T[token][head], 32 tokens per MFMA
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        const uint16_t* vp = &vt[buf][(r0 + 4 * j + (c16 >> 2)) * LDV + 16 * dt + 4 * (c16 & 3)];
                        const Op4 v0 = read_tr16(vp);
                        const Op4 v1 = read_tr16(vp + 16 * LDV);
                        const Op8 vop{{v0.w[0], v0.w[1], v1.w[0], v1.w[1]}};
                        acc[dt] = mma32<MT>(vop, pop, acc[dt]);
                        if constexpr (MT == PA_BF16) acc[dt] = mma32<MT>(vop, plo, acc[dt]);
                    }
                };
                auto compute_chunk = [&](int n, int buf) {
#pragma unroll
                    for (int g = 0; g < KT / 32; ++g) compute32(ts + n * KT + 32 * g, buf, 32 * g);
                };

                // Pipeline: register stage n mod NS holds chunk n from its load until it
                // is written to tile buffer n mod 2; step n writes chunk n + 1, loads
                // chunk n + NS into the stage just freed (past the end: masked loads of
                // the pool's first bytes, so that no branch sits between a load and its
                // wait), computes chunk n and ends with the barrier that hands both
                // buffers over.
                Stage ring[NS];
#pragma unroll
                for (int k = 0; k < NS; ++k) load_chunk(ring[k], k);
                write_chunk(ring[0], 0);
                __syncthreads();
                for (int n0 = 0; n0 < nch; n0 += NS) {
#pragma unroll
                    for (int k = 0; k < NS; ++k) {
                        const int n = n0 + k;
                        if (n < nch) {
                            write_chunk(ring[(k + 1) % NS], (n + 1) & 1);
                            load_chunk(ring[k], n + NS);
                            if (computes) compute_chunk(n, n & 1);
                            __syncthreads();
                        }
                    }
                }
            }

            // ---- per-column totals, then this tile's result for its item
            if (computes) {
                const float lt = sum_over_groups(l);
                if (hlive) {
                    const int head = kvh * G + hu;
                    const float inv_l = lt > 0.0f ? 1.0f / lt : 0.0f;
                    const int64_t r = cur.rec0 + (int64_t)hu * cur.rec_stride;
                    if (!cur.whole && j == 0) {
                        a.ws[r] = m;
                        a.ws[a.nrec + r] = lt;
                    }
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        const int d = 16 * dt + 4 * j;
                        if (cur.whole) {
                            const float f = inv_l * a.out_scale;
                            char* op = reinterpret_cast<char*>(a.out) +
                                       (((int64_t)s * a.num_heads + head) * D + d) * elem_bytes(QDT);
                            *reinterpret_cast<uint2*>(op) =
                                make_uint2(pack2<QDT>(acc[dt][0] * f, acc[dt][1] * f),
                                           pack2<QDT>(acc[dt][2] * f, acc[dt][3] * f));
                        } else {
                            float* wo = a.ws + 2 * a.nrec + r * D + d;
#pragma unroll
                            for (int i = 0; i < 4; ++i) wo[i] = acc[dt][i] * inv_l;
                        }
                    }
                }
            }
        }
    }
}

// Measured on Falcon-7B's layer (71 heads of 64, fp8): 64-token steps with
// four in flight and two workgroups per CU beat 32-token steps (three to six
// in flight) and one workgroup per CU by 3-12%.
template <int KVDT, int QDT, int D>
hipError_t launch_typed(DecodeArgs& a, hipStream_t stream) {
    constexpr int KT = 64;                              // tokens per step
    constexpr int NS = 4;                               // steps in flight per workgroup
    // workgroups per CU the registers must allow (fp8, 64 dimensions: two fit)
    constexpr int MINB = (D == 64 && KVDT == PA_FP8_E4M3) ? 2 : 1;
    auto kernel = decode_group_kernel<KVDT, QDT, D, KT, NS, MINB>;
    a.unit_heads = a.num_heads / a.num_kv_heads;        // a unit: every query head of a KV head
    a.units_per_kv = 1;
    a.seg_cost = 256;                                   // an item start, in tokens (measured)
    const int64_t grid = decode_grid(reinterpret_cast<const void*>(kernel), kGThreads,
                                     a.num_kv_heads, 0, a, kGroupMaxWorkersPerCu);
    if (grid < 0) return hipErrorOutOfMemory;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kGThreads), 0, stream, a);
    return hipGetLastError();
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

// paged_attention_decode, matrix-core path for grouped heads (2 <= G <= 16
// query heads per KV head; larger groups: decode_group.hip).
//
// When several query heads share one KV head (KV 缓存与分页注意力 §11;
// KV Cache从原理到实战 §5.3), one pass over a KV tile serves all G heads, and
// scores = K·Q^T and out = P·V become small dense contractions on the matrix
// cores: the heads (padded to 16) are one MFMA dimension, 16 tokens another.
//
// Work items come from worklist.h; each wavefront is a worker that streams
// its items in 16-token chunks.  Per chunk it
//   * loads the 16 K rows straight into the A-operand layout of
//     v_mfma_f32_16x16x32 (lane = token row, eight consecutive head_dim numbers
//     per lane, 16-byte loads) and computes S^T[token][head];
//   * runs the online softmax per head column (running maximum in log2 units,
//     combined over a column's four lanes by two lane-row swaps; the running
//     sum stays per lane and is added up at the end); the reference maximum
//     moves only when a score passes it by more than kMaxSlack, so the
//     accumulators are rescaled only on the rare chunks where it moves;
//   * stages its V rows in its own LDS slice (rows of absent tokens zeroed)
//     and reads them back with transposing LDS reads as the A operand of the
//     K=16 MFMA O^T[d][head] += V^T·P^T, whose B operand is exactly the
//     register layout the score MFMA produced (for bf16, P is split into a
//     bf16 high and low part so the weights keep ~16 significant bits).
// With blocks of 16 tokens or more a chunk lies in one block: its pool offset
// is wavefront-uniform (one table lookup per chunk) and each lane adds a fixed
// offset; smaller blocks take a per-token lookup.  The next chunk's loads are
// issued before the current one is computed.  An fp8 cache is widened exactly
// to the query's type, fp16 or bf16, in registers (value * 2^-8; the factor is
// folded into the scales).
#include "kernels.h"
#include "pa_device.h"
#include "worklist.h"
#include "mfma_util.h"

namespace pa {
namespace {

constexpr int kTableCap = 1024;     // block-table entries staged in LDS per segment
constexpr int kChunk = 16;          // tokens per wavefront step
constexpr float kNegInf = -__builtin_inff();
constexpr float kMaxSlack = 8.0f;   // log2 units a score may exceed the reference maximum by

// head_dim offset of score-operand chunk c for lane group j (the same mapping
// is used for K and for Q, so any mapping gives the same dot products; this
// one makes each lane's loads contiguous within a token row).
template <int KVDT, int D>
__device__ __forceinline__ int dmap(int c, int j) {
    if constexpr (KVDT == PA_FP8_E4M3) return (D / 4) * j + 8 * c;
    return 32 * c + 8 * j;
}

// One wavefront per SIMD may take all its registers: measured on Llama-2-70B
// (one 16-head tile), one wavefront per SIMD with three chunks in flight beats
// two wavefronts per SIMD with two (108 vs 114 us per layer): of two
// wavefronts sharing a SIMD the older one gets most of the memory pipeline,
// and the younger one finishes its equal share well after it.
template <int KVDT, int QDT, int D, int NW, int TILES, int PD, bool BIGB>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_kernel(DecodeArgs a) {
    // MFMA operand type: the cache's, or for an fp8 cache the query's (e4m3 widens
    // exactly to fp16 and to bf16, and a bf16 query keeps its range)
    constexpr int MT = (KVDT == PA_FP8_E4M3) ? QDT : KVDT;
    constexpr int EB = elem_bytes(KVDT);
    constexpr int NC = D / 32;               // score MFMAs per chunk and tile
    constexpr int NDT = D / 16;              // output d-tiles
    // LDS row stride of a staged V tile (halfs).  16-bit caches: D + 16 puts the
    // eight rows a 32-lane pass of the transposed read touches 8 banks apart (no
    // bank conflicts; D + 8 had 2-way ones on a quarter of the LDS cycles).  fp8
    // caches write 32 widened bytes per lane, which conflict less with D + 8.
    constexpr int LDV = KVDT == PA_FP8_E4M3 ? D + 8 : D + 16;
    constexpr int PPR = D * EB / 16;         // 16-byte pieces per V row
    constexpr int NPV = kChunk * PPR / 64;   // V pieces per lane per chunk
    constexpr int VEL = 16 / EB;             // numbers per V piece
    constexpr int VTILE = kChunk * LDV;      // halfs of one wavefront's V slice
    constexpr int NT = NW * 64;
    constexpr int WT = kTableCap / NW;       // block-table entries staged per wavefront
    static_assert(NPV >= 1 && (kChunk * PPR) % 64 == 0, "V staging split");

    __shared__ int32_t tbl_all[NW][WT];
    __shared__ __attribute__((aligned(16))) uint16_t smem[NW * VTILE];
    __shared__ __attribute__((aligned(8))) int32_t wl_lds[kListInts];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane >> 4;
    const int c16 = lane & 15;
    const int G = a.num_heads / a.num_kv_heads;
    const int bs = 1 << a.log2_bs;
    uint16_t* vs = smem + wave * VTILE;
    int32_t* tbl = tbl_all[wave];
    const char* kbase = reinterpret_cast<const char*>(a.k_pool);
    const char* vbase = reinterpret_cast<const char*>(a.v_pool);
    const int64_t row_bytes = (int64_t)D * EB;

    Schedule<NT> sch;
    for (int s0 = 0; s0 < a.num_seqs; s0 += kWindow) {
        sch.build(a, s0, min(kWindow, a.num_seqs - s0), a.units, wl_lds, worker_id(wave, NW),
                  gridDim.x * NW, lane == 0);
        // The query and the first block-table slice of an item are loaded while the
        // previous item streams: `pre` holds them for the item in `itm`.
        struct Prefetch {
            TablePrefetch<64, WT> tbl;
            Raw16 q[TILES][NC];
        } pre;
        auto prefetch = [&](const Item& it) {
            const int kvh = it.unit / a.units_per_kv;
            const int hg0 = (it.unit % a.units_per_kv) * a.unit_heads;
            const int nh = min(a.unit_heads, G - hg0);
            pre.tbl.issue(a.tables + (int64_t)it.s * a.max_blocks, it.t0 >> a.log2_bs,
                          table_span(a, it.t0, it.t1, WT), a.max_blocks, lane);
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
                const int hu = 16 * tt + c16;
                const char* qrow = reinterpret_cast<const char*>(a.q) +
                                   ((int64_t)it.s * a.num_heads + kvh * G + hg0 + (hu < nh ? hu : 0)) * D *
                                       elem_bytes(QDT);
#pragma unroll
                for (int c = 0; c < NC; ++c) pre.q[tt][c] = load16(qrow + dmap<KVDT, D>(c, j) * elem_bytes(QDT));
            }
        };
        Item itm;
        bool have = sch.next(a, itm);
        if (have) prefetch(itm);
        while (have) {
            // settle the prefetched loads (issued an item ago, or just now for the
            // first item); the wait-count analysis cannot see across the item loop's
            // back edge that they completed
            __builtin_amdgcn_s_waitcnt(0);
            const Item cur = itm;
            const int s = cur.s;
            const int kvh = cur.unit / a.units_per_kv;
            const int hg0 = (cur.unit % a.units_per_kv) * a.unit_heads;   // first head of the unit, within the group
            const int nh = min(a.unit_heads, G - hg0);                   // heads of the unit
            const int t0 = cur.t0, t1 = cur.t1;
            const int32_t* trow = a.tables + (int64_t)s * a.max_blocks;

            // B operands of the score MFMA: Q^T[d][head] per 16-head tile, head = 16 tt + c16
            // of the unit (zero for padding heads)
            Op8 qop[TILES][NC];
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
                const bool live = 16 * tt + c16 < nh;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    static_assert(QDT == MT, "the query is an MFMA operand as it is");
                    Op8 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o.w[q] = live ? pre.q[tt][c].w[q] : 0u;
                    qop[tt][c] = o;
                }
            }
            // the first table slice, then the next item's loads, which stream in
            // behind this item's
            const int b_first = t0 >> a.log2_bs;
            const int b_end = (t1 + bs - 1) >> a.log2_bs;
            __builtin_amdgcn_wave_barrier();
            pre.tbl.store(tbl, min(b_end, b_first + WT) - b_first, a.num_blocks, lane);
            __builtin_amdgcn_wave_barrier();
            have = sch.next(a, itm);
            if (have) prefetch(itm);

            float m[TILES], l[TILES];
            f32x4 acc[TILES][NDT];
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
                m[tt] = kNegInf;
                l[tt] = 0.0f;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc[tt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }

            for (int sb = b_first; sb < b_end; sb += WT) {
                const int se = min(b_end, sb + WT);
                if (sb != b_first) {             // later slices of a long item
                    __builtin_amdgcn_wave_barrier();
                    for (int i = lane; i < se - sb; i += 64) {
                        const int b = trow[sb + i];
                        tbl[i] = (b >= 0 && b < a.num_blocks) ? b : -1;
                    }
                    __builtin_amdgcn_wave_barrier();
                }
                const int ts = max(t0, sb << a.log2_bs);
                const int te = min(t1, se << a.log2_bs);

                // pool row (token row index) of token t, or -1 when absent; branch-free,
                // so that loads issued around it keep precise wait counts (blocks of
                // fewer than 16 tokens, where a chunk spans several blocks)
                auto row_of = [&](int t) -> int64_t {
                    const bool in = t < te;
                    const int blk = tbl[in ? (t >> a.log2_bs) - sb : 0];
                    const int64_t r = (((int64_t)blk * a.num_kv_heads + kvh) << a.log2_bs) + (t & (bs - 1));
                    return (in && blk >= 0) ? r : (int64_t)-1;
                };
                // blocks of 16 tokens or more: chunks are 16-aligned windows, so a chunk
                // lies in one block; its byte offset in the pool is wavefront-uniform
                // and every lane adds a fixed offset of its own
                const int c_begin = BIGB ? (ts & ~(kChunk - 1)) : ts;
                auto chunk_off = [&](int c0, bool& valid) -> int64_t {
                    const bool in = c0 < te;
                    const int blk = __builtin_amdgcn_readfirstlane(tbl[in ? (c0 >> a.log2_bs) - sb : 0]);
                    valid = in && blk >= 0;
                    return (((int64_t)(valid ? blk : 0) * a.num_kv_heads + kvh) << a.log2_bs) * row_bytes +
                           (int64_t)(c0 & (bs - 1)) * row_bytes;
                };
                const uint32_t k_lane = (uint32_t)(c16 * row_bytes) +
                                        (KVDT == PA_FP8_E4M3 ? (D / 4) * j : 16 * j);
                const uint32_t v_lane = (uint32_t)((lane / PPR) * row_bytes + (lane % PPR) * 16);

                // One chunk's K operands and raw V pieces.  Two sets alternate: the next
                // chunk's loads are always issued (past the end they read the pool's
                // first block and are masked) before the current chunk is computed, so
                // they overlap it and no branch sits between a load and its wait.
                struct ChunkRegs {
                    Op8 k[NC];
                    Raw16 v[NPV];
                    bool vlive[NPV];
                    bool valid;
                };
                auto load_chunk = [&](ChunkRegs& R, int c0) {
                    const char* krow;
                    const char* vrow[NPV];
                    if constexpr (BIGB) {
                        const int64_t off = chunk_off(c0, R.valid);
                        krow = kbase + off + k_lane;
#pragma unroll
                        for (int u = 0; u < NPV; ++u)
                            vrow[u] = vbase + off + v_lane + (uint32_t)(u * (64 / PPR) * row_bytes);
                    } else {
                        const int64_t r = row_of(c0 + c16);
                        krow = kbase + (r < 0 ? 0 : r) * row_bytes +
                               (KVDT == PA_FP8_E4M3 ? (D / 4) * j : 16 * j);
#pragma unroll
                        for (int u = 0; u < NPV; ++u) {
                            const int p = u * 64 + lane;
                            const int64_t rv = row_of(c0 + p / PPR);
                            R.vlive[u] = rv >= 0;
                            vrow[u] = vbase + (rv < 0 ? 0 : rv) * row_bytes + (p % PPR) * 16;
                        }
                    }
                    if constexpr (KVDT == PA_FP8_E4M3) {
#pragma unroll
                        for (int hh = 0; hh < D / 64; ++hh) {
                            const Raw16 raw = load16_stream(krow + 16 * hh);
                            // keep the raw codes; widened when used
#pragma unroll
                            for (int q = 0; q < 4; ++q) R.k[2 * hh + (q >> 1)].w[(q & 1) * 2] = raw.w[q];
                        }
                    } else {
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            const Raw16 raw = load16_stream(krow + 64 * c);
#pragma unroll
                            for (int q = 0; q < 4; ++q) R.k[c].w[q] = raw.w[q];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < NPV; ++u) R.v[u] = load16_stream(vrow[u]);
                };
                auto compute_chunk = [&](ChunkRegs& R, int c0) {
                    Op8 kop[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        if constexpr (KVDT == PA_FP8_E4M3) {
                            e4m3x4_widen<MT>(R.k[c].w[0], kop[c].w[0], kop[c].w[1]);
                            e4m3x4_widen<MT>(R.k[c].w[2], kop[c].w[2], kop[c].w[3]);
                        } else {
                            kop[c] = R.k[c];
                        }
                    }
                    // token liveness: a whole chunk of present tokens needs no masks
                    bool full = false;
                    bool live[4];
                    if constexpr (BIGB) {
                        full = R.valid && c0 >= ts && c0 + kChunk <= te;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = c0 + 4 * j + i;
                            live[i] = R.valid && t >= ts && t < te;
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) live[i] = row_of(c0 + 4 * j + i) >= 0;
                    }

                    // ---- scores S^T[token][head] of every tile (the matrix cores work on
                    // them while the vector units go on)
                    f32x4 sc[TILES];
#pragma unroll
                    for (int tt = 0; tt < TILES; ++tt) {
                        sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < NC; ++c) sc[tt] = mma32<MT>(kop[c], qop[tt][c], sc[tt]);
                    }
                    // ---- online softmax per head column.  The reference maximum moves
                    // only when a score passes it by more than kMaxSlack (weights then stay
                    // below 2^kMaxSlack); a lane's own scores tell whether that can happen,
                    // and only then (rarely, after the first chunks) are column maxima taken
                    // across the column's four lanes and the accumulators rescaled.
                    // With every token present and a positive scale the scaled maximum is
                    // the maximum scaled, and no masks are needed.
                    const bool fast = full && a.qk_scale > 0.0f;
                    float lm[TILES];
                    if (fast) {
#pragma unroll
                        for (int tt = 0; tt < TILES; ++tt)
                            lm[tt] = fmaxf(fmaxf(sc[tt][0], sc[tt][1]), fmaxf(sc[tt][2], sc[tt][3])) * a.qk_scale;
                    } else {
#pragma unroll
                        for (int tt = 0; tt < TILES; ++tt) {
                            float mx = kNegInf;
#pragma unroll
                            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, live[i] ? sc[tt][i] * a.qk_scale : kNegInf);
                            lm[tt] = mx;
                        }
                    }
                    bool grow = false;
#pragma unroll
                    for (int tt = 0; tt < TILES; ++tt) grow = grow || lm[tt] > m[tt] + kMaxSlack;
                    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                        for (int tt = 0; tt < TILES; ++tt) {
                            const float mx = max_over_groups(lm[tt]);
                            const float mn = (mx > m[tt] + kMaxSlack) ? mx : m[tt];
                            // (moving from -inf gives exp2(-inf) = 0)
                            const float alpha = mn != m[tt] ? fast_exp2(m[tt] - mn) : 1.0f;
                            if (__builtin_amdgcn_ballot_w64(mn != m[tt])) {
#pragma unroll
                                for (int dt = 0; dt < NDT; ++dt) acc[tt][dt] *= alpha;
                                l[tt] *= alpha;
                            }
                            m[tt] = mn;
                        }
                    }
                    // ---- weights -> MFMA operands; the running sum adds the weights as
                    // the matrix cores see them (fp16: the rounded values, two per dot
                    // instruction; bf16: a high and a low part that together keep ~16 bits)
                    Op4 pop[TILES], plo[TILES];
#pragma unroll
                    for (int tt = 0; tt < TILES; ++tt) {
                        float pr[4];
                        const float mn = m[tt];
                        if (fast) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(fmaf(sc[tt][i], a.qk_scale, -mn));
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                pr[i] = live[i] ? fast_exp2(fmaf(sc[tt][i], a.qk_scale, -mn)) : 0.0f;
                        }
                        pop[tt].w[0] = pack2<MT>(pr[0], pr[1]);
                        pop[tt].w[1] = pack2<MT>(pr[2], pr[3]);
                        if constexpr (MT == PA_F16) {
                            float lt = l[tt];
#pragma unroll
                            for (int q = 0; q < 2; ++q)
                                lt = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pop[tt].w[q]),
                                                            half2_t{(_Float16)1.0f, (_Float16)1.0f}, lt, false);
                            l[tt] = lt;
                        } else {
                            l[tt] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                const float h0 = __uint_as_float(pop[tt].w[q] << 16);
                                const float h1 = __uint_as_float(pop[tt].w[q] & 0xFFFF0000u);
                                plo[tt].w[q] = pack2<MT>(pr[2 * q] - h0, pr[2 * q + 1] - h1);
                            }
                        }
                    }

                    // ---- stage V rows (zero for absent tokens), read back transposed,
                    // each V^T operand serving every tile
#pragma unroll
                    for (int u = 0; u < NPV; ++u) {
                        const int p = u * 64 + lane;
                        uint16_t* dst = vs + (p / PPR) * LDV + (p % PPR) * VEL;
                        if constexpr (BIGB) {
                            const int t = c0 + p / PPR;
                            R.vlive[u] = full || (R.valid && t >= ts && t < te);
                        }
                        if constexpr (KVDT == PA_FP8_E4M3) {
                            uint32_t wv[8];
#pragma unroll
                            for (int q = 0; q < 4; ++q) e4m3x4_widen<MT>(R.v[u].w[q], wv[2 * q], wv[2 * q + 1]);
                            if (!full) {
#pragma unroll
                                for (int q = 0; q < 8; ++q) wv[q] = R.vlive[u] ? wv[q] : 0u;
                            }
                            *reinterpret_cast<uint4*>(dst) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                            *reinterpret_cast<uint4*>(dst + 8) = make_uint4(wv[4], wv[5], wv[6], wv[7]);
                        } else {
                            uint32_t wv[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) wv[q] = R.v[u].w[q];
                            if (!full) {
#pragma unroll
                                for (int q = 0; q < 4; ++q) wv[q] = R.vlive[u] ? wv[q] : 0u;
                            }
                            *reinterpret_cast<uint4*>(dst) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                        }
                    }
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        // V^T[d][token]: column d = 16 dt + c16, tokens 4j..4j+3
                        const Op4 vop = read_tr16(vs + (4 * j + (c16 >> 2)) * LDV + 16 * dt + 4 * (c16 & 3));
#pragma unroll
                        for (int tt = 0; tt < TILES; ++tt) {
                            acc[tt][dt] = mma16<MT>(vop, pop[tt], acc[tt][dt]);
                            if constexpr (MT == PA_BF16) acc[tt][dt] = mma16<MT>(vop, plo[tt], acc[tt][dt]);
                        }
                    }
                    __builtin_amdgcn_wave_barrier();
                };

                // a ring of PD register sets: chunk i lives in set i mod PD, and the
                // loads of chunk i + PD - 1 are issued just before chunk i is computed
                ChunkRegs ring[PD];
#pragma unroll
                for (int k = 0; k < PD - 1; ++k) load_chunk(ring[k], c_begin + k * kChunk);
                for (int c0 = c_begin; c0 < te; c0 += PD * kChunk) {
                    bool done = false;
#pragma unroll
                    for (int k = 0; k < PD; ++k) {
                        if (!done) {
                            load_chunk(ring[(k + PD - 1) % PD], c0 + (k + PD - 1) * kChunk);
                            compute_chunk(ring[k], c0 + k * kChunk);
                            done = c0 + (k + 1) * kChunk >= te;
                        }
                    }
                    if (done) break;
                }
            }

            // ---- per-column totals, then this wavefront's result for its item
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
                float lt = l[tt];
                lt = sum_over_groups(lt);
                const int hu = 16 * tt + c16;
                if (hu < nh) {
                    const int head = kvh * G + hg0 + hu;
                    const float inv_l = lt > 0.0f ? 1.0f / lt : 0.0f;
                    const int64_t r = cur.rec0 + (int64_t)hu * cur.rec_stride;
                    if (!cur.whole && j == 0) {
                        a.ws[r] = m[tt];
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
                                make_uint2(pack2<QDT>(acc[tt][dt][0] * f, acc[tt][dt][1] * f),
                                           pack2<QDT>(acc[tt][dt][2] * f, acc[tt][dt][3] * f));
                        } else {
                            float* wo = a.ws + 2 * a.nrec + r * D + d;
#pragma unroll
                            for (int i = 0; i < 4; ++i) wo[i] = acc[tt][dt][i] * inv_l;
                        }
                    }
                }
            }
        }
    }
}

template <int KVDT, int QDT, int D>
hipError_t launch_typed(DecodeArgs& a, hipStream_t stream) {
    constexpr int NW = 4;
    constexpr int TILES = 1;
    constexpr int PD = 3;                    // chunks in flight per wavefront (measured best)
    auto kernel = a.log2_bs >= 4 ? decode_mfma_kernel<KVDT, QDT, D, NW, TILES, PD, true>
                                 : decode_mfma_kernel<KVDT, QDT, D, NW, TILES, PD, false>;
    a.unit_heads = a.num_heads / a.num_kv_heads;        // a unit: every query head of a KV head
    a.units_per_kv = 1;
    a.seg_cost = 64;                                    // an item start, in tokens (measured)
    const int64_t grid = decode_grid(reinterpret_cast<const void*>(kernel), NW * 64,
                                     a.num_kv_heads, 1, a, kMfmaMaxWorkersPerCu);
    if (grid < 0) return hipErrorOutOfMemory;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int KVDT, int QDT>
hipError_t launch_dim(DecodeArgs& a, int head_dim, hipStream_t stream) {
    if (head_dim == 64) return launch_typed<KVDT, QDT, 64>(a, stream);
    if (head_dim == 128) return launch_typed<KVDT, QDT, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_mfma_supported(int q_dt, int kv_dt, int head_dim, int group) {
    if (group < 2 || group > 16) return false;
    if (head_dim != 64 && head_dim != 128) return false;
    if (q_dt != PA_F16 && q_dt != PA_BF16) return false;
    return kv_dt == q_dt || kv_dt == PA_FP8_E4M3;
}

hipError_t launch_decode_mfma(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
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

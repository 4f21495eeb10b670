// paged_attention_decode, vector-ALU path: one query head per work item.
//
// The new token's query is dotted with every cached key, the scores become
// softmax weights, and the weighted sum of the cached values is the head's
// output (KV Cache从原理到实战 §2.1); the keys and values are fetched block
// by block through the sequence's block table (KV 缓存与分页注意力 §07 块表).
//
// Work split.  Items come from worklist.h; each wavefront is a worker that
// streams its items.  It reads a chunk of CH tokens per step: each 16-byte
// load covers VEC numbers of one token row, LPR = head_dim / VEC lanes cover
// a row and one load instruction covers RPI = 64 / LPR consecutive token rows
// (16-byte vector loads, coalesced within a (block, head) tile).  Each lane
// keeps a running max / sum / fp32 accumulator (online softmax) over the
// tokens of its own lane-row; the row's partial dot products are summed with
// DPP and lane-rows are merged with shuffles at the end of the item.  Scores
// are kept in log2 units so that v_exp_f32 computes the exponentials.
//
// An int8 cache (group-wise codes with one scale per token and KV head) is read
// as biased codes (code + 128, see int8x16_biased): a token's score is
// (q . (c + 128) - 128 sum q) * k_scale, and its value enters the accumulator
// weighted by p * v_scale, with 128 times the sum of those weights taken off
// once at the end of the item.
//
// A cut item (split context) writes its (max, sum, normalised output) to the
// workspace and a reduction kernel below merges the pieces; an item that holds
// a whole context writes the output directly.
#include "kernels.h"
#include "pa_device.h"
#include "worklist.h"

#include <map>
#include <mutex>
#include <tuple>

namespace pa {
namespace {

constexpr int kTableCap = 1024;     // block-table entries staged in LDS per segment
constexpr float kNegInf = -__builtin_inff();

template <int KVDT, int QDT, int D, int NW, int U>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(DecodeArgs a) {
    constexpr int EB = elem_bytes(KVDT);
    constexpr int VEC = 16 / EB;             // numbers per 16-byte load
    constexpr int LPR = D / VEC;             // lanes per token row
    constexpr int RPI = 64 / LPR;            // token rows per load instruction
    constexpr int CH = RPI * U;              // tokens per wavefront step
    constexpr int NT = NW * 64;
    static_assert(LPR >= 4 && LPR <= 32, "row split");

    constexpr int WT = kTableCap / NW;       // block-table entries staged per wavefront
    __shared__ int32_t tbl_all[NW][WT];
    __shared__ __attribute__((aligned(8))) int32_t wl_lds[kListInts];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane / LPR;
    const int col = lane % LPR;
    const int bs = 1 << a.log2_bs;
    const int G = a.num_heads / a.num_kv_heads;
    const char* kbase = reinterpret_cast<const char*>(a.k_pool);
    const char* vbase = reinterpret_cast<const char*>(a.v_pool);
    int32_t* tbl = tbl_all[wave];

    Schedule<NT> sch;
    for (int s0 = 0; s0 < a.num_seqs; s0 += kWindow) {
        sch.build(a, s0, min(kWindow, a.num_seqs - s0), a.num_heads, wl_lds,
                  worker_id(wave, NW), gridDim.x * NW, lane == 0);
        Item itm;
        while (sch.next(a, itm)) {
            const int s = itm.s;
            const int h = itm.unit;
            const int kvh = h / G;
            // first loads of the item, issued together: block-table segment, query
            const int t0 = itm.t0, t1 = itm.t1;
            const int32_t* trow = a.tables + (int64_t)s * a.max_blocks;
            TablePrefetch<64, WT> tpre;
            tpre.issue(trow, t0 >> a.log2_bs, table_span(a, t0, t1, WT), a.max_blocks, lane);

            // query slice of this lane, pre-scaled into log2 units
            float qf[VEC];
            {
                const char* qp = reinterpret_cast<const char*>(a.q) +
                                 (((int64_t)s * a.num_heads + h) * D + col * VEC) * elem_bytes(QDT);
                constexpr int QV = 16 / elem_bytes(QDT);
#pragma unroll
                for (int i = 0; i < VEC; i += QV)
                    unpack16<QDT>(load16(qp + i * elem_bytes(QDT)), qf + i);
#pragma unroll
                for (int i = 0; i < VEC; ++i) qf[i] *= a.qk_scale;
            }
            __builtin_amdgcn_s_waitcnt(0);
            float qbias = 0.0f;                      // int8: 128 * this lane's sum of q
            if constexpr (KVDT == PA_INT8) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) qbias += qf[i];
                qbias *= 128.0f;
            }

            float m = kNegInf, l = 0.0f, wsum = 0.0f;   // wsum: int8, sum of p * v_scale
            float acc[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;

            const int64_t head_off = (int64_t)kvh << a.log2_bs;   // token rows within a block
            const int b_first = t0 >> a.log2_bs;
            const int b_end = (t1 + bs - 1) >> a.log2_bs;
            for (int sb = b_first; sb < b_end; sb += WT) {
                const int se = min(b_end, sb + WT);
                __builtin_amdgcn_wave_barrier();
                if (sb == b_first) {
                    tpre.store(tbl, se - sb, a.num_blocks, lane);
                } else {
                    for (int i = lane; i < se - sb; i += 64) {
                        const int b = trow[sb + i];
                        tbl[i] = (b >= 0 && b < a.num_blocks) ? b : -1;
                    }
                }
                __builtin_amdgcn_wave_barrier();
                const int ts = max(t0, sb << a.log2_bs);
                const int te = min(t1, se << a.log2_bs);
                for (int c = ts; c < te; c += CH) {
                    Raw16 kr[U], vr[U];
                    bool valid[U];
                    float kst[U], vst[U];                // int8: the tokens' scales
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int t = c + u * RPI + row;
                        int blk = -1;
                        if (t < te) blk = tbl[(t >> a.log2_bs) - sb];
                        valid[u] = blk >= 0;
                        const int64_t r = valid[u] ? ((int64_t)blk * a.num_kv_heads << a.log2_bs) +
                                                         head_off + (t & (bs - 1))
                                                   : 0;
                        const int64_t byte_off = (r * D + col * VEC) * EB;
                        kr[u] = load16_stream(kbase + byte_off);
                        vr[u] = load16_stream(vbase + byte_off);
                        if constexpr (KVDT == PA_INT8) {   // scale pools share the row index
                            kst[u] = a.k_scales[r];
                            vst[u] = a.v_scales[r];
                        }
                    }
                    float sc[U];
                    float mc = kNegInf;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float kf[VEC];
                        if constexpr (KVDT == PA_INT8) int8x16_biased(kr[u], kf);
                        else unpack16<KVDT>(kr[u], kf);
                        float dot = 0.0f;
#pragma unroll
                        for (int i = 0; i < VEC; ++i) dot = __builtin_fmaf(qf[i], kf[i], dot);
                        if constexpr (KVDT == PA_INT8) dot -= qbias;
                        dot = group_sum<LPR>(dot);
                        if constexpr (KVDT == PA_INT8) dot *= kst[u];
                        sc[u] = valid[u] ? dot : kNegInf;
                        mc = fmaxf(mc, sc[u]);
                    }
                    const float mn = fmaxf(m, mc);
                    if (mn != kNegInf) {
                        const float alpha = fast_exp2(m - mn);
                        l *= alpha;
                        if constexpr (KVDT == PA_INT8) wsum *= alpha;
#pragma unroll
                        for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            if (valid[u]) {
                                float pu = fast_exp2(sc[u] - mn);
                                l += pu;
                                float vf[VEC];
                                if constexpr (KVDT == PA_INT8) {
                                    pu *= vst[u];
                                    wsum += pu;
                                    int8x16_biased(vr[u], vf);
                                } else {
                                    unpack16<KVDT>(vr[u], vf);
                                }
#pragma unroll
                                for (int i = 0; i < VEC; ++i) acc[i] = __builtin_fmaf(pu, vf[i], acc[i]);
                            }
                        }
                        m = mn;
                    }
                }
            }
            if constexpr (KVDT == PA_INT8) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] = __builtin_fmaf(-128.0f, wsum, acc[i]);
            }

            // merge the lane-rows of this wavefront (same column, disjoint tokens)
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) {
                const float m2 = __shfl_xor(m, off, 64);
                const float l2 = __shfl_xor(l, off, 64);
                const float mn = fmaxf(m, m2);
                const float fa = (m == kNegInf) ? 0.0f : fast_exp2(m - mn);
                const float fb = (m2 == kNegInf) ? 0.0f : fast_exp2(m2 - mn);
                l = l * fa + l2 * fb;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float a2 = __shfl_xor(acc[i], off, 64);
                    acc[i] = acc[i] * fa + a2 * fb;
                }
                m = mn;
            }

            // this wavefront's result for its item (lanes of row 0 hold it)
            if (row == 0) {
                const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
                if (itm.whole) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) acc[i] *= inv_l * a.out_scale;
                    char* op = reinterpret_cast<char*>(a.out) +
                               (((int64_t)s * a.num_heads + h) * D + col * VEC) * elem_bytes(QDT);
                    store_vals<QDT>(op, acc, VEC);
                } else {
                    const int64_t r = itm.rec0;
                    if (col == 0) {
                        a.ws[r] = m;
                        a.ws[a.nrec + r] = l;
                    }
#pragma unroll
                    for (int i = 0; i < VEC; ++i) a.ws[2 * a.nrec + r * D + col * VEC + i] = acc[i] * inv_l;
                }
            }
        }
    }
}

template <int QDT>
__device__ __forceinline__ void store_one(void* out, int64_t i, float v) {
    if constexpr (QDT == PA_F32) {
        reinterpret_cast<float*>(out)[i] = v;
    } else if constexpr (QDT == PA_F16) {
        reinterpret_cast<_Float16*>(out)[i] = (_Float16)v;
    } else {
        reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// Log-sum-exp merge of n partial records (m, l, o) of one head, for this
// lane's D/64 dimensions: out = sum_k w_k o_k / sum_k w_k with
// w_k = 2^(m_k - max m) l_k, accumulated online (the running maximum rescales
// what is already summed).  Records are fetched kMergeBatch at a time so that
// their loads overlap; `rec(k)` is the index of the k-th record.
constexpr int kMergeBatch = 8;
template <int QDT, int D, typename Rec>
__device__ __forceinline__ void merge_records(const DecodeArgs& a, int n, Rec rec, int64_t out_row) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    float M = kNegInf, den = 0.0f, num[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) num[j] = 0.0f;
    for (int k0 = 0; k0 < n; k0 += kMergeBatch) {
        float mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch][PER];
#pragma unroll
        for (int q = 0; q < kMergeBatch; ++q) {
            const int64_t r = rec(min(k0 + q, n - 1));
            mv[q] = a.ws[r];
            lv[q] = a.ws[a.nrec + r];
#pragma unroll
            for (int j = 0; j < PER; ++j) ov[q][j] = a.ws[2 * a.nrec + r * D + j * 64 + lane];
        }
#pragma unroll
        for (int q = 0; q < kMergeBatch; ++q) {
            if (k0 + q < n && mv[q] != kNegInf) {
                const float Mn = fmaxf(M, mv[q]);
                const float sc = (M == kNegInf) ? 0.0f : fast_exp2(M - Mn);
                const float w = fast_exp2(mv[q] - Mn) * lv[q];
                den = den * sc + w;
#pragma unroll
                for (int j = 0; j < PER; ++j) num[j] = num[j] * sc + w * ov[q][j];
                M = Mn;
            }
        }
    }
    const float f = den > 0.0f ? a.out_scale / den : 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) store_one<QDT>(a.out, out_row * D + j * 64 + lane, num[j] * f);
}

// Partitions: merge the partitions of every (sequence, head) that has more
// than one; one wavefront per (sequence, head).
template <int QDT, int D>
__global__ __launch_bounds__(64) void lse_reduce_kernel(DecodeArgs a) {
    const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
    for (int64_t sh = blockIdx.x; sh < pairs; sh += gridDim.x) {
        const int s = (int)(sh / a.num_heads);
        const int np = parts_of(clamp_ctx(a.ctx_lens[s], a.ctx_cap), a.part_tokens);
        if (np <= 1) continue;                         // written by the attention kernel
        merge_records<QDT, D>(a, np, [&](int k) { return sh * a.num_parts + k; }, sh);
    }
}

// Balanced split: merge every segment whose tokens a worker range boundary
// cuts.  The worker whose range starts inside the segment's tokens and reaches
// past their end holds the last piece; its descriptor names the segment, and
// the pieces are held by workers first..b (first: slot 1 unless its range
// starts exactly at the segment, every other one: slot 0).  One wavefront per
// (worker, pass): it reads the worker's descriptor and, if the worker holds
// such a last piece, merges its pass's share of the unit's heads, 64 / (D / 16)
// heads with 16 consecutive dimensions of one head per lane (so every record
// is fetched in 16-byte pieces, all records of a batch at once).  The passes of
// a large unit run side by side instead of one after another.
template <int QDT, int D>
__global__ __launch_bounds__(256) void split_reduce_kernel(DecodeArgs a) {
    constexpr int LPH = D / 16;                 // lanes per head
    constexpr int HP = 64 / LPH;                // heads per pass
    constexpr int B = 4;                        // records per batch
    const int64_t windows = (a.num_seqs + kWindow - 1) / kWindow;
    const int GR = a.unit_heads;                        // record slots per unit
    const int NP = (GR + HP - 1) / HP;                  // passes per worker
    const int lane = threadIdx.x & 63;
    const int hl = lane / LPH, d0 = (lane % LPH) * 16;
    const int64_t wv = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (wv >= windows * a.workers * NP) return;
    const int pass = (int)(wv % NP);
    const int64_t wb = wv / NP;
    const int64_t win = wb / a.workers, b = wb % a.workers;
    const int h0 = pass * HP;
    // The common case, a segment cut once that started inside worker b - 1's range, has
    // its pieces in slot 1 of worker b - 1 and slot 0 of worker b: their records are
    // loaded together with the descriptor (in bounds whatever the descriptor says; used
    // only in that case).
    float smv[2], slv[2];
    float4 sov[2][4];
    {
        const int isp = min(h0 + hl, GR - 1);
        const int64_t rs[2] = {((win * a.workers + (b > 0 ? b - 1 : b)) * 2 + 1) * GR + isp,
                               ((win * a.workers + b) * 2 + 0) * GR + isp};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            smv[q] = a.ws[rs[q]];
            slv[q] = a.ws[a.nrec + rs[q]];
            const float4* op = reinterpret_cast<const float4*>(a.ws + 2 * a.nrec + rs[q] * D + d0);
#pragma unroll
            for (int v = 0; v < 4; ++v) sov[q][v] = op[v];
        }
    }
    const int64_t* d = a.desc + wb * kDescWords;
    const int64_t t0 = d[1], range = d[3];
    const int64_t run = split_run((int)d[4]);
    if (t0 <= 0 || t0 >= run) return;                   // no cut tokens end in this range
    const int64_t start = b * range - t0;               // the segment's first token, range space
    if (start + run > (b + 1) * range) return;          // a later range holds the last piece
    const int64_t first = start / range;
    const int n = (int)(b - first + 1);
    const int s = (int)(d[0] & 0xFFFFFFFF), unit = (int)(d[0] >> 32);
    const int Gq = a.num_heads / a.num_kv_heads;
    const int hg0 = (unit % a.units_per_kv) * GR;
    const int nh = min(GR, Gq - hg0);                   // heads of the unit
    const int64_t head0 = (int64_t)(unit / a.units_per_kv) * Gq + hg0;
    if (h0 >= nh) return;
    const int i = min(h0 + hl, nh - 1);                 // lanes past the unit repeat its last head
    auto rec = [&](int k) -> int64_t {
        const int64_t w = first + k;
        return ((win * a.workers + w) * 2 + (w * range >= start ? 0 : 1)) * GR + i;
    };
    float M = kNegInf, den = 0.0f, num[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) num[e] = 0.0f;
    // online merge of one piece's record (pieces in range order)
    auto take = [&](float mq, float lq, const float4* oq) {
        if (mq != kNegInf) {
            const float Mn = fmaxf(M, mq);
            const float sc = (M == kNegInf) ? 0.0f : fast_exp2(M - Mn);
            const float w = fast_exp2(mq - Mn) * lq;
            den = den * sc + w;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                num[4 * v + 0] = num[4 * v + 0] * sc + w * oq[v].x;
                num[4 * v + 1] = num[4 * v + 1] * sc + w * oq[v].y;
                num[4 * v + 2] = num[4 * v + 2] * sc + w * oq[v].z;
                num[4 * v + 3] = num[4 * v + 3] * sc + w * oq[v].w;
            }
            M = Mn;
        }
    };
    if (n == 2 && t0 < range) {                         // the records loaded up front (a segment
                                                        // starting a range keeps its slot 0 there)
        take(smv[0], slv[0], sov[0]);
        take(smv[1], slv[1], sov[1]);
    } else {
        for (int k0 = 0; k0 < n; k0 += B) {
            float mv[B], lv[B];
            float4 ov[B][4];
#pragma unroll
            for (int q = 0; q < B; ++q) {
                const int64_t r = rec(min(k0 + q, n - 1));
                mv[q] = a.ws[r];
                lv[q] = a.ws[a.nrec + r];
                const float4* op = reinterpret_cast<const float4*>(a.ws + 2 * a.nrec + r * D + d0);
#pragma unroll
                for (int v = 0; v < 4; ++v) ov[q][v] = op[v];
            }
#pragma unroll
            for (int q = 0; q < B; ++q)
                if (k0 + q < n) take(mv[q], lv[q], ov[q]);
        }
    }
    if (h0 + hl < nh) {
        const float f = den > 0.0f ? a.out_scale / den : 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) num[e] *= f;
        char* op = reinterpret_cast<char*>(a.out) +
                   (((int64_t)s * a.num_heads + head0 + i) * D + d0) * elem_bytes(QDT);
        store_vals<QDT>(op, num, 16);
    }
}

template <int KVDT, int QDT, int D>
hipError_t launch_typed(DecodeArgs& a, hipStream_t stream) {
    constexpr int NW = 4;
    constexpr int U = 4;
    auto kernel = decode_valu_kernel<KVDT, QDT, D, NW, U>;
    a.unit_heads = 1;                                   // a unit is one query head
    a.seg_cost = 16;                                    // an item start, in tokens (measured)
    a.units_per_kv = a.num_heads / a.num_kv_heads;
    const int64_t grid = decode_grid(reinterpret_cast<const void*>(kernel), NW * 64, a.num_heads, 1, a);
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

hipError_t launch_valu(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                       hipStream_t stream) {
    if (kv_dt == q_dt) {
        switch (kv_dt) {
            case PA_F32: return launch_dim<PA_F32, PA_F32>(a, head_dim, stream);
            case PA_F16: return launch_dim<PA_F16, PA_F16>(a, head_dim, stream);
            case PA_BF16: return launch_dim<PA_BF16, PA_BF16>(a, head_dim, stream);
        }
    } else if (kv_dt == PA_FP8_E4M3) {
        switch (q_dt) {
            case PA_F32: return launch_dim<PA_FP8_E4M3, PA_F32>(a, head_dim, stream);
            case PA_F16: return launch_dim<PA_FP8_E4M3, PA_F16>(a, head_dim, stream);
            case PA_BF16: return launch_dim<PA_FP8_E4M3, PA_BF16>(a, head_dim, stream);
        }
    } else if (kv_dt == PA_INT8) {
        switch (q_dt) {
            case PA_F32: return launch_dim<PA_INT8, PA_F32>(a, head_dim, stream);
            case PA_F16: return launch_dim<PA_INT8, PA_F16>(a, head_dim, stream);
            case PA_BF16: return launch_dim<PA_INT8, PA_BF16>(a, head_dim, stream);
        }
    }
    return hipErrorInvalidValue;
}

template <int QDT>
hipError_t launch_reduce(DecodeArgs& a, int head_dim, hipStream_t stream) {
    if (a.part_tokens < 0) {
        const int passes = (a.unit_heads + 64 / (head_dim / 16) - 1) / (64 / (head_dim / 16));
        const int64_t waves = (a.num_seqs + kWindow - 1) / kWindow * (int64_t)a.workers * passes;
        auto k = head_dim == 64 ? split_reduce_kernel<QDT, 64> : split_reduce_kernel<QDT, 128>;
        hipLaunchKernelGGL(k, dim3((uint32_t)((waves + 3) / 4)), dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
    if (head_dim == 64) {
        auto k = lse_reduce_kernel<QDT, 64>;
        const int64_t grid = persistent_grid(reinterpret_cast<const void*>(k), 64, pairs);
        hipLaunchKernelGGL(k, dim3((uint32_t)grid), dim3(64), 0, stream, a);
    } else {
        auto k = lse_reduce_kernel<QDT, 128>;
        const int64_t grid = persistent_grid(reinterpret_cast<const void*>(k), 64, pairs);
        hipLaunchKernelGGL(k, dim3((uint32_t)grid), dim3(64), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

int64_t persistent_grid(const void* kernel, int threads, int64_t max_items) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, int>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const auto key = std::make_tuple(dev, kernel, threads);
    int64_t cap = 0;
    {
        std::lock_guard<std::mutex> g(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            cap = it->second;
        } else {
            int cus = 0, per_cu = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                cus <= 0)
                cus = 256;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) !=
                    hipSuccess ||
                per_cu <= 0)
                per_cu = 1;
            cap = (int64_t)cus * per_cu;
            cache.emplace(key, cap);
        }
    }
    int64_t g = std::min<int64_t>(std::max<int64_t>(max_items, 1), cap);
    if (g >= 8) g -= g % 8;
    return g;
}

int device_cus() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    cache.emplace(dev, cus);
    return cus;
}

int64_t decode_grid(const void* kernel, int threads, int units, int wave_workers, DecodeArgs& a,
                    int max_workers_per_cu) {
    a.units = units;
    a.simds = device_cus() * 4;                         // four SIMDs per compute unit
    const int per_wg = wave_workers ? threads / 64 : 1;
    int64_t grid;
    if (a.part_tokens < 0) {
        grid = persistent_grid(kernel, threads, (int64_t)device_cus() * max_workers_per_cu / per_wg);
        const int64_t windows = (a.num_seqs + kWindow - 1) / kWindow;
        a.nrec = windows * grid * per_wg * 2 * a.unit_heads;
        if (a.rec_capacity >= 0 && a.nrec > a.rec_capacity) return -1;
    } else {
        grid = persistent_grid(kernel, threads, ((int64_t)a.num_seqs * units * a.num_parts + per_wg - 1) / per_wg);
    }
    a.workers = (int32_t)(grid * per_wg);
    return grid;
}

hipError_t launch_decode(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                         hipStream_t stream) {
    const int group = a.num_heads / a.num_kv_heads;
    hipError_t e;
    // the large-group kernel addresses a pool block (every KV head's rows) in 32 bits
    const uint64_t block_bytes = ((uint64_t)a.num_kv_heads << a.log2_bs) * (uint64_t)head_dim *
                                 (uint64_t)elem_bytes(kv_dt);
    if (decode_group_supported(q_dt, kv_dt, head_dim, group) && block_bytes < ((uint64_t)1 << 32))
        e = launch_decode_group(a, q_dt, kv_dt, head_dim, stream);
    else if (decode_mfma_supported(q_dt, kv_dt, head_dim, group))
        e = launch_decode_mfma(a, q_dt, kv_dt, head_dim, stream);
    else
        e = launch_valu(a, q_dt, kv_dt, head_dim, stream);
    if (e != hipSuccess || (a.part_tokens >= 0 && a.num_parts <= 1)) return e;
    switch (q_dt) {
        case PA_F32: return launch_reduce<PA_F32>(a, head_dim, stream);
        case PA_F16: return launch_reduce<PA_F16>(a, head_dim, stream);
        case PA_BF16: return launch_reduce<PA_BF16>(a, head_dim, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa

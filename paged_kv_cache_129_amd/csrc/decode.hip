// paged_attention_decode, vector-ALU path: one workgroup per (sequence,
// query head, partition).
//
// The new token's query is dotted with every cached key, the scores become
// softmax weights, and the weighted sum of the cached values is the head's
// output (KV Cache从原理到实战 §2.1); the keys and values are fetched block
// by block through the sequence's block table (KV 缓存与分页注意力 §07 块表).
//
// Work split.  A wavefront reads a chunk of CH tokens per step: each 16-byte
// load covers VEC numbers of one token row, LPR = head_dim / VEC lanes cover
// a row and one load instruction covers RPI = 64 / LPR consecutive token rows
// (16-byte vector loads, coalesced within a (block, head) tile).  Each lane
// keeps a running max / sum / fp32 accumulator (online softmax) over the
// tokens of its own lane-row; the row's partial dot products are summed with
// DPP, lane-rows are merged at the end with shuffles and the workgroup's
// waves through LDS (log-sum-exp merge).  Scores are kept in log2 units so
// that v_exp_f32 computes the exponentials.
//
// Split context: with more than one partition per sequence each workgroup
// writes its partition's (max, sum, normalised output) to the workspace and
// the reduction kernel below merges them; a sequence with one partition is
// written directly.
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

    __shared__ int32_t tbl[kTableCap];
    __shared__ float merge_ml[NW][2];
    __shared__ float merge_acc[NW][D];
    __shared__ int32_t pref[kWindow + 1];
    __shared__ int32_t scan[NT];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane / LPR;
    const int col = lane % LPR;
    const int bs = 1 << a.log2_bs;
    const int G = a.num_heads / a.num_kv_heads;
    const char* kbase = reinterpret_cast<const char*>(a.k_pool);
    const char* vbase = reinterpret_cast<const char*>(a.v_pool);

    for (int s0 = 0; s0 < a.num_seqs; s0 += kWindow) {
        const int nwin = min(kWindow, a.num_seqs - s0);
        const int total = build_prefix<NT>(a, s0, nwin, pref, scan);
        const int64_t items = (int64_t)total * a.num_heads;
        for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
            const int h = (int)(w % a.num_heads);
            const int gp = (int)(w / a.num_heads);
            const int sl = locate(pref, nwin, gp);
            const int s = s0 + sl;
            const int part = gp - pref[sl];
            const int kvh = h / G;
            // first loads of the item, issued together: block-table segment, length, query
            const int t0 = part * a.part_tokens;
            const int32_t* trow = a.tables + (int64_t)s * a.max_blocks;
            TablePrefetch<NT, kTableCap> tpre;
            tpre.issue(trow, t0 >> a.log2_bs, table_span(a, t0, kTableCap));
            const int ctx_raw = a.ctx_lens[s];

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
            const int ctx = clamp_ctx(ctx_raw, a.ctx_cap);
            const int t1 = min(ctx, t0 + a.part_tokens);
            const int nparts_s = parts_of(ctx, a.part_tokens);

            float m = kNegInf, l = 0.0f;
            float acc[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;

            const int64_t head_off = (int64_t)kvh << a.log2_bs;   // token rows within a block
            const int b_first = t0 >> a.log2_bs;
            const int b_end = (t1 + bs - 1) >> a.log2_bs;
            for (int sb = b_first; sb < b_end; sb += kTableCap) {
                const int se = min(b_end, sb + kTableCap);
                __syncthreads();
                if (sb == b_first) {
                    tpre.store(tbl, se - sb, a.num_blocks);
                } else {
                    for (int i = threadIdx.x; i < se - sb; i += NT) {
                        const int b = trow[sb + i];
                        tbl[i] = (b >= 0 && b < a.num_blocks) ? b : -1;
                    }
                }
                __syncthreads();
                const int ts = max(t0, sb << a.log2_bs);
                const int te = min(t1, se << a.log2_bs);
                for (int c = ts + wave * CH; c < te; c += NW * CH) {
                    Raw16 kr[U], vr[U];
                    bool valid[U];
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
                    }
                    float sc[U];
                    float mc = kNegInf;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float kf[VEC];
                        unpack16<KVDT>(kr[u], kf);
                        float dot = 0.0f;
#pragma unroll
                        for (int i = 0; i < VEC; ++i) dot = __builtin_fmaf(qf[i], kf[i], dot);
                        dot = group_sum<LPR>(dot);
                        sc[u] = valid[u] ? dot : kNegInf;
                        mc = fmaxf(mc, sc[u]);
                    }
                    const float mn = fmaxf(m, mc);
                    if (mn != kNegInf) {
                        const float alpha = fast_exp2(m - mn);
                        l *= alpha;
#pragma unroll
                        for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            if (valid[u]) {
                                const float pu = fast_exp2(sc[u] - mn);
                                l += pu;
                                float vf[VEC];
                                unpack16<KVDT>(vr[u], vf);
#pragma unroll
                                for (int i = 0; i < VEC; ++i) acc[i] = __builtin_fmaf(pu, vf[i], acc[i]);
                            }
                        }
                        m = mn;
                    }
                }
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

            // merge the workgroup's wavefronts through LDS
            if (row == 0) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) merge_acc[wave][col * VEC + i] = acc[i];
                if (col == 0) {
                    merge_ml[wave][0] = m;
                    merge_ml[wave][1] = l;
                }
            }
            __syncthreads();
            if (wave == 0 && row == 0) {
                float M = kNegInf;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, merge_ml[ww][0]);
                float L = 0.0f;
                float o[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i) o[i] = 0.0f;
                if (M != kNegInf) {
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) {
                        const float mw = merge_ml[ww][0];
                        const float f = (mw == kNegInf) ? 0.0f : fast_exp2(mw - M);
                        L += merge_ml[ww][1] * f;
#pragma unroll
                        for (int i = 0; i < VEC; ++i) o[i] += merge_acc[ww][col * VEC + i] * f;
                    }
                }
                const float inv_l = L > 0.0f ? 1.0f / L : 0.0f;
                if (nparts_s == 1) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) o[i] *= inv_l * a.out_scale;
                    char* op = reinterpret_cast<char*>(a.out) +
                               (((int64_t)s * a.num_heads + h) * D + col * VEC) * elem_bytes(QDT);
                    store_vals<QDT>(op, o, VEC);
                } else {
                    const int64_t idx = ((int64_t)s * a.num_heads + h) * a.num_parts + part;
                    const int64_t nslots = (int64_t)a.num_seqs * a.num_heads * a.num_parts;
                    if (col == 0) {
                        a.ws[idx] = M;
                        a.ws[nslots + idx] = L;
                    }
#pragma unroll
                    for (int i = 0; i < VEC; ++i) a.ws[2 * nslots + idx * D + col * VEC + i] = o[i] * inv_l;
                }
            }
            __syncthreads();          // merge buffers are reused by the next item
        }
    }
}

// Merge the partitions of every (sequence, head) that has more than one:
// out = sum_p w_p o_p / sum_p w_p with w_p = 2^(m_p - max m) l_p.
template <int QDT, int D>
__global__ __launch_bounds__(64) void lse_reduce_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
    const int64_t nslots = pairs * a.num_parts;
    for (int64_t sh = blockIdx.x; sh < pairs; sh += gridDim.x) {
        const int s = (int)(sh / a.num_heads);
        const int np = parts_of(clamp_ctx(a.ctx_lens[s], a.ctx_cap), a.part_tokens);
        if (np <= 1) continue;                         // written by the main kernel
        const float* ws_m = a.ws + sh * a.num_parts;
        const float* ws_l = a.ws + nslots + sh * a.num_parts;
        const float* ws_o = a.ws + 2 * nslots + sh * a.num_parts * D;
        float M = kNegInf;
        for (int p = 0; p < np; ++p) M = fmaxf(M, ws_m[p]);
        float num[PER], den = 0.0f;
#pragma unroll
        for (int j = 0; j < PER; ++j) num[j] = 0.0f;
        if (M != kNegInf) {
            for (int p = 0; p < np; ++p) {
                const float mp = ws_m[p];
                const float w = (mp == kNegInf) ? 0.0f : fast_exp2(mp - M) * ws_l[p];
                den += w;
#pragma unroll
                for (int j = 0; j < PER; ++j) num[j] += w * ws_o[p * D + j * 64 + threadIdx.x];
            }
        }
        const float f = den > 0.0f ? a.out_scale / den : 0.0f;
        char* op = reinterpret_cast<char*>(a.out) + sh * D * elem_bytes(QDT);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const float v = num[j] * f;
            const int d = j * 64 + threadIdx.x;
            if constexpr (QDT == PA_F32) {
                reinterpret_cast<float*>(op)[d] = v;
            } else if constexpr (QDT == PA_F16) {
                reinterpret_cast<_Float16*>(op)[d] = (_Float16)v;
            } else {
                reinterpret_cast<uint16_t*>(op)[d] = (uint16_t)f32_to_bf16_bits(v);
            }
        }
    }
}

template <int KVDT, int QDT, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    constexpr int NW = 4;
    constexpr int U = 4;
    auto kernel = decode_valu_kernel<KVDT, QDT, D, NW, U>;
    const int64_t grid = persistent_grid(reinterpret_cast<const void*>(kernel), NW * 64,
                                         (int64_t)a.num_seqs * a.num_heads * a.num_parts);
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int KVDT, int QDT>
hipError_t launch_dim(const DecodeArgs& a, int head_dim, hipStream_t stream) {
    if (head_dim == 64) return launch_typed<KVDT, QDT, 64>(a, stream);
    if (head_dim == 128) return launch_typed<KVDT, QDT, 128>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_valu(const DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
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
    }
    return hipErrorInvalidValue;
}

template <int QDT>
hipError_t launch_reduce(const DecodeArgs& a, int head_dim, hipStream_t stream) {
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

hipError_t launch_decode(const DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                         hipStream_t stream) {
    const int group = a.num_heads / a.num_kv_heads;
    hipError_t e;
    if (decode_mfma_supported(q_dt, kv_dt, head_dim, group))
        e = launch_decode_mfma(a, q_dt, kv_dt, head_dim, stream);
    else if (decode_mqa_supported(q_dt, kv_dt, head_dim, group))
        e = launch_decode_mqa(a, q_dt, kv_dt, head_dim, stream);
    else
        e = launch_valu(a, q_dt, kv_dt, head_dim, stream);
    if (e != hipSuccess || a.num_parts <= 1) return e;
    switch (q_dt) {
        case PA_F32: return launch_reduce<PA_F32>(a, head_dim, stream);
        case PA_F16: return launch_reduce<PA_F16>(a, head_dim, stream);
        case PA_BF16: return launch_reduce<PA_BF16>(a, head_dim, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa

// paged_attention_decode, matrix-core path for large query groups (G > 16
// query heads per KV head, e.g. multi-query attention where every head shares
// one KV head: KV 缓存与分页注意力 §11; KV Cache从原理到实战 §5.3).
//
// A work item = (sequence, KV head, partition) from the compact work list of
// worklist.h.  The workgroup has HT wavefronts, one per tile of 16 query
// heads, and they all read the same K/V: for each 32-token chunk every thread
// of the workgroup loads its share of the K and V rows (16-byte loads,
// prefetched into registers one chunk ahead), widens them to the 16-bit MFMA
// type and stores them in a double-buffered LDS pair — K row-major (the A
// operand of S^T = K·Q^T is read with 16-byte LDS loads) and V transposed
// (the A operand of O^T = V^T·P^T is read with 8-byte LDS loads).  One barrier
// per chunk.  Each wavefront then runs the score MFMAs for its 16 heads, the
// online softmax per head column (running max in log2 units) and the P·V
// MFMAs; as the wavefronts own disjoint heads, no cross-wave merge is needed.
#include "kernels.h"
#include "pa_device.h"
#include "worklist.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTableCap = 1024;
constexpr int kChunk = 32;
constexpr float kNegInf = -__builtin_inff();

struct Op8 {
    uint32_t w[4];
};

template <int MT>
__device__ __forceinline__ f32x4 mma(const Op8& a, const Op8& b, f32x4 c) {
    if constexpr (MT == PA_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    half2_t h;
    h.x = (_Float16)a;
    h.y = (_Float16)b;
    return __builtin_bit_cast(uint32_t, h);
}

template <int MT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (MT == PA_F16) return pack_f16(a, b);
    return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

template <int KVDT, int QDT, int D, int HT>
__global__ __launch_bounds__(HT * 64) void decode_mqa_kernel(DecodeArgs a) {
    constexpr int MT = (KVDT == PA_FP8_E4M3) ? PA_F16 : KVDT;
    constexpr int EB = elem_bytes(KVDT);
    constexpr int NT = HT * 64;
    constexpr int NC = D / 32;
    constexpr int NDT = D / 16;
    constexpr int LDK = D + 8;                   // K row stride in LDS (halfs)
    constexpr int LDT = kChunk + 8;              // V^T row stride in LDS (halfs)
    constexpr int VEL = 16 / EB;                 // numbers per 16-byte piece
    constexpr int PPR = D / VEL;                 // pieces per token row
    constexpr int PPC = kChunk * PPR;            // pieces per chunk, one tensor
    constexpr int NPT = (2 * PPC + NT - 1) / NT; // pieces per thread (K and V)
    constexpr int PD = NPT <= 2 ? 4 : 2;         // chunks in flight per workgroup (register ring)
    constexpr int KBUF = kChunk * LDK;
    constexpr int VBUF = D * LDT;

    __shared__ int32_t tbl[kTableCap];
    __shared__ __attribute__((aligned(16))) uint16_t kst[2][KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t vst[2][VBUF];
    __shared__ __attribute__((aligned(8))) int32_t wl_lds[kListInts];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane >> 4;
    const int c16 = lane & 15;
    const int G = a.num_heads / a.num_kv_heads;
    const int bs = 1 << a.log2_bs;
    const char* kbase = reinterpret_cast<const char*>(a.k_pool);
    const char* vbase = reinterpret_cast<const char*>(a.v_pool);
    const int64_t row_bytes = (int64_t)D * EB;

    Schedule<NT> sch;
    for (int s0 = 0; s0 < a.num_seqs; s0 += kWindow) {
        sch.build(a, s0, min(kWindow, a.num_seqs - s0), a.num_kv_heads, wl_lds, blockIdx.x,
                  gridDim.x, threadIdx.x == 0);
        Item itm;
        while (sch.next(a, itm)) {
            const int s = itm.s;
            const int kvh = itm.unit;
            // first loads of the item, issued together: block-table segment, query
            const int t0 = itm.t0, t1 = itm.t1;
            const int32_t* trow = a.tables + (int64_t)s * a.max_blocks;
            TablePrefetch<NT, kTableCap> tpre;
            tpre.issue(trow, t0 >> a.log2_bs, table_span(a, t0, t1, kTableCap), a.max_blocks,
                       threadIdx.x);
            const int hl = wave * 16 + c16;            // head within the group
            const bool head_live = hl < G;

            // B operand of the score MFMA for this wave's 16 heads
            Op8 qop[NC];
            {
                const char* qrow = reinterpret_cast<const char*>(a.q) +
                                   ((int64_t)s * a.num_heads + kvh * G + (head_live ? hl : 0)) * D *
                                       elem_bytes(QDT);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    Op8 o{{0u, 0u, 0u, 0u}};
                    if (head_live) {
                        const int d = 32 * c + 8 * j;
                        if constexpr (QDT == MT) {
                            const Raw16 r = load16(qrow + d * 2);
#pragma unroll
                            for (int q = 0; q < 4; ++q) o.w[q] = r.w[q];
                        } else {
                            float f[8];
                            unpack16<QDT>(load16(qrow + d * elem_bytes(QDT)), f);
#pragma unroll
                            for (int q = 0; q < 4; ++q) o.w[q] = pack2<MT>(f[2 * q], f[2 * q + 1]);
                        }
                    }
                    qop[c] = o;
                }
            }
            // settle the one-time loads here: the wait-count analysis cannot see across
            // the token loop's back edge that they completed, and would otherwise wait
            // for every outstanding load (the prefetches too) at the first score MFMA
            __builtin_amdgcn_s_waitcnt(0);

            float m = kNegInf, l = 0.0f;
            f32x4 acc[NDT];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

            const int b_first = t0 >> a.log2_bs;
            const int b_end = (t1 + bs - 1) >> a.log2_bs;
            for (int sb = b_first; sb < b_end; sb += kTableCap) {
                const int se = min(b_end, sb + kTableCap);
                __syncthreads();
                if (sb == b_first) {
                    tpre.store(tbl, se - sb, a.num_blocks, threadIdx.x);
                } else {
                    for (int i = threadIdx.x; i < se - sb; i += NT) {
                        const int b = trow[sb + i];
                        tbl[i] = (b >= 0 && b < a.num_blocks) ? b : -1;
                    }
                }
                __syncthreads();
                const int ts = max(t0, sb << a.log2_bs);
                const int te = min(t1, se << a.log2_bs);
                // branch-free, so that loads issued around it keep precise wait counts
                auto row_of = [&](int t) -> int64_t {
                    const bool in = t < te;
                    const int blk = tbl[in ? (t >> a.log2_bs) - sb : 0];
                    const int64_t r = (((int64_t)blk * a.num_kv_heads + kvh) << a.log2_bs) + (t & (bs - 1));
                    return (in && blk >= 0) ? r : (int64_t)-1;
                };

                // this thread's pieces of a chunk: piece q < PPC is K, else V.  A ring
                // of PD register sets keeps PD chunks in flight.
                Raw16 pre[PD][NPT];
                bool prelive[PD][NPT];
                auto fetch = [&](int slot, int c0) {
#pragma unroll
                    for (int u = 0; u < NPT; ++u) {
                        const int q = u * NT + threadIdx.x;
                        const int qq = q < PPC ? q : q - PPC;
                        const int64_t r = (q < 2 * PPC) ? row_of(c0 + qq / PPR) : -1;
                        prelive[slot][u] = r >= 0;
                        const char* base = q < PPC ? kbase : vbase;
                        pre[slot][u] = load16_stream(base + (r < 0 ? 0 : r) * row_bytes + (qq % PPR) * 16);
                    }
                };
                auto stage = [&](int slot, int buf) {
#pragma unroll
                    for (int u = 0; u < NPT; ++u) {
                        const int q = u * NT + threadIdx.x;
                        if (q >= 2 * PPC) continue;
                        const int qq = q < PPC ? q : q - PPC;
                        const int t = qq / PPR, d0 = (qq % PPR) * VEL;
                        uint32_t hw[VEL / 2];
                        if constexpr (KVDT == PA_FP8_E4M3) {
#pragma unroll
                            for (int x = 0; x < 4; ++x)
                                e4m3x4_to_f16x4(pre[slot][u].w[x], hw[2 * x], hw[2 * x + 1]);
                        } else {
#pragma unroll
                            for (int x = 0; x < 4; ++x) hw[x] = pre[slot][u].w[x];
                        }
#pragma unroll
                        for (int x = 0; x < VEL / 2; ++x) hw[x] = prelive[slot][u] ? hw[x] : 0u;
                        if (q < PPC) {
                            uint16_t* dst = &kst[buf][t * LDK + d0];
#pragma unroll
                            for (int x = 0; x < VEL / 8; ++x)
                                *reinterpret_cast<uint4*>(dst + 8 * x) =
                                    make_uint4(hw[4 * x], hw[4 * x + 1], hw[4 * x + 2], hw[4 * x + 3]);
                        } else {
#pragma unroll
                            for (int x = 0; x < VEL / 2; ++x) {
                                vst[buf][(d0 + 2 * x) * LDT + t] = (uint16_t)(hw[x] & 0xFFFFu);
                                vst[buf][(d0 + 2 * x + 1) * LDT + t] = (uint16_t)(hw[x] >> 16);
                            }
                        }
                    }
                };
                // scores, online softmax and P·V for the chunk at c0, staged in buffer buf
                auto compute = [&](int c0, int buf) {
                    f32x4 sc[2];
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            const uint4 kv = *reinterpret_cast<const uint4*>(
                                &kst[buf][(16 * tt + c16) * LDK + 32 * c + 8 * j]);
                            const Op8 ko{{kv.x, kv.y, kv.z, kv.w}};
                            sc[tt] = mma<MT>(ko, qop[c], sc[tt]);
                        }
                    }
                    float sv[8];
                    bool live[8];
                    float mx = kNegInf;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tt = e >> 2, i = e & 3;
                        live[e] = row_of(c0 + 16 * tt + 4 * j + i) >= 0;
                        sv[e] = live[e] ? sc[tt][i] * a.qk_scale : kNegInf;
                        mx = fmaxf(mx, sv[e]);
                    }
                    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                    const float mn = fmaxf(m, mx);
                    const float alpha = (m == kNegInf) ? 0.0f : fast_exp2(m - mn);
                    float pr[8];
                    float psum = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        pr[e] = live[e] ? fast_exp2(sv[e] - mn) : 0.0f;
                        psum += pr[e];
                    }
                    l = l * alpha + psum;
                    m = mn;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
                    Op8 pop, plo;
#pragma unroll
                    for (int q = 0; q < 4; ++q) pop.w[q] = pack2<MT>(pr[2 * q], pr[2 * q + 1]);
                    if constexpr (MT == PA_BF16) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float h0 = __uint_as_float(pop.w[q] << 16);
                            const float h1 = __uint_as_float(pop.w[q] & 0xFFFF0000u);
                            plo.w[q] = pack2<MT>(pr[2 * q] - h0, pr[2 * q + 1] - h1);
                        }
                    }
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        // k slots e<4: tokens 4j..4j+3 of tile 0; e>=4: of tile 1
                        const uint16_t* vrow = &vst[buf][(16 * dt + c16) * LDT];
                        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * j);
                        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * j);
                        const Op8 vo{{lo.x, lo.y, hi.x, hi.y}};
                        acc[dt] = mma<MT>(vo, pop, acc[dt]);
                        if constexpr (MT == PA_BF16) acc[dt] = mma<MT>(vo, plo, acc[dt]);
                    }
                };

                // chunk i of this segment starts at ts + i*kChunk; chunk i sits in ring
                // slot i % PD and LDS buffer i % 2 (PD is even, so both are static below)
                const int nch = (te - ts + kChunk - 1) / kChunk;
#pragma unroll
                for (int k = 0; k < PD; ++k)
                    if (k < nch) fetch(k, ts + k * kChunk);
                if (nch > 0) stage(0, 0);
                __syncthreads();
                if (PD < nch) fetch(0, ts + PD * kChunk);
                for (int i0 = 0; i0 < nch; i0 += PD) {
#pragma unroll
                    for (int k = 0; k < PD; ++k) {
                        const int i = i0 + k;
                        if (i < nch) {
                            compute(ts + i * kChunk, k & 1);
                            if (i + 1 < nch) stage((k + 1) % PD, (k + 1) & 1);
                        }
                        __syncthreads();
                        if (i + 1 + PD < nch) fetch((k + 1) % PD, ts + (i + 1 + PD) * kChunk);
                    }
                }
            }

            l += __shfl_xor(l, 16, 64);
            l += __shfl_xor(l, 32, 64);
            if (head_live) {
                const int head = kvh * G + hl;
                const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
                const int64_t r = itm.rec0 + (int64_t)hl * itm.rec_stride;
                if (!itm.whole && j == 0) {
                    a.ws[r] = m;
                    a.ws[a.nrec + r] = l;
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int d = 16 * dt + 4 * j;
                    if (itm.whole) {
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
            __syncthreads();
        }
    }
}

template <int KVDT, int QDT, int D, int HT>
hipError_t launch_ht(DecodeArgs& a, hipStream_t stream) {
    auto kernel = decode_mqa_kernel<KVDT, QDT, D, HT>;
    const int64_t grid = decode_grid(reinterpret_cast<const void*>(kernel), HT * 64, a.num_kv_heads, 0, a);
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(HT * 64), 0, stream, a);
    return hipGetLastError();
}

template <int KVDT, int QDT, int D>
hipError_t launch_d(DecodeArgs& a, int group, hipStream_t stream) {
    const int tiles = (group + 15) / 16;
    if (tiles <= 2) return launch_ht<KVDT, QDT, D, 2>(a, stream);
    if (tiles <= 4) return launch_ht<KVDT, QDT, D, 4>(a, stream);
    if (tiles <= 5) return launch_ht<KVDT, QDT, D, 5>(a, stream);
    return launch_ht<KVDT, QDT, D, 8>(a, stream);
}

template <int KVDT, int QDT>
hipError_t launch_t(DecodeArgs& a, int head_dim, int group, hipStream_t stream) {
    if (head_dim == 64) return launch_d<KVDT, QDT, 64>(a, group, stream);
    return launch_d<KVDT, QDT, 128>(a, group, stream);
}

}  // namespace

bool decode_mqa_supported(int q_dt, int kv_dt, int head_dim, int group) {
    if (group <= 16 || group > 128) return false;
    if (head_dim != 64 && head_dim != 128) return false;
    if (q_dt != PA_F16 && q_dt != PA_BF16) return false;
    return kv_dt == q_dt || kv_dt == PA_FP8_E4M3;
}

hipError_t launch_decode_mqa(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                             hipStream_t stream) {
    const int group = a.num_heads / a.num_kv_heads;
    if (kv_dt == PA_F16 && q_dt == PA_F16) return launch_t<PA_F16, PA_F16>(a, head_dim, group, stream);
    if (kv_dt == PA_BF16 && q_dt == PA_BF16) return launch_t<PA_BF16, PA_BF16>(a, head_dim, group, stream);
    if (kv_dt == PA_FP8_E4M3 && q_dt == PA_F16)
        return launch_t<PA_FP8_E4M3, PA_F16>(a, head_dim, group, stream);
    if (kv_dt == PA_FP8_E4M3 && q_dt == PA_BF16)
        return launch_t<PA_FP8_E4M3, PA_BF16>(a, head_dim, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa

// Multi-token paged attention (prompt phase, chunked prefill), matrix-core
// kernel for gfx950.
//
// The prompt phase computes a whole prompt at once (KV 缓存与分页注意力 §02);
// it is compute-bound where decode is bandwidth-bound (KV Cache从原理到实战
// §2.3), and a long prompt may be cut into chunks (§5.4).  The chunk's K/V
// are written into the paged pool first (kv_cache_write); this kernel then
// reads every token through the block table.  Query row i of a sequence with
// n cached tokens and a q_len-row chunk sits at position p = n - q_len + i and
// attends over tokens 0..p (a causal mask over the new tokens).
//
// Work split.  An item is (sequence, KV head, column block): the columns of
// a (sequence, KV head) are the pairs (query row i, head hl of the KV head's
// group of G), c = i * G + hl, so grouped heads and query rows fill the same
// matrix dimension.  A workgroup of NW wavefronts owns NW * TQ * 16 columns
// (TQ 16-column tiles per wavefront) and streams the K/V tokens 0..p_last of
// its last column in chunks of kKT tokens.  Each chunk is loaded once per
// workgroup, one chunk ahead, by direct global-to-LDS 16-byte loads
// (global_load_lds_dwordx4; block ids two chunks ahead) into double-buffered,
// bank-swizzled LDS tiles; every wavefront then runs
// on its own columns, 32 tokens at a time:
//   * S^T[token][column] = K · Q^T on v_mfma_f32_16x16x32 (K from LDS as the
//     A operand, row = token; the wavefront's queries stay in registers as B);
//   * the online softmax per column (running maximum in log2 units, moved only
//     when a score passes it by more than kMaxSlack, so rescales are rare);
//   * O^T[d][column] += V^T · P^T on v_mfma_f32_16x16x32 over two 16-token
//     halves at once, V^T read from the LDS tile with the transposing
//     ds_read_b64_tr_b16, P^T being the score results' own register layout
//     (bf16: P split into two bf16 parts).
// Sub-chunks past a tile's last position are skipped; only sub-chunks that
// reach past a tile's first position need the causal mask.  Tokens with an
// invalid block id count as absent (their V rows are zeroed in LDS).
#include "kernels.h"
#include "mfma_util.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kKT = 64;             // tokens per staged K/V chunk
constexpr float kNegInf = -__builtin_inff();
constexpr float kMaxSlack = 8.0f;   // log2 units a score may exceed the reference maximum by

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <int DT, int D, int NW, int TQ, int WPE>
__global__ __launch_bounds__(NW * 64, WPE) void prefill_mfma_kernel(PrefillArgs a) {
    constexpr int NC = D / 32;          // score MFMAs per step and tile
    constexpr int NDT = D / 16;         // output d-tiles
    constexpr int ROWB = D * 2;         // bytes of one token row
    constexpr int PPR = ROWB / 16;      // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;       // rows one wavefront load instruction fills
    constexpr int NLI = kKT / (NW * RPI);   // load instructions per wavefront, tensor and chunk
    constexpr int CB = NW * TQ * 16;    // columns per workgroup
    static_assert(NLI * NW * RPI == kKT, "chunk split");

    // K and V chunks, double-buffered, rows of ROWB bytes with no padding: piece p
    // of row r is stored at piece slot p ^ swz(r).  The mask is chosen for the two
    // reads of a tile: the 16-byte K-operand reads (16 rows, one piece each) and the
    // transposing V reads (8 bytes from two adjacent pieces of four rows per 16
    // lanes).  With 256-byte rows (128 dimensions), measured with the LDS
    // bank-conflict counters: swz = r % 16 leaves the V reads 2-way conflicted on
    // 40% of their cycles, a rotation of r clears them but conflicts the K reads;
    // the mask below (bit 3 = r0 ^ r1 ^ r3, bit 2 = r1, bit 1 = r2) has no
    // conflict in either.  128-byte rows keep r % 8.
    // Chunks arrive by direct global-to-LDS loads (no registers in between).  The two
    // buffers are separate arrays, handed to each chunk's work as restrict-qualified
    // pointers (current chunk, next chunk), so the compiler knows that the reads of the
    // current chunk do not touch the next chunk's loads in flight: with one array indexed
    // by the chunk's parity it could not tell, and waited for those loads before every
    // read (the loads then never overlapped the arithmetic).  Unrolling the loop by two
    // with the buffers named at compile time had the same effect but took 256 registers
    // against 196.
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[kKT * ROWB];
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[kKT * ROWB];
    __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[kKT * ROWB];
    __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[kKT * ROWB];
    __shared__ __attribute__((aligned(4))) uint8_t live0[kKT];
    __shared__ __attribute__((aligned(4))) uint8_t live1[kKT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane >> 4;
    const int c16 = lane & 15;
    const int G = a.num_heads / a.num_kv_heads;
    const int bs = 1 << a.log2_bs;
    auto swz = [](int r) -> int {
        if constexpr (PPR == 16)
            return (((r ^ (r >> 1) ^ (r >> 3)) & 1) << 3) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1);
        return r % PPR;
    };

    // item: KV head fastest, then sequence, then column block (last blocks first)
    int bid = blockIdx.x;
    const int g = bid % a.num_kv_heads;
    bid /= a.num_kv_heads;
    const int s = bid % a.num_seqs;
    const int cb = a.col_blocks - 1 - bid / a.num_seqs;
    const int r0 = clampi(a.query_start[s], 0, a.num_tokens);
    const int r1 = clampi(a.query_start[s + 1], r0, a.num_tokens);
    const int q_len = min(r1 - r0, a.max_query_len);
    const int ncols = q_len * G;
    const int c_first = cb * CB;
    if (c_first >= ncols) return;                       // uniform over the workgroup
    const int n = clampi(a.ctx_lens[s], 0, a.max_blocks << a.log2_bs);
    const int pos0 = n - q_len;                         // position of query row 0
    const int c_last = min(c_first + CB, ncols) - 1;
    const int kv_end = clampi(pos0 + c_last / G + 1, 0, n);   // tokens the workgroup reads
    const int nchunks = (kv_end + kKT - 1) / kKT;
    const int32_t* trow = a.tables + (int64_t)s * a.max_blocks;

    // ---- this wavefront's columns: per tile, the lane's column and its position
    const int cw0 = c_first + wave * TQ * 16;
    int pcol[TQ];                 // position of the lane's column (-1: none visible)
    int pt_min[TQ], pt_max[TQ];   // first / last position of a tile's valid columns
    Op8 qop[TQ][NC];
#pragma unroll
    for (int tt = 0; tt < TQ; ++tt) {
        const int c = cw0 + 16 * tt + c16;
        const bool valid = c < ncols;
        pcol[tt] = valid ? pos0 + c / G : -1;
        const int ct0 = cw0 + 16 * tt, ct1 = min(cw0 + 16 * tt + 15, ncols - 1);
        pt_min[tt] = pos0 + ct0 / G;
        pt_max[tt] = ct0 <= ct1 ? min(pos0 + ct1 / G, kv_end - 1) : -1;
        const int i = valid ? c / G : 0, hl = valid ? c % G : 0;
        const char* qrow = reinterpret_cast<const char*>(a.q) +
                           (((int64_t)(r0 + i) * a.num_heads + g * G + hl) * D) * 2;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const Raw16 r = load16(qrow + (32 * cc + 8 * j) * 2);
#pragma unroll
            for (int w = 0; w < 4; ++w) qop[tt][cc].w[w] = valid ? r.w[w] : 0u;
        }
    }
    // tile bounds are the same in every lane: keep them in scalar registers so that
    // the branches on them are scalar
    int p_wave_max = -1;
#pragma unroll
    for (int tt = 0; tt < TQ; ++tt) {
        pt_min[tt] = __builtin_amdgcn_readfirstlane(pt_min[tt]);
        pt_max[tt] = __builtin_amdgcn_readfirstlane(pt_max[tt]);
        p_wave_max = max(p_wave_max, pt_max[tt]);
    }

    // ---- chunk loader.  Load instruction k of wavefront w fills rows
    // (w * NLI + k) * RPI .. + RPI - 1 of a chunk: lane i lands in piece slot i % PPR
    // of row i / PPR (a direct load writes lane i's 16 bytes at base + 16 i), so it
    // fetches the piece that belongs there, (i % PPR) ^ swz(row).
    const char* kbase = reinterpret_cast<const char*>(a.k_pool);
    const char* vbase = reinterpret_cast<const char*>(a.v_pool);
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int lslot = lane % PPR;
    int lrow[NLI];
    uint32_t lpiece[NLI];
#pragma unroll
    for (int k = 0; k < NLI; ++k) {
        lrow[k] = (wu * NLI + k) * RPI + lane / PPR;
        lpiece[k] = (uint32_t)(lslot ^ swz(lrow[k])) * 16u;
    }
    int blk_next[NLI];                   // block ids of the rows of the next chunk to load
    // table loads are branch-free (index clamped into range) so that the compiler's
    // wait counts stay exact
    auto load_table = [&](int ci) {
#pragma unroll
        for (int k = 0; k < NLI; ++k) {
            const int t = min(ci * kKT + lrow[k], kv_end - 1);
            blk_next[k] = trow[t >> a.log2_bs];
        }
    };
    uint32_t absent_rows = 0;            // bit k: row of instruction k holds no token
    auto issue_chunk = [&](int ci, uint8_t* kdst, uint8_t* vdst, uint8_t* ldst) {
        absent_rows = 0;
#pragma unroll
        for (int k = 0; k < NLI; ++k) {
            const int t = ci * kKT + lrow[k];
            const int b = blk_next[k];
            const bool live = (t < kv_end) & (b >= 0) & (b < a.num_blocks);
            const int bb = live ? b : 0;            // absent: the pool's first row
            const int64_t off =
                (((int64_t)(bb * a.num_kv_heads + g) << a.log2_bs) + (live ? (t & (bs - 1)) : 0)) * ROWB +
                lpiece[k];
            const int lbase = (wu * NLI + k) * RPI * ROWB;
            __builtin_amdgcn_global_load_lds(kbase + off, (__attribute__((address_space(3))) void*)&kdst[lbase],
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(vbase + off, (__attribute__((address_space(3))) void*)&vdst[lbase],
                                             16, 0, 0);
            absent_rows |= live ? 0u : (1u << k);
            if (lslot == 0) ldst[lrow[k]] = live ? 1 : 0;
        }
    };
    // after this wavefront's loads of a chunk have landed: zero the V rows that hold
    // no token (their weights are zero, and 0 * NaN would poison the sums)
    auto settle_chunk = [&](uint8_t* vcur) {
        __builtin_amdgcn_s_waitcnt(0);           // vmcnt(0): the direct loads are in LDS
        if (absent_rows) {
#pragma unroll
            for (int k = 0; k < NLI; ++k)
                if (absent_rows & (1u << k))
                    *reinterpret_cast<uint4*>(&vcur[(wu * NLI + k) * RPI * ROWB + lane * 16]) =
                        make_uint4(0u, 0u, 0u, 0u);
        }
    };

    float m[TQ], l[TQ];
    f32x4 acc[TQ][NDT];
#pragma unroll
    for (int tt = 0; tt < TQ; ++tt) {
        m[tt] = kNegInf;
        l[tt] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[tt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (nchunks > 0) {
        load_table(0);
        issue_chunk(0, kbuf0, vbuf0, live0);
        if (nchunks > 1) load_table(1);
    }
    // one chunk: kt/vt/lt hold it, kn/vn/ln receive the next
    auto chunk = [&](int ci, const uint8_t* __restrict__ kt, uint8_t* __restrict__ vt, const uint8_t* __restrict__ lt,
                     uint8_t* __restrict__ kn, uint8_t* __restrict__ vn, uint8_t* __restrict__ ln) {
        settle_chunk(vt);
        __syncthreads();
        if (ci + 1 < nchunks) {
            issue_chunk(ci + 1, kn, vn, ln);
            if (ci + 2 < nchunks) load_table(ci + 2);
        }
        const int t0 = ci * kKT;
        // Two 32-token steps per chunk, one after the other (issuing the score MFMAs of
        // both first, so that the matrix cores work on the second step's scores while
        // the vector units run the first step's softmax, measured 3% slower once the
        // loads overlapped the arithmetic).
        const bool on0 = t0 <= p_wave_max, on1 = t0 + 32 <= p_wave_max;   // scalar
        f32x4 scs[2][TQ][2];
        uint32_t lvs[2][2];
        auto scores = [&](int sub) {
            uint32_t* lv4 = lvs[sub];
            auto& sc = scs[sub];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                lv4[h] = *reinterpret_cast<const uint32_t*>(&lt[32 * sub + 16 * h + 4 * j]);
            // scores of every tile first, so that no softmax waits on its own MFMAs; each
            // K operand is read just before the MFMAs that use it (few registers live)
#pragma unroll
            for (int tt = 0; tt < TQ; ++tt) {
                sc[tt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                sc[tt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 32 * sub + 16 * h + c16;
#pragma unroll
                for (int cc = 0; cc < NC; ++cc) {
                    const uint4 r = *reinterpret_cast<const uint4*>(
                        &kt[row * ROWB + (((4 * cc + j) ^ swz(row)) * 16)]);
                    const Op8 kop{{r.x, r.y, r.z, r.w}};
#pragma unroll
                    for (int tt = 0; tt < TQ; ++tt) sc[tt][h] = mma32<DT>(kop, qop[tt][cc], sc[tt][h]);
                }
            }
        };
        auto step = [&](int sub) {
            const int u0 = t0 + 32 * sub;
            const uint32_t* lv4 = lvs[sub];
            auto& sc = scs[sub];
            // every token of the 32 present (a wavefront-uniform test)
            const bool sub_full = __builtin_amdgcn_ballot_w64((lv4[0] & lv4[1]) != 0x01010101u) == 0;
            Op8 pop[TQ], plo[TQ];
            // The reference maximum moves only when a score passes it by more than
            // kMaxSlack; a lane's own scores tell whether that can happen, and only
            // then (rarely, after the first steps) is the column maximum taken across
            // the four lanes of the column.  Returns whether it moved (wavefront-uniform);
            // the accumulators are rescaled once, after the masked and unmasked paths
            // have joined, so that the paths share their registers.
            auto update_max = [&](int tt, float lmax, float& alpha) -> bool {
                if (__builtin_amdgcn_ballot_w64(lmax > m[tt] + kMaxSlack)) {
                    const float mx = max_over_groups(lmax);
                    const float mn = (mx > m[tt] + kMaxSlack) ? mx : m[tt];
                    alpha = mn != m[tt] ? fast_exp2(m[tt] - mn) : 1.0f;   // from -inf: 0
                    m[tt] = mn;
                    return true;
                }
                return false;
            };
            // weights -> MFMA operands; the running sum adds the weights as the MFMA
            // sees them (fp16: the rounded values, two per dot instruction)
            auto finish = [&](int tt, const float* pr) {
#pragma unroll
                for (int q = 0; q < 4; ++q) pop[tt].w[q] = pack2<DT>(pr[2 * q], pr[2 * q + 1]);
                if constexpr (DT == PA_F16) {
                    float lt = l[tt];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        lt = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pop[tt].w[q]),
                                                    half2_t{(_Float16)1.0f, (_Float16)1.0f}, lt, false);
                    l[tt] = lt;
                } else {
                    float psum = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) psum += pr[e];
                    l[tt] += psum;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float h0 = __uint_as_float(pop[tt].w[q] << 16);
                        const float h1 = __uint_as_float(pop[tt].w[q] & 0xFFFF0000u);
                        plo[tt].w[q] = pack2<DT>(pr[2 * q] - h0, pr[2 * q + 1] - h1);
                    }
                }
            };
            const bool pos_scale = a.qk_scale > 0.0f;
#pragma unroll
            for (int tt = 0; tt < TQ; ++tt) {
                // value e = 4h + i is token u0 + 16h + 4j + i
                float pr[8];
                float alpha = 1.0f;
                bool rescale;
                if (sub_full && u0 + 31 <= pt_min[tt] && pos_scale) {
                    // every token present and visible: no masks; with a positive scale
                    // the largest scaled score is the scaled largest score
                    float smax = sc[tt][0][0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) smax = fmaxf(smax, sc[tt][e >> 2][e & 3]);
                    rescale = update_max(tt, smax * a.qk_scale, alpha);
                    const float mn = m[tt];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(fmaf(sc[tt][e >> 2][e & 3], a.qk_scale, -mn));
                } else {
                    // absent tokens and the causal limit, masked without branches
                    const int lim = (u0 + 31 > pt_min[tt]) ? pcol[tt] : 0x7FFFFFFF;
                    float sv[8];
                    uint32_t live[8];
                    float lmax = kNegInf;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int h = e >> 2, i = e & 3;
                        const int t = u0 + 16 * h + 4 * j + i;
                        live[e] = ((lv4[h] >> (8 * i)) & 1u) & (uint32_t)(t <= lim);
                        sv[e] = live[e] ? sc[tt][h][i] * a.qk_scale : kNegInf;
                        lmax = fmaxf(lmax, sv[e]);
                    }
                    rescale = update_max(tt, lmax, alpha);
                    const float mn = m[tt];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = live[e] ? fast_exp2(sv[e] - mn) : 0.0f;
                }
                if (rescale) {                              // wavefront-uniform, rare
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) acc[tt][dt] *= alpha;
                    l[tt] *= alpha;
                }
                finish(tt, pr);
            }
            // O^T[d][column] += V^T[d][token] · P^T[token][column], 32 tokens per MFMA
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                // V^T operand of d-tile dt: row rr, halfs 16 dt + 4 (c16 & 3) .. + 3, i.e.
                // piece 2 dt + (c16 & 3) / 2, its first or second 8 bytes
                Op8 vop;
                {
                    const int rr = 32 * sub + 4 * j + (c16 >> 2);
                    const int pc = 2 * dt + ((c16 & 3) >> 1), hb = (c16 & 1) * 8;
                    const Op4 v0 = read_tr16(reinterpret_cast<const uint16_t*>(
                        &vt[rr * ROWB + ((pc ^ swz(rr)) * 16) + hb]));
                    const Op4 v1 = read_tr16(reinterpret_cast<const uint16_t*>(
                        &vt[(rr + 16) * ROWB + ((pc ^ swz(rr + 16)) * 16) + hb]));
                    vop.w[0] = v0.w[0];
                    vop.w[1] = v0.w[1];
                    vop.w[2] = v1.w[0];
                    vop.w[3] = v1.w[1];
                }
#pragma unroll
                for (int tt = 0; tt < TQ; ++tt) {
                    acc[tt][dt] = mma32<DT>(vop, pop[tt], acc[tt][dt]);
                    if constexpr (DT == PA_BF16) acc[tt][dt] = mma32<DT>(vop, plo[tt], acc[tt][dt]);
                }
            }
        };
        if (on0) { scores(0); step(0); }
        if (on1) { scores(1); step(1); }
        // no barrier here: the next chunk goes into the other buffer, and the
        // barrier after that store orders this chunk's reads before the buffer
        // is written again
    };
    for (int ci = 0; ci < nchunks; ++ci) {
        const bool odd = ci & 1;
        chunk(ci, odd ? kbuf1 : kbuf0, odd ? vbuf1 : vbuf0, odd ? live1 : live0,
              odd ? kbuf0 : kbuf1, odd ? vbuf0 : vbuf1, odd ? live0 : live1);
    }

    // ---- normalise and store: lane holds column c16 of each tile, d = 16 dt + 4 j .. + 3
#pragma unroll
    for (int tt = 0; tt < TQ; ++tt) {
        const float lt = sum_over_groups(l[tt]);
        const int c = cw0 + 16 * tt + c16;
        if (c < ncols) {
            const int i = c / G, hl = c % G;
            const float f = (lt > 0.0f ? 1.0f / lt : 0.0f) * a.out_scale;
            char* orow = reinterpret_cast<char*>(a.out) +
                         (((int64_t)(r0 + i) * a.num_heads + g * G + hl) * D) * 2;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int d = 16 * dt + 4 * j;
                *reinterpret_cast<uint2*>(orow + d * 2) =
                    make_uint2(pack2<DT>(acc[tt][dt][0] * f, acc[tt][dt][1] * f),
                               pack2<DT>(acc[tt][dt][2] * f, acc[tt][dt][3] * f));
            }
        }
    }
}

template <int DT, int D>
hipError_t launch_typed(PrefillArgs& a, hipStream_t stream) {
    constexpr int NW = 4, TQ = 2, WPE = 2;
    constexpr int CB = NW * TQ * 16;
    const int G = a.num_heads / a.num_kv_heads;
    a.col_blocks = (int32_t)(((int64_t)a.max_query_len * G + CB - 1) / CB);
    const int64_t grid = (int64_t)a.col_blocks * a.num_seqs * a.num_kv_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, NW, TQ, WPE>), dim3((uint32_t)grid), dim3(NW * 64),
                       0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int q_dt, int kv_dt, int head_dim) {
    return (head_dim == 64 || head_dim == 128) && q_dt == kv_dt && (q_dt == PA_F16 || q_dt == PA_BF16);
}

hipError_t launch_prefill(PrefillArgs& a, int q_dt, int kv_dt, int head_dim, hipStream_t stream) {
    if (!prefill_supported(q_dt, kv_dt, head_dim)) return hipErrorInvalidValue;
    if (q_dt == PA_F16) return head_dim == 64 ? launch_typed<PA_F16, 64>(a, stream)
                                              : launch_typed<PA_F16, 128>(a, stream);
    return head_dim == 64 ? launch_typed<PA_BF16, 64>(a, stream) : launch_typed<PA_BF16, 128>(a, stream);
}

}  // namespace pa

// kv_cache_write: scatter each new token's K and V into its pool slot.
//
// One token's keys and values are computed once and stored for every later
// step (KV 缓存与分页注意力 §02 一次写一个词元); the slot is where the
// sequence's block table puts that token (§07 块表).  Each thread moves one
// 16-byte piece of a source row: consecutive threads cover consecutive bytes
// of one token's [kv_heads][head_dim] row, so both the read of the new token
// and the write of each (block, head) row segment are 16-byte coalesced.
// An fp8 pool stores e4m3(x * (1/scale)) per number (§11).
#include "kernels.h"
#include "pa_device.h"

namespace pa {
namespace {

template <int SRC, int KV>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
    constexpr int SB = elem_bytes(SRC);
    constexpr int DB = elem_bytes(KV);
    constexpr int VEC = 16 / SB;                       // source elements per thread
    const int64_t per_token = (int64_t)a.num_kv_heads * a.head_dim / VEC;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t i = idx / per_token;
    if (i >= a.num_tokens) return;
    const int64_t e = (idx - i * per_token) * VEC;     // element within the token row
    const int64_t src = i * a.num_kv_heads * a.head_dim + e;
    // the new values do not depend on the slot: load them together with it
    const Raw16 rk = load16(reinterpret_cast<const char*>(a.k_new) + src * SB);
    const Raw16 rv = load16(reinterpret_cast<const char*>(a.v_new) + src * SB);
    const int64_t slot = a.slot_mapping[i];
    if (slot < 0 || slot >= a.num_slots) return;       // -1 (or out of range): no token
    const int64_t head = e / a.head_dim;
    const int64_t d = e - head * a.head_dim;
    const int64_t blk = slot >> a.log2_bs;
    const int64_t off = slot & ((1 << a.log2_bs) - 1);
    const int64_t dst = (((blk * a.num_kv_heads + head) << a.log2_bs) + off) * a.head_dim + d;

#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
        char* p = reinterpret_cast<char*>(kv ? a.v_pool : a.k_pool) + dst * DB;
        const Raw16 r = kv ? rv : rk;
        if constexpr (SRC == KV) {
            store16(p, r);
        } else {
            static_assert(KV == PA_FP8_E4M3, "only same-dtype copies or fp8 quantisation");
            float f[VEC];
            unpack16<SRC>(r, f);
            const float inv = kv ? a.v_inv_scale : a.k_inv_scale;
            uint32_t w[VEC / 4];
#pragma unroll
            for (int j = 0; j < VEC / 4; ++j) {
                w[j] = f32_to_e4m3(f[4 * j] * inv) | (f32_to_e4m3(f[4 * j + 1] * inv) << 8) |
                       (f32_to_e4m3(f[4 * j + 2] * inv) << 16) |
                       (f32_to_e4m3(f[4 * j + 3] * inv) << 24);
            }
            if constexpr (VEC == 8) {
                *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
            } else {
                *reinterpret_cast<uint32_t*>(p) = w[0];
            }
        }
    }
}

// int8 pools (group-wise): one wavefront per (token, KV head) quantises the head
// vector on its own: amax over the vector (wavefront reduction), scale = amax / 127,
// code = round-to-nearest-even(x / scale) clamped to [-127, 127] (codes 0 for a zero
// vector), in float32 with correctly rounded divisions; lane 0 stores the scale.
template <int SRC, int D>
__global__ __launch_bounds__(256) void kv_write_int8_kernel(WriteArgs a) {
    constexpr int PER = D / 64;                        // numbers per lane
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (token, head) pair
    const int64_t i = w / a.num_kv_heads;
    if (i >= a.num_tokens) return;
    const int64_t head = w - i * a.num_kv_heads;
    const int64_t slot = a.slot_mapping[i];
    if (slot < 0 || slot >= a.num_slots) return;
    const int64_t blk = slot >> a.log2_bs;
    const int64_t off = slot & ((1 << a.log2_bs) - 1);
    const int64_t row = ((blk * a.num_kv_heads + head) << a.log2_bs) + off;   // scale index
    const int64_t src = (i * a.num_kv_heads + head) * D + lane * PER;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
        const char* sp = reinterpret_cast<const char*>(kv ? a.v_new : a.k_new) + src * elem_bytes(SRC);
        float x[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            if constexpr (SRC == PA_F32) x[k] = reinterpret_cast<const float*>(sp)[k];
            else if constexpr (SRC == PA_F16) x[k] = (float)reinterpret_cast<const _Float16*>(sp)[k];
            else x[k] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(sp)[k] << 16);
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < PER; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const float scale = __fdiv_rn(amax, 127.0f);
        uint32_t packed = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            float q = scale > 0.0f ? __builtin_rintf(__fdiv_rn(x[k], scale)) : 0.0f;
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            packed |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * k);
        }
        char* dp = reinterpret_cast<char*>(kv ? a.v_pool : a.k_pool) + row * D + lane * PER;
        if constexpr (PER == 2) *reinterpret_cast<uint16_t*>(dp) = (uint16_t)packed;
        else *reinterpret_cast<uint8_t*>(dp) = (uint8_t)packed;
        if (lane == 0) (kv ? a.v_scales : a.k_scales)[row] = scale;
    }
}

template <int SRC>
hipError_t launch_int8(const WriteArgs& a, hipStream_t stream) {
    const int64_t waves = (int64_t)a.num_tokens * a.num_kv_heads;
    const int64_t blocks = (waves + 3) / 4;
    if (a.head_dim == 64)
        hipLaunchKernelGGL((kv_write_int8_kernel<SRC, 64>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((kv_write_int8_kernel<SRC, 128>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int SRC, int KV>
hipError_t launch(const WriteArgs& a, hipStream_t stream) {
    constexpr int VEC = 16 / elem_bytes(SRC);
    const int64_t threads = (int64_t)a.num_tokens * a.num_kv_heads * a.head_dim / VEC;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((kv_write_kernel<SRC, KV>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, int src_dt, int kv_dt, hipStream_t stream) {
    if (src_dt == kv_dt) {
        switch (kv_dt) {
            case PA_F32: return launch<PA_F32, PA_F32>(a, stream);
            case PA_F16: return launch<PA_F16, PA_F16>(a, stream);
            case PA_BF16: return launch<PA_BF16, PA_BF16>(a, stream);
            case PA_FP8_E4M3: return launch<PA_FP8_E4M3, PA_FP8_E4M3>(a, stream);
        }
    } else if (kv_dt == PA_FP8_E4M3) {
        switch (src_dt) {
            case PA_F32: return launch<PA_F32, PA_FP8_E4M3>(a, stream);
            case PA_F16: return launch<PA_F16, PA_FP8_E4M3>(a, stream);
            case PA_BF16: return launch<PA_BF16, PA_FP8_E4M3>(a, stream);
        }
    } else if (kv_dt == PA_INT8) {
        switch (src_dt) {
            case PA_F32: return launch_int8<PA_F32>(a, stream);
            case PA_F16: return launch_int8<PA_F16>(a, stream);
            case PA_BF16: return launch_int8<PA_BF16>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace pa

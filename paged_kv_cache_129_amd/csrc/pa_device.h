// Device-side helpers shared by the gfx950 kernels: storage types, 16-byte
// unpacking, wavefront row reductions through DPP, and the e4m3 codec.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int elem_bytes(int dt) {
    return dt == PA_F32 ? 4 : ((dt == PA_FP8_E4M3 || dt == PA_INT8) ? 1 : 2);
}

// The fp8 path widens e4m3 codes through an fp16 bit pattern that carries
// the value times 2^-8 (see e4m3x4_to_f16x4); this factor restores it.
constexpr float kFp8WidenFactor = 256.0f;

__host__ __device__ constexpr float dequant_factor(int kv_dt) {
    return kv_dt == PA_FP8_E4M3 ? kFp8WidenFactor : 1.0f;
}

// ---------------------------------------------------------------- loads
struct alignas(16) Raw16 {
    uint32_t w[4];
};

__device__ __forceinline__ Raw16 load16(const void* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return Raw16{{v.x, v.y, v.z, v.w}};
}

// Streaming (non-temporal) 16-byte load for K/V cache reads: every cached
// byte is read once per decode step, and on gfx950 this cache policy moves
// markedly more bytes per second than the default one (measured 7.06 vs
// 6.35 TB/s for a plain read kernel).
__device__ __forceinline__ Raw16 load16_stream(const void* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return Raw16{{v.x, v.y, v.z, v.w}};
}

__device__ __forceinline__ void store16(void* p, const Raw16& r) {
    *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
}

// Four e4m3 codes (one dword) -> four fp16 bit patterns holding value * 2^-8,
// by gfx950's scaled conversion (v_cvt_scalef32_pk_f16_fp8, scale 2^-8).
// Every finite e4m3 value times 2^-8 is an fp16 number (e4m3 subnormals land
// on fp16 subnormals), so the widening is exact; it gives the same bits as
// moving the code's exponent and mantissa into the fp16 fields (checked on
// the GPU for all 256 codes).  NaN codes give NaN; absent tokens are masked
// by selects, never by multiplication.
__device__ __forceinline__ void e4m3x4_to_f16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f / kFp8WidenFactor, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f / kFp8WidenFactor, true));
}

// The same widening to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 2^-8): bf16 has
// more significant bits than e4m3 and a wider exponent range, so this is
// exact too.  Used when the query is bf16, whose range fp16 cannot hold.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f / kFp8WidenFactor, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f / kFp8WidenFactor, true));
}

// e4m3 codes widened to the matrix-core operand type MT (fp16 or bf16)
template <int MT>
__device__ __forceinline__ void e4m3x4_widen(uint32_t w, uint32_t& lo, uint32_t& hi) {
    if constexpr (MT == PA_BF16) e4m3x4_to_bf16x4(w, lo, hi);
    else e4m3x4_to_f16x4(w, lo, hi);
}

__device__ __forceinline__ void f16x2_to_f32(uint32_t w, float& a, float& b) {
    const half2_t h = __builtin_bit_cast(half2_t, w);
    a = (float)h.x;
    b = (float)h.y;
}

// 16 raw bytes of storage type DT -> 16 / elem_bytes(DT) floats.  fp8 values
// come out multiplied by 2^-8 (kFp8WidenFactor undoes it).
template <int DT>
__device__ __forceinline__ void unpack16(const Raw16& r, float* f) {
    if constexpr (DT == PA_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r.w[i]);
    } else if constexpr (DT == PA_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f16x2_to_f32(r.w[i], f[2 * i], f[2 * i + 1]);
    } else if constexpr (DT == PA_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(r.w[i] << 16);
            f[2 * i + 1] = __uint_as_float(r.w[i] & 0xFFFF0000u);
        }
    } else {   // e4m3 straight to fp32 (v_cvt_scalef32_pk_f32_fp8, same values)
        static_assert(DT == PA_FP8_E4M3, "int8 codes go through int8x16_biased");
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.w[i], 1.0f / kFp8WidenFactor, false);
            const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.w[i], 1.0f / kFp8WidenFactor, true);
            f[4 * i] = lo[0];
            f[4 * i + 1] = lo[1];
            f[4 * i + 2] = hi[0];
            f[4 * i + 3] = hi[1];
        }
    }
}

// 16 int8 codes -> the 16 floats code + 128, each in [1, 255] for codes in
// [-127, 127].  Flipping the sign bits makes every byte the unsigned number
// code + 128, which one v_cvt_f32_ubyteN converts exactly; the caller removes
// the bias as 128 times the sum of the weights it applied.
__device__ __forceinline__ void int8x16_biased(const Raw16& r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = r.w[i] ^ 0x80808080u;
#pragma unroll
        for (int k = 0; k < 4; ++k) f[4 * i + k] = (float)((u >> (8 * k)) & 0xFFu);
    }
}

// ---------------------------------------------------------------- stores (round to nearest even)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

template <int DT>
__device__ __forceinline__ void store_vals(void* dst, const float* f, int n) {
    if constexpr (DT == PA_F32) {
        float* d = reinterpret_cast<float*>(dst);
        for (int i = 0; i < n; i += 4)
            *reinterpret_cast<float4*>(d + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
    } else if constexpr (DT == PA_F16) {
        uint32_t* d = reinterpret_cast<uint32_t*>(dst);
        for (int i = 0; i < n; i += 8) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                half2_t h;
                h.x = (_Float16)f[i + 2 * j];
                h.y = (_Float16)f[i + 2 * j + 1];
                w[j] = __builtin_bit_cast(uint32_t, h);
            }
            *reinterpret_cast<uint4*>(d + i / 2) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {   // bf16
        uint32_t* d = reinterpret_cast<uint32_t*>(dst);
        for (int i = 0; i < n; i += 8) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = f32_to_bf16_bits(f[i + 2 * j]) | (f32_to_bf16_bits(f[i + 2 * j + 1]) << 16);
            *reinterpret_cast<uint4*>(d + i / 2) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// ---------------------------------------------------------------- DPP row reductions
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES lanes (4, 8, 16 or 32); every lane of a
// group ends with the same bits.  quad_perm [1,0,3,2] and [2,3,0,1] pair
// lanes inside a quad, row_half_mirror pairs the two quads of 8 lanes,
// row_mirror the two halves of a 16-lane row.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32, "group size");
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    if constexpr (LANES >= 8) x += dpp<0x141>(x);
    if constexpr (LANES >= 16) x += dpp<0x140>(x);
    if constexpr (LANES >= 32) x += __shfl_xor(x, 16, 64);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- e4m3 encode
// float -> OCP e4m3fn code: clamp to +-448 (saturating; +-inf included), then
// round to nearest with ties to the even mantissa; NaN -> 0x7F with the sign.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;          // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;         // |x| >= 448
    if (a < 0x3C800000u) {                             // |x| < 2^-6: subnormal codes 0..8
        const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
        return sign | (uint32_t)q;
    }
    uint32_t e = (a >> 23) - 120u;                     // biased exponent 127 -> 7
    uint32_t m = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) {
        m = 0;
        ++e;
    }
    return sign | (e << 3) | m;
}

}  // namespace pa

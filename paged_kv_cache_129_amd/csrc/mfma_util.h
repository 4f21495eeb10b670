// Matrix-core helpers shared by the gfx950 attention kernels: 16x16 MFMA
// operand types and calls (f16 / bf16), fp32 -> 16-bit packing, reductions
// across the four 16-lane rows of a wavefront, and the transposing LDS read
// that turns a row-major [token][d] tile into the A operand of O^T = V^T P^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Op8 {                        // eight 16-bit MFMA operand values
    uint32_t w[4];
};
struct Op4 {                        // four 16-bit MFMA operand values
    uint32_t w[2];
};

template <int MT>
__device__ __forceinline__ f32x4 mma32(const Op8& a, const Op8& b, f32x4 c) {
    if constexpr (MT == PA_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

template <int MT>
__device__ __forceinline__ f32x4 mma16(const Op4& a, const Op4& b, f32x4 c) {
    if constexpr (MT == PA_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
    }
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    half2_t h;
    h.x = (_Float16)a;
    h.y = (_Float16)b;
    return __builtin_bit_cast(uint32_t, h);
}

// two floats -> two bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

template <int MT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (MT == PA_F16) return pack_f16(a, b);
    return pack_bf16(a, b);
}

// Lane-group reductions of a value held per (lane group j, column c16): the
// four lanes c16, c16+16, c16+32, c16+48 combine through two swaps between
// lane rows (v_permlane16_swap, v_permlane32_swap), with no LDS round trip.
__device__ __forceinline__ float max_over_groups(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane 4k + q gives the address of four consecutive 16-bit values, and lane i
// receives value i % 4 from lane 4k + i / 4, for k = 0..3.  With lane 4k + q
// of group g pointing at row 4g + k, columns 4q..4q+3 of a row-major tile,
// lane i of group g receives rows 4g..4g+3 of column i: an MFMA operand whose
// four K values run down a column.
__device__ __forceinline__ Op4 read_tr16(const uint16_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef s16x4 __attribute__((address_space(3))) * lds_ptr;
    return __builtin_bit_cast(Op4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)p));
}

}  // namespace pa

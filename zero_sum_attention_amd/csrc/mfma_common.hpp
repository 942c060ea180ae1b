// bfloat16 MFMA operand helpers shared by the matrix-core kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zeros {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two floats to a packed bfloat16 pair (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    const f32x2v f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    bf16x8 r;
    r[0] = static_cast<short>(a & 0xffff); r[1] = static_cast<short>(a >> 16);
    r[2] = static_cast<short>(b & 0xffff); r[3] = static_cast<short>(b >> 16);
    r[4] = static_cast<short>(c & 0xffff); r[5] = static_cast<short>(c >> 16);
    r[6] = static_cast<short>(d & 0xffff); r[7] = static_cast<short>(d >> 16);
    return r;
}

// acc + (sum of the squares of the two bfloat16 values packed in a)
__device__ __forceinline__ float dot2_bf16(uint32_t a, float acc) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v v = *reinterpret_cast<const bf16x2v *>(&a);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

// Transposing LDS read (ds_read_b64_tr_b16): every lane names 8 bytes (4 bfloat16), and within each
// group of 16 lanes, lane i receives element i & 3 of the 8 bytes named by lanes 4 e + (i >> 2),
// e = 0 .. 3 (measured layout). Four lanes naming 16 consecutive features of four rows thus give
// each lane its feature of the four rows.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t *p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p));
    return __builtin_bit_cast(uint2, r);
}

}  // namespace zeros

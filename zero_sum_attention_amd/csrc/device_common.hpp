// Device helpers shared by the libzeros kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zeros {

constexpr float kNegInf = -__builtin_huge_valf();

// bfloat16 storage: the upper 16 bits of an IEEE float32.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
    // round to nearest, ties to even; NaN stays a quiet NaN
    uint32_t u = __float_as_uint(x);
    bf16 r;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        r.bits = static_cast<uint16_t>((u >> 16) | 0x40u);
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);
        r.bits = static_cast<uint16_t>(u >> 16);
    }
    return r;
}

__device__ __forceinline__ float sigmoidf(float x) {
    // 1/(1+e^-x) without overflow for large |x|
    if (x >= 0.f) return 1.f / (1.f + expf(-x));
    const float e = expf(x);
    return e / (1.f + e);
}

// exp(a - b) that treats a = -inf as contributing zero (also when b = -inf).
__device__ __forceinline__ float exp_diff(float a, float b) {
    return (a == kNegInf) ? 0.f : expf(a - b);
}

// RoPE frequency of pair j expressed in revolutions per position: base^(-2j/d) / (2 pi).
__device__ __forceinline__ double rope_rev_per_pos(int j, int d, float base) {
    return pow(static_cast<double>(base), -2.0 * j / d) * 0.15915494309189535;  // 1/(2 pi)
}

// cos/sin of pos * theta_j with the angle reduced exactly enough in double precision:
// rev = pos * theta_j / (2 pi) is formed in double, its integer part dropped, and the
// remaining fraction of a turn converted to radians in [-pi, pi] before a float sincos.
__device__ __forceinline__ void rope_cos_sin(double rev_per_pos, int pos, float &c, float &s) {
    double r = static_cast<double>(pos) * rev_per_pos;
    r -= rint(r);
    const float ang = static_cast<float>(r * 6.283185307179586);
    sincosf(ang, &s, &c);
}

// DPP control codes: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror
// (lane i of 8 from lane 7 - i), row_mirror (lane i of 16 from lane 15 - i).
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane gets the sum. Within a
// row of 16 lanes the partner values come by DPP (no LDS round trip): after the two quad swaps every
// lane holds its quad's sum, and the (half-)row mirror pairs it with the other quad (or half-row),
// so each step adds the same two partial sums as a butterfly would.
template <int G> __device__ __forceinline__ float group_sum(float x) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
    if constexpr (G >= 2) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kQuadXor1, 0xf, 0xf, false));
    if constexpr (G >= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kQuadXor2, 0xf, 0xf, false));
    if constexpr (G >= 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowHalfMirror, 0xf, 0xf, false));
    if constexpr (G >= 16) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowMirror, 0xf, 0xf, false));
    if constexpr (G >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// Workgroup barrier that only waits for this wave's LDS traffic. __syncthreads() also waits for
// every outstanding global load, which would stall the prefetch of the next chunk at each barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// DPP control codes: row_shr:n, row_ror:n, row_bcast:15, row_bcast:31.
constexpr int kRowShr = 0x110, kRowRor = 0x120, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave (rows of 16 by shifts, then row broadcasts).
__device__ __forceinline__ float wave_scan_add(float v) {
    v += dpp_f<kRowShr + 1, 0xf>(0.f, v);
    v += dpp_f<kRowShr + 2, 0xf>(0.f, v);
    v += dpp_f<kRowShr + 4, 0xf>(0.f, v);
    v += dpp_f<kRowShr + 8, 0xf>(0.f, v);
    v += dpp_f<kRowBcast15, 0xa>(0.f, v);
    v += dpp_f<kRowBcast31, 0xc>(0.f, v);
    return v;
}
// Inclusive prefix maximum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_scan_max(float v) {
    v = fmaxf(v, dpp_f<kRowShr + 1, 0xf>(kNegInf, v));
    v = fmaxf(v, dpp_f<kRowShr + 2, 0xf>(kNegInf, v));
    v = fmaxf(v, dpp_f<kRowShr + 4, 0xf>(kNegInf, v));
    v = fmaxf(v, dpp_f<kRowShr + 8, 0xf>(kNegInf, v));
    v = fmaxf(v, dpp_f<kRowBcast15, 0xa>(kNegInf, v));
    v = fmaxf(v, dpp_f<kRowBcast31, 0xc>(kNegInf, v));
    return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

}  // namespace zeros

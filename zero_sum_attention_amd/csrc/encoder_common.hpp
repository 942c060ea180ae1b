// Helpers shared by the encoder kernels (encoder_mfma.hip, encoder_long.hip).
#pragma once

#include "device_common.hpp"
#include "mfma_common.hpp"

namespace zeros {

// (max, sum e^{s - max}) of two parts merged; a max of -inf marks an empty part.
__device__ __forceinline__ void lse_merge(float &m, float &e, float m2, float e2) {
    const float mm = fmaxf(m, m2);
    e = (m == kNegInf ? 0.f : e * __expf(m - mm)) + (m2 == kNegInf ? 0.f : e2 * __expf(m2 - mm));
    m = mm;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// (max, sum e^{s - max}, sum s) merged over the 64 lanes of a wave; every lane gets the result.
// Within a row of 16 lanes the partners come by DPP (the pairings of group_sum), then the four row
// results by readlane.
__device__ __forceinline__ void wave_lse_merge(float &m, float &e, float &ps) {
    lse_merge(m, e, dpp_mov<kQuadXor1>(m), dpp_mov<kQuadXor1>(e));
    ps += dpp_mov<kQuadXor1>(ps);
    lse_merge(m, e, dpp_mov<kQuadXor2>(m), dpp_mov<kQuadXor2>(e));
    ps += dpp_mov<kQuadXor2>(ps);
    lse_merge(m, e, dpp_mov<kRowHalfMirror>(m), dpp_mov<kRowHalfMirror>(e));
    ps += dpp_mov<kRowHalfMirror>(ps);
    lse_merge(m, e, dpp_mov<kRowMirror>(m), dpp_mov<kRowMirror>(e));
    ps += dpp_mov<kRowMirror>(ps);
    float M = lane_f(m, 0), E = lane_f(e, 0), P = lane_f(ps, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        lse_merge(M, E, lane_f(m, r), lane_f(e, r));
        P += lane_f(ps, r);
    }
    m = M;
    e = E;
    ps = P;
}

// float -> bfloat16 bits (round to nearest even)
__device__ __forceinline__ uint16_t bf16_bits(float x) { return static_cast<uint16_t>(pack2(x, 0.f) & 0xffffu); }

__device__ __forceinline__ void unpack8(const uint4 &x, float (&f)[8]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo_f(w[i]);
        f[2 * i + 1] = hi_f(w[i]);
    }
}

// Token column of row f in a transposed bf16 staging buffer [row][token] whose rows are 4 mod 8
// words long: rows 8 apart are then a multiple of 32 words apart, in one bank, so a staging write by
// 8 feature groups would serialise. Bits 3-5 of the token index XOR the row's 8-row group spread
// those writes over the banks while each 8-token group stays contiguous for the 16-byte MFMA
// operand reads.
__device__ __forceinline__ int eh_col(int f, int tok) { return tok ^ (((f >> 3) & 7) << 3); }

}  // namespace zeros

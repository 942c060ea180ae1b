// Internal interface between the C-ABI front end (zeros_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/zeros.h"

namespace zeros {

// Everything a kernel needs, validated by the front end. Pointers are device pointers.
struct Problem {
    const void *q, *k, *v, *u;
    const float *mu, *tau;
    const void *g1, *gh;
    void *o;
    zeros_state st;     // all NULL when no state is read or written
    int B, H, N, d, du;
    int dtype;          // zeros_dtype
    int rope;
    float rope_base;
};

hipError_t launch_causal(const Problem &p, hipStream_t stream);
hipError_t launch_encoder(const Problem &p, hipStream_t stream);
hipError_t launch_decode(const Problem &p, hipStream_t stream);

}  // namespace zeros

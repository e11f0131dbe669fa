// e4m3.h -- OCP E4M3 (FP8) encoding of one value: round to nearest, ties
// to the even code, saturating at 448; used by the MXFP8 / FP8-row encoders
// and by the attention kernel that encodes its queries.
#pragma once
#include "common.h"

namespace csa {

// E4M3 code of y (|y| may exceed 448: saturates).  With a = min(|y|, 448)
// and E = max(floor(log2 a), -6), the code is 8 (E + 6) + rne(a * 2^(3-E)):
// the rounded significand q is in [8, 16] for E > -6 (q = 16 carries into
// the next exponent), and for E = -6 it is the subnormal step count 0 .. 8.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const float a = fminf(fabsf(y), 448.f);
    int E = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // zero / subnormal: < -6
    E = E < -6 ? -6 : E;
    const float q = rintf(ldexpf(a, 3 - E));                  // exact scaling, then RNE
    const uint32_t code = (uint32_t)(8 * (E + 6)) + (uint32_t)q;
    return code | (__float_as_uint(y) >> 31 << 7);
}

}  // namespace csa

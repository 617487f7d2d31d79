// The OCP MX v1.0 E2M1 conversion rule shared by the MXFP4 quantiser and the
// indexer key append (see quant.hip for the passage and the reading).
#pragma once
#include "common.hpp"

// E2M1 magnitude code of v >= 0 (v already divided by the block scale): the
// count of grid midpoints below v, each midpoint going to the even code of
// its two neighbours (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0,
// 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0); past 5 everything is 6 (saturated).
CSA_DEV uint32_t e2m1_magnitude_code(float v) {
  return uint32_t(v > 0.25f) + uint32_t(v >= 0.75f) + uint32_t(v > 1.25f) + uint32_t(v >= 1.75f) +
         uint32_t(v > 2.5f) + uint32_t(v >= 3.5f) + uint32_t(v > 5.0f);
}

// Shared exponent of a block whose largest magnitude is amax:
// X = floor(log2(amax)) - 2 (2 being E2M1's largest exponent), at least
// -127; a zero block takes -127.  For fp32 inputs X <= 125, so 2^-X is a
// normal float.
CSA_DEV int mxfp4_block_exponent(float amax) { return amax > 0.f ? max(ilogbf(amax) - 2, -127) : -127; }

// 2^-X, exact.
CSA_DEV float mxfp4_inv_scale(int X) { return __uint_as_float(uint32_t(127 - X) << 23); }

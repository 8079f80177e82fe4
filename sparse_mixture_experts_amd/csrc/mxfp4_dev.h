// MXFP4 weight blocks.  "Phase 19: MoE - gpt-oss-20b", section 3 and the measured tensor
// layout, gives 16-byte blocks of 32 FP4 codes with one E8M0 scale byte each and
// value = fp4_lut[code] * 2^(scale - 127).  The page names the code table without printing
// it and leaves the nibble order open; this library reads the codes as OCP Microscaling
// E2M1 (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) with the low nibble of byte i
// holding element 2i (readings of the page, not statements of it).
#pragma once

#include "common.h"

namespace smoe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 2^(s - 127) as a float: the E8M0 scale.  s = 0 is 2^-127 (a subnormal float), s = 255
// is NaN.
__device__ __forceinline__ float e8m0_scale(uint32_t s) {
    const uint32_t bits = s == 0 ? 0x00400000u : (s == 255 ? 0x7FC00000u : s << 23);
    return __uint_as_float(bits);
}

// The two bf16 weights of byte B of a code word (low nibble first), times the block's
// scale: gfx950's scaled FP4 conversion.
template <int B>
__device__ __forceinline__ bf16x2_t fp4_pair_bf16(uint32_t cw, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, B);
}

// The 8 weights of a code word as 8 bf16 in element order (one 16-byte LDS chunk).
__device__ __forceinline__ uint4 fp4_word_bf16x8(uint32_t cw, float scale) {
    return make_uint4(__builtin_bit_cast(uint32_t, fp4_pair_bf16<0>(cw, scale)),
                      __builtin_bit_cast(uint32_t, fp4_pair_bf16<1>(cw, scale)),
                      __builtin_bit_cast(uint32_t, fp4_pair_bf16<2>(cw, scale)),
                      __builtin_bit_cast(uint32_t, fp4_pair_bf16<3>(cw, scale)));
}

}  // namespace smoe

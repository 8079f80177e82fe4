// Q4_K expert weight blocks (GGUF "K-quant"): device-side decoding.
//
// The pages name K-quant experts (Q3_K on "Qwen3.5-MoE Model Implementation", numeric
// status; Q4 / Q2 / Q3 GEMMs on "Engine", Prefill) without printing a block layout; the
// library reads the GGUF Q4_K definition.  A super-block holds 256 consecutive weights of
// a row in 144 bytes:
//   bytes 0-1   d     fp16, multiplier of the sub-block scales
//   bytes 2-3   dmin  fp16, multiplier of the sub-block mins
//   bytes 4-15  eight 6-bit scales sc_j and mins m_j of the 32-weight sub-blocks: for
//               j < 4 the low 6 bits of bytes 4+j (sc) and 8+j (m); for j >= 4 the low /
//               high nibble of byte 12+(j-4) gives the low 4 bits of sc_j / m_j and the
//               top 2 bits of byte 4+(j-4) / 8+(j-4) their top 2 bits
//   bytes 16-143  quants in 4 runs of 32 bytes: byte l of run c holds weight 64c + l in
//               its low nibble (sub-block 2c) and weight 64c + 32 + l in its high nibble
//   weight = d * sc_j * q - dmin * m_j
#pragma once

#include "common.h"

namespace smoe {

constexpr int kQ4kBlockBytes = 144;
constexpr int kQ4kBlockWeights = 256;

typedef __bf16 q4k_bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_f32(uint32_t h16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// Byte i (0..3, may vary per lane) of a 32-bit word.
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xFFu; }

// The multipliers of sub-block j (0..7) of a super-block whose first 16 bytes are `head`:
// a = d * sc_j (the quant multiplier) and b = dmin * m_j (the offset subtracted).
__device__ __forceinline__ void q4k_sub_scale(const uint4& head, int j, float& a, float& b) {
    const float d = half_bits_to_f32(head.x & 0xFFFFu), dmin = half_bits_to_f32(head.x >> 16);
    const int jj = j & 3;
    const uint32_t s_lo = byte_of(head.y, jj), m_lo = byte_of(head.z, jj), nib = byte_of(head.w, jj);
    uint32_t sc, mn;
    if (j < 4) {
        sc = s_lo & 63u;
        mn = m_lo & 63u;
    } else {
        sc = (nib & 15u) | ((s_lo >> 6) << 4);
        mn = (nib >> 4) | ((m_lo >> 6) << 4);
    }
    a = d * (float)sc;
    b = dmin * (float)mn;
}

// Quants as bf16 pairs offset by 128: for a word w of 4 quant bytes, pair P (0 or 1) holds
// bytes 2P and 2P+1, nibble H (0 low, 1 high), as the bf16 values 128 + q (bits 0x4300 | q,
// exact: 128 + q needs 8 significant bits).  A dot product with these pairs is
// sum (128 + q) x = sum q x + 128 sum x; the caller removes the 128 sum x term.
template <int P, int H>
__device__ __forceinline__ q4k_bf16x2_t q4k_pair(uint32_t w) {
    const uint32_t spread = __builtin_amdgcn_perm(w, w, P == 0 ? 0x0c010c00u : 0x0c030c02u);  // b0 | b1 << 16
    const uint32_t nib = H ? (spread >> 4) & 0x000F000Fu : spread & 0x000F000Fu;
    return __builtin_bit_cast(q4k_bf16x2_t, nib | 0x43004300u);
}

// The 8 weights of two quant words (nibble at bit `shift`, 0 or 4, of every byte) as a*q - b
// in bf16, element order: one 16-byte LDS chunk.
__device__ __forceinline__ uint32_t q4k_pair_bf16(uint32_t n, int byte, float a, float b) {
    q4k_bf16x2_t p;
    p[0] = (__bf16)fmaf(a, (float)((n >> (8 * byte)) & 0xFFu), -b);
    p[1] = (__bf16)fmaf(a, (float)((n >> (8 * byte + 8)) & 0xFFu), -b);
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint4 q4k_dequant8(uint32_t w0, uint32_t w1, int shift, float a, float b) {
    const uint32_t n0 = (w0 >> shift) & 0x0F0F0F0Fu, n1 = (w1 >> shift) & 0x0F0F0F0Fu;
    return make_uint4(q4k_pair_bf16(n0, 0, a, b), q4k_pair_bf16(n0, 2, a, b), q4k_pair_bf16(n1, 0, a, b),
                      q4k_pair_bf16(n1, 2, a, b));
}

}  // namespace smoe

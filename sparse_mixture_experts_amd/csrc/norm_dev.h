// Wave-level RMSNorm of one row ("Llama Forward Pass", Key Operations, RMSNorm; the mean
// square in fp32 as in "Phase 19: MoE - gpt-oss-20b", section 2), shared by the norm
// kernel and the router of the layer shell.
#pragma once

#include <math.h>

#include "common.h"

namespace smoe {

// VEC floats as one 16-byte vector of the storage type (bf16: round to nearest even).
template <typename TT>
__device__ __forceinline__ uint4 pack16(const float* f);
template <>
__device__ __forceinline__ uint4 pack16<BF16>(const float* f) {
    uint4 o;
    o.x = uint32_t(f32_to_bf16(f[0])) | (uint32_t(f32_to_bf16(f[1])) << 16);
    o.y = uint32_t(f32_to_bf16(f[2])) | (uint32_t(f32_to_bf16(f[3])) << 16);
    o.z = uint32_t(f32_to_bf16(f[4])) | (uint32_t(f32_to_bf16(f[5])) << 16);
    o.w = uint32_t(f32_to_bf16(f[6])) | (uint32_t(f32_to_bf16(f[7])) << 16);
    return o;
}
template <>
__device__ __forceinline__ uint4 pack16<F32>(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

// One wave: out[i] = row[i] / sqrt(mean(row^2) + eps) * w[i] for i < d (d a multiple of
// VEC), stored in the storage type to `out` and, when non-null, also to `out2`.  Lane l
// takes the 16-byte chunks l, l+64, ...; the sum of squares is fp32.
template <typename TT>
__device__ __forceinline__ void rmsnorm_row_wave(const typename TT::storage* __restrict__ row,
                                                 const typename TT::storage* __restrict__ w, float eps, int d,
                                                 typename TT::storage* out, typename TT::storage* out2) {
    constexpr int V = TT::VEC;
    const int lane = lane_id();
    const int nchunk = d / V;
    float ss = 0.0f;
    for (int c = lane; c < nchunk; c += kWave) {
        float f[V];
        unpack16<TT>(ld16(row + (size_t)c * V), f);
#pragma unroll
        for (int v = 0; v < V; ++v) ss = fmaf(f[v], f[v], ss);
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < nchunk; c += kWave) {
        float f[V], g[V];
        unpack16<TT>(ld16(row + (size_t)c * V), f);
        unpack16<TT>(ld16(w + (size_t)c * V), g);
#pragma unroll
        for (int v = 0; v < V; ++v) f[v] = f[v] * r * g[v];
        const uint4 o = pack16<TT>(f);
        *reinterpret_cast<uint4*>(out + (size_t)c * V) = o;
        if (out2) *reinterpret_cast<uint4*>(out2 + (size_t)c * V) = o;
    }
}

}  // namespace smoe

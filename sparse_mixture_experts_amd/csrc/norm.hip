// RMSNorm in front of the block, for the layer shell ("Llama Forward Pass", Key
// Operations, RMSNorm; "Phase 19: MoE - gpt-oss-20b", section 2, RMSNorm with the mean
// square in fp32): xn[t] = h[t] / sqrt(mean(h[t]^2) + eps) * w, stored in the layer's
// dtype (bf16 rounded to nearest even), which is what the block then reads
// ("Qwen3.5-MoE Model Implementation", Architecture: post-attention norm before the
// shared-MoE FFN).
#include <math.h>

#include "common.h"
#include "internal.h"

namespace smoe {
namespace {

// 16-byte vector of VEC floats in the storage type.
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

// One wave per row: lane l takes the 16-byte chunks l, l+64, ... of the row, sums their
// squares (fp32), and after the wave sum writes its chunks scaled by r * w.
template <typename TT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const typename TT::storage* __restrict__ h,
                                                      const typename TT::storage* __restrict__ w, float eps,
                                                      int T, int d, typename TT::storage* __restrict__ xn) {
    using S = typename TT::storage;
    constexpr int V = TT::VEC;
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    const int lane = lane_id();
    const S* row = h + (size_t)t * d;
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
    S* out = xn + (size_t)t * d;
    for (int c = lane; c < nchunk; c += kWave) {
        float f[V], g[V];
        unpack16<TT>(ld16(row + (size_t)c * V), f);
        unpack16<TT>(ld16(w + (size_t)c * V), g);
#pragma unroll
        for (int v = 0; v < V; ++v) f[v] = f[v] * r * g[v];
        *reinterpret_cast<uint4*>(out + (size_t)c * V) = pack16<TT>(f);
    }
}

}  // namespace

hipError_t launch_rmsnorm(const moe_layer& L, const void* h, int T, const void* w, float eps, void* xn,
                          hipStream_t s) {
    const dim3 grid((T + 3) / 4);
    if (L.dtype == MOE_BF16)
        rmsnorm_kernel<BF16><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w),
                                                  eps, T, L.d, static_cast<uint16_t*>(xn));
    else
        rmsnorm_kernel<F32><<<grid, 256, 0, s>>>(static_cast<const float*>(h), static_cast<const float*>(w), eps, T,
                                                 L.d, static_cast<float*>(xn));
    return hipGetLastError();
}

}  // namespace smoe

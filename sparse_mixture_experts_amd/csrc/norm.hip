// RMSNorm in front of the block, for the layer shell ("Llama Forward Pass", Key
// Operations, RMSNorm; "Phase 19: MoE - gpt-oss-20b", section 2, RMSNorm with the mean
// square in fp32): xn[t] = h[t] / sqrt(mean(h[t]^2) + eps) * w, stored in the layer's
// dtype (bf16 rounded to nearest even), which is what the block then reads
// ("Qwen3.5-MoE Model Implementation", Architecture: post-attention norm before the
// shared-MoE FFN).
#include "common.h"
#include "internal.h"
#include "norm_dev.h"

namespace smoe {
namespace {

// One wave per row.
template <typename TT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const typename TT::storage* __restrict__ h,
                                                      const typename TT::storage* __restrict__ w, float eps,
                                                      int T, int d, typename TT::storage* __restrict__ xn) {
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    rmsnorm_row_wave<TT>(h + (size_t)t * d, w, eps, d, xn + (size_t)t * d, nullptr);
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

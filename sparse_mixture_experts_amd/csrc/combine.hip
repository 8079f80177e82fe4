// Weighted combine ("Qwen3.5-MoE Model Implementation", MoE routing: out = moe_out +
// shexp_out, the residual left to the caller; "Phase 19: MoE - gpt-oss-20b", Experts:
// out = sum over the selected experts of score * y_e).
//
// y[t] = sum_{j<k} w[t,j] * Y_perm[perm_inv[t,j]] (+ sigmoid(a[t]) * Y_perm[T*k + t]),
// accumulated in fp32 in the fixed order j = 0..k-1 then the shared term, so results
// do not depend on scheduling.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace smoe {
namespace {

template <typename TT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ perm_inv,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ shared_gate, int T,
                                                      int k, int d, typename TT::storage* __restrict__ y) {
    const int t = blockIdx.x;
    const int tk = T * k;
    __shared__ int rows[32];
    __shared__ float wts[32];
    __shared__ float sg;
    if (threadIdx.x < k) {
        const int r = perm_inv[(size_t)t * k + threadIdx.x];
        rows[threadIdx.x] = (r >= 0 && r < tk) ? r : -1;
        wts[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
    }
    if (threadIdx.x == 0) sg = shared_gate ? 1.0f / (1.0f + expf(-shared_gate[t])) : 0.0f;
    __syncthreads();
    for (int i = threadIdx.x * 4; i < d; i += blockDim.x * 4) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const int r = rows[j];
            if (r < 0) continue;
            const float4 v = *reinterpret_cast<const float4*>(y_perm + (size_t)r * d + i);
            const float wj = wts[j];
            acc.x = fmaf(wj, v.x, acc.x);
            acc.y = fmaf(wj, v.y, acc.y);
            acc.z = fmaf(wj, v.z, acc.z);
            acc.w = fmaf(wj, v.w, acc.w);
        }
        if (shared_gate) {
            const float4 v = *reinterpret_cast<const float4*>(y_perm + (size_t)(tk + t) * d + i);
            acc.x = fmaf(sg, v.x, acc.x);
            acc.y = fmaf(sg, v.y, acc.y);
            acc.z = fmaf(sg, v.z, acc.z);
            acc.w = fmaf(sg, v.w, acc.w);
        }
        if constexpr (sizeof(typename TT::storage) == 2) {
            uint2 o;
            o.x = uint32_t(f32_to_bf16(acc.x)) | (uint32_t(f32_to_bf16(acc.y)) << 16);
            o.y = uint32_t(f32_to_bf16(acc.z)) | (uint32_t(f32_to_bf16(acc.w)) << 16);
            *reinterpret_cast<uint2*>(y + (size_t)t * d + i) = o;
        } else {
            *reinterpret_cast<float4*>(y + (size_t)t * d + i) = acc;
        }
    }
}

// Rows already carry their routing weight (and the shared rows their sigmoid gate):
// y[t] = sum_{j<k} Y[perm_inv[t,j]] (+ Y[T*k + t]), fp32 sum in the same fixed order.
template <typename TT>
__global__ __launch_bounds__(256) void combine_sum_kernel(const uint16_t* __restrict__ y_rows,
                                                          const int32_t* __restrict__ perm_inv, int T,
                                                          int k, int d, int shared,
                                                          typename TT::storage* __restrict__ y) {
    const int t = blockIdx.x;
    const int tk = T * k;
    __shared__ int rows[33];
    if (threadIdx.x < k) {
        const int r = perm_inv[(size_t)t * k + threadIdx.x];
        rows[threadIdx.x] = (r >= 0 && r < tk) ? r : -1;
    }
    if (threadIdx.x == 0) rows[k] = shared ? tk + t : -1;
    __syncthreads();
    for (int i = threadIdx.x * 8; i < d; i += blockDim.x * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j <= k; ++j) {
            const int r = rows[j];
            if (r < 0) continue;
            float v[8];
            unpack16<BF16>(ld16(y_rows + (size_t)r * d + i), v);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] += v[q];
        }
        if constexpr (sizeof(typename TT::storage) == 2) {
            uint4 o;
            o.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
            o.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
            o.z = uint32_t(f32_to_bf16(acc[4])) | (uint32_t(f32_to_bf16(acc[5])) << 16);
            o.w = uint32_t(f32_to_bf16(acc[6])) | (uint32_t(f32_to_bf16(acc[7])) << 16);
            *reinterpret_cast<uint4*>(y + (size_t)t * d + i) = o;
        } else {
            float4* o = reinterpret_cast<float4*>(y + (size_t)t * d + i);
            o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

}  // namespace

hipError_t launch_combine_sum(const moe_layer& L, const uint16_t* y_rows, const int32_t* perm_inv,
                              int T, void* y, hipStream_t s) {
    const int shared = L.shared_ff > 0 ? 1 : 0;
    if (L.dtype == MOE_BF16)
        combine_sum_kernel<BF16><<<T, 256, 0, s>>>(y_rows, perm_inv, T, L.k, L.d, shared,
                                                   static_cast<uint16_t*>(y));
    else
        combine_sum_kernel<F32><<<T, 256, 0, s>>>(y_rows, perm_inv, T, L.k, L.d, shared,
                                                  static_cast<float*>(y));
    return hipGetLastError();
}

hipError_t launch_combine(const moe_layer& L, const float* y_perm, const int32_t* perm_inv,
                          const float* w, const float* shared_gate, int T, void* y, hipStream_t s) {
    if (L.dtype == MOE_BF16)
        combine_kernel<BF16><<<T, 256, 0, s>>>(y_perm, perm_inv, w, shared_gate, T, L.k, L.d,
                                               static_cast<uint16_t*>(y));
    else
        combine_kernel<F32><<<T, 256, 0, s>>>(y_perm, perm_inv, w, shared_gate, T, L.k, L.d,
                                              static_cast<float*>(y));
    return hipGetLastError();
}

}  // namespace smoe

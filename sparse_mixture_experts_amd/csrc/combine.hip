// Weighted combine ("Qwen3.5-MoE Model Implementation", MoE routing: out = moe_out +
// shexp_out, the residual left to the caller of the block; "Phase 19: MoE - gpt-oss-20b",
// Experts: out = sum over the selected experts of score * y_e).
//
// y[t] = sum_{j<k} w[t,j] * Y_perm[perm_inv[t,j]] (+ sigmoid(a[t]) * Y_perm[T*k + t]),
// accumulated in fp32 in the fixed order j = 0..k-1 then the shared term, so results
// do not depend on scheduling.  The layer shell (same page, Architecture: the MoE FFN
// followed by the residual add) passes its input rows as `residual`, added last.
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
                                                      int k, int d,
                                                      const typename TT::storage* __restrict__ residual,
                                                      typename TT::storage* __restrict__ y) {
    const int t = blockIdx.x;
    const int tk = T * k;
    __shared__ int rows[40];  // k <= 32, read in batches of 8
    __shared__ float wts[40];
    __shared__ float sg;
    if (threadIdx.x < 40) {
        int r = -1;
        float wv = 0.0f;
        if (threadIdx.x < k) {
            r = perm_inv[(size_t)t * k + threadIdx.x];
            wv = w[(size_t)t * k + threadIdx.x];
        }
        rows[threadIdx.x] = (r >= 0 && r < tk) ? r : -1;
        wts[threadIdx.x] = wv;
    }
    if (threadIdx.x == 0) sg = shared_gate ? 1.0f / (1.0f + expf(-shared_gate[t])) : 0.0f;
    __syncthreads();
    for (int i = threadIdx.x * 4; i < d; i += blockDim.x * 4) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        // Up to 8 rows per batch, all loads issued before the FMAs; a missing row (-1)
        // reads row 0 with weight 0.
        for (int j0 = 0; j0 < k; j0 += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = (j0 + u < k) ? rows[j0 + u] : -1;
                v[u] = *reinterpret_cast<const float4*>(y_perm + (size_t)max(r, 0) * d + i);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bool ok = j0 + u < k && rows[j0 + u] >= 0;
                const float wj = ok ? wts[j0 + u] : 0.0f;
                acc.x = fmaf(wj, v[u].x, acc.x);
                acc.y = fmaf(wj, v[u].y, acc.y);
                acc.z = fmaf(wj, v[u].z, acc.z);
                acc.w = fmaf(wj, v[u].w, acc.w);
            }
        }
        if (shared_gate) {
            const float4 v = *reinterpret_cast<const float4*>(y_perm + (size_t)(tk + t) * d + i);
            acc.x = fmaf(sg, v.x, acc.x);
            acc.y = fmaf(sg, v.y, acc.y);
            acc.z = fmaf(sg, v.z, acc.z);
            acc.w = fmaf(sg, v.w, acc.w);
        }
        if (residual) {  // read before y is written: y may alias it
            float r[4];
            if constexpr (sizeof(typename TT::storage) == 2) {
                const uint2 q = *reinterpret_cast<const uint2*>(residual + (size_t)t * d + i);
                r[0] = bf16_lo(q.x); r[1] = bf16_hi(q.x); r[2] = bf16_lo(q.y); r[3] = bf16_hi(q.y);
            } else {
                const float4 q = *reinterpret_cast<const float4*>(residual + (size_t)t * d + i);
                r[0] = q.x; r[1] = q.y; r[2] = q.z; r[3] = q.w;
            }
            acc.x += r[0];
            acc.y += r[1];
            acc.z += r[2];
            acc.w += r[3];
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
                                                          const typename TT::storage* __restrict__ residual,
                                                          typename TT::storage* __restrict__ y) {
    const int t = blockIdx.x;
    const int tk = T * k;
    __shared__ int rows[40];  // k + 1 <= 33 rows, read in batches of 8
    if (threadIdx.x < 40) {
        int r = -1;
        if (threadIdx.x < k) {
            r = perm_inv[(size_t)t * k + threadIdx.x];
            r = (r >= 0 && r < tk) ? r : -1;
        } else if (threadIdx.x == k && shared) {
            r = tk + t;
        }
        rows[threadIdx.x] = r;
    }
    __syncthreads();
    for (int i = threadIdx.x * 8; i < d; i += blockDim.x * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // Rows j = 0..k (k+1 = shared), up to 8 per batch with the loads issued first; a
        // missing row reads row 0 and is not added.
        for (int j0 = 0; j0 <= k; j0 += 8) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = (j0 + u <= k) ? rows[j0 + u] : -1;
                v[u] = ld16(y_rows + (size_t)max(r, 0) * d + i);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u > k || rows[j0 + u] < 0) continue;
                float f[8];
                unpack16<BF16>(v[u], f);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] += f[q];
            }
        }
        if (residual) {  // read before y is written: y may alias it
            float r[8];
            const typename TT::storage* rp = residual + (size_t)t * d + i;
            if constexpr (sizeof(typename TT::storage) == 2) {
                unpack16<BF16>(ld16(rp), r);
            } else {
                unpack16<F32>(ld16(rp), r);
                unpack16<F32>(ld16(rp + 4), r + 4);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] += r[q];
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
                              int T, const void* residual, void* y, hipStream_t s) {
    const int shared = L.shared_ff > 0 ? 1 : 0;
    if (L.dtype == MOE_BF16)
        combine_sum_kernel<BF16><<<T, 256, 0, s>>>(y_rows, perm_inv, T, L.k, L.d, shared,
                                                   static_cast<const uint16_t*>(residual),
                                                   static_cast<uint16_t*>(y));
    else
        combine_sum_kernel<F32><<<T, 256, 0, s>>>(y_rows, perm_inv, T, L.k, L.d, shared,
                                                  static_cast<const float*>(residual), static_cast<float*>(y));
    return hipGetLastError();
}

hipError_t launch_combine(const moe_layer& L, const float* y_perm, const int32_t* perm_inv,
                          const float* w, const float* shared_gate, int T, const void* residual, void* y,
                          hipStream_t s) {
    if (L.dtype == MOE_BF16)
        combine_kernel<BF16><<<T, 256, 0, s>>>(y_perm, perm_inv, w, shared_gate, T, L.k, L.d,
                                               static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(y));
    else
        combine_kernel<F32><<<T, 256, 0, s>>>(y_perm, perm_inv, w, shared_gate, T, L.k, L.d,
                                              static_cast<const float*>(residual), static_cast<float*>(y));
    return hipGetLastError();
}

}  // namespace smoe

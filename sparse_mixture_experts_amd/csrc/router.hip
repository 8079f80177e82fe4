// Router: logits z = W_r x (+ b_r), the shared-expert gate input w_sg . x, and the
// wave-level top-k with the routing weights of either mode.
//
// "Qwen3.5-MoE Model Implementation", MoE routing: router matrix [n_expert, n_embd],
// softmax, top-8, renormalisation, expert_weights_scale; the shared expert's scalar
// sigmoid gate [n_embd].  "Phase 19: MoE - gpt-oss-20b", Router: logits with bias,
// top-k first, softmax over the k selected.
#include <math.h>

#include "internal.h"
#include "rowdot.h"

namespace smoe {
namespace {

constexpr int kRouterTokChunk = 64;  // tokens per block along grid.y
constexpr int kRouterNT = 4;         // tokens per rows_dot call

// One wave per router row (rows 0..E-1 are experts, row E the shared gate vector),
// looping over a chunk of tokens.  Writes logits[t * ld + row].
template <int KB, typename TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(
    const typename TT::storage* __restrict__ x, const typename TT::storage* __restrict__ w_router,
    const float* __restrict__ b_router, const typename TT::storage* __restrict__ w_sg, int T, int d,
    int E, int n_rows, float* __restrict__ logits, int ld) {
    const int row = blockIdx.x * 4 + threadIdx.x / kWave;
    if (row >= n_rows) return;
    const typename TT::storage* const wr[1] = {row < E ? w_router + (size_t)row * d : w_sg};
    const float bias = (row < E && b_router) ? b_router[row] : 0.0f;
    const int t_end = min(T, (int)(blockIdx.y + 1) * kRouterTokChunk);
    for (int t0 = blockIdx.y * kRouterTokChunk; t0 < t_end; t0 += kRouterNT) {
        const int nt = min(kRouterNT, t_end - t0);
        const typename TT::storage* ar[kRouterNT];
#pragma unroll
        for (int t = 0; t < kRouterNT; ++t) ar[t] = x + (size_t)min(t0 + t, T - 1) * d;
        float acc[1][kRouterNT] = {};
        rows_dot<1, kRouterNT, KB, TT, TT>(wr, ar, nt, d, acc);
#pragma unroll
        for (int t = 0; t < kRouterNT; ++t) {
            const float z = wave_sum(acc[0][t]);
            if (lane_id() == 0 && t < nt) logits[(size_t)(t0 + t) * ld + row] = z + bias;
        }
    }
}

// Does (va, ia) rank before (vb, ib)?  Larger logit first, ties to the lower index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

constexpr int kMaxPerLane = 8;  // E <= 512

// One wave per token: k rounds of a wave arg-max by xor shuffles, then the weights.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int ld, int T,
                                                   int E, int k, int mode, float scale,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ w_out,
                                                   float* __restrict__ sg_out) {
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const float* z = logits + (size_t)t * ld;
    float v[kMaxPerLane];
    int id[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + i * kWave;
        v[i] = e < E ? z[e] : -INFINITY;
        id[i] = e < E ? e : INT32_MAX;
    }
    float my_v = -INFINITY;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = INT32_MAX;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if (ranks_before(v[i], id[i], bv, bi)) { bv = v[i]; bi = id[i]; }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        // Non-finite logits can leave no candidate: keep the index in range.
        if (bi >= E) bi = 0;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if (id[i] == bi) { v[i] = -INFINITY; id[i] = INT32_MAX; }
        if (lane == j) { my_v = bv; my_i = bi; }
    }
    // Weights over the selected logits: exp(z_j - z_0) / sum_j' exp(z_j' - z_0).  In
    // mode SOFTMAX_TOPK_RENORM the full-softmax denominator cancels in the
    // renormalisation, so both modes share this form; mode A then applies the scale.
    const float zmax = __shfl(my_v, 0, kWave);
    const float ex = lane < k ? expf(my_v - zmax) : 0.0f;
    const float den = wave_sum(ex);
    if (lane < k) {
        float w = ex / den;
        if (mode == MOE_ROUTE_SOFTMAX_TOPK_RENORM) w *= scale;
        idx_out[(size_t)t * k + lane] = my_i;
        w_out[(size_t)t * k + lane] = w;
    }
    if (sg_out && lane == 0) sg_out[t] = z[E];
}

template <typename TT>
hipError_t launch_router_t(const moe_layer& L, const void* x, int T, float* logits, int ld,
                           hipStream_t s) {
    using S = typename TT::storage;
    const int n_rows = L.n_expert + (L.shared_ff > 0 ? 1 : 0);
    dim3 grid((n_rows + 3) / 4, (T + kRouterTokChunk - 1) / kRouterTokChunk);
    const S* xs = static_cast<const S*>(x);
    const S* wr = static_cast<const S*>(L.w_router);
    const S* wsg = static_cast<const S*>(L.ws_gate_inp);
    switch (pick_kb(L.d, TT::VEC)) {
#define SMOE_ROUTER_CASE(KB)                                                                   \
    case KB:                                                                                   \
        router_gemv_kernel<KB, TT><<<grid, 256, 0, s>>>(xs, wr, L.b_router, wsg, T, L.d,        \
                                                        L.n_expert, n_rows, logits, ld);       \
        break;
        SMOE_ROUTER_CASE(1)
        SMOE_ROUTER_CASE(2)
        SMOE_ROUTER_CASE(4)
        SMOE_ROUTER_CASE(8)
#undef SMOE_ROUTER_CASE
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const moe_layer& L, const void* x, int T, float* logits, int ld,
                                hipStream_t s) {
    return L.dtype == MOE_BF16 ? launch_router_t<BF16>(L, x, T, logits, ld, s)
                               : launch_router_t<F32>(L, x, T, logits, ld, s);
}

hipError_t launch_topk(const moe_layer& L, const float* logits, int ld, int T, int32_t* idx,
                       float* w, float* shared_gate, hipStream_t s) {
    topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ld, T, L.n_expert, L.k, L.route,
                                             L.route_scale, idx, w, shared_gate);
    return hipGetLastError();
}

}  // namespace smoe

// Wave-level top-k over one token's router logits ("Qwen3.5-MoE Model Implementation",
// MoE routing: softmax, top-8, renormalisation, expert_weights_scale; "Phase 19: MoE -
// gpt-oss-20b", Router: top-k, then softmax over the selected logits).
#pragma once

#include <math.h>

#include "common.h"
#include "internal.h"
#include "rowdot.h"

namespace smoe {

constexpr int kRouterNT = 4;  // tokens per rows_dot call

// One wave: router row `row` (rows 0..E-1 are experts, row E the shared-gate vector) over
// tokens [t0, t_end), written to logits[t * ld + row] (+ the expert's bias).
template <int KB, typename TT>
__device__ __forceinline__ void router_row_wave(const typename TT::storage* __restrict__ x,
                                                const typename TT::storage* __restrict__ w_router,
                                                const float* __restrict__ b_router,
                                                const typename TT::storage* __restrict__ w_sg, int T, int d,
                                                int E, int row, int t0, int t_end, float* __restrict__ logits,
                                                int ld) {
    const typename TT::storage* const wr[1] = {row < E ? w_router + (size_t)row * d : w_sg};
    const float bias = (row < E && b_router) ? b_router[row] : 0.0f;
    for (; t0 < t_end; t0 += kRouterNT) {
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

// Lane moves inside 16-lane rows (DPP): quad permutes [1,0,3,2] and [2,3,0,1], the
// half-row mirror (lane i <- 7-i within 8) and the row mirror (lane i <- 15-i).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
    const float ov = __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
    const int oi = dpp_i<CTRL>(i);
    if (ranks_before(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Wave-wide best (value, index) under ranks_before, returned to every lane: four DPP
// steps make each 16-lane row uniform, then the four row winners are read and compared.
// The order is strict (indices are distinct), so both sides of every step agree.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_step<0xB1>(v, i);
    argmax_step<0x4E>(v, i);
    argmax_step<0x141>(v, i);
    argmax_step<0x140>(v, i);
    float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (ranks_before(rv, ri, bv, bi)) {
            bv = rv;
            bi = ri;
        }
    }
    v = bv;
    i = bi;
}

constexpr int kMaxPerLane = 8;  // E <= 512

// Called by a whole wave for one token's logits z[0..E).  Lane j < k receives the j-th
// selected expert (descending logit, ties to the lower index) and its weight.
// Selection: k rounds; each lane keeps the best of its E/64 logits, a wave arg-max finds
// the wave's best, whose owner retires it.
// Weights: exp(z_j - z_0) / sum_j' exp(z_j' - z_0) over the k selected.  In mode
// SOFTMAX_TOPK_RENORM the full-softmax denominator cancels in the renormalisation, so
// both modes share this form; that mode then applies the expert weight scale.
__device__ __forceinline__ void topk_wave(const float* z, int E, int k, int mode, float scale,
                                          int* out_i, float* out_w) {
    const int lane = lane_id();
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
        wave_argmax(bv, bi);
        // Non-finite logits can leave no candidate: keep the index in range.
        if (bi >= E) bi = 0;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if (id[i] == bi) { v[i] = -INFINITY; id[i] = INT32_MAX; }
        if (lane == j) { my_v = bv; my_i = bi; }
    }
    const float zmax = __shfl(my_v, 0, kWave);
    const float ex = lane < k ? expf(my_v - zmax) : 0.0f;
    const float den = wave_sum(ex);
    float w = ex / den;
    if (mode == MOE_ROUTE_SOFTMAX_TOPK_RENORM) w *= scale;
    *out_i = my_i;
    *out_w = w;
}

}  // namespace smoe

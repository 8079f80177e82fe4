// Wave-level top-k over one token's router logits ("Qwen3.5-MoE Model Implementation",
// MoE routing: softmax, top-8, renormalisation, expert_weights_scale; "Phase 19: MoE -
// gpt-oss-20b", Router: top-k, then softmax over the selected logits).
#pragma once

#include <math.h>

#include "common.h"
#include "internal.h"

namespace smoe {

// Does (va, ia) rank before (vb, ib)?  Larger logit first, ties to the lower index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

constexpr int kMaxPerLane = 8;  // E <= 512

// Called by a whole wave for one token's logits z[0..E).  Lane j < k receives the j-th
// selected expert (descending logit, ties to the lower index) and its weight.
// Selection: k rounds; each lane keeps the best of its E/64 logits, a 6-step xor-shuffle
// arg-max finds the wave's best, whose owner retires it.
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
    const float zmax = __shfl(my_v, 0, kWave);
    const float ex = lane < k ? expf(my_v - zmax) : 0.0f;
    const float den = wave_sum(ex);
    float w = ex / den;
    if (mode == MOE_ROUTE_SOFTMAX_TOPK_RENORM) w *= scale;
    *out_i = my_i;
    *out_w = w;
}

}  // namespace smoe

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
constexpr int kRouterNR = 4;  // router rows per wave (a few tokens: 1, for more waves)

// One wave: router rows row0 .. row0+NR-1 (rows 0..E-1 are experts, row E the shared-gate
// vector; rows past n_rows repeat the last and are not written) over tokens
// [t0, t_end), written to logits[t * ld + row] (+ the expert's bias).  Token t's row is
// x + (t - x_first) * d.
template <int KB, typename TT, int NR>
__device__ __forceinline__ void router_rows_wave(const typename TT::storage* __restrict__ x,
                                                 const typename TT::storage* __restrict__ w_router,
                                                 const float* __restrict__ b_router,
                                                 const typename TT::storage* __restrict__ w_sg, int T, int d,
                                                 int E, int n_rows, int row0, int t0, int t_end,
                                                 float* __restrict__ logits, int ld, int x_first = 0) {
    using S = typename TT::storage;
    constexpr int NT = kRouterNT, N = NR * NT;
    constexpr int SH = 6 - ilog2(N);
    const S* wr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int row = min(row0 + r, n_rows - 1);
        wr[r] = row < E ? w_router + (size_t)row * d : w_sg;
    }
    const S* const (&wrc)[NR] = wr;
    // After the reduction lane l holds value (t * NR + r) = l >> SH.
    const int lane = lane_id();
    const int my_t = (lane >> SH) / NR, my_row = row0 + (lane >> SH) % NR;
    const bool writer = (lane & ((1 << SH) - 1)) == 0 && my_row < n_rows;
    const float bias = (writer && my_row < E && b_router) ? b_router[my_row] : 0.0f;
    for (; t0 < t_end; t0 += NT) {
        const int nt = min(NT, t_end - t0);
        const S* ar[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) ar[t] = x + (size_t)(min(t0 + t, T - 1) - x_first) * d;
        const S* const (&arc)[NT] = ar;
        float acc[NR][NT] = {};
        rows_dot<NR, NT, KB, TT, TT>(wrc, arc, nt, d, acc);
        float v[N];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) v[t * NR + r] = acc[r][t];
        const float z = wave_reduce_scatter<N>(v);
        if (writer && my_t < nt) logits[(size_t)(t0 + my_t) * ld + my_row] = z + bias;
    }
}

// Order-preserving 32-bit key of a logit: unsigned comparison of keys is the float order
// (-0 and +0 share one key, as they compare equal).  NaN gets key 1, below every other
// value (-inf included) and above key 0, which marks retired and absent entries.
__device__ __forceinline__ unsigned logit_key(float v) {
    v = v + 0.0f;  // -0 -> +0
    unsigned u = __float_as_uint(v);
    u ^= static_cast<unsigned>(static_cast<int>(u) >> 31) | 0x80000000u;
    return v != v ? 1u : u;
}

__device__ __forceinline__ float key_logit(unsigned key) {
    const unsigned u = (key >> 31) ? (key & 0x7FFFFFFFu) : ~key;
    return key == 1u ? __uint_as_float(0x7FC00000u) : __uint_as_float(u);
}

// Lane-to-lane max through DPP.  The zero `old` operand is the identity of unsigned max,
// which lets the compiler fold each move into one v_max_u32_dpp.  Inside 16-lane rows:
// quad permutes [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors leave every
// lane with its row's max; the two row broadcasts (lane 15 into rows 1 and 3, lane 31
// into rows 2 and 3) carry the wave max to lane 63.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ unsigned dpp_max(unsigned m) {
    return max(m, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), CTRL, ROW_MASK,
                                                                      0xF, false)));
}

__device__ __forceinline__ unsigned wave_max_key(unsigned m) {
    m = dpp_max<0xB1>(m);
    m = dpp_max<0x4E>(m);
    m = dpp_max<0x141>(m);
    m = dpp_max<0x140>(m);
    m = dpp_max<0x142, 0xA>(m);
    m = dpp_max<0x143, 0xC>(m);
    return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(m), 63));
}

// Top-k of one token's logits z[0..E) on one wave (E <= 64 * PL).  Lane j < k returns
// the j-th selected expert (descending logit, ties to the lower index) and its weight.
// Selection: k rounds of a wave max over the keys; the lowest expert index holding the
// max (ballot per register slot, expert = lane + 64 * slot) is taken and retired.
// Weights: exp(z_j - z_0) / sum_j' exp(z_j' - z_0) over the k selected.  In mode
// SOFTMAX_TOPK_RENORM the full-softmax denominator cancels in the renormalisation, so
// both modes share this form; that mode then applies the expert weight scale.
// Requires 1 <= k <= min(E, 64).
template <int PL>
__device__ __forceinline__ void topk_wave_pl(const float* z, int E, int k, int mode, float scale,
                                             int* out_i, float* out_w) {
    const int lane = lane_id();
    unsigned key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + i * kWave;
        key[i] = e < E ? logit_key(z[e]) : 0u;
    }
    unsigned my_key = 0;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
        unsigned m = key[0];
#pragma unroll
        for (int i = 1; i < PL; ++i) m = max(m, key[i]);
        m = wave_max_key(m);
        int slot = 0;
        unsigned long long owners = 0;
#pragma unroll
        for (int i = PL - 1; i >= 0; --i) {
            const unsigned long long b = __ballot(key[i] == m);
            if (b) {
                slot = i;
                owners = b;
            }
        }
        const int owner = __builtin_ctzll(owners);
        const bool mine = lane == owner;
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (i == slot && mine) key[i] = 0u;
        if (lane == j) {
            my_key = m;
            my_i = owner + slot * kWave;
        }
    }
    if (my_i >= E) my_i = 0;  // unreachable for k <= E; keeps the index in range
    const float my_v = key_logit(my_key);
    const float zmax = __shfl(my_v, 0, kWave);
    const float ex = lane < k ? expf(my_v - zmax) : 0.0f;
    const float den = wave_sum(ex);
    float w = ex / den;
    if (mode == MOE_ROUTE_SOFTMAX_TOPK_RENORM) w *= scale;
    *out_i = my_i;
    *out_w = w;
}

constexpr int kMaxPerLane = 8;  // E <= 512

__device__ __forceinline__ void topk_wave(const float* z, int E, int k, int mode, float scale, int* out_i,
                                          float* out_w) {
    if (E <= kWave) topk_wave_pl<1>(z, E, k, mode, scale, out_i, out_w);
    else if (E <= 2 * kWave) topk_wave_pl<2>(z, E, k, mode, scale, out_i, out_w);
    else if (E <= 4 * kWave) topk_wave_pl<4>(z, E, k, mode, scale, out_i, out_w);
    else topk_wave_pl<kMaxPerLane>(z, E, k, mode, scale, out_i, out_w);
}

}  // namespace smoe

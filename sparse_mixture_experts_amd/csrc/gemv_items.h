// Wave-level work items of the decode GEMVs (the kernels of expert_gemv.hip).
//
// "Qwen3.5-MoE Model Implementation", MoE routing: each routed expert is a SwiGLU,
// silu(gate . x) * (up . x) then down; the shared expert is one more SwiGLU over every
// token.  "Phase 19: MoE - gpt-oss-20b", Experts: fused interleaved gate_up with bias,
// clamps, (up + 1) * gate * sigmoid(alpha * gate), down with bias.
//
// up_item: a wave owns 2 hidden units f, f+1 of one group: it streams the 4 weight rows
// (gate f, gate f+1, up f, up f+1 -- or the 4 interleaved gate_up rows) and dots them
// with the group's rows of x, then applies the activation and writes H[row, f..f+1] in
// fp32.  down_item: a wave owns 4 output dims i..i+3 of one group: it streams the 4 rows
// of W_d and dots them with the group's rows of H, writing Y_perm[row, i..i+3].
#pragma once

#include "internal.h"
#include "rowdot.h"

namespace smoe {

constexpr int kNT = 4;  // rows per rows_dot call

struct GemvUp {
    const void* x;
    const int32_t* perm_token;
    const Group* groups;
    const void* w_gate;     // SWIGLU [E, ff, d]
    const void* w_up;
    const void* w_gate_up;  // OAI [E, 2ff, d]
    const void* b_gate_up;  // OAI [E, 2ff]
    const void* ws_gate;    // shared [ffs, d]
    const void* ws_up;
    float* H;
    int hstride, T, d, ff, ffs;
    float alpha, limit;
};

struct GemvDown {
    const float* H;
    const Group* groups;
    const void* w_down;   // [E, d, ff]
    const void* b_down;   // OAI [E, d] or null
    const void* ws_down;  // [d, ffs]
    float* y;
    int hstride, d, ff, ffs;
};

// One wave: hidden units f0, f0+1 (f0 even, f0 < the group's hidden width) of group g,
// for every row of the group.  RESIDENT: the whole K axis fits one KB-chunk register
// batch, so the 4 weight rows are streamed once and every row is served from registers.
template <int KB, typename TT, bool OAI, bool RESIDENT>
__device__ __forceinline__ void up_item(const GemvUp& a, const Group& g, int f0) {
    using S = typename TT::storage;
    const bool shared = g.e < 0;
    const size_t d = a.d;
    // The shared expert is always a plain SwiGLU, also in a layer of clamped experts.
    const bool oai = OAI && !shared;
    const S* wr[4];
    if (oai) {
        const S* base = static_cast<const S*>(a.w_gate_up) + ((size_t)g.e * 2 * a.ff + 2 * f0) * d;
        // rows: gate f0, up f0, gate f0+1, up f0+1
        for (int r = 0; r < 4; ++r) wr[r] = base + r * d;
    } else {
        const S* gb = shared ? static_cast<const S*>(a.ws_gate) : static_cast<const S*>(a.w_gate) + (size_t)g.e * a.ff * d;
        const S* ub = shared ? static_cast<const S*>(a.ws_up) : static_cast<const S*>(a.w_up) + (size_t)g.e * a.ff * d;
        // rows: gate f0, gate f0+1, up f0, up f0+1
        wr[0] = gb + f0 * d;
        wr[1] = gb + (f0 + 1) * d;
        wr[2] = ub + f0 * d;
        wr[3] = ub + (f0 + 1) * d;
    }
    const S* const wrc[4] = {wr[0], wr[1], wr[2], wr[3]};
    float bg[2] = {0.f, 0.f}, bu[2] = {0.f, 0.f};
    if (oai) {
        const S* b = static_cast<const S*>(a.b_gate_up) + (size_t)g.e * 2 * a.ff + 2 * f0;
        for (int f = 0; f < 2; ++f) {
            if constexpr (sizeof(S) == 2) {
                bg[f] = bf16_to_f32(b[2 * f]);
                bu[f] = bf16_to_f32(b[2 * f + 1]);
            } else {
                bg[f] = b[2 * f];
                bu[f] = b[2 * f + 1];
            }
        }
    }
    const S* x = static_cast<const S*>(a.x);
    const int lane = lane_id();
    // Whole K in one register batch: stream the 4 weight rows once and loop over every
    // row of the group from registers.
    uint4 wv[RESIDENT ? KB : 1][4];
    if constexpr (RESIDENT) load_w_batch<4, KB, TT, true>(wrc, a.d, 0, wv);
    for (int tb = 0; tb < g.n; tb += kNT) {
        const int nt = min(kNT, g.n - tb);
        const S* ar[kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            const int r = min(tb + t, g.n - 1);
            int tok = shared ? r : a.perm_token[g.row0 + r];
            tok = min(max(tok, 0), a.T - 1);
            ar[t] = x + (size_t)tok * d;
        }
        const S* const arc[kNT] = {ar[0], ar[1], ar[2], ar[3]};
        float acc[4][kNT] = {};
        if constexpr (RESIDENT) dot_w_batch<4, kNT, KB, TT, TT>(wv, arc, nt, a.d, 0, acc);
        else rows_dot<4, kNT, KB, TT, TT, true>(wrc, arc, nt, a.d, acc);
        float h[2][kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            if (t >= nt) continue;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                if (oai) {
                    float gv = wave_sum(acc[2 * f][t]) + bg[f];
                    float uv = wave_sum(acc[2 * f + 1][t]) + bu[f];
                    gv = fminf(gv, a.limit);
                    uv = fminf(fmaxf(uv, -a.limit), a.limit);
                    h[f][t] = (uv + 1.0f) * gv * sigmoidf_(a.alpha * gv);
                } else {
                    const float gv = wave_sum(acc[f][t]);
                    const float uv = wave_sum(acc[2 + f][t]);
                    h[f][t] = gv * sigmoidf_(gv) * uv;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
            for (int f = 0; f < 2; ++f)
                if (lane == f + 2 * t && t < nt) a.H[(size_t)(g.row0 + tb + t) * a.hstride + f0 + f] = h[f][t];
    }
}

// One wave: output dims i0..i0+3 (i0 < d, d a multiple of 4) of group g, for every row.
template <int KB, typename TT, bool OAI, bool RESIDENT>
__device__ __forceinline__ void down_item(const GemvDown& a, const Group& g, int i0) {
    using S = typename TT::storage;
    const bool shared = g.e < 0;
    const int K = shared ? a.ffs : a.ff;
    const S* base = shared ? static_cast<const S*>(a.ws_down) + (size_t)i0 * K
                           : static_cast<const S*>(a.w_down) + ((size_t)g.e * a.d + i0) * K;
    const S* const wr[4] = {base, base + K, base + 2 * (size_t)K, base + 3 * (size_t)K};
    float bias[4] = {0.f, 0.f, 0.f, 0.f};
    if (OAI && !shared && a.b_down) {
        const S* b = static_cast<const S*>(a.b_down) + (size_t)g.e * a.d + i0;
        for (int r = 0; r < 4; ++r) {
            if constexpr (sizeof(S) == 2) bias[r] = bf16_to_f32(b[r]);
            else bias[r] = b[r];
        }
    }
    const int lane = lane_id();
    uint4 wv[RESIDENT ? KB : 1][4];
    if constexpr (RESIDENT) load_w_batch<4, KB, TT, true>(wr, K, 0, wv);
    for (int tb = 0; tb < g.n; tb += kNT) {
        const int nt = min(kNT, g.n - tb);
        const float* ar[kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) ar[t] = a.H + (size_t)(g.row0 + min(tb + t, g.n - 1)) * a.hstride;
        const float* const arc[kNT] = {ar[0], ar[1], ar[2], ar[3]};
        float acc[4][kNT] = {};
        if constexpr (RESIDENT) dot_w_batch<4, kNT, KB, TT, F32>(wv, arc, nt, K, 0, acc);
        else rows_dot<4, kNT, KB, TT, F32, true>(wr, arc, nt, K, acc);
        float out[4][kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            if (t >= nt) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r][t] = wave_sum(acc[r][t]) + bias[r];
        }
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (lane == r + 4 * t && t < nt) a.y[(size_t)(g.row0 + tb + t) * a.d + i0 + r] = out[r][t];
    }
}

}  // namespace smoe

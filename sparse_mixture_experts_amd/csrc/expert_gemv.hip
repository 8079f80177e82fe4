// Expert FFNs as HBM-streaming GEMVs over the active groups only (the decode path).
//
// "Qwen3.5-MoE Model Implementation", MoE routing: each routed expert is a SwiGLU,
// silu(gate . x) * (up . x) then down; the shared expert is one more SwiGLU over every
// token.  "Phase 19: MoE - gpt-oss-20b", Experts: fused interleaved gate_up with bias,
// clamps, (up + 1) * gate * sigmoid(alpha * gate), down with bias.  The group list is
// the union of experts the batch selected ("Engine", Address tables): only their
// weights are read, each once per block of up to 4 routed rows.
//
// Kernel 1 (up): a wave owns 2 hidden units f, f+1 of one group: it streams the 4
// weight rows (gate f, gate f+1, up f, up f+1 -- or the 4 interleaved gate_up rows)
// and dots them with the group's rows of x, then applies the activation and writes
// H[row, f..f+1] in fp32.
// Kernel 2 (down): a wave owns 4 output dims i..i+3 of one group: it streams the 4
// rows of W_d and dots them with the group's rows of H, writing Y_perm[row, i..i+3].
// Grids are sized for the largest possible number of groups; blocks beyond the
// device-side group count return at once, so no host synchronisation is needed.
#include "internal.h"
#include "rowdot.h"

namespace smoe {
namespace {

constexpr int kNT = 4;  // rows per rows_dot call

struct UpArgs {
    const void* x;
    const int32_t* perm_token;
    const Group* groups;
    const PlanMeta* meta;
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

struct DownArgs {
    const float* H;
    const Group* groups;
    const PlanMeta* meta;
    const void* w_down;   // [E, d, ff]
    const void* b_down;   // OAI [E, d] or null
    const void* ws_down;  // [d, ffs]
    float* y;
    int hstride, d, ff, ffs;
};

// Group handled by grid row y.  With a shared expert (always the last group, and the
// one with the most rows) grid row 0 takes it, so its longer work starts first.
__device__ __forceinline__ int group_of_row(int y, int n_groups, bool has_shared) {
    return has_shared ? (y == 0 ? n_groups - 1 : y - 1) : y;
}

// RESIDENT: the whole K axis fits one KB-chunk register batch (chosen at launch).
template <int KB, typename TT, bool OAI, bool RESIDENT>
__global__ __launch_bounds__(256) void expert_up_gemv_kernel(UpArgs a) {
    using S = typename TT::storage;
    const PlanMeta meta = *a.meta;
    if ((int)blockIdx.y >= meta.n_groups) return;
    const Group g = a.groups[group_of_row(blockIdx.y, meta.n_groups, a.ffs > 0)];
    const bool shared = g.e < 0;
    const int ffg = shared ? a.ffs : a.ff;
    const int f0 = (blockIdx.x * 4 + threadIdx.x / kWave) * 2;
    if (f0 >= ffg) return;
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

template <int KB, typename TT, bool OAI, bool RESIDENT>
__global__ __launch_bounds__(256) void expert_down_gemv_kernel(DownArgs a) {
    using S = typename TT::storage;
    const PlanMeta meta = *a.meta;
    if ((int)blockIdx.y >= meta.n_groups) return;
    const Group g = a.groups[group_of_row(blockIdx.y, meta.n_groups, a.ffs > 0)];
    const bool shared = g.e < 0;
    const int K = shared ? a.ffs : a.ff;
    const int i0 = (blockIdx.x * 4 + threadIdx.x / kWave) * 4;
    if (i0 >= a.d) return;
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

template <typename TT, bool OAI>
hipError_t launch_t(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                    const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                    hipStream_t s) {
    const bool shared = L.shared_ff > 0;
    const int gmax = max_groups(L.n_expert, T, L.k, shared);
    UpArgs u{x, perm_token, groups, meta, L.w_gate, L.w_up, L.w_gate_up, L.b_gate_up,
             L.ws_gate, L.ws_up, H, hstride, T, L.d, L.ff, L.shared_ff, L.oai_alpha, L.oai_limit};
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    dim3 gu((ffmax + 7) / 8, gmax);
    const bool up_res = chunks(L.d, TT::VEC) <= 8;
    switch (pick_kb(L.d, TT::VEC)) {
#define SMOE_UP_CASE(KB)                                                                      \
    case KB:                                                                                  \
        if (up_res) expert_up_gemv_kernel<KB, TT, OAI, true><<<gu, 256, 0, s>>>(u);           \
        else expert_up_gemv_kernel<KB, TT, OAI, false><<<gu, 256, 0, s>>>(u);                 \
        break;
        SMOE_UP_CASE(1)
        SMOE_UP_CASE(2)
        SMOE_UP_CASE(4)
        SMOE_UP_CASE(8)
#undef SMOE_UP_CASE
    }
    DownArgs dn{H, groups, meta, L.w_down, L.b_down, L.ws_down, y_perm, hstride, L.d, L.ff, L.shared_ff};
    dim3 gd((L.d + 15) / 16, gmax);
    const bool dn_res = chunks(ffmax, TT::VEC) <= 8;
    switch (pick_kb(ffmax, TT::VEC)) {
#define SMOE_DOWN_CASE(KB)                                                                    \
    case KB:                                                                                  \
        if (dn_res) expert_down_gemv_kernel<KB, TT, OAI, true><<<gd, 256, 0, s>>>(dn);        \
        else expert_down_gemv_kernel<KB, TT, OAI, false><<<gd, 256, 0, s>>>(dn);              \
        break;
        SMOE_DOWN_CASE(1)
        SMOE_DOWN_CASE(2)
        SMOE_DOWN_CASE(4)
        SMOE_DOWN_CASE(8)
#undef SMOE_DOWN_CASE
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gemv(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                              const Group* groups, const PlanMeta* meta, float* H, int hstride,
                              float* y_perm, hipStream_t s) {
    const bool oai = L.act == MOE_ACT_SWIGLU_OAI;
    if (L.dtype == MOE_BF16)
        return oai ? launch_t<BF16, true>(L, x, T, perm_token, groups, meta, H, hstride, y_perm, s)
                   : launch_t<BF16, false>(L, x, T, perm_token, groups, meta, H, hstride, y_perm, s);
    return oai ? launch_t<F32, true>(L, x, T, perm_token, groups, meta, H, hstride, y_perm, s)
               : launch_t<F32, false>(L, x, T, perm_token, groups, meta, H, hstride, y_perm, s);
}

}  // namespace smoe

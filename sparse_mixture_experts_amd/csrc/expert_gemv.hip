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
#include "gemv_items.h"

namespace smoe {
namespace {

// Group handled by grid row y.  With a shared expert (always the last group, and the
// one with the most rows) grid row 0 takes it, so its longer work starts first.
__device__ __forceinline__ int group_of_row(int y, int n_groups, bool has_shared) {
    return has_shared ? (y == 0 ? n_groups - 1 : y - 1) : y;
}

template <int KB, typename TT, bool OAI, bool RESIDENT>
__global__ __launch_bounds__(256) void expert_up_gemv_kernel(GemvUp a, const PlanMeta* meta_p) {
    const PlanMeta meta = *meta_p;
    if ((int)blockIdx.y >= meta.n_groups) return;
    const Group g = a.groups[group_of_row(blockIdx.y, meta.n_groups, a.ffs > 0)];
    const int ffg = g.e < 0 ? a.ffs : a.ff;
    const int f0 = (blockIdx.x * 4 + threadIdx.x / kWave) * 2;
    if (f0 < ffg) up_item<KB, TT, OAI, RESIDENT>(a, g, f0);
}

template <int KB, typename TT, bool OAI, bool RESIDENT>
__global__ __launch_bounds__(256) void expert_down_gemv_kernel(GemvDown a, const PlanMeta* meta_p) {
    const PlanMeta meta = *meta_p;
    if ((int)blockIdx.y >= meta.n_groups) return;
    const Group g = a.groups[group_of_row(blockIdx.y, meta.n_groups, a.ffs > 0)];
    const int i0 = (blockIdx.x * 4 + threadIdx.x / kWave) * 4;
    if (i0 < a.d) down_item<KB, TT, OAI, RESIDENT>(a, g, i0);
}

template <typename TT, bool OAI>
hipError_t launch_t(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                    const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                    hipStream_t s) {
    const bool shared = L.shared_ff > 0;
    const int gmax = max_groups(L.n_expert, T, L.k, shared);
    GemvUp u{x, perm_token, groups, L.w_gate, L.w_up, L.w_gate_up, L.b_gate_up,
             L.ws_gate, L.ws_up, H, hstride, T, L.d, L.ff, L.shared_ff, L.oai_alpha, L.oai_limit};
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    dim3 gu((ffmax + 7) / 8, gmax);
    const bool up_res = chunks(L.d, TT::VEC) <= 8;
    switch (pick_kb(L.d, TT::VEC)) {
#define SMOE_UP_CASE(KB)                                                                      \
    case KB:                                                                                  \
        if (up_res) expert_up_gemv_kernel<KB, TT, OAI, true><<<gu, 256, 0, s>>>(u, meta);           \
        else expert_up_gemv_kernel<KB, TT, OAI, false><<<gu, 256, 0, s>>>(u, meta);                 \
        break;
        SMOE_UP_CASE(1)
        SMOE_UP_CASE(2)
        SMOE_UP_CASE(4)
        SMOE_UP_CASE(8)
#undef SMOE_UP_CASE
    }
    GemvDown dn{H, groups, L.w_down, L.b_down, L.ws_down, y_perm, hstride, L.d, L.ff, L.shared_ff};
    dim3 gd((L.d + 15) / 16, gmax);
    const bool dn_res = chunks(ffmax, TT::VEC) <= 8;
    switch (pick_kb(ffmax, TT::VEC)) {
#define SMOE_DOWN_CASE(KB)                                                                    \
    case KB:                                                                                  \
        if (dn_res) expert_down_gemv_kernel<KB, TT, OAI, true><<<gd, 256, 0, s>>>(dn, meta);        \
        else expert_down_gemv_kernel<KB, TT, OAI, false><<<gd, 256, 0, s>>>(dn, meta);              \
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

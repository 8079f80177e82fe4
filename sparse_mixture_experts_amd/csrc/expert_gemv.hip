// Expert FFNs as HBM-streaming GEMVs over the active groups only (the decode path).
//
// "Qwen3.5-MoE Model Implementation", MoE routing: each routed expert is a SwiGLU,
// silu(gate . x) * (up . x) then down; the shared expert is one more SwiGLU over every
// token.  "Phase 19: MoE - gpt-oss-20b", Experts: fused interleaved gate_up with bias,
// clamps, (up + 1) * gate * sigmoid(alpha * gate), down with bias.  The group list is
// the union of experts the batch selected ("Engine", Address tables): only their
// weights are read, each once per block of up to 4 routed rows.
//
// Kernel 1 (up): a wave owns 2 hidden units of one group: it streams their gate
// and up weight rows (or the interleaved gate_up rows) and dots them with the group's
// rows of x, then applies the activation and writes H[row, f..] in fp32.
// Kernel 2 (down): a wave owns up to 16 output dims of one group: it streams those rows
// of W_d and dots them with the group's rows of H, writing Y_perm[row, i..].
// Grids are sized for the largest possible number of groups; blocks beyond the
// device-side group count return at once, so no host synchronisation is needed.
#include "gemv_items.h"

namespace smoe {
namespace {

template <int KB, typename TT, bool OAI, bool RESIDENT, int U, bool EXACT>
__global__ __launch_bounds__(256) void expert_up_gemv_kernel(GemvUp a, const PlanMeta* meta) {
    Group g;
    if (!gemv_group(a.groups, meta, a.ffs > 0, a.T, a.tk, g)) return;
    const int ffg = g.e < 0 ? a.ffs : a.ff;
    const int f0 = (blockIdx.x * 4 + wave_id()) * U;
    if (f0 < ffg) up_item<KB, TT, OAI, RESIDENT, U, EXACT>(a, g, f0);
}

template <int KB, typename TT, bool OAI, bool RESIDENT, int NR, bool EXACT>
__global__ __launch_bounds__(256) void expert_down_gemv_kernel(GemvDown a, const PlanMeta* meta) {
    Group g;
    if (!gemv_group(a.groups, meta, a.ffs > 0, a.T, a.tk, g)) return;
    const int i0 = (blockIdx.x * 4 + wave_id()) * NR;
    if (i0 < a.d) down_item<KB, TT, OAI, RESIDENT, NR, down_step_rows<NR>(), EXACT>(a, g, i0);
}

template <typename TT, bool OAI>
hipError_t launch_t(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                    const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                    hipStream_t s) {
    const bool shared = L.shared_ff > 0;
    const int gmax = max_groups(L.n_expert, T, L.k, shared);
    GemvUp u{x, perm_token, groups, L.w_gate, L.w_up, L.w_gate_up, L.b_gate_up,
             L.ws_gate, L.ws_up, H, hstride, T, T * L.k, L.d, L.ff, L.shared_ff, L.oai_alpha, L.oai_limit};
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    const bool up_res = chunks(L.d, TT::VEC) <= 8;
    const dim3 gu((ffmax + 4 * kUpUnits - 1) / (4 * kUpUnits), gmax);
    // Rows longer than one 8-chunk batch stream in batches of 4 chunks per lane.
    switch (up_res ? pick_kb(L.d, TT::VEC) : 4) {
#define SMOE_UP_LAUNCH(KB, RES, EX) \
    expert_up_gemv_kernel<KB, TT, OAI, RES, kUpUnits, EX><<<gu, 256, 0, s>>>(u, meta)
#define SMOE_UP_CASE(KB)                                                                       \
    case KB:                                                                                   \
        if (exact_k(L.d, TT::VEC, KB)) {                                                       \
            if (up_res) SMOE_UP_LAUNCH(KB, true, true);                                        \
            else SMOE_UP_LAUNCH(KB, false, true);                                              \
        } else {                                                                               \
            if (up_res) SMOE_UP_LAUNCH(KB, true, false);                                       \
            else SMOE_UP_LAUNCH(KB, false, false);                                             \
        }                                                                                      \
        break;
        SMOE_UP_CASE(1)
        SMOE_UP_CASE(2)
        SMOE_UP_CASE(4)
        SMOE_UP_CASE(8)
#undef SMOE_UP_CASE
#undef SMOE_UP_LAUNCH
    }
    GemvDown dn{H, groups, L.w_down, L.b_down, L.ws_down, y_perm, hstride, T, T * L.k, L.d, L.ff, L.shared_ff};
    const bool dn_res = chunks(ffmax, TT::VEC) <= 8;
    // Fewer than 64 possible groups (T*k + shared below 64 rows): 4 rows per wave, for
    // more waves in flight.
    const bool wide = gmax >= 64;
    // The down K axis is ff for routed experts and shared_ff for the shared one: exact
    // only when both are.
    const auto dn_exact = [&](int kb) {
        return exact_k(L.ff, TT::VEC, kb) && (L.shared_ff == 0 || exact_k(L.shared_ff, TT::VEC, kb));
    };
    switch (dn_res ? pick_kb(ffmax, TT::VEC) : 4) {
#define SMOE_DOWN_LAUNCH(KB, NR, RES, EX)                                                      \
    expert_down_gemv_kernel<KB, TT, OAI, RES, NR, EX>                                          \
        <<<dim3((L.d + 4 * (NR) - 1) / (4 * (NR)), gmax), 256, 0, s>>>(dn, meta)
#define SMOE_DOWN_NR(KB, NR)                                                                   \
    if (dn_exact(KB)) {                                                                        \
        if (dn_res) SMOE_DOWN_LAUNCH(KB, NR, true, true);                                      \
        else SMOE_DOWN_LAUNCH(KB, NR, false, true);                                            \
    } else {                                                                                   \
        if (dn_res) SMOE_DOWN_LAUNCH(KB, NR, true, false);                                     \
        else SMOE_DOWN_LAUNCH(KB, NR, false, false);                                           \
    }
#define SMOE_DOWN_CASE(KB)                                                                     \
    case KB:                                                                                   \
        if (wide) {                                                                            \
            SMOE_DOWN_NR(KB, down_rows_wide<KB>())                                             \
        } else {                                                                               \
            SMOE_DOWN_NR(KB, 4)                                                                \
        }                                                                                      \
        break;
        SMOE_DOWN_CASE(1)
        SMOE_DOWN_CASE(2)
        SMOE_DOWN_CASE(4)
        SMOE_DOWN_CASE(8)
#undef SMOE_DOWN_CASE
#undef SMOE_DOWN_NR
#undef SMOE_DOWN_LAUNCH
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

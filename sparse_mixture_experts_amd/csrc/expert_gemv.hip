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
#include "route_dev.h"

namespace smoe {
namespace {

// NT: group rows per step (1 for one token: every group then has one row).  PLAN: the
// wave finds its group from the expert offsets and the kernel writes the list for the down
// kernel (used for one token, where a separate planning launch costs more than the scan).
// The decode-batch form (two rows per step, resident weight rows of at most 4 chunks per
// lane, plain SwiGLU) fits 128 VGPRs without spilling when asked to, i.e. four waves per
// SIMD instead of three (130 registers unconstrained): a third more weight bytes in flight
// per CU.  The other forms would spill and keep the compiler's choice.
template <int KB, bool OAI, bool RESIDENT, bool EXACT, int NT>
constexpr int up_gemv_min_blocks() { return NT == 2 && !OAI && RESIDENT && EXACT && KB <= 4 ? 4 : 1; }

template <int KB, typename TT, bool OAI, bool RESIDENT, int U, bool EXACT, int NT, bool PLAN = false>
__global__ __launch_bounds__(256, (up_gemv_min_blocks<KB, OAI, RESIDENT, EXACT, NT>())) void expert_up_gemv_kernel(
    GemvUp a, const PlanMeta* meta, GemvPlan plan) {
    Group g;
    if constexpr (PLAN) {
        if (!plan_group(plan, a.ffs > 0, a.T, a.tk, g)) return;
    } else {
        if (!gemv_group(a.groups, meta, a.ffs > 0, a.T, a.tk, a.sh_rows, g)) return;
    }
    const int ffg = g.e < 0 ? a.ffs : a.ff;
    const int f0 = (blockIdx.x * 4 + wave_id()) * U;
    if (f0 < ffg) up_item<KB, TT, OAI, RESIDENT, U, EXACT, NT>(a, g, f0);
}

template <int KB, typename TT, bool OAI, bool RESIDENT, int NR, bool EXACT, int NT>
__global__ __launch_bounds__(256) void expert_down_gemv_kernel(GemvDown a, const PlanMeta* meta) {
    Group g;
    if (!gemv_group(a.groups, meta, a.ffs > 0, a.T, a.tk, a.sh_rows, g)) return;
    const int i0 = (blockIdx.x * 4 + wave_id()) * NR;
    if (i0 < a.d) down_item<KB, TT, OAI, RESIDENT, NR, NT, EXACT>(a, g, i0);
}

// One token: routing and the up projection in one kernel.  With shared_row, grid row 0
// is the shared expert, hidden row k, and starts streaming at once (without it, the
// shared expert's up GEMV ran in the router launch, or there is none); grid row y of a
// pick j = y - 1 (or y) runs the token's top-k on every wave (the same wave top-k as the
// routing kernels) and takes its j-th pick, hidden row j.  Block 0 of each pick row
// records the pick (idx[j], w[j]) for the down kernel.  (One top-k per block, handed to
// the other waves through LDS, measured no faster: the waves wait for the logits either
// way, and the top-k's arithmetic is not what the kernel waits on.)
template <int KB, typename TT, bool OAI, bool RESIDENT, int U, bool EXACT>
__global__ __launch_bounds__(256) void token1_up_kernel(GemvUp a, const float* __restrict__ logits, int E,
                                                        int k, int mode, float scale, int32_t* __restrict__ idx,
                                                        float* __restrict__ w, int shared_row) {
    const bool has_shared = a.ffs > 0 && shared_row;
    const int y = blockIdx.y;
    const int f0 = (blockIdx.x * 4 + wave_id()) * U;
    Group g;
    if (has_shared && y == 0) {
        g = Group{-1, k, 1, 0};
    } else {
        if (f0 >= a.ff) return;  // never block 0's first wave, which records the pick
        const int j = has_shared ? y - 1 : y;
        int my_i;
        float my_w;
        topk_wave(logits, E, k, mode, scale, &my_i, &my_w);
        if (blockIdx.x == 0 && wave_id() == 0 && lane_id() == j) {
            idx[j] = my_i;
            w[j] = my_w;
        }
        const int e = __builtin_amdgcn_readlane(my_i, j);
        g = Group{min(max(e, 0), E - 1), j, 1, 0};
    }
    const int ffg = g.e < 0 ? a.ffs : a.ff;
    // Every group holds the one token: one row per step.
    if (f0 < ffg) up_item<KB, TT, OAI, RESIDENT, U, EXACT, 1>(a, g, f0);
}

// One token with a shared expert: the router rows and the shared expert's up GEMV in one
// launch (the shared expert does not depend on the routing, so its weights stream while
// the router's do).  Blocks 0 .. n_sh-1 (a multiple of 8) run the shared expert's gate and
// up rows, hidden row k; block n_sh + b runs router row group b as router_gemv_kernel does
// for one token (rows 0..E-1 experts, row E the shared gate; row group b on XCD b % 8,
// which n_sh being a multiple of 8 keeps).
template <int KB, bool EXACT>
__global__ __launch_bounds__(256) void token1_router_shared_kernel(GemvUp a, const uint16_t* __restrict__ w_router,
                                                                   const float* __restrict__ b_router,
                                                                   const uint16_t* __restrict__ w_sg, int E,
                                                                   int n_sh, float* __restrict__ logits) {
    if ((int)blockIdx.x < n_sh) {
        const int f0 = (blockIdx.x * 4 + wave_id()) * kUpUnits;
        if (f0 < a.ffs) up_item<KB, BF16, false, true, kUpUnits, EXACT, 1>(a, Group{-1, a.tk, 1, 0}, f0);
        return;
    }
    const int row0 = (blockIdx.x - n_sh) * 4 + wave_id();
    if (row0 > E) return;
    router_rows_wave<KB, BF16, 1>(static_cast<const uint16_t*>(a.x), w_router, b_router, w_sg, 1, a.d, E, E + 1,
                                  row0, 0, 1, logits, E + 1);
}

// A few tokens: the down projection of every pick and of the shared expert, and the
// weighted combine, in one kernel.  Block (b, t) owns output dims i0 = b*NR .. i0+NR-1 of
// token t.  Wave j < k takes the token's j-th pick (expert idx[t*k+j], weight w[t*k+j],
// hidden row perm_inv[t*k+j], or row j for a single token without perm_inv); wave k (when
// there is a shared expert) takes hidden row T*k + t with weight sigmoid(gate[t]).
// Each wave leaves its NR dot products (+ the down bias) in LDS; the first NR threads then
// sum them in the combine's fixed order, picks 0..k-1 and then the shared expert: the
// separate down GEMV and combine compute the same sums (up to the order of the cross-lane
// reduction of each dot product).
constexpr int kToken1MaxWaves = 16;
constexpr int kToken1Rows = 4;

template <int KB, typename TT, bool OAI, int NR, bool EXACT>
__global__ __launch_bounds__(kToken1MaxWaves * kWave) void token1_down_combine_kernel(
    GemvDown a, const int32_t* __restrict__ idx, const float* __restrict__ w,
    const int32_t* __restrict__ perm_inv, const float* __restrict__ shared_gate, int gate_ld, int E, int k,
    const typename TT::storage* __restrict__ residual, typename TT::storage* __restrict__ y) {
    using S = typename TT::storage;
    __shared__ float part[kToken1MaxWaves][NR];
    __shared__ float wts[kToken1MaxWaves];
    const int j = wave_id(), lane = lane_id();
    const bool shared = j >= k;
    const int i0 = blockIdx.x * NR, t = blockIdx.y;
    int e = 0, row = a.tk + t;
    float weight;
    if (shared) {
        weight = 1.0f / (1.0f + expf(-shared_gate[(size_t)t * gate_ld]));
    } else {
        // A pick without a valid hidden row contributes nothing (its weight is zero).
        const int p = t * k + j;
        const int ei = idx[p], r = perm_inv ? perm_inv[p] : j;
        const bool ok = ei >= 0 && ei < E && r >= 0 && r < a.tk;
        e = ok ? ei : 0;
        row = ok ? r : 0;
        weight = ok ? w[p] : 0.0f;
    }
    const int K = shared ? a.ffs : a.ff;
    const S* base = shared ? static_cast<const S*>(a.ws_down) : static_cast<const S*>(a.w_down) + (size_t)e * a.d * K;
    const S* wr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) wr[r] = base + (size_t)min(i0 + r, a.d - 1) * K;
    const S* const (&wrc)[NR] = wr;
    const float* ar[1] = {a.H + (size_t)row * a.hstride};
    const float* const (&arc)[1] = ar;
    float acc[NR][1] = {};
    rows_dot<NR, 1, KB, TT, F32, true, EXACT>(wrc, arc, 1, K, acc);
    float v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = acc[r][0];
    // After the reduction lane l holds row l >> SH.
    constexpr int SH = 6 - ilog2(NR);
    const float sum = wave_reduce_scatter<NR>(v);
    const int my_r = lane >> SH;
    float bias = 0.0f;
    if (OAI && !shared && a.b_down && i0 + my_r < a.d) {
        const S* b = static_cast<const S*>(a.b_down) + (size_t)e * a.d + i0 + my_r;
        if constexpr (sizeof(S) == 2) bias = bf16_to_f32(*b);
        else bias = *b;
    }
    if ((lane & ((1 << SH) - 1)) == 0) part[j][my_r] = sum + bias;
    if (lane == 0) wts[j] = weight;
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < NR && i0 + tid < a.d) {
        const int nw = blockDim.x / kWave;
        float o = 0.0f;
        for (int jj = 0; jj < nw; ++jj) o = fmaf(wts[jj], part[jj][tid], o);
        const size_t at = (size_t)t * a.d + i0 + tid;
        if (residual) {  // read before y is written: y may alias it
            if constexpr (sizeof(S) == 2) o += bf16_to_f32(residual[at]);
            else o += residual[at];
        }
        if constexpr (sizeof(S) == 2) y[at] = f32_to_bf16(o);
        else y[at] = o;
    }
}

// shared_only: only the shared expert's grid rows, for layers whose routed experts run on
// other kernels; its rows are then cut into chunks of kSharedRows rows (one grid row
// each), so that the whole expert is not one grid row's serial loop over T tokens.
constexpr int kSharedRows = 16;

template <typename TT, bool OAI>
hipError_t launch_up_t(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                       const Group* groups, const PlanMeta* meta, float* H, int hstride, const GemvPlan& plan,
                       hipStream_t s, bool shared_only = false) {
    const bool shared = L.shared_ff > 0;
    const int sh_rows = shared_only ? kSharedRows : 0;
    const int gmax = (shared_only ? 0 : max_groups(L.n_expert, T, L.k, false)) +
                     (!shared ? 0 : shared_only ? (T + kSharedRows - 1) / kSharedRows : 1);
    GemvUp u{x, perm_token, groups, L.w_gate, L.w_up, L.w_gate_up, L.b_gate_up,
             L.ws_gate, L.ws_up, H, hstride, T, T * L.k, L.d, L.ff, L.shared_ff, L.oai_alpha, L.oai_limit,
             sh_rows};
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    const bool up_res = chunks(L.d, TT::VEC) <= 8;
    // Rows longer than one 8-chunk batch stream in batches of 4 chunks per lane.  One
    // token: one row per step, and one hidden unit per wave for rows of 8 chunks per lane
    // (the resident weights are used once, so fewer registers buy more waves).  Decode
    // batches (groups of a row or two): two rows per step, which measured faster than
    // four at 8 and 64 tokens (fewer registers, no duplicated rows); larger batches four.
    const int kb = up_res ? pick_kb(L.d, TT::VEC) : 4;
    const bool one = T == 1;
    if (plan.offsets && !one) return hipErrorInvalidValue;  // the in-kernel list is for one token
    const int units = one && kb == 8 ? 1 : kUpUnits;
    const dim3 gu((ffmax + 4 * units - 1) / (4 * units), gmax);
    switch (kb) {
#define SMOE_UP_LAUNCH(KB, RES, EX)                                                            \
    do {                                                                                       \
        if (one && plan.offsets)                                                               \
            expert_up_gemv_kernel<KB, TT, OAI, RES, KB == 8 ? 1 : kUpUnits, EX, 1, true>       \
                <<<gu, 256, 0, s>>>(u, meta, plan);                                            \
        else if (one)                                                                          \
            expert_up_gemv_kernel<KB, TT, OAI, RES, KB == 8 ? 1 : kUpUnits, EX, 1>             \
                <<<gu, 256, 0, s>>>(u, meta, plan);                                            \
        else if (T <= 64)                                                                      \
            expert_up_gemv_kernel<KB, TT, OAI, RES, kUpUnits, EX, 2><<<gu, 256, 0, s>>>(u, meta, plan); \
        else                                                                                   \
            expert_up_gemv_kernel<KB, TT, OAI, RES, kUpUnits, EX, kNT><<<gu, 256, 0, s>>>(u, meta, plan); \
    } while (0)
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
        SMOE_UP_CASE(6)
        SMOE_UP_CASE(8)
        default:
            return hipErrorInvalidValue;
#undef SMOE_UP_CASE
#undef SMOE_UP_LAUNCH
    }
    return hipGetLastError();
}

template <typename TT, bool OAI>
hipError_t launch_down_t(const moe_layer& L, int T, const Group* groups, const PlanMeta* meta, const float* H,
                         int hstride, float* y_perm, hipStream_t s, bool shared_only = false) {
    const bool shared = L.shared_ff > 0;
    const int sh_rows = shared_only ? kSharedRows : 0;
    const int gmax = (shared_only ? 0 : max_groups(L.n_expert, T, L.k, false)) +
                     (!shared ? 0 : shared_only ? (T + kSharedRows - 1) / kSharedRows : 1);
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    GemvDown dn{H, groups, L.w_down, L.b_down, L.ws_down, y_perm, hstride, T, T * L.k, L.d, L.ff, L.shared_ff,
                sh_rows};
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
    do {                                                                                       \
        const dim3 gd((L.d + 4 * (NR) - 1) / (4 * (NR)), gmax);                               \
        if (T == 1)                                                                            \
            expert_down_gemv_kernel<KB, TT, OAI, RES, NR, EX, 1><<<gd, 256, 0, s>>>(dn, meta);   \
        else                                                                                   \
            expert_down_gemv_kernel<KB, TT, OAI, RES, NR, EX, down_step_rows<NR>()>            \
                <<<gd, 256, 0, s>>>(dn, meta);                                                 \
    } while (0)
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
        SMOE_DOWN_CASE(6)
        SMOE_DOWN_CASE(8)
        default:
            return hipErrorInvalidValue;
#undef SMOE_DOWN_CASE
#undef SMOE_DOWN_NR
#undef SMOE_DOWN_LAUNCH
    }
    return hipGetLastError();
}


template <typename TT, bool OAI>
hipError_t launch_token1_up_t(const moe_layer& L, const void* x, const float* logits, int32_t* idx, float* w,
                              float* H, int hstride, bool shared_done, hipStream_t s) {
    const bool shared = L.shared_ff > 0 && !shared_done;
    GemvUp u{x, nullptr, nullptr, L.w_gate, L.w_up, L.w_gate_up, L.b_gate_up,
             L.ws_gate, L.ws_up, H, hstride, 1, L.k, L.d, L.ff, L.shared_ff, L.oai_alpha, L.oai_limit};
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    const bool up_res = chunks(L.d, TT::VEC) <= 8;
    // One token gives the resident weights no reuse: rows of 8 chunks per lane take one
    // hidden unit per wave (64 weight registers) for more waves in flight.
    const int kb = up_res ? pick_kb(L.d, TT::VEC) : 4;
    const int units = kb == 8 ? 1 : kUpUnits;
    const dim3 gu((ffmax + 4 * units - 1) / (4 * units), L.k + (shared ? 1 : 0));
    switch (kb) {
#define SMOE_UP_LAUNCH(KB, RES, EX)                                                              \
    token1_up_kernel<KB, TT, OAI, RES, KB == 8 ? 1 : kUpUnits, EX>                               \
        <<<gu, 256, 0, s>>>(u, logits, L.n_expert, L.k, L.route, L.route_scale, idx, w, shared ? 1 : 0)
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
        SMOE_UP_CASE(6)
        SMOE_UP_CASE(8)
        default:
            return hipErrorInvalidValue;
#undef SMOE_UP_CASE
#undef SMOE_UP_LAUNCH
    }
    return hipGetLastError();
}

template <typename TT, bool OAI>
hipError_t launch_token1_t(const moe_layer& L, int T, const float* H, int hstride, const int32_t* idx,
                           const float* w, const int32_t* perm_inv, const float* shared_gate, int gate_ld,
                           const void* residual, void* y, hipStream_t s) {
    const bool shared = L.shared_ff > 0;
    GemvDown dn{H, nullptr, L.w_down, L.b_down, L.ws_down, nullptr, hstride, T, T * L.k, L.d, L.ff, L.shared_ff};
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    const dim3 grid((L.d + kToken1Rows - 1) / kToken1Rows, T);
    const dim3 block((L.k + (shared ? 1 : 0)) * kWave);
    auto* yo = static_cast<typename TT::storage*>(y);
    const auto* ro = static_cast<const typename TT::storage*>(residual);
    const auto exact = [&](int kb) {
        return exact_k(L.ff, TT::VEC, kb) && (L.shared_ff == 0 || exact_k(L.shared_ff, TT::VEC, kb));
    };
    // Weight batches of at most 2 chunks per lane: the block may hold 16 waves, which
    // leaves 128 registers per lane.
    switch (min(pick_kb(ffmax, TT::VEC), 2)) {
#define SMOE_T1_CASE(KB)                                                                        \
    case KB:                                                                                    \
        if (exact(KB))                                                                          \
            token1_down_combine_kernel<KB, TT, OAI, kToken1Rows, true>                          \
                <<<grid, block, 0, s>>>(dn, idx, w, perm_inv, shared_gate, gate_ld, L.n_expert, L.k, ro, yo); \
        else                                                                                    \
            token1_down_combine_kernel<KB, TT, OAI, kToken1Rows, false>                         \
                <<<grid, block, 0, s>>>(dn, idx, w, perm_inv, shared_gate, gate_ld, L.n_expert, L.k, ro, yo); \
        break;
        SMOE_T1_CASE(1)
        SMOE_T1_CASE(2)
        default:
            return hipErrorInvalidValue;
#undef SMOE_T1_CASE
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gemv(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                              Group* groups, PlanMeta* meta, float* H, int hstride, float* y_perm,
                              const int32_t* plan_offsets, hipStream_t s) {
    if (L.expert_format == MOE_EXPERTS_MXFP4) {
        if (plan_offsets) return hipErrorInvalidValue;
        return launch_expert_gemv_mx(L, x, T, perm_token, groups, meta, H, hstride, y_perm, s);
    }
    if (L.expert_format == MOE_EXPERTS_Q4K) {
        if (plan_offsets) return hipErrorInvalidValue;
        return launch_expert_gemv_q4k(L, x, T, perm_token, groups, meta, H, hstride, y_perm, s);
    }
    const GemvPlan plan{plan_offsets, L.n_expert, groups, meta};
    const bool oai = L.act == MOE_ACT_SWIGLU_OAI;
    hipError_t e;
    if (L.dtype == MOE_BF16)
        e = oai ? launch_up_t<BF16, true>(L, x, T, perm_token, groups, meta, H, hstride, plan, s)
                : launch_up_t<BF16, false>(L, x, T, perm_token, groups, meta, H, hstride, plan, s);
    else
        e = oai ? launch_up_t<F32, true>(L, x, T, perm_token, groups, meta, H, hstride, plan, s)
                : launch_up_t<F32, false>(L, x, T, perm_token, groups, meta, H, hstride, plan, s);
    if (e != hipSuccess) return e;
    if (L.dtype == MOE_BF16)
        return oai ? launch_down_t<BF16, true>(L, T, groups, meta, H, hstride, y_perm, s)
                   : launch_down_t<BF16, false>(L, T, groups, meta, H, hstride, y_perm, s);
    return oai ? launch_down_t<F32, true>(L, T, groups, meta, H, hstride, y_perm, s)
               : launch_down_t<F32, false>(L, T, groups, meta, H, hstride, y_perm, s);
}

hipError_t launch_shared_gemv_up(const moe_layer& L, const void* x, int T, const Group* groups, const PlanMeta* meta,
                                 float* H, int hstride, hipStream_t s) {
    if (L.shared_ff <= 0 || L.dtype != MOE_BF16 || L.act != MOE_ACT_SWIGLU) return hipErrorInvalidValue;
    const GemvPlan plan{nullptr, L.n_expert, nullptr, nullptr};
    return launch_up_t<BF16, false>(L, x, T, nullptr, groups, meta, H, hstride, plan, s, true);
}

hipError_t launch_shared_gemv_down(const moe_layer& L, int T, const Group* groups, const PlanMeta* meta,
                                   const float* H, int hstride, float* y_perm, hipStream_t s) {
    if (L.shared_ff <= 0 || L.dtype != MOE_BF16 || L.act != MOE_ACT_SWIGLU) return hipErrorInvalidValue;
    return launch_down_t<BF16, false>(L, T, groups, meta, H, hstride, y_perm, s, true);
}

hipError_t launch_expert_up_gemv(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                 const Group* groups, const PlanMeta* meta, float* H, int hstride,
                                 hipStream_t s) {
    const GemvPlan plan{nullptr, L.n_expert, nullptr, nullptr};
    const bool oai = L.act == MOE_ACT_SWIGLU_OAI;
    if (L.dtype == MOE_BF16)
        return oai ? launch_up_t<BF16, true>(L, x, T, perm_token, groups, meta, H, hstride, plan, s)
                   : launch_up_t<BF16, false>(L, x, T, perm_token, groups, meta, H, hstride, plan, s);
    return oai ? launch_up_t<F32, true>(L, x, T, perm_token, groups, meta, H, hstride, plan, s)
               : launch_up_t<F32, false>(L, x, T, perm_token, groups, meta, H, hstride, plan, s);
}

hipError_t launch_token1_up(const moe_layer& L, const void* x, const float* logits, int32_t* idx, float* w,
                            float* H, int hstride, bool shared_done, hipStream_t s) {
    if (!token1_fits(L)) return hipErrorInvalidValue;
    const bool oai = L.act == MOE_ACT_SWIGLU_OAI;
    if (L.dtype == MOE_BF16)
        return oai ? launch_token1_up_t<BF16, true>(L, x, logits, idx, w, H, hstride, shared_done, s)
                   : launch_token1_up_t<BF16, false>(L, x, logits, idx, w, H, hstride, shared_done, s);
    return oai ? launch_token1_up_t<F32, true>(L, x, logits, idx, w, H, hstride, shared_done, s)
               : launch_token1_up_t<F32, false>(L, x, logits, idx, w, H, hstride, shared_done, s);
}

// The router and the shared expert in one launch: bf16 layers with a shared expert whose
// rows take one register batch of at most 4 chunks per lane (the router kernel's batch),
// dense routed experts on the one-token kernels or Q4_K routed experts (whose shared
// expert is bf16).
bool token1_router_shared_fits(const moe_layer& L) {
    const bool experts_ok = L.expert_format == MOE_EXPERTS_DENSE ? token1_fits(L)
                                                                  : L.expert_format == MOE_EXPERTS_Q4K;
    return experts_ok && L.shared_ff > 0 && L.dtype == MOE_BF16 && pick_kb(L.d, BF16::VEC) <= 4 &&
           chunks(L.d, BF16::VEC) <= 8;
}

hipError_t launch_token1_router_shared(const moe_layer& L, const void* x, float* logits, int ld, float* H,
                                       int hstride, hipStream_t s) {
    if (!token1_router_shared_fits(L) || ld != L.n_expert + 1) return hipErrorInvalidValue;
    GemvUp u{x, nullptr, nullptr, L.w_gate, L.w_up, L.w_gate_up, L.b_gate_up,
             L.ws_gate, L.ws_up, H, hstride, 1, L.k, L.d, L.ff, L.shared_ff, L.oai_alpha, L.oai_limit, 0};
    const int n_sh = 8 * ((L.shared_ff + 4 * kUpUnits * 8 - 1) / (4 * kUpUnits * 8));
    const int n_router = (L.n_expert + 1 + 3) / 4;
    const dim3 grid(n_sh + n_router);
    const auto* wr = static_cast<const uint16_t*>(L.w_router);
    const auto* wsg = static_cast<const uint16_t*>(L.ws_gate_inp);
    switch (pick_kb(L.d, BF16::VEC)) {
#define SMOE_RS_CASE(KB)                                                                                   \
    case KB:                                                                                              \
        if (exact_k(L.d, BF16::VEC, KB))                                                                  \
            token1_router_shared_kernel<KB, true><<<grid, 256, 0, s>>>(u, wr, L.b_router, wsg, L.n_expert, n_sh, logits); \
        else                                                                                              \
            token1_router_shared_kernel<KB, false><<<grid, 256, 0, s>>>(u, wr, L.b_router, wsg, L.n_expert, n_sh, logits); \
        break;
        SMOE_RS_CASE(1)
        SMOE_RS_CASE(2)
        SMOE_RS_CASE(4)
        default:
            return hipErrorInvalidValue;
#undef SMOE_RS_CASE
    }
    return hipGetLastError();
}

bool token1_fits(const moe_layer& L) {
    return L.expert_format == MOE_EXPERTS_DENSE && L.k + (L.shared_ff > 0 ? 1 : 0) <= kToken1MaxWaves;
}

hipError_t launch_token_down_combine(const moe_layer& L, int T, const float* H, int hstride, const int32_t* idx,
                                     const float* w, const int32_t* perm_inv, const float* shared_gate,
                                     int gate_ld, const void* residual, void* y, hipStream_t s) {
    if (!token1_fits(L) || T < 1 || (!perm_inv && T != 1)) return hipErrorInvalidValue;
    const bool oai = L.act == MOE_ACT_SWIGLU_OAI;
    if (L.dtype == MOE_BF16)
        return oai ? launch_token1_t<BF16, true>(L, T, H, hstride, idx, w, perm_inv, shared_gate, gate_ld, residual, y, s)
                   : launch_token1_t<BF16, false>(L, T, H, hstride, idx, w, perm_inv, shared_gate, gate_ld, residual, y, s);
    return oai ? launch_token1_t<F32, true>(L, T, H, hstride, idx, w, perm_inv, shared_gate, gate_ld, residual, y, s)
               : launch_token1_t<F32, false>(L, T, H, hstride, idx, w, perm_inv, shared_gate, gate_ld, residual, y, s);
}

}  // namespace smoe

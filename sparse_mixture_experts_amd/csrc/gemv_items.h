// Wave-level work items of the decode GEMVs (the kernels of expert_gemv.hip).
//
// "Qwen3.5-MoE Model Implementation", MoE routing: each routed expert is a SwiGLU,
// silu(gate . x) * (up . x) then down; the shared expert is one more SwiGLU over every
// token.  "Phase 19: MoE - gpt-oss-20b", Experts: fused interleaved gate_up with bias,
// clamps, (up + 1) * gate * sigmoid(alpha * gate), down with bias.
//
// up_item: a wave owns U hidden units f.. of one group: it streams their 2U weight rows
// (gate and up, or the interleaved gate_up rows) and dots them with the group's rows of
// x, then applies the activation and writes H[row, f..] in fp32.  down_item: a wave owns NR output dims i.. of one group: it streams those NR rows
// of W_d and dots them with the group's rows of H, writing Y_perm[row, i..].  Each
// 4-row step ends in one butterfly reduce-scatter of all the wave's partial sums.
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
    int hstride, T, tk, d, ff, ffs;  // tk = T * k routed rows
    float alpha, limit;
    int sh_rows;  // shared-expert rows per grid row (0: all T in one)
};

struct GemvDown {
    const float* H;
    const Group* groups;
    const void* w_down;   // [E, d, ff]
    const void* b_down;   // OAI [E, d] or null
    const void* ws_down;  // [d, ffs]
    float* y;
    int hstride, T, tk, d, ff, ffs;
    int sh_rows;  // shared-expert rows per grid row (0: all T in one)
};

// Grid rows of the shared expert: its T rows cut into chunks of sh_rows (0: one chunk).
__device__ __forceinline__ int shared_grid_rows(bool has_shared, int T, int sh_rows) {
    return !has_shared ? 0 : sh_rows > 0 ? (T + sh_rows - 1) / sh_rows : 1;
}

// Group of grid row blockIdx.y.  The shared expert (when there is one) is the last group
// of the list and always holds rows tk .. tk+T-1; the first grid rows take it, in chunks
// of sh_rows rows (built here without a load), so that its longer work starts first.  The
// grid rows after them take routed groups 0, 1, ...  The group entry and the group count
// are loaded together, before the count is checked (the list has room for every grid
// row), so the two reads cost one memory latency.  Returns false for rows past the count.
__device__ __forceinline__ bool gemv_group(const Group* groups, const PlanMeta* meta, bool has_shared,
                                           int T, int tk, int sh_rows, Group& g) {
    const int y = blockIdx.y;
    const int n_sh = shared_grid_rows(has_shared, T, sh_rows);
    const int gi = max(y - n_sh, 0);
    // Loaded on every row, so that nothing branches before the loads are issued; both
    // values are needed at the asm, so the compiler may not sink either load past a check.
    const Group cand = groups[gi];
    const int n_groups = meta->n_groups;
    asm volatile("" ::"s"(cand.e), "s"(cand.row0), "s"(cand.n), "s"(n_groups));
    if (y < n_sh) {
        const int r0 = sh_rows > 0 ? y * sh_rows : 0;
        g = Group{-1, tk + r0, sh_rows > 0 ? min(sh_rows, T - r0) : T, 0};
        return true;
    }
    if (gi >= n_groups - (has_shared ? 1 : 0)) return false;
    g = cand;
    return true;
}

// One wave: hidden units f0 .. f0+U-1 of group g (those below the group's hidden width),
// for every row of the group.  RESIDENT: the whole K axis fits one KB-chunk register
// batch, so the 2U weight rows are streamed once and every row is served from registers.
// The group list built inside the up kernel instead of by a separate planning launch
// (expert offsets from the caller): where the offsets are, and where the list and its
// count go for the down kernel.
struct GemvPlan {
    const int32_t* offsets;  // [E + 1], or null: the list is already built
    int E;
    Group* groups;
    PlanMeta* meta;
};

// Routed group gi of the expert offsets, found by one wave: the gi-th expert (ascending
// id) with rows, its rows clamped to 0 .. tk the same way as the planning kernel does.
// Lane l scans experts l*epl .. l*epl+epl-1 (epl = ceil(E / 64) <= 8); a wave prefix sum
// of the per-lane counts names the lane that holds group gi.  Returns the number of
// routed groups; g is set when gi is below it.  gi must be wave-uniform.
__device__ __forceinline__ int offsets_group(const int32_t* __restrict__ offsets, int E, int tk, int gi,
                                             Group& g) {
    const int epl = (E + kWave - 1) / kWave;
    const int e0 = lane_id() * epl;
    int o[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) o[i] = offsets[min(e0 + i, E)];
    const auto rows_of = [&](int i, int& r0, int& n) {
        r0 = min(max(o[i], 0), tk);
        n = (i < epl && e0 + i < E) ? min(max(o[i + 1] - r0, 0), tk - r0) : 0;
    };
    unsigned flags = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int r0, n;
        rows_of(i, r0, n);
        flags |= (n > 0 ? 1u : 0u) << i;
    }
    const int cnt = __popc(flags);
    const int incl = wave_inclusive_sum(cnt);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int excl = incl - cnt;
    const unsigned long long holder = __ballot(gi >= excl && gi < incl);
    if (holder == 0ull) return total;
    const int src = __ffsll((long long)holder) - 1;
    int t = gi - excl, pe = 0, pr = 0, pn = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int r0, n;
        rows_of(i, r0, n);
        if ((flags >> i) & 1u) {
            if (t == 0) {
                pe = e0 + i;
                pr = r0;
                pn = n;
            }
            --t;
        }
    }
    g = Group{__builtin_amdgcn_readlane(pe, src), __builtin_amdgcn_readlane(pr, src),
              __builtin_amdgcn_readlane(pn, src), 0};
    return total;
}

// gemv_group for a kernel that builds the list itself from p.offsets (same grid-row
// order).  Thread 0 of block 0 of each grid row records its routed group, and grid row 0
// the shared group and the count, for the down kernel that follows.
__device__ __forceinline__ bool plan_group(const GemvPlan& p, bool has_shared, int T, int tk, Group& g) {
    const int y = blockIdx.y;
    const int gi = has_shared ? max(y - 1, 0) : y;
    Group cand{0, 0, 0, 0};
    const int n_routed = offsets_group(p.offsets, p.E, tk, gi, cand);
    const bool shared_row = has_shared && y == 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (y == 0) {
            *p.meta = PlanMeta{n_routed + (has_shared ? 1 : 0), 0, 0, 0};
            if (has_shared) p.groups[n_routed] = Group{-1, tk, T, 0};
        }
        if (!shared_row && gi < n_routed) p.groups[gi] = cand;
    }
    if (shared_row) {
        g = Group{-1, tk, T, 0};
        return true;
    }
    if (gi >= n_routed) return false;
    g = cand;
    return true;
}

// v of the lane SHIFT lanes higher: a DPP row shift inside 16-lane rows (lanes whose
// source lies outside their row get 0; callers only use lanes whose source is inside),
// a bpermute for shifts of a whole row or more.
template <int SHIFT>
__device__ __forceinline__ float lanes_down(float v) {
    if constexpr (SHIFT < 16)
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + SHIFT, 0xF, 0xF, false));
    else
        return __shfl_down(v, SHIFT, kWave);
}

template <int KB, typename TT, bool OAI, bool RESIDENT, int U, bool EXACT, int NT = kNT>
__device__ __forceinline__ void up_item(const GemvUp& a, const Group& g, int f0) {
    using S = typename TT::storage;
    constexpr int NR = 2 * U;
    const bool shared = g.e < 0;
    const size_t d = a.d;
    const int ffg = shared ? a.ffs : a.ff;
    // The shared expert is always a plain SwiGLU, also in a layer of clamped experts.
    const bool oai = OAI && !shared;
    // Weight rows: gate f0.., then up f0.. (two matrices), or the interleaved gate_up rows
    // gate f0, up f0, gate f0+1, ... (one matrix).  Units past the width repeat the last.
    const S* wr[NR];
    if (oai) {
        const S* base = static_cast<const S*>(a.w_gate_up) + (size_t)g.e * 2 * a.ff * d;
#pragma unroll
        for (int r = 0; r < NR; ++r) wr[r] = base + (size_t)(2 * min(f0 + r / 2, ffg - 1) + (r & 1)) * d;
    } else {
        const S* gb = shared ? static_cast<const S*>(a.ws_gate) : static_cast<const S*>(a.w_gate) + (size_t)g.e * a.ff * d;
        const S* ub = shared ? static_cast<const S*>(a.ws_up) : static_cast<const S*>(a.w_up) + (size_t)g.e * a.ff * d;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wr[u] = gb + (size_t)min(f0 + u, ffg - 1) * d;
            wr[U + u] = ub + (size_t)min(f0 + u, ffg - 1) * d;
        }
    }
    const S* const (&wrc)[NR] = wr;
    // After the reduction lane l holds value (t * NR + r) = l >> SH: row t of the step,
    // weight row r = (l >> SH) % NR.  The up row matching a gate row sits U values on (two
    // matrices) or 1 value on (interleaved), (U << SH) or (1 << SH) lanes higher.
    constexpr int N = NR * NT;
    constexpr int SH = 6 - ilog2(N);
    const int lane = lane_id();
    const int my_t = (lane >> SH) / NR, my_r = (lane >> SH) % NR;
    const bool gate_lane = oai ? (my_r & 1) == 0 : my_r < U;
    const int my_f = oai ? my_r / 2 : my_r;  // unit offset of a gate lane
    const bool writer = gate_lane && (lane & ((1 << SH) - 1)) == 0 && f0 + my_f < ffg;
    float bg = 0.f, bu = 0.f;
    if (oai && writer) {
        const S* b = static_cast<const S*>(a.b_gate_up) + (size_t)g.e * 2 * a.ff + 2 * (f0 + my_f);
        if constexpr (sizeof(S) == 2) {
            bg = bf16_to_f32(b[0]);
            bu = bf16_to_f32(b[1]);
        } else {
            bg = b[0];
            bu = b[1];
        }
    }
    const S* x = static_cast<const S*>(a.x);
    // Token of row tb + (lane % NT), one vector load per step, issued before the weight
    // loads so that waiting for it does not wait for them.
    auto step_tokens = [&](int tb) {
        const int r = min(tb + (lane & (NT - 1)), g.n - 1);
        // Shared rows are the tokens in order (row tk + t is token t); with one token
        // every row is token 0.
        const int tok = shared ? g.row0 - a.tk + r : a.T == 1 ? r : a.perm_token[g.row0 + r];
        return min(max(tok, 0), a.T - 1);
    };
    auto step = [&](int tb, int tok_v, const uint4 (&wv)[RESIDENT ? KB : 1][NR]) {
        const int nt = min(NT, g.n - tb);
        const S* ar[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) ar[t] = x + (size_t)__builtin_amdgcn_readlane(tok_v, t) * d;
        const S* const (&arc)[NT] = ar;
        float acc[NR][NT] = {};
        if constexpr (RESIDENT) dot_w_batch<NR, NT, KB, TT, TT, EXACT>(wv, arc, nt, a.d, 0, acc);
        else rows_dot<NR, NT, KB, TT, TT, true, EXACT>(wrc, arc, nt, a.d, acc);
        float v[N];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) v[t * NR + r] = acc[r][t];
        const float sum = wave_reduce_scatter<N>(v);
        const float up_two = lanes_down<(U << SH)>(sum);
        const float up_one = lanes_down<(1 << SH)>(sum);
        float h;
        if (oai) {
            float gv = sum + bg;
            float uv = up_one + bu;
            gv = fminf(gv, a.limit);
            uv = fminf(fmaxf(uv, -a.limit), a.limit);
            h = (uv + 1.0f) * gv * sigmoidf_(a.alpha * gv);
        } else {
            h = sum * sigmoidf_(sum) * up_two;
        }
        if (writer && my_t < nt) a.H[(size_t)(g.row0 + tb + my_t) * a.hstride + f0 + my_f] = h;
    };
    // The first step runs outside the loop: straight-line code lets the compiler wait for
    // the token load alone (not the weights behind it) before the activation loads.
    const int tok0 = step_tokens(0);
    uint4 wv[RESIDENT ? KB : 1][NR];
    if constexpr (RESIDENT) load_w_batch<NR, KB, TT, true, EXACT>(wrc, a.d, 0, wv);
    __builtin_amdgcn_sched_barrier(0);  // the token's readlanes stay behind the weight loads
    step(0, tok0, wv);
    for (int tb = NT; tb < g.n; tb += NT) step(tb, step_tokens(tb), wv);
}

// Hidden units per up-projection wave.  Four units (8 weight rows, x re-read half as
// often) measured slower at 64 decode tokens than two: the larger register batch halves
// the waves in flight.
constexpr int kUpUnits = 2;

// One wave: output dims i0 .. i0+NR-1 of group g (those below d), for every row, NT
// rows of H per step.
template <int KB, typename TT, bool OAI, bool RESIDENT, int NR, int NT, bool EXACT>
__device__ __forceinline__ void down_item(const GemvDown& a, const Group& g, int i0) {
    using S = typename TT::storage;
    const bool shared = g.e < 0;
    const int K = shared ? a.ffs : a.ff;
    const S* base = shared ? static_cast<const S*>(a.ws_down) : static_cast<const S*>(a.w_down) + (size_t)g.e * a.d * K;
    const S* wr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) wr[r] = base + (size_t)min(i0 + r, a.d - 1) * K;
    const S* const (&wrc)[NR] = wr;
    // After the reduction lane l holds value (t * NR + r) = l >> SH.
    constexpr int N = NR * NT;
    constexpr int SH = 6 - ilog2(N);
    const int lane = lane_id();
    const int my_t = (lane >> SH) / NR, my_i = i0 + (lane >> SH) % NR;
    const bool writer = (lane & ((1 << SH) - 1)) == 0 && my_i < a.d;
    float bias = 0.f;
    if (OAI && !shared && a.b_down && my_i < a.d) {
        const S* b = static_cast<const S*>(a.b_down) + (size_t)g.e * a.d + my_i;
        if constexpr (sizeof(S) == 2) bias = bf16_to_f32(*b);
        else bias = *b;
    }
    uint4 wv[RESIDENT ? KB : 1][NR];
    if constexpr (RESIDENT) load_w_batch<NR, KB, TT, true, EXACT>(wrc, K, 0, wv);
    for (int tb = 0; tb < g.n; tb += NT) {
        const int nt = min(NT, g.n - tb);
        const float* ar[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) ar[t] = a.H + (size_t)(g.row0 + min(tb + t, g.n - 1)) * a.hstride;
        const float* const (&arc)[NT] = ar;
        float acc[NR][NT] = {};
        if constexpr (RESIDENT) dot_w_batch<NR, NT, KB, TT, F32, EXACT>(wv, arc, nt, K, 0, acc);
        else rows_dot<NR, NT, KB, TT, F32, true, EXACT>(wrc, arc, nt, K, acc);
        float v[N];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) v[t * NR + r] = acc[r][t];
        const float out = wave_reduce_scatter<N>(v) + bias;
        if (writer && my_t < nt) a.y[(size_t)(g.row0 + tb + my_t) * a.d + my_i] = out;
    }
}

// Output rows per down-projection wave for "wide" launches: 8 (a K axis of one or two
// register chunks per lane; 16 and 4 measured slower at 64 decode tokens), 4 for longer
// axes so that the weight batch stays at 64 registers or below.  Launches over very few
// groups use 4 rows per wave instead, for more waves in flight.
template <int KB>
constexpr int down_rows_wide() { return KB <= 2 ? 8 : 4; }

// H rows per down-projection step: 2 beside 8 or more weight rows (decode groups hold a
// row or two; fewer registers), else 4.
template <int NR>
constexpr int down_step_rows() { return NR >= 8 ? 2 : kNT; }

}  // namespace smoe

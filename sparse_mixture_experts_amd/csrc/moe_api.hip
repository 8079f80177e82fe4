// C ABI of libsmoe.so: argument checks, workspace layout, and the stream-ordered
// sequence of launches of each entry point.  Every check happens on the host before
// any HIP call, so a rejected call enqueues nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

namespace smoe {
namespace {

constexpr int kMaxExperts = 512;
constexpr int kMaxK = 32;
constexpr int32_t kMaxTokens = 1 << 22;
constexpr int kDecodeMaxT = 64;  // MOE_PATH_AUTO takes the grouped path above this T
// ... and at or below it when the expected rows per active expert reach this many: the
// GEMVs' per-row arithmetic then outgrows their weight stream, MFMA tiles do not.
constexpr double kGroupedMinRows = 4.0;
// Dense experts whose gate/up weights reach 16 MB take the grouped path from 2 expected rows
// per active expert: each expert's tiles then run long enough that streaming its weights once
// per N-tile beats once per row pair (Mixtral-shaped T=8 546 -> 435 us, gpt-oss-shaped T=16
// 274 -> 259 us; the Qwen-shaped layer's 4 MB experts at T=64 stay faster on the GEMVs).
constexpr double kGroupedMinRowsWide = 2.0;
constexpr double kWideExpertBytes = 16.0 * (1 << 20);
// Q4_K experts keep the GEMVs up to this many tokens while the expected rows per active expert
// stay below 8: the GEMVs decode each quant once per step, the grouped kernels expand every
// weight of a tile into LDS (Qwen-shaped: T=96 209 vs 260 us, T=128 244 vs 264 us; grouped
// faster from T=192, 304 vs 315 us).
constexpr int kDecodeMaxTQ4k = 128;
constexpr double kQ4kGroupedMinRows = 8.0;
// Split-K of the grouped down projection at decode-sized batches: at most this many K
// slices per tile, chosen to bring the expected down blocks up to two per CU (256 CUs).
constexpr int kMaxKSplit = 4;
constexpr double kTargetDownBlocks = 512.0;
constexpr int kTileM = kGroupTileM;  // M-tile size recorded in the group plan
// Largest batch whose down projection runs per token, fused with the combine.
constexpr int kTokenDownMaxT = 8;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte offsets of every scratch buffer inside the caller's workspace.
struct Layout {
    size_t logits, idx, w, sg, counts, base, offsets, perm_token, perm_inv, groups, meta, tiles,
        row_w, H, yperm, xn, partial;
    size_t total;
    int ld, hstride, rows;
};

Layout layout_for(const moe_layer& L, int T) {
    Layout o{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += round_up(bytes ? bytes : 1, 256);
        return at;
    };
    const bool shared = L.shared_ff > 0;
    const size_t tk = (size_t)T * L.k;
    const size_t n_chunks = ((size_t)T + kPermChunk - 1) / kPermChunk;
    o.ld = L.n_expert + (shared ? 1 : 0);
    o.hstride = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    o.rows = (int)(tk + (shared ? T : 0));
    o.logits = take((size_t)T * o.ld * 4);
    o.idx = take(tk * 4);
    o.w = take(tk * 4);
    o.sg = take((size_t)T * 4);
    o.counts = take(n_chunks * L.n_expert * 4);
    o.base = take((n_chunks + 1) * L.n_expert * 4);
    o.offsets = take(((size_t)L.n_expert + 1) * 4);
    o.perm_token = take(tk * 4);
    o.perm_inv = take(tk * 4);
    o.groups = take(((size_t)L.n_expert + 1) * sizeof(Group));
    o.meta = take(sizeof(PlanMeta));
    o.tiles = take((size_t)grouped_max_mtiles(L.n_expert, T, L.k, shared) * sizeof(TileDesc));
    o.row_w = take((size_t)o.rows * 4);
    // H: fp32 on the GEMV path, bf16 on the grouped path (same region).
    o.H = take((size_t)o.rows * o.hstride * 4);
    o.yperm = take((size_t)o.rows * L.d * 4);
    // Normalised rows of the layer shell, in the layer's dtype.
    o.xn = take((size_t)T * L.d * (L.dtype == MOE_BF16 ? 2 : 4));
    // fp32 planes of the split-K down projection (decode-sized bf16 batches only).
    const bool split_possible = T <= kDecodeMaxT && L.dtype == MOE_BF16;
    o.partial = take(split_possible ? (size_t)kMaxKSplit * o.rows * L.d * 4 : 0);
    o.total = off;
    return o;
}

template <typename P>
inline P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

moe_status check_layer(const moe_layer* L) {
    if (!L) return MOE_ERR_ARG;
    if (L->d <= 0 || L->n_expert <= 0 || L->ff <= 0 || L->k < 1 || L->k > L->n_expert ||
        L->shared_ff < 0)
        return MOE_ERR_ARG;
    if (L->dtype != MOE_F32 && L->dtype != MOE_BF16) return MOE_ERR_ARG;
    if (L->route != MOE_ROUTE_SOFTMAX_TOPK_RENORM && L->route != MOE_ROUTE_TOPK_SOFTMAX) return MOE_ERR_ARG;
    if (L->act != MOE_ACT_SWIGLU && L->act != MOE_ACT_SWIGLU_OAI) return MOE_ERR_ARG;
    if (L->path != MOE_PATH_AUTO && L->path != MOE_PATH_DECODE && L->path != MOE_PATH_GROUPED)
        return MOE_ERR_ARG;
    if (!isfinite(L->route_scale) || !isfinite(L->oai_alpha) || !isfinite(L->oai_limit))
        return MOE_ERR_ARG;
    if (!L->w_router || !L->w_down) return MOE_ERR_ARG;
    if (L->act == MOE_ACT_SWIGLU && (!L->w_gate || !L->w_up)) return MOE_ERR_ARG;
    // Expert biases belong to the clamped variant only; a plain SwiGLU layer that carried
    // one would see it on some kernel paths and not on others.
    if (L->act == MOE_ACT_SWIGLU && (L->b_gate_up || L->b_down)) return MOE_ERR_ARG;
    if (L->act == MOE_ACT_SWIGLU_OAI && (!L->w_gate_up || !L->b_gate_up)) return MOE_ERR_ARG;
    if (L->shared_ff > 0 && (!L->ws_gate || !L->ws_up || !L->ws_down || !L->ws_gate_inp))
        return MOE_ERR_ARG;
    if (L->d % 64 || L->ff % 64 || L->shared_ff % 64) return MOE_ERR_UNSUPPORTED;
    if (L->n_expert > kMaxExperts || L->k > kMaxK) return MOE_ERR_UNSUPPORTED;
    if (L->path == MOE_PATH_GROUPED && L->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (L->expert_format != MOE_EXPERTS_DENSE && L->expert_format != MOE_EXPERTS_MXFP4 &&
        L->expert_format != MOE_EXPERTS_Q4K)
        return MOE_ERR_ARG;
    if (L->reserved0 != 0) return MOE_ERR_ARG;
    if (L->grouped_pack && L->expert_format == MOE_EXPERTS_DENSE && L->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (!aligned(L->grouped_pack, 16)) return MOE_ERR_UNSUPPORTED;
    if (L->expert_format == MOE_EXPERTS_MXFP4) {
        if (!L->w_gate_up_scales || !L->w_down_scales) return MOE_ERR_ARG;
        if (L->dtype != MOE_BF16 || L->act != MOE_ACT_SWIGLU_OAI || L->shared_ff != 0 || !mx_fits(*L))
            return MOE_ERR_UNSUPPORTED;
    }
    if (L->expert_format == MOE_EXPERTS_Q4K) {
        if (L->w_gate_up_scales || L->w_down_scales) return MOE_ERR_ARG;
        if (L->dtype != MOE_BF16 || L->act != MOE_ACT_SWIGLU || !q4k_fits(*L)) return MOE_ERR_UNSUPPORTED;
    }
    const void* vec_ptrs[] = {L->w_router, L->w_gate, L->w_up, L->w_gate_up, L->w_down,
                              L->ws_gate, L->ws_up, L->ws_down, L->ws_gate_inp};
    for (const void* p : vec_ptrs)
        if (!aligned(p, 16)) return MOE_ERR_UNSUPPORTED;
    const size_t es = L->dtype == MOE_BF16 ? 2 : 4;
    if (!aligned(L->b_router, 4) || !aligned(L->b_gate_up, es) || !aligned(L->b_down, es))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_tokens(int32_t T) {
    if (T < 0) return MOE_ERR_ARG;
    if (T > kMaxTokens) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

inline moe_status status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

#define SMOE_TRY(expr)                          \
    do {                                        \
        hipError_t err_ = (expr);               \
        if (err_ != hipSuccess) return MOE_ERR_DEVICE; \
    } while (0)

// Expected number of distinct experts that T tokens select, k each, if every expert were
// equally likely: E * (1 - (1 - k/E)^T).
double expected_active(int E, int k, int T) { return E * (1.0 - pow(1.0 - (double)k / E, (double)T)); }

// The grouped MFMA path (bf16; dense or MXFP4 experts) or the decode GEMV path.
bool use_grouped(const moe_layer& L, int T) {
    if (L.dtype != MOE_BF16) return false;
    if (L.path == MOE_PATH_GROUPED) return true;
    if (L.path != MOE_PATH_AUTO) return false;
    const double rows = (double)T * L.k / expected_active(L.n_expert, L.k, T);
    if (T > kDecodeMaxT)
        return !(L.expert_format == MOE_EXPERTS_Q4K && T <= kDecodeMaxTQ4k && rows < kQ4kGroupedMinRows);
    const bool wide = L.expert_format == MOE_EXPERTS_DENSE && 2.0 * L.ff * L.d * 2 >= kWideExpertBytes;
    return rows >= (wide ? kGroupedMinRowsWide : kGroupedMinRows);
}

// Large bf16 batches compute the router logits on MFMA (experts only; top-k then forms
// the shared-gate input itself); otherwise the GEMV router fills every column.
// K slices per tile of the grouped down projection.  Up to 64 tokens a group holds at most
// 64 rows, so every active expert is one M-tile; with few of them (layers with few experts)
// the down grid would leave CUs idle.  The slices must be whole 32-wide K-steps of both the
// routed and the shared expert's K.
int down_ksplit(const moe_layer& L, int T) {
    if (T > kDecodeMaxT) return 1;
    const double tiles = expected_active(L.n_expert, L.k, T) + (L.shared_ff > 0 ? 1 : 0);
    const double blocks = tiles * ((L.d + 255) / 256);
    int s = (int)ceil(kTargetDownBlocks / blocks);
    s = s < kMaxKSplit ? s : kMaxKSplit;
    while (s > 1 && (L.ff % (32 * s) || (L.shared_ff > 0 && L.shared_ff % (32 * s)))) --s;
    return s > 1 ? s : 1;
}

bool router_on_mfma(const moe_layer& L, int T) { return use_grouped(L, T) && T > kPermChunk; }
bool router_leaves_shared_gate(const moe_layer& L, int T) {
    return router_on_mfma(L, T) && L.shared_ff > 0;
}
hipError_t run_router(const moe_layer& L, const void* x, int T, float* logits, int ld, hipStream_t s,
                      const RouterNorm* norm = nullptr) {
    if (norm) return launch_router_logits(L, x, T, logits, ld, s, norm);
    return router_on_mfma(L, T) ? launch_router_mfma(L, x, T, logits, ld, s)
                                : launch_router_logits(L, x, T, logits, ld, s);
}

// Expert FFNs over the grouped rows.  `planned`: the group list is already in the
// workspace (the fused decode routing kernel wrote it).  Grouped path: `row_w` non-null
// scales each row by its routing weight and `y_bf16` stores bf16 rows; the GEMV path
// always writes unweighted fp32 rows.
moe_status run_experts(const moe_layer& L, const void* x, int T, const int32_t* offsets,
                       const int32_t* perm_token, void* y_rows, const float* row_w, bool y_bf16,
                       void* ws, const Layout& o, bool planned, hipStream_t s) {
    Group* groups = at<Group>(ws, o.groups);
    PlanMeta* meta = at<PlanMeta>(ws, o.meta);
    TileDesc* tiles = at<TileDesc>(ws, o.tiles);
    const bool grouped = use_grouped(L, T);
    // One token on the dense GEMVs: the up kernel finds its groups from the offsets itself
    // (a planning launch costs more than that scan there; at more tokens the scan in front
    // of every wave's loads costs more than the launch).
    const bool plan_in_up = !planned && !grouped && T == 1 && L.expert_format == MOE_EXPERTS_DENSE;
    if (!planned && !plan_in_up)
        SMOE_TRY(launch_plan(offsets, L.n_expert, T, L.k, L.shared_ff > 0, kTileM, groups, meta,
                             tiles, s));
    if (grouped) {
        const int ksplit = down_ksplit(L, T);
        SMOE_TRY(launch_grouped_ffn(L, x, T, perm_token, groups, meta, tiles, at<uint16_t>(ws, o.H),
                                    o.hstride, row_w, y_rows, y_bf16, ksplit,
                                    ksplit > 1 ? at<float>(ws, o.partial) : nullptr, s));
    } else {
        SMOE_TRY(launch_expert_gemv(L, x, T, perm_token, groups, meta, at<float>(ws, o.H), o.hstride,
                                    static_cast<float*>(y_rows), plan_in_up ? offsets : nullptr, s));
    }
    return MOE_OK;
}

// The layer after the argument checks: route, group, expert FFNs, combine (plus
// residual[t] when it is non-null), reading x and writing y.  With `norm` the router
// reads residual (the shell's h), normalises it and writes the rows the experts read to
// x (= norm->xn).
moe_status forward_body(const moe_layer* L, const void* x, int32_t T, const void* residual, void* y, void* ws,
                        const Layout& o, hipStream_t s, const RouterNorm* norm = nullptr) {
    const bool shared = L->shared_ff > 0;
    float* logits = at<float>(ws, o.logits);
    int32_t* idx = at<int32_t>(ws, o.idx);
    float* w = at<float>(ws, o.w);
    float* sg = shared ? at<float>(ws, o.sg) : nullptr;
    int32_t* offsets = at<int32_t>(ws, o.offsets);
    int32_t* perm_token = at<int32_t>(ws, o.perm_token);
    int32_t* perm_inv = at<int32_t>(ws, o.perm_inv);
    const bool grouped = use_grouped(*L, T);
    // Grouped path: rows carry their routing weight and are stored in bf16.
    float* row_w = grouped ? at<float>(ws, o.row_w) : nullptr;
    void* y_rows = at<void>(ws, o.yperm);
    const bool dense = L->expert_format == MOE_EXPERTS_DENSE;
    const bool q4k_token = L->expert_format == MOE_EXPERTS_Q4K && !grouped && q4k_token_fits(*L);
    // One token with a shared expert: its up GEMV streams in the router launch.
    const bool router_shared = T == 1 && !grouped && (dense || q4k_token) && !norm && o.ld == L->n_expert + 1 &&
                               token1_router_shared_fits(*L);
    if (router_shared)
        SMOE_TRY(launch_token1_router_shared(*L, x, logits, o.ld, at<float>(ws, o.H), o.hstride, s));
    else
        SMOE_TRY(run_router(*L, norm ? residual : x, T, logits, o.ld, s, norm));
    if (T == 1 && !grouped && dense && token1_fits(*L)) {
        // One token: top-k inside the up GEMV, then the down GEMVs and the combine in one
        // kernel (no grouping: hidden row j holds pick j).
        SMOE_TRY(launch_token1_up(*L, x, logits, idx, w, at<float>(ws, o.H), o.hstride, router_shared, s));
        SMOE_TRY(launch_token_down_combine(*L, 1, at<float>(ws, o.H), o.hstride, idx, w, nullptr,
                                           shared ? logits + L->n_expert : nullptr, o.ld, residual, y, s));
        return MOE_OK;
    }
    if (T == 1 && q4k_token && (router_shared || !shared)) {
        // The same three launches over Q4_K routed experts (the shared expert's up ran in
        // the router launch).
        SMOE_TRY(launch_token1_up_q4k(*L, x, logits, idx, w, at<float>(ws, o.H), o.hstride, s));
        SMOE_TRY(launch_token_down_combine_q4k(*L, 1, at<float>(ws, o.H), o.hstride, idx, w, nullptr,
                                               shared ? logits + L->n_expert : nullptr, o.ld, residual, y, s));
        return MOE_OK;
    }
    const bool mxfp4 = L->expert_format == MOE_EXPERTS_MXFP4;
    if (T == 1 && !grouped && mxfp4 && token1_mx_fits(*L)) {
        // The same three launches over MXFP4 expert weights.
        SMOE_TRY(launch_token1_up_mx(*L, x, logits, idx, w, at<float>(ws, o.H), o.hstride, s));
        SMOE_TRY(launch_token_down_combine_mx(*L, 1, at<float>(ws, o.H), o.hstride, idx, w, nullptr, residual, y, s));
        return MOE_OK;
    }
    const bool fused_route = T <= kPermChunk;
    if (fused_route) {
        SMOE_TRY(launch_decode_route(*L, logits, o.ld, T, idx, w, sg, offsets, perm_token, perm_inv,
                                     row_w, kTileM, at<Group>(ws, o.groups), at<PlanMeta>(ws, o.meta),
                                     at<TileDesc>(ws, o.tiles), s));
    } else {
        SMOE_TRY(launch_topk(*L, logits, o.ld, T, idx, w, sg, row_w,
                             router_leaves_shared_gate(*L, T) ? x : nullptr, s));
        SMOE_TRY(launch_permute(idx, T, L->k, L->n_expert, offsets, perm_token, perm_inv,
                                at<int32_t>(ws, o.counts), at<int32_t>(ws, o.base), w, row_w, s));
    }
    if (fused_route && !grouped && dense && T <= kTokenDownMaxT && token1_fits(*L)) {
        // A few tokens: up GEMV over the groups, then per token the down GEMVs of its picks
        // and the combine in one kernel.
        SMOE_TRY(launch_expert_up_gemv(*L, x, T, perm_token, at<Group>(ws, o.groups), at<PlanMeta>(ws, o.meta),
                                       at<float>(ws, o.H), o.hstride, s));
        SMOE_TRY(launch_token_down_combine(*L, T, at<float>(ws, o.H), o.hstride, idx, w, perm_inv, sg, 1, residual,
                                           y, s));
        return MOE_OK;
    }
    if (fused_route && q4k_token && T <= kTokenDownMaxT) {
        SMOE_TRY(launch_expert_up_gemv_q4k(*L, x, T, perm_token, at<Group>(ws, o.groups), at<PlanMeta>(ws, o.meta),
                                           at<float>(ws, o.H), o.hstride, s));
        SMOE_TRY(launch_token_down_combine_q4k(*L, T, at<float>(ws, o.H), o.hstride, idx, w, perm_inv, sg, 1,
                                               residual, y, s));
        return MOE_OK;
    }
    if (fused_route && !grouped && mxfp4 && T <= kTokenDownMaxT && token1_mx_fits(*L)) {
        SMOE_TRY(launch_expert_up_gemv_mx(*L, x, T, perm_token, at<Group>(ws, o.groups), at<PlanMeta>(ws, o.meta),
                                          at<float>(ws, o.H), o.hstride, s));
        SMOE_TRY(launch_token_down_combine_mx(*L, T, at<float>(ws, o.H), o.hstride, idx, w, perm_inv, residual, y, s));
        return MOE_OK;
    }
    const moe_status st = run_experts(*L, x, T, offsets, perm_token, y_rows, row_w, grouped, ws, o, fused_route, s);
    if (st != MOE_OK) return st;
    if (grouped)
        SMOE_TRY(launch_combine_sum(*L, static_cast<const uint16_t*>(y_rows), perm_inv, T, residual, y, s));
    else
        SMOE_TRY(launch_combine(*L, static_cast<const float*>(y_rows), perm_inv, w, sg, T, residual, y, s));
    return MOE_OK;
}

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" {

int32_t moe_abi_version(void) { return 4; }

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape, alignment or dtype/path combination";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_DEVICE: return "HIP launch failed";
        default: return "unknown status";
    }
}

moe_status moe_grouped_pack_size(const moe_layer* L, size_t* bytes) {
    const moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_ARG;
    if (L->expert_format == MOE_EXPERTS_MXFP4) *bytes = mx_pack_layout(*L).total;
    else if (L->expert_format == MOE_EXPERTS_Q4K) *bytes = q4k_pack_layout(*L).total;
    else if (L->dtype == MOE_BF16) *bytes = dense_pack_layout(*L).total;
    else return MOE_ERR_UNSUPPORTED;  // fp32 layers never take the grouped path
    return MOE_OK;
}

moe_status moe_grouped_pack(const moe_layer* L, void* dst, size_t bytes, void* stream) {
    size_t need = 0;
    const moe_status st = moe_grouped_pack_size(L, &need);
    if (st != MOE_OK) return st;
    if (!dst) return MOE_ERR_ARG;
    if (!aligned(dst, 16)) return MOE_ERR_UNSUPPORTED;
    if (bytes < need) return MOE_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = L->expert_format == MOE_EXPERTS_MXFP4 ? launch_mx_pack(*L, dst, s)
                         : L->expert_format == MOE_EXPERTS_Q4K ? launch_q4k_pack(*L, dst, s)
                                                                : launch_dense_pack(*L, dst, s);
    return status_of(e);
}

moe_status moe_workspace_size(const moe_layer* L, int32_t T, size_t* bytes) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if ((st = check_tokens(T)) != MOE_OK) return st;
    if (!bytes) return MOE_ERR_ARG;
    // The split-K planes exist only up to kDecodeMaxT tokens, so the layout of a smaller
    // batch can be larger: the size covers every batch of at most T tokens.
    const size_t own = layout_for(*L, T).total;
    const size_t small = layout_for(*L, T < kDecodeMaxT ? T : kDecodeMaxT).total;
    *bytes = own > small ? own : small;
    return MOE_OK;
}

moe_status moe_route(const moe_layer* L, const void* x, int32_t T, int32_t* topk_idx,
                     float* topk_w, float* shared_gate, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if ((st = check_tokens(T)) != MOE_OK) return st;
    if (shared_gate && L->shared_ff == 0) return MOE_ERR_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !topk_idx || !topk_w || !ws) return MOE_ERR_ARG;
    if (!aligned(x, 16)) return MOE_ERR_UNSUPPORTED;
    const Layout o = layout_for(*L, T);
    if (ws_bytes < o.total) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    float* logits = at<float>(ws, o.logits);
    SMOE_TRY(run_router(*L, x, T, logits, o.ld, s));
    SMOE_TRY(launch_topk(*L, logits, o.ld, T, topk_idx, topk_w, shared_gate, nullptr,
                         router_leaves_shared_gate(*L, T) ? x : nullptr, s));
    return MOE_OK;
}

moe_status moe_permute_workspace_size(int32_t T, int32_t k, int32_t E, size_t* bytes) {
    if (T < 0 || k < 1 || E < 1 || k > E || !bytes) return MOE_ERR_ARG;
    if (E > kMaxExperts || k > kMaxK || T > kMaxTokens) return MOE_ERR_UNSUPPORTED;
    const size_t n_chunks = ((size_t)T + kPermChunk - 1) / kPermChunk;
    *bytes = round_up(n_chunks * E * 4, 256) + round_up((n_chunks + 1) * E * 4, 256);
    return MOE_OK;
}

moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                       int32_t* expert_offsets, int32_t* perm_token, int32_t* perm_inv, void* ws,
                       size_t ws_bytes, void* stream) {
    size_t need = 0;
    moe_status st = moe_permute_workspace_size(T, k, E, &need);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !expert_offsets || !perm_token || !perm_inv || !ws) return MOE_ERR_ARG;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const size_t n_chunks = ((size_t)T + kPermChunk - 1) / kPermChunk;
    int32_t* counts = static_cast<int32_t*>(ws);
    int32_t* base = at<int32_t>(ws, round_up(n_chunks * E * 4, 256));
    return status_of(launch_permute(topk_idx, T, k, E, expert_offsets, perm_token, perm_inv, counts,
                                    base, nullptr, nullptr, s));
}

moe_status moe_expert_ffn(const moe_layer* L, const void* x, int32_t T,
                          const int32_t* expert_offsets, const int32_t* perm_token, float* y_perm,
                          void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if ((st = check_tokens(T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!x || !expert_offsets || !perm_token || !y_perm || !ws) return MOE_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y_perm, 16)) return MOE_ERR_UNSUPPORTED;
    const Layout o = layout_for(*L, T);
    if (ws_bytes < o.total) return MOE_ERR_WORKSPACE;
    (void)hipGetLastError();
    return run_experts(*L, x, T, expert_offsets, perm_token, y_perm, nullptr, false, ws, o, false,
                       static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_layer* L, const float* y_perm, const int32_t* perm_inv,
                       const float* topk_w, const float* shared_gate, int32_t T, void* y,
                       void* stream) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if ((st = check_tokens(T)) != MOE_OK) return st;
    if ((shared_gate != nullptr) != (L->shared_ff > 0)) return MOE_ERR_ARG;
    if (T == 0) return MOE_OK;
    if (!y_perm || !perm_inv || !topk_w || !y) return MOE_ERR_ARG;
    if (!aligned(y_perm, 16) || !aligned(y, 16)) return MOE_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    return status_of(launch_combine(*L, y_perm, perm_inv, topk_w, shared_gate, T, nullptr, y,
                                    static_cast<hipStream_t>(stream)));
}

moe_status moe_forward(const moe_layer* L, const void* x, int32_t T, void* y, void* ws,
                       size_t ws_bytes, void* stream) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if ((st = check_tokens(T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!x || !y || !ws) return MOE_ERR_ARG;
    if (x == y) return MOE_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 16)) return MOE_ERR_UNSUPPORTED;
    const Layout o = layout_for(*L, T);
    if (ws_bytes < o.total) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return forward_body(L, x, T, nullptr, y, ws, o, s);
}

moe_status moe_forward_shell(const moe_layer* L, const void* h, int32_t T, const void* norm_w, float eps,
                             void* out, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if ((st = check_tokens(T)) != MOE_OK) return st;
    if (!isfinite(eps) || eps < 0.0f) return MOE_ERR_ARG;
    if (T == 0) return MOE_OK;
    if (!h || !norm_w || !out || !ws) return MOE_ERR_ARG;
    // out may be h itself, but may not overlap it partially.
    const size_t row_bytes = (size_t)T * L->d * (L->dtype == MOE_BF16 ? 2 : 4);
    const uintptr_t hb = reinterpret_cast<uintptr_t>(h), ob = reinterpret_cast<uintptr_t>(out);
    if (hb != ob && hb < ob + row_bytes && ob < hb + row_bytes) return MOE_ERR_ARG;
    if (!aligned(h, 16) || !aligned(out, 16) || !aligned(ws, 16) || !aligned(norm_w, 16))
        return MOE_ERR_UNSUPPORTED;
    const Layout o = layout_for(*L, T);
    if (ws_bytes < o.total) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    void* xn = at<void>(ws, o.xn);
    // h is read by the norm (or the router that normalises) and then only by the final
    // kernel, element by element before out is written there, so out may alias h.
    if (T <= kDecodeMaxT && !router_on_mfma(*L, T) && router_norm_fits(*L)) {
        // Decode batches: the router GEMV normalises its token chunk itself.
        const RouterNorm norm{norm_w, eps, xn};
        return forward_body(L, xn, T, h, out, ws, o, s, &norm);
    }
    SMOE_TRY(launch_rmsnorm(*L, h, T, norm_w, eps, xn, s));
    return forward_body(L, xn, T, h, out, ws, o, s);
}

}  // extern "C"

// ------------------------------------------------------------------------------------
// Allocation-free forward: the workspace is a fixed device array of this library.
// ------------------------------------------------------------------------------------
namespace smoe {
namespace {

// One copy per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel or a copy (on the host that name is only a stand-in); it uses the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up once per device
// (with that device current); null if the lookup fails.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace smoe

extern "C" moe_status moe_forward_noalloc(const moe_layer* L, const void* x, int32_t T, void* y, void* stream) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if ((st = check_tokens(T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!x || !y) return MOE_ERR_ARG;
    if (x == y) return MOE_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y, 16)) return MOE_ERR_UNSUPPORTED;
    const Layout o = layout_for(*L, T);
    if (o.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    (void)hipGetLastError();
    void* ws = scratch_on_current_device();
    if (!ws) return MOE_ERR_DEVICE;
    // Every workspace region is written before it is read within one forward (no kernel
    // expects zeroed memory), so what an earlier call left in the array does not matter.
    return forward_body(L, x, T, nullptr, y, ws, o, static_cast<hipStream_t>(stream));
}

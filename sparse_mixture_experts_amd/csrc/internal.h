// Host-side launchers shared between the translation units of libsmoe.so.
// Every launcher only enqueues work on `s`; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace smoe {

// Tokens per permute chunk: one 64-bit token mask per expert and chunk.
constexpr int kPermChunk = 64;
// Rows per M-tile of the grouped MFMA kernels.
constexpr int kGroupTileM = 128;

// One group of grouped rows handled by the expert kernels: expert e (-1 = shared
// expert), its first grouped row, its row count and its first M-tile.
struct Group {
    int32_t e, row0, n, tile0;
};

// Plan metadata written next to the group list: number of groups, number of M-tiles.
struct PlanMeta {
    int32_t n_groups, n_tiles, pad0, pad1;
};

// One M-tile of the grouped kernels: expert e (-1 = shared), first grouped row, rows
// (1 .. kGroupTileM), index of its group in the group list.
struct TileDesc {
    int32_t e, row0, n, group;
};

inline int max_groups(int E, int T, int k, bool shared) {
    long long tk = (long long)T * k;
    return int((tk < E ? tk : E) + (shared ? 1 : 0));
}

// RMSNorm fused in front of the router GEMV (the layer shell): x is then the un-normalised
// input h; the router reads RMSNorm(h) * w and writes it to xn [T, d] in the layer dtype.
// Only for batches of at most 256 tokens (chunks of 4 tokens) whose 4 rows fit 64 KB of LDS.
struct RouterNorm {
    const void* w;
    float eps;
    void* xn;
};
constexpr size_t kRouterNormMaxLds = 64 * 1024;
bool router_norm_fits(const moe_layer& L);
hipError_t launch_router_logits(const moe_layer& L, const void* x, int T, float* logits, int ld,
                                hipStream_t s, const RouterNorm* norm = nullptr);
// row_w (optional, [T*k (+T)]): per grouped row routing weight, and sigmoid of the
// shared gate for the shared rows T*k + t; lets the down GEMM apply the weights.
// Router logits on MFMA (bf16, experts only: the shared-gate column is left to top-k).
hipError_t launch_router_mfma(const moe_layer& L, const void* x, int T, float* logits, int ld,
                              hipStream_t s);
// x_sg (optional, bf16 x): top-k computes the shared-gate input w_sg . x itself instead of
// reading logits column E.
hipError_t launch_topk(const moe_layer& L, const float* logits, int ld, int T, int32_t* idx,
                       float* w, float* shared_gate, float* row_w, const void* x_sg, hipStream_t s);
hipError_t launch_decode_route(const moe_layer& L, const float* logits, int ld, int T, int32_t* idx,
                               float* w, float* shared_gate, int32_t* offsets, int32_t* perm_token,
                               int32_t* perm_inv, float* row_w, int tile_m, Group* groups,
                               PlanMeta* meta, TileDesc* tiles, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* perm_token, int32_t* perm_inv, int32_t* counts, int32_t* base,
                          const float* w, float* row_w, hipStream_t s);
hipError_t launch_plan(const int32_t* offsets, int E, int T, int k, bool shared, int tile_m,
                       Group* groups, PlanMeta* meta, TileDesc* tiles, hipStream_t s);
int grouped_max_mtiles(int E, int T, int k, bool shared);
// The grouped copy of MXFP4 expert weights (moe_grouped_pack): byte offsets of its four
// regions (256-aligned) and its tile and slice counts.  Up: NTu N-tiles of 128 hidden units
// (256 gate/up rows) times Su = d/64 slices, 512 16-byte blocks and 512 scale bytes per
// (expert, N-tile, slice).  Down: NTd N-tiles of 256 output rows times Sd = ff/32 slices,
// 256 blocks and 256 scale bytes each.
struct MxPackLayout {
    size_t up_codes, up_scales, dn_codes, dn_scales, total;
    int ntu, su, ntd, sd;
};
MxPackLayout mx_pack_layout(const moe_layer& L);
hipError_t launch_mx_pack(const moe_layer& L, void* dst, hipStream_t s);
// The grouped copy of Q4_K expert weights: up region (NTu N-tiles of 128 units x d/256
// super-blocks) at `up`, down region (NTd N-tiles of 256 rows x ff/256) at `dn`; each
// (expert, N-tile, super-block) group holds 256 rows' 16-byte headers, then quant run
// c = 0..3 of every row as 32 bytes (256 x 144 bytes in all).
struct Q4kPackLayout {
    size_t up, dn, total;
    int ntu, ntd;
};
Q4kPackLayout q4k_pack_layout(const moe_layer& L);
hipError_t launch_q4k_pack(const moe_layer& L, void* dst, hipStream_t s);
// The grouped copy of dense bf16 down weights: routed W_d at `dn` as [E][NTd][ff/32][256][32]
// (NTd N-tiles of 256 output rows, 32-input slices; rows past d repeat the last), the
// shared expert's at `sh` as [NTd][shared_ff/32][256][32].
struct DensePackLayout {
    size_t dn, sh, total;
    int ntd;
};
DensePackLayout dense_pack_layout(const moe_layer& L);
hipError_t launch_dense_pack(const moe_layer& L, void* dst, hipStream_t s);
// Grouped up + down.  ksplit > 1: the down projection cuts each tile's K axis into that
// many slices, summing them through `partial` (fp32, ksplit * rows * d floats).
hipError_t launch_grouped_ffn(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                              const Group* groups, const PlanMeta* meta, const TileDesc* tiles,
                              uint16_t* H, int hstride, const float* row_w, void* y, bool y_bf16,
                              int ksplit, float* partial, hipStream_t s);
// Combine of pre-weighted bf16 rows: y[t] = sum_j Y[perm_inv[t,j]] (+ Y[T*k + t]).
hipError_t launch_combine_sum(const moe_layer& L, const uint16_t* y_rows, const int32_t* perm_inv,
                              int T, const void* residual, void* y, hipStream_t s);
// Decode GEMVs (up then down; fp32 H and unweighted fp32 rows).  With plan_offsets (the
// expert offsets; dense experts and one token only) the up kernel builds the group list
// and count into groups / meta itself, so no planning launch has to come first.
hipError_t launch_expert_gemv(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                              Group* groups, PlanMeta* meta, float* H, int hstride, float* y_perm,
                              const int32_t* plan_offsets, hipStream_t s);
// GEMVs over MXFP4 expert weights (up then down; H in bf16 in the fp32 H region;
// unweighted fp32 rows), for layers with MOE_EXPERTS_MXFP4; mx_fits: the widths the
// kernels take (K <= 4096).
bool mx_fits(const moe_layer& L);
hipError_t launch_expert_gemv_mx(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                 const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                                 hipStream_t s);
// The MXFP4 up GEMV alone (bf16 H rows), and the one-token / few-token fused kernels of
// the MXFP4 layer: top-k inside the up GEMV (one token; hidden row j = pick j), and the
// down GEMVs of every pick with the weighted combine written straight to y (hidden rows
// perm_inv[t*k+j], or row j for one token).  token1_mx_fits: k <= 16, no shared expert.
hipError_t launch_expert_up_gemv_mx(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                    const Group* groups, const PlanMeta* meta, float* H, int hstride,
                                    hipStream_t s);
bool token1_mx_fits(const moe_layer& L);
// GEMVs over Q4_K routed experts (fp32 H and unweighted fp32 rows, as the dense GEMVs);
// a bf16 shared expert as wide as the routed experts runs in the same launches (its H rows
// rounded to bf16 for the down GEMV, as the routed ones), one of another width on the dense
// kernels restricted to its grid row (launch_shared_gemv_*).  q4k_fits: d and ff multiples
// of 256, at most 4096.
bool q4k_fits(const moe_layer& L);
hipError_t launch_expert_gemv_q4k(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                  const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                                  hipStream_t s);
// The Q4_K up GEMVs alone (routed and shared H rows), and the one-token / few-token
// kernels of the Q4_K layer: top-k inside the up GEMV (one token, routed picks only: the
// shared expert's up runs in the router launch), and the down GEMVs of every pick and of
// the shared expert with the weighted combine written straight to y (hidden rows
// perm_inv[t*k+j], or row j for one token; shared row T*k + t, gate shared_gate[t*gate_ld]).
// q4k_token_fits: k (+1 with a shared expert) <= 16 and k staged H rows (ff bf16 and ff/32
// fp32 sums each) within 64 KB of LDS.
bool q4k_token_fits(const moe_layer& L);
hipError_t launch_expert_up_gemv_q4k(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                     const Group* groups, const PlanMeta* meta, float* H, int hstride,
                                     hipStream_t s);
hipError_t launch_token1_up_q4k(const moe_layer& L, const void* x, const float* logits, int32_t* idx, float* w,
                                float* H, int hstride, hipStream_t s);
hipError_t launch_token_down_combine_q4k(const moe_layer& L, int T, const float* H, int hstride, const int32_t* idx,
                                         const float* w, const int32_t* perm_inv, const float* shared_gate,
                                         int gate_ld, const void* residual, void* y, hipStream_t s);
hipError_t launch_shared_gemv_up(const moe_layer& L, const void* x, int T, const Group* groups, const PlanMeta* meta,
                                 float* H, int hstride, hipStream_t s);
hipError_t launch_shared_gemv_down(const moe_layer& L, int T, const Group* groups, const PlanMeta* meta,
                                   const float* H, int hstride, float* y_perm, hipStream_t s);
hipError_t launch_token1_up_mx(const moe_layer& L, const void* x, const float* logits, int32_t* idx, float* w,
                               float* H, int hstride, hipStream_t s);
hipError_t launch_token_down_combine_mx(const moe_layer& L, int T, const float* H, int hstride, const int32_t* idx,
                                        const float* w, const int32_t* perm_inv, const void* residual, void* y,
                                        hipStream_t s);
// Up GEMV alone (H rows), for callers that finish the layer themselves.
hipError_t launch_expert_up_gemv(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                 const Group* groups, const PlanMeta* meta, float* H, int hstride,
                                 hipStream_t s);
// One token (T = 1): top-k on the router logits fused into the up GEMV (hidden row j for
// pick j, row k for the shared expert; the picks go to idx / w).  A few tokens: the down
// GEMVs of every pick and of the shared expert plus the weighted combine, written straight
// to y; hidden rows perm_inv[t*k+j] (null for one token: row j) and T*k + t (shared, gate
// shared_gate[t * gate_ld]).  Both need k (+1 with a shared expert) <= 16.
bool token1_fits(const moe_layer& L);
hipError_t launch_token1_up(const moe_layer& L, const void* x, const float* logits, int32_t* idx, float* w,
                            float* H, int hstride, bool shared_done, hipStream_t s);
// One token, bf16 with a shared expert: the router logits (ld = E + 1) and the shared
// expert's up GEMV (hidden row k) in one launch; token1_up then runs with shared_done.
bool token1_router_shared_fits(const moe_layer& L);
hipError_t launch_token1_router_shared(const moe_layer& L, const void* x, float* logits, int ld, float* H,
                                       int hstride, hipStream_t s);
hipError_t launch_token_down_combine(const moe_layer& L, int T, const float* H, int hstride, const int32_t* idx,
                                     const float* w, const int32_t* perm_inv, const float* shared_gate,
                                     int gate_ld, const void* residual, void* y, hipStream_t s);
// residual (optional, [T, d] in the layer's dtype) is added to every output row.
hipError_t launch_combine(const moe_layer& L, const float* y_perm, const int32_t* perm_inv,
                          const float* w, const float* shared_gate, int T, const void* residual, void* y,
                          hipStream_t s);
// xn[t] = RMSNorm(h[t]) * w in the layer's dtype (the layer shell's norm).
hipError_t launch_rmsnorm(const moe_layer& L, const void* h, int T, const void* w, float eps, void* xn,
                          hipStream_t s);


}  // namespace smoe

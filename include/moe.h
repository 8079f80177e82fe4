/*
 * moe.h -- C ABI of libsmoe.so, the sparse mixture-of-experts FFN layer on one
 * MI355X (gfx950).
 *
 * The layer (per token t, input x[t] of width d):
 *   z      = W_r x (+ b_r)                                   router logits, E of them
 *   S, w   = the k experts with the largest logits and their routing weights
 *   out    = sum_j w_j FFN_{S_j}(x) (+ sigmoid(w_sg . x) FFN_shared(x))
 * as defined on "Qwen3.5-MoE Model Implementation" (section "MoE routing": router,
 * top-8, renormalisation, SwiGLU experts, sigmoid-gated shared expert, combine with
 * the residual left to the caller), "Llama Forward Pass" (section "Mixture of
 * Experts (Mixtral)") and "Phase 19: MoE - gpt-oss-20b" (section 2, Router and
 * Experts: top-k before softmax with a router bias; interleaved, clamped
 * (up + 1) * gate * sigmoid(alpha * gate) experts with biases).  The grouped
 * evaluation (each expert run once over the rows routed to it, the results returned to
 * their tokens) follows "Engine" (Cherenkov), section "Prefill".
 *
 * Conventions (every entry point):
 *  - Every pointer argument and every pointer inside moe_layer is DEVICE memory
 *    unless stated otherwise; the moe_layer struct itself and size_t* out-arguments
 *    are HOST memory.  The caller owns all memory; the library borrows it for the
 *    duration of the enqueued work and never allocates, frees or synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls
 *    only enqueue kernels; results are valid once the stream's work has completed.
 *  - Tensors are dense, row-major, with no padding.  Weights are [out, in]
 *    (the input dimension is contiguous).
 *  - Argument checks happen on the host before anything is enqueued.  On any error
 *    the call returns without enqueuing work and without writing any output.
 *    T == 0 is a no-op that returns MOE_OK.
 *  - Results are deterministic: no floating-point atomics, fixed reduction orders.
 *  - The functions hold no state and may be called from several host threads
 *    (moe_forward_noalloc shares one scratch array per GPU; see there).
 */
#ifndef SMOE_MOE_H
#define SMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,          /* null required pointer, bad enum, k < 1, k > E, T < 0, ... */
    MOE_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle (see below)    */
    MOE_ERR_WORKSPACE = 3,    /* workspace smaller than the size query returned           */
    MOE_ERR_DEVICE = 4        /* a HIP launch failed (hipGetLastError after enqueue)      */
};

/* dtype of x, y and every weight except the router bias (always fp32). */
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Routing mode.
 *  SOFTMAX_TOPK_RENORM ("Qwen3.5-MoE Model Implementation", MoE routing; "Llama Forward
 *    Pass", Mixture of Experts): p = softmax(z) over all E experts, S = top-k, weights
 *    w_j = route_scale * p_{S_j} / sum_j' p_{S_j'}.
 *  TOPK_SOFTMAX ("Phase 19: MoE - gpt-oss-20b", Router): S = top-k of z, weights
 *    w = softmax over the k selected logits (route_scale is ignored).
 *  In both modes S is ordered by descending logit and ties go to the lower expert
 *  index; a router bias, when given, is added to z before selection. */
enum { MOE_ROUTE_SOFTMAX_TOPK_RENORM = 0, MOE_ROUTE_TOPK_SOFTMAX = 1 };

/* Expert activation.
 *  SWIGLU: h = silu(W_g x) * (W_u x), y = W_d h ("Llama Forward Pass", SwiGLU FFN).
 *  SWIGLU_OAI ("Phase 19: MoE - gpt-oss-20b", Experts): v = W_gu x + b_gu with rows of
 *    W_gu interleaved (row 2m = gate m, row 2m+1 = up m); gate = min(v_2m, limit);
 *    up = clamp(v_2m+1, -limit, limit); h = (up + 1) * gate * sigmoid(alpha * gate);
 *    y = W_d h + b_d (the down bias is inside the routing-weighted sum). */
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_SWIGLU_OAI = 1 };

/* Kernel path.  AUTO: the grouped MFMA path for T > 64 (Q4K experts: T > 128, or from 65
 * tokens once the expected rows per active expert reach 8), and also for smaller batches
 * (bf16) whose expected rows per active expert reach 4 (2 for dense experts whose gate and
 * up weights take 16 MB or more), taking E * (1 - (1 - k/E)^T) distinct experts as for
 * uniform routing; else the decode GEMV path.  DECODE / GROUPED force one path at any T
 * (GROUPED requires MOE_BF16). */
enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_GROUPED = 2 };

/* Storage of the routed experts' gate_up and down weights.
 *  DENSE: in `dtype`, as described at each field.
 *  MXFP4 ("Phase 19: MoE - gpt-oss-20b", section 3 and the measured tensor layout):
 *    w_gate_up = blocks [E, 2*ff, d/32, 16] uint8 with scales w_gate_up_scales
 *    [E, 2*ff, d/32] uint8, and w_down = blocks [E, d, ff/32, 16] uint8 with scales
 *    w_down_scales [E, d, ff/32] uint8.  Each 16-byte block holds the 32 FP4 (E2M1,
 *    OCP Microscaling) codes of 32 consecutive inputs, the low nibble of byte i being
 *    element 2i; each scale is an E8M0 exponent: value = fp4(code) * 2^(scale - 127).
 *    Requires MOE_BF16, MOE_ACT_SWIGLU_OAI, no shared expert and d, ff <= 4096.  The
 *    GEMV path expands the blocks in registers; the grouped path expands each K-slice of
 *    a weight tile into LDS as bf16 for the bf16 MFMA (activations stay bf16).  Biases,
 *    router, x and y stay bf16.
 *  Q4K (K-quant experts named on "Qwen3.5-MoE Model Implementation", numeric status, and
 *    "Engine", Prefill; the block layout is GGUF's Q4_K, not printed on the pages):
 *    w_gate, w_up = [E, ff, d/256, 144] and w_down = [E, d, ff/256, 144] uint8 super-blocks
 *    of 256 consecutive inputs each: fp16 d and dmin (bytes 0-3), eight packed 6-bit
 *    scales and mins of the 32-input sub-blocks (bytes 4-15), 4-bit quants in 4 runs of 32
 *    bytes (low nibble of byte l of run c = input 64c + l, high nibble = input 64c+32+l);
 *    weight = d * scale_j * q - dmin * min_j.  Requires MOE_BF16, MOE_ACT_SWIGLU, d and ff
 *    multiples of 256 and at most 4096, and NULL *_scales fields.  The shared expert, router,
 *    x and y stay bf16.  The GEMV path decodes the quants in registers and meets them with
 *    activations held as bf16 (the hidden rows H rounded to bf16, as on the grouped path;
 *    also the shared expert's, when it is as wide as the routed experts and runs in the same
 *    GEMVs); the grouped path expands each K-slice of a weight tile into LDS as bf16 for
 *    the bf16 MFMA. */
enum { MOE_EXPERTS_DENSE = 0, MOE_EXPERTS_MXFP4 = 1, MOE_EXPERTS_Q4K = 2 };

/* One MoE layer.  Fixed layout: 9 int32, 3 float, then 12 pointers (offset 48), then
 * 2 int32 and 3 pointers (offset 144).  No field depends on a build flag.  All pointers
 * are device memory, 16-byte aligned (b_router, b_gate_up, b_down and the MXFP4 scales:
 * element-aligned suffices). */
typedef struct moe_layer {
    int32_t d;            /* model width; multiple of 64                               */
    int32_t n_expert;     /* E, 1..512                                                 */
    int32_t ff;           /* expert hidden width; multiple of 64                       */
    int32_t k;            /* experts per token, 1..min(E, 32)                          */
    int32_t shared_ff;    /* shared expert hidden width; 0 = no shared expert; %64==0  */
    int32_t dtype;        /* MOE_F32 | MOE_BF16                                        */
    int32_t route;        /* MOE_ROUTE_*                                               */
    int32_t act;          /* MOE_ACT_*                                                 */
    int32_t path;         /* MOE_PATH_*                                                */
    float route_scale;    /* expert weight scale of mode SOFTMAX_TOPK_RENORM (1.0)     */
    float oai_alpha;      /* 1.702 for SWIGLU_OAI                                      */
    float oai_limit;      /* 7.0 for SWIGLU_OAI                                        */
    const void* w_router;     /* [E, d]                                                */
    const float* b_router;    /* [E] fp32, or NULL                                     */
    const void* w_gate;       /* SWIGLU: [E, ff, d]                                    */
    const void* w_up;         /* SWIGLU: [E, ff, d]                                    */
    const void* w_gate_up;    /* SWIGLU_OAI: [E, 2*ff, d], rows gate,up interleaved    */
    const void* b_gate_up;    /* SWIGLU_OAI: [E, 2*ff]; must be NULL for SWIGLU        */
    const void* w_down;       /* [E, d, ff]                                            */
    const void* b_down;       /* SWIGLU_OAI: [E, d] or NULL; must be NULL for SWIGLU   */
    const void* ws_gate;      /* shared expert: [shared_ff, d]                         */
    const void* ws_up;        /* shared expert: [shared_ff, d]                         */
    const void* ws_down;      /* shared expert: [d, shared_ff]                         */
    const void* ws_gate_inp;  /* shared expert sigmoid gate vector: [d]                */
    int32_t expert_format;    /* MOE_EXPERTS_*                                         */
    int32_t reserved0;        /* 0                                                     */
    const uint8_t* w_gate_up_scales;  /* MXFP4: [E, 2*ff, d/32] E8M0, else NULL        */
    const uint8_t* w_down_scales;     /* MXFP4: [E, d, ff/32] E8M0, else NULL          */
    const void* grouped_pack;         /* the grouped path's copy of expert weights
                                         written by moe_grouped_pack, or NULL (the
                                         grouped kernels then read the fields above);
                                         bf16 layers only                              */
} moe_layer;

/* ABI version of this header (bumped on any layout or signature change). */
int32_t moe_abi_version(void);

/* Static description of a status code.  Never NULL. */
const char* moe_status_string(moe_status s);

/* Workspace bytes needed by moe_route, moe_expert_ffn, moe_forward and
 * moe_forward_shell for this layer and up to T tokens (one size covers all of them).  Writes *bytes (host).  Errors:
 * MOE_ERR_ARG / MOE_ERR_UNSUPPORTED as for moe_forward. */
moe_status moe_workspace_size(const moe_layer* L, int32_t T, size_t* bytes);

/* Router and top-k ("Qwen3.5-MoE Model Implementation", MoE routing; "Phase 19",
 * Router).
 *   x           [T, d] in L->dtype
 *   topk_idx    [T, k] int32 out: selected experts, descending logit, ties -> lower id
 *   topk_w      [T, k] fp32 out: routing weights of the layer's mode
 *   shared_gate [T] fp32 out: w_sg . x (the sigmoid's input), or NULL; must be NULL
 *               when the layer has no shared expert
 *   ws          device workspace of at least moe_workspace_size(L, T) bytes */
moe_status moe_route(const moe_layer* L, const void* x, int32_t T, int32_t* topk_idx,
                     float* topk_w, float* shared_gate, void* ws, size_t ws_bytes,
                     void* stream);

/* Workspace bytes needed by moe_permute. */
moe_status moe_permute_workspace_size(int32_t T, int32_t k, int32_t E, size_t* bytes);

/* Reorder the T*k (token, slot) pairs so that each expert's rows are contiguous
 * ("Engine", section "Prefill").
 *   topk_idx        [T, k] int32 in, entries in [0, E), distinct within a row
 *   expert_offsets  [E+1] int32 out: exclusive prefix sum of per-expert counts
 *   perm_token      [T*k] int32 out: token of grouped row r (expert-major rows, tokens
 *                   ascending inside an expert)
 *   perm_inv        [T*k] int32 out: grouped row of (t, j), at index t*k + j
 * Entries outside [0, E) are ignored (not counted; their perm_inv is -1). */
moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                       int32_t* expert_offsets, int32_t* perm_token, int32_t* perm_inv,
                       void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs over the grouped rows ("Qwen3.5-MoE Model Implementation", MoE
 * routing: SwiGLU experts and the shared expert; "Phase 19", Experts).
 *   expert_offsets, perm_token  as produced by moe_permute for this T and k
 *   y_perm  [T*k + (shared_ff ? T : 0), d] fp32 out: row r < T*k holds
 *           FFN_e(x[perm_token[r]]) for the expert e owning row r (down bias included,
 *           routing weight NOT applied); row T*k + t holds the shared expert's output
 *           for token t without its sigmoid gate. */
moe_status moe_expert_ffn(const moe_layer* L, const void* x, int32_t T,
                          const int32_t* expert_offsets, const int32_t* perm_token,
                          float* y_perm, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine ("Qwen3.5-MoE Model Implementation", MoE routing: out = moe_out +
 * shexp_out, no residual):
 *   y[t] = sum_{j<k} topk_w[t,j] * y_perm[perm_inv[t*k+j]]
 *          (+ sigmoid(shared_gate[t]) * y_perm[T*k + t])
 * summed in fp32 in the order j = 0..k-1, then the shared term; y [T, d] in L->dtype.
 * shared_gate must be non-NULL exactly when the layer has a shared expert. */
moe_status moe_combine(const moe_layer* L, const float* y_perm, const int32_t* perm_inv,
                       const float* topk_w, const float* shared_gate, int32_t T, void* y,
                       void* stream);

/* The whole layer: route, group, expert FFNs, combine.  x [T, d] and y [T, d] in
 * L->dtype (y must not alias x); ws of at least moe_workspace_size(L, T) bytes.
 * Unsupported: d, ff or shared_ff not a multiple of 64; E > 512; k > 32;
 * MOE_PATH_GROUPED with MOE_F32. */
moe_status moe_forward(const moe_layer* L, const void* x, int32_t T, void* y, void* ws,
                       size_t ws_bytes, void* stream);

/* The FFN half of a decoder layer around the block ("Qwen3.5-MoE Model Implementation",
 * Architecture: post-attention norm, shared-MoE FFN, residual add; RMSNorm as in "Llama
 * Forward Pass", Key Operations):
 *     out[t] = h[t] + MoE(RMSNorm(h[t]) * norm_w),  RMSNorm(v) = v / sqrt(mean(v^2) + eps).
 * The normalised rows are computed in fp32 and stored in L->dtype (bf16: rounded to
 * nearest even) in the workspace; the block reads them as moe_forward reads x, and the
 * residual is added to the fp32 sum before the output is stored.
 *   h       [T, d] in L->dtype (the layer input and the residual)
 *   norm_w  [d] in L->dtype, 16-byte aligned
 *   eps     finite, >= 0 (the pages use 1e-5)
 *   out     [T, d] in L->dtype; may equal h (in-place residual update), must not overlap
 *           it otherwise
 *   ws      as for moe_forward: moe_workspace_size(L, T) bytes cover this call too
 * Errors as moe_forward; MOE_ERR_ARG for a negative or non-finite eps. */
moe_status moe_forward_shell(const moe_layer* L, const void* h, int32_t T, const void* norm_w, float eps,
                             void* out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the library's fixed device scratch array used by moe_forward_noalloc (one
 * array per GPU, allocated when the library's code is loaded on that GPU and held until
 * the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* The grouped (MFMA) path's copy of expert weights ("Engine" (Cherenkov), Prefill: the
 * experts evaluated as tiled GEMMs).  Each K-slice of a weight tile that the grouped
 * kernels load is stored as contiguous runs, in the order the threads of a block read
 * them, so a wave's loads cover whole cache lines; in the checkpoint layouts a slice is a
 * few bytes of every row.  What is copied:
 *  - MXFP4 and Q4K: the routed experts' gate_up / gate, up and down blocks (rows of
 *    16-byte MXFP4 blocks, "Phase 19: MoE - gpt-oss-20b", section 3; rows of 144-byte
 *    Q4_K super-blocks), codes, scales and headers unchanged;
 *  - dense bf16 experts: the down weights only (routed and shared), whose 32-input slices
 *    are half a cache line of each row in place; the up weights' 64-input slices already
 *    cover whole lines and are read in place.
 * Same values, so results are bit for bit those of the checkpoint layout.  The decode
 * GEMVs keep reading the checkpoint layout, which suits their whole-row reads.
 * moe_grouped_pack_size writes the copy's size to *bytes (host): about the size of the
 * copied weights.  Errors: MOE_ERR_ARG / MOE_ERR_UNSUPPORTED as for moe_forward;
 * MOE_ERR_UNSUPPORTED for fp32 layers (they have no grouped path).
 * moe_grouped_pack enqueues on `stream` the kernels that write the copy to `dst` (device,
 * 16-byte aligned, at least that size; it must not overlap the layer's weights).  The
 * caller owns `dst`; store it in moe_layer.grouped_pack for the calls that should use it
 * and keep it alive while they run.  L->grouped_pack itself is ignored here.  Errors as
 * moe_grouped_pack_size, plus MOE_ERR_ARG for a null dst, MOE_ERR_UNSUPPORTED for a
 * misaligned one, MOE_ERR_WORKSPACE when `bytes` is below the size, and MOE_ERR_DEVICE. */
moe_status moe_grouped_pack_size(const moe_layer* L, size_t* bytes);
moe_status moe_grouped_pack(const moe_layer* L, void* dst, size_t bytes, void* stream);

/* moe_forward without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same layer, same kernels and same results as moe_forward; the workspace is the fixed
 * array above.  The call itself allocates and frees nothing.
 *   x [T, d], y [T, d] in L->dtype; y must not alias x.
 * Errors as moe_forward, plus MOE_ERR_WORKSPACE when the batch needs more workspace than
 * MOE_NOALLOC_SCRATCH_BYTES (moe_workspace_size(L, T) reports the need; 64 MiB covers
 * every batch of up to 64 tokens of the Qwen-, gpt-oss- and Mixtral-shaped layers), and
 * MOE_ERR_DEVICE when the array's device address cannot be obtained.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (on different streams, or from several host threads without ordering) race and give
 * undefined results.  Calls ordered on one stream are safe. */
moe_status moe_forward_noalloc(const moe_layer* L, const void* x, int32_t T, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_MOE_H */

// Router: logits z = W_r x (+ b_r), the shared-expert gate input w_sg . x, and the
// wave-level top-k with the routing weights of either mode.
//
// "Qwen3.5-MoE Model Implementation", MoE routing: router matrix [n_expert, n_embd],
// softmax, top-8, renormalisation, expert_weights_scale; the shared expert's scalar
// sigmoid gate [n_embd].  "Phase 19: MoE - gpt-oss-20b", Router: logits with bias,
// top-k first, softmax over the k selected.
#include <math.h>

#include "internal.h"
#include "norm_dev.h"
#include "permute_dev.h"
#include "route_dev.h"
#include "rowdot.h"

namespace smoe {
namespace {

// NR router rows per wave (rows 0..E-1 are experts, row E the shared gate vector),
// looping over a chunk of tokens.  Writes logits[t * ld + row].  The 1-D grid holds
// n_groups row groups (4 waves each) times n_chunks token chunks, ordered so that every
// token chunk of a row group runs on the same XCD (blocks go to the 8 XCDs round-robin by
// id): each XCD then fetches its row groups' router rows into its own L2 once, instead of
// every XCD fetching the whole router matrix.
constexpr int kRouterXcds = 8;

template <int KB, typename TT, int NR>
__global__ __launch_bounds__(256) void router_gemv_kernel(
    const typename TT::storage* __restrict__ x, const typename TT::storage* __restrict__ w_router,
    const float* __restrict__ b_router, const typename TT::storage* __restrict__ w_sg, int T, int d,
    int E, int n_rows, int tok_chunk, int n_chunks, float* __restrict__ logits, int ld) {
    const int xcd = blockIdx.x % kRouterXcds, slot = blockIdx.x / kRouterXcds;
    const int group = xcd + kRouterXcds * (slot / n_chunks), chunk = slot % n_chunks;
    const int row0 = (group * 4 + wave_id()) * NR;
    if (row0 >= n_rows) return;
    const int t0 = chunk * tok_chunk;
    if (t0 >= T) return;
    router_rows_wave<KB, TT, NR>(x, w_router, b_router, w_sg, T, d, E, n_rows, row0, t0, min(T, t0 + tok_chunk),
                             logits, ld);
}

// The same over the RMSNorm of the rows (the layer shell, chunks of kRouterNT tokens):
// wave w first normalises token t0 + w of h into LDS (and, in the blocks of grid column
// 0, into xn for the expert kernels), then the block's router rows read the LDS rows.
template <int KB, typename TT, int NR>
__global__ __launch_bounds__(256) void router_norm_gemv_kernel(
    const typename TT::storage* __restrict__ h, const typename TT::storage* __restrict__ norm_w, float eps,
    typename TT::storage* __restrict__ xn, const typename TT::storage* __restrict__ w_router,
    const float* __restrict__ b_router, const typename TT::storage* __restrict__ w_sg, int T, int d, int E,
    int n_rows, float* __restrict__ logits, int ld) {
    using S = typename TT::storage;
    extern __shared__ uint4 smem_rows[];  // kRouterNT rows of d elements
    S* xs = reinterpret_cast<S*>(smem_rows);
    const int t0 = blockIdx.y * kRouterNT;
    const int w = wave_id(), t = t0 + w;
    if (t < T)
        rmsnorm_row_wave<TT>(h + (size_t)t * d, norm_w, eps, d, xs + (size_t)w * d,
                             blockIdx.x == 0 ? xn + (size_t)t * d : nullptr);
    __syncthreads();
    const int row0 = (blockIdx.x * 4 + w) * NR;
    if (row0 >= n_rows) return;
    router_rows_wave<KB, TT, NR>(xs, w_router, b_router, w_sg, T, d, E, n_rows, row0, t0, min(T, t0 + kRouterNT),
                                 logits, ld, t0);
}

// One wave per token: the wave top-k, the weights, and the shared-expert gate input.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int ld, int T,
                                                   int E, int k, int mode, float scale,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ w_out,
                                                   float* __restrict__ sg_out,
                                                   float* __restrict__ row_w,
                                                   const uint16_t* __restrict__ x_sg,
                                                   const uint16_t* __restrict__ w_sg, int d) {
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    const float* z = logits + (size_t)t * ld;
    int my_i;
    float my_w;
    topk_wave(z, E, k, mode, scale, &my_i, &my_w);
    const int lane = lane_id();
    if (lane < k) {
        idx_out[(size_t)t * k + lane] = my_i;
        w_out[(size_t)t * k + lane] = my_w;
    }
    if (sg_out) {
        float a;
        if (x_sg) {  // shared-gate input w_sg . x[t], bf16 products, fp32 sum
            float acc = 0.0f;
            const uint16_t* xr = x_sg + (size_t)t * d;
            for (int i = lane * 8; i < d; i += kWave * 8) {
                float xv[8], wv[8];
                unpack16<BF16>(ld16(xr + i), xv);
                unpack16<BF16>(ld16(w_sg + i), wv);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc = fmaf(xv[q], wv[q], acc);
            }
            a = wave_sum(acc);
        } else {
            a = z[E];
        }
        if (lane == 0) {
            sg_out[t] = a;
            if (row_w) row_w[(size_t)T * k + t] = 1.0f / (1.0f + expf(-a));
        }
    }
}

// Decode (T <= 64): the expert grouping and the group plan in one block of 1024 threads,
// after the top-k of every token, done here (topk_here, one wave per token) for small T or
// beforehand by topk_kernel, whose blocks spread the tokens over many compute units.
__global__ __launch_bounds__(1024) void decode_route_kernel(
    const float* __restrict__ logits, int ld, int T, int E, int k, int mode, float scale,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, float* __restrict__ sg_out,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token, int32_t* __restrict__ perm_inv,
    float* __restrict__ row_w, int shared, int tile_m, Group* __restrict__ groups,
    PlanMeta* __restrict__ meta, TileDesc* __restrict__ tiles, int tile_cap, int topk_here) {
    __shared__ float s_w[kPermChunk * 32];
    __shared__ int32_t s_idx[kPermChunk * 32];
    __shared__ unsigned long long mask[kMaxE];
    __shared__ int32_t base_row[kMaxE + 1];
    __shared__ int tmp[2 * 1024 / kWave];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    if (!topk_here) {  // top-k already done by topk_kernel: idx_out / w_out hold it
        for (int p = threadIdx.x; p < T * k; p += blockDim.x) {
            s_idx[p] = idx_out[p];
            s_w[p] = w_out[p];
        }
    }
    for (int t = wave; topk_here && t < T; t += 1024 / kWave) {
        const float* z = logits + (size_t)t * ld;
        int my_i;
        float my_w;
        topk_wave(z, E, k, mode, scale, &my_i, &my_w);
        if (lane < k) {
            idx_out[(size_t)t * k + lane] = my_i;
            w_out[(size_t)t * k + lane] = my_w;
            s_idx[t * k + lane] = my_i;
            s_w[t * k + lane] = my_w;
        }
        if (sg_out && lane == 0) {
            sg_out[t] = z[E];
            if (row_w) row_w[T * k + t] = 1.0f / (1.0f + expf(-z[E]));
        }
    }
    __syncthreads();
    if (T * k <= kWave && tile_m >= kWave) {
        // One wave groups every routed row; expert offsets are not needed by the forward.
        if (wave == 0)
            group_wave_small(s_idx, s_w, T, k, E, shared, perm_token, perm_inv, row_w, groups, meta, tiles,
                             tile_cap);
        return;
    }
    build_masks(s_idx, T, k, E, 0, mask);
    const int e = threadIdx.x;
    const int cnt = e < E ? __popcll(mask[e]) : 0;
    int total;
    const int off = block_exclusive_scan(cnt, tmp, &total);
    if (e < E) {
        base_row[e] = off;
        offsets[e] = off;
    }
    if (e == 0) {
        base_row[E] = total;
        offsets[E] = total;
    }
    __syncthreads();
    scatter_chunk(s_idx, T, k, E, 0, mask, base_row, perm_token, perm_inv, s_w, row_w);
    plan_block(base_row, E, T, k, shared, tile_m, groups, meta, tiles, tile_cap, tmp);
}

template <typename TT>
hipError_t launch_router_t(const moe_layer& L, const void* x, int T, float* logits, int ld,
                           const RouterNorm* norm, hipStream_t s) {
    using S = typename TT::storage;
    const int n_rows = L.n_expert + (L.shared_ff > 0 ? 1 : 0);
    // Small batches: one 4-token chunk per block row, so that every wave issues its
    // loads at once; large batches: 64 tokens per block to reuse the router row.  Up to
    // 64 tokens (decode batches), one row per wave: four times the waves in flight.
    const int tok_chunk = T <= 256 ? kRouterNT : 64;
    const bool one_row = T <= 64;
    const int nr = one_row ? 1 : kRouterNR;
    const int n_groups = (n_rows + 4 * nr - 1) / (4 * nr);
    const int n_chunks = (T + tok_chunk - 1) / tok_chunk;
    dim3 grid(n_groups, n_chunks);  // the normalising variant's 2-D grid
    // The plain variant's 1-D grid: whole rounds of kRouterXcds row groups per chunk set.
    const unsigned flat = (unsigned)(kRouterXcds * ((n_groups + kRouterXcds - 1) / kRouterXcds) * n_chunks);
    const S* xs = static_cast<const S*>(x);
    const S* wr = static_cast<const S*>(L.w_router);
    // The normalising variant works on chunks of kRouterNT tokens held in LDS.
    if (norm && (tok_chunk != kRouterNT || !router_norm_fits(L))) return hipErrorInvalidValue;
    const size_t norm_lds = norm ? (size_t)kRouterNT * L.d * sizeof(S) : 0;
    const S* wsg = static_cast<const S*>(L.ws_gate_inp);
    // Weight batches of at most 4 chunks per lane (longer rows loop over batches).
    switch (min(pick_kb(L.d, TT::VEC), 4)) {
#define SMOE_ROUTER_LAUNCH(KB, NR)                                                             \
    do {                                                                                       \
        if (norm)                                                                              \
            router_norm_gemv_kernel<KB, TT, NR><<<grid, 256, norm_lds, s>>>(                   \
                xs, static_cast<const S*>(norm->w), norm->eps, static_cast<S*>(norm->xn), wr,   \
                L.b_router, wsg, T, L.d, L.n_expert, n_rows, logits, ld);                     \
        else                                                                                   \
            router_gemv_kernel<KB, TT, NR><<<flat, 256, 0, s>>>(xs, wr, L.b_router, wsg, T,     \
                                                                L.d, L.n_expert, n_rows,       \
                                                                tok_chunk, n_chunks, logits, ld); \
    } while (0)
#define SMOE_ROUTER_CASE(KB)                                                                   \
    case KB:                                                                                   \
        if (one_row) SMOE_ROUTER_LAUNCH(KB, 1);                                                \
        else SMOE_ROUTER_LAUNCH(KB, kRouterNR);                                                \
        break;
        SMOE_ROUTER_CASE(1)
        SMOE_ROUTER_CASE(2)
        SMOE_ROUTER_CASE(4)
        default:
            return hipErrorInvalidValue;
#undef SMOE_ROUTER_CASE
#undef SMOE_ROUTER_LAUNCH
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_route(const moe_layer& L, const float* logits, int ld, int T, int32_t* idx,
                               float* w, float* shared_gate, int32_t* offsets, int32_t* perm_token,
                               int32_t* perm_inv, float* row_w, int tile_m, Group* groups,
                               PlanMeta* meta, TileDesc* tiles, hipStream_t s) {
    // One block holds 16 waves: beyond 16 tokens the top-k runs as its own launch.
    const bool topk_here = T <= 1024 / kWave;
    if (!topk_here) {
        const hipError_t e = launch_topk(L, logits, ld, T, idx, w, shared_gate, row_w, nullptr, s);
        if (e != hipSuccess) return e;
    }
    decode_route_kernel<<<1, 1024, 0, s>>>(logits, ld, T, L.n_expert, L.k, L.route, L.route_scale, idx,
                                           w, shared_gate, offsets, perm_token, perm_inv, row_w,
                                           L.shared_ff > 0 ? 1 : 0, tile_m, groups, meta, tiles,
                                           grouped_max_mtiles(L.n_expert, T, L.k, L.shared_ff > 0),
                                           topk_here ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_router_logits(const moe_layer& L, const void* x, int T, float* logits, int ld,
                                hipStream_t s, const RouterNorm* norm) {
    return L.dtype == MOE_BF16 ? launch_router_t<BF16>(L, x, T, logits, ld, norm, s)
                               : launch_router_t<F32>(L, x, T, logits, ld, norm, s);
}

bool router_norm_fits(const moe_layer& L) {
    return (size_t)kRouterNT * L.d * (L.dtype == MOE_BF16 ? 2 : 4) <= kRouterNormMaxLds;
}

hipError_t launch_topk(const moe_layer& L, const float* logits, int ld, int T, int32_t* idx,
                       float* w, float* shared_gate, float* row_w, const void* x_sg, hipStream_t s) {
    topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ld, T, L.n_expert, L.k, L.route,
                                             L.route_scale, idx, w, shared_gate, row_w,
                                             static_cast<const uint16_t*>(x_sg),
                                             static_cast<const uint16_t*>(L.ws_gate_inp), L.d);
    return hipGetLastError();
}

}  // namespace smoe

// Expert FFN GEMVs over MXFP4 expert weights (the decode path of a gpt-oss-shaped layer
// stored as its checkpoint stores it).
//
// "Phase 19: MoE - gpt-oss-20b", section 3 and the measured tensor layout: gate_up
// [E, 2ff, d/32, 16] and down [E, d, ff/32, 16] uint8 blocks, each 16-byte block the 32
// FP4 (E2M1) codes of 32 consecutive inputs (low nibble first) sharing one E8M0 scale;
// value = fp4(code) * 2^(scale - 127).  Experts as in section 2: interleaved gate/up
// rows with biases, gate clamped from above, up clamped both ways, (up + 1) * gate *
// sigmoid(alpha * gate), down projection with bias.
//
// The weights are never expanded in memory: each lane loads whole 16-byte blocks plus
// their scale byte (0.53 bytes per weight instead of 2) and gfx950's scaled conversions
// expand them in registers, two codes per instruction, to bf16 pairs that meet the bf16
// activations in v_dot2 (fp32 accumulation).  H rows are stored in bf16 here, as on the
// grouped path.  Lane l takes blocks l, l+64, ... of a row.
#include "gemv_items.h"
#include "mxfp4_dev.h"
#include "route_dev.h"

namespace smoe {
namespace {


// A code word's 8 weights against NT activation rows at once: each converted pair
// serves every row.
template <int NT>
__device__ __forceinline__ void word_dot_bf16_rows(uint32_t cw, float scale, const uint4 (&xw)[NT], float (&acc)[NT]) {
    const bf16x2_t p0 = fp4_pair_bf16<0>(cw, scale), p1 = fp4_pair_bf16<1>(cw, scale);
    const bf16x2_t p2 = fp4_pair_bf16<2>(cw, scale), p3 = fp4_pair_bf16<3>(cw, scale);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float a = acc[t];
        a = __builtin_amdgcn_fdot2_f32_bf16(p0, __builtin_bit_cast(bf16x2_t, xw[t].x), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(p1, __builtin_bit_cast(bf16x2_t, xw[t].y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(p2, __builtin_bit_cast(bf16x2_t, xw[t].z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(p3, __builtin_bit_cast(bf16x2_t, xw[t].w), a, false);
        acc[t] = a;
    }
}

// acc[t] += sum over the block's 32 elements of w * x_t for NT activation rows x_t (each
// 32 bf16 in four 16-byte pieces): every FP4 pair is converted once for all rows.
template <int NT>
__device__ __forceinline__ void block_dot_bf16_rows(const uint4& codes, float scale, const uint4 (&xq)[NT][4],
                                                    float (&acc)[NT]) {
    uint4 xw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) xw[t] = xq[t][0];
    word_dot_bf16_rows<NT>(codes.x, scale, xw, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t) xw[t] = xq[t][1];
    word_dot_bf16_rows<NT>(codes.y, scale, xw, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t) xw[t] = xq[t][2];
    word_dot_bf16_rows<NT>(codes.z, scale, xw, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t) xw[t] = xq[t][3];
    word_dot_bf16_rows<NT>(codes.w, scale, xw, acc);
}

constexpr int kMxUnits = 2;   // hidden units per up wave (4 interleaved rows)
constexpr int kMxUpNT = 2;    // group rows per up step
constexpr int kMxDownNR = 4;  // output dims per down wave
constexpr int kMxDownNT = 2;  // H rows per down step
constexpr int kMxNB = 2;      // blocks per lane and row held at once (K up to 4096)
constexpr int kToken1MxMaxWaves = 16;  // picks per token of the fused one-token kernels

__device__ const uint16_t kZeroBf16 = 0;

struct MxArgs {
    const uint16_t* x;          // [T, d] bf16
    const int32_t* perm_token;
    const Group* groups;
    const uint8_t* w_gate_up;   // blocks [E, 2ff, d/32, 16]
    const uint8_t* s_gate_up;   // [E, 2ff, d/32]
    const uint16_t* b_gate_up;  // [E, 2ff] bf16
    const uint8_t* w_down;      // blocks [E, d, ff/32, 16]
    const uint8_t* s_down;      // [E, d, ff/32]
    const uint16_t* b_down;     // [E, d] bf16 or null
    uint16_t* H;                // bf16 [rows, hstride]
    float* y;
    int hstride, T, tk, d, ff;
    float alpha, limit;
};

// Block i of this lane (block index lane + 64 i) of `rows` weight rows: codes and the raw
// scale byte.  Nothing is done with them here, so that no wait for these loads comes
// before the activation loads are issued; blocks past nblk read block 0 and are given a
// zero scale where they are used (mx_scale).
template <int NR, int NB>
__device__ __forceinline__ void load_mx_rows(const uint8_t* const (&wrow)[NR], const uint8_t* const (&srow)[NR],
                                             int nblk, uint4 (&codes)[NR][NB], uint32_t (&sbyte)[NR][NB]) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int b = lane + kWave * i;
        const int bc = b < nblk ? b : 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            codes[r][i] = ld16(wrow[r] + (size_t)bc * 16);
            sbyte[r][i] = srow[r][bc];
        }
    }
}

// The block's scale, or 0 for a block past the row (its codes were block 0's).
__device__ __forceinline__ float mx_scale(uint32_t sbyte, int b, int nblk) {
    return b < nblk ? e8m0_scale(sbyte) : 0.0f;
}

// One wave: hidden units f0, f0+1 of routed group g (interleaved rows 2f0 .. 2f0+3), every
// row of the group, NT rows per step (1 for a one-token group, whose second row would repeat
// the first).
template <int NB, int NT = kMxUpNT>
__device__ __forceinline__ void mx_up_item(const MxArgs& a, const Group& g, int f0) {
    constexpr int NR = 2 * kMxUnits, N = NR * NT;
    constexpr int SH = 6 - ilog2(N);
    const int nblk = a.d / 32;
    const size_t row_blocks = (size_t)nblk;
    const uint8_t* wrow[NR];
    const uint8_t* srow[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int f = min(f0 + r / 2, a.ff - 1);
        const size_t R = (size_t)g.e * 2 * a.ff + 2 * f + (r & 1);
        wrow[r] = a.w_gate_up + R * row_blocks * 16;
        srow[r] = a.s_gate_up + R * row_blocks;
    }
    const uint8_t* const (&wc)[NR] = wrow;
    const uint8_t* const (&sc)[NR] = srow;
    // Token of each row of a step (unconditional loads: perm_token always holds the group's
    // rows; with one token the row is token 0).  The first step's are loaded before the
    // weights: vector loads complete in issue order, so a token index loaded after the
    // weights could only be used once the weights had arrived.
    // Lane l loads the token of row tb + l % NT: a per-lane load keeps the value in a
    // vector register, read out with readlane only where the activation addresses need it.
    const int lane = lane_id();
    auto step_tokens = [&](int tb) { return a.perm_token[g.row0 + min(tb + (lane & (NT - 1)), g.n - 1)]; };
    const int tok0 = step_tokens(0);
    __builtin_amdgcn_sched_barrier(0);
    uint4 codes[NR][NB];
    uint32_t sbyte[NR][NB];
    load_mx_rows<NR, NB>(wc, sc, nblk, codes, sbyte);
    // After the reduction lane l holds value v = t * NR + r = l >> SH; the up row of gate
    // row r sits one value on, 1 << SH lanes higher (in the same 16-lane row for NT = 2).
    const int my_t = (lane >> SH) / NR, my_r = (lane >> SH) % NR;
    const int my_f = f0 + my_r / 2;
    const bool writer = (my_r & 1) == 0 && (lane & ((1 << SH) - 1)) == 0 && my_f < a.ff;
    // Every lane loads a bias pair (branch-free, clamped): a load behind a branch would make
    // the compiler wait for all loads in flight at the join.
    const uint32_t bpair = *reinterpret_cast<const uint32_t*>(a.b_gate_up + (size_t)g.e * 2 * a.ff +
                                                              2 * min(my_f, a.ff - 1));
    for (int tb = 0; tb < g.n; tb += NT) {
        const int nt = min(NT, g.n - tb);
        float acc[NR][NT] = {};
        const int tok_v = tb == 0 ? tok0 : step_tokens(tb);
        const uint16_t* xr[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int tok = __builtin_amdgcn_readlane(tok_v, t);
            xr[t] = a.x + (size_t)min(max(a.T == 1 ? 0 : tok, 0), a.T - 1) * a.d;
        }
        // All activation loads of the step first; then the codes pass an opaque asm, so
        // that their conversion is neither hoisted out of the loop (which would wait for
        // the weights before the first activation load and hold 4x the registers) nor
        // moved above the activation loads.
        uint4 xq[NB][NT][4];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = lane + kWave * i;
            const int bc = b < nblk ? b : 0;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) xq[i][t][q] = ld16(xr[t] + (size_t)bc * 32 + q * 8);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = lane + kWave * i;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                block_dot_bf16_rows<NT>(opaque(codes[r][i]), mx_scale(sbyte[r][i], b, nblk), xq[i], acc[r]);
        }
        float v[N];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) v[t * NR + r] = acc[r][t];
        const float sum = wave_reduce_scatter<N>(v);
        float up;
        if constexpr (SH < 4)  // inside a 16-lane row: a DPP row shift
            up = __int_as_float(
                __builtin_amdgcn_update_dpp(0, __float_as_int(sum), 0x100 + (1 << SH), 0xF, 0xF, false));
        else
            up = __shfl(sum, (lane + (1 << SH)) & 63, kWave);
        if (writer && my_t < nt) {
            float gv = fminf(sum + bf16_lo(bpair), a.limit);
            float uv = fminf(fmaxf(up + bf16_hi(bpair), -a.limit), a.limit);
            a.H[(size_t)(g.row0 + tb + my_t) * a.hstride + my_f] =
                f32_to_bf16((uv + 1.0f) * gv * sigmoidf_(a.alpha * gv));
        }
    }
}

// One wave: output dims i0 .. i0+NR-1 of routed group g, kMxDownNT H rows per step.
template <int NB>
__device__ __forceinline__ void mx_down_item(const MxArgs& a, const Group& g, int i0) {
    constexpr int NR = kMxDownNR, NT = kMxDownNT, N = NR * NT;
    constexpr int SH = 6 - ilog2(N);
    const int nblk = a.ff / 32;
    const uint8_t* wrow[NR];
    const uint8_t* srow[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const size_t R = (size_t)g.e * a.d + min(i0 + r, a.d - 1);
        wrow[r] = a.w_down + R * nblk * 16;
        srow[r] = a.s_down + R * nblk;
    }
    const uint8_t* const (&wc)[NR] = wrow;
    const uint8_t* const (&sc)[NR] = srow;
    uint4 codes[NR][NB];
    uint32_t sbyte[NR][NB];
    load_mx_rows<NR, NB>(wc, sc, nblk, codes, sbyte);
    // After the reduction lane l holds value v = t * NR + r = l >> SH.
    const int lane = lane_id();
    const int my_t = (lane >> SH) / NR, my_i = i0 + (lane >> SH) % NR;
    const bool writer = (lane & ((1 << SH) - 1)) == 0 && my_i < a.d;
    // Branch-free bias load (see mx_up_item); a layer without down bias reads a zero.
    const uint16_t* bd = a.b_down ? a.b_down + (size_t)g.e * a.d + min(my_i, a.d - 1) : &kZeroBf16;
    const float bias = bf16_to_f32(*bd);
    for (int tb = 0; tb < g.n; tb += NT) {
        const int nt = min(NT, g.n - tb);
        float acc[NR][NT] = {};
        const uint16_t* hr[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) hr[t] = a.H + (size_t)(g.row0 + min(tb + t, g.n - 1)) * a.hstride;
        // As in mx_up_item: the step's H loads first, then the codes through an opaque asm.
        uint4 hq[NB][NT][4];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = lane + kWave * i;
            const int bc = b < nblk ? b : 0;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) hq[i][t][q] = ld16(hr[t] + (size_t)bc * 32 + q * 8);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = lane + kWave * i;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                block_dot_bf16_rows<NT>(opaque(codes[r][i]), mx_scale(sbyte[r][i], b, nblk), hq[i], acc[r]);
        }
        float v[N];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) v[t * NR + r] = acc[r][t];
        const float sum = wave_reduce_scatter<N>(v);
        if (writer && my_t < nt) a.y[(size_t)(g.row0 + tb + my_t) * a.d + my_i] = sum + bias;
    }
}

// Grid row y takes routed group y (there is no shared expert with MXFP4 experts).
__device__ __forceinline__ bool mx_group(const MxArgs& a, const PlanMeta* meta, Group& g) {
    return gemv_group(a.groups, meta, false, a.T, a.tk, 0, g);
}

template <int NB>
__global__ __launch_bounds__(256) void expert_up_gemv_mx_kernel(MxArgs a, const PlanMeta* meta) {
    Group g;
    if (!mx_group(a, meta, g)) return;
    const int f0 = (blockIdx.x * 4 + wave_id()) * kMxUnits;
    if (f0 < a.ff) mx_up_item<NB>(a, g, f0);
}

template <int NB>
__global__ __launch_bounds__(256) void expert_down_gemv_mx_kernel(MxArgs a, const PlanMeta* meta) {
    Group g;
    if (!mx_group(a, meta, g)) return;
    const int i0 = (blockIdx.x * 4 + wave_id()) * kMxDownNR;
    if (i0 < a.d) mx_down_item<NB>(a, g, i0);
}

// Token index of every hidden row of a one-token batch (hidden row j = pick j).
__device__ const int32_t kTokenZero[kToken1MxMaxWaves] = {};

// One token: the top-k and the up projection in one kernel.  Grid row j: every wave runs
// the token's top-k on the router logits and takes pick j (hidden row j); block 0 of the
// row records the pick for the down kernel.  No planning or grouping launch.
template <int NB>
__global__ __launch_bounds__(256) void token1_up_mx_kernel(MxArgs a, const float* __restrict__ logits, int E,
                                                           int k, int mode, float scale,
                                                           int32_t* __restrict__ idx, float* __restrict__ w) {
    const int j = blockIdx.y;
    const int f0 = (blockIdx.x * 4 + wave_id()) * kMxUnits;
    if (f0 >= a.ff) return;  // never block 0's first wave, which records the pick
    int my_i;
    float my_w;
    topk_wave(logits, E, k, mode, scale, &my_i, &my_w);
    if (blockIdx.x == 0 && wave_id() == 0 && lane_id() == j) {
        idx[j] = my_i;
        w[j] = my_w;
    }
    const int e = __builtin_amdgcn_readlane(my_i, j);
    MxArgs b = a;
    b.perm_token = kTokenZero;
    mx_up_item<NB, 1>(b, Group{min(max(e, 0), E - 1), j, 1, 0}, f0);
}

// A few tokens: the down projection of every pick (MXFP4 W_d) and the weighted combine
// in one kernel, as token1_down_combine_kernel does for dense experts.  Block (b, t) owns
// output dims i0 = 4b .. i0+3 of token t; wave j takes pick j (expert idx[t*k+j], weight
// w[t*k+j], bf16 hidden row perm_inv[t*k+j], or row j for one token without perm_inv) and
// leaves its 4 sums (+ down bias) in LDS; 4 threads then add them in pick order.
template <int NB>
__global__ __launch_bounds__(kToken1MxMaxWaves * kWave) void token_down_combine_mx_kernel(
    MxArgs a, const int32_t* __restrict__ idx, const float* __restrict__ w, const int32_t* __restrict__ perm_inv,
    int E, int k, const uint16_t* __restrict__ residual, uint16_t* __restrict__ y) {
    constexpr int NR = kMxDownNR, SH = 6 - ilog2(NR);
    __shared__ float part[kToken1MxMaxWaves][NR];
    __shared__ float wts[kToken1MxMaxWaves];
    const int j = wave_id(), lane = lane_id();
    const int i0 = blockIdx.x * NR, t = blockIdx.y;
    // A pick without a valid hidden row contributes nothing (its weight is zero).
    const int p = t * k + j;
    const int ei = idx[p], r = perm_inv ? perm_inv[p] : j;
    const bool ok = ei >= 0 && ei < E && r >= 0 && r < a.tk;
    const int e = ok ? ei : 0, row = ok ? r : 0;
    const float weight = ok ? w[p] : 0.0f;
    const int nblk = a.ff / 32;
    const uint8_t* wrow[NR];
    const uint8_t* srow[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
        const size_t R = (size_t)e * a.d + min(i0 + q, a.d - 1);
        wrow[q] = a.w_down + R * nblk * 16;
        srow[q] = a.s_down + R * nblk;
    }
    const uint8_t* const (&wc)[NR] = wrow;
    const uint8_t* const (&sc)[NR] = srow;
    uint4 codes[NR][NB];
    uint32_t sbyte[NR][NB];
    load_mx_rows<NR, NB>(wc, sc, nblk, codes, sbyte);
    const int my_r = lane >> SH;
    const uint16_t* bd = a.b_down ? a.b_down + (size_t)e * a.d + min(i0 + my_r, a.d - 1) : &kZeroBf16;
    const float bias = bf16_to_f32(*bd);
    const uint16_t* hr = a.H + (size_t)row * a.hstride;
    uint4 hq[NB][1][4];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int b = lane + kWave * i;
        const int bc = b < nblk ? b : 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) hq[i][0][q] = ld16(hr + (size_t)bc * 32 + q * 8);
    }
    float acc[NR][1] = {};
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int b = lane + kWave * i;
#pragma unroll
        for (int q = 0; q < NR; ++q)
            block_dot_bf16_rows<1>(opaque(codes[q][i]), mx_scale(sbyte[q][i], b, nblk), hq[i], acc[q]);
    }
    float v[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) v[q] = acc[q][0];
    const float sum = wave_reduce_scatter<NR>(v);
    if ((lane & ((1 << SH) - 1)) == 0) part[j][my_r] = sum + bias;
    if (lane == 0) wts[j] = weight;
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < NR && i0 + tid < a.d) {
        float o = 0.0f;
        for (int jj = 0; jj < k; ++jj) o = fmaf(wts[jj], part[jj][tid], o);
        const size_t at = (size_t)t * a.d + i0 + tid;
        if (residual) o += bf16_to_f32(residual[at]);  // read before y is written: y may alias it
        y[at] = f32_to_bf16(o);
    }
}

int blocks_per_lane(int K) { return (K / 32 + kWave - 1) / kWave; }

MxArgs mx_args(const moe_layer& L, const void* x, int T, const int32_t* perm_token, const Group* groups, float* H,
               int hstride, float* y_perm) {
    return MxArgs{static_cast<const uint16_t*>(x), perm_token, groups,
                  static_cast<const uint8_t*>(L.w_gate_up), L.w_gate_up_scales, static_cast<const uint16_t*>(L.b_gate_up),
                  static_cast<const uint8_t*>(L.w_down), L.w_down_scales, static_cast<const uint16_t*>(L.b_down),
                  reinterpret_cast<uint16_t*>(H), y_perm, hstride, T, T * L.k, L.d, L.ff, L.oai_alpha, L.oai_limit};
}

}  // namespace

bool mx_fits(const moe_layer& L) {
    return blocks_per_lane(L.d) <= kMxNB && blocks_per_lane(L.ff) <= kMxNB && L.d % 32 == 0 && L.ff % 32 == 0;
}

hipError_t launch_expert_gemv_mx(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                 const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                                 hipStream_t s) {
    if (!mx_fits(L)) return hipErrorInvalidValue;
    const hipError_t e = launch_expert_up_gemv_mx(L, x, T, perm_token, groups, meta, H, hstride, s);
    if (e != hipSuccess) return e;
    const MxArgs a = mx_args(L, x, T, perm_token, groups, H, hstride, y_perm);
    const int gmax = max_groups(L.n_expert, T, L.k, false);
    const dim3 gd((L.d + 4 * kMxDownNR - 1) / (4 * kMxDownNR), gmax);
    if (blocks_per_lane(L.ff) == 1) expert_down_gemv_mx_kernel<1><<<gd, 256, 0, s>>>(a, meta);
    else expert_down_gemv_mx_kernel<2><<<gd, 256, 0, s>>>(a, meta);
    return hipGetLastError();
}

hipError_t launch_expert_up_gemv_mx(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                    const Group* groups, const PlanMeta* meta, float* H, int hstride,
                                    hipStream_t s) {
    if (!mx_fits(L)) return hipErrorInvalidValue;
    const MxArgs a = mx_args(L, x, T, perm_token, groups, H, hstride, nullptr);
    const int gmax = max_groups(L.n_expert, T, L.k, false);
    const dim3 gu((L.ff + 4 * kMxUnits - 1) / (4 * kMxUnits), gmax);
    if (blocks_per_lane(L.d) == 1) expert_up_gemv_mx_kernel<1><<<gu, 256, 0, s>>>(a, meta);
    else expert_up_gemv_mx_kernel<2><<<gu, 256, 0, s>>>(a, meta);
    return hipGetLastError();
}

bool token1_mx_fits(const moe_layer& L) {
    return L.expert_format == MOE_EXPERTS_MXFP4 && mx_fits(L) && L.k <= kToken1MxMaxWaves && L.shared_ff == 0;
}

hipError_t launch_token1_up_mx(const moe_layer& L, const void* x, const float* logits, int32_t* idx, float* w,
                               float* H, int hstride, hipStream_t s) {
    if (!token1_mx_fits(L)) return hipErrorInvalidValue;
    const MxArgs a = mx_args(L, x, 1, nullptr, nullptr, H, hstride, nullptr);
    const dim3 gu((L.ff + 4 * kMxUnits - 1) / (4 * kMxUnits), L.k);
    if (blocks_per_lane(L.d) == 1)
        token1_up_mx_kernel<1><<<gu, 256, 0, s>>>(a, logits, L.n_expert, L.k, L.route, L.route_scale, idx, w);
    else
        token1_up_mx_kernel<2><<<gu, 256, 0, s>>>(a, logits, L.n_expert, L.k, L.route, L.route_scale, idx, w);
    return hipGetLastError();
}

hipError_t launch_token_down_combine_mx(const moe_layer& L, int T, const float* H, int hstride, const int32_t* idx,
                                        const float* w, const int32_t* perm_inv, const void* residual, void* y,
                                        hipStream_t s) {
    if (!token1_mx_fits(L) || T < 1 || (!perm_inv && T != 1)) return hipErrorInvalidValue;
    const MxArgs a = mx_args(L, nullptr, T, nullptr, nullptr, const_cast<float*>(H), hstride, nullptr);
    const dim3 grid((L.d + kMxDownNR - 1) / kMxDownNR, T);
    const dim3 block(L.k * kWave);
    const auto* ro = static_cast<const uint16_t*>(residual);
    auto* yo = static_cast<uint16_t*>(y);
    if (blocks_per_lane(L.ff) == 1)
        token_down_combine_mx_kernel<1><<<grid, block, 0, s>>>(a, idx, w, perm_inv, L.n_expert, L.k, ro, yo);
    else
        token_down_combine_mx_kernel<2><<<grid, block, 0, s>>>(a, idx, w, perm_inv, L.n_expert, L.k, ro, yo);
    return hipGetLastError();
}

}  // namespace smoe

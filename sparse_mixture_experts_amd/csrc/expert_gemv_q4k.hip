// Expert FFN GEMVs over Q4_K expert weights (the decode path of a SwiGLU layer whose
// routed experts are stored as GGUF K-quant blocks; block layout in q4k_dev.h).
//
// "Qwen3.5-MoE Model Implementation", MoE routing: each routed expert is a SwiGLU,
// silu(gate . x) * (up . x) then down.  The weights are never expanded in memory: a lane
// takes 64-weight units of a row (one 32-byte quant run of a super-block plus the block's
// 16-byte header), 0.56 bytes per weight.  With U = K / 64 units per row, LPR lanes (U
// rounded up to a power of two, at most 64) share a row and a wave covers 64 / LPR rows
// at once, so short rows still occupy every lane.
//
// Up: the quants become bf16 pairs 128 + q (exact), which meet the bf16 activations in
// v_dot2 (fp32 accumulation); per sub-block, sum q x = dot - 128 sum x, and the unit's
// contribution is d sc (sum q x) - dmin m (sum x) for each of its two sub-blocks.  Down:
// H is fp32 on this path, so the quants are widened to fp32 and meet H in FMAs.  Each
// row's LPR partial sums meet in a butterfly over the LPR lanes.  The shared expert (bf16)
// runs on the dense GEMV kernels.
#include "internal.h"
#include "q4k_dev.h"

namespace smoe {
namespace {

struct Q4kArgs {
    const uint16_t* x;          // [T, d] bf16
    const int32_t* perm_token;  // token of each grouped row
    const Group* groups;
    const PlanMeta* meta;
    const uint8_t* w_gate;      // [E, ff, d/256, 144]
    const uint8_t* w_up;
    const uint8_t* w_down;      // [E, d, ff/256, 144]
    float* H;                   // fp32 [rows, hstride]
    float* y;                   // fp32 [rows, d]
    int hstride, T, tk, d, ff, has_shared;
};

// Routed group of grid row blockIdx.y (the shared expert, last in the list, is not taken
// here).  The entry and the count are loaded before the count is checked.
__device__ __forceinline__ bool q4k_group(const Q4kArgs& a, Group& g) {
    const int gi = blockIdx.y;
    const Group cand = a.groups[gi];
    const int n_groups = a.meta->n_groups;
    asm volatile("" ::"s"(cand.e), "s"(cand.row0), "s"(cand.n), "s"(n_groups));
    if (gi >= n_groups - a.has_shared) return false;
    g = cand;
    return true;
}

// Sum over each group of LPR consecutive lanes (every lane of the group gets the total).
template <int LPR>
__device__ __forceinline__ float segment_sum(float v) {
    if constexpr (LPR > 1) v = butterfly_full<0>(v);
    if constexpr (LPR > 2) v = butterfly_full<1>(v);
    if constexpr (LPR > 4) v = butterfly_full<2>(v);
    if constexpr (LPR > 8) v = butterfly_full<3>(v);
    if constexpr (LPR > 16) v = butterfly_full<4>(v);
    if constexpr (LPR > 32) v = butterfly_full<5>(v);
    return v;
}

// One unit (64 weights) of a row: the header and the 32-byte quant run.
struct Q4kUnit {
    uint4 head, q0, q1;
};

__device__ __forceinline__ Q4kUnit load_unit(const uint8_t* row, int unit) {
    const uint8_t* blk = row + (size_t)(unit >> 2) * kQ4kBlockBytes;
    const uint8_t* run = blk + 16 + 32 * (unit & 3);
    return Q4kUnit{ld16(blk), ld16(run), ld16(run + 16)};
}

__device__ __forceinline__ uint32_t word_of(const Q4kUnit& u, int i) {
    const uint4& q = i < 4 ? u.q0 : u.q1;
    const int k = i & 3;
    return k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
}

__device__ __forceinline__ uint32_t word4(const uint4& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// sum over the sub-block half H (0: weights 0..31 of the unit, 1: 32..63) of (128 + q) x,
// x given as 4 16-byte pieces of 8 bf16.
template <int H>
__device__ __forceinline__ float q_dot_half(const Q4kUnit& u, const uint4 (&xs)[4]) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t w = word_of(u, i);
        const uint4& xv = xs[i >> 1];
        const uint32_t x01 = (i & 1) ? xv.z : xv.x, x23 = (i & 1) ? xv.w : xv.y;
        acc = __builtin_amdgcn_fdot2_f32_bf16(q4k_pair<0, H>(w), __builtin_bit_cast(q4k_bf16x2_t, x01), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(q4k_pair<1, H>(w), __builtin_bit_cast(q4k_bf16x2_t, x23), acc, false);
    }
    return acc;
}

__device__ __forceinline__ float bf16_sum(const uint4 (&xs)[4]) {
    const q4k_bf16x2_t one = __builtin_bit_cast(q4k_bf16x2_t, 0x3F803F80u);
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(q4k_bf16x2_t, word4(xs[k], c)), one, acc, false);
    return acc;
}

template <int LPR>
struct Lanes {
    static constexpr int P = 64 / LPR;             // rows a wave covers at once
    static constexpr int NR = P > 4 ? P : 4;       // rows per wave
    static constexpr int NP = NR / P;              // passes
};

// One wave: hidden units f0 .. f0 + NR/2 - 1 of routed group g.  Row r of the wave is the
// gate (r even) or up (r odd) row of unit f0 + r / 2; in pass p, lane l serves row
// p * P + l / LPR, unit l % LPR.  NT group rows per step.
template <int LPR, int NT>
__device__ __forceinline__ void q4k_up_item(const Q4kArgs& a, const Group& g, int f0) {
    using LN = Lanes<LPR>;
    constexpr int P = LN::P, NP = LN::NP;
    const int lane = lane_id();
    const int sr = lane / LPR, ul = lane % LPR;
    const int units = a.d / 64;
    const bool active = ul < units;
    const int uc = active ? ul : 0;
    const int nsb = a.d / kQ4kBlockWeights;
    Q4kUnit w[NP];
    float sa[NP], ma[NP], sb[NP], mb[NP];
    int row_f[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = p * P + sr;
        const int f = min(f0 + r / 2, a.ff - 1);
        row_f[p] = f0 + r / 2;
        const uint8_t* base = (r & 1) ? a.w_up : a.w_gate;
        w[p] = load_unit(base + ((size_t)g.e * a.ff + f) * nsb * kQ4kBlockBytes, uc);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int c = uc & 3;
        q4k_sub_scale(w[p].head, 2 * c, sa[p], ma[p]);
        q4k_sub_scale(w[p].head, 2 * c + 1, sb[p], mb[p]);
    }
    for (int tb = 0; tb < g.n; tb += NT) {
        const int nt = min(NT, g.n - tb);
        uint4 xa[NT][4], xb[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int row = g.row0 + min(tb + t, g.n - 1);
            int tok = a.T == 1 ? 0 : a.perm_token[row];
            tok = min(max(tok, 0), a.T - 1);
            const uint16_t* xr = a.x + (size_t)tok * a.d + 64 * uc;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                xa[t][k] = ld16(xr + 8 * k);
                xb[t][k] = ld16(xr + 32 + 8 * k);
            }
        }
        float acc[NP][NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float sxa = bf16_sum(xa[t]), sxb = bf16_sum(xb[t]);
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float da = q_dot_half<0>(w[p], xa[t]), db = q_dot_half<1>(w[p], xb[t]);
                float v = sa[p] * da + sb[p] * db - (128.0f * sa[p] + ma[p]) * sxa - (128.0f * sb[p] + mb[p]) * sxb;
                acc[p][t] = active ? v : 0.0f;
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[p][t] = segment_sum<LPR>(acc[p][t]);
        // Gate of unit u and its up row: with P >= 2 the up row is the next sub-row (LPR
        // lanes on); with P == 1 it is the next pass, in the same lane.
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float gate = acc[p][t], up;
                bool writer;
                int f;
                if constexpr (P >= 2) {
                    up = __shfl(gate, (lane + LPR) & 63, kWave);
                    writer = ul == 0 && (sr & 1) == 0;
                    f = row_f[p];
                } else {
                    if (p & 1) continue;
                    up = acc[p + 1][t];
                    writer = lane == 0;
                    f = row_f[p];
                }
                if (writer && t < nt && f < a.ff)
                    a.H[(size_t)(g.row0 + tb + t) * a.hstride + f] = gate * sigmoidf_(gate) * up;
            }
        }
    }
}

// One wave: output dims i0 .. i0 + NR - 1 of routed group g (row r = dim i0 + r), NT H
// rows per step.
template <int LPR, int NT>
__device__ __forceinline__ void q4k_down_item(const Q4kArgs& a, const Group& g, int i0) {
    using LN = Lanes<LPR>;
    constexpr int P = LN::P, NP = LN::NP;
    const int lane = lane_id();
    const int sr = lane / LPR, ul = lane % LPR;
    const int units = a.ff / 64;
    const bool active = ul < units;
    const int uc = active ? ul : 0;
    const int nsb = a.ff / kQ4kBlockWeights;
    Q4kUnit w[NP];
    float sa[NP], ma[NP], sb[NP], mb[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int i = min(i0 + p * P + sr, a.d - 1);
        w[p] = load_unit(a.w_down + ((size_t)g.e * a.d + i) * nsb * kQ4kBlockBytes, uc);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int c = uc & 3;
        q4k_sub_scale(w[p].head, 2 * c, sa[p], ma[p]);
        q4k_sub_scale(w[p].head, 2 * c + 1, sb[p], mb[p]);
    }
    for (int tb = 0; tb < g.n; tb += NT) {
        const int nt = min(NT, g.n - tb);
        float4 ha[NT][8], hb[NT][8];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float* hr = a.H + (size_t)(g.row0 + min(tb + t, g.n - 1)) * a.hstride + 64 * uc;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                ha[t][k] = *reinterpret_cast<const float4*>(hr + 4 * k);
                hb[t][k] = *reinterpret_cast<const float4*>(hr + 32 + 4 * k);
            }
        }
        float acc[NP][NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float sha = 0.0f, shb = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sha += (ha[t][k].x + ha[t][k].y) + (ha[t][k].z + ha[t][k].w);
                shb += (hb[t][k].x + hb[t][k].y) + (hb[t][k].z + hb[t][k].w);
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float da = 0.0f, db = 0.0f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t wd = word_of(w[p], k);
                    const uint32_t lo = wd & 0x0F0F0F0Fu, hi = (wd >> 4) & 0x0F0F0F0Fu;
                    da = fmaf((float)(lo & 0xFFu), ha[t][k].x, da);
                    da = fmaf((float)((lo >> 8) & 0xFFu), ha[t][k].y, da);
                    da = fmaf((float)((lo >> 16) & 0xFFu), ha[t][k].z, da);
                    da = fmaf((float)(lo >> 24), ha[t][k].w, da);
                    db = fmaf((float)(hi & 0xFFu), hb[t][k].x, db);
                    db = fmaf((float)((hi >> 8) & 0xFFu), hb[t][k].y, db);
                    db = fmaf((float)((hi >> 16) & 0xFFu), hb[t][k].z, db);
                    db = fmaf((float)(hi >> 24), hb[t][k].w, db);
                }
                const float v = sa[p] * da - ma[p] * sha + sb[p] * db - mb[p] * shb;
                acc[p][t] = active ? v : 0.0f;
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float s = segment_sum<LPR>(acc[p][t]);
                const int i = i0 + p * P + sr;
                if (ul == 0 && t < nt && i < a.d) a.y[(size_t)(g.row0 + tb + t) * a.d + i] = s;
            }
    }
}

template <int LPR, int NT>
__global__ __launch_bounds__(256) void expert_up_gemv_q4k_kernel(Q4kArgs a) {
    Group g;
    if (!q4k_group(a, g)) return;
    const int f0 = (blockIdx.x * 4 + wave_id()) * (Lanes<LPR>::NR / 2);
    if (f0 < a.ff) q4k_up_item<LPR, NT>(a, g, f0);
}

template <int LPR, int NT>
__global__ __launch_bounds__(256) void expert_down_gemv_q4k_kernel(Q4kArgs a) {
    Group g;
    if (!q4k_group(a, g)) return;
    const int i0 = (blockIdx.x * 4 + wave_id()) * Lanes<LPR>::NR;
    if (i0 < a.d) q4k_down_item<LPR, NT>(a, g, i0);
}

// Lanes per row for a K axis: K / 64 units rounded up to a power of two (K <= 4096).
int lanes_per_row(int K) {
    const int u = K / 64;
    int l = 4;
    while (l < u) l *= 2;
    return l;
}

template <int NT>
hipError_t launch_q4k_t(const Q4kArgs& a, int gmax, hipStream_t s) {
#define SMOE_Q4K_UP(LPR)                                                                                  \
    case LPR: {                                                                                           \
        const dim3 g((a.ff + 4 * (Lanes<LPR>::NR / 2) - 1) / (4 * (Lanes<LPR>::NR / 2)), gmax);          \
        expert_up_gemv_q4k_kernel<LPR, NT><<<g, 256, 0, s>>>(a);                                          \
        break;                                                                                            \
    }
    switch (lanes_per_row(a.d)) {
        SMOE_Q4K_UP(4)
        SMOE_Q4K_UP(8)
        SMOE_Q4K_UP(16)
        SMOE_Q4K_UP(32)
        SMOE_Q4K_UP(64)
        default:
            return hipErrorInvalidValue;
    }
#undef SMOE_Q4K_UP
    return hipGetLastError();
}

template <int NT>
hipError_t launch_q4k_down_t(const Q4kArgs& a, int gmax, hipStream_t s) {
#define SMOE_Q4K_DOWN(LPR)                                                                                \
    case LPR: {                                                                                           \
        const dim3 g((a.d + 4 * Lanes<LPR>::NR - 1) / (4 * Lanes<LPR>::NR), gmax);                        \
        expert_down_gemv_q4k_kernel<LPR, NT><<<g, 256, 0, s>>>(a);                                        \
        break;                                                                                            \
    }
    switch (lanes_per_row(a.ff)) {
        SMOE_Q4K_DOWN(4)
        SMOE_Q4K_DOWN(8)
        SMOE_Q4K_DOWN(16)
        SMOE_Q4K_DOWN(32)
        SMOE_Q4K_DOWN(64)
        default:
            return hipErrorInvalidValue;
    }
#undef SMOE_Q4K_DOWN
    return hipGetLastError();
}

}  // namespace

bool q4k_fits(const moe_layer& L) {
    return L.d % kQ4kBlockWeights == 0 && L.ff % kQ4kBlockWeights == 0 && L.d <= 4096 && L.ff <= 4096;
}

hipError_t launch_expert_gemv_q4k(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                  const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                                  hipStream_t s) {
    if (!q4k_fits(L)) return hipErrorInvalidValue;
    const bool shared = L.shared_ff > 0;
    const Q4kArgs a{static_cast<const uint16_t*>(x), perm_token, groups, meta,
                    static_cast<const uint8_t*>(L.w_gate), static_cast<const uint8_t*>(L.w_up),
                    static_cast<const uint8_t*>(L.w_down), H, y_perm, hstride, T, T * L.k, L.d, L.ff,
                    shared ? 1 : 0};
    const int routed = max_groups(L.n_expert, T, L.k, false);
    hipError_t e = T == 1 ? launch_q4k_t<1>(a, routed, s) : launch_q4k_t<2>(a, routed, s);
    if (e != hipSuccess) return e;
    if (shared && (e = launch_shared_gemv_up(L, x, T, groups, meta, H, hstride, s)) != hipSuccess) return e;
    e = T == 1 ? launch_q4k_down_t<1>(a, routed, s) : launch_q4k_down_t<2>(a, routed, s);
    if (e != hipSuccess) return e;
    if (shared) return launch_shared_gemv_down(L, T, groups, meta, H, hstride, y_perm, s);
    return hipSuccess;
}

}  // namespace smoe

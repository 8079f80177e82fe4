// Expert FFN GEMVs over Q4_K expert weights (the decode path of a SwiGLU layer whose
// routed experts are stored as GGUF K-quant blocks; block layout in q4k_dev.h).
//
// "Qwen3.5-MoE Model Implementation", MoE routing: each routed expert is a SwiGLU,
// silu(gate . x) * (up . x) then down.  The weights are never expanded in memory: a lane
// takes 64-weight units of a row (one 32-byte quant run of a super-block plus the block's
// 16-byte header), 0.56 bytes per weight.  With U = K / 64 units per row, LPR lanes (U
// rounded up to a power of two, at most 64) share a row and a wave covers P = 64 / LPR
// rows at once, in NP passes.
//
// A block (4 waves) serves one group.  Each wave loads its rows' units once and turns the
// quants into bf16 pairs 128 + q (exact), kept in registers for every row of the group.
// The block stages the group's activations in LDS as bf16, up to 4 rows at a time (x for
// the up kernel; for the down kernel H, fp32 in memory, rounded to bf16 as on the grouped
// path), so the waves read them from LDS rather than each from the L2.  Per row a lane
// dots its unit with the activations in v_dot2 (fp32 accumulation); per sub-block,
// sum q x = dot - 128 sum x, and the unit's contribution is d sc (sum q x) - dmin m (sum x)
// for each of its two sub-blocks.  Each weight row's LPR partial sums meet in a butterfly
// over its LPR lanes.
//
// A bf16 shared expert as wide as the routed experts runs in the same launches: its units
// are the 64 weights themselves as bf16 pairs, with multiplier 1 and offset term 0, and the
// first grid rows take it in chunks of kQ4kSharedRows tokens (the other rows the routed
// groups), so its longer blocks start first.  A shared expert of another width runs on the
// dense GEMV kernels.
#include "gemv_items.h"
#include "q4k_dev.h"
#include "route_dev.h"
#include "rowdot.h"

namespace smoe {
namespace {

constexpr int kQ4kStepRows = 4;     // activation rows staged in LDS per step (T > 1)
constexpr int kQ4kSharedRows = 16;  // tokens per grid row of a fused shared expert

struct Q4kArgs {
    const uint16_t* x;          // [T, d] bf16
    const int32_t* perm_token;  // token of each grouped row
    const Group* groups;
    const PlanMeta* meta;
    const uint8_t* w_gate;      // [E, ff, d/256, 144]
    const uint8_t* w_up;
    const uint8_t* w_down;      // [E, d, ff/256, 144]
    const uint16_t* ws_gate;    // shared expert, bf16 [ff, d] (fuse_shared)
    const uint16_t* ws_up;
    const uint16_t* ws_down;    // bf16 [d, ff]
    float* H;                   // fp32 [rows, hstride]
    float* y;                   // fp32 [rows, d]
    int hstride, T, tk, d, ff, has_shared, fuse_shared;
};

// Group of grid row blockIdx.y.  With fuse_shared the first grid rows take the shared
// expert in chunks (gemv_group); otherwise the shared expert, last in the list, is not
// taken here.  The entry and the count are loaded before the count is checked.
__device__ __forceinline__ bool q4k_group(const Q4kArgs& a, Group& g) {
    if (a.fuse_shared) return gemv_group(a.groups, a.meta, true, a.T, a.tk, kQ4kSharedRows, g);
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

__device__ __forceinline__ uint32_t word4(const uint4& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// One unit of a row, decoded: lo[j] / hi[j] hold weights 2j, 2j+1 of the unit's first /
// second sub-block as bf16 pairs 128 + q; sa, ma / sb, mb are d sc and dmin m of the two.
struct Q4kDec {
    uint32_t lo[16], hi[16];
    float sa, ma, sb, mb;
};

__device__ __forceinline__ void load_unit(const uint8_t* row, int unit, uint4& head, uint4& q0, uint4& q1) {
    const uint8_t* blk = row + (size_t)(unit >> 2) * kQ4kBlockBytes;
    const uint8_t* run = blk + 16 + 32 * (unit & 3);
    head = ld16(blk);
    q0 = ld16(run);
    q1 = ld16(run + 16);
}

// Byte l of the run holds weight l (low nibble) and 32 + l (high nibble): word i of the
// run gives weights 4i .. 4i+3 of both sub-blocks.
__device__ __forceinline__ void decode_unit(int unit, const uint4& head, const uint4& q0, const uint4& q1,
                                            Q4kDec& u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t w = word4(i < 4 ? q0 : q1, i & 3);
        u.lo[2 * i] = __builtin_bit_cast(uint32_t, q4k_pair<0, 0>(w));
        u.lo[2 * i + 1] = __builtin_bit_cast(uint32_t, q4k_pair<1, 0>(w));
        u.hi[2 * i] = __builtin_bit_cast(uint32_t, q4k_pair<0, 1>(w));
        u.hi[2 * i + 1] = __builtin_bit_cast(uint32_t, q4k_pair<1, 1>(w));
    }
    const int c = unit & 3;
    q4k_sub_scale(head, 2 * c, u.sa, u.ma);
    q4k_sub_scale(head, 2 * c + 1, u.sb, u.mb);
}

// A unit of a bf16 row (the shared expert): lo / hi take the 64 weights as they are, with
// multiplier 1 and offset 128 * 1 - 128 = 0, so unit_dot gives the plain dot product.
__device__ __forceinline__ void load_bf16_unit(const uint16_t* row, int unit, Q4kDec& u) {
    const uint16_t* p = row + 64 * unit;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint4 a = ld16(p + 8 * c), b = ld16(p + 32 + 8 * c);
        u.lo[4 * c] = a.x;
        u.lo[4 * c + 1] = a.y;
        u.lo[4 * c + 2] = a.z;
        u.lo[4 * c + 3] = a.w;
        u.hi[4 * c] = b.x;
        u.hi[4 * c + 1] = b.y;
        u.hi[4 * c + 2] = b.z;
        u.hi[4 * c + 3] = b.w;
    }
    u.sa = 1.0f;
    u.sb = 1.0f;
    u.ma = -128.0f;
    u.mb = -128.0f;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(q4k_bf16x2_t, a), __builtin_bit_cast(q4k_bf16x2_t, b),
                                           acc, false);
}

// One unit's 64 activations as bf16 pairs: xa (elements 0..31), xb (32..63), and the sums
// of each half.
struct Q4kAct {
    uint32_t xa[16], xb[16];
    float sxa, sxb;
};

// LDS layout of a staged activation row: unit u's 16-byte chunk c sits at chunk position
// c ^ (u & 7) of the unit's 128 bytes, so that the LPR lanes of a row (units 128 bytes
// apart) read different banks.
__device__ __forceinline__ int act_chunk(int u, int c) { return u * 8 + (c ^ (u & 7)); }

// LDS bytes of nt staged rows of K activations.
constexpr size_t q4k_stage_bytes(int K, int nt) { return (size_t)nt * (size_t)K * 2; }

// The unit's activations and the sums of its two halves (each lane adds its own: sums
// staged once per row by one thread per sub-block ran slower, the staging being what the
// kernels wait on).
__device__ __forceinline__ void read_act(const uint4* row, int unit, Q4kAct& x) {
    const uint32_t one = 0x3F803F80u;  // bf16 pair (1, 1)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint4 v = row[act_chunk(unit, c)];
        uint32_t* dst = c < 4 ? x.xa : x.xb;
        const int o = 4 * (c & 3);
        dst[o] = v.x;
        dst[o + 1] = v.y;
        dst[o + 2] = v.z;
        dst[o + 3] = v.w;
    }
    x.sxa = 0.0f;
    x.sxb = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        x.sxa = dot2(x.xa[j], one, x.sxa);
        x.sxb = dot2(x.xb[j], one, x.sxb);
    }
}

// The unit's contribution to its row's dot product.
__device__ __forceinline__ float unit_dot(const Q4kDec& u, const Q4kAct& x) {
    float da = 0.0f, db = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        da = dot2(u.lo[j], x.xa[j], da);
        db = dot2(u.hi[j], x.xb[j], db);
    }
    return u.sa * da + u.sb * db - (128.0f * u.sa + u.ma) * x.sxa - (128.0f * u.sb + u.mb) * x.sxb;
}

// 8 fp32 values as a 16-byte chunk of bf16 (rounded to nearest even).
__device__ __forceinline__ uint4 bf16_chunk(const float* src) {
    const float4 f0 = *reinterpret_cast<const float4*>(src);
    const float4 f1 = *reinterpret_cast<const float4*>(src + 4);
    q4k_bf16x2_t p0, p1, p2, p3;
    p0[0] = (__bf16)f0.x;
    p0[1] = (__bf16)f0.y;
    p1[0] = (__bf16)f0.z;
    p1[1] = (__bf16)f0.w;
    p2[0] = (__bf16)f1.x;
    p2[1] = (__bf16)f1.y;
    p3[0] = (__bf16)f1.z;
    p3[1] = (__bf16)f1.w;
    return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                      __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

// Stage group rows tb .. tb+nt-1 in LDS as bf16 rows of K (layout act_chunk): x rows
// (bf16, by token; the shared expert's row r is token r - tk) or H rows (fp32, rounded to
// nearest even).
template <bool FROM_H>
__device__ __forceinline__ void stage_rows(const Q4kArgs& a, const Group& g, int tb, int nt, int K, uint4* lds) {
    const int chunks = K / 8;  // 16-byte bf16 chunks per row
    for (int i = threadIdx.x; i < nt * chunks; i += blockDim.x) {
        const int t = i / chunks, ch = i - t * chunks;
        const int row = g.row0 + tb + t;
        uint4 v;
        if constexpr (FROM_H) {
            v = bf16_chunk(a.H + (size_t)row * a.hstride + 8 * ch);
        } else {
            int tok = a.T == 1 ? 0 : g.e < 0 ? row - a.tk : a.perm_token[row];
            tok = min(max(tok, 0), a.T - 1);
            v = ld16(a.x + (size_t)tok * a.d + 8 * ch);
        }
        lds[t * chunks + act_chunk(ch >> 3, ch & 7)] = v;
    }
}

template <int LPR, int NP>
struct Lanes {
    static constexpr int P = 64 / LPR;  // rows a wave covers at once
    static constexpr int NR = P * NP;   // rows per wave
};

// Up: one wave owns hidden units f0 .. f0 + NR/2 - 1 of group g.  Row r of the
// wave is the gate (r even) or up (r odd) row of unit f0 + r / 2; in pass p, lane l serves
// row p * P + l / LPR, unit l % LPR.  With P >= 2 the up row is the next sub-row (LPR
// lanes on); with P == 1 it is the next pass, in the same lane.  Every wave of the block
// runs this with the same group (the staging barriers are the block's).
template <int LPR, int NP, int NT>
__device__ __forceinline__ void q4k_up_body(const Q4kArgs& a, const Group& g, int f0, uint4* act) {
    constexpr int P = Lanes<LPR, NP>::P;
    static_assert(P >= 2 || NP % 2 == 0, "gate and up rows pair up");
    const int lane = lane_id();
    const int sr = lane / LPR, ul = lane % LPR;
    const bool active = ul < a.d / 64;
    const int uc = active ? ul : 0;
    const int nsb = a.d / kQ4kBlockWeights;
    Q4kDec w[NP];
    if (g.e < 0) {  // the shared expert (bf16 rows)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = p * P + sr;
            const int f = min(f0 + r / 2, a.ff - 1);
            load_bf16_unit(((r & 1) ? a.ws_up : a.ws_gate) + (size_t)f * a.d, uc, w[p]);
        }
    } else {
        uint4 hd[NP], q0[NP], q1[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = p * P + sr;
            const int f = min(f0 + r / 2, a.ff - 1);
            const uint8_t* base = (r & 1) ? a.w_up : a.w_gate;
            load_unit(base + ((size_t)g.e * a.ff + f) * nsb * kQ4kBlockBytes, uc, hd[p], q0[p], q1[p]);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) decode_unit(uc, hd[p], q0[p], q1[p], w[p]);
    }
    const int chunks = a.d / 8;
    for (int tb = 0; tb < g.n; tb += NT) {
        const int nt = min(NT, g.n - tb);
        if (tb > 0) __syncthreads();  // every wave is done with the previous rows
        stage_rows<false>(a, g, tb, nt, a.d, act);
        __syncthreads();
        if (f0 >= a.ff) continue;
        for (int t = 0; t < nt; ++t) {
            Q4kAct x;
            read_act(act + t * chunks, uc, x);
            float acc[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) acc[p] = segment_sum<LPR>(active ? unit_dot(w[p], x) : 0.0f);
            const size_t hrow = (size_t)(g.row0 + tb + t) * a.hstride;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int f = f0 + (p * P + sr) / 2;
                if constexpr (P >= 2) {
                    const float up = __shfl(acc[p], (lane + LPR) & 63, kWave);
                    if (ul == 0 && (sr & 1) == 0 && f < a.ff) a.H[hrow + f] = acc[p] * sigmoidf_(acc[p]) * up;
                } else if ((p & 1) == 0) {
                    if (lane == 0 && f < a.ff) a.H[hrow + f] = acc[p] * sigmoidf_(acc[p]) * acc[p + 1];
                }
            }
        }
    }
}

template <int LPR, int NP, int NT>
__global__ __launch_bounds__(256) void expert_up_gemv_q4k_kernel(Q4kArgs a) {
    extern __shared__ uint4 act[];
    Group g;
    if (!q4k_group(a, g)) return;
    q4k_up_body<LPR, NP, NT>(a, g, (blockIdx.x * 4 + wave_id()) * (Lanes<LPR, NP>::NR / 2), act);
}

// One token: the top-k in front of the up GEMV.  Every wave of grid row j runs the wave
// top-k of the routing kernels on the logits and takes pick j (hidden row j); block 0 of
// the row records the pick (idx[j], w[j]) for the down kernel.
template <int LPR, int NP>
__global__ __launch_bounds__(256) void token1_up_q4k_kernel(Q4kArgs a, const float* __restrict__ logits, int E,
                                                            int k, int mode, float scale,
                                                            int32_t* __restrict__ idx, float* __restrict__ w) {
    extern __shared__ uint4 act[];
    const int j = blockIdx.y;
    int my_i;
    float my_w;
    topk_wave(logits, E, k, mode, scale, &my_i, &my_w);
    if (blockIdx.x == 0 && wave_id() == 0 && lane_id() == j) {
        idx[j] = my_i;
        w[j] = my_w;
    }
    const int e = __builtin_amdgcn_readlane(my_i, j);
    q4k_up_body<LPR, NP, 1>(a, Group{min(max(e, 0), E - 1), j, 1, 0},
                            (blockIdx.x * 4 + wave_id()) * (Lanes<LPR, NP>::NR / 2), act);
}

// Down: one wave owns output dims i0 .. i0 + NR - 1 of group g (dim i0 + p * P + l / LPR
// in pass p).
template <int LPR, int NP, int NT>
__global__ __launch_bounds__(256) void expert_down_gemv_q4k_kernel(Q4kArgs a) {
    using LN = Lanes<LPR, NP>;
    constexpr int P = LN::P, NR = LN::NR;
    extern __shared__ uint4 act[];
    Group g;
    if (!q4k_group(a, g)) return;
    const int i0 = (blockIdx.x * 4 + wave_id()) * NR;
    const int lane = lane_id();
    const int sr = lane / LPR, ul = lane % LPR;
    const bool active = ul < a.ff / 64;
    const int uc = active ? ul : 0;
    const int nsb = a.ff / kQ4kBlockWeights;
    Q4kDec w[NP];
    if (g.e < 0) {  // the shared expert (bf16 rows)
#pragma unroll
        for (int p = 0; p < NP; ++p)
            load_bf16_unit(a.ws_down + (size_t)min(i0 + p * P + sr, a.d - 1) * a.ff, uc, w[p]);
    } else {
        uint4 hd[NP], q0[NP], q1[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int i = min(i0 + p * P + sr, a.d - 1);
            load_unit(a.w_down + ((size_t)g.e * a.d + i) * nsb * kQ4kBlockBytes, uc, hd[p], q0[p], q1[p]);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) decode_unit(uc, hd[p], q0[p], q1[p], w[p]);
    }
    const int chunks = a.ff / 8;
    for (int tb = 0; tb < g.n; tb += NT) {
        const int nt = min(NT, g.n - tb);
        if (tb > 0) __syncthreads();
        stage_rows<true>(a, g, tb, nt, a.ff, act);
        __syncthreads();
        if (i0 >= a.d) continue;
        for (int t = 0; t < nt; ++t) {
            Q4kAct h;
            read_act(act + t * chunks, uc, h);
            const size_t yrow = (size_t)(g.row0 + tb + t) * a.d;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float s = segment_sum<LPR>(active ? unit_dot(w[p], h) : 0.0f);
                const int i = i0 + p * P + sr;
                if (ul == 0 && i < a.d) a.y[yrow + i] = s;
            }
        }
    }
}

// A few tokens: the down projection of every pick (Q4_K W_d) and of the shared expert
// (bf16) with the weighted combine, in one kernel, as the dense and MXFP4 layers do.
// Block (b, t) owns output dims i0 = NR b .. i0 + NR - 1 of token t.  Wave j < k takes
// pick j: expert idx[t k + j], weight w[t k + j], hidden row perm_inv[t k + j] (row j for
// one token); it stages that H row in its own LDS slice as bf16 (as the down GEMV does)
// and serves its NR rows with the decoded units.  Wave k, with a shared expert, takes hidden
// row T k + t with weight sigmoid(shared_gate[t gate_ld]) and streams the bf16 rows of the
// shared W_d against the fp32 H row.  The waves leave their NR sums in LDS; NR threads then
// add them in the combine's order (picks 0..k-1, then the shared expert).
constexpr int kQ4kTokenMaxWaves = 16;

template <int LPR, int NP, int KBS, bool EXS>
__global__ __launch_bounds__(kQ4kTokenMaxWaves * kWave) void token_down_combine_q4k_kernel(
    Q4kArgs a, const uint16_t* __restrict__ ws_down, int ffs, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const int32_t* __restrict__ perm_inv, const float* __restrict__ shared_gate,
    int gate_ld, int E, int k, const uint16_t* __restrict__ residual, uint16_t* __restrict__ y) {
    using LN = Lanes<LPR, NP>;
    constexpr int P = LN::P, NR = LN::NR;
    __shared__ float part[kQ4kTokenMaxWaves][NR];
    __shared__ float wts[kQ4kTokenMaxWaves];
    extern __shared__ uint4 act[];
    const int j = wave_id(), lane = lane_id();
    const int i0 = blockIdx.x * NR, t = blockIdx.y;
    if (j < k) {
        const int p = t * k + j;
        const int ei = idx[p], r = perm_inv ? perm_inv[p] : j;
        const bool ok = ei >= 0 && ei < E && r >= 0 && r < a.tk;  // else weight 0
        const int e = ok ? ei : 0, row = ok ? r : 0;
        const int sr = lane / LPR, ul = lane % LPR;
        const bool active = ul < a.ff / 64;
        const int uc = active ? ul : 0;
        const int nsb = a.ff / kQ4kBlockWeights;
        uint4 hd[NP], q0[NP], q1[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int i = min(i0 + q * P + sr, a.d - 1);
            load_unit(a.w_down + ((size_t)e * a.d + i) * nsb * kQ4kBlockBytes, uc, hd[q], q0[q], q1[q]);
        }
        // This wave's H row as bf16 in its LDS slice (layout act_chunk); the wave reads back
        // only what it wrote.
        const int chunks = a.ff / 8;
        uint4* mine = act + j * chunks;
        const float* hr = a.H + (size_t)row * a.hstride;
        for (int ch = lane; ch < chunks; ch += kWave) mine[act_chunk(ch >> 3, ch & 7)] = bf16_chunk(hr + 8 * ch);
        Q4kDec wd[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) decode_unit(uc, hd[q], q0[q], q1[q], wd[q]);
        Q4kAct h;
        read_act(mine, uc, h);
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const float sum = segment_sum<LPR>(active ? unit_dot(wd[q], h) : 0.0f);
            if (ul == 0) part[j][q * P + sr] = sum;
        }
        if (lane == 0) wts[j] = ok ? w[p] : 0.0f;
    } else {
        // The shared expert: NR bf16 rows of the shared W_d against hidden row T k + t.
        constexpr int SH = 6 - ilog2(NR);
        const uint16_t* wr[NR];
#pragma unroll
        for (int q = 0; q < NR; ++q) wr[q] = ws_down + (size_t)min(i0 + q, a.d - 1) * ffs;
        const uint16_t* const (&wrc)[NR] = wr;
        const float* ar[1] = {a.H + (size_t)(a.tk + t) * a.hstride};
        const float* const (&arc)[1] = ar;
        float acc[NR][1] = {};
        rows_dot<NR, 1, KBS, BF16, F32, true, EXS>(wrc, arc, 1, ffs, acc);
        float v[NR];
#pragma unroll
        for (int q = 0; q < NR; ++q) v[q] = acc[q][0];
        const float sum = wave_reduce_scatter<NR>(v);
        if ((lane & ((1 << SH) - 1)) == 0) part[j][lane >> SH] = sum;
        if (lane == 0) wts[j] = 1.0f / (1.0f + expf(-shared_gate[(size_t)t * gate_ld]));
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < NR && i0 + tid < a.d) {
        const int nw = blockDim.x / kWave;
        float o = 0.0f;
        for (int jj = 0; jj < nw; ++jj) o = fmaf(wts[jj], part[jj][tid], o);
        const size_t at = (size_t)t * a.d + i0 + tid;
        if (residual) o += bf16_to_f32(residual[at]);  // read before y is written: y may alias it
        y[at] = f32_to_bf16(o);
    }
}

// Lanes per row for a K axis: K / 64 units rounded up to a power of two (K <= 4096).
int lanes_per_row(int K) {
    const int u = K / 64;
    int l = 4;
    while (l < u) l *= 2;
    return l;
}

// Passes per wave: NP = R / P, at most 4 (128 registers of decoded weights), for R rows
// per wave: 8 for one token; for more, 4 in the up kernel and 16 in the down kernel.  (Up
// kernel at the Qwen shape, K = 2048: 4 rows per wave hold 64 registers of decoded weights
// and leave about four waves per SIMD to hide the weight loads; 8 rows, two waves per
// SIMD, ran the T=64 forward at 180 us against 169 us, 2 rows at 182 us.)  P == 1 gives
// 4 passes, even as the up kernel needs.
constexpr int q4k_passes(int P, bool many, bool down = false) {
    const int r = many ? (down ? 16 : 4) : 8;
    return r / P > 4 ? 4 : (r / P < 1 ? 1 : r / P);
}

template <int LPR, bool MANY>
hipError_t launch_q4k_lpr(const Q4kArgs& a, int gmax, bool down, hipStream_t s) {
    constexpr int NT = MANY ? kQ4kStepRows : 1;
    if (!down) {
        constexpr int NP = q4k_passes(64 / LPR, MANY, false);
        constexpr int NR = Lanes<LPR, NP>::NR;
        const int units_per_block = 4 * (NR / 2);
        const dim3 grid((a.ff + units_per_block - 1) / units_per_block, gmax);
        expert_up_gemv_q4k_kernel<LPR, NP, NT><<<grid, 256, q4k_stage_bytes(a.d, NT), s>>>(a);
    } else {
        constexpr int NP = q4k_passes(64 / LPR, MANY, true);
        constexpr int NR = Lanes<LPR, NP>::NR;
        const dim3 grid((a.d + 4 * NR - 1) / (4 * NR), gmax);
        expert_down_gemv_q4k_kernel<LPR, NP, NT><<<grid, 256, q4k_stage_bytes(a.ff, NT), s>>>(a);
    }
    return hipGetLastError();
}

template <bool MANY>
hipError_t launch_q4k(const Q4kArgs& a, int gmax, bool down, hipStream_t s) {
    switch (lanes_per_row(down ? a.ff : a.d)) {
        case 4: return launch_q4k_lpr<4, MANY>(a, gmax, down, s);
        case 8: return launch_q4k_lpr<8, MANY>(a, gmax, down, s);
        case 16: return launch_q4k_lpr<16, MANY>(a, gmax, down, s);
        case 32: return launch_q4k_lpr<32, MANY>(a, gmax, down, s);
        case 64: return launch_q4k_lpr<64, MANY>(a, gmax, down, s);
        default: return hipErrorInvalidValue;
    }
}

template <int LPR>
hipError_t launch_token1_up_q4k_lpr(const Q4kArgs& a, const moe_layer& L, const float* logits, int32_t* idx,
                                    float* w, hipStream_t s) {
    constexpr int NP = q4k_passes(64 / LPR, false);
    constexpr int units_per_block = 4 * (Lanes<LPR, NP>::NR / 2);
    const dim3 grid((a.ff + units_per_block - 1) / units_per_block, L.k);
    token1_up_q4k_kernel<LPR, NP><<<grid, 256, q4k_stage_bytes(a.d, 1), s>>>(a, logits, L.n_expert, L.k, L.route, L.route_scale,
                                                            idx, w);
    return hipGetLastError();
}

template <int LPR>
hipError_t launch_down_combine_q4k_lpr(const Q4kArgs& a, const moe_layer& L, int T, const int32_t* idx,
                                       const float* w, const int32_t* perm_inv, const float* shared_gate,
                                       int gate_ld, const void* residual, void* y, hipStream_t s) {
    constexpr int NP = q4k_passes(64 / LPR, false);
    constexpr int NR = Lanes<LPR, NP>::NR;
    const bool shared = L.shared_ff > 0;
    const dim3 grid((a.d + NR - 1) / NR, T);
    const dim3 block((L.k + (shared ? 1 : 0)) * kWave);
    const size_t lds = q4k_stage_bytes(a.ff, L.k);
    const auto* wsd = static_cast<const uint16_t*>(L.ws_down);
    const auto* ro = static_cast<const uint16_t*>(residual);
    auto* yo = static_cast<uint16_t*>(y);
    const int ffs = shared ? L.shared_ff : kWave * BF16::VEC;
    // Shared rows in batches of at most 2 chunks per lane, 1 for 16 rows per wave (the
    // block may hold 16 waves, 128 registers each).
    const int kbs = NR >= 16 || pick_kb(ffs, BF16::VEC) < 2 ? 1 : 2;
    const bool ex = exact_k(ffs, BF16::VEC, kbs);
#define SMOE_Q4K_DC(KBS, EX)                                                                           \
    token_down_combine_q4k_kernel<LPR, NP, KBS, EX><<<grid, block, lds, s>>>(                           \
        a, wsd, ffs, idx, w, perm_inv, shared ? shared_gate : nullptr, gate_ld, L.n_expert, L.k, ro, yo)
    if constexpr (NR >= 16) {
        if (ex) SMOE_Q4K_DC(1, true);
        else SMOE_Q4K_DC(1, false);
    } else if (kbs == 1) {
        if (ex) SMOE_Q4K_DC(1, true);
        else SMOE_Q4K_DC(1, false);
    } else {
        if (ex) SMOE_Q4K_DC(2, true);
        else SMOE_Q4K_DC(2, false);
    }
#undef SMOE_Q4K_DC
    return hipGetLastError();
}

// The shared expert rides in the Q4_K launches when it is as wide as the routed experts.
bool q4k_fuse_shared(const moe_layer& L) { return L.shared_ff > 0 && L.shared_ff == L.ff; }

Q4kArgs q4k_args(const moe_layer& L, const void* x, int T, const int32_t* perm_token, const Group* groups,
                 const PlanMeta* meta, float* H, int hstride, float* y_perm) {
    return Q4kArgs{static_cast<const uint16_t*>(x), perm_token, groups, meta,
                   static_cast<const uint8_t*>(L.w_gate), static_cast<const uint8_t*>(L.w_up),
                   static_cast<const uint8_t*>(L.w_down), static_cast<const uint16_t*>(L.ws_gate),
                   static_cast<const uint16_t*>(L.ws_up), static_cast<const uint16_t*>(L.ws_down), H, y_perm,
                   hstride, T, T * L.k, L.d, L.ff, L.shared_ff > 0 ? 1 : 0, q4k_fuse_shared(L) ? 1 : 0};
}

// Grid rows of a Q4_K GEMV launch: every routed group, and the fused shared expert's chunks.
int q4k_grid_rows(const moe_layer& L, int T) {
    return max_groups(L.n_expert, T, L.k, false) + (q4k_fuse_shared(L) ? (T + kQ4kSharedRows - 1) / kQ4kSharedRows : 0);
}

}  // namespace

bool q4k_fits(const moe_layer& L) {
    return L.d % kQ4kBlockWeights == 0 && L.ff % kQ4kBlockWeights == 0 && L.d <= 4096 && L.ff <= 4096;
}

bool q4k_token_fits(const moe_layer& L) {
    return L.expert_format == MOE_EXPERTS_Q4K && q4k_fits(L) &&
           L.k + (L.shared_ff > 0 ? 1 : 0) <= kQ4kTokenMaxWaves && q4k_stage_bytes(L.ff, L.k) <= (64u << 10);
}

hipError_t launch_expert_up_gemv_q4k(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                     const Group* groups, const PlanMeta* meta, float* H, int hstride,
                                     hipStream_t s) {
    if (!q4k_fits(L)) return hipErrorInvalidValue;
    const Q4kArgs a = q4k_args(L, x, T, perm_token, groups, meta, H, hstride, nullptr);
    const int rows = q4k_grid_rows(L, T);
    const hipError_t e = T == 1 ? launch_q4k<false>(a, rows, false, s) : launch_q4k<true>(a, rows, false, s);
    if (e != hipSuccess || L.shared_ff <= 0 || a.fuse_shared) return e;
    return launch_shared_gemv_up(L, x, T, groups, meta, H, hstride, s);
}

hipError_t launch_expert_gemv_q4k(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                                  const Group* groups, const PlanMeta* meta, float* H, int hstride, float* y_perm,
                                  hipStream_t s) {
    hipError_t e = launch_expert_up_gemv_q4k(L, x, T, perm_token, groups, meta, H, hstride, s);
    if (e != hipSuccess) return e;
    const Q4kArgs a = q4k_args(L, x, T, perm_token, groups, meta, H, hstride, y_perm);
    const int rows = q4k_grid_rows(L, T);
    e = T == 1 ? launch_q4k<false>(a, rows, true, s) : launch_q4k<true>(a, rows, true, s);
    if (e != hipSuccess || L.shared_ff <= 0 || a.fuse_shared) return e;
    return launch_shared_gemv_down(L, T, groups, meta, H, hstride, y_perm, s);
}

hipError_t launch_token1_up_q4k(const moe_layer& L, const void* x, const float* logits, int32_t* idx, float* w,
                                float* H, int hstride, hipStream_t s) {
    if (!q4k_token_fits(L)) return hipErrorInvalidValue;
    const Q4kArgs a = q4k_args(L, x, 1, nullptr, nullptr, nullptr, H, hstride, nullptr);
    switch (lanes_per_row(L.d)) {
        case 4: return launch_token1_up_q4k_lpr<4>(a, L, logits, idx, w, s);
        case 8: return launch_token1_up_q4k_lpr<8>(a, L, logits, idx, w, s);
        case 16: return launch_token1_up_q4k_lpr<16>(a, L, logits, idx, w, s);
        case 32: return launch_token1_up_q4k_lpr<32>(a, L, logits, idx, w, s);
        case 64: return launch_token1_up_q4k_lpr<64>(a, L, logits, idx, w, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_token_down_combine_q4k(const moe_layer& L, int T, const float* H, int hstride, const int32_t* idx,
                                         const float* w, const int32_t* perm_inv, const float* shared_gate,
                                         int gate_ld, const void* residual, void* y, hipStream_t s) {
    if (!q4k_token_fits(L) || T < 1 || (!perm_inv && T != 1) || (L.shared_ff > 0 && !shared_gate))
        return hipErrorInvalidValue;
    const Q4kArgs a = q4k_args(L, nullptr, T, nullptr, nullptr, nullptr, const_cast<float*>(H), hstride, nullptr);
    switch (lanes_per_row(L.ff)) {
#define SMOE_DC_CASE(LPR) \
    case LPR: return launch_down_combine_q4k_lpr<LPR>(a, L, T, idx, w, perm_inv, shared_gate, gate_ld, residual, y, s);
        SMOE_DC_CASE(4)
        SMOE_DC_CASE(8)
        SMOE_DC_CASE(16)
        SMOE_DC_CASE(32)
        SMOE_DC_CASE(64)
#undef SMOE_DC_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace smoe

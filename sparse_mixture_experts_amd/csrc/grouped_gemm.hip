// Grouped GEMMs of the expert FFNs on bf16 MFMA (the prefill path).
//
// "Engine" (Cherenkov), Prefill: tokens are grouped by expert, gathered, projected and
// scattered back; its kernels use token tiles, half-precision weights and float
// accumulation.  Here every group (one expert's rows, or the shared expert over all
// tokens) is cut into 128-row M-tiles; a block computes one 128-row tile against one
// slice of the expert's weights with v_mfma_f32_16x16x32_bf16 and fp32 accumulation.
//
// Up kernel: rows of x gathered through perm_token, times the 64 gate rows and the 64
// matching up rows of a 64-unit slice of the hidden layer (for the clamped variant the
// interleaved gate_up rows are de-interleaved while staging), then the activation of
// "Qwen3.5-MoE Model Implementation" (silu(gate) * up) or of "Phase 19: MoE -
// gpt-oss-20b", Experts (biases, clamps, (up + 1) * gate * sigmoid(alpha * gate)) in
// the epilogue; H is stored in bf16.
// Down kernel: H rows times a 128-column slice of W_d (+ down bias), optionally scaled
// by each row's routing weight (or the shared expert's sigmoid gate) so that the
// combine is a plain sum; output bf16 or fp32.
//
// Block: 256 threads = 4 waves in a 2 x 2 grid, each wave a 64 x 64 output tile =
// 4 x 4 MFMA tiles.  K advances 64 per step through a double-buffered LDS stage: the
// next step's global loads are issued before the current step's MFMAs.  LDS rows are
// padded to 72 bf16 (144 B) so the 16-row fragment reads hit distinct banks.
#include "common.h"
#include "internal.h"

namespace smoe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = kGroupTileM;  // rows per M-tile
constexpr int BN = 128;          // weight rows per block
constexpr int BK = 64;           // K per pipeline step
constexpr int LDS_STRIDE = BK + 8;
constexpr int kThreads = 256;

struct UpArgs {
    const uint16_t* x;
    const int32_t* perm_token;
    const Group* groups;
    const PlanMeta* meta;
    const int32_t* tile_map;
    const uint16_t* w_gate;     // [E, ff, d]
    const uint16_t* w_up;
    const uint16_t* w_gate_up;  // [E, 2ff, d]
    const uint16_t* b_gate_up;  // [E, 2ff]
    const uint16_t* ws_gate;    // [ffs, d]
    const uint16_t* ws_up;
    uint16_t* H;                // bf16 [rows, hstride]
    int hstride, T, d, ff, ffs, n_ntiles;
    float alpha, limit;
};

struct DownArgs {
    const uint16_t* H;
    const Group* groups;
    const PlanMeta* meta;
    const int32_t* tile_map;
    const uint16_t* w_down;   // [E, d, ff]
    const uint16_t* b_down;   // [E, d] or null
    const uint16_t* ws_down;  // [d, ffs]
    const float* row_w;       // per grouped row weight, or null (unweighted)
    void* y;                  // [rows, d], bf16 or fp32
    int hstride, d, ff, ffs, n_ntiles;
};

__device__ __forceinline__ float ld_bf16(const uint16_t* p) { return bf16_to_f32(*p); }

// Stage one BK-wide slice: this thread's 4 rows (tile rows tid/8 + 32 i) at chunk tid%8.
__device__ __forceinline__ void load_slice(const uint16_t* const (&rows)[4], int k0, uint4 (&r)[4]) {
    const int c = (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ld16(rows[i] + k0 + c);
}

__device__ __forceinline__ void store_slice(uint16_t* lds, const uint4 (&r)[4]) {
    const int c = (threadIdx.x & 7) * 8;
    const int r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(lds + (r0 + 32 * i) * LDS_STRIDE + c) = r[i];
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* lds, int row, int col) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + row * LDS_STRIDE + col));
}

// One pipeline step on K-slice kt, using LDS buffer / register set B (= kt & 1, a
// compile-time constant so the register arrays are never indexed dynamically).
template <int B>
__device__ __forceinline__ void pipeline_step(const uint16_t* const (&a_rows)[4],
                                              const uint16_t* const (&b_rows)[4], int kt, int nk,
                                              const int (&brow)[4], uint4 (&ra)[2][4], uint4 (&rb)[2][4],
                                              uint16_t (&sA)[2][BM * LDS_STRIDE],
                                              uint16_t (&sB)[2][BN * LDS_STRIDE], floatx4 (&acc)[4][4]) {
    const int lane = lane_id();
    const int wm = (threadIdx.x / kWave) >> 1;
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    if (kt + 2 < nk) {
        load_slice(a_rows, (kt + 2) * BK, ra[B]);
        load_slice(b_rows, (kt + 2) * BK, rb[B]);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) af[mi] = lds_frag(sA[B], wm * 64 + mi * 16 + fr, kk + fk);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) bfr[ni] = lds_frag(sB[B], brow[ni] + fr, kk + fk);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) {
        store_slice(sA[B ^ 1], ra[B ^ 1]);
        store_slice(sB[B ^ 1], rb[B ^ 1]);
    }
    __syncthreads();
}

// acc[mi][ni] += A[64 wave rows] x B[4 x 16 rows given by brow[ni]]^T over K.
// Slice s (K range [s*BK, (s+1)*BK)) is loaded into registers two steps before it is
// used (register set s & 1), written to LDS buffer s & 1 one step before, and consumed
// from LDS: each global load has two steps of MFMA work to arrive.
__device__ __forceinline__ void mainloop(const uint16_t* const (&a_rows)[4], const uint16_t* const (&b_rows)[4],
                                         int K, const int (&brow)[4], floatx4 (&acc)[4][4]) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDS_STRIDE];
    const int nk = K / BK;
    uint4 ra[2][4], rb[2][4];
    load_slice(a_rows, 0, ra[0]);
    load_slice(b_rows, 0, rb[0]);
    if (nk > 1) {
        load_slice(a_rows, BK, ra[1]);
        load_slice(b_rows, BK, rb[1]);
    }
    store_slice(sA[0], ra[0]);
    store_slice(sB[0], rb[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        pipeline_step<0>(a_rows, b_rows, kt, nk, brow, ra, rb, sA, sB, acc);
        if (kt + 1 < nk) pipeline_step<1>(a_rows, b_rows, kt + 1, nk, brow, ra, rb, sA, sB, acc);
    }
}

// XCD-aware tile order.  Workgroups are dispatched to the 8 XCDs round-robin by block
// id, and each XCD has its own L2.  Block b runs slot b / 8 of XCD b % 8; every XCD owns
// a contiguous range of M-tiles (groups are contiguous in tile order, so an expert spans
// at most a few XCDs) and runs all N-tiles of one M-tile back to back.  The gathered A
// tile is then fetched into one L2 and reused by all N-tiles, and an expert's weight
// slices are reused by its consecutive M-tiles inside the same L2.
constexpr int kXcds = 8;

inline int grid_blocks(int max_mtiles, int n_ntiles) {
    return kXcds * ((max_mtiles + kXcds - 1) / kXcds) * n_ntiles;
}

// Resolve this block's (group, first row, N-tile).  Returns false if the block is idle.
__device__ __forceinline__ bool locate(const PlanMeta* meta, const int32_t* tile_map, const Group* groups,
                                       int n_ntiles, Group& g, int& m0, int& nt) {
    const int n_tiles = meta->n_tiles;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int per_xcd = (n_tiles + kXcds - 1) / kXcds;
    const int local = slot / n_ntiles;
    const int mt = xcd * per_xcd + local;
    nt = slot % n_ntiles;
    if (local >= per_xcd || mt >= n_tiles) return false;
    g = groups[tile_map[mt]];
    m0 = (mt - g.tile0) * BM;
    return true;
}

template <bool OAI>
__global__ __launch_bounds__(kThreads, 2) void gg_up_kernel(UpArgs a) {
    Group g;
    int m0, nt;
    if (!locate(a.meta, a.tile_map, a.groups, a.n_ntiles, g, m0, nt)) return;
    const bool shared = g.e < 0;
    const int ffg = shared ? a.ffs : a.ff;
    const int f0 = nt * 64;
    if (f0 >= ffg) return;
    const bool oai = OAI && !shared;
    const size_t d = a.d;
    const int r0 = threadIdx.x >> 3;

    const uint16_t* a_rows[4];
    const uint16_t* b_rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = min(m0 + r0 + 32 * i, g.n - 1);  // ragged tail: re-read the last row
        int tok = shared ? m : a.perm_token[g.row0 + m];
        tok = min(max(tok, 0), a.T - 1);
        a_rows[i] = a.x + (size_t)tok * d;
        const int j = r0 + 32 * (i & 1);  // hidden unit within the slice
        const bool up = i >= 2;
        if (oai) {
            b_rows[i] = a.w_gate_up + ((size_t)g.e * 2 * a.ff + 2 * (f0 + j) + (up ? 1 : 0)) * d;
        } else {
            const uint16_t* base = shared ? (up ? a.ws_up : a.ws_gate)
                                          : (up ? a.w_up : a.w_gate) + (size_t)g.e * a.ff * d;
            b_rows[i] = base + (size_t)(f0 + j) * d;
        }
    }
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    // B tile rows: 0..63 gate units, 64..127 up units; wave n-tiles 0,1 gate, 2,3 up.
    const int brow[4] = {wn * 32, wn * 32 + 16, 64 + wn * 32, 64 + wn * 32 + 16};
    floatx4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* const (&ar)[4] = a_rows;
    const uint16_t* const (&br)[4] = b_rows;
    mainloop(ar, br, a.d, brow, acc);

    // Epilogue: lane holds D[4*(lane/16) + i][lane%16] of each 16x16 tile.
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int f = f0 + wn * 32 + ni * 16 + (lane & 15);
        float bg = 0.f, bu = 0.f;
        if (oai) {
            bg = ld_bf16(a.b_gate_up + (size_t)g.e * 2 * a.ff + 2 * f);
            bu = ld_bf16(a.b_gate_up + (size_t)g.e * 2 * a.ff + 2 * f + 1);
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
                float gv = acc[mi][ni][i], uv = acc[mi][ni + 2][i], h;
                if (oai) {
                    gv = fminf(gv + bg, a.limit);
                    uv = fminf(fmaxf(uv + bu, -a.limit), a.limit);
                    h = (uv + 1.0f) * gv * sigmoidf_(a.alpha * gv);
                } else {
                    h = gv * sigmoidf_(gv) * uv;
                }
                if (m < g.n) a.H[(size_t)(g.row0 + m) * a.hstride + f] = f32_to_bf16(h);
            }
        }
    }
}

template <typename TY>
__global__ __launch_bounds__(kThreads, 2) void gg_down_kernel(DownArgs a) {
    Group g;
    int m0, nt;
    if (!locate(a.meta, a.tile_map, a.groups, a.n_ntiles, g, m0, nt)) return;
    const bool shared = g.e < 0;
    const int K = shared ? a.ffs : a.ff;
    const int n0 = nt * BN;
    const int r0 = threadIdx.x >> 3;
    const uint16_t* a_rows[4];
    const uint16_t* b_rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = min(m0 + r0 + 32 * i, g.n - 1);
        a_rows[i] = a.H + (size_t)(g.row0 + m) * a.hstride;
        const int n = min(n0 + r0 + 32 * i, a.d - 1);  // partial last N-tile: re-read
        b_rows[i] = shared ? a.ws_down + (size_t)n * K : a.w_down + ((size_t)g.e * a.d + n) * K;
    }
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
    floatx4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* const (&ar)[4] = a_rows;
    const uint16_t* const (&br)[4] = b_rows;
    mainloop(ar, br, K, brow, acc);

    float rw[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = min(m0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i, g.n - 1);
            rw[mi][i] = a.row_w ? a.row_w[g.row0 + m] : 1.0f;
        }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int n = n0 + wn * 64 + ni * 16 + (lane & 15);
        if (n >= a.d) continue;
        const float bias = (!shared && a.b_down) ? ld_bf16(a.b_down + (size_t)g.e * a.d + n) : 0.0f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
                if (m >= g.n) continue;
                const float v = (acc[mi][ni][i] + bias) * rw[mi][i];
                const size_t o = (size_t)(g.row0 + m) * a.d + n;
                if constexpr (sizeof(TY) == 2) static_cast<uint16_t*>(a.y)[o] = f32_to_bf16(v);
                else static_cast<float*>(a.y)[o] = v;
            }
    }
}

// Router logits of a large batch on MFMA: logits[t, e] = x[t] . W_r[e] (+ b[e]) for
// e < E ("Qwen3.5-MoE Model Implementation", MoE routing; "Phase 19: MoE - gpt-oss-20b",
// Router).  Same tiling as the down kernel: 128 tokens x 128 experts per block.
__global__ __launch_bounds__(kThreads, 2) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ w_router,
                                                                  const float* __restrict__ b_router,
                                                                  int T, int d, int E, int n_ntiles,
                                                                  float* __restrict__ logits, int ld) {
    const int m0 = (blockIdx.x / n_ntiles) * BM;
    const int n0 = (blockIdx.x % n_ntiles) * BN;
    const int r0 = threadIdx.x >> 3;
    const uint16_t* a_rows[4];
    const uint16_t* b_rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_rows[i] = x + (size_t)min(m0 + r0 + 32 * i, T - 1) * d;
        b_rows[i] = w_router + (size_t)min(n0 + r0 + 32 * i, E - 1) * d;
    }
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
    floatx4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* const (&ar)[4] = a_rows;
    const uint16_t* const (&br)[4] = b_rows;
    mainloop(ar, br, d, brow, acc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int n = n0 + wn * 64 + ni * 16 + (lane & 15);
        if (n >= E) continue;
        const float bias = b_router ? b_router[n] : 0.0f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
                if (m < T) logits[(size_t)m * ld + n] = acc[mi][ni][i] + bias;
            }
    }
}

}  // namespace

hipError_t launch_router_mfma(const moe_layer& L, const void* x, int T, float* logits, int ld,
                              hipStream_t s) {
    const int nn = (L.n_expert + BN - 1) / BN;
    const int nm = (T + BM - 1) / BM;
    router_mfma_kernel<<<nm * nn, kThreads, 0, s>>>(static_cast<const uint16_t*>(x),
                                                    static_cast<const uint16_t*>(L.w_router), L.b_router, T,
                                                    L.d, L.n_expert, nn, logits, ld);
    return hipGetLastError();
}

int grouped_max_mtiles(int E, int T, int k, bool shared) {
    const long long tk = (long long)T * k;
    long long b = tk / BM + (tk < E ? tk : E) + 1;
    if (shared) b += (T + BM - 1) / BM;
    return (int)b;
}

hipError_t launch_grouped_ffn(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                              const Group* groups, const PlanMeta* meta, const int32_t* tile_map,
                              uint16_t* H, int hstride, const float* row_w, void* y, bool y_bf16,
                              hipStream_t s) {
    const bool shared = L.shared_ff > 0;
    const int mt = grouped_max_mtiles(L.n_expert, T, L.k, shared);
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    UpArgs u{static_cast<const uint16_t*>(x), perm_token, groups, meta, tile_map,
             static_cast<const uint16_t*>(L.w_gate), static_cast<const uint16_t*>(L.w_up),
             static_cast<const uint16_t*>(L.w_gate_up), static_cast<const uint16_t*>(L.b_gate_up),
             static_cast<const uint16_t*>(L.ws_gate), static_cast<const uint16_t*>(L.ws_up), H, hstride, T,
             L.d, L.ff, L.shared_ff, ffmax / 64, L.oai_alpha, L.oai_limit};
    const dim3 gu((unsigned)grid_blocks(mt, ffmax / 64));
    if (L.act == MOE_ACT_SWIGLU_OAI)
        gg_up_kernel<true><<<gu, kThreads, 0, s>>>(u);
    else
        gg_up_kernel<false><<<gu, kThreads, 0, s>>>(u);
    const int nn = (L.d + BN - 1) / BN;
    DownArgs dn{H, groups, meta, tile_map, static_cast<const uint16_t*>(L.w_down),
                static_cast<const uint16_t*>(L.b_down), static_cast<const uint16_t*>(L.ws_down), row_w, y,
                hstride, L.d, L.ff, L.shared_ff, nn};
    const dim3 gd((unsigned)grid_blocks(mt, nn));
    if (y_bf16)
        gg_down_kernel<uint16_t><<<gd, kThreads, 0, s>>>(dn);
    else
        gg_down_kernel<float><<<gd, kThreads, 0, s>>>(dn);
    return hipGetLastError();
}

}  // namespace smoe

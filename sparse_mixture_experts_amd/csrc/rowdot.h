// Wave-level multi-row dot products: the building block of the HBM-streaming GEMV
// kernels (router logits, decode expert projections).
#pragma once

#include "common.h"

namespace smoe {

// The value itself, hidden from the optimiser: widening of register-resident weights is
// then done where it is written, not hoisted out of the row loop (which would hold the
// fp32 copy -- twice the registers).  The asm also pins instruction order, so every load
// of a step is issued before the first use of this.
__device__ __forceinline__ uint4 opaque(uint4 v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
    return v;
}

// One lane's activation chunk of V elements, as loaded (16-byte pieces, not widened).
template <typename TA, int V>
struct ARaw {
    static constexpr int Q = (V * (int)sizeof(typename TA::storage) + 15) / 16;
    uint4 q[Q];
};

template <typename TA, int V>
__device__ __forceinline__ void load_a(const typename TA::storage* p, ARaw<TA, V>& r) {
#pragma unroll
    for (int i = 0; i < ARaw<TA, V>::Q; ++i) r.q[i] = ld16(p + i * TA::VEC);
}

template <typename TA, int V>
__device__ __forceinline__ void widen_a(const ARaw<TA, V>& r, float (&f)[V]) {
#pragma unroll
    for (int i = 0; i < ARaw<TA, V>::Q; ++i) unpack16<TA>(r.q[i], f + i * TA::VEC);
}

// acc[r][t] += W_r . A_t over one 16-byte weight chunk per row (V = TW::VEC elements),
// from registers.  The operand with fewer rows is widened to fp32 in full first and the
// other one row at a time, which keeps the fewest floats live: weights first for
// NR <= NT, activations first for taller weight blocks.
template <int NR, int NT, typename TW, typename TA>
__device__ __forceinline__ void fma_chunk(const uint4 (&wv)[NR], const ARaw<TA, TW::VEC> (&av)[NT],
                                          float (&acc)[NR][NT]) {
    constexpr int V = TW::VEC;
    if constexpr (NR <= NT) {
        float wf[NR][V];
#pragma unroll
        for (int r = 0; r < NR; ++r) unpack16<TW>(opaque(wv[r]), wf[r]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float af[V];
            widen_a<TA, V>(av[t], af);
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int v = 0; v < V; ++v) acc[r][t] = fmaf(wf[r][v], af[v], acc[r][t]);
        }
    } else {
        float af[NT][V];
#pragma unroll
        for (int t = 0; t < NT; ++t) widen_a<TA, V>(av[t], af[t]);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float wf[V];
            unpack16<TW>(opaque(wv[r]), wf);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int v = 0; v < V; ++v) acc[r][t] = fmaf(wf[v], af[t][v], acc[r][t]);
        }
    }
}

// All-ones for a lane whose chunk starting at element e0 lies inside K, else zero, hidden
// from the optimiser: zeroing a loaded chunk with it cannot be turned back into an
// exec-masked load behind a branch (after which the compiler no longer counts the loads
// in flight and, at its next wait, waits for all of them).
__device__ __forceinline__ unsigned in_range_mask(int e0, int K) {
    unsigned m = e0 < K ? ~0u : 0u;
    asm("" : "+v"(m));
    return m;
}

__device__ __forceinline__ uint4 and_mask(uint4 q, unsigned m) {
    return make_uint4(q.x & m, q.y & m, q.z & m, q.w & m);
}

// Activation chunks of NT rows for the KB-chunk batch starting at chunk c0.  EXACT: every
// chunk of the batch lies inside K; otherwise chunks past K read the last in-range chunk
// and are zeroed (K >= V).
template <int NT, int KB, typename TW, typename TA, bool EXACT>
__device__ __forceinline__ void load_a_batch(const typename TA::storage* const (&a)[NT], int K, int c0,
                                             ARaw<TA, TW::VEC> (&av)[KB][NT]) {
    constexpr int V = TW::VEC;
    const int lane = lane_id();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int e0 = ((c0 + kb) * kWave + lane) * V;
        const int ec = EXACT ? e0 : min(e0, K - V);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            load_a<TA, V>(a[t] + ec, av[kb][t]);
            if constexpr (!EXACT) {
                const unsigned m = in_range_mask(e0, K);
#pragma unroll
                for (int i = 0; i < ARaw<TA, V>::Q; ++i) av[kb][t].q[i] = and_mask(av[kb][t].q[i], m);
            }
        }
    }
}

// Weights of NR rows held in registers: the KB-chunk batch starting at chunk c0 (EXACT
// and the tail as for load_a_batch).
template <int NR, int KB, typename TW, bool STREAM_W, bool EXACT>
__device__ __forceinline__ void load_w_batch(const typename TW::storage* const (&w)[NR], int K, int c0,
                                             uint4 (&wv)[KB][NR]) {
    constexpr int V = TW::VEC;
    const int lane = lane_id();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int e0 = ((c0 + kb) * kWave + lane) * V;
        const int ec = EXACT ? e0 : min(e0, K - V);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint4 q = STREAM_W ? ld16_stream(w[r] + ec) : ld16(w[r] + ec);
            if constexpr (EXACT) wv[kb][r] = q;
            else wv[kb][r] = and_mask(q, in_range_mask(e0, K));
        }
    }
}

// Activation chunks per load sub-batch: the largest divisor of KB that keeps it at most
// 16 16-byte pieces (64 registers).
template <int NT, int KB, typename TW, typename TA>
constexpr int act_sub_batch() {
    constexpr int per_chunk = NT * ARaw<TA, TW::VEC>::Q;
    int n = 16 / per_chunk;
    if (n > KB) n = KB;
    while (n > 1 && KB % n != 0) --n;
    return n < 1 ? 1 : n;
}

// acc[r][t] += W-batch (registers) . A_t over the batch's K range (same contract on a[t],
// nt and EXACT as rows_dot).  Chunks past K hold zero weights and activations.  The
// activations are loaded in sub-batches of at most 64 registers, each loaded in full
// before its arithmetic.
template <int NR, int NT, int KB, typename TW, typename TA, bool EXACT = false>
__device__ __forceinline__ void dot_w_batch(const uint4 (&wv)[KB][NR], const typename TA::storage* const (&a)[NT],
                                            int nt, int K, int c0, float (&acc)[NR][NT]) {
    (void)nt;
    constexpr int KBA = act_sub_batch<NT, KB, TW, TA>();
    static_assert(KB % KBA == 0, "sub-batches must tile the chunk batch");
#pragma unroll
    for (int k0 = 0; k0 < KB; k0 += KBA) {
        ARaw<TA, TW::VEC> av[KBA][NT];
        load_a_batch<NT, KBA, TW, TA, EXACT>(a, K, c0 + k0, av);
#pragma unroll
        for (int kb = 0; kb < KBA; ++kb) fma_chunk<NR, NT, TW, TA>(wv[k0 + kb], av[kb], acc);
    }
}

// acc[r][t] += sum_i W_r[i] * A_t[i] over i < K, for NR weight rows and NT activation
// rows, computed by one wave.  The K axis is cut into 16-byte chunks of W (TW::VEC
// elements); lane l takes chunks l, l+64, l+128, ...  Per batch of KB chunks, all
// NR*KB weight loads and NT*KB activation loads of a lane are issued before any
// arithmetic.  STREAM_W marks the W loads non-temporal (for weights read once per call).
// EXACT: K is a multiple of the batch span (64 * KB chunks), so no chunk needs a bound.
// Every a[t] must be readable over K (callers repeat their last row to fill NT); sums of
// rows t >= nt are computed and left for the caller to drop.
// The partial sums are per lane; the caller reduces them across the wave.
template <int NR, int NT, int KB, typename TW, typename TA, bool STREAM_W = false, bool EXACT = false>
__device__ __forceinline__ void rows_dot(const typename TW::storage* const (&w)[NR],
                                         const typename TA::storage* const (&a)[NT], int nt,
                                         int K, float (&acc)[NR][NT]) {
    static_assert(TW::VEC % TA::VEC == 0, "activation loads must tile the weight vector");
    (void)nt;
    const int nchunk = (K / TW::VEC + kWave - 1) / kWave;
    for (int c0 = 0; c0 < nchunk; c0 += KB) {
        uint4 wv[KB][NR];
        load_w_batch<NR, KB, TW, STREAM_W, EXACT>(w, K, c0, wv);
        dot_w_batch<NR, NT, KB, TW, TA, EXACT>(wv, a, nt, K, c0, acc);
    }
}

// Is K a whole number of KB-chunk batches (64 lanes x KB chunks of `vec` elements)?
inline bool exact_k(int K, int vec, int kb) { return K % (kWave * vec * kb) == 0; }

// 16-byte chunks per lane along a K axis of the given length.
inline int chunks(int K, int vec) { return (K / vec + 63) / 64; }

// Chunk-batch size for a K axis of the given length: the smallest of 1, 2, 4, 6, 8 that
// covers it in one batch, capped at 8 (longer axes loop over batches).  6 serves axes of
// 5-6 chunks per lane (K = 2880 in bf16 is 5.6) with a quarter fewer padded chunks than 8.
inline int pick_kb(int K, int vec) {
    int nchunk = (K / vec + 63) / 64;
    if (nchunk <= 1) return 1;
    if (nchunk <= 2) return 2;
    if (nchunk <= 4) return 4;
    if (nchunk <= 6) return 6;
    return 8;
}

}  // namespace smoe

// Wave-level multi-row dot products: the building block of the HBM-streaming GEMV
// kernels (router logits, decode expert projections).
#pragma once

#include "common.h"

namespace smoe {

// acc[r][t] += sum_i W_r[i] * A_t[i] over i < K, for NR weight rows and up to NT
// activation rows, computed by one wave.  The K axis is cut into 16-byte chunks of W
// (TW::VEC elements); lane l takes chunks l, l+64, l+128, ...  KB chunks per lane are
// loaded into registers before any arithmetic so that NR*KB independent 16-byte loads
// per lane are in flight.  STREAM_W marks the W loads non-temporal (for weights read
// once per call).  Tokens t >= nt are skipped.
// The partial sums are per lane; the caller reduces them across the wave.
template <int NR, int NT, int KB, typename TW, typename TA, bool STREAM_W = false>
__device__ __forceinline__ void rows_dot(const typename TW::storage* const (&w)[NR],
                                         const typename TA::storage* const (&a)[NT], int nt,
                                         int K, float (&acc)[NR][NT]) {
    constexpr int V = TW::VEC;
    static_assert(V % TA::VEC == 0, "activation loads must tile the weight vector");
    const int lane = lane_id();
    const int nchunk = (K / V + kWave - 1) / kWave;
    for (int c0 = 0; c0 < nchunk; c0 += KB) {
        uint4 wv[KB][NR];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int e0 = ((c0 + kb) * kWave + lane) * V;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                wv[kb][r] = (e0 < K) ? (STREAM_W ? ld16_stream(w[r] + e0) : ld16(w[r] + e0))
                                      : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int e0 = ((c0 + kb) * kWave + lane) * V;
            if (e0 >= K) continue;
            float wf[NR][V];
#pragma unroll
            for (int r = 0; r < NR; ++r) unpack16<TW>(wv[kb][r], wf[r]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t >= nt) continue;
                float af[V];
                load_as_f32<TA, V>(a[t] + e0, af);
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int v = 0; v < V; ++v) acc[r][t] = fmaf(wf[r][v], af[v], acc[r][t]);
            }
        }
    }
}

// Weights of NR rows held in registers: the KB-chunk batch starting at chunk c0.
template <int NR, int KB, typename TW, bool STREAM_W>
__device__ __forceinline__ void load_w_batch(const typename TW::storage* const (&w)[NR], int K, int c0,
                                             uint4 (&wv)[KB][NR]) {
    constexpr int V = TW::VEC;
    const int lane = lane_id();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int e0 = ((c0 + kb) * kWave + lane) * V;
#pragma unroll
        for (int r = 0; r < NR; ++r)
            wv[kb][r] = (e0 < K) ? (STREAM_W ? ld16_stream(w[r] + e0) : ld16(w[r] + e0))
                                  : make_uint4(0, 0, 0, 0);
    }
}

// acc[r][t] += W-batch (registers) . A_t over the batch's K range, tokens t < nt.
template <int NR, int NT, int KB, typename TW, typename TA>
__device__ __forceinline__ void dot_w_batch(const uint4 (&wv)[KB][NR], const typename TA::storage* const (&a)[NT],
                                            int nt, int K, int c0, float (&acc)[NR][NT]) {
    constexpr int V = TW::VEC;
    const int lane = lane_id();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int e0 = ((c0 + kb) * kWave + lane) * V;
        if (e0 >= K) continue;
        float wf[NR][V];
#pragma unroll
        for (int r = 0; r < NR; ++r) unpack16<TW>(wv[kb][r], wf[r]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t >= nt) continue;
            float af[V];
            load_as_f32<TA, V>(a[t] + e0, af);
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int v = 0; v < V; ++v) acc[r][t] = fmaf(wf[r][v], af[v], acc[r][t]);
        }
    }
}

// 16-byte chunks per lane along a K axis of the given length.
inline int chunks(int K, int vec) { return (K / vec + 63) / 64; }

// Chunk-batch size for a K axis of the given length: the smallest of 1, 2, 4, 8 that
// covers it in one batch, capped at 8 (longer axes loop over batches).
inline int pick_kb(int K, int vec) {
    int nchunk = (K / vec + 63) / 64;
    if (nchunk <= 1) return 1;
    if (nchunk <= 2) return 2;
    if (nchunk <= 4) return 4;
    return 8;
}

}  // namespace smoe

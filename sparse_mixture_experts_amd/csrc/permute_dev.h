// Device helpers of the expert grouping, shared by the permute kernels and the fused
// decode routing kernel.  See permute.hip for the method.
#pragma once

#include "common.h"
#include "internal.h"

namespace smoe {

constexpr int kMaxE = 512;

__device__ __forceinline__ void build_masks(const int32_t* __restrict__ idx, int T, int k, int E,
                                            int chunk, unsigned long long* mask) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
    const int t0 = chunk * kPermChunk;
    const int n = min(kPermChunk, T - t0) * k;
    for (int p = threadIdx.x; p < n; p += blockDim.x) {
        const int tl = p / k;
        const int e = idx[(size_t)t0 * k + p];
        if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << tl);
    }
    __syncthreads();
}

__device__ __forceinline__ void scatter_chunk(const int32_t* __restrict__ idx, int T, int k, int E,
                                              int chunk, const unsigned long long* mask,
                                              const int32_t* base_row, int32_t* __restrict__ perm_token,
                                              int32_t* __restrict__ perm_inv, const float* __restrict__ w,
                                              float* __restrict__ row_w) {
    const int t0 = chunk * kPermChunk;
    const int n = min(kPermChunk, T - t0) * k;
    for (int p = threadIdx.x; p < n; p += blockDim.x) {
        const int tl = p / k;
        const size_t flat = (size_t)t0 * k + p;
        const int e = idx[flat];
        if (e >= 0 && e < E) {
            const int rank = __popcll(mask[e] & ((1ull << tl) - 1ull));
            const int pos = base_row[e] + rank;
            perm_token[pos] = t0 + tl;
            perm_inv[flat] = pos;
            if (row_w) row_w[pos] = w[flat];
        } else {
            perm_inv[flat] = -1;
        }
    }
}

// Group list for the expert kernels: every non-empty expert in ascending id, then the
// shared expert (e = -1) over rows T*k .. T*k+T-1.  tile0 = first M-tile of the group
// when groups are cut into tiles of tile_m rows; tiles (optional) gets the descriptor of
// every M-tile (at most tile_cap entries).
// Runs on one block with blockDim.x >= E; `tmp` holds 2 * blockDim.x / 64 ints of LDS.
__device__ __forceinline__ void plan_block(const int32_t* offsets, int E, int T, int k, int shared,
                                           int tile_m, Group* __restrict__ groups,
                                           PlanMeta* __restrict__ meta, TileDesc* __restrict__ tiles_out,
                                           int tile_cap, int* tmp) {
    const int e = threadIdx.x;
    // Offsets may come from the caller: clamp them so every group stays inside the
    // T*k grouped rows whatever they hold.
    const int tk = T * k;
    const int row0 = e < E ? min(max(offsets[e], 0), tk) : 0;
    const int n = e < E ? min(max(offsets[e + 1] - row0, 0), tk - row0) : 0;
    const int flag = n > 0 ? 1 : 0;
    const int tiles = n > 0 ? (n + tile_m - 1) / tile_m : 0;
    const int in[2] = {flag, tiles};
    int ex[2], tot[2];
    block_exclusive_scan_n<2>(in, tmp, ex, tot);
    const int pos = ex[0], tile0 = ex[1], n_active = tot[0], n_tiles = tot[1];
    if (flag) {
        groups[pos] = Group{e, row0, n, tile0};
        if (tiles_out)
            for (int i = 0; i < tiles && tile0 + i < tile_cap; ++i)
                tiles_out[tile0 + i] = TileDesc{e, row0 + i * tile_m, min(tile_m, n - i * tile_m), pos};
    }
    if (e == 0) {
        int ng = n_active, nt = n_tiles;
        if (shared) {
            groups[ng] = Group{-1, T * k, T, nt};
            const int st = (T + tile_m - 1) / tile_m;
            if (tiles_out)
                for (int i = 0; i < st && nt + i < tile_cap; ++i)
                    tiles_out[nt + i] = TileDesc{-1, T * k + i * tile_m, min(tile_m, T - i * tile_m), ng};
            ++ng;
            nt += st;
        }
        meta->n_groups = ng;
        // Offsets from a caller may overlap; never hand out tiles beyond the map.
        meta->n_tiles = min(nt, tile_cap);
        meta->pad0 = meta->pad1 = 0;
    }
}


// Grouping, group list and M-tile descriptors of at most 64 routed rows (T * k <= 64,
// tile_m >= 64) by one wave, for the decode routing kernel.  Lane p holds entry p (token
// p / k, slot p % k, expert idx[p]); the order is the same as the chunked path's:
// ascending expert, then ascending p (ascending token).  A radix rank over the expert id
// bits (ballots from the top bit down) gives each entry the number of entries with a
// smaller expert and, among those with the same expert, the ones before it.  Each group
// holds at most 64 rows, so it is one M-tile.  Out-of-range ids get perm_inv = -1.
__device__ __forceinline__ void group_wave_small(const int32_t* idx, const float* w, int T, int k, int E,
                                                 int shared, int32_t* __restrict__ perm_token,
                                                 int32_t* __restrict__ perm_inv, float* __restrict__ row_w,
                                                 Group* __restrict__ groups, PlanMeta* __restrict__ meta,
                                                 TileDesc* __restrict__ tiles, int tile_cap) {
    const int lane = lane_id();
    const int n = T * k;
    const bool valid = lane < n;
    const int e = valid ? idx[lane] : -1;
    const bool ok = valid && e >= 0 && e < E;
    unsigned long long eq = __ballot(ok), less = 0ull;
#pragma unroll
    for (int b = 9; b >= 0; --b) {  // E <= 512 < 2^10
        const bool bit = (e >> b) & 1;
        const unsigned long long B = __ballot(ok && bit);
        less = bit ? (less | (eq & ~B)) : less;
        eq = bit ? (eq & B) : (eq & ~B);
    }
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(less) + __popcll(eq & below);
    const bool first = ok && (eq & below) == 0ull;
    const unsigned long long firsts = __ballot(first);
    const int gi = __popcll(firsts & less);
    if (ok) {
        perm_token[rank] = lane / k;
        if (row_w) row_w[rank] = w[lane];
    }
    if (valid) perm_inv[lane] = ok ? rank : -1;
    if (first) {
        const int cnt = __popcll(eq);
        groups[gi] = Group{e, rank, cnt, gi};
        if (tiles && gi < tile_cap) tiles[gi] = TileDesc{e, rank, cnt, gi};
    }
    if (lane == 0) {
        int ng = __popcll(firsts);
        if (shared) {
            groups[ng] = Group{-1, n, T, ng};
            if (tiles && ng < tile_cap) tiles[ng] = TileDesc{-1, n, T, ng};
            ++ng;
        }
        meta->n_groups = ng;
        meta->n_tiles = min(ng, tile_cap);
        meta->pad0 = meta->pad1 = 0;
    }
}

}  // namespace smoe

// Expert grouping ("Engine" (Cherenkov), section "Prefill"): the T*k (token, slot) pairs
// are reordered so that each expert's rows are contiguous, by a deterministic counting
// sort with the tokens in ascending order inside each expert.
//
// Tokens are cut into chunks of 64.  For each chunk and expert an LDS 64-bit mask marks
// the chunk's tokens that selected the expert (LDS atomic OR: order-free, so the
// result is deterministic).  counts = popcount(mask); a scan down each expert's column
// of chunk counts plus a scan of the expert totals give every chunk's base row per
// expert; the rank of token t inside its chunk is popcount(mask & bits below t).  A token selects an expert at most once,
// so this rank is exactly the stable (token-ascending) position.
//
// Also here: the plan kernel that turns expert offsets into the list of non-empty
// groups (and M-tiles) the expert kernels iterate over, the decode view of the
// "Engine" page's address table (the union of the experts a batch selects).
#include "common.h"
#include "internal.h"
#include "permute_dev.h"

namespace smoe {
namespace {

// Pass 1 (several chunks): per-chunk counts[chunk][e].
__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx, int T,
                                                            int k, int E, int32_t* __restrict__ counts) {
    __shared__ unsigned long long mask[kMaxE];
    build_masks(idx, T, k, E, blockIdx.x, mask);
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        counts[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
}

// Pass 2 (one block per expert e): base[chunk][e] = rows of expert e in earlier chunks
// (a block-wide scan down the column), and totals[e] = rows of expert e (row n_chunks
// of `base`).
__global__ __launch_bounds__(256) void permute_colscan_kernel(const int32_t* __restrict__ counts,
                                                              int n_chunks, int E, int32_t* __restrict__ base) {
    __shared__ int tmp[256 / kWave];
    const int e = blockIdx.x;
    int carry = 0;
    for (int c0 = 0; c0 < n_chunks; c0 += blockDim.x) {
        const int c = c0 + threadIdx.x;
        const int v = c < n_chunks ? counts[(size_t)c * E + e] : 0;
        int total;
        const int excl = block_exclusive_scan(v, tmp, &total);
        if (c < n_chunks) base[(size_t)c * E + e] = carry + excl;
        carry += total;
    }
    if (threadIdx.x == 0) base[(size_t)n_chunks * E + e] = carry;
}

// Pass 3 (several chunks): stable scatter.
// Every block first turns the expert totals into offsets (exclusive scan over E <= 512
// in LDS, two experts per thread); block 0 also writes them out.
__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t* __restrict__ idx, int T,
                                                              int k, int E, int n_chunks,
                                                              const int32_t* __restrict__ base,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm_token,
                                                              int32_t* __restrict__ perm_inv,
                                                              const float* __restrict__ w,
                                                              float* __restrict__ row_w) {
    __shared__ unsigned long long mask[kMaxE];
    __shared__ int32_t base_row[kMaxE];
    __shared__ int tmp[256 / kWave];
    build_masks(idx, T, k, E, blockIdx.x, mask);
    const int32_t* totals = base + (size_t)n_chunks * E;
    const int e0 = 2 * threadIdx.x;
    const int v0 = e0 < E ? totals[e0] : 0, v1 = e0 + 1 < E ? totals[e0 + 1] : 0;
    int all;
    const int off0 = block_exclusive_scan(v0 + v1, tmp, &all);
    if (e0 < E) base_row[e0] = off0 + base[(size_t)blockIdx.x * E + e0];
    if (e0 + 1 < E) base_row[e0 + 1] = off0 + v0 + base[(size_t)blockIdx.x * E + e0 + 1];
    if (blockIdx.x == 0) {
        if (e0 < E) offsets[e0] = off0;
        if (e0 + 1 < E) offsets[e0 + 1] = off0 + v0;
        if (threadIdx.x == 0) offsets[E] = all;
    }
    __syncthreads();
    scatter_chunk(idx, T, k, E, blockIdx.x, mask, base_row, perm_token, perm_inv, w, row_w);
}

// T <= 64: all three passes in one block of 512 threads.
__global__ __launch_bounds__(512) void permute_single_kernel(const int32_t* __restrict__ idx, int T,
                                                             int k, int E, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm_token,
                                                             int32_t* __restrict__ perm_inv,
                                                             const float* __restrict__ w,
                                                             float* __restrict__ row_w) {
    __shared__ unsigned long long mask[kMaxE];
    __shared__ int32_t base_row[kMaxE];
    __shared__ int tmp[512 / kWave];
    build_masks(idx, T, k, E, 0, mask);
    const int e = threadIdx.x;
    const int cnt = e < E ? __popcll(mask[e]) : 0;
    int total;
    const int off = block_exclusive_scan(cnt, tmp, &total);
    if (e < E) {
        base_row[e] = off;
        offsets[e] = off;
    }
    if (e == 0) offsets[E] = total;
    __syncthreads();
    scatter_chunk(idx, T, k, E, 0, mask, base_row, perm_token, perm_inv, w, row_w);
}

__global__ __launch_bounds__(512) void plan_kernel(const int32_t* __restrict__ offsets, int E, int T,
                                                   int k, int shared, int tile_m, Group* __restrict__ groups,
                                                   PlanMeta* __restrict__ meta,
                                                   TileDesc* __restrict__ tiles, int tile_cap) {
    __shared__ int tmp[2 * 512 / kWave];
    plan_block(offsets, E, T, k, shared, tile_m, groups, meta, tiles, tile_cap, tmp);
}

}  // namespace

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* perm_token, int32_t* perm_inv, int32_t* counts, int32_t* base,
                          const float* w, float* row_w, hipStream_t s) {
    const int n_chunks = (T + kPermChunk - 1) / kPermChunk;
    if (n_chunks == 1) {
        permute_single_kernel<<<1, 512, 0, s>>>(idx, T, k, E, offsets, perm_token, perm_inv, w, row_w);
        return hipGetLastError();
    }
    permute_count_kernel<<<n_chunks, 256, 0, s>>>(idx, T, k, E, counts);
    permute_colscan_kernel<<<E, 256, 0, s>>>(counts, n_chunks, E, base);
    permute_scatter_kernel<<<n_chunks, 256, 0, s>>>(idx, T, k, E, n_chunks, base, offsets, perm_token,
                                                    perm_inv, w, row_w);
    return hipGetLastError();
}

hipError_t launch_plan(const int32_t* offsets, int E, int T, int k, bool shared, int tile_m,
                       Group* groups, PlanMeta* meta, TileDesc* tiles, hipStream_t s) {
    plan_kernel<<<1, 512, 0, s>>>(offsets, E, T, k, shared ? 1 : 0, tile_m, groups, meta, tiles,
                                  grouped_max_mtiles(E, T, k, shared));
    return hipGetLastError();
}

}  // namespace smoe

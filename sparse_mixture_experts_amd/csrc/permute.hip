// Expert grouping ("Engine" (Cherenkov), Prefill: tokens grouped by expert, gathered,
// projected, scattered back) as a deterministic counting sort of the T*k (token, slot)
// pairs by expert, tokens ascending inside each expert.
//
// Tokens are cut into chunks of 64.  For each chunk and expert an LDS 64-bit mask marks
// the chunk's tokens that selected the expert (LDS atomic OR: order-free, so the
// result is deterministic).  counts = popcount(mask); an exclusive scan over
// (expert, chunk) gives every chunk's base row per expert; the rank of token t inside
// its chunk is popcount(mask & bits below t).  A token selects an expert at most once,
// so this rank is exactly the stable (token-ascending) position.
//
// Also here: the plan kernel that turns expert offsets into the list of non-empty
// groups (and M-tiles) the expert kernels iterate over, the decode view of the
// "Engine" page's address table (the union of the experts a batch selects).
#include "common.h"
#include "internal.h"

namespace smoe {
namespace {

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
                                              int32_t* __restrict__ perm_inv) {
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
        } else {
            perm_inv[flat] = -1;
        }
    }
}

// Pass 1 (several chunks): per-chunk counts[chunk][e].
__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx, int T,
                                                            int k, int E, int32_t* __restrict__ counts) {
    __shared__ unsigned long long mask[kMaxE];
    build_masks(idx, T, k, E, blockIdx.x, mask);
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        counts[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
}

// Pass 2 (one block of 512 threads, E <= 512): base[chunk][e] = offsets[e] + rows of
// expert e in earlier chunks; offsets[E+1] = exclusive scan of the expert totals.
__global__ __launch_bounds__(512) void permute_scan_kernel(const int32_t* __restrict__ counts,
                                                           int n_chunks, int E, int32_t* __restrict__ base,
                                                           int32_t* __restrict__ offsets) {
    __shared__ int tmp[512 / kWave];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E)
        for (int c = 0; c < n_chunks; ++c) {
            const int v = counts[(size_t)c * E + e];
            base[(size_t)c * E + e] = run;
            run += v;
        }
    int total;
    const int off = block_exclusive_scan(e < E ? run : 0, tmp, &total);
    if (e < E) {
        offsets[e] = off;
        for (int c = 0; c < n_chunks; ++c) base[(size_t)c * E + e] += off;
    }
    if (e == 0) offsets[E] = total;
}

// Pass 3 (several chunks): stable scatter.
__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t* __restrict__ idx, int T,
                                                              int k, int E, const int32_t* __restrict__ base,
                                                              int32_t* __restrict__ perm_token,
                                                              int32_t* __restrict__ perm_inv) {
    __shared__ unsigned long long mask[kMaxE];
    __shared__ int32_t base_row[kMaxE];
    build_masks(idx, T, k, E, blockIdx.x, mask);
    for (int e = threadIdx.x; e < E; e += blockDim.x) base_row[e] = base[(size_t)blockIdx.x * E + e];
    __syncthreads();
    scatter_chunk(idx, T, k, E, blockIdx.x, mask, base_row, perm_token, perm_inv);
}

// T <= 64: all three passes in one block of 512 threads.
__global__ __launch_bounds__(512) void permute_single_kernel(const int32_t* __restrict__ idx, int T,
                                                             int k, int E, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm_token,
                                                             int32_t* __restrict__ perm_inv) {
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
    scatter_chunk(idx, T, k, E, 0, mask, base_row, perm_token, perm_inv);
}

// Group list for the expert kernels: every non-empty expert in ascending id, then the
// shared expert (e = -1) over rows T*k .. T*k+T-1.  tile0 = first M-tile of the group
// when groups are cut into tiles of tile_m rows.
__global__ __launch_bounds__(512) void plan_kernel(const int32_t* __restrict__ offsets, int E, int T,
                                                   int k, int shared, int tile_m, Group* __restrict__ groups,
                                                   PlanMeta* __restrict__ meta) {
    __shared__ int tmp[512 / kWave];
    const int e = threadIdx.x;
    // Offsets may come from the caller: clamp them so every group stays inside the
    // T*k grouped rows whatever they hold.
    const int tk = T * k;
    const int row0 = e < E ? min(max(offsets[e], 0), tk) : 0;
    const int n = e < E ? min(max(offsets[e + 1] - row0, 0), tk - row0) : 0;
    const int flag = n > 0 ? 1 : 0;
    const int tiles = n > 0 ? (n + tile_m - 1) / tile_m : 0;
    int n_active, n_tiles;
    const int pos = block_exclusive_scan(flag, tmp, &n_active);
    const int tile0 = block_exclusive_scan(tiles, tmp, &n_tiles);
    if (flag) groups[pos] = Group{e, row0, n, tile0};
    if (e == 0) {
        int ng = n_active, nt = n_tiles;
        if (shared) {
            groups[ng] = Group{-1, T * k, T, nt};
            ++ng;
            nt += (T + tile_m - 1) / tile_m;
        }
        meta->n_groups = ng;
        meta->n_tiles = nt;
        meta->pad0 = meta->pad1 = 0;
    }
}

}  // namespace

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* perm_token, int32_t* perm_inv, int32_t* counts, int32_t* base,
                          hipStream_t s) {
    const int n_chunks = (T + kPermChunk - 1) / kPermChunk;
    if (n_chunks == 1) {
        permute_single_kernel<<<1, 512, 0, s>>>(idx, T, k, E, offsets, perm_token, perm_inv);
        return hipGetLastError();
    }
    permute_count_kernel<<<n_chunks, 256, 0, s>>>(idx, T, k, E, counts);
    permute_scan_kernel<<<1, 512, 0, s>>>(counts, n_chunks, E, base, offsets);
    permute_scatter_kernel<<<n_chunks, 256, 0, s>>>(idx, T, k, E, base, perm_token, perm_inv);
    return hipGetLastError();
}

hipError_t launch_plan(const int32_t* offsets, int E, int T, int k, bool shared, int tile_m,
                       Group* groups, PlanMeta* meta, hipStream_t s) {
    plan_kernel<<<1, 512, 0, s>>>(offsets, E, T, k, shared ? 1 : 0, tile_m, groups, meta);
    return hipGetLastError();
}

}  // namespace smoe

// Host-side launchers shared between the translation units of libsmoe.so.
// Every launcher only enqueues work on `s`; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace smoe {

// Tokens per permute chunk: one 64-bit token mask per expert and chunk.
constexpr int kPermChunk = 64;

// One group of grouped rows handled by the expert kernels: expert e (-1 = shared
// expert), its first grouped row, its row count and its first M-tile.
struct Group {
    int32_t e, row0, n, tile0;
};

// Plan metadata written next to the group list: number of groups, number of M-tiles.
struct PlanMeta {
    int32_t n_groups, n_tiles, pad0, pad1;
};

inline int max_groups(int E, int T, int k, bool shared) {
    long long tk = (long long)T * k;
    return int((tk < E ? tk : E) + (shared ? 1 : 0));
}

hipError_t launch_router_logits(const moe_layer& L, const void* x, int T, float* logits, int ld,
                                hipStream_t s);
hipError_t launch_topk(const moe_layer& L, const float* logits, int ld, int T, int32_t* idx,
                       float* w, float* shared_gate, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* perm_token, int32_t* perm_inv, int32_t* counts, int32_t* base,
                          hipStream_t s);
hipError_t launch_plan(const int32_t* offsets, int E, int T, int k, bool shared, int tile_m,
                       Group* groups, PlanMeta* meta, hipStream_t s);
hipError_t launch_expert_gemv(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                              const Group* groups, const PlanMeta* meta, float* H, int hstride,
                              float* y_perm, hipStream_t s);
hipError_t launch_combine(const moe_layer& L, const float* y_perm, const int32_t* perm_inv,
                          const float* w, const float* shared_gate, int T, void* y, hipStream_t s);

}  // namespace smoe

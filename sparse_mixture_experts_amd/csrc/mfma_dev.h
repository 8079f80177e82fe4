// Device helpers of the MFMA kernels: fragment types, the swizzled LDS row layouts,
// wait-count and barrier primitives.
#pragma once

#include "common.h"

namespace smoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ float ld_bf16(const uint16_t* p) { return bf16_to_f32(*p); }

// LDS row layouts.  Rows of 64 bf16 (8 chunks of 16 B): chunk c of row r at
// c ^ ((r >> 1) & 7).  Rows of 32 bf16 (4 chunks): chunk c of row r at c ^ ((r >> 2) & 3).
// Either way 16 rows read at one logical chunk cover 64 distinct banks.
template <int KW>
__device__ __forceinline__ int swz_chunk(int r, int c) {
    if constexpr (KW == 64) return c ^ ((r >> 1) & 7);
    else return c ^ ((r >> 2) & 3);
}

template <int KW>
__device__ __forceinline__ int swz(int r, int c) {
    return r * KW + (swz_chunk<KW>(r, c) << 3);
}

template <int KW>
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* lds, int row, int chunk) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + swz<KW>(row, chunk)));
}

template <int MI, int NI>
__device__ __forceinline__ void zero(floatx4 (&acc)[MI][NI]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt: no wait): this lane's vector-memory ops but the
// newest N are done, and all of its LDS ops are.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (whose release would
// drain the direct loads still in flight); the memory clobber keeps the compiler from
// moving LDS accesses across it.  Ordering of the direct LDS loads is by wait_vm_lgkm.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) only (LDS and scalar counters not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait for this wave's LDS (and scalar) operations, then a workgroup barrier: LDS writes
// of every wave are visible afterwards.  Vector-memory operations stay in flight.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("s_barrier" ::: "memory");
}

}  // namespace smoe

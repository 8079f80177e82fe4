// Device helpers shared by the kernels of libsmoe.so (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smoe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 <-> fp32
// bf16 values are carried as raw uint16 bits; widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32 (the compiler packs two
// neighbouring conversions into one instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Element type tags: the kernels are templated on the storage type of weights and
// activations.  VEC = elements per 16-byte load.
struct BF16 { using storage = uint16_t; static constexpr int VEC = 8; };
struct F32  { using storage = float;    static constexpr int VEC = 4; };

// Unpack one 16-byte vector into VEC floats.
template <typename TT> __device__ __forceinline__ void unpack16(const uint4& v, float* out);
template <> __device__ __forceinline__ void unpack16<BF16>(const uint4& v, float* o) {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
}
template <> __device__ __forceinline__ void unpack16<F32>(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Streaming load for weights that are read once per call.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Load N consecutive elements of type TT starting at p as floats (N a multiple of VEC).
template <typename TT, int N>
__device__ __forceinline__ void load_as_f32(const typename TT::storage* p, float* out) {
#pragma unroll
    for (int i = 0; i < N / TT::VEC; ++i) unpack16<TT>(ld16(p + i * TT::VEC), out + i * TT::VEC);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave index in the block, marked wave-uniform so that addresses built from it stay in
// scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// 1 / (1 + e^-a) with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE
// division: ten instructions fewer per value in the activation epilogues.
__device__ __forceinline__ float sigmoidf_(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// ---------------------------------------------------------------- wave reduce-scatter
// Butterfly sum of N values per lane across the wave (N a power of two, 1..64), in
// 63 lane exchanges for N = 64 instead of 6 per value.  Step b (lane bit 5 down to 0)
// pairs each lane with the lane differing in bit b -- through v_permlane32_swap and
// v_permlane16_swap for bits 5 and 4, through DPP row mirror, half-row mirror and quad
// permutes for bits 3..0 (those partners also differ in lower bits, which no earlier
// step has used) -- and, while more than one value remains, each lane keeps the half of
// the values named by its bit and adds its partner's copy of that half.  On return every
// lane holds the wave total of value index lane >> (6 - log2 N).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int B>
__device__ __forceinline__ void lane_pair_swap(float& a, float& b) {
    // After the swap, a + b sums the lower-half value in lanes with bit B clear and the
    // upper-half value in lanes with bit B set, each with its partner's copy.
    if constexpr (B == 5) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    }
}

template <int B>
constexpr int lane_pair_dpp() {
    return B == 3 ? 0x140 : B == 2 ? 0x141 : B == 1 ? 0x4E : 0xB1;
}

template <int B, int H>
__device__ __forceinline__ void butterfly_split(float* v) {
    if constexpr (B >= 4) {
#pragma unroll
        for (int i = 0; i < H; ++i) {
            float a = v[i], b = v[H + i];
            lane_pair_swap<B>(a, b);
            v[i] = a + b;
        }
    } else {
        const bool upper = (lane_id() >> B) & 1;
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float keep = upper ? v[H + i] : v[i];
            const float give = upper ? v[i] : v[H + i];
            v[i] = keep + dpp_f32<lane_pair_dpp<B>()>(give);
        }
    }
}

template <int B>
__device__ __forceinline__ float butterfly_full(float x) {
    if constexpr (B >= 4) {
        float a = x, b = x;
        lane_pair_swap<B>(a, b);
        return a + b;
    } else {
        return x + dpp_f32<lane_pair_dpp<B>()>(x);
    }
}

template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[N]) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
    if constexpr (N >= 2) butterfly_split<5, N / 2>(v);
    if constexpr (N >= 4) butterfly_split<4, N / 4>(v);
    if constexpr (N >= 8) butterfly_split<3, N / 8>(v);
    if constexpr (N >= 16) butterfly_split<2, N / 16>(v);
    if constexpr (N >= 32) butterfly_split<1, N / 32>(v);
    if constexpr (N >= 64) butterfly_split<0, N / 64>(v);
    float x = v[0];
    if constexpr (N < 2) x = butterfly_full<5>(x);
    if constexpr (N < 4) x = butterfly_full<4>(x);
    if constexpr (N < 8) x = butterfly_full<3>(x);
    if constexpr (N < 16) x = butterfly_full<2>(x);
    if constexpr (N < 32) x = butterfly_full<1>(x);
    if constexpr (N < 64) x = butterfly_full<0>(x);
    return x;
}

// log2 of a power of two, at compile time.
constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// ---------------------------------------------------------------- scans
// Inclusive prefix sum over the wave through DPP: shifts right by 1, 2, 4 and 8 lanes
// inside each 16-lane row (lanes without a source add the zero `old`), then the row
// broadcasts add row 0's total into row 1, row 2's into row 3, and rows 0-1's into rows
// 2-3.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
    return v;
}

// Exclusive prefix sums of N ints per thread over the whole block (blockDim.x <= 1024, a
// multiple of 64), all N in one pass.  `tmp` must hold N * blockDim.x / 64 ints of LDS.
// excl[i] receives the exclusive prefix of v[i], total[i] the block total.
template <int N>
__device__ __forceinline__ void block_exclusive_scan_n(const int (&v)[N], int* tmp, int (&excl)[N],
                                                       int (&total)[N]) {
    const int lane = lane_id(), wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
    int incl[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        incl[i] = wave_inclusive_sum(v[i]);
        if (lane == kWave - 1) tmp[i * nw + wave] = incl[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        int wave_base = 0, all = 0;
        for (int w = 0; w < nw; ++w) {
            const int s = tmp[i * nw + w];
            if (w < wave) wave_base += s;
            all += s;
        }
        excl[i] = wave_base + incl[i] - v[i];
        total[i] = all;
    }
    __syncthreads();
}

// One value per thread: returns the exclusive prefix, *total the block total.  `tmp` must
// hold blockDim.x / 64 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
    const int in[1] = {v};
    int ex[1], tot[1];
    block_exclusive_scan_n<1>(in, tmp, ex, tot);
    *total = tot[0];
    return ex[0];
}

}  // namespace smoe

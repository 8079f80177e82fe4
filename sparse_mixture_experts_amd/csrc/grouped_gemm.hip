// Grouped GEMMs of the expert FFNs on bf16 MFMA (the prefill path), and the dense router
// GEMM of large batches.
//
// "Engine" (Cherenkov), section "Prefill", evaluates an expert once over all the tokens
// routed to it, with token tiles, half-precision weights and float accumulation.  Here
// every group (one expert's rows, or the shared expert over all
// tokens) is cut into 128-row M-tiles; a block computes one 128-row tile against one
// 256-row slice of the expert's weights with v_mfma_f32_16x16x32_bf16 and fp32
// accumulation.
//
// Up kernel: rows of x gathered through perm_token, times the 128 gate rows and the 128
// matching up rows of a 128-unit slice of the hidden layer (for the clamped variant the
// interleaved gate_up rows are de-interleaved while staging), then the activation of
// "Qwen3.5-MoE Model Implementation" (silu(gate) * up) or of "Phase 19: MoE -
// gpt-oss-20b", Experts (biases, clamps, (up + 1) * gate * sigmoid(alpha * gate)) in
// the epilogue; H is stored in bf16.
// Down kernel: H rows times a 256-column slice of W_d (+ down bias), optionally scaled
// by each row's routing weight (or the shared expert's sigmoid gate) so that the
// combine is a plain sum; output bf16 or fp32.
//
// Grouped block: 512 threads = 8 waves in a 2 x 4 grid over a 128 x 256 output tile, each
// wave a 64 x 64 tile = 4 x 4 MFMA tiles.  K advances one slice (64 for the up kernel,
// 32 for the down kernel) per step through a 3-stage LDS ring filled straight from global
// memory by global_load_lds_dwordx4 (no register round trip, no LDS store instructions);
// slice s is issued two steps before it is used, and one barrier per step both publishes
// slice s and frees the stage that the next issue overwrites.  Ring rows of 64 bf16
// (8 chunks of 16 B) store chunk c of row r at c ^ ((r >> 1) & 7), rows of 32 bf16 at
// c ^ ((r >> 2) & 3): 16 rows read at one logical chunk touch 64 distinct banks.  A wave's
// direct load writes 64 consecutive 16-byte slots (8 or 16 rows), so each lane fetches the
// global chunk that belongs in its slot.  Whole 128-byte rows per slice halve the L2
// requests of 64-byte rows (each request returns a full cache line); that pays in the up
// kernel's long K loop.  Epilogues go through LDS so that every lane
// stores whole 16-byte chunks of output rows.
//
// The router GEMM (128, 64 or 32 tokens x 128 experts per block) keeps a 4-wave,
// register-staged pipeline: with E = 256 experts a 256-wide tile would leave too few
// blocks.  MXFP4 expert weights take the same loops with their B slices expanded from FP4
// blocks into the ring, and Q4_K weights from their super-blocks (see
// grouped_mainloop_regb).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_dev.h"
#include "mxfp4_dev.h"
#include "q4k_dev.h"

namespace smoe {
namespace {

constexpr int BM = kGroupTileM;  // rows per M-tile

// 32 K of one wave's (16 MI) x 64 tile: MI A and 4 B fragments from LDS, 4 MI MFMAs.
// Fragment layout of v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 of its
// 16-row block and the 8 K values of chunk (l / 16); A and B use the same chunk map, so
// the order of K inside the 32 does not matter.
template <int KW, int MI = 4>
__device__ __forceinline__ void mfma_k32(const uint16_t* sa, const uint16_t* sb, int arow0,
                                         const int (&brow)[4], int kc, floatx4 (&acc)[MI][4]) {
    const int lane = lane_id();
    const int fr = lane & 15, fc = lane >> 4;
    bf16x8 af[MI], bfr[4];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) af[mi] = lds_frag<KW>(sa, arow0 + mi * 16 + fr, kc + fc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) bfr[ni] = lds_frag<KW>(sb, brow[ni] + fr, kc + fc);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
}

// =====================================================================================
// Grouped GEMM: 8 waves, 128 x 256 block tile, direct-to-LDS 3-stage ring of K-slices
// KW wide.  Up: KW = 64 (128-byte LDS rows, whole cache lines per row; 144 KB of LDS, one
// block per CU).  Down (K = ff, a few slices per tile): KW = 32 (72 KB, two blocks per
// CU, so one block's prologue and epilogue overlap the other's main loop).
// =====================================================================================
constexpr int GBN = 256;
constexpr int kGThreads = 512;
constexpr int kStages = 3;
constexpr int kUpKW = 64;
constexpr int kDownKW = 32;

template <int KW>
struct Ring {
    static constexpr int kRowsPerSeg = 1024 / (KW * 2);  // LDS rows per 1 KB direct-load segment
    static constexpr int kChunksPerRow = KW / 8;
    static constexpr int kSegA = BM / kRowsPerSeg;        // segments per A slice
    static constexpr int kSegB = GBN / kRowsPerSeg;       // ... per B slice
    static constexpr int kLoadsA = kSegA / 8, kLoadsB = kSegB / 8;  // per wave (8 waves)
    static constexpr int kLoads = kLoadsA + kLoadsB;                  // direct loads per lane per slice
};

constexpr int kUpStage = 128 + 8;       // bf16 H tile 128 x 128
constexpr int kDownStageH = GBN + 8;    // bf16 output tile 128 x 256
constexpr int kDownStageF = GBN / 2 + 4;  // fp32 output tile, one 128-column half at a time

template <int KW>
struct GSmem {
    union {
        struct {
            uint16_t a[kStages][BM * KW];
            uint16_t b[kStages][GBN * KW];
        } k;
        uint16_t up[BM * kUpStage];
        uint16_t down_h[BM * kDownStageH];
        float down_f[BM * kDownStageF];
    };
    float row_w[BM];  // down epilogue: the tile rows' routing weights
};

// Blocks that fit one CU's 160 KB of LDS (at most 2).
template <int KW>
constexpr int blocks_per_cu() { return sizeof(GSmem<KW>) * 2 <= 160 * 1024 ? 2 : 1; }

// Source pointers of this lane's direct loads: A segments w + 8j, B segments w + 8j
// (segment s holds tile rows s * kRowsPerSeg ..).  row_a / row_b map a tile row to its
// global row.
// Slice s of load j starts at src[j] + s * KW * mul (mul_a for the A loads, mul_b for B):
// mul 1 for row-major operands, the row count for operands stored slice-major (the bf16
// hidden rows H of the grouped path; the grouped copy of dense W_d).
template <int KW>
struct LoadPlan {
    const uint16_t* src[Ring<KW>::kLoads];
    int mul_a, mul_b;
};

// A_ONLY: B comes from MXFP4 blocks through registers (mx_load / mx_store), so only the A
// segments are direct loads; row_b is not called.
template <int KW, bool A_ONLY = false, typename RowA, typename RowB>
__device__ __forceinline__ LoadPlan<KW> make_plan(RowA row_a, RowB row_b) {
    using R = Ring<KW>;
    LoadPlan<KW> p;
    p.mul_a = 1;
    p.mul_b = 1;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < R::kLoads; ++j) {
        const bool is_a = j < R::kLoadsA;
        const int seg = wave + 8 * (is_a ? j : j - R::kLoadsA);
        const int r = seg * R::kRowsPerSeg + lane / R::kChunksPerRow;
        const int slot = lane % R::kChunksPerRow;
        const int c = swz_chunk<KW>(r, slot);  // logical chunk that belongs in this slot (the map is an involution)
        if (A_ONLY && !is_a) p.src[j] = nullptr;
        else p.src[j] = (is_a ? row_a(r) : row_b(r)) + c * 8;
    }
    return p;
}

// The direct loads of one K-slice (from src[j] + k0) into ring stage (a_stage, b_stage).
// NTB: the weight (B) loads are non-temporal -- for launches whose every weight slice is read
// by one block only (batches of at most 128 tokens: no group has a second M-tile), where the
// streaming loads reach a higher HBM rate; with several M-tiles per expert they would evict
// the slices the later M-tiles re-read from L2.
template <int KW, bool NTB = false>
__device__ __forceinline__ void issue_stage(uint16_t* a_stage, uint16_t* b_stage, const uint16_t* const* src, int k0) {
    using R = Ring<KW>;
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < R::kLoads; ++j) {
        const bool is_a = j < R::kLoadsA;
        const int seg = wave + 8 * (is_a ? j : j - R::kLoadsA);
        uint16_t* dst = is_a ? a_stage + seg * 512 : b_stage + seg * 512;  // 1 KB
        if (NTB && !is_a) __builtin_amdgcn_global_load_lds(src[j] + k0, (lds_ptr_t)dst, 16, 0, 2);  // nt
        else __builtin_amdgcn_global_load_lds(src[j] + k0, (lds_ptr_t)dst, 16, 0, 0);
    }
}

template <int KW, bool NTB = false>
__device__ __forceinline__ void issue_slice(GSmem<KW>& sm, const LoadPlan<KW>& p, int stage, int k0) {
    const uint16_t* srcs[Ring<KW>::kLoads];
#pragma unroll
    for (int j = 0; j < Ring<KW>::kLoads; ++j)
        srcs[j] = p.src[j] + (size_t)k0 * (j < Ring<KW>::kLoadsA ? p.mul_a : p.mul_b);
    issue_stage<KW, NTB>(sm.k.a[stage], sm.k.b[stage], srcs, 0);
}

// The A segments of a slice only (B comes through registers): n 1 KB segments of this
// wave, segment j at dst + (wave + 8 j) * 512 elements, fetched from src[j] + k0.
__device__ __forceinline__ void issue_a_segments(uint16_t* dst, const uint16_t* const* src, int n, int k0, int mul) {
    const int wave = threadIdx.x / kWave;
    for (int j = 0; j < n; ++j)
        __builtin_amdgcn_global_load_lds(src[j] + (size_t)k0 * mul, (lds_ptr_t)(dst + (wave + 8 * j) * 512), 16, 0, 0);
}

// Fragments of 32 K of one wave's 64 x 64 tile, read from LDS apart from their MFMAs.
struct Frags {
    bf16x8 a[4], b[4];
};

// MI: the wave's 16-row fragments that hold tile rows (the others are padding past the
// group's last row, skipped).
template <int KW, int MI = 4>
__device__ __forceinline__ void read_frags(const uint16_t* sa, const uint16_t* sb, int arow0, const int (&brow)[4],
                                           int kc, Frags& f) {
    const int lane = lane_id();
    const int fr = lane & 15, fc = lane >> 4;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) f.a[mi] = lds_frag<KW>(sa, arow0 + mi * 16 + fr, kc + fc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) f.b[ni] = lds_frag<KW>(sb, brow[ni] + fr, kc + fc);
}

template <int MI = 4>
__device__ __forceinline__ void mfma_frags(const Frags& f, floatx4 (&acc)[4][4]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
}

// acc += A[wave rows] x B[rows brow[ni] + 0..15]^T over K.  Step kt: wait for this lane's
// loads of slice kt, barrier (everyone's slice kt has landed and everyone has finished
// step kt-1, whose stage the next issue reuses), compute slice kt, then issue slice kt+2
// (clamped near the end, so the body stays uniform).  Issuing the loads behind the
// step's LDS reads and MFMAs instead of in front of them measured ~20% faster per step in
// a probe of this loop (L2-resident operands): the fragment reads start right after the
// barrier instead of queueing behind the direct loads' LDS writes.  Ends with all loads
// drained and a barrier, so the caller may reuse the LDS.
template <int KW, bool NTB = false>
__device__ __forceinline__ void grouped_mainloop_plain(GSmem<KW>& sm, const LoadPlan<KW>& p, int K, int arow0,
                                                       const int (&brow)[4], floatx4 (&acc)[4][4]) {
    const int nk = K / KW;
    issue_slice<KW, NTB>(sm, p, 0, 0);
    issue_slice<KW, NTB>(sm, p, 1, min(1, nk - 1) * KW);
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
        wait_vm_lgkm<Ring<KW>::kLoads>();
        lds_barrier();
#pragma unroll
        for (int kc = 0; kc < KW / 8; kc += 4) mfma_k32<KW>(sm.k.a[st], sm.k.b[st], arow0, brow, kc, acc);
        const int pre = st == 0 ? 2 : st - 1;  // (kt + 2) % 3
        issue_slice<KW, NTB>(sm, p, pre, min(kt + 2, nk - 1) * KW);
        st = st == 2 ? 0 : st + 1;
    }
    wait_vm_lgkm<0>();
    __syncthreads();
}

// 32-wide slices in M halves: A rows 0-31 of the wave tile (lo) with all four B fragments,
// then A rows 32-63 (hi) with the same B.  b0 / b1 hold the B fragments of alternate slices.
struct HalfFrags {
    bf16x8 lo[2], hi[2], b0[4], b1[4];
};

// MI (0, 2 or 4): the wave's live 16-row fragments, as in read_frags; 2 keeps the lo half.
template <int KW, int MI = 4>
__device__ __forceinline__ void read_half_lo(GSmem<KW>& sm, int stg, int arow0, const int (&brow)[4], HalfFrags& h,
                                             bf16x8 (&b)[4]) {
    if constexpr (MI == 0) return;
    const int lane = lane_id();
    const int fr = lane & 15, fc = lane >> 4;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) h.lo[mi] = lds_frag<KW>(sm.k.a[stg], arow0 + mi * 16 + fr, fc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) b[ni] = lds_frag<KW>(sm.k.b[stg], brow[ni] + fr, fc);
}

__device__ __forceinline__ void mfma_half(const bf16x8 (&a)[2], const bf16x8 (&b)[4], floatx4 (&acc)[4][4], int m0) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            acc[m0 + mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[m0 + mi][ni], 0, 0, 0);
}

// Step kt of a 32-wide loop: B fragments of slice kt in bc, those of slice kt+1 go to bn.
template <int KW, int MI = 4, bool NTB = false>
__device__ __forceinline__ void half_step(GSmem<KW>& sm, const LoadPlan<KW>& p, int kt, int nk, int& st, int arow0,
                                          const int (&brow)[4], HalfFrags& h, bf16x8 (&bc)[4], bf16x8 (&bn)[4],
                                          floatx4 (&acc)[4][4]) {
    const int lane = lane_id();
    const int fr = lane & 15, fc = lane >> 4;
    if constexpr (MI == 4) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) h.hi[mi] = lds_frag<KW>(sm.k.a[st], arow0 + (mi + 2) * 16 + fr, fc);
    }
    if constexpr (MI >= 2) mfma_half(h.lo, bc, acc, 0);
    wait_vm_lgkm<Ring<KW>::kLoads>();  // slice kt+1 has landed, this wave's reads of slice kt are done
    lds_barrier();
    const int nx = st == 2 ? 0 : st + 1;
    read_half_lo<KW, MI>(sm, nx, arow0, brow, h, bn);
    if constexpr (MI == 4) mfma_half(h.hi, bc, acc, 2);
    issue_slice<KW, NTB>(sm, p, st, min(kt + 3, nk - 1) * KW);
    st = nx;
}

// The same product with each step straddling the barrier, in two halves: the fragments of
// a step's second half are read while its first half's MFMAs run, and after the barrier the
// next slice's first-half fragments while the second half's MFMAs run, so no wave meets the
// barrier with its LDS reads still to issue and none waits at the top of a step for reads
// it has just issued.  64-wide slices split into their two 32-wide K halves; 32-wide slices
// into M halves (A rows 0-31 with all B fragments, then A rows 32-63 with the same B, so the
// next slice's B fragments take a second set of registers).  The stage of slice kt is
// overwritten (by slice kt + 3) only after the barrier that follows every wave's last read
// of it; the slices stay two ahead.  Each accumulator still takes the slices, and the halves
// of a slice, in K order, so the sums are those of grouped_mainloop_plain.
template <int KW, int MI = 4, bool NTB = false>
__device__ __forceinline__ void grouped_mainloop(GSmem<KW>& sm, const LoadPlan<KW>& p, int K, int arow0,
                                                 const int (&brow)[4], floatx4 (&acc)[4][4]) {
    static_assert(KW == 32 || KW == 64, "slice width");
    constexpr int NL = Ring<KW>::kLoads;
    const int nk = K / KW;
    issue_slice<KW, NTB>(sm, p, 0, 0);
    issue_slice<KW, NTB>(sm, p, 1, min(1, nk - 1) * KW);
    wait_vm_lgkm<NL>();
    lds_barrier();
    int st = 0;
    if constexpr (KW == 64) {
        Frags f0, f1;
        read_frags<KW, MI>(sm.k.a[0], sm.k.b[0], arow0, brow, 0, f0);
        issue_slice<KW, NTB>(sm, p, 2, min(2, nk - 1) * KW);
        for (int kt = 0; kt < nk; ++kt) {
            read_frags<KW, MI>(sm.k.a[st], sm.k.b[st], arow0, brow, 4, f1);
            mfma_frags<MI>(f0, acc);
            wait_vm_lgkm<NL>();  // slice kt+1 has landed, this wave's reads of slice kt are done
            lds_barrier();
            const int nx = st == 2 ? 0 : st + 1;  // (kt + 1) % 3; past the last slice, a clamped re-load
            read_frags<KW, MI>(sm.k.a[nx], sm.k.b[nx], arow0, brow, 0, f0);
            mfma_frags<MI>(f1, acc);
            issue_slice<KW, NTB>(sm, p, st, min(kt + 3, nk - 1) * KW);
            st = nx;
        }
    } else {
        static_assert(MI == 0 || MI == 2 || MI == 4, "32-wide slices skip whole 32-row halves");
        HalfFrags h;
        read_half_lo<KW, MI>(sm, 0, arow0, brow, h, h.b0);
        issue_slice<KW, NTB>(sm, p, 2, min(2, nk - 1) * KW);
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            half_step<KW, MI, NTB>(sm, p, kt, nk, st, arow0, brow, h, h.b0, h.b1, acc);
            half_step<KW, MI, NTB>(sm, p, kt + 1, nk, st, arow0, brow, h, h.b1, h.b0, acc);
        }
        if (kt < nk) half_step<KW, MI, NTB>(sm, p, kt, nk, st, arow0, brow, h, h.b0, h.b1, acc);
    }
    wait_vm_lgkm<0>();
    __syncthreads();
}

// MXFP4 weights ("Phase 19: MoE - gpt-oss-20b", section 3): B rows are 16-byte blocks of
// 32 FP4 codes with one E8M0 scale byte each.  They cannot be direct-loaded into the bf16
// ring, so each thread loads its share of a K-slice into registers -- row threadIdx.x / 2
// of the N-tile, half threadIdx.x & 1 of the slice's KW codes (KW / 4 bytes) and the
// block's scale -- and one step later expands it with gfx950's scaled FP4 conversion into
// the slice's bf16 LDS rows (same swizzled layout as the direct loads).  The weights then
// cost 0.53 bytes each from memory instead of 2.  The thread's piece of slice s sits at
// codes + s * cstride and its scale at scales + s * sstride: in the checkpoint layout
// (rows of blocks) each thread of a wave reads another row, one cache line per row for a
// few bytes of it; in the grouped copy (mx_pack_layout) the pieces of one slice of one
// tile are contiguous, in thread order, so a wave reads whole lines.
struct MxRow {
    const uint8_t* codes;   // this thread's piece of slice 0
    const uint8_t* scales;  // the scale byte of that piece
    int cstride, sstride;   // bytes between the pieces of consecutive slices
};

// Vector loads into registers that the compiler does not track.  Its wait-count model
// does not count the direct-to-LDS loads in flight, so a wait it places before the first
// use of a register load drains those as well (vmcnt(0)), and the A slice meant to be two
// steps ahead has to land within the step.  The register-staged loop issues B through
// these and places its own waits (reg_wait), which name the number of younger loads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void vload16(u32x4& dst, const void* p) {
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(dst) : "v"(p) : "memory");
}
__device__ __forceinline__ void vload8(u32x2& dst, const void* p) {
    asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(dst) : "v"(p) : "memory");
}
__device__ __forceinline__ void vload_u8(uint32_t& dst, const void* p) {
    asm volatile("global_load_ubyte %0, %1, off" : "=v"(dst) : "v"(p) : "memory");
}
// Wait until at most N of this wave's vector-memory operations are outstanding; the
// registers named are tied to the wait, so no use of them moves above it.  The assembly
// names them in a comment ("tied ..."), which tests/test_asm_waits.py reads.
template <int N>
__device__ __forceinline__ void reg_wait(u32x4& a, uint32_t& b) {
    asm volatile("s_waitcnt vmcnt(%2) ; tied %0 %1" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void reg_wait(u32x2& a, uint32_t& b) {
    asm volatile("s_waitcnt vmcnt(%2) ; tied %0 %1" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void reg_wait(u32x4& a, u32x4& b) {
    asm volatile("s_waitcnt vmcnt(%2) ; tied %0 %1" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void reg_wait(u32x4& a, u32x4& b, u32x4& c) {
    asm volatile("s_waitcnt vmcnt(%3) ; tied %0 %1 %2" : "+v"(a), "+v"(b), "+v"(c) : "n"(N) : "memory");
}
// A 16-byte LDS store the compiler does not see as one: it orders every LDS store it sees
// after all direct-to-LDS loads in flight (vmcnt(0)), not knowing that the expanded B rows
// and the loads' A stages never overlap.  The loop's wait before each barrier
// (lgkmcnt(0)) completes these stores.
__device__ __forceinline__ void lds_write16(uint16_t* dst, const uint4& v) {
    const u32x4 d = {v.x, v.y, v.z, v.w};
    asm volatile("ds_write_b128 %0, %1" ::"v"((__attribute__((address_space(3))) void*)dst), "v"(d) : "memory");
}

template <int KW>
struct MxRegs {
    typename std::conditional<KW == 64, u32x4, u32x2>::type w;  // KW / 2 codes
    uint32_t s;                                                 // scale byte
};
constexpr int kMxLoads = 2;  // vector loads per thread per slice (codes, scale)

template <int KW>
__device__ __forceinline__ void mx_load(const MxRow& m, int k0, MxRegs<KW>& r) {
    static_assert(KW == 64 || KW == 32, "MXFP4 slices are one or two blocks wide");
    const int sl = k0 / KW;
    if constexpr (KW == 64) vload16(r.w, m.codes + (size_t)sl * m.cstride);  // one whole block
    else vload8(r.w, m.codes + (size_t)sl * m.cstride);                      // half a block
    vload_u8(r.s, m.scales + (size_t)sl * m.sstride);
}

template <int KW>
__device__ __forceinline__ void mx_store(GSmem<KW>& sm, int stage, const MxRegs<KW>& r) {
    const int row = threadIdx.x >> 1, h = threadIdx.x & 1;
    const float scale = e8m0_scale(r.s & 0xFFu);
#pragma unroll
    for (int i = 0; i < KW / 16; ++i)
        lds_write16(&sm.k.b[stage][swz<KW>(row, h * (KW / 16) + i)], fp4_word_bf16x8(r.w[i], scale));
}

// Weight sources of the register-staged main loop: load(k0, r) issues this thread's loads
// of the K-slice at k0 (thread t: tile row t / 2, half t & 1 of the slice) into r;
// ready<N>(r) waits for them with N younger vector-memory operations allowed in flight;
// store() expands r into the slice's bf16 LDS rows (the swizzled layout of the direct
// loads).  kLoads: vector loads per thread per slice.
template <int KW>
struct MxSrc {
    MxRow m;
    using Regs = MxRegs<KW>;
    static constexpr int kLoads = kMxLoads;
    __device__ __forceinline__ void load(int k0, Regs& r) const { mx_load<KW>(m, k0, r); }
    template <int N>
    __device__ __forceinline__ void ready(Regs& r) const { reg_wait<N>(r.w, r.s); }
    __device__ __forceinline__ void store(GSmem<KW>& sm, int stage, const Regs& r) const { mx_store<KW>(sm, stage, r); }
};

// Q4_K weights (layout in q4k_dev.h).  A 64-wide slice is one quant run c (two
// sub-blocks): half h of a row takes sub-block 2c + h, i.e. nibble h of all 32 run bytes.
// A 32-wide slice is one sub-block j: half h takes its weights 16h .. 16h+15, i.e. bytes
// 16h .. of run j / 2, nibble j & 1.  Either way the super-block's 16-byte header comes
// along.  `kbase` is the absolute input index of the call's K = 0 (split-K slices start
// inside a super-block).  Checkpoint layout: each thread's row is a run of 144-byte
// super-blocks, so the threads of a wave read 32 rows, a line or two per row for 48 bytes
// of it.  Grouped copy (q4k_pack_layout): per tile and super-block, the 256 tile rows'
// headers (16 bytes each) and then the four runs, each as 256 rows of 32 bytes, so a wave
// reads whole lines.
template <int KW>
struct Q4kRegs {
    u32x4 head;
    u32x4 q[KW == 64 ? 2 : 1];
    int j;  // sub-block whose scale and min apply
};

// Addresses: the header of super-block sb at head0 + sb * hs, quant run c of it at that
// header + qoff + c * cs.  Checkpoint: head0 = the thread's row, hs = 144, qoff = 16,
// cs = 32.  Grouped copy: head0 = the tile's first group + row * 16, hs = 256 * 144,
// qoff = 256 * 16 + row * 16 (the run rows follow the 256 headers), cs = 256 * 32.  A
// 32-wide slice adds 16h to qoff (its half of the run).
template <int KW>
struct Q4kSrc {
    const uint8_t* head0;
    int qoff, hs, cs;
    int kbase;
    using Regs = Q4kRegs<KW>;
    static constexpr int kLoads = KW == 64 ? 3 : 2;
    static_assert(KW == 64 || KW == 32, "Q4_K slices are one run or one sub-block wide");
    __device__ __forceinline__ static Q4kSrc make(const uint8_t* tile_or_row, bool packed, int kbase) {
        const int row = threadIdx.x >> 1, half = KW == 32 ? 16 * (threadIdx.x & 1) : 0;
        if (packed)
            return Q4kSrc{tile_or_row + row * 16, (kGThreads / 2) * 16 + row * 16 + half, (kGThreads / 2) * kQ4kBlockBytes,
                          (kGThreads / 2) * 32, kbase};
        return Q4kSrc{tile_or_row, 16 + half, kQ4kBlockBytes, 32, kbase};
    }
    __device__ __forceinline__ void load(int k0, Regs& r) const {
        const int k = kbase + k0, h = threadIdx.x & 1;
        const int j = (k % kQ4kBlockWeights) / 32;
        const uint8_t* head = head0 + (size_t)(k / kQ4kBlockWeights) * hs;
        const uint8_t* run = head + qoff + (j / 2) * cs;
        vload16(r.head, head);
        if constexpr (KW == 64) {
            vload16(r.q[0], run);
            vload16(r.q[1], run + 16);
            r.j = j + h;
        } else {
            vload16(r.q[0], run);
            r.j = j;
        }
    }
    template <int N>
    __device__ __forceinline__ void ready(Regs& r) const {
        if constexpr (KW == 64) reg_wait<N>(r.head, r.q[0], r.q[1]);
        else reg_wait<N>(r.head, r.q[0]);
    }
    __device__ __forceinline__ void store(GSmem<KW>& sm, int stage, const Regs& r) const {
        const int row_l = threadIdx.x >> 1, h = threadIdx.x & 1;
        float a, b;
        const uint4 head = make_uint4(r.head[0], r.head[1], r.head[2], r.head[3]);
        q4k_sub_scale(head, r.j, a, b);
        const int shift = 4 * (r.j & 1);
        constexpr int NC = KW / 16;  // 16-byte LDS chunks per thread
#pragma unroll
        for (int q = 0; q < NC; ++q) {
            const u32x4& v = r.q[q / 2];
            const uint32_t w0 = (q & 1) ? v[2] : v[0], w1 = (q & 1) ? v[3] : v[1];
            lds_write16(&sm.k.b[stage][swz<KW>(row_l, h * NC + q)], q4k_dequant8(w0, w1, shift, a, b));
        }
    }
};

// The main loop with B from a register-staged source.  Slice s: A direct-loaded two steps
// ahead as in grouped_mainloop; B loaded into registers two steps ahead and expanded into
// LDS at the end of step s - 1 (its stage held slice s - 3, finished by every wave at the
// barrier of step s - 1).  Each step issues its B loads, then its A segments, so the
// expansion of slice s waits with slice s's A segments still in flight (kLoadsA younger
// operations); the prologue's first expansion has A of slices 0 and 1 and B of slice 1
// behind it.  The wait before each step allows the newest slice's loads (B registers and
// A) in flight.  The B registers of the clamped re-load on the last step stay tied until
// every load has drained.  (With the compiler's own waits, which drained every load at the
// first use of the B registers: gpt-oss-shaped MXFP4 T=4096 1252 -> 1170 us per forward,
// Q4_K prefill T=8192 1056 -> 1038 us.)
// MI: the wave's live 16-row fragments (as in read_frags; the rest are padding).
template <int KW, int MI = 4, typename Src>
__device__ __forceinline__ void grouped_mainloop_regb(GSmem<KW>& sm, const LoadPlan<KW>& p, const Src& src, int K,
                                                      int arow0, const int (&brow)[4], floatx4 (&acc)[4][4]) {
    constexpr int LA = Ring<KW>::kLoadsA;
    const int nk = K / KW;
    typename Src::Regs first, nxt;
    src.load(0, first);
    issue_a_segments(sm.k.a[0], p.src, LA, 0, p.mul_a);
    src.load(min(1, nk - 1) * KW, nxt);
    issue_a_segments(sm.k.a[1], p.src, LA, min(1, nk - 1) * KW, p.mul_a);
    src.template ready<2 * LA + Src::kLoads>(first);
    src.store(sm, 0, first);
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
        wait_vm_lgkm<LA + Src::kLoads>();
        lds_barrier();
        if constexpr (MI > 0) {
#pragma unroll
            for (int kc = 0; kc < KW / 8; kc += 4) {
                Frags f;
                read_frags<KW, MI>(sm.k.a[st], sm.k.b[st], arow0, brow, kc, f);
                mfma_frags<MI>(f, acc);
            }
        }
        const int nx = st == 2 ? 0 : st + 1;   // (kt + 1) % 3
        src.template ready<LA>(nxt);
        src.store(sm, nx, nxt);                // B of slice kt+1 (clamped re-load on the last step)
        src.load(min(kt + 2, nk - 1) * KW, nxt);
        const int pre = st == 0 ? 2 : st - 1;  // (kt + 2) % 3
        issue_a_segments(sm.k.a[pre], p.src, LA, min(kt + 2, nk - 1) * KW, p.mul_a);
        st = nx;
    }
    wait_vm_lgkm<0>();
    src.template ready<0>(nxt);
    __syncthreads();
}

// Storage of the routed experts' weights in the grouped kernels.
constexpr int kWDense = 0, kWMx = 1, kWQ4k = 2;

struct UpArgs {
    const uint16_t* x;
    const int32_t* perm_token;
    const Group* groups;
    const PlanMeta* meta;
    const TileDesc* tiles;
    const uint16_t* w_gate;     // [E, ff, d]
    const uint16_t* w_up;
    const uint16_t* w_gate_up;  // [E, 2ff, d]
    const uint16_t* b_gate_up;  // [E, 2ff]
    const uint16_t* ws_gate;    // [ffs, d]
    const uint16_t* ws_up;
    const uint8_t* mx_w;        // MXFP4 gate_up blocks [E, 2ff, d/32, 16], or null
    const uint8_t* mx_s;        // ... and scales [E, 2ff, d/32]
    const uint8_t* q4_gate;     // Q4_K gate / up super-blocks [E, ff, d/256, 144], or null
    const uint8_t* q4_up;
    uint16_t* H;                // bf16 hidden rows, slice-major: [hstride / 32][h_rows][32]
    int hstride, T, d, ff, ffs, n_ntiles;
    float alpha, limit;
    int mx_packed;              // mx_w / mx_s point into the grouped copy (mx_pack_layout)
    int q4_packed;              // q4_gate points at the grouped copy's up region (q4k_pack_layout)
    int h_rows;                 // rows of H (T * k, plus T with a shared expert)
};

struct DownArgs {
    const uint16_t* H;
    const Group* groups;
    const PlanMeta* meta;
    const TileDesc* tiles;
    const uint16_t* w_down;   // [E, d, ff]
    const uint16_t* b_down;   // [E, d] or null
    const uint16_t* ws_down;  // [d, ffs]
    const uint8_t* mx_w;      // MXFP4 down blocks [E, d, ff/32, 16], or null
    const uint8_t* mx_s;      // ... and scales [E, d, ff/32]
    const uint8_t* q4_down;   // Q4_K down super-blocks [E, d, ff/256, 144], or null
    const float* row_w;       // per grouped row weight, or null (unweighted)
    void* y;                  // [rows, d], bf16 or fp32; with ksplit > 1 fp32 [ksplit][rows][d]
    int hstride, d, ff, ffs, n_ntiles;
    int ksplit, rows;         // K slices per tile (each block sums K / ksplit), grouped rows
    int mx_packed;            // mx_w / mx_s, or q4_down, point into the grouped copy
    const uint16_t* wd_pack;  // dense bf16: routed W_d in the grouped copy (dense_pack_layout), or null
    const uint16_t* wsd_pack; // ... and the shared expert's W_d, or null
};

// XCD-aware tile order.  Workgroups are dispatched to the 8 XCDs round-robin by block
// id, and each XCD has its own L2.  Block b runs slot b / 8 of XCD b % 8; every XCD owns
// a contiguous range of M-tiles (groups are contiguous in tile order, so an expert spans
// at most a few XCDs) and walks it in groups of kGroupM M-tiles: all N-tiles of a group,
// N-tile by N-tile, each N-tile over the group's M-tiles.  The blocks in flight on one XCD
// (32 to 64) then share a few gathered A tiles and a few weight slices in its L2.  With
// a single M-tile per step of the walk, a layer with wide experts (tens of N-tiles) would
// stream a different weight slice into every block and re-read each expert's weights
// from HBM once per M-tile.  (A walk that instead runs every group of the XCD through a
// window of 4 N-tiles before the next window measured no faster anywhere and fetched
// twice the bytes on the 8-expert, 14336-wide layer.)
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

inline int grid_blocks(int max_mtiles, int n_ntiles) {
    return kXcds * ((max_mtiles + kXcds - 1) / kXcds) * n_ntiles;
}

// Resolve this block's (group, first row, N-tile).  Returns false if the block is idle.
// Slots of one XCD: group q = slot / (kGroupM * n_ntiles) holds that XCD's M-tiles
// q*kGroupM .. +gm-1 (gm = kGroupM but for the last group); inside it slot s takes N-tile
// s / gm of M-tile s % gm.  The grid has ceil(max_mtiles / 8) * n_ntiles slots per XCD,
// which covers every (M-tile, N-tile) pair of the XCD's range exactly once.
__device__ __forceinline__ bool locate(const PlanMeta* meta, const TileDesc* tiles, const Group* groups,
                                       int n_ntiles, Group& g, int& m0, int& nt) {
    const int n_tiles = meta->n_tiles;
    if (n_tiles <= 0) return false;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int per_xcd = (n_tiles + kXcds - 1) / kXcds;
    const int q = slot / (kGroupM * n_ntiles), s = slot % (kGroupM * n_ntiles);
    const int gm = min(kGroupM, per_xcd - q * kGroupM);
    if (gm <= 0) return false;
    nt = s / gm;
    const int mt = xcd * per_xcd + q * kGroupM + s % gm;
    if (nt >= n_ntiles || mt >= n_tiles) return false;
    g = groups[tiles[mt].group];
    m0 = (mt - g.tile0) * BM;
    return true;
}

// 16-row fragments of wave row wm's 64 tile rows that hold group rows (0 .. 4); the rest of
// a partial tile is padding, whose MFMAs and fragment reads are skipped (its loads are not:
// every wave issues its share of each slice).
__device__ __forceinline__ int up_live(const Group& g, int m0, int wm) {
    return __builtin_amdgcn_readfirstlane(min(max((g.n - m0 - wm * 64 + 15) / 16, 0), 4));
}

// The register-staged loop with the padded fragments skipped.
template <int KW, typename Src>
__device__ __forceinline__ void regb_live(GSmem<KW>& sm, const LoadPlan<KW>& p, const Src& src, int K, int live,
                                          int arow0, const int (&brow)[4], floatx4 (&acc)[4][4]) {
    switch (live) {
        case 4: grouped_mainloop_regb<KW, 4>(sm, p, src, K, arow0, brow, acc); break;
        case 3: grouped_mainloop_regb<KW, 3>(sm, p, src, K, arow0, brow, acc); break;
        case 2: grouped_mainloop_regb<KW, 2>(sm, p, src, K, arow0, brow, acc); break;
        case 1: grouped_mainloop_regb<KW, 1>(sm, p, src, K, arow0, brow, acc); break;
        default: grouped_mainloop_regb<KW, 0>(sm, p, src, K, arow0, brow, acc); break;
    }
}

// Down kernel, register-staged B: padded fragments skipped by whole 32-row halves for bf16
// rows; fp32 rows keep the one full loop (more instances would cost that kernel its second
// block per CU).
template <typename TY, typename Src>
__device__ __forceinline__ void down_regb(GSmem<kDownKW>& sm, const LoadPlan<kDownKW>& p, const Src& src, int K,
                                          int live, int arow0, const int (&brow)[4], floatx4 (&acc)[4][4]) {
    if constexpr (sizeof(TY) == 2) {
        if (live > 2) grouped_mainloop_regb<kDownKW, 4>(sm, p, src, K, arow0, brow, acc);
        else if (live > 0) grouped_mainloop_regb<kDownKW, 2>(sm, p, src, K, arow0, brow, acc);
        else grouped_mainloop_regb<kDownKW, 0>(sm, p, src, K, arow0, brow, acc);
    } else {
        grouped_mainloop_regb<kDownKW, 4>(sm, p, src, K, arow0, brow, acc);
    }
}

// WF: storage of the routed gate/up weights.  kWMx: MXFP4 gate_up blocks (a.mx_w, a.mx_s;
// clamped variant, no shared expert).  kWQ4k: Q4_K w_gate / w_up super-blocks (SwiGLU);
// the shared expert's tiles stay on the bf16 direct loads.
template <bool OAI, int WF, bool NTB>
__global__ __launch_bounds__(kGThreads, blocks_per_cu<kUpKW>()) void gg_up_kernel(UpArgs a) {
    __shared__ GSmem<kUpKW> sm;
    Group g;
    int m0, nt;
    if (!locate(a.meta, a.tiles, a.groups, a.n_ntiles, g, m0, nt)) return;
    const bool shared = g.e < 0;
    const int ffg = shared ? a.ffs : a.ff;
    const int f0 = nt * 128;
    if (f0 >= ffg) return;
    const bool oai = OAI && !shared;
    const size_t d = a.d;

    // Tile rows of A: gathered token rows (ragged tail re-reads the last row).  Tile rows
    // of B: 0..127 gate units f0.., 128..255 up units f0.. (units past ffg re-read the last).
    auto row_a = [&](int r) {
        const int m = min(m0 + r, g.n - 1);
        int tok = shared ? m : a.perm_token[g.row0 + m];
        tok = min(max(tok, 0), a.T - 1);
        return a.x + (size_t)tok * d;
    };
    auto row_b = [&](int r) {
        const bool up = r >= 128;
        const int f = min(f0 + (r & 127), ffg - 1);
        if (oai) return a.w_gate_up + ((size_t)g.e * 2 * a.ff + 2 * f + (up ? 1 : 0)) * d;
        const uint16_t* base = shared ? (up ? a.ws_up : a.ws_gate)
                                      : (up ? a.w_up : a.w_gate) + (size_t)g.e * a.ff * d;
        return base + (size_t)f * d;
    };
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int wm = wave >> 2, wn = wave & 3;
    // Wave n-tiles 0,1 are gate units wn*32.., 2,3 the matching up units.
    const int brow[4] = {wn * 32, wn * 32 + 16, 128 + wn * 32, 128 + wn * 32 + 16};
    floatx4 acc[4][4];
    zero(acc);
    if constexpr (WF == kWMx) {
        // This thread's B row (tile row threadIdx.x / 2), in the interleaved gate_up rows.
        const LoadPlan<kUpKW> plan = make_plan<kUpKW, true>(row_a, row_b);
        const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
        MxRow m;
        if (a.mx_packed) {
            const size_t tile = (size_t)max(g.e, 0) * ((a.ff + 127) / 128) + nt, slices = d / kUpKW;
            m = MxRow{a.mx_w + (tile * slices * kGThreads + threadIdx.x) * 16, a.mx_s + tile * slices * kGThreads + threadIdx.x,
                      kGThreads * 16, kGThreads};
        } else {
            const int f = min(f0 + (r & 127), ffg - 1);
            const size_t R = (size_t)max(g.e, 0) * 2 * a.ff + 2 * f + (r >= 128 ? 1 : 0);
            const size_t nblk = d / 32;
            m = MxRow{a.mx_w + (R * nblk + h) * 16, a.mx_s + R * nblk + h, 32, 2};
        }
        const MxSrc<kUpKW> src{m};
        regb_live<kUpKW>(sm, plan, src, a.d, up_live(g, m0, wm), wm * 64, brow, acc);
    } else if constexpr (WF == kWQ4k) {
        if (!shared) {
            const LoadPlan<kUpKW> plan = make_plan<kUpKW, true>(row_a, row_b);
            const int r = threadIdx.x >> 1;
            const size_t nsb = d / kQ4kBlockWeights;
            const uint8_t* base;
            if (a.q4_packed) {
                base = a.q4_gate + ((size_t)g.e * ((a.ff + 127) / 128) + nt) * nsb * (kGThreads / 2) * kQ4kBlockBytes;
            } else {
                const int f = min(f0 + (r & 127), ffg - 1);
                base = (r >= 128 ? a.q4_up : a.q4_gate) + ((size_t)g.e * a.ff + f) * nsb * kQ4kBlockBytes;
            }
            const Q4kSrc<kUpKW> src = Q4kSrc<kUpKW>::make(base, a.q4_packed != 0, 0);
            regb_live<kUpKW>(sm, plan, src, a.d, up_live(g, m0, wm), wm * 64, brow, acc);
        } else {
            const LoadPlan<kUpKW> plan = make_plan<kUpKW, false>(row_a, row_b);
            grouped_mainloop<kUpKW, 4, NTB>(sm, plan, a.d, wm * 64, brow, acc);
        }
    } else {
        const LoadPlan<kUpKW> plan = make_plan<kUpKW, false>(row_a, row_b);
        switch (up_live(g, m0, wm)) {
            case 4: grouped_mainloop<kUpKW, 4, NTB>(sm, plan, a.d, wm * 64, brow, acc); break;
            case 3: grouped_mainloop<kUpKW, 3, NTB>(sm, plan, a.d, wm * 64, brow, acc); break;
            case 2: grouped_mainloop<kUpKW, 2, NTB>(sm, plan, a.d, wm * 64, brow, acc); break;
            case 1: grouped_mainloop<kUpKW, 1, NTB>(sm, plan, a.d, wm * 64, brow, acc); break;
            default: grouped_mainloop<kUpKW, 0, NTB>(sm, plan, a.d, wm * 64, brow, acc); break;
        }
    }

    // Epilogue: lane holds D[4*(lane/16) + i][lane%16] of each 16x16 tile.  Activation,
    // bf16, staged in LDS as the 128 x 128 H tile.
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int fl = wn * 32 + ni * 16 + (lane & 15);
        float bg = 0.f, bu = 0.f;
        if (oai) {
            const int f = min(f0 + fl, ffg - 1);
            bg = ld_bf16(a.b_gate_up + (size_t)g.e * 2 * a.ff + 2 * f);
            bu = ld_bf16(a.b_gate_up + (size_t)g.e * 2 * a.ff + 2 * f + 1);
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ml = wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
                float gv = acc[mi][ni][i], uv = acc[mi][ni + 2][i], h;
                if (oai) {
                    gv = fminf(gv + bg, a.limit);
                    uv = fminf(fmaxf(uv + bu, -a.limit), a.limit);
                    h = (uv + 1.0f) * gv * sigmoidf_(a.alpha * gv);
                } else {
                    h = gv * sigmoidf_(gv) * uv;
                }
                sm.up[ml * kUpStage + fl] = f32_to_bf16(h);
            }
        }
    }
    __syncthreads();
    // 128 rows x 16 chunks; 512 threads = 32 rows per pass.  H is slice-major (32 columns
    // per slice, the down kernel's K-slice): chunk c goes to slice (f0 + 8c) / 32, so a
    // wave's 4 rows x 64 bytes per slice are contiguous.
    const int c = threadIdx.x & 15;
    const int f = f0 + c * 8;
    uint16_t* hs = a.H + ((size_t)(f / 32) * a.h_rows + g.row0 + m0) * 32 + f % 32;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int ml = (threadIdx.x >> 4) + 32 * p;
        if (m0 + ml < g.n && f < ffg)
            *reinterpret_cast<uint4*>(hs + (size_t)ml * 32) = *reinterpret_cast<const uint4*>(sm.up + ml * kUpStage + c * 8);
    }
}

// With ksplit > 1 (few tiles: decode-sized batches of layers with few experts) the K axis
// of every tile is cut into ksplit slices, one block each (N-tile-major: the slices of an
// N-tile are consecutive block slots), and each block stores its raw fp32 sums to slice
// plane ks of y; splitk_reduce_kernel adds the planes, the bias and the routing weight.
// WF: storage of the routed down weights (kWMx: MXFP4 blocks a.mx_w, a.mx_s; kWQ4k: Q4_K
// super-blocks a.q4_down, the shared expert's tiles on the bf16 direct loads).
template <typename TY, int WF, bool NTB>
__global__ __launch_bounds__(kGThreads, blocks_per_cu<kDownKW>()) void gg_down_kernel(DownArgs a) {
    __shared__ GSmem<kDownKW> sm;
    Group g;
    int m0, nt;
    if (!locate(a.meta, a.tiles, a.groups, a.n_ntiles * a.ksplit, g, m0, nt)) return;
    const int ks = nt % a.ksplit;
    nt /= a.ksplit;
    const bool shared = g.e < 0;
    const int Kfull = shared ? a.ffs : a.ff;
    const int K = Kfull / a.ksplit;  // the host picks ksplit so that slices are whole K-steps
    const int kb = ks * K;
    const int n0 = nt * GBN;
    // H is slice-major: slice s of row m at H + (s * rows + m) * 32; this split starts at slice kb / 32.
    auto row_a = [&](int r) { return a.H + ((size_t)(kb / kDownKW) * a.rows + g.row0 + min(m0 + r, g.n - 1)) * kDownKW; };
    // Dense weights in the grouped copy: slice s of N-tile nt is 256 rows x 32 contiguous, so
    // row r of this split's first slice sits at ((tile * slices + kb / 32) * 256 + r) * 32.
    const uint16_t* wpack = shared ? a.wsd_pack : a.wd_pack;
    auto row_b = [&](int r) {
        if (wpack) {
            const size_t tile = shared ? (size_t)nt : (size_t)g.e * a.n_ntiles + nt;
            return wpack + ((tile * (Kfull / kDownKW) + kb / kDownKW) * GBN + r) * kDownKW;
        }
        const int n = min(n0 + r, a.d - 1);  // partial last N-tile: re-read
        return (shared ? a.ws_down + (size_t)n * Kfull : a.w_down + ((size_t)g.e * a.d + n) * Kfull) + kb;
    };
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int wm = wave >> 2, wn = wave & 3;
    const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
    // The routing weight of tile row threadIdx.x, loaded now so that its latency hides behind
    // the main loop; it goes to LDS after the loop, where the epilogue reads it.
    float my_rw = 1.0f;
    if (a.row_w && threadIdx.x < BM) my_rw = a.row_w[g.row0 + min(m0 + (int)threadIdx.x, g.n - 1)];
    floatx4 acc[4][4];
    zero(acc);
    if constexpr (WF == kWMx) {
        // This thread's B row (tile row threadIdx.x / 2) of W_d, from this split's first block.
        LoadPlan<kDownKW> plan = make_plan<kDownKW, true>(row_a, row_b);
        plan.mul_a = a.rows;
        const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
        MxRow m;
        if (a.mx_packed) {
            const size_t tile = (size_t)max(g.e, 0) * a.n_ntiles + nt, slices = Kfull / kDownKW;
            const size_t first = tile * slices + kb / kDownKW;  // this split's first slice
            m = MxRow{a.mx_w + (first * GBN + r) * 16 + 8 * h, a.mx_s + first * GBN + r, GBN * 16, GBN};
        } else {
            const int n = min(n0 + r, a.d - 1);
            const size_t R = (size_t)max(g.e, 0) * a.d + n;
            const size_t nblk = Kfull / 32;
            m = MxRow{a.mx_w + (R * nblk + kb / 32) * 16 + 8 * h, a.mx_s + R * nblk + kb / 32, 16, 1};
        }
        const MxSrc<kDownKW> src{m};
        down_regb<TY>(sm, plan, src, K, up_live(g, m0, wm), wm * 64, brow, acc);
    } else if constexpr (WF == kWQ4k) {
        if (!shared) {
            LoadPlan<kDownKW> plan = make_plan<kDownKW, true>(row_a, row_b);
            plan.mul_a = a.rows;
            const size_t nsb = Kfull / kQ4kBlockWeights;
            const uint8_t* base;
            if (a.mx_packed) {
                base = a.q4_down + ((size_t)g.e * a.n_ntiles + nt) * nsb * GBN * kQ4kBlockBytes;
            } else {
                const int n = min(n0 + (int)(threadIdx.x >> 1), a.d - 1);
                base = a.q4_down + ((size_t)g.e * a.d + n) * nsb * kQ4kBlockBytes;
            }
            const Q4kSrc<kDownKW> src = Q4kSrc<kDownKW>::make(base, a.mx_packed != 0, kb);
            down_regb<TY>(sm, plan, src, K, up_live(g, m0, wm), wm * 64, brow, acc);
        } else {  // the plain loop: the second set of B registers would cost this kernel occupancy
            LoadPlan<kDownKW> plan = make_plan<kDownKW, false>(row_a, row_b);
            plan.mul_a = a.rows;
            grouped_mainloop_plain<kDownKW, NTB>(sm, plan, K, wm * 64, brow, acc);
        }
    } else {
        // As in the up kernel, padding rows past the group's last row run no MFMAs, here by
        // whole 32-row halves of the wave's 64 rows (bf16 rows only: the three instances
        // would take the fp32-row kernel past 128 VGPRs, i.e. to one block per CU).
        LoadPlan<kDownKW> plan = make_plan<kDownKW, false>(row_a, row_b);
        plan.mul_a = a.rows;
        plan.mul_b = wpack ? GBN : 1;
        if constexpr (sizeof(TY) == 2) {
            const int live = up_live(g, m0, wm);
            if (live > 2) grouped_mainloop<kDownKW, 4, NTB>(sm, plan, K, wm * 64, brow, acc);
            else if (live > 0) grouped_mainloop<kDownKW, 2, NTB>(sm, plan, K, wm * 64, brow, acc);
            else grouped_mainloop<kDownKW, 0, NTB>(sm, plan, K, wm * 64, brow, acc);
        } else {
            grouped_mainloop<kDownKW, 4, NTB>(sm, plan, K, wm * 64, brow, acc);
        }
    }

    if (threadIdx.x < BM) sm.row_w[threadIdx.x] = my_rw;
    __syncthreads();
    float rw[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) rw[mi][i] = sm.row_w[wm * 64 + mi * 16 + 4 * (lane >> 4) + i];
    constexpr bool kHalf = sizeof(TY) == 2;
    // bf16: the whole 128 x 256 tile is staged at once; fp32: two 128-column halves (the
    // waves with wn < 2, then the others), each followed by coalesced 16-byte stores.
    constexpr int kHalves = kHalf ? 1 : 2;
    constexpr int kCols = GBN / kHalves;
    constexpr int kStride = kHalf ? kDownStageH : kDownStageF;
    constexpr int kChunks = kCols * (int)sizeof(TY) / 16;
    constexpr int kPer = 16 / (int)sizeof(TY);
    constexpr int kRowsPerPass = kGThreads / kChunks;
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
        if (kHalves == 1 || (wn >> 1) == h) {
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int nl = wn * 64 + ni * 16 + (lane & 15);
                const int n = min(n0 + nl, a.d - 1);
                const float bias = (!shared && a.b_down) ? ld_bf16(a.b_down + (size_t)g.e * a.d + n) : 0.0f;
                const int sc = nl - h * kCols;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ml = wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
                        const float v = (acc[mi][ni][i] + bias) * rw[mi][i];
                        if constexpr (kHalf) sm.down_h[ml * kStride + sc] = f32_to_bf16(v);
                        else sm.down_f[ml * kStride + sc] = v;
                    }
            }
        }
        __syncthreads();
        const int c = threadIdx.x % kChunks;
#pragma unroll
        for (int p = 0; p < BM / kRowsPerPass; ++p) {
            const int ml = threadIdx.x / kChunks + kRowsPerPass * p;
            const int n = n0 + h * kCols + c * kPer;
            if (m0 + ml < g.n && n < a.d) {
                TY* dst = static_cast<TY*>(a.y) + ((size_t)ks * a.rows + g.row0 + m0 + ml) * a.d + n;
                u32x4_t v;
                if constexpr (kHalf) v = *reinterpret_cast<const u32x4_t*>(sm.down_h + ml * kStride + c * kPer);
                else v = *reinterpret_cast<const u32x4_t*>(sm.down_f + ml * kStride + c * kPer);
                // Streamed out: the rows are read again only by a later launch.
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
            }
        }
        if (h + 1 < kHalves) __syncthreads();
    }
}

// Sum of the ksplit fp32 planes of split-K down tiles, in plane order, plus the down bias,
// times the row's routing weight: the same value the unsplit epilogue stores, summed in
// another order.  Block (c, i, m) takes row m of M-tile i of the tile map and 1024 output
// columns from c * 1024, four per thread; every plane's load is issued before the sum.
constexpr int kMaxSplitPlanes = 4;

template <typename TY>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int ksplit, int rows,
                                                           const PlanMeta* __restrict__ meta,
                                                           const TileDesc* __restrict__ tiles,
                                                           const uint16_t* __restrict__ b_down,
                                                           const float* __restrict__ row_w, TY* __restrict__ y,
                                                           int d) {
    if ((int)blockIdx.y >= meta->n_tiles) return;
    const TileDesc td = tiles[blockIdx.y];
    const int m = blockIdx.z;
    const int n = blockIdx.x * 1024 + threadIdx.x * 4;
    if (m >= td.n || n >= d) return;
    const size_t row = (size_t)td.row0 + m;
    float4 v[kMaxSplitPlanes];
#pragma unroll
    for (int s = 0; s < kMaxSplitPlanes; ++s)
        v[s] = s < ksplit ? *reinterpret_cast<const float4*>(part + ((size_t)s * rows + row) * d + n)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    float bias[4] = {0.f, 0.f, 0.f, 0.f};
    if (td.e >= 0 && b_down) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bias[j] = ld_bf16(b_down + (size_t)td.e * d + n + j);
    }
    const float rw = row_w ? row_w[row] : 1.0f;
    float4 acc = v[0];
#pragma unroll
    for (int s = 1; s < kMaxSplitPlanes; ++s) {
        if (s < ksplit) {
            acc.x += v[s].x;
            acc.y += v[s].y;
            acc.z += v[s].z;
            acc.w += v[s].w;
        }
    }
    const float o[4] = {(acc.x + bias[0]) * rw, (acc.y + bias[1]) * rw, (acc.z + bias[2]) * rw,
                        (acc.w + bias[3]) * rw};
    if constexpr (sizeof(TY) == 2) {
        const uint2 pk = make_uint2(uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16),
                                    uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16));
        *reinterpret_cast<uint2*>(y + row * d + n) = pk;
    } else {
        *reinterpret_cast<float4*>(y + row * d + n) = make_float4(o[0], o[1], o[2], o[3]);
    }
}

// =====================================================================================
// Router GEMM: 4 waves, MT x 128 block tile (MT = 128, 64 or 32 token rows: the largest
// that still gives every CU a block), register-staged double-buffered LDS.
// =====================================================================================
constexpr int RBN = 128;
constexpr int RBK = 64;
constexpr int kRThreads = 256;

template <int MT>
struct RSmem {
    uint16_t a[2][MT * RBK];
    uint16_t b[2][RBN * RBK];
};

// This thread's N rows (tile rows tid/8 + 32 i) at chunk tid%8.
template <int N>
__device__ __forceinline__ void load_slice(const uint16_t* const (&rows)[N], int k0, uint4 (&r)[N]) {
    const int c = (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = ld16(rows[i] + k0 + c);
}

template <int N>
__device__ __forceinline__ void store_slice(uint16_t* lds, const uint4 (&r)[N]) {
    const int c = threadIdx.x & 7;
    const int r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < N; ++i) *reinterpret_cast<uint4*>(lds + swz<RBK>(r0 + 32 * i, c)) = r[i];
}

// One step on K-slice kt with buffer / register set B (compile-time, so register arrays
// are never indexed dynamically).  Straight-line on purpose: the prefetch (slice kt+2,
// clamped) and the store (slice kt+1; a dead store into the idle buffer on the last step)
// are unconditional, and a scheduling fence keeps the prefetch above the store, so the
// wait before the store leaves this step's prefetch in flight.  NA: A rows per thread
// (MT / 32); MI: A fragments per wave (MT / 32).
template <int B, int MT>
__device__ __forceinline__ void router_step(RSmem<MT>& sm, const uint16_t* const (&a_rows)[MT / 32],
                                            const uint16_t* const (&b_rows)[4], int kt, int nk, int arow0,
                                            const int (&brow)[4], uint4 (&ra)[2][MT / 32], uint4 (&rb)[2][4],
                                            floatx4 (&acc)[MT / 32][4]) {
    constexpr int MI = MT / 32;
    const int pre = min(kt + 2, nk - 1) * RBK;
    load_slice(a_rows, pre, ra[B]);
    load_slice(b_rows, pre, rb[B]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_k32<RBK, MI>(sm.a[B], sm.b[B], arow0, brow, 0, acc);
    mfma_k32<RBK, MI>(sm.a[B], sm.b[B], arow0, brow, 4, acc);
    store_slice(sm.a[B ^ 1], ra[B ^ 1]);
    store_slice(sm.b[B ^ 1], rb[B ^ 1]);
    __syncthreads();
}

// Router logits of a large batch on MFMA: logits[t, e] = x[t] . W_r[e] (+ b[e]) for
// e < E ("Qwen3.5-MoE Model Implementation", MoE routing; "Phase 19: MoE - gpt-oss-20b",
// Router).  Waves in a 2 x 2 grid of (MT / 2) x 64 tiles.
template <int MT>
__global__ __launch_bounds__(kRThreads, 2) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w_router,
                                                                   const float* __restrict__ b_router,
                                                                   int T, int d, int E, int n_ntiles,
                                                                   float* __restrict__ logits, int ld) {
    constexpr int NA = MT / 32, MI = MT / 32, WM = MT / 2;
    __shared__ RSmem<MT> sm;
    const int m0 = (blockIdx.x / n_ntiles) * MT;
    const int n0 = (blockIdx.x % n_ntiles) * RBN;
    const int r0 = threadIdx.x >> 3;
    const uint16_t* a_rows[NA];
    const uint16_t* b_rows[4];
#pragma unroll
    for (int i = 0; i < NA; ++i) a_rows[i] = x + (size_t)min(m0 + r0 + 32 * i, T - 1) * d;
#pragma unroll
    for (int i = 0; i < 4; ++i) b_rows[i] = w_router + (size_t)min(n0 + r0 + 32 * i, E - 1) * d;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
    floatx4 acc[MI][4];
    zero(acc);
    const uint16_t* const (&ar)[NA] = a_rows;
    const uint16_t* const (&br)[4] = b_rows;
    const int nk = d / RBK;
    uint4 ra[2][NA], rb[2][4];
    load_slice(ar, 0, ra[0]);
    load_slice(br, 0, rb[0]);
    load_slice(ar, min(1, nk - 1) * RBK, ra[1]);
    load_slice(br, min(1, nk - 1) * RBK, rb[1]);
    store_slice(sm.a[0], ra[0]);
    store_slice(sm.b[0], rb[0]);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        router_step<0, MT>(sm, ar, br, kt, nk, wm * WM, brow, ra, rb, acc);
        router_step<1, MT>(sm, ar, br, kt + 1, nk, wm * WM, brow, ra, rb, acc);
    }
    if (kt < nk) router_step<0, MT>(sm, ar, br, kt, nk, wm * WM, brow, ra, rb, acc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int n = n0 + wn * 64 + ni * 16 + (lane & 15);
        if (n >= E) continue;
        const float bias = b_router ? b_router[n] : 0.0f;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * WM + mi * 16 + 4 * (lane >> 4) + i;
                if (m < T) logits[(size_t)m * ld + n] = acc[mi][ni][i] + bias;
            }
    }
}

// The grouped copy of MXFP4 expert weights (moe_grouped_pack), one thread per 16-byte
// block.  Up: piece i = ((e * NTu + nt) * Su + s) * 512 + t holds the block that thread t
// of the up kernel's block for N-tile nt reads in slice s (tile row r = t / 2: gate unit
// nt * 128 + r for r < 128, else up unit nt * 128 + r - 128, clamped to the last unit;
// block 2s + t % 2 of that row), its scale byte at the same index.  Down: piece
// i = ((e * NTd + nt) * Sd + s) * 256 + r holds block s of output row nt * 256 + r
// (clamped to the last row).  Units and rows past the matrix repeat the last one, as the
// kernels' own clamps do.
__global__ __launch_bounds__(256) void mx_pack_up_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ sc,
                                                         int ff, int d, long long pieces, int ntu, int su,
                                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const size_t nblk = d / 32;
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < pieces; i += (long long)gridDim.x * 256) {
        const int t = (int)(i % kGThreads);
        long long rest = i / kGThreads;
        const int sl = (int)(rest % su);
        rest /= su;
        const int nt = (int)(rest % ntu);
        const long long e = rest / ntu;
        const int r = t >> 1;
        const int f = min(nt * 128 + (r & 127), ff - 1);
        const size_t R = (size_t)e * 2 * ff + 2 * f + (r >= 128 ? 1 : 0);
        const size_t blk = R * nblk + 2 * sl + (t & 1);
        *reinterpret_cast<uint4*>(codes + (size_t)i * 16) = *reinterpret_cast<const uint4*>(w + blk * 16);
        scales[i] = sc[blk];
    }
}

__global__ __launch_bounds__(256) void mx_pack_down_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ sc,
                                                           int ff, int d, long long pieces, int ntd, int sd,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const size_t nblk = ff / 32;
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < pieces; i += (long long)gridDim.x * 256) {
        const int r = (int)(i % GBN);
        long long rest = i / GBN;
        const int sl = (int)(rest % sd);
        rest /= sd;
        const int nt = (int)(rest % ntd);
        const long long e = rest / ntd;
        const int n = min(nt * GBN + r, d - 1);
        const size_t blk = ((size_t)e * d + n) * nblk + sl;
        *reinterpret_cast<uint4*>(codes + (size_t)i * 16) = *reinterpret_cast<const uint4*>(w + blk * 16);
        scales[i] = sc[blk];
    }
}

// The grouped copy of Q4_K expert weights, one thread per (tile row, super-block): per
// (expert, N-tile, super-block) group of 256 tile rows, the rows' 16-byte headers, then
// quant run c (c = 0..3) of every row as 32 bytes.  Up tiles: rows 0..127 are gate units
// nt * 128 + r, rows 128..255 the up units (clamped to the last unit); down tiles: output
// rows nt * 256 + r (clamped to the last row).
__global__ __launch_bounds__(256) void q4k_pack_kernel(const uint8_t* __restrict__ w_a, const uint8_t* __restrict__ w_b,
                                                       int rows, int tile_rows, int half, long long items, int nt_n,
                                                       int nsb, uint8_t* __restrict__ out) {
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < items; i += (long long)gridDim.x * 256) {
        const int r = (int)(i % GBN);
        long long rest = i / GBN;
        const int sb = (int)(rest % nsb);
        rest /= nsb;
        const int nt = (int)(rest % nt_n);
        const long long e = rest / nt_n;
        // half > 0: rows >= half come from w_b (the up units of an up tile)
        const bool second = half > 0 && r >= half;
        const int local = half > 0 ? (second ? r - half : r) : r;
        const int n = min(nt * tile_rows + local, rows - 1);
        const uint8_t* src = (second ? w_b : w_a) + (((size_t)e * rows + n) * nsb + sb) * kQ4kBlockBytes;
        uint8_t* grp = out + (((size_t)e * nt_n + nt) * nsb + sb) * GBN * kQ4kBlockBytes;
        *reinterpret_cast<uint4*>(grp + r * 16) = *reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint8_t* dst = grp + GBN * 16 + (size_t)c * GBN * 32 + r * 32;
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src + 16 + 32 * c);
            *reinterpret_cast<uint4*>(dst + 16) = *reinterpret_cast<const uint4*>(src + 32 + 32 * c);
        }
    }
}

// The grouped copy of dense bf16 down weights (moe_grouped_pack): piece
// i = ((tile * slices + s) * 256 + r) holds the 32 inputs 32s .. 32s+31 of output row
// min(nt * 256 + r, d - 1) of the tile's expert, where tile = e * NTd + nt; one thread per
// piece (64 bytes).
__global__ __launch_bounds__(256) void dense_down_pack_kernel(const uint16_t* __restrict__ w, int d, int K,
                                                              long long pieces, int ntd, uint16_t* __restrict__ out) {
    const int slices = K / kDownKW;
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < pieces; i += (long long)gridDim.x * 256) {
        const int r = (int)(i % GBN);
        long long rest = i / GBN;
        const int sl = (int)(rest % slices);
        rest /= slices;
        const int nt = (int)(rest % ntd);
        const long long e = rest / ntd;
        const int n = min(nt * GBN + r, d - 1);
        const uint4* src = reinterpret_cast<const uint4*>(w + ((size_t)e * d + n) * K + (size_t)sl * kDownKW);
        uint4* dst = reinterpret_cast<uint4*>(out + (size_t)i * kDownKW);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = src[q];
    }
}

}  // namespace

hipError_t launch_router_mfma(const moe_layer& L, const void* x, int T, float* logits, int ld,
                              hipStream_t s) {
    const int nn = (L.n_expert + RBN - 1) / RBN;
    // The tallest token tile that still makes one block per CU (256 CUs), else 32 rows.
    const auto blocks = [&](int mt) { return ((T + mt - 1) / mt) * nn; };
    const int mt = blocks(128) >= 256 ? 128 : blocks(64) >= 256 ? 64 : 32;
    const auto* xs = static_cast<const uint16_t*>(x);
    const auto* wr = static_cast<const uint16_t*>(L.w_router);
    if (mt == 128)
        router_mfma_kernel<128><<<blocks(128), kRThreads, 0, s>>>(xs, wr, L.b_router, T, L.d, L.n_expert, nn, logits, ld);
    else if (mt == 64)
        router_mfma_kernel<64><<<blocks(64), kRThreads, 0, s>>>(xs, wr, L.b_router, T, L.d, L.n_expert, nn, logits, ld);
    else
        router_mfma_kernel<32><<<blocks(32), kRThreads, 0, s>>>(xs, wr, L.b_router, T, L.d, L.n_expert, nn, logits, ld);
    return hipGetLastError();
}

int grouped_max_mtiles(int E, int T, int k, bool shared) {
    const long long tk = (long long)T * k;
    long long b = tk / BM + (tk < E ? tk : E) + 1;
    if (shared) b += (T + BM - 1) / BM;
    return (int)b;
}

MxPackLayout mx_pack_layout(const moe_layer& L) {
    MxPackLayout p{};
    p.ntu = (L.ff + 127) / 128;
    p.su = L.d / kUpKW;
    p.ntd = (L.d + GBN - 1) / GBN;
    p.sd = L.ff / kDownKW;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return at;
    };
    const size_t E = (size_t)L.n_expert;
    p.up_codes = take(E * p.ntu * p.su * kGThreads * 16);
    p.up_scales = take(E * p.ntu * p.su * kGThreads);
    p.dn_codes = take(E * p.ntd * p.sd * GBN * 16);
    p.dn_scales = take(E * p.ntd * p.sd * GBN);
    p.total = off;
    return p;
}

DensePackLayout dense_pack_layout(const moe_layer& L) {
    DensePackLayout p{};
    p.ntd = (L.d + GBN - 1) / GBN;
    const size_t routed = (size_t)L.n_expert * p.ntd * GBN * L.ff * 2;
    p.dn = 0;
    p.sh = (routed + 255) / 256 * 256;
    p.total = p.sh + (size_t)p.ntd * GBN * L.shared_ff * 2;
    return p;
}

hipError_t launch_dense_pack(const moe_layer& L, void* dst, hipStream_t s) {
    const DensePackLayout p = dense_pack_layout(L);
    uint8_t* base = static_cast<uint8_t*>(dst);
    auto blocks = [](long long n) { return (unsigned)std::min<long long>((n + 255) / 256, 8192); };
    const long long routed = (long long)L.n_expert * p.ntd * (L.ff / kDownKW) * GBN;
    dense_down_pack_kernel<<<blocks(routed), 256, 0, s>>>(static_cast<const uint16_t*>(L.w_down), L.d, L.ff, routed,
                                                          p.ntd, reinterpret_cast<uint16_t*>(base + p.dn));
    if (L.shared_ff > 0) {
        const long long sh = (long long)p.ntd * (L.shared_ff / kDownKW) * GBN;
        dense_down_pack_kernel<<<blocks(sh), 256, 0, s>>>(static_cast<const uint16_t*>(L.ws_down), L.d, L.shared_ff, sh,
                                                          p.ntd, reinterpret_cast<uint16_t*>(base + p.sh));
    }
    return hipGetLastError();
}

Q4kPackLayout q4k_pack_layout(const moe_layer& L) {
    Q4kPackLayout p{};
    p.ntu = (L.ff + 127) / 128;
    p.ntd = (L.d + GBN - 1) / GBN;
    const size_t group = (size_t)GBN * kQ4kBlockBytes, E = (size_t)L.n_expert;
    const size_t up = E * p.ntu * (L.d / kQ4kBlockWeights) * group;
    p.up = 0;
    p.dn = (up + 255) / 256 * 256;
    p.total = p.dn + E * p.ntd * (L.ff / kQ4kBlockWeights) * group;
    return p;
}

hipError_t launch_q4k_pack(const moe_layer& L, void* dst, hipStream_t s) {
    const Q4kPackLayout p = q4k_pack_layout(L);
    uint8_t* base = static_cast<uint8_t*>(dst);
    const int nsb_u = L.d / kQ4kBlockWeights, nsb_d = L.ff / kQ4kBlockWeights;
    const long long up = (long long)L.n_expert * p.ntu * nsb_u * GBN;
    const long long dn = (long long)L.n_expert * p.ntd * nsb_d * GBN;
    auto blocks = [](long long n) { return (unsigned)std::min<long long>((n + 255) / 256, 8192); };
    q4k_pack_kernel<<<blocks(up), 256, 0, s>>>(static_cast<const uint8_t*>(L.w_gate), static_cast<const uint8_t*>(L.w_up),
                                               L.ff, 128, 128, up, p.ntu, nsb_u, base + p.up);
    q4k_pack_kernel<<<blocks(dn), 256, 0, s>>>(static_cast<const uint8_t*>(L.w_down), nullptr, L.d, GBN, 0, dn, p.ntd,
                                               nsb_d, base + p.dn);
    return hipGetLastError();
}

hipError_t launch_mx_pack(const moe_layer& L, void* dst, hipStream_t s) {
    const MxPackLayout p = mx_pack_layout(L);
    uint8_t* base = static_cast<uint8_t*>(dst);
    const long long up = (long long)L.n_expert * p.ntu * p.su * kGThreads;
    const long long dn = (long long)L.n_expert * p.ntd * p.sd * GBN;
    auto blocks = [](long long n) { return (unsigned)std::min<long long>((n + 255) / 256, 8192); };
    mx_pack_up_kernel<<<blocks(up), 256, 0, s>>>(static_cast<const uint8_t*>(L.w_gate_up), L.w_gate_up_scales, L.ff,
                                                 L.d, up, p.ntu, p.su, base + p.up_codes, base + p.up_scales);
    mx_pack_down_kernel<<<blocks(dn), 256, 0, s>>>(static_cast<const uint8_t*>(L.w_down), L.w_down_scales, L.ff, L.d,
                                                   dn, p.ntd, p.sd, base + p.dn_codes, base + p.dn_scales);
    return hipGetLastError();
}

hipError_t launch_grouped_ffn(const moe_layer& L, const void* x, int T, const int32_t* perm_token,
                              const Group* groups, const PlanMeta* meta, const TileDesc* tiles,
                              uint16_t* H, int hstride, const float* row_w, void* y, bool y_bf16,
                              int ksplit, float* partial, hipStream_t s) {
    const bool shared = L.shared_ff > 0;
    const int mt = grouped_max_mtiles(L.n_expert, T, L.k, shared);
    const int ffmax = L.ff > L.shared_ff ? L.ff : L.shared_ff;
    const int nn_up = (ffmax + 127) / 128;
    // MXFP4 experts: the clamped variant without a shared expert (checked by the caller);
    // w_gate_up / w_down hold the FP4 blocks, the *_scales fields their E8M0 scales.
    // Q4_K experts: SwiGLU, w_gate / w_up / w_down hold the super-blocks (K multiple of 256).
    const bool mx = L.expert_format == MOE_EXPERTS_MXFP4;
    const bool q4 = L.expert_format == MOE_EXPERTS_Q4K;
    if (mx && (L.act != MOE_ACT_SWIGLU_OAI || shared || L.d % 64 || L.ff % 32)) return hipErrorInvalidValue;
    if (q4 && (L.act != MOE_ACT_SWIGLU || L.d % kQ4kBlockWeights || L.ff % kQ4kBlockWeights))
        return hipErrorInvalidValue;
    // With the grouped copy (MXFP4 or Q4_K), both GEMMs read their weight slices from it.
    const bool packed = L.grouped_pack != nullptr;
    const DensePackLayout pdn = packed && !mx && !q4 ? dense_pack_layout(L) : DensePackLayout{};
    const uint16_t* wd_pack = packed && !mx && !q4 ? reinterpret_cast<const uint16_t*>(
                                                         static_cast<const uint8_t*>(L.grouped_pack) + pdn.dn) : nullptr;
    const uint16_t* wsd_pack = wd_pack && shared ? reinterpret_cast<const uint16_t*>(
                                                       static_cast<const uint8_t*>(L.grouped_pack) + pdn.sh) : nullptr;
    const uint8_t* pack = static_cast<const uint8_t*>(L.grouped_pack);
    const Q4kPackLayout pq = q4 && packed ? q4k_pack_layout(L) : Q4kPackLayout{};
    const auto* q4_gate = q4 ? (packed ? pack + pq.up : static_cast<const uint8_t*>(L.w_gate)) : nullptr;
    const auto* q4_up = q4 && !packed ? static_cast<const uint8_t*>(L.w_up) : nullptr;
    const auto* q4_down = q4 ? (packed ? pack + pq.dn : static_cast<const uint8_t*>(L.w_down)) : nullptr;
    UpArgs u{static_cast<const uint16_t*>(x), perm_token, groups, meta, tiles,
             static_cast<const uint16_t*>(L.w_gate), static_cast<const uint16_t*>(L.w_up),
             static_cast<const uint16_t*>(L.w_gate_up), static_cast<const uint16_t*>(L.b_gate_up),
             static_cast<const uint16_t*>(L.ws_gate), static_cast<const uint16_t*>(L.ws_up),
             mx ? static_cast<const uint8_t*>(L.w_gate_up) : nullptr, mx ? L.w_gate_up_scales : nullptr, q4_gate,
             q4_up, H, hstride, T, L.d, L.ff, L.shared_ff, nn_up, L.oai_alpha, L.oai_limit};
    const bool mx_packed = mx && packed;
    const MxPackLayout pk = mx_packed ? mx_pack_layout(L) : MxPackLayout{};
    if (mx_packed) {
        u.mx_w = pack + pk.up_codes;
        u.mx_s = pack + pk.up_scales;
        u.mx_packed = 1;
    }
    u.q4_packed = q4 && packed ? 1 : 0;
    u.h_rows = T * L.k + (shared ? T : 0);
    const dim3 gu((unsigned)grid_blocks(mt, nn_up));
    // A group holds at most T rows: up to 128 tokens every weight slice is read by one block.
    const bool ntb = T <= BM;
#define SMOE_GG_UP(OAI, WF)                                                          \
    do {                                                                             \
        if (ntb) gg_up_kernel<OAI, WF, true><<<gu, kGThreads, 0, s>>>(u);            \
        else gg_up_kernel<OAI, WF, false><<<gu, kGThreads, 0, s>>>(u);               \
    } while (0)
    if (mx) SMOE_GG_UP(true, kWMx);
    else if (q4) SMOE_GG_UP(false, kWQ4k);
    else if (L.act == MOE_ACT_SWIGLU_OAI) SMOE_GG_UP(true, kWDense);
    else SMOE_GG_UP(false, kWDense);
#undef SMOE_GG_UP
    const uint8_t* mx_dw = mx_packed ? pack + pk.dn_codes : mx ? static_cast<const uint8_t*>(L.w_down) : nullptr;
    const uint8_t* mx_ds = mx_packed ? pack + pk.dn_scales : mx ? L.w_down_scales : nullptr;
    const int nn = (L.d + GBN - 1) / GBN;
    const int rows = T * L.k + (shared ? T : 0);
    const auto* b_down = static_cast<const uint16_t*>(L.b_down);
    const int wf = mx ? kWMx : q4 ? kWQ4k : kWDense;
    if (ksplit > 1) {
        // The reduce grid has a z-slice per tile row: min(BM, T*k) covers every row of a tile
        // (a group never holds more than the T*k routed rows).
        if (!partial || ksplit > kMaxSplitPlanes || (L.ff / ksplit) % kDownKW ||
            (shared && (L.shared_ff / ksplit) % kDownKW) || L.ff % ksplit || L.shared_ff % ksplit)
            return hipErrorInvalidValue;
        DownArgs dn{H, groups, meta, tiles, static_cast<const uint16_t*>(L.w_down), nullptr,
                    static_cast<const uint16_t*>(L.ws_down), mx_dw, mx_ds, q4_down, nullptr, partial, hstride, L.d,
                    L.ff, L.shared_ff, nn, ksplit, rows, (mx || q4) && packed ? 1 : 0, wd_pack, wsd_pack};
        const dim3 gs((unsigned)grid_blocks(mt, nn * ksplit));
#define SMOE_GG_SPLIT(WF)                                                            \
    do {                                                                             \
        if (ntb) gg_down_kernel<float, WF, true><<<gs, kGThreads, 0, s>>>(dn);       \
        else gg_down_kernel<float, WF, false><<<gs, kGThreads, 0, s>>>(dn);          \
    } while (0)
        if (wf == kWMx) SMOE_GG_SPLIT(kWMx);
        else if (wf == kWQ4k) SMOE_GG_SPLIT(kWQ4k);
        else SMOE_GG_SPLIT(kWDense);
#undef SMOE_GG_SPLIT
        const dim3 gr((unsigned)((L.d + 1023) / 1024), (unsigned)mt, (unsigned)min(BM, T * L.k));
        if (y_bf16)
            splitk_reduce_kernel<uint16_t><<<gr, 256, 0, s>>>(partial, ksplit, rows, meta, tiles, b_down, row_w,
                                                              static_cast<uint16_t*>(y), L.d);
        else
            splitk_reduce_kernel<float><<<gr, 256, 0, s>>>(partial, ksplit, rows, meta, tiles, b_down, row_w,
                                                           static_cast<float*>(y), L.d);
        return hipGetLastError();
    }
    DownArgs dn{H, groups, meta, tiles, static_cast<const uint16_t*>(L.w_down), b_down,
                static_cast<const uint16_t*>(L.ws_down), mx_dw, mx_ds, q4_down, row_w, y, hstride, L.d, L.ff,
                L.shared_ff, nn, 1, rows, (mx || q4) && packed ? 1 : 0, wd_pack, wsd_pack};
    const dim3 gd((unsigned)grid_blocks(mt, nn));
#define SMOE_GG_DOWN(WF)                                                              \
    do {                                                                              \
        if (y_bf16 && ntb) gg_down_kernel<uint16_t, WF, true><<<gd, kGThreads, 0, s>>>(dn);   \
        else if (y_bf16) gg_down_kernel<uint16_t, WF, false><<<gd, kGThreads, 0, s>>>(dn);    \
        else if (ntb) gg_down_kernel<float, WF, true><<<gd, kGThreads, 0, s>>>(dn);           \
        else gg_down_kernel<float, WF, false><<<gd, kGThreads, 0, s>>>(dn);                   \
    } while (0)
    if (wf == kWMx) SMOE_GG_DOWN(kWMx);
    else if (wf == kWQ4k) SMOE_GG_DOWN(kWQ4k);
    else SMOE_GG_DOWN(kWDense);
#undef SMOE_GG_DOWN
    return hipGetLastError();
}

}  // namespace smoe

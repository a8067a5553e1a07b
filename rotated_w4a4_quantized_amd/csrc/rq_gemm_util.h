// rq_gemm_util.h -- device helpers shared by the matrix-core GEMMs that stream
// operands through LDS with direct-to-LDS loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace rq {
namespace gemm {

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its global loads in flight (the prefetched stages).
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>):
// accumulator registers must only ever be indexed by compile-time constants.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One direct-to-LDS load of 16 bytes per active lane
// (global_load_lds_dwordx4): lane l's bytes, from sbase + voff, land at LDS
// byte lds_addr + 16 l.  M0 holds the LDS address (saved and restored: the
// compiler reserves M0 and does not expect it to change; one wait state
// after writing it); the load has no VGPR result, so its completion is
// counted by hand with wait_vm.  Every scalar operand must be wave-uniform.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds_addr)
        : "memory");
}

// Tile id for workgroup `bid`: contiguous id ranges per XCD (workgroup id
// mod 8), then groups of 8 token tiles x all channel tiles, for L2 reuse.
__device__ inline void tile_of(int bid, int nblk, int tiles_t, int tiles_n, int &tt, int &tn) {
    int id = bid;
    const int full = (nblk / 8) * 8;
    if (bid < full) id = (bid % 8) * (full / 8) + bid / 8;
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = id / per_group;
    const int first = group * GM;
    const int gsize = min(tiles_t - first, GM);
    const int in = id - group * per_group;
    tt = first + in % gsize;
    tn = in / gsize;
}

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 (round to nearest even), one instruction
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    const f2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

}  // namespace gemm
}  // namespace rq

// rq_gemm_fp6.hip -- W4A4 GEMM with the per-token x per-channel rescale on
// gfx950's FP6 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4, E2M3 operands).
//
// Math ("TR-DQ" section 3.1: Y = X W with per-token activation and
// per-channel weight scales):
//   acc[t][n] = sum_{k < Kq} qa[t][k] qw[n][koff + k]        (exact)
//   RPBH:  Y = s_a[t] s_w[n] acc / b
//   DENSE: Y = s_w[n] (lr[t][n] + s_a[t] acc),  lr = sum_{j<r} bf16(u)[t][j] qw[n][j]
//
// Why FP6 carries INT4 exactly.  An E2M3 element (sign, 2 exponent bits with
// bias 1, 3 mantissa bits) whose 6-bit code is an unsigned value u < 16 with
// the two top bits clear decodes to u / 8: codes 0..7 are the subnormals
// m / 8, codes 8..15 have exponent 1 and decode to 1 + m / 8.  So:
//   * activations: u = q + 8, which is the two's-complement nibble with its
//     top bit flipped (one XOR per eight codes), placed in the low four bits
//     of a 6-bit field;
//   * weights (packed offline): sign-magnitude codes (q < 0) << 5 | |q|,
//     i.e. subnormal q / 8.
// With both E8M0 block scales at 2^3 the matrix core returns
// sum_k (qa + 8) qw = acc + 8 wsum[n], where wsum[n] = sum_k qw[n][k] is
// stored in the weight blob.  Every product and partial sum is an integer of
// magnitude <= 15 * 7 * 16384 < 2^24, so the fp32 accumulation is exact in
// any order, and acc is recovered exactly as a float.
//
// Operand layout of one 32x32x64 MFMA with 6-bit elements: lane l supplies
// row (A) / column (B) l % 32 and 32 consecutive-in-K elements of half
// l / 32, six dwords, element e at bits [6e, 6e + 6).  Which k feeds which
// element only has to agree between A and B.  The activation side takes the
// 32 codes of a 16-byte chunk (canonical order: low nibble = even k) and
// spreads them into 6-bit fields with a fixed permutation that needs no
// per-element shifts (to_fp6 below); the offline weight packer
// (rq_host.cpp) lays the weight codes out in the same permutation, already
// in per-lane fragment order.
//
// Tiling: a workgroup owns BT tokens x BN channels, waves WT x WN.  Per
// 128-k stage the LDS holds the activation nibbles [BT/32][2][64 lanes][16 B]
// and the weight fragments [BN/32][3][64 lanes][16 B]; both are filled by
// direct-to-LDS loads (global_load_lds_dwordx4, 1 KB per instruction) into
// NBUF rotating buffers, and every fragment read is a conflict-free
// ds_read_b128 of 64 consecutive 16-byte slots.  MFMA A = weight rows,
// MFMA B = token rows, so each lane of the accumulator owns one token and
// runs of four consecutive output channels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "rq_internal.h"

namespace rq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kActStageBytes = 64;      // nibble bytes per token row per stage
constexpr uint32_t kScale2p3 = 130u * 0x01010101u;   // E8M0 2^3 in every byte

struct Fp6Args {
    const uint8_t *A;      // activation codes [T][lda]
    const uint8_t *Bmma;   // weight fragments [ntiles][S][3][64][16]
    const uint8_t *Bcan;   // canonical weight codes [N][ldb] (low-rank part)
    const float *sa;       // [T]
    const float *sw;       // [N]
    const int32_t *wsum;   // [N]
    const uint16_t *top;   // bf16 [T][r] or null
    const float *bias;     // [N] or null
    void *Y;               // [T][N]
    int64_t T;
    int N;
    int lda;               // bytes per activation row (Kq / 2)
    int ldb;               // bytes per canonical weight row (K / 2)
    int S;                 // 128-k stages (weight blob)
    int ntiles;            // 32-row weight tiles in the blob
    int r;                 // low-rank width (multiple of 32) or 0
    int ydt;               // rq_dtype
    int tiles_t, tiles_n;
    float post;            // 1 / b_div
};

__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 canonical nibble codes (a: k 0..7, b: k 8..15 of a group) -> sixteen
// 6-bit fields holding q + 8, in three dwords.  Field f takes canonical
// offset {0,1,3,4,6,7,9,10,12,13,15,8,2,11,5,14}[f]: with that order each
// field is a nibble of a or b shifted by 0 or 2 bits, so three masks per
// output dword do the spreading.
__device__ inline void to_fp6(uint32_t a, uint32_t b, uint32_t &d0, uint32_t &d1, uint32_t &d2) {
    a ^= 0x88888888u;
    b ^= 0x88888888u;
    const uint32_t a2 = a << 2, b2 = b << 2;
    d0 = (a & 0x0F00F00Fu) | (a2 & 0xC03C03C0u);
    d1 = (a >> 30) | (b & 0xF00F00F0u) | (b2 & 0x03C03C00u);
    d2 = (a & 0x00F00F00u) | (b2 & 0x3C03C03Cu);
}

__device__ inline uint32_t bf16_rne_bits(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;   // finite x
}

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>):
// accumulator registers must only ever be indexed by compile-time constants
// (a runtime index sends the whole array to scratch memory).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BT_, int BN_, int WT_, int WN_, int NBUF_, int OCC_>
struct Cfg {
    static constexpr int BT = BT_, BN = BN_, WT = WT_, WN = WN_, NBUF = NBUF_, OCC = OCC_;
    static constexpr int NW = WT * WN;
    static constexpr int NTH = 64 * NW;
    static constexpr int FT = BT / WT / 32;   // token fragments per wave
    static constexpr int FN = BN / WN / 32;   // channel fragments per wave
    static constexpr int ACT_STAGE = BT * kActStageBytes;
    static constexpr int W_STAGE = BN * 96;
    static constexpr int LDS_STAGE = ACT_STAGE + W_STAGE;
    static constexpr int NQA = BT / 16;       // 1 KB activation loads per stage
    static constexpr int NQW = BN / 32 * 3;   // 1 KB weight loads per stage
    static constexpr int NA = NQA / NW;       // ... issued by each wave
    static constexpr int NB = NQW / NW;
    static constexpr int IPW = NA + NB;
    static constexpr int OUT_STRIDE = BN * 2 + 16;
    static constexpr int LDS_BYTES =
        NBUF * LDS_STAGE > BT * OUT_STRIDE ? NBUF * LDS_STAGE : BT * OUT_STRIDE;
    static_assert(BT % (32 * WT) == 0 && BN % (32 * WN) == 0, "tile shape");
    static_assert(NA * NW == NQA && NB * NW == NQW, "load split");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Direct-to-LDS loads of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's bytes land at LDS byte lds_addr + 16 l.  Inline asm so that the
// compiler does not see an LDS store it cannot tell apart from the fragment
// reads (it would otherwise wait for every load in flight, the prefetched
// stages too, before each read); completion is tracked by hand with
// s_waitcnt vmcnt.  M0 holds the LDS address (saved and restored, one wait
// state after writing it); the loads have no VGPR result.
//   dma16_s: address = 64-bit scalar base + 32-bit per-lane offset
//   dma16_v: 64-bit per-lane address
__device__ inline void dma16_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
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
__device__ inline void dma16_v(const void *gptr, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_addr)
        : "memory");
}

// a wave-uniform pointer, forced into scalar registers
__device__ inline const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t *>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// sixteen zero bytes: the source of activation chunks past the end of a row
__device__ __attribute__((aligned(16))) uint8_t g_zero16_fp6[16];

// Tile id for workgroup `bid`: contiguous id ranges per XCD (workgroup id
// mod 8), then groups of GM token tiles x all channel tiles, for L2 reuse.
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

// Epilogue of four consecutive channels nb .. nb + 3 (those below N) of
// token t: remove the offset-binary term, rescale, store as rq_dtype.
template <bool HAS_LR>
__device__ __forceinline__ void store4(const Fp6Args &a, int64_t t, int nb, float sat, float c0,
                                       float c1, float c2, float c3, const float (&lr4)[4]) {
    const float c[4] = {c0, c1, c2, c3};
    int32_t iv[4];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int n = nb + e < a.N ? nb + e : a.N - 1;
        const float accn = c[e] - (float)(8 * a.wsum[n]);   // exact: integers below 2^24
        iv[e] = (int32_t)accn;
        const float swn = a.sw[n];
        const float bn = a.bias ? a.bias[n] : 0.0f;
        if constexpr (HAS_LR)
            y[e] = swn * (lr4[e] + sat * accn) + bn;
        else
            y[e] = (accn * a.post) * (sat * swn) + bn;
    }
    const int64_t o = t * a.N + nb;
    if ((a.N % 4) == 0) {
        if (a.ydt == RQ_I32) {
            *reinterpret_cast<int4 *>(static_cast<int32_t *>(a.Y) + o) = make_int4(iv[0], iv[1], iv[2], iv[3]);
        } else if (a.ydt == RQ_F32) {
            *reinterpret_cast<float4 *>(static_cast<float *>(a.Y) + o) = make_float4(y[0], y[1], y[2], y[3]);
        } else {
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.Y) + o) =
                make_uint2(bf16_rne_bits(y[0]) | (bf16_rne_bits(y[1]) << 16),
                           bf16_rne_bits(y[2]) | (bf16_rne_bits(y[3]) << 16));
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (nb + e < a.N) {
            if (a.ydt == RQ_I32)
                static_cast<int32_t *>(a.Y)[o + e] = iv[e];
            else if (a.ydt == RQ_F32)
                static_cast<float *>(a.Y)[o + e] = y[e];
            else
                static_cast<uint16_t *>(a.Y)[o + e] = (uint16_t)bf16_rne_bits(y[e]);
        }
    }
}

template <class C, bool HAS_LR, bool TAIL>
__global__ void __launch_bounds__(C::NTH, C::OCC)
gemm_fp6_kernel(Fp6Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wt = wave / C::WN, wn = wave % C::WN;
    const int li = lane & 31, lg = lane >> 5;
    int tile_t, tile_n;
    tile_of(blockIdx.x, gridDim.x, a.tiles_t, a.tiles_n, tile_t, tile_n);
    const int64_t t0 = (int64_t)tile_t * C::BT;
    const int n0 = tile_n * C::BN;

    // This wave's direct-to-LDS loads: NA activation loads, then NB weight
    // loads.  Activation load q = wave NA + i fills fragment slot
    // (tf, ks) = (q / 2, q % 2): lane l brings bytes [32 ks + 16 (l / 32), +16)
    // of the stage's 64-byte slice of token t0 + 32 tf + l % 32 (rows past T
    // read row T - 1; their outputs are never stored).  Weight load
    // q = wave NB + i, (ntl, part) = (q / 3, q % 3), copies 1 KB of tile
    // n0 / 32 + ntl of the blob, already in fragment order.
    uint32_t aoff[C::NA];   // activation: byte offset from the tile's first row
#pragma unroll
    for (int i = 0; i < C::NA; ++i) {
        const int q = wave * C::NA + i;
        const int tf = q >> 1, ks = q & 1;
        int64_t t = t0 + 32 * tf + li;
        if (t >= a.T) t = a.T - 1;
        aoff[i] = (uint32_t)((t - t0) * a.lda + 32 * ks + 16 * lg);
    }
    const uint8_t *abase = uniform_ptr(a.A + t0 * a.lda);
    const uint32_t woff = lane * 16;
    const int nstage = a.S;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    auto issue = [&](int s, int buf) {
        const uint32_t lb = lds_base + buf * C::LDS_STAGE;
#pragma unroll
        for (int i = 0; i < C::NA; ++i) {
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lb + (wave * C::NA + i) * 1024);
            if constexpr (TAIL) {
                // a chunk past the end of the row reads sixteen zero bytes
                const int col = 32 * ((wave * C::NA + i) & 1) + 16 * lg;
                const uint8_t *p = s * kActStageBytes + col >= a.lda
                                       ? g_zero16_fp6
                                       : abase + aoff[i] + (int64_t)s * kActStageBytes;
                dma16_v(p, dst);
            } else {
                dma16_s(abase + (int64_t)s * kActStageBytes, aoff[i], dst);
            }
        }
#pragma unroll
        for (int i = 0; i < C::NB; ++i) {
            const int q = wave * C::NB + i;
            int nt = n0 / 32 + q / 3;
            if (nt >= a.ntiles) nt = a.ntiles - 1;
            const uint8_t *src = uniform_ptr(a.Bmma + (((int64_t)nt * a.S + s) * 3 + q % 3) * 1024);
            dma16_s(src, woff, __builtin_amdgcn_readfirstlane(lb + C::ACT_STAGE + q * 1024));
        }
    };
    // s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
    auto wait_vm = [](auto nc) {
        constexpr int n = decltype(nc)::value;
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
    };
    constexpr int D = C::NBUF - 1;
    auto wait_pending = [&](int pending) {
        if constexpr (D >= 3) if (pending >= 2) { wait_vm(std::integral_constant<int, 2 * C::IPW>()); return; }
        if constexpr (D >= 2) if (pending >= 1) { wait_vm(std::integral_constant<int, C::IPW>()); return; }
        wait_vm(std::integral_constant<int, 0>());
    };

    v16f acc[C::FN][C::FT];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    for (int p = 0; p < D && p < nstage; ++p) issue(p, p);
    wait_pending((nstage < D ? nstage : D) - 1);
    lds_barrier();

    int buf = 0;
    for (int s = 0; s < nstage; ++s) {
        if (s + D < nstage) issue(s + D, buf == 0 ? D : buf - 1);
        const uint8_t *L = lds + buf * C::LDS_STAGE;
        const uint8_t *LW = L + C::ACT_STAGE + wn * C::FN * 3 * 1024 + lane * 16;
        const uint8_t *LA = L + wt * C::FT * 2 * 1024 + lane * 16;
        // k-step 0 uses weight parts 0 and 1.xy, k-step 1 parts 1.zw and 2
        uint4 w0[C::FN], w1[C::FN];
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            w0[i] = *reinterpret_cast<const uint4 *>(LW + (i * 3 + 0) * 1024);
            w1[i] = *reinterpret_cast<const uint4 *>(LW + (i * 3 + 1) * 1024);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8i bt[C::FT];
#pragma unroll
            for (int j = 0; j < C::FT; ++j) {
                const uint4 an = *reinterpret_cast<const uint4 *>(LA + (j * 2 + ks) * 1024);
                uint32_t d0, d1, d2, d3, d4, d5;
                to_fp6(an.x, an.y, d0, d1, d2);
                to_fp6(an.z, an.w, d3, d4, d5);
                bt[j] = v8i{(int)d0, (int)d1, (int)d2, (int)d3, (int)d4, (int)d5, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < C::FN; ++i) {
                v8i wa;
                if (ks == 0) {
                    wa = v8i{(int)w0[i].x, (int)w0[i].y, (int)w0[i].z, (int)w0[i].w,
                             (int)w1[i].x, (int)w1[i].y, 0, 0};
                } else {
                    const uint4 w2 = *reinterpret_cast<const uint4 *>(LW + (i * 3 + 2) * 1024);
                    wa = v8i{(int)w1[i].z, (int)w1[i].w, (int)w2.x, (int)w2.y, (int)w2.z, (int)w2.w, 0, 0};
                }
#pragma unroll
                for (int j = 0; j < C::FT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        wa, bt[j], acc[i][j], 2, 2, 0, (int)kScale2p3, 0, (int)kScale2p3);
            }
        }
        {
            const int last = (s + D < nstage ? s + D : nstage - 1);   // newest stage issued
            wait_pending(last - (s + 1) > 0 ? last - (s + 1) : 0);
        }
        lds_barrier();
        buf = buf == D ? 0 : buf + 1;
    }

    // low-rank term (DENSE weights): lr[n][t] = sum_{j < r} qw[n][j] * bf16(top[t][j])
    v16f lr[HAS_LR ? C::FN : 1][HAS_LR ? C::FT : 1];
    if constexpr (HAS_LR) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int j = 0; j < C::FT; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) lr[i][j][e] = 0.0f;
        for (int k0 = 0; k0 < a.r; k0 += 16) {
            v8bf wa[C::FN], tb[C::FT];
#pragma unroll
            for (int i = 0; i < C::FN; ++i) {
                int n = n0 + wn * C::FN * 32 + i * 32 + li;
                if (n >= a.N) n = a.N - 1;
                const uint32_t w = *reinterpret_cast<const uint32_t *>(a.Bcan + (int64_t)n * a.ldb +
                                                                      (k0 + 8 * lg) / 2);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int q = ((int)(w << (28 - 4 * e))) >> 28;   // sign-extended nibble
                    wa[i][e] = (__bf16)(float)q;                       // exact: |q| <= 8
                }
            }
#pragma unroll
            for (int j = 0; j < C::FT; ++j) {
                int64_t t = t0 + wt * C::FT * 32 + j * 32 + li;
                if (t >= a.T) t = a.T - 1;
                const uint4 v = *reinterpret_cast<const uint4 *>(a.top + t * a.r + k0 + 8 * lg);
                tb[j] = __builtin_bit_cast(v8bf, v);
            }
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FT; ++j)
                    lr[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[i], tb[j], lr[i][j], 0, 0, 0);
        }
    }

    // Epilogue for a full tile with bf16 output: the scaled tile is staged
    // in LDS (free after the last barrier) and written back as whole row
    // segments; the accumulator layout alone would give every store
    // instruction 32 separate 8-byte pieces in 32 different rows.
    constexpr int kOutStride = C::OUT_STRIDE;
    if constexpr (!HAS_LR) {
        if (a.ydt == RQ_BF16 && t0 + C::BT <= a.T && n0 + C::BN <= a.N && (a.N % 8) == 0 &&
            a.bias == nullptr) {
            static_for<C::FN>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                static_for<4>([&](auto qc) {
                    constexpr int q = decltype(qc)::value;
                    const int nl = wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg;
                    const float4 sw4 = *reinterpret_cast<const float4 *>(a.sw + n0 + nl);
                    const int4 ws4 = *reinterpret_cast<const int4 *>(a.wsum + n0 + nl);
                    const float o0 = (float)(8 * ws4.x), o1 = (float)(8 * ws4.y);
                    const float o2 = (float)(8 * ws4.z), o3 = (float)(8 * ws4.w);
                    static_for<C::FT>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        const int tl = wt * C::FT * 32 + j * 32 + li;
                        const float sat = a.sa[t0 + tl] * a.post;
                        const float y0 = (acc[i][j][4 * q + 0] - o0) * (sat * sw4.x);
                        const float y1 = (acc[i][j][4 * q + 1] - o1) * (sat * sw4.y);
                        const float y2 = (acc[i][j][4 * q + 2] - o2) * (sat * sw4.z);
                        const float y3 = (acc[i][j][4 * q + 3] - o3) * (sat * sw4.w);
                        *reinterpret_cast<uint2 *>(lds + tl * kOutStride + 2 * nl) =
                            make_uint2(bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16),
                                       bf16_rne_bits(y2) | (bf16_rne_bits(y3) << 16));
                    });
                });
            });
            lds_barrier();
            constexpr int kChunksPerRow = C::BN * 2 / 16;
            constexpr int kChunks = C::BT * kChunksPerRow;
#pragma unroll 4
            for (int c = tid; c < kChunks; c += C::NTH) {
                const int row = c / kChunksPerRow, cc = c % kChunksPerRow;
                const uint4 v = *reinterpret_cast<const uint4 *>(lds + row * kOutStride + 16 * cc);
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.Y) + (t0 + row) * a.N + n0 + 8 * cc) = v;
            }
            return;
        }
    }

    // general epilogue: lane owns token t = ... + li and channels n = ... + 8 q + 4 lg + (0..3)
    static_for<C::FT>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int64_t t = t0 + wt * C::FT * 32 + j * 32 + li;
        const bool t_ok = t < a.T;
        const float sat = a.sa[t_ok ? t : a.T - 1];
        static_for<C::FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const int nb = n0 + wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg;
                float lr4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (HAS_LR) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) lr4[e] = lr[i][j][4 * q + e];
                }
                if (t_ok && nb < a.N)
                    store4<HAS_LR>(a, t, nb, sat, acc[i][j][4 * q + 0], acc[i][j][4 * q + 1],
                                   acc[i][j][4 * q + 2], acc[i][j][4 * q + 3], lr4);
            });
        });
    });
}

template <class C, bool HAS_LR>
hipError_t launch_cfg(Fp6Args a, hipStream_t s) {
    a.tiles_t = (int)((a.T + C::BT - 1) / C::BT);
    a.tiles_n = (a.N + C::BN - 1) / C::BN;
    const int nblk = a.tiles_t * a.tiles_n;
    if (a.lda % kActStageBytes)
        hipLaunchKernelGGL((gemm_fp6_kernel<C, HAS_LR, true>), dim3(nblk), dim3(C::NTH), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_fp6_kernel<C, HAS_LR, false>), dim3(nblk), dim3(C::NTH), 0, s, a);
    return hipGetLastError();
}

// 256 x 256 tiles, four waves of 64 tokens x 256 channels, one workgroup per
// CU: each token fragment is converted to FP6 by exactly one wave.
using CfgBig = Cfg<256, 256, 4, 1, 3, 1>;
// 128 x 128 tiles, four waves of 64 x 64, two workgroups per CU: small
// shapes and the low-rank path (which needs registers for its own sums).
using CfgMid = Cfg<128, 128, 2, 2, 3, 2>;

}  // namespace

int launch_gemm_fp6(const uint8_t *codes, const float *scale, const uint16_t *top, int64_t T,
                    const rq_weight_header *hdr, const void *blob, const float *bias, void *Y,
                    int y_dtype, void *stream) {
    Fp6Args a;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
    a.A = codes;
    a.Bmma = base + hdr->mma_offset;
    a.Bcan = base + hdr->codes_offset;
    a.sa = scale;
    a.sw = reinterpret_cast<const float *>(base + hdr->scale_offset);
    a.wsum = reinterpret_cast<const int32_t *>(base + hdr->wsum_offset);
    a.top = top;
    a.bias = bias;
    a.Y = Y;
    a.T = T;
    a.N = hdr->N;
    a.lda = (hdr->K - hdr->r) / 2;
    a.ldb = hdr->row_bytes;
    a.S = hdr->mma_stages;
    a.ntiles = hdr->mma_ntiles;
    a.r = hdr->r;
    a.ydt = y_dtype;
    a.post = 1.0f / (float)hdr->b_div;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.r > 0) return (int)launch_cfg<CfgMid, true>(a, s);
    if (T >= 256 && hdr->N >= 256) return (int)launch_cfg<CfgBig, false>(a, s);
    return (int)launch_cfg<CfgMid, false>(a, s);
}

}  // namespace rq

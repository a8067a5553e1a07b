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
// stored in the weight blob.  Asymmetric activations ("TR-DQ" section 3.1,
// codes u in [0, 15] with a per-token zero point z) are carried as u itself,
// and the epilogue removes z[t] wsum[n] instead of 8 wsum[n].  Every product and partial sum is an integer of
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

#include "rq_fp6.h"
#include "rq_internal.h"

namespace rq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kActStageBytes = 64;      // nibble bytes per token row per stage
constexpr uint32_t kScale2p3 = 130u * 0x01010101u;   // E8M0 2^3 in every byte

struct Fp6Args {
    const uint8_t *A;      // activation codes [T][lda] (canonical nibbles)
    const uint8_t *Amma;   // activation codes in FP6 fragment layout (rq_fp6.h), or null
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
    const float *za;       // asymmetric activations: zero point per token [T], else null
    uint32_t flip;         // canonical nibble -> FP6 field: XOR 0x88888888 (signed) or 0
};

__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
// token t: remove the offset term zt wsum[n] (zt = 8, or the token's zero
// point), rescale, store as rq_dtype.
template <bool HAS_LR>
__device__ __forceinline__ void store4(const Fp6Args &a, int64_t t, int nb, float sat, float zt,
                                       float c0, float c1, float c2, float c3,
                                       const float (&lr4)[4]) {
    const float c[4] = {c0, c1, c2, c3};
    int32_t iv[4];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int n = nb + e < a.N ? nb + e : a.N - 1;
        const float accn = c[e] - zt * (float)a.wsum[n];   // exact: integers below 2^24
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
    // loads d0 .. d1 - 1 of this wave's IPW loads for stage s into buffer buf
    // (activation loads first, then weight loads)
    auto issue_range = [&](int s, int buf, int d0, int d1) {
        const uint32_t lb = lds_base + buf * C::LDS_STAGE;
#pragma unroll
        for (int i = 0; i < C::NA; ++i) {
            if (i < d0 || i >= d1) continue;
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lb + (wave * C::NA + i) * 1024);
            if constexpr (TAIL) {
                // a chunk past the end of the row reads sixteen zero bytes
                const int col = 32 * ((wave * C::NA + i) & 1) + 16 * lg;
                const uint8_t *p = s * kActStageBytes + col >= a.lda
                                       ? g_zero16_fp6
                                       : abase + aoff[i] + (int64_t)s * kActStageBytes;
                dma16_v(p, dst);
            } else {
                dma16_s(uniform_ptr(abase + (int64_t)s * kActStageBytes), aoff[i], dst);
            }
        }
#pragma unroll
        for (int i = 0; i < C::NB; ++i) {
            if (C::NA + i < d0 || C::NA + i >= d1) continue;
            const int q = wave * C::NB + i;
            int nt = n0 / 32 + q / 3;
            if (nt >= a.ntiles) nt = a.ntiles - 1;
            const uint8_t *src = uniform_ptr(a.Bmma + (((int64_t)nt * a.S + s) * 3 + q % 3) * 1024);
            dma16_s(src, woff, __builtin_amdgcn_readfirstlane(lb + C::ACT_STAGE + q * 1024));
        }
    };
    auto issue = [&](int s, int buf) { issue_range(s, buf, 0, C::IPW); };
    // s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
    auto wait_vm = [](auto nc) {
        constexpr int n = decltype(nc)::value;
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
    };

    v16f acc[C::FN][C::FT];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Fragments of one stage: part 0 and 1 of every weight fragment plus the
    // k-step-0 activation chunks (R0), part 2 plus the k-step-1 chunks (R1).
    // k-step 0 multiplies parts 0 and 1.xy, k-step 1 parts 1.zw and 2.
    struct R0t { uint4 w0[C::FN], w1[C::FN], a[C::FT]; };
    struct R1t { uint4 w2[C::FN], a[C::FT]; };
    const uint8_t *LWb = lds + C::ACT_STAGE + wn * C::FN * 3 * 1024 + lane * 16;
    const uint8_t *LAb = lds + wt * C::FT * 2 * 1024 + lane * 16;
    auto read_r0 = [&](int b, R0t &r) {
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
            r.a[j] = *reinterpret_cast<const uint4 *>(LAb + b * C::LDS_STAGE + (j * 2 + 0) * 1024);
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            r.w0[i] = *reinterpret_cast<const uint4 *>(LWb + b * C::LDS_STAGE + (i * 3 + 0) * 1024);
            r.w1[i] = *reinterpret_cast<const uint4 *>(LWb + b * C::LDS_STAGE + (i * 3 + 1) * 1024);
        }
    };
    auto read_r1 = [&](int b, R1t &r) {
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
            r.a[j] = *reinterpret_cast<const uint4 *>(LAb + b * C::LDS_STAGE + (j * 2 + 1) * 1024);
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
            r.w2[i] = *reinterpret_cast<const uint4 *>(LWb + b * C::LDS_STAGE + (i * 3 + 2) * 1024);
    };
    auto convert = [&](const uint4 (&an)[C::FT], v8i (&bt)[C::FT]) {
#pragma unroll
        for (int j = 0; j < C::FT; ++j) {
            uint32_t d0, d1, d2, d3, d4, d5;
            to_fp6(an[j].x, an[j].y, d0, d1, d2, a.flip);
            to_fp6(an[j].z, an[j].w, d3, d4, d5, a.flip);
            bt[j] = v8i{(int)d0, (int)d1, (int)d2, (int)d3, (int)d4, (int)d5, 0, 0};
        }
    };
    auto mfma_row = [&](int i, const v8i &wa, const v8i (&bt)[C::FT]) {
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wa, bt[j], acc[i][j], 2, 2, 0, (int)kScale2p3, 0, (int)kScale2p3);
    };

    // Software pipeline over the NBUF = 3 LDS buffers, stage s in buffer
    // s % 3.  Per stage: k-step 0 MFMAs; wait until stage s + 1 has landed
    // and every wave is done reading buffer s % 3 (one barrier); read all
    // fragments of stage s + 1 while the k-step 1 MFMAs run, and start the
    // loads of stage s + 3 into buffer s % 3 between them.  So three stages
    // of global loads are in flight and the LDS reads of a stage overlap the
    // previous stage's MFMAs.
    static_assert(C::NBUF == 3, "pipeline written for three buffers");
    const int npre = nstage < 3 ? nstage : 3;
    for (int p = 0; p < npre; ++p) issue(p, p);
    if (npre == 3) wait_vm(std::integral_constant<int, 2 * C::IPW>());
    else if (npre == 2) wait_vm(std::integral_constant<int, C::IPW>());
    else wait_vm(std::integral_constant<int, 0>());
    lds_barrier();
    R0t r0;
    R1t r1;
    read_r0(0, r0);
    read_r1(0, r1);

    // One stage.  PF: issue the loads of stage s + 3; WAIT_IPW: at the
    // mid-stage wait, this wave's loads of stage s + 2 may still be in
    // flight.  Both compile-time, so the body is one basic block.
    int b = 0;
    auto stage = [&](int s, auto pf_c, auto wait_c) {
        constexpr bool PF = decltype(pf_c)::value;
        constexpr bool WAIT_IPW = decltype(wait_c)::value;
        const int bn = b == 2 ? 0 : b + 1;
        v8i bt0[C::FT], bt1[C::FT];
        convert(r0.a, bt0);
        // k-step 0
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            const v8i wa = v8i{(int)r0.w0[i].x, (int)r0.w0[i].y, (int)r0.w0[i].z, (int)r0.w0[i].w,
                               (int)r0.w1[i].x, (int)r0.w1[i].y, 0, 0};
            mfma_row(i, wa, bt0);
        }
        convert(r1.a, bt1);
        // stage s + 1 has landed (own loads, then every wave's), and every
        // wave's reads of buffer b are complete
        if constexpr (WAIT_IPW) wait_vm(std::integral_constant<int, C::IPW>());
        else wait_vm(std::integral_constant<int, 0>());
        lds_barrier();
        R0t r0n;
        R1t r1n;
        read_r0(bn, r0n);   // the last stage reads a stale buffer; never used
        read_r1(bn, r1n);
        // k-step 1, with the loads of stage s + 3 (into buffer b) between its MFMAs
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            const v8i wa = v8i{(int)r0.w1[i].z, (int)r0.w1[i].w, (int)r1.w2[i].x, (int)r1.w2[i].y,
                               (int)r1.w2[i].z, (int)r1.w2[i].w, 0, 0};
            mfma_row(i, wa, bt1);
            if constexpr (PF) issue_range(s + 3, b, (i * C::IPW) / C::FN, ((i + 1) * C::IPW) / C::FN);
        }
        r0 = r0n;
        r1 = r1n;
        b = bn;
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    for (int s = 0; s + 3 < nstage; ++s) stage(s, T_{}, T_{});
    // the last three stages: no further loads; at the wait of stage S - 3
    // the loads of stage S - 1 may still be in flight
    if (nstage >= 3) stage(nstage - 3, F_{}, T_{});
    if (nstage >= 2) stage(nstage - 2, F_{}, F_{});
    stage(nstage - 1, F_{}, F_{});

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
                    const float w0 = (float)ws4.x, w1 = (float)ws4.y, w2 = (float)ws4.z, w3 = (float)ws4.w;
                    static_for<C::FT>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        const int tl = wt * C::FT * 32 + j * 32 + li;
                        const float sat = a.sa[t0 + tl] * a.post;
                        const float zt = a.za ? a.za[t0 + tl] : 8.0f;   // zt * w exact
                        const float y0 = (acc[i][j][4 * q + 0] - zt * w0) * (sat * sw4.x);
                        const float y1 = (acc[i][j][4 * q + 1] - zt * w1) * (sat * sw4.y);
                        const float y2 = (acc[i][j][4 * q + 2] - zt * w2) * (sat * sw4.z);
                        const float y3 = (acc[i][j][4 * q + 3] - zt * w3) * (sat * sw4.w);
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
        const float zt = a.za ? a.za[t_ok ? t : a.T - 1] : 8.0f;
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
                    store4<HAS_LR>(a, t, nb, sat, zt, acc[i][j][4 * q + 0], acc[i][j][4 * q + 1],
                                   acc[i][j][4 * q + 2], acc[i][j][4 * q + 3], lr4);
            });
        });
    });
}

// ---------------------------------------------------------------------------
// The same GEMM on activations that rq_rotate_quant already wrote in the FP6
// fragment layout (rq_fp6.h): no conversion, so the main loop is MFMAs, LDS
// fragment reads and direct-to-LDS loads only (on gfx950 VALU work does not
// overlap the FP6 matrix core, so every VALU instruction in the loop costs
// MFMA time).  Both operands stream through LDS as [32 rows][3 pieces][64
// lanes][16 B] per 128-coordinate stage; a lane's three pieces are the
// twelve dwords of its k-step-0 and k-step-1 fragments, so the MFMA operands
// are plain sub-ranges of the loaded registers.
// ---------------------------------------------------------------------------
template <int BT_, int BN_, int WT_, int WN_>
struct MmaCfg {
    static constexpr int BT = BT_, BN = BN_, WT = WT_, WN = WN_;
    static constexpr int NW = WT * WN;
    static constexpr int NTH = 64 * NW;
    static constexpr int FT = BT / WT / 32;
    static constexpr int FN = BN / WN / 32;
    static constexpr int ACT_STAGE = BT / 32 * 3 * 1024;
    static constexpr int W_STAGE = BN / 32 * 3 * 1024;
    static constexpr int LDS_STAGE = ACT_STAGE + W_STAGE;
    static constexpr int NA = BT / 32 * 3 / NW;   // activation loads per wave per stage
    static constexpr int NB = BN / 32 * 3 / NW;   // weight loads per wave per stage
    static constexpr int IPW = NA + NB;
    // after the stage buffers (which the epilogue reuses for its output
    // slabs): the tile's per-token scales, per-channel scales, code sums and
    // per-token zero points, 1 KB each
    static constexpr int EPI_OFF = 3 * LDS_STAGE;
    static constexpr int LDS_BYTES = EPI_OFF + 4 * 1024;
    static_assert(BT == 256 && BN == 256, "one 1 KB direct-to-LDS load per epilogue array");
    static_assert(NW >= 4, "four waves load the epilogue arrays");
    static_assert(NA * NW == BT / 32 * 3 && NB * NW == BN / 32 * 3, "load split");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 (round to nearest even), one instruction
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    const f2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// one lane's three 16-byte pieces of a 32-row fragment pair
struct Frag {
    v4i p[3];
};
__device__ __forceinline__ v8i frag_k0(const Frag &f) {
    const v8i lo = __builtin_shufflevector(f.p[0], f.p[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, 4, 5, -1, -1);
}
__device__ __forceinline__ v8i frag_k1(const Frag &f) {
    const v8i hi = __builtin_shufflevector(f.p[1], f.p[2], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_shufflevector(hi, hi, 2, 3, 4, 5, 6, 7, -1, -1);
}
// An empty asm that "redefines" the fragment: code that uses the result
// cannot be scheduled above the asm, and the asm stays below the barrier
// before it (volatile asm keeps its order).
__device__ __forceinline__ void pin(Frag &f) {
    asm volatile("" : "+v"(f.p[0]), "+v"(f.p[1]), "+v"(f.p[2]));
}

template <class C, bool HAS_LR>
__global__ void __launch_bounds__(C::NTH, 1)
gemm_fp6_mma_kernel(Fp6Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar address math
    const int wt = wave / C::WN, wn = wave % C::WN;
    const int li = lane & 31, lg = lane >> 5;
    int tile_t, tile_n;
    tile_of(blockIdx.x, gridDim.x, a.tiles_t, a.tiles_n, tile_t, tile_n);
    const int64_t t0 = (int64_t)tile_t * C::BT;
    const int n0 = tile_n * C::BN;
    const int nstage = a.S;

    // Direct-to-LDS loads of this wave per stage: NA activation loads, then
    // NB weight loads, each one contiguous 1 KB piece: activation load
    // q = wave NA + i copies piece q % 3 of token tile t0 / 32 + q / 3 (tiles
    // past the last token are clamped to it; their outputs are never
    // stored), weight load q = wave NB + i piece q % 3 of weight tile
    // n0 / 32 + q / 3.
    const int atiles = (int)((a.T + 31) / 32);
    const uint32_t loff = lane * 16;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    auto issue = [&](int s, int buf) {
        const uint32_t lb = lds_base + buf * C::LDS_STAGE;
#pragma unroll
        for (int i = 0; i < C::NA; ++i) {
            const int q = wave * C::NA + i;
            int tt = (int)(t0 / 32) + q / 3;
            if (tt >= atiles) tt = atiles - 1;
            dma16_s(a.Amma + (((int64_t)tt * a.S + s) * 3 + q % 3) * 1024, loff, lb + q * 1024);
        }
#pragma unroll
        for (int i = 0; i < C::NB; ++i) {
            const int q = wave * C::NB + i;
            int nt = n0 / 32 + q / 3;
            if (nt >= a.ntiles) nt = a.ntiles - 1;
            dma16_s(a.Bmma + (((int64_t)nt * a.S + s) * 3 + q % 3) * 1024, loff, lb + C::ACT_STAGE + q * 1024);
        }
    };
    auto wait_vm = [](auto nc) {
        constexpr int n = decltype(nc)::value;
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
    };

    v16f acc[C::FN][C::FT];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const uint8_t *LA = lds + wt * C::FT * 3 * 1024 + lane * 16;
    const uint8_t *LW = lds + C::ACT_STAGE + wn * C::FN * 3 * 1024 + lane * 16;
    auto rd = [](const uint8_t *p) {
        Frag f;
#pragma unroll
        for (int part = 0; part < 3; ++part) f.p[part] = *reinterpret_cast<const v4i *>(p + part * 1024);
        return f;
    };
    auto rd_act = [&](int buf, int j) { return rd(LA + buf * C::LDS_STAGE + j * 3 * 1024); };
    auto rd_w = [&](int buf, int i) { return rd(LW + buf * C::LDS_STAGE + i * 3 * 1024); };
    // the MFMAs of weight fragment i: both k-steps, all token fragments
    auto mfma_frag = [&](auto ic, const Frag &w, const Frag (&act)[C::FT]) {
        constexpr int i = decltype(ic)::value;
        const v8i w0 = frag_k0(w), w1 = frag_k1(w);
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                w0, frag_k0(act[j]), acc[i][j], 2, 2, 0, (int)kScale2p3, 0, (int)kScale2p3);
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                w1, frag_k1(act[j]), acc[i][j], 2, 2, 0, (int)kScale2p3, 0, (int)kScale2p3);
    };

    // Three LDS buffers, stage s in buffer s % 3.  Within a stage the weight
    // fragments are consumed one at a time with the next one's LDS read in
    // flight; once every read of stage s has landed in registers, one
    // barrier (also covering: this wave's loads of stage s + 1 complete)
    // lets all waves read stage s + 1 -- issued before the last fragment's
    // MFMAs, so their latency hides behind them -- and frees buffer s % 3
    // for the loads of stage s + 3.
    static_assert(C::FN == 4, "pipeline written for four weight fragments per wave");
    // Full bf16 tiles take the staged epilogue; its per-token and
    // per-channel arrays are loaded to LDS ahead of the stage-0 loads (the
    // prologue's wait covers them).
    const bool fast = a.ydt == RQ_BF16 && t0 + C::BT <= a.T && n0 + C::BN <= a.N && (a.N % 8) == 0 &&
                      a.bias == nullptr;
    // zero points follow the scales ([2][T]): a 16-byte aligned start only
    // when T % 4 == 0, else they are read from global memory at the end
    const bool za_lds = a.za != nullptr && (reinterpret_cast<uintptr_t>(a.za) & 15) == 0;
    // Low-rank operands of the first 32 coordinates (every DENSE blob has
    // r >= 32), loaded ahead of the stage loads so that the prologue's wait
    // covers them: per weight fragment i and k-step kk the lane's eight
    // nibbles of channel row ..+ li, coordinates 16 kk + 8 lg .. + 7; per
    // token fragment j its eight bf16 top coefficients.
    uint32_t lrw[HAS_LR ? C::FN : 1][2];
    uint4 lrt[HAS_LR ? C::FT : 1][2];
    auto lr_load = [&](int k0, uint32_t (&w)[HAS_LR ? C::FN : 1], uint4 (&tv)[HAS_LR ? C::FT : 1]) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            int n = n0 + wn * C::FN * 32 + i * 32 + li;
            if (n >= a.N) n = a.N - 1;
            w[i] = *reinterpret_cast<const uint32_t *>(a.Bcan + (int64_t)n * a.ldb + (k0 + 8 * lg) / 2);
        }
#pragma unroll
        for (int j = 0; j < C::FT; ++j) {
            int64_t t = t0 + wt * C::FT * 32 + j * 32 + li;
            if (t >= a.T) t = a.T - 1;
            tv[j] = *reinterpret_cast<const uint4 *>(a.top + t * a.r + k0 + 8 * lg);
        }
    };
    if constexpr (HAS_LR) {
        if (a.ydt != RQ_I32) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint32_t w[C::FN];
                uint4 tv[C::FT];
                lr_load(16 * kk, w, tv);
#pragma unroll
                for (int i = 0; i < C::FN; ++i) lrw[i][kk] = w[i];
#pragma unroll
                for (int j = 0; j < C::FT; ++j) lrt[j][kk] = tv[j];
            }
        }
    }
    if (fast && (wave < 3 || (wave == 3 && za_lds))) {
        const void *src = wave == 0   ? static_cast<const void *>(a.sa + t0)
                          : wave == 1 ? static_cast<const void *>(a.sw + n0)
                          : wave == 2 ? static_cast<const void *>(a.wsum + n0)
                                      : static_cast<const void *>(a.za + t0);
        dma16_s(src, loff, lds_base + C::EPI_OFF + wave * 1024);
    }
    const int npre = nstage < 3 ? nstage : 3;
    for (int p = 0; p < npre; ++p) issue(p, p);
    if (npre == 3) wait_vm(std::integral_constant<int, 2 * C::IPW>());
    else if (npre == 2) wait_vm(std::integral_constant<int, C::IPW>());
    else wait_vm(std::integral_constant<int, 0>());
    lds_barrier();
    // Full bf16 tiles start the accumulators at -zt wsum[n] (zt = 8, or the
    // token's zero point): the MFMAs then leave acc - zt wsum, and every
    // partial sum is an integer of magnitude below 2^24, so this is exact and
    // the epilogue only rescales.
    if (fast) {
        const int32_t *e_ws = reinterpret_cast<const int32_t *>(lds + C::EPI_OFF + 2048);
        const float *e_za = reinterpret_cast<const float *>(lds + C::EPI_OFF + 3072);
        float zt[C::FT];
#pragma unroll
        for (int j = 0; j < C::FT; ++j) {
            const int tl = wt * C::FT * 32 + j * 32 + li;
            zt[j] = !a.za ? 8.0f : za_lds ? e_za[tl] : a.za[t0 + tl];
        }
        static_for<C::FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const int4 ws4 = *reinterpret_cast<const int4 *>(e_ws + wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg);
                const float w[4] = {(float)ws4.x, (float)ws4.y, (float)ws4.z, (float)ws4.w};
#pragma unroll
                for (int j = 0; j < C::FT; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[i][j][4 * q + c] = -(zt[j] * w[c]);
            });
        });
    }
    Frag A[C::FT], W0, W1;
#pragma unroll
    for (int j = 0; j < C::FT; ++j) A[j] = rd_act(0, j);
    W0 = rd_w(0, 0);
    W1 = rd_w(0, 1);

    int b = 0;
    auto stage = [&](int s, auto pf_c, auto wait_c) {
        constexpr bool PF = decltype(pf_c)::value;
        constexpr bool WAIT_IPW = decltype(wait_c)::value;
        const int bn = b == 2 ? 0 : b + 1;
        const Frag W2 = rd_w(b, 2);
        mfma_frag(std::integral_constant<int, 0>(), W0, A);
        Frag W3 = rd_w(b, 3);
        mfma_frag(std::integral_constant<int, 1>(), W1, A);
        mfma_frag(std::integral_constant<int, 2>(), W2, A);
        if constexpr (WAIT_IPW) wait_vm(std::integral_constant<int, C::IPW>());
        else wait_vm(std::integral_constant<int, 0>());
        lds_barrier();
        pin(W3);
        Frag An[C::FT];
#pragma unroll
        for (int j = 0; j < C::FT; ++j) An[j] = rd_act(bn, j);   // stale after the last stage; unused
        const Frag W0n = rd_w(bn, 0), W1n = rd_w(bn, 1);
        mfma_frag(std::integral_constant<int, 3>(), W3, A);
        if constexpr (PF) issue(s + 3, b);
#pragma unroll
        for (int j = 0; j < C::FT; ++j) A[j] = An[j];
        W0 = W0n;
        W1 = W1n;
        b = bn;
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    for (int s = 0; s + 3 < nstage; ++s) stage(s, T_{}, T_{});
    if (nstage >= 3) stage(nstage - 3, F_{}, T_{});
    if (nstage >= 2) stage(nstage - 2, F_{}, F_{});
    stage(nstage - 1, F_{}, F_{});

    // keep the epilogue below the main loop's last MFMAs (register pressure)
    __builtin_amdgcn_sched_barrier(0);
    // Low-rank term (DENSE weights, float outputs):
    //   Y = s_w[n] (s_a[t] acc + sum_{j < r} bf16(u)[t][j] qw[n][j])
    // The accumulators are first rescaled in place to s_a[t] (acc - zt
    // wsum[n]) (on full bf16 tiles the offset is already in them); the
    // bf16 matrix core then adds the products of the top coefficients and
    // the weights' leading r codes (exact in bf16: |q| <= 8) into the same
    // registers -- its 32x32 output layout is the FP6 one.  Raw int32
    // accumulators skip this.
    const bool lr_on = HAS_LR && a.ydt != RQ_I32;
    if constexpr (HAS_LR) {
        if (lr_on) {
            const float *e_sa = reinterpret_cast<const float *>(lds + C::EPI_OFF);
            static_for<C::FT>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const int tl = wt * C::FT * 32 + j * 32 + li;
                const int64_t t = t0 + tl < a.T ? t0 + tl : a.T - 1;
                const float sat = fast ? e_sa[tl] : a.sa[t];
                const float zt = a.za ? a.za[t] : 8.0f;
                static_for<C::FN>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    static_for<4>([&](auto qc) {
                        constexpr int q = decltype(qc)::value;
                        const int nb = n0 + wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg;
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int n = nb + c < a.N ? nb + c : a.N - 1;
                            const float off = fast ? 0.0f : zt * (float)a.wsum[n];   // exact
                            acc[i][j][4 * q + c] = (acc[i][j][4 * q + c] - off) * sat;
                        }
                    });
                });
            });
            auto lr_mfma = [&](const uint32_t (&w)[C::FN], const uint4 (&tv)[C::FT]) {
                v8bf wa[C::FN];
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int q = ((int)(w[i] << (28 - 4 * e))) >> 28;   // sign-extended nibble
                        wa[i][e] = (__bf16)(float)q;
                    }
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            wa[i], __builtin_bit_cast(v8bf, tv[j]), acc[i][j], 0, 0, 0);
            };
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint32_t w[C::FN];
                uint4 tv[C::FT];
#pragma unroll
                for (int i = 0; i < C::FN; ++i) w[i] = lrw[i][kk];
#pragma unroll
                for (int j = 0; j < C::FT; ++j) tv[j] = lrt[j][kk];
                lr_mfma(w, tv);
            }
            for (int k0 = 32; k0 < a.r; k0 += 16) {
                uint32_t w[C::FN];
                uint4 tv[C::FT];
                lr_load(k0, w, tv);
                lr_mfma(w, tv);
            }
        }
    }

    // Epilogue.  Full bf16 tiles: each wave scales its 64 tokens x 128
    // channels into a private slab of the stage buffers (every fragment read
    // of the last stage completed before that stage's barrier; the reads
    // issued after it are stale and unused), then copies the slab out as
    // 256-byte row segments.  No workgroup barrier.  Other tiles take the
    // general path.
    if (fast) {
        constexpr int kRowBytes = C::BN / C::WN * 2;      // one token's channels
        constexpr int kSlabStride = kRowBytes + 16;       // padded LDS row
        constexpr int kRows = C::FT * 32;
        static_assert(C::NW * kRows * kSlabStride <= 3 * C::LDS_STAGE, "slabs fit the stage buffers");
        uint8_t *slab = lds + wave * kRows * kSlabStride;
        const float *e_sa = reinterpret_cast<const float *>(lds + C::EPI_OFF);
        const float *e_sw = reinterpret_cast<const float *>(lds + C::EPI_OFF + 1024);
        // y = (acc - zt wsum[n]) (s_a post s_w); the offset is already in
        // acc (with the low-rank term: y = acc s_w, acc already final)
        float sat[C::FT];
#pragma unroll
        for (int j = 0; j < C::FT; ++j) sat[j] = HAS_LR ? 1.0f : e_sa[wt * C::FT * 32 + j * 32 + li] * a.post;
        static_for<C::FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const int nw = i * 32 + 8 * q + 4 * lg;   // channel within the wave's 128
                const float4 sw4 = *reinterpret_cast<const float4 *>(e_sw + wn * C::FN * 32 + nw);
                static_for<C::FT>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const float y0 = acc[i][j][4 * q + 0] * (sat[j] * sw4.x);
                    const float y1 = acc[i][j][4 * q + 1] * (sat[j] * sw4.y);
                    const float y2 = acc[i][j][4 * q + 2] * (sat[j] * sw4.z);
                    const float y3 = acc[i][j][4 * q + 3] * (sat[j] * sw4.w);
                    *reinterpret_cast<uint2 *>(slab + (j * 32 + li) * kSlabStride + 2 * nw) =
                        make_uint2(bf16x2_rne(y0, y1), bf16x2_rne(y2, y3));
                });
            });
        });
        // the slab's writes come from this wave only: order them before the reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // copy-out: one instruction moves 64 / kChunksPerRow rows of 16-byte
        // chunks; lane l takes chunk l % kChunksPerRow of row l / kChunksPerRow
        constexpr int kChunksPerRow = kRowBytes / 16;
        constexpr int kRowsPerInst = 64 / kChunksPerRow;
        static_assert(kRows % (8 * kRowsPerInst) == 0, "whole batches of eight instructions");
        const int lr = lane / kChunksPerRow, lc = lane % kChunksPerRow;
        const uint8_t *src = slab + lr * kSlabStride + 16 * lc;
        uint16_t *dst = static_cast<uint16_t *>(a.Y) + (t0 + wt * kRows + lr) * a.N + n0 +
                        wn * (kRowBytes / 2) + 8 * lc;
        // eight LDS reads in flight, then their eight stores (named values: an
        // array here was kept in scratch memory)
        auto ld = [&](int r) { return *reinterpret_cast<const uint4 *>(src + r * kSlabStride); };
        auto st = [&](int r, const uint4 &v) { *reinterpret_cast<uint4 *>(dst + (int64_t)r * a.N) = v; };
        constexpr int R = kRowsPerInst;
#pragma unroll 1
        for (int r0 = 0; r0 < kRows; r0 += 8 * R) {
            const uint4 v0 = ld(r0), v1 = ld(r0 + R), v2 = ld(r0 + 2 * R), v3 = ld(r0 + 3 * R);
            const uint4 v4 = ld(r0 + 4 * R), v5 = ld(r0 + 5 * R), v6 = ld(r0 + 6 * R), v7 = ld(r0 + 7 * R);
            st(r0, v0);
            st(r0 + R, v1);
            st(r0 + 2 * R, v2);
            st(r0 + 3 * R, v3);
            st(r0 + 4 * R, v4);
            st(r0 + 5 * R, v5);
            st(r0 + 6 * R, v6);
            st(r0 + 7 * R, v7);
        }
        return;
    }
    // general epilogue (with the low-rank term the accumulators are already
    // s_a (acc - zt wsum) + lr: only s_w remains, post is 1 for DENSE)
    static_for<C::FT>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int64_t t = t0 + wt * C::FT * 32 + j * 32 + li;
        const bool t_ok = t < a.T;
        const float sat = lr_on ? 1.0f : a.sa[t_ok ? t : a.T - 1];
        const float zt = lr_on ? 0.0f : a.za ? a.za[t_ok ? t : a.T - 1] : 8.0f;
        static_for<C::FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const int nb = n0 + wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg;
                const float lr4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (t_ok && nb < a.N)
                    store4<false>(a, t, nb, sat, zt, acc[i][j][4 * q + 0], acc[i][j][4 * q + 1],
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

// 256 x 256 tiles, eight waves of 64 tokens x 128 channels, one workgroup per
// CU: two waves per SIMD (128 accumulators each) hide each other's waits.
// Each token fragment is converted by the two waves that use it; four
// waves of 64 x 256 (one conversion per fragment, 256 accumulators, one
// wave per SIMD) were 11% slower.
using CfgBig = Cfg<256, 256, 4, 2, 3, 1>;
// 128 x 128 tiles, four waves of 64 x 64, two workgroups per CU: small
// shapes and the low-rank path (which needs registers for its own sums).
using CfgMid = Cfg<128, 128, 2, 2, 3, 2>;

}  // namespace

int launch_gemm_fp6(const uint8_t *codes, const uint8_t *codes_mma, const float *scale,
                    const float *zero, const uint16_t *top, int64_t T,
                    const rq_weight_header *hdr, const void *blob, const float *bias, void *Y,
                    int y_dtype, void *stream) {
    Fp6Args a;
    a.za = zero;
    a.flip = zero ? 0u : 0x88888888u;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
    a.A = codes;
    a.Amma = codes_mma;
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
    if (codes_mma) {
        // Activations already in the FP6 fragment layout (RPBH, or DENSE
        // with the low-rank term in the epilogue).
        // 256 x 256 tiles on eight waves of 64 tokens x 128 channels: 128
        // accumulators and about 200 registers per lane, so two waves share
        // each SIMD and one wave's LDS and barrier waits overlap the other's
        // MFMAs.  Four waves of 128 x 128 (256 accumulators, one wave per
        // SIMD) read a third less from LDS but were 14% slower.
        using C = MmaCfg<256, 256, 4, 2>;
        a.tiles_t = (int)((T + C::BT - 1) / C::BT);
        a.tiles_n = (a.N + C::BN - 1) / C::BN;
        if (a.r > 0)
            hipLaunchKernelGGL((gemm_fp6_mma_kernel<C, true>), dim3(a.tiles_t * a.tiles_n), dim3(C::NTH), 0, s, a);
        else
            hipLaunchKernelGGL((gemm_fp6_mma_kernel<C, false>), dim3(a.tiles_t * a.tiles_n), dim3(C::NTH), 0, s, a);
        return (int)hipGetLastError();
    }
    if (a.r > 0) return (int)launch_cfg<CfgMid, true>(a, s);
    // 256 x 256 tiles only when they fill at least half of the CUs; a
    // smaller layer runs on four times as many 128 x 128 tiles
    const int64_t big_tiles = ((T + 255) / 256) * (int64_t)((hdr->N + 255) / 256);
    if (T >= 256 && hdr->N >= 256 && big_tiles >= device_cus() / 2) return (int)launch_cfg<CfgBig, false>(a, s);
    return (int)launch_cfg<CfgMid, false>(a, s);
}

}  // namespace rq

// rq_gemm_w4a4.hip -- W4A4 GEMM with the per-token x per-channel rescale,
// on gfx950 int8 MFMA.
//
// Math ("TR-DQ" section 3.1: Y = X W with per-token activation and
// per-channel weight scales):
//   acc[t][n] = sum_{k < Kq} qa[t][k] qw[n][koff + k]        (exact)
//   RPBH:  Y = s_a[t] s_w[n] acc / b
//   DENSE: Y = s_w[n] (lr[t][n] + s_a[t] acc),  lr = sum_{j<r} bf16(u)[t][j] qw[n][j]
//
// This is the int8 engine of the INT4 GEMM (rq_w4a4_linear_engine with
// RQ_ENGINE_INT8); the default runs on the FP6 matrix cores
// (rq_gemm_fp6.hip) at twice the rate, with the same accumulators.
//
// 8-bit activations have their own kernel on fragment-ordered operands
// (rq_gemm_i8.hip).
//
// Widening: gfx950 has no 4-bit MFMA.  For a packed word p (eight nibbles,
// low nibble = even k), (p << 4) & 0xF0F0F0F0 holds 16 q for the even k and
// p & 0xF0F0F0F0 holds 16 q for the odd k, as int8 lanes.  Both operands
// are widened the same way, so v_mfma_i32_32x32x32_i8 returns 256 acc
// exactly (|256 acc| <= 256 * 49 * 16384 < 2^31).  How the 32 k-values of
// one MFMA are spread over lanes and bytes only has to agree between the two
// operands, and it does: lane group g of both operands carries bytes
// [32 g, 32 g + 32) of the stage's 64-byte row slice.
//
// Operand roles: MFMA A = weight rows (n), MFMA B = token rows (t), so the
// 32 x 32 accumulator gives each lane one token column and four runs of four
// consecutive output channels -> 8-byte (bf16) / 16-byte (fp32) stores of
// Y[t][n..n+3].
//
// Tiling: workgroup BT tokens x BN channels, waves arranged WT x WN, 128 k
// (64 bytes of codes per row) per stage, double-buffered LDS rows padded to
// 80 bytes (16-byte fragment reads of eight consecutive rows hit all 32
// banks), next stage prefetched into registers during the MFMAs.  Tiles are
// numbered so that each XCD (workgroup id mod 8) works on a compact block of
// the output, and inside that in groups of eight token tiles, for L2 reuse.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rq_internal.h"

namespace rq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kStageBytes = 64;  // bytes of packed codes per row per stage (128 k)

struct W4A4Args {
    const uint8_t *A;      // activation codes [T][lda]
    const uint8_t *B;      // weight codes [N][ldb]
    const float *sa;       // [T]
    const float *sw;       // [N]
    const uint16_t *top;   // bf16 [T][r] or null
    const float *bias;     // [N] or null
    void *Y;               // [T][N]
    int64_t T;
    int N;
    int lda;               // bytes per activation row (Kq / 2)
    int ldb;               // bytes per weight row (K / 2)
    int koff;              // byte offset of the quantized part in a weight row (r / 2)
    int r;                 // low-rank width (multiple of 32) or 0
    int ydt;               // rq_dtype
    int tiles_t, tiles_n;
    float post;            // 1 / b_div
};

// Workgroup barrier ordering LDS only: waits for this wave's LDS traffic,
// not for global loads in flight (the next stages' prefetch).
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ inline v4i widen(uint32_t w0, uint32_t w1) {
    const uint32_t M = 0xF0F0F0F0u;
    v4i r;
    r[0] = (int)((w0 << 4) & M);
    r[1] = (int)(w0 & M);
    r[2] = (int)((w1 << 4) & M);
    r[3] = (int)(w1 & M);
    return r;
}

__device__ inline uint32_t bf16_rne_bits(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;   // finite x
}

template <int BT_, int BN_, int WT_, int WN_, int NBUF_, int OCC_ = 2>
struct Cfg {
    static constexpr int OCC = OCC_;          // workgroups per CU the register budget is sized for
    static constexpr int BT = BT_, BN = BN_, WT = WT_, WN = WN_;
    static constexpr int NBUF = NBUF_;        // LDS stage buffers (prefetch distance NBUF - 1)
    static constexpr int NW = WT * WN;
    static constexpr int NTH = 64 * NW;
    static constexpr int FT = BT / WT / 32;   // token fragments per wave
    static constexpr int FN = BN / WN / 32;   // channel fragments per wave
    static constexpr int ROWS = BT + BN;      // token rows, then weight rows
    static constexpr int LDS_STAGE = ROWS * kStageBytes;
    static constexpr int NQ = ROWS / 16;      // 1 KB direct-to-LDS loads per stage
    static constexpr int IPW = NQ / NW;       // ... issued by each wave
    static constexpr int OUT_STRIDE = BN * 2 + 16;            // bytes per staged bf16 output row
    static constexpr int LDS_BYTES = NBUF * LDS_STAGE > BT * OUT_STRIDE ? NBUF * LDS_STAGE : BT * OUT_STRIDE;
    static_assert(BT % (32 * WT) == 0 && BN % (32 * WN) == 0, "tile shape");
    static_assert(IPW * NW == NQ, "load split");
};

// LDS rows hold 64 bytes of packed nibbles; 16-byte chunk c of row r sits at
// c ^ ((r >> 1) & 3), which keeps the 16-byte accesses of eight consecutive
// lanes on distinct bank groups.
__device__ inline int row_slot(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4); }

// One direct-to-LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's bytes land at LDS offset lds_addr + 16 l.  Written as inline asm so that
// the compiler does not see an LDS store it cannot tell apart from the
// fragment reads -- it would otherwise wait for every load in flight (the
// prefetched stages too) before each read.  Completion is tracked by hand
// with s_waitcnt vmcnt.  M0 holds the LDS address (saved and restored; one
// wait state between the M0 write and the load); the load has no VGPR result.
__device__ inline void dma16(const void *gptr, uint32_t lds_addr) {
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

// Source of K-tail chunks: sixteen zero bytes in global memory, so that the
// direct-to-LDS loads need no branch.
__device__ __attribute__((aligned(16))) uint8_t g_zero16[16];

// Tile id for workgroup `bid`: contiguous id ranges per XCD, then grouped
// ordering (GM token tiles x all channel tiles per group).
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

template <class C, bool HAS_LR, bool TAIL>
__global__ void __launch_bounds__(C::NTH, C::OCC)
gemm_w4a4_kernel(W4A4Args a) {
    // the accumulator holds 256 acc (nibbles widened to 16 q)
    constexpr int kAccShift = 8;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wt = wave / C::WN, wn = wave % C::WN;
    const int li = lane & 31, lg = lane >> 5;
    int tile_t, tile_n;
    tile_of(blockIdx.x, gridDim.x, a.tiles_t, a.tiles_n, tile_t, tile_n);
    const int64_t t0 = (int64_t)tile_t * C::BT;
    const int n0 = tile_n * C::BN;

    // Loads: every stage is NQ direct-to-LDS instructions of 1 KB (16 rows x
    // 64 bytes); lane l of instruction q fills physical chunk l & 3 of row
    // 16 q + l / 4, i.e. logical chunk (l & 3) ^ ((row >> 1) & 3).
    const uint8_t *gsrc[C::IPW];
    int col[C::IPW];
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) {
        const int q = wave * C::IPW + i;
        const int row = 16 * q + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 1) & 3);
        col[i] = 16 * ch;
        if (row < C::BT) {
            int64_t t = t0 + row;
            if (t >= a.T) t = a.T - 1;
            gsrc[i] = a.A + t * a.lda + col[i];
        } else {
            int n = n0 + row - C::BT;
            if (n >= a.N) n = a.N - 1;
            gsrc[i] = a.B + (int64_t)n * a.ldb + a.koff + col[i];
        }
    }
    const int nstage = (a.lda + kStageBytes - 1) / kStageBytes;
    // LDS byte offset of the buffer (the low half of its flat address), wave-uniform
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    auto issue = [&](int s, int buf) {
        const int kb = s * kStageBytes;
#pragma unroll
        for (int i = 0; i < C::IPW; ++i) {
            const uint8_t *p = gsrc[i] + kb;
            if (TAIL && kb + col[i] >= a.lda) p = g_zero16;
            dma16(p, __builtin_amdgcn_readfirstlane(lds_base + buf * C::LDS_STAGE + (wave * C::IPW + i) * 1024));
        }
    };
    // s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
    auto wait_vm = [](auto nc) {
        constexpr int n = decltype(nc)::value;
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
    };

    v16i acc[C::FN][C::FT];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    // NBUF LDS buffers: stage s is multiplied while stages s + 1 .. s + D
    // (D = NBUF - 1) are in flight; before the barrier that ends step s only
    // stage s + 1 must have landed, i.e. at most (pending - 1) stages of IPW
    // loads each may remain outstanding
    constexpr int D = C::NBUF - 1;
    auto wait_pending = [&](int pending) {
        // pending: stages in flight after stage s + 1 (0 .. D - 1)
        if constexpr (D >= 4) if (pending >= 3) { wait_vm(std::integral_constant<int, 3 * C::IPW>()); return; }
        if constexpr (D >= 3) if (pending == 2) { wait_vm(std::integral_constant<int, 2 * C::IPW>()); return; }
        if constexpr (D >= 2) if (pending == 1) { wait_vm(std::integral_constant<int, C::IPW>()); return; }
        wait_vm(std::integral_constant<int, 0>());
    };
    for (int p = 0; p < D && p < nstage; ++p) issue(p, p);
    wait_pending((nstage < D ? nstage : D) - 1);
    lds_barrier();
    const int rT0 = wt * C::FT * 32 + li;
    const int rN0 = C::BT + wn * C::FN * 32 + li;
    int toff[2], noff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        toff[h] = row_slot(rT0, 2 * lg + h);
        noff[h] = row_slot(rN0, 2 * lg + h);
    }
    int buf = 0;
    for (int s = 0; s < nstage; ++s) {
        if (s + D < nstage) issue(s + D, buf == 0 ? D : buf - 1);
        const uint8_t *L = lds + buf * C::LDS_STAGE;
        // fragments of both half-stages are read up front so the second
        // half's LDS latency hides under the first half's MFMAs
        uint4 fn_[2][C::FN], ft_[2][C::FT];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
                fn_[half][i] = *reinterpret_cast<const uint4 *>(L + noff[half] + i * 32 * 64);
#pragma unroll
            for (int j = 0; j < C::FT; ++j)
                ft_[half][j] = *reinterpret_cast<const uint4 *>(L + toff[half] + j * 32 * 64);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                v4i xn[C::FN], xt[C::FT];
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
                    xn[i] = k ? widen(fn_[half][i].z, fn_[half][i].w) : widen(fn_[half][i].x, fn_[half][i].y);
#pragma unroll
                for (int j = 0; j < C::FT; ++j)
                    xt[j] = k ? widen(ft_[half][j].z, ft_[half][j].w) : widen(ft_[half][j].x, ft_[half][j].y);
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xn[i], xt[j], acc[i][j], 0, 0, 0);
            }
        }
        // stage s + 1 has landed; stages s + 2 .. may still be in flight
        {
            const int last = (s + D < nstage ? s + D : nstage - 1);   // newest stage issued
            wait_pending(last - (s + 1) > 0 ? last - (s + 1) : 0);
        }
        lds_barrier();
        buf = buf == D ? 0 : buf + 1;
    }

    // low-rank term (DENSE weights): lr[n][t] = sum_{j < r} qw[n][j] * bf16(top[t][j])
    constexpr bool has_lr = HAS_LR;
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
                const uint32_t w = *reinterpret_cast<const uint32_t *>(a.B + (int64_t)n * a.ldb +
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
    // in LDS (free after the last barrier) and written back as 256-byte row
    // segments -- the accumulator layout alone would give every store
    // instruction 32 separate 16-byte pieces in 32 different rows.
    constexpr int kOutStride = C::OUT_STRIDE;
    if constexpr (!HAS_LR) {
        if (a.ydt == RQ_BF16 && t0 + C::BT <= a.T && n0 + C::BN <= a.N && (a.N % 8) == 0 &&
            a.bias == nullptr) {
#pragma unroll
            for (int j = 0; j < C::FT; ++j) {
                const int tl = wt * C::FT * 32 + j * 32 + li;
                const float sat = a.sa[t0 + tl] * a.post;
#pragma unroll
                for (int i = 0; i < C::FN; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg;
                        const float4 sw4 = *reinterpret_cast<const float4 *>(a.sw + n0 + nl);
                        const float y0 = (float)(acc[i][j][4 * q + 0] >> kAccShift) * (sat * sw4.x);
                        const float y1 = (float)(acc[i][j][4 * q + 1] >> kAccShift) * (sat * sw4.y);
                        const float y2 = (float)(acc[i][j][4 * q + 2] >> kAccShift) * (sat * sw4.z);
                        const float y3 = (float)(acc[i][j][4 * q + 3] >> kAccShift) * (sat * sw4.w);
                        *reinterpret_cast<uint2 *>(lds + tl * kOutStride + 2 * nl) =
                            make_uint2(bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16),
                                       bf16_rne_bits(y2) | (bf16_rne_bits(y3) << 16));
                    }
                }
            }
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
    const bool vec_ok = (a.N % 4) == 0;
#pragma unroll
    for (int j = 0; j < C::FT; ++j) {
        const int64_t t = t0 + wt * C::FT * 32 + j * 32 + li;
        if (t >= a.T) continue;
        const float sat = a.sa[t];
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nb = n0 + wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg;
                if (nb >= a.N) continue;
                const int64_t o = t * a.N + nb;
                int32_t iv[4];
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    iv[e] = acc[i][j][4 * q + e] >> kAccShift;   // nibbles: the MFMA returned 256 acc
                    const int n = nb + e < a.N ? nb + e : a.N - 1;
                    const float swn = a.sw[n];
                    const float bn = a.bias ? a.bias[n] : 0.0f;
                    if constexpr (has_lr)
                        y[e] = swn * (lr[i][j][4 * q + e] + sat * (float)iv[e]) + bn;
                    else
                        y[e] = ((float)iv[e] * a.post) * (sat * swn) + bn;
                }
                if (vec_ok) {
                    if (a.ydt == RQ_I32) {
                        *reinterpret_cast<int4 *>(static_cast<int32_t *>(a.Y) + o) =
                            make_int4(iv[0], iv[1], iv[2], iv[3]);
                    } else if (a.ydt == RQ_F32) {
                        *reinterpret_cast<float4 *>(static_cast<float *>(a.Y) + o) =
                            make_float4(y[0], y[1], y[2], y[3]);
                    } else {
                        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.Y) + o) =
                            make_uint2(bf16_rne_bits(y[0]) | (bf16_rne_bits(y[1]) << 16),
                                       bf16_rne_bits(y[2]) | (bf16_rne_bits(y[3]) << 16));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (nb + e >= a.N) break;
                        if (a.ydt == RQ_I32)
                            static_cast<int32_t *>(a.Y)[o + e] = iv[e];
                        else if (a.ydt == RQ_F32)
                            static_cast<float *>(a.Y)[o + e] = y[e];
                        else
                            static_cast<uint16_t *>(a.Y)[o + e] = (uint16_t)bf16_rne_bits(y[e]);
                    }
                }
            }
        }
    }
}

template <class C, bool HAS_LR>
hipError_t launch_cfg(W4A4Args a, hipStream_t s) {
    a.tiles_t = (int)((a.T + C::BT - 1) / C::BT);
    a.tiles_n = (a.N + C::BN - 1) / C::BN;
    const int nblk = a.tiles_t * a.tiles_n;
    if (a.lda % kStageBytes)
        hipLaunchKernelGGL((gemm_w4a4_kernel<C, HAS_LR, true>), dim3(nblk), dim3(C::NTH), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_w4a4_kernel<C, HAS_LR, false>), dim3(nblk), dim3(C::NTH), 0, s, a);
    return hipGetLastError();
}

// Two workgroups per CU (2 waves per SIMD): one workgroup's barrier waits and
// epilogue overlap the other's MFMAs.  (A 256 x 256 tile with one 8-wave
// workgroup per CU stages fewer bytes per MFMA but measured slower.)
using CfgBig = Cfg<256, 128, 4, 1, 3>;    // 4 waves of 64 x 128, two workgroups per CU
using CfgMid = Cfg<128, 128, 2, 2, 3>;    // 4 waves of 64 x 64

}  // namespace

int launch_gemm_w4a4(const uint8_t *codes, const float *scale, const uint16_t *top, int64_t T,
                     const rq_weight_header *hdr, const void *blob, const float *bias, void *Y,
                     int y_dtype, void *stream) {
    W4A4Args a;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
    if (hdr->a_bits != 4) return (int)hipErrorInvalidValue;   // 8-bit activations: rq_gemm_i8.hip
    a.A = codes;
    a.B = base + hdr->codes_offset;
    a.sa = scale;
    a.sw = reinterpret_cast<const float *>(base + hdr->scale_offset);
    a.top = top;
    a.bias = bias;
    a.Y = Y;
    a.T = T;
    a.N = hdr->N;
    a.r = hdr->r;
    a.lda = (hdr->K - hdr->r) / 2;
    a.ldb = hdr->row_bytes;
    a.koff = hdr->r / 2;
    a.ydt = y_dtype;
    a.post = 1.0f / (float)hdr->b_div;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the low-rank term needs registers for its own accumulators: mid tile
    if (a.r > 0) return (int)launch_cfg<CfgMid, true>(a, s);
    if (T >= 256) return (int)launch_cfg<CfgBig, false>(a, s);
    return (int)launch_cfg<CfgMid, false>(a, s);
}

}  // namespace rq

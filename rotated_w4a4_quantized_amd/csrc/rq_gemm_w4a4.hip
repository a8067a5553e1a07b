// rq_gemm_w4a4.hip -- W4A4 GEMM with the per-token x per-channel rescale,
// on gfx950 int8 MFMA.
//
// Math ("TR-DQ" section 3.1: Y = X W with per-token activation and
// per-channel weight scales):
//   acc[t][n] = sum_{k < Kq} qa[t][k] qw[n][koff + k]        (exact)
//   RPBH:  Y = s_a[t] s_w[n] acc / b
//   DENSE: Y = s_w[n] (lr[t][n] + s_a[t] acc),  lr = sum_{j<r} bf16(u)[t][j] qw[n][j]
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

#include "rq_internal.h"

namespace rq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kStageBytes = 64;  // bytes of packed codes per row per stage (128 k)
constexpr int kRowStride = 80;   // padded LDS row stride

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
    int koff;              // byte offset of the INT4 part in a weight row (r / 2)
    int r;                 // low-rank width (multiple of 32) or 0
    int ydt;               // rq_dtype
    int tiles_t, tiles_n;
    float post;            // 1 / (256 * b_div)
    float post_lr;         // 1 / 256
};

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

template <int BT_, int BN_, int WT_, int WN_>
struct Cfg {
    static constexpr int BT = BT_, BN = BN_, WT = WT_, WN = WN_;
    static constexpr int NW = WT * WN;
    static constexpr int NTH = 64 * NW;
    static constexpr int FT = BT / WT / 32;   // token fragments per wave
    static constexpr int FN = BN / WN / 32;   // channel fragments per wave
    static constexpr int ROWS = BT + BN;
    static constexpr int CHUNKS = ROWS * (kStageBytes / 16);
    static constexpr int CPT = (CHUNKS + NTH - 1) / NTH;
    static constexpr int LDS_STAGE = ROWS * kRowStride;
    static_assert(BT % (32 * WT) == 0 && BN % (32 * WN) == 0, "tile shape");
};

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

template <class C, bool HAS_LR>
__global__ void __launch_bounds__(C::NTH, 2)
gemm_w4a4_kernel(W4A4Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::LDS_STAGE];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wt = wave / C::WN, wn = wave % C::WN;
    const int li = lane & 31, lg = lane >> 5;
    int tile_t, tile_n;
    tile_of(blockIdx.x, gridDim.x, a.tiles_t, a.tiles_n, tile_t, tile_n);
    const int64_t t0 = (int64_t)tile_t * C::BT;
    const int n0 = tile_n * C::BN;

    // global source of every 16-byte chunk this thread stages
    const uint8_t *src[C::CPT];
    int dst[C::CPT];
    bool live[C::CPT];
#pragma unroll
    for (int h = 0; h < C::CPT; ++h) {
        const int c = tid + C::NTH * h;
        live[h] = c < C::CHUNKS;
        const int row = c >> 2, col = (c & 3) * 16;
        dst[h] = row * kRowStride + col;
        if (row < C::BT) {
            int64_t t = t0 + row;
            if (t >= a.T) t = a.T - 1;
            src[h] = a.A + t * a.lda + col;
        } else {
            int n = n0 + row - C::BT;
            if (n >= a.N) n = a.N - 1;
            src[h] = a.B + (int64_t)n * a.ldb + a.koff + col;
        }
    }
    const int nstage = (a.lda + kStageBytes - 1) / kStageBytes;
    uint4 pre[C::CPT];
    auto fetch = [&](int s) {
        const int kb = s * kStageBytes;
#pragma unroll
        for (int h = 0; h < C::CPT; ++h) {
            const int col = (dst[h] % kRowStride);
            if (live[h] && kb + col < a.lda)
                pre[h] = *reinterpret_cast<const uint4 *>(src[h] + kb);
            else
                pre[h] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int h = 0; h < C::CPT; ++h)
            if (live[h]) *reinterpret_cast<uint4 *>(lds + buf * C::LDS_STAGE + dst[h]) = pre[h];
    };

    v16i acc[C::FN][C::FT];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    fetch(0);
    stash(0);
    __syncthreads();
    // LDS row offsets of this lane's fragments (token rows first, then channels)
    const int rowT = (wt * C::FT * 32 + li) * kRowStride + 32 * lg;
    const int rowN = (C::BT + wn * C::FN * 32 + li) * kRowStride + 32 * lg;
    for (int s = 0; s < nstage; ++s) {
        const int buf = s & 1;
        if (s + 1 < nstage) fetch(s + 1);
        const uint8_t *L = lds + buf * C::LDS_STAGE;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint4 fn_[C::FN], ft_[C::FT];
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
                fn_[i] = *reinterpret_cast<const uint4 *>(L + rowN + i * 32 * kRowStride + 16 * half);
#pragma unroll
            for (int j = 0; j < C::FT; ++j)
                ft_[j] = *reinterpret_cast<const uint4 *>(L + rowT + j * 32 * kRowStride + 16 * half);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v4i xn[C::FN], xt[C::FT];
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
                    xn[i] = ks ? widen(fn_[i].z, fn_[i].w) : widen(fn_[i].x, fn_[i].y);
#pragma unroll
                for (int j = 0; j < C::FT; ++j)
                    xt[j] = ks ? widen(ft_[j].z, ft_[j].w) : widen(ft_[j].x, ft_[j].y);
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xn[i], xt[j], acc[i][j], 0, 0, 0);
            }
        }
        if (s + 1 < nstage) stash(buf ^ 1);
        __syncthreads();
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

    // epilogue: lane owns token t = ... + li and channels n = ... + 8 q + 4 lg + (0..3)
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
                    iv[e] = acc[i][j][4 * q + e];
                    const int n = nb + e < a.N ? nb + e : a.N - 1;
                    const float swn = a.sw[n];
                    const float bn = a.bias ? a.bias[n] : 0.0f;
                    if constexpr (has_lr)
                        y[e] = swn * (lr[i][j][4 * q + e] + sat * ((float)iv[e] * a.post_lr)) + bn;
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
    hipLaunchKernelGGL((gemm_w4a4_kernel<C, HAS_LR>), dim3(nblk), dim3(C::NTH), 0, s, a);
    return hipGetLastError();
}

using CfgBig = Cfg<256, 128, 4, 1>;    // 256 tokens x 128 channels, waves 4 x 1 (64 x 128 each)
using CfgMid = Cfg<128, 128, 2, 2>;    // 128 x 128, waves 2 x 2 (64 x 64 each)

}  // namespace

int launch_gemm_w4a4(const uint8_t *codes, const float *scale, const uint16_t *top, int64_t T,
                     const rq_weight_header *hdr, const void *blob, const float *bias, void *Y,
                     int y_dtype, void *stream) {
    W4A4Args a;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
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
    a.post = 1.0f / (256.0f * (float)hdr->b_div);
    a.post_lr = 1.0f / 256.0f;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the low-rank term needs registers for its own accumulators: mid tile
    if (a.r > 0) return (int)launch_cfg<CfgMid, true>(a, s);
    // 512 workgroup slots (256 CUs x 2): pick the tile that leaves the
    // smaller idle fraction in the last round of tiles
    const int64_t big = ((T + 255) / 256) * ((hdr->N + 127) / 128);
    const int64_t mid = ((T + 127) / 128) * ((hdr->N + 127) / 128);
    const double eff_big = (double)big / (double)(((big + 511) / 512) * 512);
    const double eff_mid = (double)mid / (double)(((mid + 511) / 512) * 512) * 0.92;
    if (T >= 256 && eff_big >= eff_mid) return (int)launch_cfg<CfgBig, false>(a, s);
    return (int)launch_cfg<CfgMid, false>(a, s);
}

}  // namespace rq

// rq_gemm_i8.hip -- GEMM of 8-bit activations (TR-DQ's W4A8 and W8A8
// settings) on gfx950's int8 matrix cores, with the per-token x per-channel
// rescale.
//
// Math ("TR-DQ" section 3.1: Y = X W with per-token activation and
// per-channel weight scales):
//   acc[t][n] = sum_k qa[t][k] qw[n][k]                        (exact, int32)
//   Y = s_a[t] s_w[n] acc / b
// Symmetric activation codes are int8; asymmetric ones are u in [0, 255]
// with a per-token zero point z, entered as u - 128 (the top bit flipped)
// and corrected in the epilogue by (128 - z[t]) wsum[n], so acc = sum (u - z) qw.
// Operands in the matrix core's order (v_mfma_i32_32x32x32_i8: lane l
// supplies row l % 32, bytes 16 (l / 32) .. + 15 of the 32-coordinate k-step):
// the weights are the blob's int8 copy of the codes (4- or 8-bit) laid out
// offline as [N / 32][K / 32][64 lanes][16 B], and the activations either
// rq_rotate_quant's codes_mma in the same order or the canonical row-major
// codes (then each lane's 16 bytes are one contiguous piece of its row).
// Direct-to-LDS loads (global_load_lds_dwordx4) copy one fragment, 1 KB, per
// instruction into LDS slots [fragment][k-step][lane][16 B]; every fragment
// read is one conflict-free ds_read_b128 and no VALU touches an operand
// (asymmetric activations: one XOR per dword).  A copy from the fragment
// order is one contiguous KB; from the row-major codes it touches 32 rows,
// and the kernel was a third slower that way (455 against 338 us on the
// FLUX up-projection).
//
// Tiling: 256 tokens x 256 channels per workgroup on eight waves of 64 x 128
// (two token fragments x four channel fragments, 128 int32 accumulators, two
// waves per SIMD); 64 coordinates per stage (32 KB of LDS), four stage buffers:
// the copies of stage s + 3 are issued at the start of stage s, after the one
// barrier that makes stage s visible and frees the buffer of stage s - 1.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rq_gemm_util.h"
#include "rq_internal.h"

namespace rq {
namespace {

using namespace gemm;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct I8Args {
    const uint8_t *A;      // activation codes [T][K] (int8, or uint8 when asymmetric), or null
    const uint8_t *Amma;   // the same in fragment order [T/32][K/32][64][16], or null
    const uint8_t *B;      // weight codes in fragment order [N/32][K/32][64][16]
    const float *sa;       // [T]
    const float *sw;       // [N]
    const float *za;       // asymmetric: zero points [T], else null
    const int32_t *wsum;   // [N]
    const float *bias;     // [N] or null
    void *Y;               // [T][N]
    int64_t T;
    int N, K, ydt;
    float post;            // 1 / b_div
    int tiles_t, tiles_n;
};

constexpr int BT = 256, BN = 256, WT = 4, WN = 2;
constexpr int NW = WT * WN, NTH = 64 * NW;
constexpr int FT = BT / WT / 32;   // token fragments per wave (2)
constexpr int FN = BN / WN / 32;   // channel fragments per wave (4)
constexpr int KS = 64;             // k per stage
constexpr int NKS = KS / 32;       // MFMA k-steps per stage
constexpr int NBUF = 4;
constexpr int OPND = BT / 32 * NKS * 1024;   // one operand's fragments per stage (16 KB)
constexpr int STAGE = 2 * OPND;              // activations, then weights
constexpr int EPI_OFF = NBUF * STAGE;        // then s_a, s_w, wsum, z: 1 KB each
constexpr int LDS_BYTES = EPI_OFF + 4 * 1024;
constexpr int PIECES = 2 * (BT / 32) * NKS;  // 1 KB copies per stage (32)
constexpr int PPW = PIECES / NW;             // ... per wave (4)
static_assert(BT == BN && PPW * NW == PIECES, "load split");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

// sixteen zero bytes: the source of k-steps past K
__device__ __attribute__((aligned(16))) uint8_t g_zero16_i8[16];

__device__ __forceinline__ uint32_t slot(int f, int ks) { return (uint32_t)((f * NKS + ks) * 1024); }

template <bool ASYM, bool ROWMAJOR>
__global__ void __launch_bounds__(NTH, 1)
gemm_i8_kernel(I8Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave / WN, wn = wave % WN;
    const int li = lane & 31, lg = lane >> 5;
    int tile_t, tile_n;
    tile_of(blockIdx.x, gridDim.x, a.tiles_t, a.tiles_n, tile_t, tile_n);
    const int64_t t0 = (int64_t)tile_t * BT;
    const int n0 = tile_n * BN;
    const int K = a.K;
    const int nstage = (K + KS - 1) / KS;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);

    // This wave's copies: piece p = PPW wave + i; p < 16: activation fragment
    // f = p / 2, k-step p % 2; else weight fragment (p - 16) / 2.  Row tiles
    // past T (N) repeat the last one, rows of the canonical codes past T
    // repeat the last row; their outputs are never stored.
    const int atiles = (int)((a.T + 31) / 32), wtiles = (a.N + 31) / 32, nkb = K / 32;
    uint32_t voff[PPW];      // canonical activation codes: lane offset from the tile's first row
    const uint8_t *src0[PPW];   // the piece's k-step 0 (wave-uniform)
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        const int p = wave * PPW + i;
        const bool act = p < PIECES / 2;
        const int f = (act ? p : p - PIECES / 2) / NKS;
        const int ks = (act ? p : p - PIECES / 2) % NKS;
        voff[i] = lane * 16;
        if (act && ROWMAJOR) {
            int64_t t = t0 + 32 * f + li;
            if (t >= a.T) t = a.T - 1;
            voff[i] = (uint32_t)((t - t0) * K + 16 * lg);
            src0[i] = a.A + t0 * K + 32 * ks;
        } else {
            int tile = (act ? (int)(t0 / 32) : n0 / 32) + f;
            const int ntile = act ? atiles : wtiles;
            if (tile >= ntile) tile = ntile - 1;
            src0[i] = (act ? a.Amma : a.B) + ((int64_t)tile * nkb + ks) * 1024;
        }
    }
    auto issue = [&](int s, int buf) {
#pragma unroll
        for (int i = 0; i < PPW; ++i) {
            const int p = wave * PPW + i;
            const bool act = p < PIECES / 2;
            const int q = act ? p : p - PIECES / 2;
            const int f = q / NKS, ks = q % NKS;
            const uint32_t dst = lds_base + buf * STAGE + (act ? 0 : OPND) + slot(f, ks);
            const bool in = s * KS + 32 * ks < K;   // wave-uniform
            // k-step s NKS + ks: 32 bytes further in a row, one KB further in a tile
            const int64_t step = (act && ROWMAJOR) ? (int64_t)s * KS : (int64_t)s * NKS * 1024;
            dma16(in ? src0[i] + step : g_zero16_i8, in ? voff[i] : 0u, dst);
        }
    };

    // Full bf16 tiles take the staged epilogue; its per-token and per-channel
    // arrays are copied to LDS ahead of the first stages (the first wait
    // covers them).
    const bool fast = a.ydt == RQ_BF16 && t0 + BT <= a.T && n0 + BN <= a.N && (a.N % 8) == 0 &&
                      a.bias == nullptr;
    const bool za_lds = ASYM && (reinterpret_cast<uintptr_t>(a.za) & 15) == 0;
    if (fast && (wave < 3 || (wave == 3 && za_lds))) {
        const void *src = wave == 0   ? static_cast<const void *>(a.sa + t0)
                          : wave == 1 ? static_cast<const void *>(a.sw + n0)
                          : wave == 2 ? static_cast<const void *>(a.wsum + n0)
                                      : static_cast<const void *>(a.za + t0);
        dma16(src, lane * 16, lds_base + EPI_OFF + wave * 1024);
    }

    v16i acc[FN][FT];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    const uint8_t *LA = lds + lane * 16;
    const uint8_t *LW = lds + OPND + lane * 16;
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p)
        if (p < nstage) issue(p, p);

    // One stage: wait until this wave's copies of stage s landed (those of
    // s + 1 and s + 2 may be in flight: WAIT copies), barrier (every wave's
    // landed; every read of stage s - 1 done), copies of stage s + 3 into
    // the buffer of stage s - 1 (PF), then both k-steps.
    auto stage = [&](int s, auto wait_c, auto pf_c) {
        constexpr int WAIT = decltype(wait_c)::value;
        constexpr bool PF = decltype(pf_c)::value;
        wait_vm<WAIT>();
        lds_barrier();
        if constexpr (PF) issue(s + NBUF - 1, (s + NBUF - 1) % NBUF);
        const int buf = s % NBUF;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            v4i tf[FT], wf[FN];
#pragma unroll
            for (int j = 0; j < FT; ++j) {
                tf[j] = *reinterpret_cast<const v4i *>(LA + buf * STAGE + slot(wt * FT + j, ks));
                if constexpr (ASYM) tf[j] ^= (int)0x80808080u;
            }
#pragma unroll
            for (int i = 0; i < FN; ++i)
                wf[i] = *reinterpret_cast<const v4i *>(LW + buf * STAGE + slot(wn * FN + i, ks));
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[i], tf[j], acc[i][j], 0, 0, 0);
        }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    using W2 = std::integral_constant<int, 2 * PPW>;
    using W1 = std::integral_constant<int, PPW>;
    using W0 = std::integral_constant<int, 0>;
    int s = 0;
    for (; s + NBUF - 1 < nstage; ++s) stage(s, W2{}, T_{});
    // the last three stages issue no copies
    if (s + 2 < nstage) stage(s++, W2{}, F_{});
    if (s + 1 < nstage) stage(s++, W1{}, F_{});
    if (s < nstage) stage(s++, W0{}, F_{});
    lds_barrier();   // every read of the last stage done: the buffers are free

    // Epilogue: acc (+ (128 - z) wsum for asymmetric codes) -> Y.
    if (fast) {
        const float *e_sa = reinterpret_cast<const float *>(lds + EPI_OFF);
        const float *e_sw = reinterpret_cast<const float *>(lds + EPI_OFF + 1024);
        const int32_t *e_ws = reinterpret_cast<const int32_t *>(lds + EPI_OFF + 2048);
        const float *e_za = reinterpret_cast<const float *>(lds + EPI_OFF + 3072);
        uint8_t *slab = lds + wave * (64 * 256);   // this wave's 64 tokens x 128 channels
        static_for<FT>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int q = j * 32 + li;   // row in the slab
            const int tl = wt * 64 + q;
            const float sat = e_sa[tl] * a.post;
            const int zoff = ASYM ? 128 - (int)(za_lds ? e_za[tl] : a.za[t0 + tl]) : 0;
            static_for<FN>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                static_for<4>([&](auto gc) {
                    constexpr int g = decltype(gc)::value;
                    const int nl = wn * 128 + i * 32 + 8 * g + 4 * lg;
                    const float4 w4 = *reinterpret_cast<const float4 *>(e_sw + nl);
                    float y[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        int v = acc[i][j][4 * g + c];
                        if constexpr (ASYM) v += zoff * e_ws[nl + c];
                        const float swc = c == 0 ? w4.x : c == 1 ? w4.y : c == 2 ? w4.z : w4.w;
                        y[c] = (float)v * (sat * swc);
                    }
                    const int chunk = 4 * i + g;
                    *reinterpret_cast<uint2 *>(slab + q * 256 + ((chunk ^ (q & 15)) * 16) + 8 * lg) =
                        make_uint2(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]));
                });
            });
        });
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int lr = lane >> 4, lc = lane & 15;
        uint16_t *dst = static_cast<uint16_t *>(a.Y) + (t0 + wt * 64 + lr) * a.N + n0 + wn * 128 + 8 * lc;
#pragma unroll 4
        for (int q0 = 0; q0 < 64; q0 += 4) {
            const int q = q0 + lr;
            const uint4 v = *reinterpret_cast<const uint4 *>(slab + q * 256 + ((lc ^ (q & 15)) * 16));
            *reinterpret_cast<uint4 *>(dst + (int64_t)q0 * a.N) = v;
        }
        return;
    }
    static_for<FT>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int64_t t = t0 + wt * 64 + j * 32 + li;
        if (t >= a.T) return;
        const float sat = a.sa[t] * a.post;
        const int zoff = ASYM ? 128 - (int)a.za[t] : 0;
        static_for<FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                const int n = n0 + wn * 128 + i * 32 + 8 * g + 4 * lg;
                int32_t iv[4];
                float y[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int nc = n + c < a.N ? n + c : a.N - 1;
                    int v = acc[i][j][4 * g + c];
                    if constexpr (ASYM) v += zoff * a.wsum[nc];
                    iv[c] = v;
                    y[c] = (float)v * (sat * a.sw[nc]) + (a.bias ? a.bias[nc] : 0.0f);
                }
                const int64_t o = t * a.N + n;
                if (n + 3 < a.N && (a.N % 4) == 0) {
                    if (a.ydt == RQ_I32)
                        *reinterpret_cast<int4 *>(static_cast<int32_t *>(a.Y) + o) = make_int4(iv[0], iv[1], iv[2], iv[3]);
                    else if (a.ydt == RQ_F32)
                        *reinterpret_cast<float4 *>(static_cast<float *>(a.Y) + o) = make_float4(y[0], y[1], y[2], y[3]);
                    else
                        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.Y) + o) =
                            make_uint2(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]));
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (n + c >= a.N) break;
                        if (a.ydt == RQ_I32)
                            static_cast<int32_t *>(a.Y)[o + c] = iv[c];
                        else if (a.ydt == RQ_F32)
                            static_cast<float *>(a.Y)[o + c] = y[c];
                        else
                            static_cast<uint16_t *>(a.Y)[o + c] = (uint16_t)(bf16x2_rne(y[c], 0.0f) & 0xFFFFu);
                    }
                }
            });
        });
    });
}

}  // namespace

int launch_gemm_i8(const uint8_t *codes, const uint8_t *codes_mma, const float *scale,
                   const float *zero, int64_t T, const rq_weight_header *hdr, const void *blob,
                   const float *bias, void *Y, int y_dtype, void *stream) {
    I8Args a;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
    a.A = codes;
    a.Amma = codes_mma;
    a.B = base + hdr->i8_offset;
    a.sa = scale;
    a.sw = reinterpret_cast<const float *>(base + hdr->scale_offset);
    a.za = zero;
    a.wsum = reinterpret_cast<const int32_t *>(base + hdr->wsum_offset);
    a.bias = bias;
    a.Y = Y;
    a.T = T;
    a.N = hdr->N;
    a.K = hdr->K;
    a.ydt = y_dtype;
    a.post = 1.0f / (float)hdr->b_div;
    a.tiles_t = (int)((T + BT - 1) / BT);
    a.tiles_n = (hdr->N + BN - 1) / BN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)(a.tiles_t * a.tiles_n));
    if (codes_mma) {
        if (zero) hipLaunchKernelGGL((gemm_i8_kernel<true, false>), grid, dim3(NTH), 0, s, a);
        else hipLaunchKernelGGL((gemm_i8_kernel<false, false>), grid, dim3(NTH), 0, s, a);
    } else {
        if (zero) hipLaunchKernelGGL((gemm_i8_kernel<true, true>), grid, dim3(NTH), 0, s, a);
        else hipLaunchKernelGGL((gemm_i8_kernel<false, true>), grid, dim3(NTH), 0, s, a);
    }
    return (int)hipGetLastError();
}

}  // namespace rq

// rq_gemm_codebook.hip -- codebook GEMM of the Lloyd-Max variant for gfx950.
//
// "OrbitQuant" abstract: tokens and weight rows are quantized in a
// normalized rotated basis with fixed Lloyd-Max codebooks; the output is
//   Y[t][n] = sigma[t] tau[n] / b * sum_k a_levels[ia[t][k]] w_levels[iw[n][k]]
// Every level is a bf16 value, so the products are exact in the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16) and only the fp32 accumulation rounds.
//
// Tiling: a workgroup owns 256 tokens x 256 channels on eight waves of 64
// tokens x 128 channels (two token fragments x four channel fragments, 128
// accumulators per lane, two waves per SIMD).  K advances in stages of 64.
// Operands that arrive as bf16 levels in the matrix-core fragment order
// [fragment][k-step][lane][16 bytes] -- the activations from rq_rotate_quant's
// codes_mma, the weights from the packed blob's copy -- are copied for stage
// s + 1 with direct-to-LDS loads while stage s is multiplied.  Operands given
// as packed indices are loaded into registers for stage s + 2 and decoded for
// stage s + 1 through LDS look-up tables (one entry per packed byte: two
// 4-bit activation indices -> two bf16, four 2-bit weight indices -> four
// bf16) into the same fragment order of the other LDS buffer.  Every
// fragment read is one conflict-free 1 KB ds_read_b128 and each stage needs
// one workgroup barrier.
//
// Accumulator element e of the 32x32 MFMA held by lane l: column l % 32,
// row 8 (e / 4) + 4 (l / 32) + e % 4.  The weight fragment is the A operand
// and the token fragment the B operand, so a lane owns one token and runs of
// four consecutive output channels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rq_gemm_util.h"
#include "rq_internal.h"

namespace rq {
namespace {

using namespace gemm;

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct CodebookArgs {
    const uint8_t *A;      // activation indices, 4-bit, [T][K/2]
    const uint8_t *Amma;   // or their bf16 levels in fragment order (rq_rotate_quant's codes_mma)
    const uint8_t *B;      // weight indices, w_bits, [N][ldb]
    const uint8_t *Bmma;   // or their bf16 levels in fragment order (the blob's copy)
    const float *sigma;    // [T]
    const float *tau;      // [N]
    const float *bias;     // [N] or null
    const float *a_levels; // device, inside the blob header (16)
    const float *w_levels; // device (2^w_bits)
    void *Y;
    int64_t T;
    int N, K, ldb, ydt;
    float post;            // 1 / b_div
    int tiles_t, tiles_n;
};

constexpr int BT = 256, BN = 256;       // tile: tokens x channels
constexpr int WT = 4, WN = 2;           // waves along tokens x channels
constexpr int NTH = 64 * WT * WN;
constexpr int FT = BT / WT / 32;        // token fragments per wave (2)
constexpr int FN = BN / WN / 32;        // channel fragments per wave (4)
constexpr int KS = 64;                  // k per stage
constexpr int NKS = KS / 16;            // MFMA k-steps per stage
constexpr int OPND = BT / 32 * NKS * 1024;   // one operand's fragments per stage (32 KB)
constexpr int STAGE = 2 * OPND;              // activations, then weights
constexpr int LUT_OFF = 2 * STAGE;           // two stage buffers, then the tables
constexpr int LDS_BYTES = LUT_OFF + 1024 + 2048;
static_assert(BT == BN, "one fragment layout for both operands");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

// LDS byte offset of the 16-byte slot of (fragment f, k-step ks, lane l)
__device__ __forceinline__ uint32_t frag_slot(int f, int ks, int l) {
    return (uint32_t)(((f * NKS + ks) * 64 + l) * 16);
}

template <bool W4, bool AMMA, bool BMMA>
__global__ void __launch_bounds__(NTH, 1)
gemm_cb_kernel(CodebookArgs a) {
    // index loads per load() call (activation and weight rows still packed)
    constexpr int LDN = (AMMA ? 0 : 1) + (BMMA ? 0 : 1);
    constexpr bool COPY = AMMA || BMMA;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    uint32_t *lutA = reinterpret_cast<uint32_t *>(lds + LUT_OFF);   // byte -> two bf16
    uint2 *lutB = reinterpret_cast<uint2 *>(lds + LUT_OFF + 1024);  // byte -> four (two) bf16
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave / WN, wn = wave % WN;
    const int li = lane & 31, lg = lane >> 5;
    int tile_t, tile_n;
    tile_of(blockIdx.x, gridDim.x, a.tiles_t, a.tiles_n, tile_t, tile_n);
    const int64_t t0 = (int64_t)tile_t * BT;
    const int n0 = tile_n * BN;
    const int nstage = a.K / KS;

    if (tid < 256) {
        const uint32_t lo = __float_as_uint(a.a_levels[tid & 15]) >> 16;
        const uint32_t hi = __float_as_uint(a.a_levels[tid >> 4]) >> 16;
        lutA[tid] = lo | (hi << 16);
        if constexpr (W4) {
            const uint32_t wl = __float_as_uint(a.w_levels[tid & 15]) >> 16;
            const uint32_t wh = __float_as_uint(a.w_levels[tid >> 4]) >> 16;
            lutB[tid] = make_uint2(wl | (wh << 16), 0u);
        } else {
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = __float_as_uint(a.w_levels[(tid >> (2 * e)) & 3]) >> 16;
            lutB[tid] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
    }

    // Decode work of this thread: row r = tid / 2 of the tile (tokens past
    // T and channels past N repeat the last row; their outputs are never
    // stored), coordinates 32 h .. 32 h + 31 of the stage, h = tid % 2, as
    // four 8-coordinate chunks c -> slot (row / 32, k-step 2 h + c / 2,
    // lane row % 32 + 32 (c % 2)).
    const int r = tid >> 1, h = tid & 1;
    int64_t ar = t0 + r;
    if (ar >= a.T) ar = a.T - 1;
    int br = n0 + r;
    if (br >= a.N) br = a.N - 1;
    const uint8_t *ap = a.A + ar * (a.K / 2) + 16 * h;                       // 16 bytes per stage
    const uint8_t *bp = a.B + (int64_t)br * a.ldb + (W4 ? 16 : 8) * h;       // 16 (8) bytes per stage
    uint32_t dslot[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) dslot[c] = frag_slot(r >> 5, 2 * h + (c >> 1), (r & 31) + 32 * (c & 1));

    uint4 ra = make_uint4(0u, 0u, 0u, 0u), rb = make_uint4(0u, 0u, 0u, 0u);
    auto load = [&](int s) {
        if constexpr (!AMMA) ra = *reinterpret_cast<const uint4 *>(ap + (int64_t)s * (KS / 2));
        if constexpr (BMMA) {
        } else if constexpr (W4) {
            rb = *reinterpret_cast<const uint4 *>(bp + (int64_t)s * (KS / 2));
        } else {
            const uint2 v = *reinterpret_cast<const uint2 *>(bp + (int64_t)s * (KS / 4));
            rb = make_uint4(v.x, v.y, 0u, 0u);
        }
    };
    // indices in ra / rb -> bf16 fragments of stage buffer buf
    auto decode = [&](int buf) {
        uint8_t *base = lds + buf * STAGE;
        if constexpr (!AMMA) {
            const uint32_t wa[4] = {ra.x, ra.y, ra.z, ra.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w = wa[c];
                const uint4 v = make_uint4(lutA[w & 0xFFu], lutA[(w >> 8) & 0xFFu],
                                           lutA[(w >> 16) & 0xFFu], lutA[w >> 24]);
                *reinterpret_cast<uint4 *>(base + dslot[c]) = v;
            }
        }
        if constexpr (BMMA) {
        } else if constexpr (W4) {
            const uint32_t wb[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w = wb[c];
                const uint4 v = make_uint4(lutB[w & 0xFFu].x, lutB[(w >> 8) & 0xFFu].x,
                                           lutB[(w >> 16) & 0xFFu].x, lutB[w >> 24].x);
                *reinterpret_cast<uint4 *>(base + OPND + dslot[c]) = v;
            }
        } else {
            const uint32_t wb[2] = {rb.x, rb.y};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w = wb[c >> 1] >> (16 * (c & 1));
                const uint2 p0 = lutB[w & 0xFFu], p1 = lutB[(w >> 8) & 0xFFu];
                *reinterpret_cast<uint4 *>(base + OPND + dslot[c]) = make_uint4(p0.x, p0.y, p1.x, p1.y);
            }
        }
    };

    v16f acc[FN][FT];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // AMMA: the activation fragments of stage s are copied as they are,
    // four 1 KB pieces (k-steps) per 32-token tile and stage, by direct-to-LDS
    // loads: piece q = 4 wave + i of the stage is k-step q % 4 of token tile
    // q / 4 (tiles past the last token repeat it; their outputs are never
    // stored)
    const int atiles = (int)((a.T + 31) / 32);
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    auto dma_act = [&](int s, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = wave * 4 + i;
            int tt = (int)(t0 / 32) + q / 4;
            if (tt >= atiles) tt = atiles - 1;
            const uint8_t *src = a.Amma + (((int64_t)tt * (a.K / 16) + s * NKS + (q & 3)) * 64) * 16;
            dma16(src, lane * 16, lds_base + buf * STAGE + frag_slot(q / 4, q & 3, 0));
        }
    };
    // BMMA: the weight fragments likewise, piece q of the stage is k-step
    // q % 4 of channel tile q / 4 (tiles past the last channel repeat it)
    const int btiles = (a.N + 31) / 32;
    auto dma_w = [&](int s, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = wave * 4 + i;
            int nt = n0 / 32 + q / 4;
            if (nt >= btiles) nt = btiles - 1;
            const uint8_t *src = a.Bmma + (((int64_t)nt * (a.K / 16) + s * NKS + (q & 3)) * 64) * 16;
            dma16(src, lane * 16, lds_base + buf * STAGE + OPND + frag_slot(q / 4, q & 3, 0));
        }
    };
    if constexpr (AMMA) dma_act(0, 0);
    if constexpr (BMMA) dma_w(0, 0);
    load(0);
    __syncthreads();   // tables ready
    decode(0);
    if (nstage > 1) load(1);
    if constexpr (COPY) {
        // the stage-0 copies have landed (stage 1's index loads, issued
        // after them, may still be in flight)
        if (nstage > 1) wait_vm<LDN>();
        else wait_vm<0>();
    }
    lds_barrier();

    const uint8_t *LA = lds + lane * 16;
    const uint8_t *LW = lds + OPND + lane * 16;
    // One stage: four k-steps of eight MFMAs from buffer s % 2; between them
    // the next stage's operands are copied or decoded into the other buffer
    // (every read of it finished before the previous stage's barrier) (DEC)
    // and the indices of the stage after that are fetched (LD).
    auto stage = [&](int s, auto dec_c, auto ld_c) {
        constexpr bool DEC = decltype(dec_c)::value;
        constexpr bool LD = decltype(ld_c)::value;
        const int cur = s & 1;
        const uint8_t *la = LA + cur * STAGE, *lw = LW + cur * STAGE;
        if constexpr (AMMA && DEC) dma_act(s + 1, cur ^ 1);
        if constexpr (BMMA && DEC) dma_w(s + 1, cur ^ 1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            v8bf tf[FT], wf[FN];
#pragma unroll
            for (int j = 0; j < FT; ++j)
                tf[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4 *>(la + frag_slot(wt * FT + j, ks, 0)));
#pragma unroll
            for (int i = 0; i < FN; ++i)
                wf[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4 *>(lw + frag_slot(wn * FN + i, ks, 0)));
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], tf[j], acc[i][j], 0, 0, 0);
            if constexpr (DEC) {
                if (ks == 1) decode(cur ^ 1);
            }
            if constexpr (LD) {
                if (ks == 2) load(s + 2);
            }
        }
        // the copies of stage s + 1 have landed (the index loads of stage
        // s + 2, issued after them, may still be in flight)
        if constexpr (COPY && DEC) {
            if constexpr (LD) wait_vm<LDN>();
            else wait_vm<0>();
        }
        lds_barrier();
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    for (int s = 0; s + 2 < nstage; ++s) stage(s, T_{}, T_{});
    if (nstage >= 2) stage(nstage - 2, T_{}, F_{});
    stage(nstage - 1, F_{}, F_{});

    // Epilogue.  Full bf16 tiles: each wave scales its 64 tokens x 128
    // channels into a private 16 KB slab of the stage buffers (free after the
    // last barrier), 256-byte rows whose 16-byte chunks are rotated by the
    // row (chunk c of row q at (c ^ (q % 16)) * 16), and copies the rows out
    // as whole segments.
    const bool fast = a.ydt == RQ_BF16 && t0 + BT <= a.T && n0 + BN <= a.N && (a.N % 8) == 0 &&
                      a.bias == nullptr;
    if (fast) {
        uint8_t *slab = lds + wave * (64 * 256);
        static_for<FT>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int q = j * 32 + li;   // row in the slab
            const float st = a.sigma[t0 + wt * 64 + q] * a.post;
            static_for<FN>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                static_for<4>([&](auto gc) {
                    constexpr int g = decltype(gc)::value;
                    const int nl = wn * 128 + i * 32 + 8 * g + 4 * lg;
                    const float4 t4 = *reinterpret_cast<const float4 *>(a.tau + n0 + nl);
                    const float y0 = acc[i][j][4 * g + 0] * (st * t4.x);
                    const float y1 = acc[i][j][4 * g + 1] * (st * t4.y);
                    const float y2 = acc[i][j][4 * g + 2] * (st * t4.z);
                    const float y3 = acc[i][j][4 * g + 3] * (st * t4.w);
                    const int chunk = 4 * i + g;
                    *reinterpret_cast<uint2 *>(slab + q * 256 + ((chunk ^ (q & 15)) * 16) + 8 * lg) =
                        make_uint2(bf16x2_rne(y0, y1), bf16x2_rne(y2, y3));
                });
            });
        });
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // four rows per instruction: lane l -> row l / 16, chunk l % 16
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
        const float st = a.sigma[t];
        static_for<FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                const int n = n0 + wn * 128 + i * 32 + 8 * g + 4 * lg;
                float y[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int nc = n + c < a.N ? n + c : a.N - 1;
                    const float tn = a.tau[nc] * a.post;
                    const float bn = a.bias ? a.bias[nc] : 0.0f;
                    y[c] = acc[i][j][4 * g + c] * (st * tn) + bn;
                }
                const int64_t o = t * a.N + n;
                if (n + 3 < a.N && (a.N % 4) == 0) {
                    if (a.ydt == RQ_F32)
                        *reinterpret_cast<float4 *>(static_cast<float *>(a.Y) + o) = make_float4(y[0], y[1], y[2], y[3]);
                    else
                        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.Y) + o) =
                            make_uint2(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]));
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (n + c >= a.N) break;
                        if (a.ydt == RQ_F32)
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

int launch_gemm_codebook(const uint8_t *codes, const uint8_t *codes_mma, const float *sigma, int64_t T,
                         const rq_weight_header *hdr, const void *blob, const float *bias,
                         void *Y, int y_dtype, void *stream) {
    CodebookArgs a;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
    a.A = codes;
    a.Amma = codes_mma;
    a.B = base + hdr->codes_offset;
    // the weights' bf16 fragments (blobs of 16-level weight books)
    a.Bmma = hdr->mma_offset ? base + hdr->mma_offset : nullptr;
    a.sigma = sigma;
    a.tau = reinterpret_cast<const float *>(base + hdr->scale_offset);
    a.bias = bias;
    a.a_levels = reinterpret_cast<const float *>(base + offsetof(rq_weight_header, a_levels));
    a.w_levels = reinterpret_cast<const float *>(base + offsetof(rq_weight_header, w_levels));
    a.Y = Y;
    a.T = T;
    a.N = hdr->N;
    a.K = hdr->K;
    a.ldb = hdr->row_bytes;
    a.ydt = y_dtype;
    a.post = 1.0f / (float)hdr->b_div;
    a.tiles_t = (int)((T + BT - 1) / BT);
    a.tiles_n = (hdr->N + BN - 1) / BN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)(a.tiles_t * a.tiles_n));
    const bool w4 = hdr->w_bits == 4, am = codes_mma != nullptr, bm = a.Bmma != nullptr;
    if (bm) {
        // the weights' index width no longer matters
        if (am)
            hipLaunchKernelGGL((gemm_cb_kernel<true, true, true>), grid, dim3(NTH), 0, s, a);
        else
            hipLaunchKernelGGL((gemm_cb_kernel<true, false, true>), grid, dim3(NTH), 0, s, a);
    } else if (am) {
        if (w4)
            hipLaunchKernelGGL((gemm_cb_kernel<true, true, false>), grid, dim3(NTH), 0, s, a);
        else
            hipLaunchKernelGGL((gemm_cb_kernel<false, true, false>), grid, dim3(NTH), 0, s, a);
    } else {
        if (w4)
            hipLaunchKernelGGL((gemm_cb_kernel<true, false, false>), grid, dim3(NTH), 0, s, a);
        else
            hipLaunchKernelGGL((gemm_cb_kernel<false, false, false>), grid, dim3(NTH), 0, s, a);
    }
    return (int)hipGetLastError();
}

}  // namespace rq

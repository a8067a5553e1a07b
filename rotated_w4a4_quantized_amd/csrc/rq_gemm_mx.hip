// rq_gemm_mx.hip -- the MXFP4 GEMM on gfx950's scaled FP4 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands).
//
// Math (the FP4 variant, "DiRotQ" abstract, later version; read as OCP MX
// MXFP4): activations and weights are E2M1 codes with one E8M0 scale per 32
// consecutive coordinates, and
//   Y[t][n] = 1/b * sum_c 2^(ea[t][c] + ew[n][c]) sum_{k in c} a[t][k] w[n][k]
// (b: the RPBH block -- the unnormalized block Hadamard scales dot products
// by b).  One MFMA takes 32 rows x 64 coordinates per operand: lane l holds
// row l % 32 and the 32 coordinates of half h = l / 32 as sixteen bytes (one
// 32-coordinate block, so one scale per lane), and the instruction multiplies
// each lane's elements by 2^(scale - 127) before the fp32 accumulation.  The
// per-lane scale byte of each operand comes from a VGPR, its byte chosen by
// the instruction's op_sel (k-step 0 or 1 of a 128-coordinate stage).
//
// Operand layouts (written by rq_rotate_quant and rq_pack_weights):
//   codes   [tile of 32 rows][K/32 blocks][32 rows][16 bytes]: the 1 KB of a
//           (tile, stage s, k-step ks) operand is blocks 4 s + 2 ks and
//           4 s + 2 ks + 1, lane order l = 32 h + row -- one contiguous
//           direct-to-LDS load
//   scales  [stage][tile][64 lanes][2 bytes]: byte ks of lane l is the E8M0
//           code of that lane's block in k-step ks
// Tiling as the FP6 GEMM: 256 tokens x 256 channels per workgroup, eight waves
// of 64 tokens x 128 channels (two per SIMD), 128-coordinate stages in three
// LDS buffers filled by direct-to-LDS loads, one barrier per stage.  MFMA A =
// weight rows, B = token rows, so each lane of an accumulator owns one token
// and runs of four consecutive channels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq_gemm_util.h"
#include "rq_internal.h"

namespace rq {
namespace {

using namespace gemm;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFmtFp4 = 4;   // matrix-core operand format code of E2M1

struct MxArgs {
    const uint8_t *A;      // activation codes, tiled
    const uint8_t *As;     // activation scales, tiled
    const uint8_t *B;      // weight codes, tiled
    const uint8_t *Bs;     // weight scales, tiled
    const float *bias;     // [N] or null
    void *Y;               // [T][N]
    int64_t T;
    int N;
    int nch;               // K / 32
    int S;                 // K / 128 stages
    int atiles, wtiles;    // 32-row tiles of activations / weights
    int ydt;               // rq_dtype (RQ_F32 or RQ_BF16)
    int tiles_t, tiles_n;
    float post;            // 1 / b_div
};

template <int BT_, int BN_, int WT_, int WN_>
struct MxCfg {
    static constexpr int BT = BT_, BN = BN_, WT = WT_, WN = WN_;
    static constexpr int NW = WT * WN;
    static constexpr int NTH = 64 * NW;
    static constexpr int FT = BT / WT / 32;   // token fragments per wave
    static constexpr int FN = BN / WN / 32;   // channel fragments per wave
    static constexpr int ACT_STAGE = BT / 32 * 2 * 1024;
    static constexpr int W_STAGE = BN / 32 * 2 * 1024;
    static constexpr int SC_STAGE = (BT + BN) / 32 * 128;   // both operands' scales
    static constexpr int LDS_STAGE = ACT_STAGE + W_STAGE + SC_STAGE;
    static constexpr int NA = BT / 32 * 2 / NW;   // activation loads per wave per stage
    static constexpr int NB = BN / 32 * 2 / NW;   // weight loads per wave per stage
    static constexpr int IPW = NA + NB + 1;       // + one 256-byte scale load
    // the epilogue's per-wave output slabs (64 rows of 128 bf16 + 16 pad bytes)
    // reuse the stage buffers and may run past them
    static constexpr int SLABS = NW * (BT / WT) * (BN / WN * 2 + 16);
    static constexpr int LDS_BYTES = 3 * LDS_STAGE > SLABS ? 3 * LDS_STAGE : SLABS;
    static_assert(NA * NW == BT / 32 * 2 && NB * NW == BN / 32 * 2, "load split");
    static_assert(BT == 256 && BN == 256 && NW == 8, "scale loads: 256 bytes per wave");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// one lane's two 16-byte k-step pieces of a 32-row fragment
struct Frag {
    v4i k[2];
};

__device__ __forceinline__ v8i as_op(const v4i &x) {
    return __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1);
}

template <class C>
__global__ void __launch_bounds__(C::NTH, 1)
gemm_mx_kernel(MxArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave / C::WN, wn = wave % C::WN;
    const int li = lane & 31, lg = lane >> 5;
    int tile_t, tile_n;
    tile_of(blockIdx.x, gridDim.x, a.tiles_t, a.tiles_n, tile_t, tile_n);
    const int64_t t0 = (int64_t)tile_t * C::BT;
    const int n0 = tile_n * C::BN;
    const int at0 = (int)(t0 / 32), wt0 = n0 / 32;
    const int nstage = a.S;

    // This wave's direct-to-LDS loads per stage: NA activation and NB weight
    // loads of 1 KB (load q: tile q / 2, k-step q % 2; tiles past the last
    // are clamped to it -- their outputs are never stored), then 256 bytes of
    // scales from 16 lanes: waves 0-3 the activation scales, 4-7 the weight
    // scales, lane l of wave w covering the 16 bytes of tile 2 (w % 4) + l / 8
    // at offset 16 (l % 8) (clamped per lane as above).
    const uint32_t loff = lane * 16;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    const bool sc_w = wave >= 4;
    const int sc_tile = 2 * (wave & 3) + (lane >> 3);   // 0..7 for lanes below 16
    uint32_t sc_off;
    {
        const int base_tile = sc_w ? wt0 : at0;
        const int last = (sc_w ? a.wtiles : a.atiles) - 1;
        int tile = base_tile + sc_tile;
        tile = tile > last ? last : tile;
        sc_off = (uint32_t)((tile - base_tile) * 128 + 16 * (lane & 7));
    }
    const uint8_t *sc_src = sc_w ? a.Bs : a.As;
    const int sc_tiles = sc_w ? a.wtiles : a.atiles;
    const int sc_first = sc_w ? wt0 : at0;
    const uint32_t sc_dst = C::ACT_STAGE + C::W_STAGE + (sc_w ? C::BT / 32 * 128 : 0) + 256 * (wave & 3);
    auto issue = [&](int s, int buf) {
        const uint32_t lb = lds_base + buf * C::LDS_STAGE;
#pragma unroll
        for (int i = 0; i < C::NA; ++i) {
            const int q = wave * C::NA + i;
            int tt = at0 + q / 2;
            if (tt >= a.atiles) tt = a.atiles - 1;
            dma16(a.A + ((int64_t)tt * a.nch + 4 * s + 2 * (q % 2)) * 512, loff, lb + q * 1024);
        }
#pragma unroll
        for (int i = 0; i < C::NB; ++i) {
            const int q = wave * C::NB + i;
            int nt = wt0 + q / 2;
            if (nt >= a.wtiles) nt = a.wtiles - 1;
            dma16(a.B + ((int64_t)nt * a.nch + 4 * s + 2 * (q % 2)) * 512, loff, lb + C::ACT_STAGE + q * 1024);
        }
        const uint8_t *src = sc_src + ((int64_t)s * sc_tiles + sc_first) * 128;
        if (lane < 16) dma16(src, sc_off, lb + sc_dst);
    };

    v16f acc[C::FN][C::FT];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const uint8_t *LA = lds + wt * C::FT * 2 * 1024 + lane * 16;
    const uint8_t *LW = lds + C::ACT_STAGE + wn * C::FN * 2 * 1024 + lane * 16;
    const uint8_t *LSA = lds + C::ACT_STAGE + C::W_STAGE + (wt * C::FT) * 128 + lane * 2;
    const uint8_t *LSW = lds + C::ACT_STAGE + C::W_STAGE + C::BT / 32 * 128 + (wn * C::FN) * 128 + lane * 2;
    auto rd = [](const uint8_t *p) {
        Frag f;
        f.k[0] = *reinterpret_cast<const v4i *>(p);
        f.k[1] = *reinterpret_cast<const v4i *>(p + 1024);
        return f;
    };
    auto rd_sc = [](const uint8_t *p) { return (int)*reinterpret_cast<const uint16_t *>(p); };

    struct StageRegs {
        Frag A[C::FT], W[C::FN];
        int sa[C::FT], sw[C::FN];
    };
    auto read_stage = [&](int buf, StageRegs &r) {
        const int o = buf * C::LDS_STAGE;
#pragma unroll
        for (int j = 0; j < C::FT; ++j) {
            r.A[j] = rd(LA + o + j * 2 * 1024);
            r.sa[j] = rd_sc(LSA + o + j * 128);
        }
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            r.W[i] = rd(LW + o + i * 2 * 1024);
            r.sw[i] = rd_sc(LSW + o + i * 128);
        }
    };
    // the MFMAs of k-step KS of weight fragment I against every token fragment
    auto mfma_ks = [&](auto ic, auto ksc, const StageRegs &r) {
        constexpr int i = decltype(ic)::value;
        constexpr int ks = decltype(ksc)::value;
        const v8i w = as_op(r.W[i].k[ks]);
#pragma unroll
        for (int j = 0; j < C::FT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                w, as_op(r.A[j].k[ks]), acc[i][j], kFmtFp4, kFmtFp4, ks, r.sw[i], ks, r.sa[j]);
    };

    // Three LDS buffers, stage s in buffer s % 3: the stage's MFMAs run on
    // registers read after the previous barrier; one barrier per stage (stage
    // s + 1 landed for this wave, every wave done reading buffer s % 3), then
    // the next stage's reads, then the loads of stage s + 3 into the freed
    // buffer.
    const int npre = nstage < 3 ? nstage : 3;
    for (int p = 0; p < npre; ++p) issue(p, p);
    if (npre == 3) wait_vm<2 * C::IPW>();
    else if (npre == 2) wait_vm<C::IPW>();
    else wait_vm<0>();
    lds_barrier();
    StageRegs cur;
    read_stage(0, cur);

    int b = 0;
    auto stage = [&](int s, auto pf_c, auto wait_c) {
        constexpr bool PF = decltype(pf_c)::value;
        constexpr bool WAIT_IPW = decltype(wait_c)::value;
        const int bn = b == 2 ? 0 : b + 1;
        static_for<C::FN>([&](auto ic) {
            mfma_ks(ic, std::integral_constant<int, 0>(), cur);
            mfma_ks(ic, std::integral_constant<int, 1>(), cur);
        });
        if constexpr (WAIT_IPW) wait_vm<C::IPW>();
        else wait_vm<0>();
        lds_barrier();
        read_stage(bn, cur);   // after the last stage: a stale buffer, unused
        if constexpr (PF) issue(s + 3, b);
        b = bn;
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    for (int s = 0; s + 3 < nstage; ++s) stage(s, T_{}, T_{});
    if (nstage >= 3) stage(nstage - 3, F_{}, T_{});
    if (nstage >= 2) stage(nstage - 2, F_{}, F_{});
    stage(nstage - 1, F_{}, F_{});

    // Epilogue: Y = acc / b (+ bias).  Full bf16 tiles without bias: each
    // wave stages its 64 x 128 slab in the (free) stage buffers and copies it
    // out as 256-byte row segments.
    const bool fast = a.ydt == RQ_BF16 && t0 + C::BT <= a.T && n0 + C::BN <= a.N && (a.N % 8) == 0 &&
                      a.bias == nullptr;
    if (fast) {
        constexpr int kRowBytes = C::BN / C::WN * 2;
        constexpr int kSlabStride = kRowBytes + 16;
        constexpr int kRows = C::FT * 32;
        static_assert(C::NW * kRows * kSlabStride <= C::LDS_BYTES, "slabs fit");
        // every wave's reads of the last stage completed before its final
        // barrier; the reads issued after it are stale and unused
        uint8_t *slab = lds + wave * kRows * kSlabStride;
        static_for<C::FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const int nw = i * 32 + 8 * q + 4 * lg;
#pragma unroll
                for (int j = 0; j < C::FT; ++j) {
                    const float y0 = acc[i][j][4 * q + 0] * a.post;
                    const float y1 = acc[i][j][4 * q + 1] * a.post;
                    const float y2 = acc[i][j][4 * q + 2] * a.post;
                    const float y3 = acc[i][j][4 * q + 3] * a.post;
                    *reinterpret_cast<uint2 *>(slab + (j * 32 + li) * kSlabStride + 2 * nw) =
                        make_uint2(bf16x2_rne(y0, y1), bf16x2_rne(y2, y3));
                }
            });
        });
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int kChunksPerRow = kRowBytes / 16;
        constexpr int kRowsPerInst = 64 / kChunksPerRow;
        const int lr = lane / kChunksPerRow, lc = lane % kChunksPerRow;
        const uint8_t *src = slab + lr * kSlabStride + 16 * lc;
        uint16_t *dst = static_cast<uint16_t *>(a.Y) + (t0 + wt * kRows + lr) * a.N + n0 +
                        wn * (kRowBytes / 2) + 8 * lc;
#pragma unroll 4
        for (int r = 0; r < kRows; r += kRowsPerInst)
            *reinterpret_cast<uint4 *>(dst + (int64_t)r * a.N) =
                *reinterpret_cast<const uint4 *>(src + r * kSlabStride);
        return;
    }
    // general epilogue: lane owns token t = ... + li and channels n = ... + 8 q + 4 lg + (0..3)
    static_for<C::FT>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int64_t t = t0 + wt * C::FT * 32 + j * 32 + li;
        if (t >= a.T) return;
        static_for<C::FN>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<4>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const int nb = n0 + wn * C::FN * 32 + i * 32 + 8 * q + 4 * lg;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = nb + e;
                    if (n >= a.N) continue;
                    const float y = acc[i][j][4 * q + e] * a.post + (a.bias ? a.bias[n] : 0.0f);
                    if (a.ydt == RQ_F32)
                        static_cast<float *>(a.Y)[t * a.N + n] = y;
                    else
                        static_cast<uint16_t *>(a.Y)[t * a.N + n] = (uint16_t)(bf16x2_rne(y, 0.0f) & 0xFFFFu);
                }
            });
        });
    });
}

}  // namespace

int launch_gemm_mx(const uint8_t *codes_mma, int64_t T, const rq_weight_header *hdr,
                   const void *blob, const float *bias, void *Y, int y_dtype, void *stream) {
    using C = MxCfg<256, 256, 4, 2>;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
    MxArgs a;
    a.T = T;
    a.N = hdr->N;
    a.nch = hdr->K / 32;
    a.S = hdr->K / 128;
    a.atiles = (int)((T + 31) / 32);
    a.wtiles = hdr->mma_ntiles;
    a.A = codes_mma;
    a.As = codes_mma + (int64_t)a.atiles * a.nch * 512;
    a.B = base + hdr->mma_offset;
    a.Bs = base + hdr->mxs_offset;
    a.bias = bias;
    a.Y = Y;
    a.ydt = y_dtype;
    a.post = 1.0f / (float)hdr->b_div;
    a.tiles_t = (int)((T + C::BT - 1) / C::BT);
    a.tiles_n = (a.N + C::BN - 1) / C::BN;
    hipLaunchKernelGGL((gemm_mx_kernel<C>), dim3(a.tiles_t * a.tiles_n), dim3(C::NTH), 0,
                       static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace rq

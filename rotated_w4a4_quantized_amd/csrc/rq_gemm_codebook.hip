// rq_gemm_codebook.hip -- codebook GEMM of the Lloyd-Max variant for gfx950.
//
// "OrbitQuant" abstract: tokens and weight rows are quantized in a
// normalized rotated basis with fixed Lloyd-Max codebooks; the output is
//   Y[t][n] = sigma[t] tau[n] / b * sum_k a_levels[ia[t][k]] w_levels[iw[n][k]]
// 4-bit activation and 2-bit (or 4-bit) weight level indices are decoded to
// bf16 through LDS look-up tables (one entry per packed byte), staged as bf16
// tiles, and multiplied on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq_internal.h"

namespace rq {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128;

// Output element e of a 32x32 MFMA accumulator held by lane l: column
// l % 32, row 8 * (e / 4) + 4 * (l / 32) + e % 4.  The weight fragment is the
// MFMA's A operand and the token fragment its B operand, so a lane owns one
// token and runs of four consecutive output channels.

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 (round to nearest even), one instruction
__device__ inline uint32_t bf16x2_rne(float lo, float hi) {
    const f2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}


// ---------------------------------------------------------------------------
// Codebook GEMM (W2A4 / W4A4 Lloyd-Max)
// ---------------------------------------------------------------------------
struct CodebookArgs {
    const uint8_t *A;      // activation indices, 4-bit, [T][K/2]
    const uint8_t *B;      // weight indices, w_bits, [N][ldb]
    const float *sigma;    // [T]
    const float *tau;      // [N]
    const float *bias;
    const float *a_levels; // device, inside the blob header (16)
    const float *w_levels; // device (16)
    void *Y;
    int64_t T;
    int N, K, ldb, w_bits, ydt;
    float post;            // 1 / b_div
};

constexpr int CBK = 64;                // k per stage
constexpr int CLDS = CBK * 2 + 16;     // bf16 tile row stride in bytes (padded)

__global__ void __launch_bounds__(256)
gemm_codebook_kernel(CodebookArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t As[BM * CLDS];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * CLDS];
    __shared__ uint32_t lutA[256];   // packed byte of two 4-bit indices -> two bf16
    __shared__ uint2 lutB[256];      // packed byte of four 2-bit indices -> four bf16, or
                                     // of two 4-bit indices -> two bf16 (x)
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int li = lane & 31, lg = lane >> 5;
    {
        const uint32_t lo = __float_as_uint(a.a_levels[tid & 15]) >> 16;
        const uint32_t hi = __float_as_uint(a.a_levels[tid >> 4]) >> 16;
        lutA[tid] = lo | (hi << 16);
        if (a.w_bits == 2) {
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = __float_as_uint(a.w_levels[(tid >> (2 * e)) & 3]) >> 16;
            lutB[tid] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else {
            const uint32_t wl = __float_as_uint(a.w_levels[tid & 15]) >> 16;
            const uint32_t wh = __float_as_uint(a.w_levels[tid >> 4]) >> 16;
            lutB[tid] = make_uint2(wl | (wh << 16), 0u);
        }
    }
    __syncthreads();
    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // This thread's rows of the tile (clamped past the edges; those outputs
    // are not stored): token row tid / 2 (16 bytes of indices per stage) and
    // weight row tid / 2 (8 or 16 bytes).  The next stage's indices are
    // loaded into registers before the current stage's MFMAs.
    const int row = tid >> 1;
    int64_t ar = m0 + row;
    if (ar >= a.T) ar = a.T - 1;
    int br = n0 + row;
    if (br >= a.N) br = a.N - 1;
    const uint8_t *ap = a.A + ar * (a.K / 2) + (tid & 1) * 16;
    const uint8_t *bp = a.B + (int64_t)br * a.ldb + (a.w_bits == 2 ? (tid & 1) * 8 : (tid & 1) * 16);
    uint4 ra, rb;
    auto load = [&](int k0) {
        ra = *reinterpret_cast<const uint4 *>(ap + k0 / 2);
        if (a.w_bits == 2) {
            const uint2 v = *reinterpret_cast<const uint2 *>(bp + k0 / 4);
            rb = make_uint4(v.x, v.y, 0u, 0u);
        } else {
            rb = *reinterpret_cast<const uint4 *>(bp + k0 / 2);
        }
    };
    load(0);
    for (int k0 = 0; k0 < a.K; k0 += CBK) {
        // A: 128 rows x 32 bytes; thread -> row tid / 2, 16 bytes at (tid & 1) * 16
        {
            const int cb = (tid & 1) * 16;
            const uint32_t w[4] = {ra.x, ra.y, ra.z, ra.w};
            uint32_t d[16];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int by = 0; by < 4; ++by) d[4 * q + by] = lutA[(w[q] >> (8 * by)) & 0xFFu];
            uint4 *dst = reinterpret_cast<uint4 *>(As + row * CLDS + cb * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
        }
        // B: 128 rows x 64 k
        if (a.w_bits == 2) {
            const int cb = (tid & 1) * 8;   // 8 bytes = 32 k
            const uint32_t w[2] = {rb.x, rb.y};
            uint2 d[8];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int by = 0; by < 4; ++by) d[4 * q + by] = lutB[(w[q] >> (8 * by)) & 0xFFu];
            uint4 *dst = reinterpret_cast<uint4 *>(Bs + row * CLDS + cb * 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = make_uint4(d[2 * q].x, d[2 * q].y, d[2 * q + 1].x, d[2 * q + 1].y);
        } else {
            const int cb = (tid & 1) * 16;  // 16 bytes = 32 k (4-bit weights)
            const uint32_t w[4] = {rb.x, rb.y, rb.z, rb.w};
            uint32_t d[16];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int by = 0; by < 4; ++by) d[4 * q + by] = lutB[(w[q] >> (8 * by)) & 0xFFu].x;
            uint4 *dst = reinterpret_cast<uint4 *>(Bs + row * CLDS + cb * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
        }
        if (k0 + CBK < a.K) load(k0 + CBK);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < CBK / 16; ++ks) {
            v8bf fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4 *>(
                                                     As + (wm * 64 + i * 32 + li) * CLDS + (ks * 16 + 8 * lg) * 2));
                fb[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4 *>(
                                                     Bs + (wn * 64 + i * 32 + li) * CLDS + (ks * 16 + 8 * lg) * 2));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // acc[i][j]: tokens wm 64 + 32 i + (lane % 32), channels
    // wn 64 + 32 j + 8 g + 4 (lane / 32) + c for element 4 g + c
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = m0 + wm * 64 + i * 32 + li;
        if (t >= a.T) continue;
        const float st = a.sigma[t];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 64 + j * 32 + 8 * g + 4 * lg;
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
            }
        }
    }
}

}  // namespace

int launch_gemm_codebook(const uint8_t *codes, const float *sigma, int64_t T,
                         const rq_weight_header *hdr, const void *blob, const float *bias,
                         void *Y, int y_dtype, void *stream) {
    CodebookArgs a;
    const uint8_t *base = static_cast<const uint8_t *>(blob);
    a.A = codes;
    a.B = base + hdr->codes_offset;
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
    a.w_bits = hdr->w_bits;
    a.ydt = y_dtype;
    a.post = 1.0f / (float)hdr->b_div;
    dim3 grid((hdr->N + BN - 1) / BN, (unsigned)((T + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_codebook_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace rq

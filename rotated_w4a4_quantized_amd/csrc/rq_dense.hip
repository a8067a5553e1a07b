// rq_dense.hip -- DiRotQ runtime activation path for gfx950: rotate each
// token into the dense (PCA) basis and quantize the coordinates past the
// top r to INT4, keeping the top r in bf16.
//
// "DiRotQ" abstract: activations are rotated into a calibration-derived
// orthogonal PCA basis at inference, the leading principal coefficients are
// kept at higher precision and the rest quantized to 4 bits.  Arithmetic
// (the reading this library fixes so results are reproducible): every
// rotated coordinate is one fp32 fused multiply-add chain over k ascending,
// starting from +0; quantization is symmetric INT4 with s = fl32(amax / 7),
// q = clamp(rne(fl32(u * fl32(7 / amax))), -7, 7).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rq_fp6.h"
#include "rq_internal.h"

namespace rq {
namespace {

// ---------------------------------------------------------------------------
// DENSE ("DiRotQ" abstract): u = x R as one fp32 fma chain per output over k
// ascending (register-tiled: each thread owns an 8 x 8 block of (token,
// column) outputs and walks k in order), then per-token quantization of the
// coordinates [r, K) with the top r kept in bf16.
// ---------------------------------------------------------------------------
constexpr int kDT = 128;   // tokens per tile
constexpr int kDJ = 128;   // output columns per tile
constexpr int kDK = 16;    // k per LDS stage

template <bool BF16>
__global__ void __launch_bounds__(256)
dense_rotate_kernel(const void *__restrict__ X, int64_t T, int K, const float *__restrict__ R,
                    float *__restrict__ U) {
    __shared__ float xs[kDK][kDT + 4];  // x^T tile: [k][token]
    __shared__ float rs[kDK][kDJ + 4];  // R tile:   [k][column]
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;  // 16 x 16 threads, 8 x 8 outputs each
    const int64_t t0 = (int64_t)blockIdx.y * kDT;
    const int j0 = blockIdx.x * kDJ;
    float acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += kDK) {
        // x tile: 128 tokens x 16 k; thread loads 8 values
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int li = tid + 256 * e;   // 0..2047
            const int tt = li / kDK, kk = li % kDK;
            int64_t tok = t0 + tt;
            if (tok >= T) tok = T - 1;
            float xv;
            if constexpr (BF16)
                xv = __uint_as_float((uint32_t)static_cast<const uint16_t *>(X)[tok * K + k0 + kk] << 16);
            else
                xv = static_cast<const float *>(X)[tok * K + k0 + kk];
            xs[kk][tt] = xv;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int li = tid + 256 * e;
            const int kk = li / kDJ, jj = li % kDJ;
            const int j = j0 + jj;
            rs[kk][jj] = j < K ? R[(int64_t)(k0 + kk) * K + j] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kDK; ++kk) {
            float xa[8], rb[8];
#pragma unroll
            for (int a = 0; a < 8; ++a) xa[a] = xs[kk][ty * 8 + a];
#pragma unroll
            for (int b = 0; b < 8; ++b) rb[b] = rs[kk][tx * 8 + b];
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int b = 0; b < 8; ++b) acc[a][b] = fmaf(xa[a], rb[b], acc[a][b]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const int64_t tok = t0 + ty * 8 + a;
        if (tok >= T) continue;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int j = j0 + tx * 8 + b;
            if (j < K) U[tok * K + j] = acc[a][b];
        }
    }
}

__device__ inline uint16_t f32_to_bf16_rne(float x) {
    const uint32_t b = __float_as_uint(x);
    const uint32_t lower = b & 0xFFFFu, upper = b >> 16;
    return (uint16_t)(upper + ((lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) ? 1u : 0u));
}

// One 64-lane wave per token.  Lane l quantizes the 32-coordinate chunks
// c = l, l + 64, ... of the token's Kq = K - r quantized coordinates and
// writes them as sixteen canonical nibble bytes and/or in the GEMM's FP6
// fragment layout (rq_fp6.h; signed codes, carried as q + 8).
__global__ void __launch_bounds__(256)
dense_quant_kernel(const float *__restrict__ U, int64_t T, int K, int r,
                   uint8_t *__restrict__ codes, float *__restrict__ scale,
                   uint16_t *__restrict__ top, uint8_t *__restrict__ codes_mma) {
    const int lane = threadIdx.x & 63;
    const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= T) return;
    const float *u = U + tok * K;
    float m = 0.0f;
    for (int j = r + lane; j < K; j += 64) m = fmaxf(m, fabsf(u[j]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    for (int j = lane; j < r; j += 64) top[tok * r + j] = f32_to_bf16_rne(u[j]);
    const int Kq = K - r, nch = Kq / 32, S = (Kq + 127) / 128;
    const float inv = m > 0.0f ? 7.0f / m : 0.0f;
    for (int c = lane; c < nch; c += 64) {
        const float4 *src = reinterpret_cast<const float4 *>(u + r + 32 * c);
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float4 v0 = src[2 * d], v1 = src[2 * d + 1];
            const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t b = 0;
            if (m > 0.0f) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float q = rintf(v[e] * inv);
                    q = fminf(7.0f, fmaxf(-7.0f, q));
                    b |= ((uint32_t)(int)q & 0xFu) << (4 * e);   // low nibble = even coordinate
                }
            }
            w[d] = b;
        }
        const uint4 w4 = make_uint4(w[0], w[1], w[2], w[3]);
        if (codes) *reinterpret_cast<uint4 *>(codes + tok * (int64_t)(Kq / 2) + 16 * c) = w4;
        if (codes_mma) store_chunk_mma(codes_mma, tok, S, c, w4, 0x88888888u);
    }
    if (lane == 0) scale[tok] = m > 0.0f ? m / 7.0f : 0.0f;
}

// Device scratch of the allocation-free entry point (rq_rotate_quant_noalloc):
// the fp32 rotated tokens of a DENSE call, kDenseScratchBytes at most.  One
// copy per device, held from the module's load until the process ends.  In
// host code the name is only a stand-in: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kDenseScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxScratchDevices];   // per device, null until looked up

}  // namespace

int dense_scratch(float **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxScratchDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return (int)hipSuccess;
}

int launch_dense_rotate(const void *X, int x_bf16, int64_t T, int K, const float *R, float *U,
                        void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    dim3 grid((K + kDJ - 1) / kDJ, (unsigned)((T + kDT - 1) / kDT));
    if (x_bf16)
        hipLaunchKernelGGL(dense_rotate_kernel<true>, grid, dim3(256), 0, s, X, T, K, R, U);
    else
        hipLaunchKernelGGL(dense_rotate_kernel<false>, grid, dim3(256), 0, s, X, T, K, R, U);
    return (int)hipGetLastError();
}

int launch_dense_quant(const float *U, int64_t T, int K, int r, uint8_t *codes, float *scale,
                       uint16_t *top, uint8_t *codes_mma, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(dense_quant_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, U, T,
                       K, r, codes, scale, top, codes_mma);
    return (int)hipGetLastError();
}

}  // namespace rq

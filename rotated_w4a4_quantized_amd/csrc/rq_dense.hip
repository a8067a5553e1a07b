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
// ascending (register-tiled: each thread owns an 8 x CW block of (token,
// column) outputs and walks k in order), then per-token quantization of the
// coordinates [r, K) with the top r kept in bf16.
//
// A workgroup computes 128 tokens x 16 CW columns in chunks of 16 k: the
// chunk's x tile (transposed, [k][token]) and R tile ([k][column]) sit in one
// of two LDS buffers while the next chunk's tiles are loaded into registers
// (16-byte global loads) and written to the other, so each chunk takes one
// barrier.  The column-tile width (CW = 8, 6 or 4 columns per thread) is
// chosen per shape so that the workgroups spread evenly over the CUs: every
// workgroup is resident at once and a CU holding one more than the others
// sets the time.
// ---------------------------------------------------------------------------
constexpr int kDT = 128;   // tokens per tile
constexpr int kDK = 16;    // k per LDS chunk

// an empty asm that takes and returns a row of sums: code before it must
// have produced them
template <int CW>
__device__ __forceinline__ void pin_row(float (&r)[CW]) {
    if constexpr (CW == 8)
        asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]));
    else if constexpr (CW == 6)
        asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]));
    else
        asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
}

template <bool BF16, int CW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
dense_rotate_kernel(const void *__restrict__ X, int64_t T, int K, const float *__restrict__ R,
                    float *__restrict__ U) {
    constexpr int DJ = 16 * CW;                 // columns per tile
    constexpr int XL = BF16 ? 1 : 2;            // 16-byte x loads per thread per chunk
    constexpr int RL = (kDK * DJ / 4 + 255) / 256;   // 16-byte R loads per thread per chunk
    __shared__ __attribute__((aligned(16))) float xs[2][kDK][kDT + 4];  // x^T: [k][token]
    __shared__ __attribute__((aligned(16))) float rs[2][kDK][DJ + 4];   // R:   [k][column]
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;    // 16 x 16 threads, 8 x CW outputs each
    const int64_t t0 = (int64_t)blockIdx.y * kDT;
    const int j0 = blockIdx.x * DJ;
    float acc[8][CW];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < CW; ++b) acc[a][b] = 0.0f;

    // x: load i of thread tid covers token (tid + 256 i) / Q, k-quarter
    // (tid + 256 i) % Q of the chunk (Q = 2 for bf16: 8 values per 16 bytes;
    // 4 for fp32); R: load i covers row q / (DJ / 4), columns 4 (q % (DJ / 4))
    // of the chunk, q = tid + 256 i (loads past the tile or the matrix are
    // skipped; their slots hold zeros that no output reads)
    constexpr int Q = BF16 ? 2 : 4;
    uint4 xr[XL];
    float4 rr[RL];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int q = tid + 256 * i;
            int64_t tok = t0 + q / Q;
            if (tok >= T) tok = T - 1;
            const int kq = (q % Q) * (16 / (BF16 ? 2 : 4));   // first k of this load
            const uint8_t *src = static_cast<const uint8_t *>(X) + (tok * K + k0 + kq) * (BF16 ? 2 : 4);
            xr[i] = *reinterpret_cast<const uint4 *>(src);
        }
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int q = tid + 256 * i;
            const int kk = q / (DJ / 4), jj = 4 * (q % (DJ / 4));
            rr[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (kk < kDK && j0 + jj < K)
                rr[i] = *reinterpret_cast<const float4 *>(R + (int64_t)(k0 + kk) * K + j0 + jj);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int q = tid + 256 * i;
            const int tt = q / Q;
            const int kq = (q % Q) * (16 / (BF16 ? 2 : 4));
            const uint32_t w[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
            if constexpr (BF16) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xs[buf][kq + e][tt] = __uint_as_float(e & 1 ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) xs[buf][kq + e][tt] = __uint_as_float(w[e]);
            }
        }
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int q = tid + 256 * i;
            const int kk = q / (DJ / 4), jj = 4 * (q % (DJ / 4));
            if (kk < kDK) *reinterpret_cast<float4 *>(&rs[buf][kk][jj]) = rr[i];
        }
    };

    const int nchunk = K / kDK;
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
        const int buf = c & 1;
        if (c + 1 < nchunk) load((c + 1) * kDK);   // in flight during the FMAs
        // operands of step kk + 1 are read while step kk's FMAs run (two
        // register sets; the empty asm statements, which the compiler may not
        // move memory accesses across, keep it from hoisting every read of
        // the chunk, which would cost occupancy)
        float xa[2][8], rb[2][CW];
        auto rd = [&](int kk, int p) {
#pragma unroll
            for (int a = 0; a < 8; ++a) xa[p][a] = xs[buf][kk][ty * 8 + a];
#pragma unroll
            for (int b = 0; b < CW; ++b) rb[p][b] = rs[buf][kk][tx * CW + b];
        };
        rd(0, 0);
#pragma unroll
        for (int kk = 0; kk < kDK; ++kk) {
            if (kk + 1 < kDK) rd(kk + 1, (kk + 1) & 1);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int b = 0; b < CW; ++b) acc[a][b] = fmaf(xa[kk & 1][a], rb[kk & 1][b], acc[a][b]);
            // the step's sums are due here (else the compiler sinks every FMA
            // of the chunk below its last read)
#pragma unroll
            for (int a = 0; a < 8; ++a) pin_row(acc[a]);
        }
        // the other buffer was last read before the previous barrier
        if (c + 1 < nchunk) store(buf ^ 1);
        __syncthreads();
    }
    // this thread's columns jb .. jb + CW - 1 (those below K), rows t0 + 8 ty + a
    const int jb = j0 + tx * CW;
    const bool full = jb + CW <= K;
    float *u = U + (t0 + ty * 8) * K + jb;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        if (t0 + ty * 8 + a >= T) break;
        if (full) {
            if constexpr (CW % 4 == 0) {
#pragma unroll
                for (int b = 0; b < CW; b += 4)
                    *reinterpret_cast<float4 *>(u + b) = make_float4(acc[a][b], acc[a][b + 1], acc[a][b + 2], acc[a][b + 3]);
            } else {
#pragma unroll
                for (int b = 0; b < CW; b += 2) *reinterpret_cast<float2 *>(u + b) = make_float2(acc[a][b], acc[a][b + 1]);
            }
        } else {
#pragma unroll
            for (int b = 0; b < CW; ++b)
                if (jb + b < K) u[b] = acc[a][b];
        }
        u += K;
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
    // columns per thread: the width whose workgroup count spreads most evenly
    // over the CUs (every workgroup is resident at once), ties to the wider
    const int64_t ttiles = (T + kDT - 1) / kDT;
    const int64_t cus = device_cus();
    int cw = 8;
    double best = -1.0;
    for (int c : {8, 6, 4}) {
        const int64_t n = ttiles * ((K + 16 * c - 1) / (16 * c));
        const double eff = (double)n / (double)(((n + cus - 1) / cus) * cus);
        if (eff > best + 1e-9) {
            best = eff;
            cw = c;
        }
    }
    const dim3 grid((unsigned)((K + 16 * cw - 1) / (16 * cw)), (unsigned)ttiles);
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, X, T, K, R, U); };
    if (x_bf16) {
        if (cw == 8) go(dense_rotate_kernel<true, 8>);
        else if (cw == 6) go(dense_rotate_kernel<true, 6>);
        else go(dense_rotate_kernel<true, 4>);
    } else {
        if (cw == 8) go(dense_rotate_kernel<false, 8>);
        else if (cw == 6) go(dense_rotate_kernel<false, 6>);
        else go(dense_rotate_kernel<false, 4>);
    }
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

// rq_rotate.hip -- runtime activation kernels for gfx950: rotate each token
// and quantize it to 4 bits.
//
// RPBH ("OrbitQuant" abstract; block structure "TR-DQ" Eq.(8)):
//   y[j] = sign[j] * x[perm[j]], then the unnormalized Sylvester transform of
//   every b-block with radix-2 fp32 butterflies (lo, hi) -> (lo + hi, lo - hi)
//   in ascending stage order h = 1, 2, ..., b/2.  Within one stage all
//   butterflies are independent, so any schedule that keeps the stage order
//   and computes lo + hi / lo - hi in fp32 reproduces the same bits.
//
// Work decomposition: one workgroup holds a whole token (K/16 threads, 16
// coordinates per thread); workgroups stride over tokens.  The token is
// staged in LDS (coalesced 16-byte loads), gathered through the permutation
// into registers, and the log2(b) stages run in passes of up to four stages
// on sixteen registers, exchanging through LDS between passes:
//   pass 0  : the thread holds 16 consecutive coordinates (stages 1..8)
//   pass p>0: the thread holds the coordinates whose index bits [4p, 4p+4)
//             vary (plus the lowest bits when fewer than four remain)
// Then the per-token statistic, the quantizer and the nibble pack.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq_internal.h"

namespace rq {
namespace {

constexpr int kPer = 16;  // coordinates per thread per pass

__host__ __device__ constexpr int npass(int L) { return L <= 4 ? 1 : 1 + (L - 4 + 3) / 4; }
__host__ __device__ constexpr int pass_lo(int p) { return 4 * p; }
__host__ __device__ constexpr int pass_hi(int L, int p) {
    return p == 0 ? (L < 4 ? L : 4) : (4 * p + 4 < L ? 4 * p + 4 : L);
}
// Index bit of the block-local coordinate carried by register bit k in pass p.
__host__ __device__ constexpr int vbit(int L, int p, int k) {
    return p == 0 ? k
                  : (k < 4 - (pass_hi(L, p) - pass_lo(p)) ? k
                                                           : pass_lo(p) + k - (4 - (pass_hi(L, p) - pass_lo(p))));
}
__host__ __device__ constexpr int reg_offset(int L, int p, int r) {
    return ((r & 1) << vbit(L, p, 0)) | (((r >> 1) & 1) << vbit(L, p, 1)) |
           (((r >> 2) & 1) << vbit(L, p, 2)) | (((r >> 3) & 1) << vbit(L, p, 3));
}
__host__ __device__ constexpr bool is_vbit(int L, int p, int pos) {
    return vbit(L, p, 0) == pos || vbit(L, p, 1) == pos || vbit(L, p, 2) == pos ||
           vbit(L, p, 3) == pos;
}
// Register bit that carries index bit s in pass p.
__host__ __device__ constexpr int reg_bit_of(int L, int p, int s) {
    return vbit(L, p, 0) == s ? 0 : vbit(L, p, 1) == s ? 1 : vbit(L, p, 2) == s ? 2 : 3;
}

// First coordinate (row-relative) of thread t's set in pass p; the set is
// base + reg_offset(p, r) for r = 0..15.
template <int L, int P>
__device__ inline int pass_base(int t) {
    if constexpr (P == 0) {
        return kPer * t;
    } else {
        const int c = t >> (L - 4);        // block index
        int f = t & ((1 << (L - 4)) - 1);  // the thread's fixed index bits
        int i = 0;
#pragma unroll
        for (int pos = 0; pos < L; ++pos) {
            if (is_vbit(L, P, pos)) continue;
            i |= (f & 1) << pos;
            f >>= 1;
        }
        return (c << L) + i;
    }
}

// Butterflies of pass p on the sixteen registers.
template <int L, int P>
__device__ inline void pass_stages(float (&v)[kPer]) {
#pragma unroll
    for (int s = pass_lo(P); s < pass_hi(L, P); ++s) {
        const int kb = reg_bit_of(L, P, s);
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            if (r & (1 << kb)) continue;
            const float lo = v[r], hi = v[r | (1 << kb)];
            v[r] = lo + hi;
            v[r | (1 << kb)] = lo - hi;
        }
    }
}

template <int L, int P>
__device__ inline void run_pass(float (&v)[kPer], float *us, int t) {
    if constexpr (P > 0) {
        const int prev = pass_base<L, P - 1>(t);
#pragma unroll
        for (int r = 0; r < kPer; ++r) us[prev + reg_offset(L, P - 1, r)] = v[r];
        __syncthreads();
        const int cur = pass_base<L, P>(t);
#pragma unroll
        for (int r = 0; r < kPer; ++r) v[r] = us[cur + reg_offset(L, P, r)];
    }
    pass_stages<L, P>(v);
}

template <int L>
__device__ inline void rpbh_transform(float (&v)[kPer], float *us, int t) {
    run_pass<L, 0>(v, us, t);
    if constexpr (npass(L) > 1) run_pass<L, 1>(v, us, t);
    if constexpr (npass(L) > 2) run_pass<L, 2>(v, us, t);
    static_assert(npass(L) <= 3, "block too large");
}

// Stage one token row [K] (fp32 or bf16) into LDS as fp32: thread t copies
// coordinates [16t, 16t + 16).
template <bool BF16>
__device__ inline void stage_row(const void *X, int64_t tok, int K, float *xs, int t) {
    if constexpr (BF16) {
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(X) +
                                                           tok * (int64_t)K + kPer * t);
        const uint4 a = src[0], b = src[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float4 *dst = reinterpret_cast<float4 *>(xs + kPer * t);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w0 = w[2 * q], w1 = w[2 * q + 1];
            dst[q] = make_float4(__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                                 __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u));
        }
    } else {
        const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(X) +
                                                             tok * (int64_t)K + kPer * t);
        float4 *dst = reinterpret_cast<float4 *>(xs + kPer * t);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = src[q];
    }
}

// Per-thread gather table: coordinates 16t + r read x[perm[16t + r]] with
// the sign of coordinate 16t + r.
struct Gather {
    int idx[kPer];
    uint32_t neg;
};
__device__ inline Gather load_gather(const int8_t *sign, const int32_t *perm, int t) {
    Gather g;
    g.neg = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        g.idx[r] = perm[kPer * t + r];
        g.neg |= (sign[kPer * t + r] < 0 ? 1u : 0u) << r;
    }
    return g;
}

// ---------------------------------------------------------------------------
// RPBH + symmetric INT4
// ---------------------------------------------------------------------------
template <int L, bool BF16>
__global__ void __launch_bounds__(1024)
rpbh_int4_kernel(const void *__restrict__ X, int64_t T, int K, const int8_t *__restrict__ sign,
                 const int32_t *__restrict__ perm, uint8_t *__restrict__ codes,
                 float *__restrict__ scale) {
    extern __shared__ float smem[];
    float *xs = smem;       // staged token [K]
    float *us = smem + K;   // pass exchange / final values [K]
    __shared__ unsigned red[2];
    const int t = threadIdx.x;
    const Gather g = load_gather(sign, perm, t);
    int it = 0;
    for (int64_t tok = blockIdx.x; tok < T; tok += gridDim.x, ++it) {
        if (t == 0) red[it & 1] = 0u;
        stage_row<BF16>(X, tok, K, xs, t);
        __syncthreads();
        float v[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const float x = xs[g.idx[r]];
            v[r] = ((g.neg >> r) & 1u) ? -x : x;
        }
        rpbh_transform<L>(v, us, t);
        // per-token absmax (|u| >= 0, so the fp32 bits order like the values)
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < kPer; ++r) m = fmaxf(m, fabsf(v[r]));
        atomicMax(&red[it & 1], __float_as_uint(m));
        const int fin = pass_base<L, npass(L) - 1>(t);
#pragma unroll
        for (int r = 0; r < kPer; ++r) us[fin + reg_offset(L, npass(L) - 1, r)] = v[r];
        __syncthreads();
        const float amax = __uint_as_float(red[it & 1]);
        // quantize coordinates [16t, 16t + 16): q = clamp(rne(fl32(u * inv)), -7, 7)
        uint32_t packed[2] = {0u, 0u};
        if (amax > 0.0f) {
            const float inv = 7.0f / amax;
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                float q = rintf(us[kPer * t + r] * inv);
                q = fminf(7.0f, fmaxf(-7.0f, q));
                packed[r >> 3] |= ((uint32_t)(int)q & 0xFu) << (4 * (r & 7));
            }
        }
        *reinterpret_cast<uint2 *>(codes + tok * (int64_t)(K / 2) + (kPer / 2) * t) =
            make_uint2(packed[0], packed[1]);
        if (t == 0) scale[tok] = amax > 0.0f ? amax / 7.0f : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// RPBH + Lloyd-Max codebook on the normalized token ("OrbitQuant" abstract)
//   d = |u|^2 on an exact integer grid: with E = ilogb(max|u|), every
//   u^2 * 2^(36 - 2E) is rounded to an integer (< 2^38) and the integers are
//   summed in uint64 -- exact and independent of the order.
//   g = (float)sqrt(K / d);  index = #{ thresholds < fl32(u * g) }
//   sigma = (float)sqrt(d / K)
// ---------------------------------------------------------------------------
struct Thresholds {
    float v[15];
};

template <int L, bool BF16>
__global__ void __launch_bounds__(1024)
rpbh_lloydmax_kernel(const void *__restrict__ X, int64_t T, int K,
                     const int8_t *__restrict__ sign, const int32_t *__restrict__ perm,
                     Thresholds th, int nth, uint8_t *__restrict__ codes,
                     float *__restrict__ sigma) {
    extern __shared__ float smem[];
    float *xs = smem;
    float *us = smem + K;
    __shared__ unsigned red[2];
    __shared__ unsigned long long acc[2];
    const int t = threadIdx.x;
    const Gather g = load_gather(sign, perm, t);
    int it = 0;
    for (int64_t tok = blockIdx.x; tok < T; tok += gridDim.x, ++it) {
        if (t == 0) {
            red[it & 1] = 0u;
            acc[it & 1] = 0ull;
        }
        stage_row<BF16>(X, tok, K, xs, t);
        __syncthreads();
        float v[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const float x = xs[g.idx[r]];
            v[r] = ((g.neg >> r) & 1u) ? -x : x;
        }
        rpbh_transform<L>(v, us, t);
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < kPer; ++r) m = fmaxf(m, fabsf(v[r]));
        atomicMax(&red[it & 1], __float_as_uint(m));
        __syncthreads();
        const float M = __uint_as_float(red[it & 1]);
        if (M > 0.0f) {
            const int E = ilogbf(M);
            unsigned long long s = 0;
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const double sq = (double)v[r] * (double)v[r];
                s += (unsigned long long)rint(ldexp(sq, 36 - 2 * E));
            }
            atomicAdd(&acc[it & 1], s);
        }
        const int fin = pass_base<L, npass(L) - 1>(t);
#pragma unroll
        for (int r = 0; r < kPer; ++r) us[fin + reg_offset(L, npass(L) - 1, r)] = v[r];
        __syncthreads();
        uint32_t packed[2] = {0u, 0u};
        float sg = 0.0f;
        if (M > 0.0f) {
            const int E = ilogbf(M);
            const double d = ldexp((double)acc[it & 1], 2 * E - 36);
            const float gain = (float)sqrt((double)K / d);
            sg = (float)sqrt(d / (double)K);
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const float x = us[kPer * t + r] * gain;
                uint32_t idx = 0;
                for (int i = 0; i < nth; ++i) idx += (x > th.v[i]) ? 1u : 0u;
                packed[r >> 3] |= idx << (4 * (r & 7));
            }
        }
        *reinterpret_cast<uint2 *>(codes + tok * (int64_t)(K / 2) + (kPer / 2) * t) =
            make_uint2(packed[0], packed[1]);
        if (t == 0) sigma[tok] = sg;
    }
}

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

// One 64-lane wave per token.
__global__ void __launch_bounds__(256)
dense_quant_kernel(const float *__restrict__ U, int64_t T, int K, int r,
                   uint8_t *__restrict__ codes, float *__restrict__ scale,
                   uint16_t *__restrict__ top) {
    const int lane = threadIdx.x & 63;
    const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= T) return;
    const float *u = U + tok * K;
    float m = 0.0f;
    for (int j = r + lane; j < K; j += 64) m = fmaxf(m, fabsf(u[j]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    for (int j = lane; j < r; j += 64) top[tok * r + j] = f32_to_bf16_rne(u[j]);
    const int Kq = K - r;
    uint8_t *crow = codes + tok * (int64_t)(Kq / 2);
    const float inv = m > 0.0f ? 7.0f / m : 0.0f;
    for (int p = lane; p < Kq / 2; p += 64) {
        uint32_t b = 0;
        if (m > 0.0f) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float q = rintf(u[r + 2 * p + e] * inv);
                q = fminf(7.0f, fmaxf(-7.0f, q));
                b |= ((uint32_t)(int)q & 0xFu) << (4 * e);
            }
        }
        crow[p] = (uint8_t)b;
    }
    if (lane == 0) scale[tok] = m > 0.0f ? m / 7.0f : 0.0f;
}

int grid_for_tokens(int64_t T, int threads) {
    // enough workgroups to fill 256 CUs several times over, never more than T
    int per_cu = threads <= 256 ? 8 : threads <= 512 ? 4 : 2;
    int64_t g = (int64_t)256 * per_cu;
    if (g > T) g = T;
    return (int)(g < 1 ? 1 : g);
}

template <int L, bool BF16>
hipError_t launch_int4_L(const void *X, int64_t T, int K, const int8_t *sign,
                         const int32_t *perm, uint8_t *codes, float *scale, hipStream_t s) {
    const int threads = K / kPer;
    const size_t lds = (size_t)2 * K * sizeof(float);
    auto kern = rpbh_int4_kernel<L, BF16>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid_for_tokens(T, threads)), dim3(threads), lds, s, X, T, K,
                       sign, perm, codes, scale);
    return hipGetLastError();
}

template <int L, bool BF16>
hipError_t launch_lm_L(const void *X, int64_t T, int K, const int8_t *sign, const int32_t *perm,
                       const Thresholds &th, int nth, uint8_t *codes, float *sigma,
                       hipStream_t s) {
    const int threads = K / kPer;
    const size_t lds = (size_t)2 * K * sizeof(float);
    auto kern = rpbh_lloydmax_kernel<L, BF16>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid_for_tokens(T, threads)), dim3(threads), lds, s, X, T, K,
                       sign, perm, th, nth, codes, sigma);
    return hipGetLastError();
}

}  // namespace

#define RQ_DISPATCH_L(FN, BF, ...)                         \
    switch (L) {                                           \
        case 1: return (int)FN<1, BF>(__VA_ARGS__);        \
        case 2: return (int)FN<2, BF>(__VA_ARGS__);        \
        case 3: return (int)FN<3, BF>(__VA_ARGS__);        \
        case 4: return (int)FN<4, BF>(__VA_ARGS__);        \
        case 5: return (int)FN<5, BF>(__VA_ARGS__);        \
        case 6: return (int)FN<6, BF>(__VA_ARGS__);        \
        case 7: return (int)FN<7, BF>(__VA_ARGS__);        \
        case 8: return (int)FN<8, BF>(__VA_ARGS__);        \
        case 9: return (int)FN<9, BF>(__VA_ARGS__);        \
        case 10: return (int)FN<10, BF>(__VA_ARGS__);      \
        default: return (int)hipErrorInvalidValue;         \
    }

int launch_rpbh_int4(const void *X, int x_bf16, int64_t T, int K, int block, const int8_t *sign,
                     const int32_t *perm, uint8_t *codes, float *scale, void *stream) {
    const int L = ilog2(block);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (x_bf16) {
        RQ_DISPATCH_L(launch_int4_L, true, X, T, K, sign, perm, codes, scale, s)
    } else {
        RQ_DISPATCH_L(launch_int4_L, false, X, T, K, sign, perm, codes, scale, s)
    }
}

int launch_rpbh_lloydmax(const void *X, int x_bf16, int64_t T, int K, int block,
                         const int8_t *sign, const int32_t *perm, const float *thresholds,
                         int n_thresholds, uint8_t *codes, float *sigma, void *stream) {
    const int L = ilog2(block);
    hipStream_t s = static_cast<hipStream_t>(stream);
    Thresholds th;
    for (int i = 0; i < 15; ++i) th.v[i] = i < n_thresholds ? thresholds[i] : 0.0f;
    if (x_bf16) {
        RQ_DISPATCH_L(launch_lm_L, true, X, T, K, sign, perm, th, n_thresholds, codes, sigma, s)
    } else {
        RQ_DISPATCH_L(launch_lm_L, false, X, T, K, sign, perm, th, n_thresholds, codes, sigma, s)
    }
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
                       uint16_t *top, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(dense_quant_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, U, T,
                       K, r, codes, scale, top);
    return (int)hipGetLastError();
}

}  // namespace rq

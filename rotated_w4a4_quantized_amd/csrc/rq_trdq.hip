// rq_trdq.hip -- TR-DQ's runtime activation rotation for gfx950, with the
// per-token integer quantizer.
//
// "TR-DQ: Time-Rotation Diffusion Quantization", section 3.2, Eq.(9)-(10):
// G(X) = (X Delta) R1 P R2 -- a per-channel smoothing multiplier, a block
// rotation R1 (Eq.(8): b x b blocks), the zigzag permutation P and a second
// block rotation R2; quantization parameters are computed online per token
// from the extremes (section 3.2; the quantizer of section 3.1 Eq.(1)-(3)).
// Arithmetic (the reading this library fixes so that codes are
// reproducible): y = fl32(x * smooth); every rotated coordinate is one fp32
// fused multiply-add chain over its block's inputs ascending, from +0; the
// permutation is a gather, p[j] = z[perm[j]].  The chains stay on the VALU:
// the matrix cores' summation order is unspecified, and the codes depend on
// every bit of u.
//
// Work decomposition.  A workgroup owns TOK consecutive tokens; their rows
// live in LDS as fp32 (TOK * K * 4 bytes).  For a block rotation, b / 4
// threads take one block, four output columns each, for all TOK tokens: per
// block input i a thread loads R[c][i][4 g .. 4 g + 3] (16 bytes, coalesced
// across the block's threads) and reads y[t][c b + i] from LDS (the same word
// for all of the block's threads), then TOK x 4 fused multiply-adds.  The
// 256 threads cover 1024 / b blocks at once and loop over the rest, holding
// every output in registers (K / 1024 blocks x TOK tokens x 4 columns).
//   load     x -> y = x * smooth, into LDS
//   R1       z in registers; barrier; z written over y (each block reads only
//            its own inputs, so the in-place write waits for one barrier)
//   R2       inputs gathered from z through perm; u stays in registers
//   stat     per-token max |u| (or min and max) by shuffles and LDS atomics
//   codes    per (block, token) four consecutive codes: one 2- or 4-byte store

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rq_internal.h"

namespace rq {
namespace {

constexpr int kThreads = 256;

// Order-preserving 32-bit key of a float (LDS atomic min / max of either sign).
__device__ inline unsigned fkey(float f) {
    const unsigned b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float fkey_inv(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

struct TrdqArgs {
    const void *X;
    int64_t T;
    int K;
    int b;                 // block
    const float *smooth;   // [K]
    const float *R1;       // [K/b][b][b]
    const int32_t *perm;   // [K]
    const float *R2;       // [K/b][b][b]
    uint8_t *codes;        // [T][K a_bits / 8]
    float *scale;          // [T] (asymmetric: s [T] then z [T])
};

// TOK tokens per workgroup, NBMAX = the most blocks one thread handles,
// QB code bits (4 or 8), ASYM zero point.
template <int TOK, int NBMAX, bool BF16, int QB, bool ASYM>
__global__ void __launch_bounds__(kThreads)
trdq_quant_kernel(TrdqArgs a) {
    extern __shared__ __attribute__((aligned(16))) float buf[];   // [TOK][K]
    __shared__ unsigned red_max[TOK], red_min[TOK];
    const int K = a.K, b = a.b;
    const int tid = threadIdx.x;
    const int tpb = b / 4;                 // threads per block
    const int slots = kThreads / tpb;      // blocks processed at once
    const int slot = tid / tpb, g = tid - slot * tpb;
    const int nblk = K / b;
    const int64_t t0 = (int64_t)blockIdx.x * TOK;

    if (tid < TOK) {
        red_max[tid] = 0u;
        red_min[tid] = 0xFFFFFFFFu;
    }
    // load and smooth: y = fl32(x * smooth)
    {
        constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
        const int cpr = K / EPC;            // chunks per row
        for (int c = tid; c < TOK * cpr; c += kThreads) {
            const int t = c / cpr, k0 = (c - t * cpr) * EPC;
            int64_t tok = t0 + t;
            if (tok >= a.T) tok = a.T - 1;
            float x[EPC];
            if constexpr (BF16) {
                const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.X) + tok * K + k0);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = __uint_as_float(ww[e] << 16);
                    x[2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
                }
            } else {
                const float4 w = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.X) + tok * K + k0);
                x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) buf[t * K + k0 + e] = x[e] * a.smooth[k0 + e];
        }
    }
    __syncthreads();

    float v[NBMAX][TOK][4];
    // one block rotation over LDS rows: v[bi] = (inputs of block c) R[c]
    // columns 4 g .. 4 g + 3, inputs y[t][c b + i] or, with GATHER,
    // y[t][perm[c b + i]]
    auto rotate = [&](const float *R, auto gather_c) {
        constexpr bool GATHER = decltype(gather_c)::value;
#pragma unroll
        for (int bi = 0; bi < NBMAX; ++bi) {
            const int c = slot + bi * slots;
            if (c >= nblk) break;
            float acc[TOK][4];
#pragma unroll
            for (int t = 0; t < TOK; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[t][e] = 0.0f;
            const float *Rc = R + (size_t)c * b * b + 4 * g;
            const int32_t *pc = a.perm + c * b;
#pragma unroll 4
            for (int i = 0; i < b; ++i) {
                const float4 r = *reinterpret_cast<const float4 *>(Rc + (size_t)i * b);
                const int src = GATHER ? pc[i] : c * b + i;
#pragma unroll
                for (int t = 0; t < TOK; ++t) {
                    const float y = buf[t * K + src];
                    acc[t][0] = fmaf(y, r.x, acc[t][0]);
                    acc[t][1] = fmaf(y, r.y, acc[t][1]);
                    acc[t][2] = fmaf(y, r.z, acc[t][2]);
                    acc[t][3] = fmaf(y, r.w, acc[t][3]);
                }
            }
#pragma unroll
            for (int t = 0; t < TOK; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) v[bi][t][e] = acc[t][e];
        }
    };

    rotate(a.R1, std::false_type{});
    __syncthreads();   // every block's inputs are read
#pragma unroll
    for (int bi = 0; bi < NBMAX; ++bi) {
        const int c = slot + bi * slots;
        if (c >= nblk) break;
#pragma unroll
        for (int t = 0; t < TOK; ++t)
            *reinterpret_cast<float4 *>(buf + t * K + c * b + 4 * g) =
                make_float4(v[bi][t][0], v[bi][t][1], v[bi][t][2], v[bi][t][3]);
    }
    __syncthreads();
    rotate(a.R2, std::true_type{});

    // per-token statistic
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
        float hi = ASYM ? -INFINITY : 0.0f, lo = INFINITY;
#pragma unroll
        for (int bi = 0; bi < NBMAX; ++bi) {
            if (slot + bi * slots >= nblk) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ASYM) {
                    hi = fmaxf(hi, v[bi][t][e]);
                    lo = fminf(lo, v[bi][t][e]);
                } else {
                    hi = fmaxf(hi, fabsf(v[bi][t][e]));
                }
            }
        }
        unsigned khi = ASYM ? fkey(hi) : __float_as_uint(hi);   // |u| >= 0 orders as unsigned
        unsigned klo = fkey(lo);
        for (int off = 32; off > 0; off >>= 1) {
            khi = max(khi, (unsigned)__shfl_xor((int)khi, off, 64));
            if constexpr (ASYM) klo = min(klo, (unsigned)__shfl_xor((int)klo, off, 64));
        }
        if ((tid & 63) == 0) {
            atomicMax(&red_max[t], khi);
            if constexpr (ASYM) atomicMin(&red_min[t], klo);
        }
    }
    __syncthreads();

    constexpr float kQ = ASYM ? (QB == 8 ? 255.0f : 15.0f) : (QB == 8 ? 127.0f : 7.0f);
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
        const int64_t tok = t0 + t;
        if (tok >= a.T) break;
        float inv = 0.0f, sc = 0.0f, zp = 0.0f;
        bool zero_row;
        if constexpr (ASYM) {
            // s = fl32(d / L), inv = fl32(L / d), z = clamp(-rne(fl32(lo inv)), 0, L)
            const float lo = fkey_inv(red_min[t]), hi = fkey_inv(red_max[t]);
            const float d = hi - lo;
            zero_row = d == 0.0f;
            if (!zero_row) {
                inv = kQ / d;
                sc = d / kQ;
                const float zr = rintf(lo * inv);
                zp = zr >= 0.0f ? 0.0f : (zr < -kQ ? kQ : -zr);
            }
        } else {
            // s = fl32(amax / qmax), inv = fl32(qmax / amax)
            const float amax = __uint_as_float(red_max[t]);
            zero_row = amax == 0.0f;
            if (!zero_row) {
                inv = kQ / amax;
                sc = amax / kQ;
            }
        }
        if (tid == 0) {
            a.scale[tok] = sc;
            if constexpr (ASYM) a.scale[a.T + tok] = zp;
        }
#pragma unroll
        for (int bi = 0; bi < NBMAX; ++bi) {
            const int c = slot + bi * slots;
            if (c >= nblk) break;
            uint32_t q[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float r = rintf(v[bi][t][e] * inv);
                if constexpr (ASYM) r = fminf(fmaxf(r + zp, 0.0f), kQ);
                else r = fminf(fmaxf(r, -kQ), kQ);
                q[e] = zero_row ? 0u : ((uint32_t)(int)r & (QB == 8 ? 0xFFu : 0xFu));
            }
            const int k = c * b + 4 * g;
            if constexpr (QB == 8)
                *reinterpret_cast<uint32_t *>(a.codes + tok * K + k) =
                    q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
            else
                *reinterpret_cast<uint16_t *>(a.codes + tok * (K / 2) + k / 2) =
                    (uint16_t)(q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12));
        }
    }
}

template <int TOK, int NBMAX, bool BF16>
hipError_t launch_tok(const TrdqArgs &a, int asym, int a_bits, hipStream_t s) {
    const size_t lds = (size_t)TOK * a.K * sizeof(float);
    const dim3 grid((unsigned)((a.T + TOK - 1) / TOK));
    auto go = [&](auto kern) -> hipError_t {
        const hipError_t e = (hipError_t)ensure_dyn_lds((const void *)kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
        return hipGetLastError();
    };
    if (a_bits == 8)
        return asym ? go(trdq_quant_kernel<TOK, NBMAX, BF16, 8, true>)
                    : go(trdq_quant_kernel<TOK, NBMAX, BF16, 8, false>);
    return asym ? go(trdq_quant_kernel<TOK, NBMAX, BF16, 4, true>)
                : go(trdq_quant_kernel<TOK, NBMAX, BF16, 4, false>);
}

}  // namespace

int launch_trdq(const void *X, int x_bf16, int64_t T, int K, int block, const float *smooth,
                const float *R1, const int32_t *perm, const float *R2, uint8_t *codes,
                float *scale, int asym, int a_bits, void *stream) {
    TrdqArgs a{X, T, K, block, smooth, R1, perm, R2, codes, scale};
    hipStream_t s = static_cast<hipStream_t>(stream);
    // a thread holds ceil(K / 1024) blocks x TOK tokens x 4 columns
    if (K <= 4096)
        return (int)(x_bf16 ? launch_tok<4, 4, true>(a, asym, a_bits, s)
                            : launch_tok<4, 4, false>(a, asym, a_bits, s));
    if (K <= 8192)
        return (int)(x_bf16 ? launch_tok<4, 8, true>(a, asym, a_bits, s)
                            : launch_tok<4, 8, false>(a, asym, a_bits, s));
    return (int)(x_bf16 ? launch_tok<2, 16, true>(a, asym, a_bits, s)
                        : launch_tok<2, 16, false>(a, asym, a_bits, s));
}

}  // namespace rq

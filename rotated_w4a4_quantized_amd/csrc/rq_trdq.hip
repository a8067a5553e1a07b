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
    uint8_t *codes;        // [T][K / 2] (4-bit) or [T][K] (6- and 8-bit), or null
    uint8_t *codes_mma;    // byte codes in the int8 GEMM's fragment order, or null
    float *scale;          // [T] (asymmetric: s [T] then z [T])
    float qbyte;           // byte codes: symmetric qmax 31 / 127 or asymmetric top code 63 / 255
};

// 8-bit code of (token t, coordinate k) in the int8 GEMM's fragment order
// [t / 32][k / 32][lane t % 32 + 32 (k % 32 / 16)][k % 16]
__device__ __forceinline__ int64_t i8_frag_offset(int64_t t, int k, int K) {
    return (((t >> 5) * (K / 32) + (k >> 5)) * 64 + (t & 31) + 32 * ((k & 31) >> 4)) * 16 + (k & 15);
}

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

    // QB: code container (4: nibbles, 8: bytes holding 6- or 8-bit codes)
    const float kQ = QB == 8 ? a.qbyte : (ASYM ? 15.0f : 7.0f);
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
            if constexpr (QB == 8) {
                const uint32_t w = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
                if (a.codes) *reinterpret_cast<uint32_t *>(a.codes + tok * K + k) = w;
                if (a.codes_mma) *reinterpret_cast<uint32_t *>(a.codes_mma + i8_frag_offset(tok, k, K)) = w;
            } else {
                *reinterpret_cast<uint16_t *>(a.codes + tok * (K / 2) + k / 2) =
                    (uint16_t)(q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12));
            }
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
    if (a_bits != 4)   // 6- or 8-bit codes, one per byte
        return asym ? go(trdq_quant_kernel<TOK, NBMAX, BF16, 8, true>)
                    : go(trdq_quant_kernel<TOK, NBMAX, BF16, 8, false>);
    return asym ? go(trdq_quant_kernel<TOK, NBMAX, BF16, 4, true>)
                : go(trdq_quant_kernel<TOK, NBMAX, BF16, 4, false>);
}

// ---------------------------------------------------------------------------
// Tiled form (a workspace is given): three launches.
//   rot 1   z = (x * smooth) BlockDiag(R1)          -> Zt, fp32 [K][Tp], token
//           index fastest (Tp = T rounded up to 128), so that rot 2 gathers
//           whole 512-byte column runs
//   rot 2   u = z[perm] BlockDiag(R2)               -> U, fp32 [T][K], and the
//           per-token extremes (atomics on [2][T] keys)
//   quant   codes and scales from U and the extremes
// A rotation workgroup owns 128 tokens x DJ = 16 CW columns of one block and
// walks that block's b inputs in chunks of 16: the chunk's input tile
// (transposed, [k][token]) and R tile sit in one of two LDS buffers while the
// next chunk is loaded into registers and written to the other (one barrier
// per chunk); each thread keeps 8 tokens x CW columns of sums.  Every output
// is the same FMA chain as in the one-pass kernel (the block's inputs
// ascending from +0), so the codes agree bit for bit; R is read once per 128
// tokens instead of once per workgroup of 2 or 4 tokens.
// ---------------------------------------------------------------------------
constexpr int kTT = 128;   // tokens per rotation tile
constexpr int kTK = 16;    // k per chunk

struct TileArgs {
    const void *X;          // STEP 1: x [T][K] (bf16 or fp32); STEP 2: Zt
    float *Out;             // STEP 1: Zt; STEP 2: U
    const float *smooth;    // STEP 1
    const int32_t *perm;    // STEP 2
    const float *R;         // [K/b][b][b]
    unsigned *stat;         // [2][T]: max key, then min key (asymmetric)
    int64_t T;
    int64_t Tp;             // Zt row stride (T rounded up to 128)
    int K, b;
};

template <int CW>
__device__ __forceinline__ void pin_sums(float (&r)[CW]) {
    if constexpr (CW == 8)
        asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]));
    else if constexpr (CW == 4)
        asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
    else if constexpr (CW == 2)
        asm volatile("" : "+v"(r[0]), "+v"(r[1]));
    else
        asm volatile("" : "+v"(r[0]));
}

// STEP 1: inputs x * smooth (BF16: x is bf16); STEP 2: inputs Z[perm[k]],
// per-token extremes of the outputs (ASYM: min and max, else max |u|).
template <int STEP, bool BF16, int CW, bool ASYM>
__global__ void __launch_bounds__(256)
trdq_tile_kernel(TileArgs a) {
    constexpr int DJ = 16 * CW;
    constexpr int RL = (kTK * DJ / 4 + 255) / 256;   // 16-byte R loads per thread per chunk
    __shared__ __attribute__((aligned(16))) float xs[2][kTK][kTT + 4];
    __shared__ __attribute__((aligned(16))) float rs[2][kTK][DJ + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t t0 = (int64_t)blockIdx.y * kTT;
    const int K = a.K, b = a.b;
    const int j0 = blockIdx.x * DJ;           // first output column
    const int c = j0 / b;                     // its block (DJ divides b)
    const int kb = c * b;                     // the block's first input
    const float *Rc = a.R + (size_t)c * b * b + (j0 - kb);

    if constexpr (STEP == 1) {
        // the extremes of rot 2 start from the atomics' identities
        if (blockIdx.x == 0 && tid < kTT && t0 + tid < a.T) {
            a.stat[t0 + tid] = 0u;
            a.stat[a.T + t0 + tid] = 0xFFFFFFFFu;
        }
    }

    // input loads: STEP 1 x as 16-byte pieces (thread -> token tid / 2, k
    // 8 (tid % 2) .. + 7: one piece of bf16, two of fp32); STEP 2 the
    // gathered columns of Zt (thread -> k tid / 16, tokens 8 (tid % 16) .. + 7:
    // two pieces)
    constexpr int XW = STEP == 1 ? (BF16 ? 4 : 8) : 8;   // 32-bit words per thread
    uint32_t xr[XW];
    float4 rr[RL];
    const int lt = tid >> 1, lh = tid & 1;
    int64_t ltok = t0 + lt;
    if (ltok >= a.T) ltok = a.T - 1;
    auto load = [&](int k0) {
        if constexpr (STEP == 1) {
            if constexpr (BF16) {
                const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.X) + ltok * K + k0 + 8 * lh);
                xr[0] = w.x; xr[1] = w.y; xr[2] = w.z; xr[3] = w.w;
            } else {
                const float *src = static_cast<const float *>(a.X) + ltok * K + k0 + 8 * lh;
                const uint4 w0 = *reinterpret_cast<const uint4 *>(src);
                const uint4 w1 = *reinterpret_cast<const uint4 *>(src + 4);
                xr[0] = w0.x; xr[1] = w0.y; xr[2] = w0.z; xr[3] = w0.w;
                xr[4] = w1.x; xr[5] = w1.y; xr[6] = w1.z; xr[7] = w1.w;
            }
        } else {
            const float *col = static_cast<const float *>(a.X) + (int64_t)a.perm[k0 + (tid >> 4)] * a.Tp + t0 +
                               8 * (tid & 15);
            const uint4 w0 = *reinterpret_cast<const uint4 *>(col);
            const uint4 w1 = *reinterpret_cast<const uint4 *>(col + 4);
            xr[0] = w0.x; xr[1] = w0.y; xr[2] = w0.z; xr[3] = w0.w;
            xr[4] = w1.x; xr[5] = w1.y; xr[6] = w1.z; xr[7] = w1.w;
        }
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int q = tid + 256 * i;
            const int kk = q / (DJ / 4), jj = 4 * (q % (DJ / 4));
            if (kk < kTK) rr[i] = *reinterpret_cast<const float4 *>(Rc + (size_t)(k0 - kb + kk) * b + jj);
        }
    };
    auto store = [&](int buf, int k0) {
        const int kq = 8 * lh;
        if constexpr (STEP == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x;
                if constexpr (BF16)
                    x = __uint_as_float(e & 1 ? (xr[e >> 1] & 0xFFFF0000u) : (xr[e >> 1] << 16));
                else
                    x = __uint_as_float(xr[e]);
                xs[buf][kq + e][lt] = x * a.smooth[k0 + kq + e];
            }
        } else {
            float *d = &xs[buf][tid >> 4][8 * (tid & 15)];
            *reinterpret_cast<uint4 *>(d) = make_uint4(xr[0], xr[1], xr[2], xr[3]);
            *reinterpret_cast<uint4 *>(d + 4) = make_uint4(xr[4], xr[5], xr[6], xr[7]);
        }
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int q = tid + 256 * i;
            const int kk = q / (DJ / 4), jj = 4 * (q % (DJ / 4));
            if (kk < kTK) *reinterpret_cast<float4 *>(&rs[buf][kk][jj]) = rr[i];
        }
    };

    float acc[8][CW];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < CW; ++e) acc[t][e] = 0.0f;
    const int nchunk = b / kTK;
    load(kb);
    store(0, kb);
    __syncthreads();
    for (int ch = 0; ch < nchunk; ++ch) {
        const int buf = ch & 1;
        const int k0 = kb + ch * kTK;
        if (ch + 1 < nchunk) load(k0 + kTK);
        float xa[2][8], rb[2][CW];
        auto rd = [&](int kk, int p) {
#pragma unroll
            for (int t = 0; t < 8; ++t) xa[p][t] = xs[buf][kk][ty * 8 + t];
#pragma unroll
            for (int e = 0; e < CW; ++e) rb[p][e] = rs[buf][kk][tx * CW + e];
        };
        rd(0, 0);
#pragma unroll
        for (int kk = 0; kk < kTK; ++kk) {
            if (kk + 1 < kTK) rd(kk + 1, (kk + 1) & 1);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < CW; ++e) acc[t][e] = fmaf(xa[kk & 1][t], rb[kk & 1][e], acc[t][e]);
#pragma unroll
            for (int t = 0; t < 8; ++t) pin_sums(acc[t]);
        }
        if (ch + 1 < nchunk) store(buf ^ 1, k0 + kTK);
        __syncthreads();
    }

    // outputs: tokens t0 + 8 ty + t, columns j0 + CW tx .. + CW - 1
    if constexpr (STEP == 1) {
        // Zt: per column, the thread's eight tokens are 32 contiguous bytes
        // (the padding rows past T are written too; nothing reads them for
        // a real token)
#pragma unroll
        for (int e = 0; e < CW; ++e) {
            float *d = a.Out + (int64_t)(j0 + tx * CW + e) * a.Tp + t0 + ty * 8;
            *reinterpret_cast<float4 *>(d) = make_float4(acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
            *reinterpret_cast<float4 *>(d + 4) = make_float4(acc[4][e], acc[5][e], acc[6][e], acc[7][e]);
        }
        return;
    }
    float *o = a.Out + (t0 + ty * 8) * K + j0 + tx * CW;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t tok = t0 + ty * 8 + t;
        const bool ok = tok < a.T;
        if (ok) {
            if constexpr (CW % 4 == 0) {
#pragma unroll
                for (int e = 0; e < CW; e += 4)
                    *reinterpret_cast<float4 *>(o + e) = make_float4(acc[t][e], acc[t][e + 1], acc[t][e + 2], acc[t][e + 3]);
            } else {
#pragma unroll
                for (int e = 0; e < CW; ++e) o[e] = acc[t][e];
            }
        }
        o += K;
        if constexpr (STEP == 2) {
            // this token's extremes over the tile: the thread's CW columns,
            // then the 16 threads (lanes) of its row group
            float hi = ASYM ? -INFINITY : 0.0f, lo = INFINITY;
#pragma unroll
            for (int e = 0; e < CW; ++e) {
                if constexpr (ASYM) {
                    hi = fmaxf(hi, acc[t][e]);
                    lo = fminf(lo, acc[t][e]);
                } else {
                    hi = fmaxf(hi, fabsf(acc[t][e]));
                }
            }
            unsigned khi = ASYM ? fkey(hi) : __float_as_uint(hi);
            unsigned klo = fkey(lo);
            for (int off = 1; off < 16; off <<= 1) {
                khi = max(khi, (unsigned)__shfl_xor((int)khi, off, 64));
                if constexpr (ASYM) klo = min(klo, (unsigned)__shfl_xor((int)klo, off, 64));
            }
            if (tx == 0 && ok) {
                atomicMax(&a.stat[tok], khi);
                if constexpr (ASYM) atomicMin(&a.stat[a.T + tok], klo);
            }
        }
    }
}

// codes and scales of U: one wave per token, four consecutive coordinates per
// lane and step (the one-pass kernel's quantizer, formula for formula)
template <int QB, bool ASYM>
__global__ void __launch_bounds__(256)
trdq_quant_tiled_kernel(const float *__restrict__ U, const unsigned *__restrict__ stat, int64_t T, int K,
                        uint8_t *__restrict__ codes, uint8_t *__restrict__ codes_mma,
                        float *__restrict__ scale, float qbyte) {
    const int lane = threadIdx.x & 63;
    const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= T) return;
    // QB: code container (4: nibbles, 8: bytes holding 6- or 8-bit codes)
    const float kQ = QB == 8 ? qbyte : (ASYM ? 15.0f : 7.0f);
    float inv = 0.0f, sc = 0.0f, zp = 0.0f;
    bool zero_row;
    if constexpr (ASYM) {
        const float lo = fkey_inv(stat[T + tok]), hi = fkey_inv(stat[tok]);
        const float d = hi - lo;
        zero_row = d == 0.0f;
        if (!zero_row) {
            inv = kQ / d;
            sc = d / kQ;
            const float zr = rintf(lo * inv);
            zp = zr >= 0.0f ? 0.0f : (zr < -kQ ? kQ : -zr);
        }
    } else {
        const float amax = __uint_as_float(stat[tok]);
        zero_row = amax == 0.0f;
        if (!zero_row) {
            inv = kQ / amax;
            sc = amax / kQ;
        }
    }
    if (lane == 0) {
        scale[tok] = sc;
        if constexpr (ASYM) scale[T + tok] = zp;
    }
    const float *u = U + tok * K;
    for (int k = 4 * lane; k < K; k += 256) {
        const float4 v4 = *reinterpret_cast<const float4 *>(u + k);
        const float v[4] = {v4.x, v4.y, v4.z, v4.w};
        uint32_t q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float r = rintf(v[e] * inv);
            if constexpr (ASYM) r = fminf(fmaxf(r + zp, 0.0f), kQ);
            else r = fminf(fmaxf(r, -kQ), kQ);
            q[e] = zero_row ? 0u : ((uint32_t)(int)r & (QB == 8 ? 0xFFu : 0xFu));
        }
        if constexpr (QB == 8) {
            const uint32_t w = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
            if (codes) *reinterpret_cast<uint32_t *>(codes + tok * K + k) = w;
            if (codes_mma) *reinterpret_cast<uint32_t *>(codes_mma + i8_frag_offset(tok, k, K)) = w;
        } else
            *reinterpret_cast<uint16_t *>(codes + tok * (K / 2) + k / 2) =
                (uint16_t)(q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12));
    }
}

template <int STEP, bool BF16, bool ASYM>
hipError_t launch_tile_step(const TileArgs &a, hipStream_t s) {
    // widest column tile that divides the block
    const int cw = a.b >= 128 ? 8 : a.b / 16;
    const dim3 grid((unsigned)(a.K / (16 * cw)), (unsigned)((a.T + kTT - 1) / kTT));
    switch (cw) {
        case 8: hipLaunchKernelGGL((trdq_tile_kernel<STEP, BF16, 8, ASYM>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((trdq_tile_kernel<STEP, BF16, 4, ASYM>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((trdq_tile_kernel<STEP, BF16, 2, ASYM>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((trdq_tile_kernel<STEP, BF16, 1, ASYM>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

int launch_trdq(const void *X, int x_bf16, int64_t T, int K, int block, const float *smooth,
                const float *R1, const int32_t *perm, const float *R2, uint8_t *codes,
                uint8_t *codes_mma, float *scale, int asym, int a_bits, void *stream) {
    const float qbyte = asym ? (float)((1 << a_bits) - 1) : (float)((1 << (a_bits - 1)) - 1);
    TrdqArgs a{X, T, K, block, smooth, R1, perm, R2, codes, codes_mma, scale, qbyte};
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

size_t trdq_workspace_bytes(int64_t T, int K) {
    const size_t Tp = (size_t)((T + kTT - 1) / kTT) * kTT;
    return Tp * (size_t)K * 4 + (size_t)T * (size_t)K * 4 + (size_t)T * 8;
}

int launch_trdq_tiled(const void *X, int x_bf16, int64_t T, int K, int block, const float *smooth,
                      const float *R1, const int32_t *perm, const float *R2, uint8_t *codes,
                      uint8_t *codes_mma, float *scale, int asym, int a_bits, void *workspace,
                      void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t Tp = (T + kTT - 1) / kTT * kTT;
    float *Zt = static_cast<float *>(workspace);
    float *U = Zt + (size_t)Tp * K;
    unsigned *stat = reinterpret_cast<unsigned *>(U + (size_t)T * K);
    TileArgs a1{X, Zt, smooth, perm, R1, stat, T, Tp, K, block};
    TileArgs a2{Zt, U, smooth, perm, R2, stat, T, Tp, K, block};
    hipError_t e;
    if (x_bf16) e = asym ? launch_tile_step<1, true, true>(a1, s) : launch_tile_step<1, true, false>(a1, s);
    else e = asym ? launch_tile_step<1, false, true>(a1, s) : launch_tile_step<1, false, false>(a1, s);
    if (e != hipSuccess) return (int)e;
    e = asym ? launch_tile_step<2, false, true>(a2, s) : launch_tile_step<2, false, false>(a2, s);
    if (e != hipSuccess) return (int)e;
    const dim3 grid((unsigned)((T + 3) / 4));
    const float qb = asym ? (float)((1 << a_bits) - 1) : (float)((1 << (a_bits - 1)) - 1);
    if (a_bits != 4) {   // 6- or 8-bit codes, one per byte
        if (asym) hipLaunchKernelGGL((trdq_quant_tiled_kernel<8, true>), grid, dim3(256), 0, s, U, stat, T, K, codes, codes_mma, scale, qb);
        else hipLaunchKernelGGL((trdq_quant_tiled_kernel<8, false>), grid, dim3(256), 0, s, U, stat, T, K, codes, codes_mma, scale, qb);
    } else {
        if (asym) hipLaunchKernelGGL((trdq_quant_tiled_kernel<4, true>), grid, dim3(256), 0, s, U, stat, T, K, codes, codes_mma, scale, qb);
        else hipLaunchKernelGGL((trdq_quant_tiled_kernel<4, false>), grid, dim3(256), 0, s, U, stat, T, K, codes, codes_mma, scale, qb);
    }
    return (int)hipGetLastError();
}

}  // namespace rq

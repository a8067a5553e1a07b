// rq_rpbh.hip -- runtime activation path for gfx950 with the randomized
// permuted block-Hadamard (RPBH) rotation, then per-token 4-bit
// quantization: symmetric INT4, asymmetric INT4 with a zero point ("TR-DQ"
// section 3.1, Eq.(1)-(3)), or the Lloyd-Max codebook on the
// norm-normalized token.
//
// Rotation ("OrbitQuant" abstract; block structure "TR-DQ" Eq.(8)):
//   y[j] = sign[j] * x[perm[j]]; then on every b-block the unnormalized
//   Sylvester transform by radix-2 fp32 butterflies (lo, hi) -> (lo + hi,
//   lo - hi), stages h = 1, 2, ..., b/2 in that order.  Inside one stage the
//   butterflies are independent, so any schedule that keeps the stage order
//   and evaluates lo + hi and lo - hi in fp32 gives the same bits.
//
// Work decomposition.  A token is owned by K/32 threads, 32 coordinates
// each; a workgroup holds `tpw` tokens.  Per token:
//   staging  the row is read from HBM one iteration ahead (coalesced 16-byte
//            loads into registers), the sign of the coordinate each source
//            element will land on is applied with one XOR per 32-bit word,
//            and the row is written to LDS in its natural order;
//   gather   each thread reads its 32 permuted inputs from LDS;
//   pass 0   stages on bits 0..4 of the block index, in registers;
//   pass p   one exchange inside the wave (two rounds through LDS, see
//            exchange()), then up to four more stages in registers; the
//            register set of every pass after the first also carries index
//            bit 0, so the final values of each nibble pair sit in one thread;
//   stat     per-token absmax (asymmetric: min and max; for the codebook
//            also the exact integer-grid squared norm) by shuffles and one
//            LDS atomic per lane group;
//   codes    nibbles are packed from registers and regrouped through LDS
//            into 16 contiguous bytes per 32 coordinates; the canonical
//            layout is stored with one 16-byte store per thread.  For the
//            GEMM's FP6 fragment layout (rq_fp6.h) a workgroup takes its
//            tokens in groups of at least four consecutive ones, keeps the
//            group's codes in LDS, and once the group is complete spreads
//            them so that the four tokens' 16-byte slots of one piece -- 64
//            contiguous bytes -- come from four adjacent lanes: whole-request
//            stores instead of sixteen-byte writes to scattered lines.
// Two workgroup barriers per iteration of `tpw` tokens (three for the
// codebook).  A per-workgroup prologue reads perm and sign and builds the
// source-side sign masks in LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq_fp6.h"
#include "rq_internal.h"

namespace rq {
namespace {

constexpr int kE = 32;   // coordinates per thread
constexpr int kMaxTpw = 16;
// Threads per workgroup: bf16 input up to twelve waves, three per SIMD (at
// most 168 registers per lane, which the kernel fits); fp32 input stages
// twice the words per thread and keeps the 256-register budget of eight.
template <bool BF16>
constexpr int kMaxThreads = BF16 ? 768 : 512;
// relative time per token of a workgroup that shares its CU with others
// (their LDS, memory and VALU phases overlap), against one alone on the CU
constexpr double kOverlap = 0.75;

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its global loads and stores (a __syncthreads() would
// also drain the next token's prefetch and the code stores in flight).
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int L>
struct Plan {
    static constexpr int NP = L <= 5 ? 1 : 1 + (L - 5 + 3) / 4;
    __host__ __device__ static constexpr int lo(int p) { return p == 0 ? 0 : 5 + 4 * (p - 1); }
    __host__ __device__ static constexpr int hi(int p) {
        return p == 0 ? (L < 5 ? L : 5) : (5 + 4 * p < L ? 5 + 4 * p : L);
    }
    // index bit carried by register bit k in pass p
    __host__ __device__ static constexpr int vbit(int p, int k) {
        return p == 0 ? k : (k < 5 - (hi(p) - lo(p)) ? k : lo(p) + k - (5 - (hi(p) - lo(p))));
    }
    __host__ __device__ static constexpr int roff(int p, int r) {
        int o = 0;
        for (int k = 0; k < 5; ++k)
            if ((r >> k) & 1) o |= 1 << vbit(p, k);
        return o;
    }
    __host__ __device__ static constexpr bool isv(int p, int pos) {
        for (int k = 0; k < 5; ++k)
            if (vbit(p, k) == pos) return true;
        return false;
    }
    __host__ __device__ static constexpr int rbit(int p, int s) {
        for (int k = 0; k < 5; ++k)
            if (vbit(p, k) == s) return k;
        return -1;
    }
};

// First coordinate of thread tt's set in pass P (the set is base + roff(P, r)).
template <int L, int P>
__device__ inline int pbase(int tt) {
    if constexpr (P == 0) {
        return kE * tt;
    } else {
        const int c = tt >> (L - 5);
        int f = tt & ((1 << (L - 5)) - 1);
        int i = 0;
#pragma unroll
        for (int pos = 0; pos < L; ++pos) {
            if (Plan<L>::isv(P, pos)) continue;
            i |= (f & 1) << pos;
            f >>= 1;
        }
        return (c << L) + i;
    }
}

template <int L, int P>
__device__ inline void stages(float (&v)[kE]) {
#pragma unroll
    for (int s = Plan<L>::lo(P); s < Plan<L>::hi(P); ++s) {
        const int kb = Plan<L>::rbit(P, s);
#pragma unroll
        for (int r = 0; r < kE; ++r) {
            if (r & (1 << kb)) continue;
            const float lo = v[r], hi = v[r | (1 << kb)];
            v[r] = lo + hi;
            v[r | (1 << kb)] = lo - hi;
        }
    }
}

// Exchanges.  A block's 2^(L-5) threads are adjacent lanes of one wave, so
// every exchange stays inside a wave and needs only wave-level ordering (LDS
// operations of one wave complete in issue order).  It runs in two rounds:
// round h moves the coordinates with index bit 0 = h, which sit in the
// registers of parity h in every pass, so one round needs a buffer of half a
// token.  Half-coordinate m = j >> 1 lives at hslot(m).  In every pass a
// thread's coordinates are base | roff(r) with disjoint bit fields, so the
// slot splits into a per-thread base plus a per-register constant (an
// immediate offset of the LDS instruction).  The pads put the 64 lanes of one
// instruction on distinct banks in both access patterns for b >= 512, with at
// most a two-way conflict for b = 64..256 (checked for 32 and 64 four-byte
// banks).
template <int L>
__host__ __device__ constexpr int hslot(int m) {
    return L == 6 ? m + 8 * (m >> 4) + (m >> 6) : L == 7 ? m + 4 * (m >> 4) + (m >> 7) : m + (m >> 4);
}
// exchange words per token (blocks up to 32 need none)
template <int L>
__host__ __device__ constexpr int xwords(int K) {
    return L <= 5 ? 0 : ((hslot<L>(K / 2 - 1) + 1 + 3) & ~3);
}

template <int L, int P, int H>
__device__ inline void put(float *us, int tt, const float (&v)[kE]) {
    float *p = us + hslot<L>(pbase<L, P>(tt) >> 1);
#pragma unroll
    for (int r = H; r < kE; r += 2) p[hslot<L>(Plan<L>::roff(P, r) >> 1)] = v[r];
}
template <int L, int P, int H>
__device__ inline void get(const float *us, int tt, float (&v)[kE]) {
    const float *p = us + hslot<L>(pbase<L, P>(tt) >> 1);
#pragma unroll
    for (int r = H; r < kE; r += 2) v[r] = p[hslot<L>(Plan<L>::roff(P, r) >> 1)];
}
// orders this wave's LDS accesses at the compiler level (the hardware keeps
// one wave's LDS operations in order)
__device__ inline void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// pass P -> pass P + 1; round 0's put may already have been issued
template <int L, int P, bool PUT0>
__device__ inline void exchange(float *us, int tt, float (&v)[kE]) {
    if constexpr (PUT0) put<L, P, 0>(us, tt, v);
    wave_lds_order();
    get<L, P + 1, 0>(us, tt, v);
    wave_lds_order();
    put<L, P, 1>(us, tt, v);
    wave_lds_order();
    get<L, P + 1, 1>(us, tt, v);
}

// Code staging layout: code byte q at q + 16 (q >> (L - 1)), i.e. 16 pad
// bytes after every block (b / 2 bytes), which spreads the byte writes of one
// instruction over the banks and keeps every 16-byte chunk aligned.
template <int L>
__host__ __device__ constexpr int cpad(int q) { return q + 16 * (q >> (L - 1)); }
template <int L>
__host__ __device__ constexpr int cbytes(int K) { return L <= 5 ? K / 2 : K / 2 + 16 * (K >> L) + 16; }
// byte offset of the 16-byte code chunk c (coordinates 32 c .. 32 c + 31)
// in a token's staging slot
template <int L>
__host__ __device__ constexpr int chunk_off(int c) { return L <= 5 ? 16 * c : cpad<L>(16 * c); }

// Order-preserving 32-bit key of a float (for LDS atomic min / max over
// values of either sign) and its inverse.
__device__ inline unsigned fkey(float f) {
    const unsigned b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float fkey_inv(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// x of the lane that the data-parallel-primitive control CTRL selects inside
// x's row of 16 lanes (0 where that lane is inactive; the runs reduced below
// are all active or all inactive).
template <int CTRL>
__device__ inline unsigned dpp_peer(unsigned x) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
// Max (MAX) or min of x over every aligned run of g lanes (g = 1, 2, 4, 8 or
// 16): swaps inside each quad, then the half-row and row mirrors.  Every lane
// of a run ends with the run's result.
template <bool MAX>
__device__ inline unsigned run_reduce(unsigned x, int g) {
    auto op = [](unsigned p, unsigned q) { return MAX ? (p > q ? p : q) : (p < q ? p : q); };
    if (g >= 2) x = op(x, dpp_peer<0xB1>(x));    // quad lanes 1 0 3 2
    if (g >= 4) x = op(x, dpp_peer<0x4E>(x));    // quad lanes 2 3 0 1
    if (g >= 8) x = op(x, dpp_peer<0x141>(x));   // mirror inside each half row
    if (g >= 16) x = op(x, dpp_peer<0x140>(x));  // mirror inside the row
    return x;
}

struct RpbhArgs {
    const void *X;
    int64_t T;
    int K;
    int tpt;              // threads per token (K / 32)
    int tpw;              // tokens per workgroup
    const int8_t *sign;
    const int32_t *perm;
    uint8_t *codes;       // canonical [T][K/2], or null
    uint8_t *codes_mma;   // FP6 fragment layout (rq_fp6.h), or null (INT4 only)
    int mma_stages;       // 128-coordinate stages of the MMA layout
    int grouped;          // MMA codes written per group (else per token)
    int gsz_log2;         // tokens per group: a workgroup's unit of work
    int ipg_log2;         // iterations per group (group size / tpw)
    int64_t ngroups;
    float *scale;         // s or sigma [T]; asymmetric INT4: s [T] then z [T]
    float th[15];         // codebook thresholds (Lloyd-Max)
    int th_sym;           // th[7] == 0 and th[i] == -th[14 - i] exactly
};

template <bool BF16>
struct Src {
    // 32-bit words of input a thread stages per token, in 16-byte chunks
    static constexpr int WORDS = BF16 ? 16 : 32;
    static constexpr int CHUNKS = WORDS / 4;
    static constexpr int ELEMS_PER_CHUNK = BF16 ? 8 : 4;
    static constexpr int XB = BF16 ? 2 : 4;
};

template <int L, bool BF16, int QK>
__global__ void __launch_bounds__(kMaxThreads<BF16>)
rpbh_quant_kernel(RpbhArgs a) {
    using S = Src<BF16>;
    // Staged nibbles are the MMA-layout fields: a symmetric code is held as
    // q + 8, an unsigned one (asymmetric, codebook) as it is.  The canonical
    // layout holds a symmetric q in two's complement: the nibble's top bit
    // flipped.
    constexpr uint32_t kCanonFlip = QK == 0 ? 0x88888888u : 0u;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ unsigned red_max[2][kMaxTpw];
    __shared__ unsigned red_min[2][kMaxTpw];   // asymmetric INT4 (keys)
    __shared__ unsigned long long red_sum[2][kMaxTpw];
    const int K = a.K;
    const int tid = threadIdx.x;
    const int tl = tid / a.tpt;
    const int tt = tid - tl * a.tpt;
    uint8_t *xs = smem + (size_t)tl * K * S::XB;
    const int xw = xwords<L>(K);
    const int cb = (cbytes<L>(K) + 15) & ~15;
    float *us = reinterpret_cast<float *>(smem + (size_t)a.tpw * K * S::XB) + (size_t)tl * xw;
    // code staging: one slot per token of the group
    uint8_t *const cs0 = smem + (size_t)a.tpw * (K * S::XB + 4 * xw);

    // Workgroup b runs on XCD b % 8: number the workgroups XCD-major so that
    // each XCD works on a contiguous range of tokens, whose 32-token tiles of
    // the MMA-layout codes are then written from one L2.
    int vb = blockIdx.x;
    if (gridDim.x % 8 == 0) vb = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
    // Iteration k of this workgroup takes group vb + (k / ipg) * grid, and in
    // it tokens (k % ipg) tpw .. (k % ipg) tpw + tpw - 1; -1 past the end.
    const int ipg_mask = (1 << a.ipg_log2) - 1;
    auto first_tok = [&](int k) -> int64_t {
        const int64_t g = vb + (int64_t)(k >> a.ipg_log2) * gridDim.x;
        return g < a.ngroups ? (g << a.gsz_log2) + (int64_t)(k & ipg_mask) * a.tpw : -1;
    };
    int64_t base = first_tok(0);
    uint4 pre[S::CHUNKS];
    auto fetch = [&](int64_t b) {
        int64_t tok = b + tl;
        if (tok >= a.T) tok = a.T - 1;
        const uint8_t *row = static_cast<const uint8_t *>(a.X) + tok * (int64_t)K * S::XB;
#pragma unroll
        for (int q = 0; q < S::CHUNKS; ++q)
            pre[q] = *reinterpret_cast<const uint4 *>(row + (size_t)16 * (tt + q * a.tpt));
    };
    // the first token's row is in flight while the prologue runs
    if (base >= 0) fetch(base);

    // ---- prologue: gather offsets, source-side sign masks -----------------
    // Thread tt owns destination coordinates j = 32 tt + r: it reads perm[j]
    // and sign[j] contiguously, and writes the sign bit that source element
    // perm[j] must carry into a table in the first token's staging row (one
    // element per staging element, so the 16 bytes of the table that cover a
    // staged 16-byte chunk are that chunk's XOR mask).  Only the first
    // token's threads write it; every thread then reads its chunks' masks.
    int gofs[kE];
    {
        int pj[kE];
        int8_t sj[kE];
#pragma unroll
        for (int r = 0; r < kE; r += 4) {
            const int4 p4 = *reinterpret_cast<const int4 *>(a.perm + kE * tt + r);
            pj[r] = p4.x;
            pj[r + 1] = p4.y;
            pj[r + 2] = p4.z;
            pj[r + 3] = p4.w;
        }
#pragma unroll
        for (int r = 0; r < kE; r += 16) {
            const int4 s4 = *reinterpret_cast<const int4 *>(a.sign + kE * tt + r);
            const int w[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int e = 0; e < 16; ++e) sj[r + e] = (int8_t)(w[e >> 2] >> (8 * (e & 3)));
        }
#pragma unroll
        for (int r = 0; r < kE; ++r) gofs[r] = pj[r] * S::XB;
        if (tl == 0) {
#pragma unroll
            for (int r = 0; r < kE; ++r) {
                if constexpr (BF16)
                    *reinterpret_cast<uint16_t *>(smem + 2 * pj[r]) = sj[r] < 0 ? 0x8000u : 0u;
                else
                    *reinterpret_cast<uint32_t *>(smem + 4 * pj[r]) = sj[r] < 0 ? 0x80000000u : 0u;
            }
        }
    }
    __syncthreads();
    uint32_t smask[S::WORDS];
#pragma unroll
    for (int q = 0; q < S::CHUNKS; ++q) {
        const uint4 m = *reinterpret_cast<const uint4 *>(smem + (size_t)16 * (tt + q * a.tpt));
        smask[4 * q] = m.x;
        smask[4 * q + 1] = m.y;
        smask[4 * q + 2] = m.z;
        smask[4 * q + 3] = m.w;
    }
    __syncthreads();

    auto stage = [&]() {
#pragma unroll
        for (int q = 0; q < S::CHUNKS; ++q) {
            uint4 w = pre[q];
            w.x ^= smask[4 * q];
            w.y ^= smask[4 * q + 1];
            w.z ^= smask[4 * q + 2];
            w.w ^= smask[4 * q + 3];
            *reinterpret_cast<uint4 *>(xs + (size_t)16 * (tt + q * a.tpt)) = w;
        }
    };
    if (base >= 0) {
        stage();
        const int64_t b1 = first_tok(1);
        if (b1 >= 0) fetch(b1);
    }
    __syncthreads();

    // MMA-layout codes of group g (complete in the slots, LDS writes ordered
    // by a barrier): item i is (stage s, half h) = (i >> gsz_log2) and token
    // j = i % group size, so four adjacent lanes write one 64-byte run.
    // A group (at most 16 tokens, aligned) lies inside one 32-token tile.
    auto flush = [&](int64_t g) {
        const int items = a.mma_stages * 2 << a.gsz_log2;
        const int nth = a.tpw * a.tpt;
        const int nch = K / kE;
        const int gsz = 1 << a.gsz_log2;
        const int64_t t0 = g << a.gsz_log2;
        const int nvalid = a.T - t0 < gsz ? (int)(a.T - t0) : gsz;
        uint8_t *const tile = a.codes_mma + (t0 >> 5) * (int64_t)a.mma_stages * kMmaTileStageBytes;
        const int t32 = (int)(t0 & 31);
        for (int i = tid; i < items; i += nth) {
            const int j = i & (gsz - 1);
            const int sh = i >> a.gsz_log2;
            if (j >= nvalid) continue;
            const uint8_t *slot = cs0 + (size_t)j * cb;
            // chunks c0 (k-step 0) and c1 (k-step 1); those past the last
            // coordinate are not written
            const int c0 = 2 * (sh & ~1) + (sh & 1), c1 = c0 + 2;
            if (c0 >= nch) continue;
            const uint4 w0 = *reinterpret_cast<const uint4 *>(slot + chunk_off<L>(c0));
            const uint4 w1 = c1 < nch ? *reinterpret_cast<const uint4 *>(slot + chunk_off<L>(c1))
                                      : make_uint4(0u, 0u, 0u, 0u);
            store_pair_mma_in_tile(tile, sh >> 1, t32 + j, sh & 1, w0, w1, c1 < nch, 0u);
        }
    };
    const bool grouped = QK != 1 && a.grouped;

    // lane groups of one token for the shuffle reductions
    int grp = 64;
    while (a.tpt % grp) grp >>= 1;
    // the same runs cut to one row of 16 lanes (max / min reductions)
    const int rg = grp < 16 ? grp : 16;

    int it = 0;
    for (; base >= 0; ++it) {
        const int64_t tok = base + tl;
        const bool valid = tok < a.T;
        uint8_t *const cs = cs0 + (size_t)(((it & ipg_mask) * a.tpw) + tl) * cb;
        if (tt == 0) {
            red_max[it & 1][tl] = 0u;
            if constexpr (QK == 1) red_sum[it & 1][tl] = 0ull;
            if constexpr (QK == 2) red_min[it & 1][tl] = 0xFFFFFFFFu;
        }
        float v[kE];
#pragma unroll
        for (int r = 0; r < kE; ++r) {
            if constexpr (BF16)
                v[r] = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t *>(xs + gofs[r])) << 16);
            else
                v[r] = *reinterpret_cast<const float *>(xs + gofs[r]);
        }
        stages<L, 0>(v);
        if constexpr (Plan<L>::NP > 1) put<L, 0, 0>(us, tt, v);   // exchange round 0
        lds_barrier();  // B1: every gather of this token is done
        const int64_t next = first_tok(it + 1);
        if (next >= 0) {
            stage();                                        // next token -> LDS
            const int64_t b2 = first_tok(it + 2);
            if (b2 >= 0) fetch(b2);
        }
        // the previous group is complete: its packs are ordered by B1
        if (grouped && it > 0 && (it & ipg_mask) == 0)
            flush(vb + (int64_t)((it - 1) >> a.ipg_log2) * gridDim.x);
        if constexpr (Plan<L>::NP > 1) {
            exchange<L, 0, false>(us, tt, v);
            stages<L, 1>(v);
        }
        if constexpr (Plan<L>::NP > 2) {
            exchange<L, 1, true>(us, tt, v);
            stages<L, 2>(v);
        }
        static_assert(Plan<L>::NP <= 3, "block too large");
        constexpr int PL = Plan<L>::NP - 1;

        if constexpr (QK == 2) {
            float lo = v[0], hi = v[0];
#pragma unroll
            for (int r = 1; r < kE; ++r) {
                lo = fminf(lo, v[r]);
                hi = fmaxf(hi, v[r]);
            }
            const unsigned klo = run_reduce<false>(fkey(lo), rg);
            const unsigned khi = run_reduce<true>(fkey(hi), rg);
            if ((tid & (rg - 1)) == 0) {
                atomicMin(&red_min[it & 1][tl], klo);
                atomicMax(&red_max[it & 1][tl], khi);
            }
        } else {
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < kE; ++r) m = fmaxf(m, fabsf(v[r]));
            // m >= 0: its bits order as unsigned integers
            const unsigned km = run_reduce<true>(__float_as_uint(m), rg);
            if ((tid & (rg - 1)) == 0) atomicMax(&red_max[it & 1][tl], km);
        }
        lds_barrier();  // B2: statistic complete, next token staged
        const float amax = __uint_as_float(red_max[it & 1][tl]);

        uint32_t nib[kE];
        float sc = 0.0f, zp = 0.0f;
        if constexpr (QK == 2) {
            // s = fl32(d / 15), inv = fl32(15 / d), z = clamp(-rne(fl32(lo inv)), 0, 15),
            // q = clamp(rne(fl32(u inv)) + z, 0, 15); the float sum is exact
            // wherever the clamp does not bind
            const float lo = fkey_inv(red_min[it & 1][tl]);
            const float hi = fkey_inv(red_max[it & 1][tl]);
            const float d = hi - lo;
            if (d != 0.0f) {
                const float inv = 15.0f / d;
                sc = d / 15.0f;
                const float zr = rintf(lo * inv);
                zp = zr > 0.0f ? 0.0f : (zr < -15.0f ? 15.0f : -zr);
#pragma unroll
                for (int r = 0; r < kE; ++r) {
                    const float t = fminf(fmaxf(rintf(v[r] * inv) + zp, 0.0f), 15.0f);
                    nib[r] = (uint32_t)t;
                }
            } else {
#pragma unroll
                for (int r = 0; r < kE; ++r) nib[r] = 0u;
            }
        } else if constexpr (QK == 0) {
            // q = rne(fl32(u * inv)) lands in [-7, 7]: |u * inv| <= fl32(7 (1 + 2^-24)) = 7,
            // so no clamp is needed.  Adding 1.5 * 2^23 + 8 (even) rounds to
            // an integer, nearest-even, and leaves q + 8 in bits 0..3 with
            // bits 4..21 clear.
            const float inv = amax > 0.0f ? 7.0f / amax : 0.0f;
#pragma unroll
            for (int r = 0; r < kE; ++r) {
                const float mq = v[r] * inv;
                nib[r] = __float_as_uint(mq + 12582920.0f);   // q + 8 in bits 0..3
            }
            sc = amax > 0.0f ? amax / 7.0f : 0.0f;
        } else {
            // exact squared norm on the grid 2^(2E - 36), E = ilogb(max |u|)
            const int E = amax > 0.0f ? ilogbf(amax) : 0;
            unsigned long long s = 0;
            if (amax > 0.0f) {
#pragma unroll
                for (int r = 0; r < kE; ++r) {
                    const double sq = (double)v[r] * (double)v[r];
                    s += (unsigned long long)rint(ldexp(sq, 36 - 2 * E));
                }
            }
            for (int off = 1; off < grp; off <<= 1) s += __shfl_xor(s, off, 64);
            if ((tid & (grp - 1)) == 0 && s) atomicAdd(&red_sum[it & 1][tl], s);
            lds_barrier();  // B3
            const unsigned long long S = red_sum[it & 1][tl];
            if (amax > 0.0f) {
                const double d = ldexp((double)S, 2 * E - 36);
                const float g = (float)sqrt((double)K / d);
                sc = (float)sqrt(d / (double)K);
#pragma unroll
                for (int r = 0; r < kE; ++r) {
                    const float x = v[r] * g;
                    uint32_t idx = 0;
                    if (a.th_sym) {
                        // Symmetric book: for x > 0 the eight thresholds up to
                        // th[7] = 0 lie below x; for x <= 0, th[i] < x exactly
                        // when th[14 - i] > |x|, and th[j] <= |x| exactly when
                        // th[j] < nextup(|x|).  Seven compares either way.
                        const float ax = fabsf(x);
                        const float vv = x > 0.0f ? ax : __uint_as_float(__float_as_uint(ax) + 1u);
                        uint32_t c = 0;
#pragma unroll
                        for (int j = 8; j < 15; ++j) c += (vv > a.th[j]) ? 1u : 0u;
                        idx = x > 0.0f ? 8u + c : 7u - c;
                    } else {
#pragma unroll
                        for (int i = 0; i < 15; ++i) idx += (x > a.th[i]) ? 1u : 0u;
                    }
                    nib[r] = idx;
                }
            } else {
#pragma unroll
                for (int r = 0; r < kE; ++r) nib[r] = 0u;
            }
        }

        // pack: register bit 0 carries index bit 0, so registers (2m, 2m + 1)
        // hold a nibble pair; bits 4..7 of every code word are clear
        uint4 chunk = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (Plan<L>::NP == 1) {
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t x = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) x |= (nib[8 * q + e] & 0xFu) << (4 * e);
                w[q] = x;
            }
            chunk = make_uint4(w[0], w[1], w[2], w[3]);
            if (grouped) *reinterpret_cast<uint4 *>(cs + 16 * tt) = chunk;
        } else {
            uint8_t *p = cs + cpad<L>(pbase<L, PL>(tt) >> 1);
#pragma unroll
            for (int mm = 0; mm < kE / 2; ++mm)
                p[Plan<L>::roff(PL, 2 * mm) >> 1] = (uint8_t)(nib[2 * mm] | (nib[2 * mm + 1] << 4));
            if (a.codes || (a.codes_mma && !grouped)) {
                // the 16 bytes this thread stores were written by lanes of its
                // own wave (its RPBH block): order the LDS writes before the read
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                chunk = *reinterpret_cast<const uint4 *>(cs + cpad<L>(16 * tt));
            }
        }
        if (valid) {
            if (a.codes)
                *reinterpret_cast<uint4 *>(a.codes + tok * (int64_t)(K / 2) + 16 * tt) =
                    make_uint4(chunk.x ^ kCanonFlip, chunk.y ^ kCanonFlip, chunk.z ^ kCanonFlip,
                               chunk.w ^ kCanonFlip);
            if constexpr (QK != 1)
                if (a.codes_mma && !grouped) store_chunk_mma(a.codes_mma, tok, a.mma_stages, tt, chunk, 0u);
            if (tt == 0) {
                a.scale[tok] = sc;
                if constexpr (QK == 2) a.scale[a.T + tok] = zp;
            }
        }
        base = next;
    }
    if (grouped && it > 0) {
        lds_barrier();
        flush(vb + (int64_t)((it - 1) >> a.ipg_log2) * gridDim.x);
    }
}

int g_num_cus = 0;

int num_cus() {
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            g_num_cus = n;
        else
            g_num_cus = 256;
    }
    return g_num_cus;
}

template <int L, bool BF16, int QK>
hipError_t launch_L(RpbhArgs a, hipStream_t s) {
    const int xb = BF16 ? 2 : 4;
    const size_t per_tok = (size_t)a.K * xb + 4 * (size_t)xwords<L>(a.K);
    const size_t slot_bytes = (size_t)((cbytes<L>(a.K) + 15) & ~15);
    // the dynamic LDS a workgroup may take (160 KB less the static arrays)
    constexpr size_t kLdsMax = 159 * 1024;
    // MMA-layout codes are written per group of >= 4 consecutive tokens when
    // the group's code slots fit, else per token
    const bool grouped = QK != 1 && a.codes_mma != nullptr && per_tok + 4 * slot_bytes <= kLdsMax;
    a.grouped = grouped ? 1 : 0;
    // per-token code staging: the regrouping exchange (blocks > 32), or the
    // group's slots
    const size_t slot = (L <= 5 && !grouped) ? 0 : slot_bytes;
    auto group_of = [&](int tpw) { return grouped && tpw < 4 ? 4 : tpw; };
    auto lds_of = [&](int tpw) { return per_tok * tpw + slot * group_of(tpw); };
    auto kern = rpbh_quant_kernel<L, BF16, QK>;
    // waves one SIMD holds given the kernel's registers (512 per lane)
    static int simd_waves = 0;
    if (simd_waves == 0) {
        hipFuncAttributes fa;
        int w = 2;
        if (hipFuncGetAttributes(&fa, (const void *)kern) == hipSuccess && fa.numRegs > 0) {
            w = 512 / ((fa.numRegs + 7) & ~7);
            w = w < 1 ? 1 : (w > 8 ? 8 : w);
        }
        simd_waves = w;
    }
    // Tokens per workgroup (<= 768 or 512 threads, <= 159 KB of LDS) and workgroups
    // per CU (as many as LDS and registers allow, or fewer).  A workgroup of
    // w waves puts ceil(w / 4) of them on some SIMD, and co-resident
    // workgroups are counted as landing on the same SIMDs (a pair of six-wave
    // workgroups at three waves per SIMD was measured not to co-reside).
    // Every workgroup stays resident and loops over groups.  The candidate
    // with the fewest tokens on the busiest CU wins, counting a CU that runs
    // several workgroups at once as kOverlap times as fast per workgroup as
    // one that runs a single one; ties go to more waves per CU, then to the
    // larger workgroup (fewer barriers per token).
    const int cus = num_cus();
    int best_tpw = 1, best_occ = 1, best_waves = 0;
    double best_cost = -1.0;
    for (int tpw = 1; tpw <= kMaxTpw; tpw *= 2) {
        if (tpw > 1 && (tpw * a.tpt > kMaxThreads<BF16> || lds_of(tpw) > kLdsMax)) break;
        const int wpw = (tpw * a.tpt + 63) / 64;
        int occ_max = (int)((160 * 1024) / (lds_of(tpw) + 1024));
        const int by_regs = simd_waves / ((wpw + 3) / 4);
        if (occ_max > by_regs) occ_max = by_regs;
        if (occ_max < 1) occ_max = 1;
        const int gs = group_of(tpw);
        const int64_t groups = (a.T + gs - 1) / gs;
        for (int occ = 1; occ <= occ_max; ++occ) {
            const int64_t wgs = (int64_t)cus * occ;
            const int64_t load = (int64_t)occ * ((groups + wgs - 1) / wgs) * gs;
            const double cost = (double)load * (occ > 1 ? kOverlap : 1.0);
            const int waves = occ * wpw;
            if (best_cost < 0 || cost < best_cost || (cost == best_cost && waves >= best_waves)) {
                best_cost = cost;
                best_waves = waves;
                best_tpw = tpw;
                best_occ = occ;
            }
        }
    }
    a.tpw = best_tpw;
    const int gs = group_of(best_tpw);
    a.gsz_log2 = ilog2(gs);
    a.ipg_log2 = ilog2(gs / best_tpw);
    a.ngroups = (a.T + gs - 1) / gs;
    const size_t lds = lds_of(best_tpw);
    const int64_t resident = (int64_t)cus * best_occ;
    const int grid = (int)(a.ngroups < resident ? a.ngroups : resident);
    // raise the dynamic-LDS limit once per instantiation (the call is not free)
    static size_t lds_set = 0;
    if (lds > 64 * 1024 && lds > lds_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_set = lds;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(a.tpw * a.tpt), lds, s, a);
    return hipGetLastError();
}

template <bool BF16, int QK>
hipError_t dispatch(int L, RpbhArgs a, hipStream_t s) {
    switch (L) {
        case 1: return launch_L<1, BF16, QK>(a, s);
        case 2: return launch_L<2, BF16, QK>(a, s);
        case 3: return launch_L<3, BF16, QK>(a, s);
        case 4: return launch_L<4, BF16, QK>(a, s);
        case 5: return launch_L<5, BF16, QK>(a, s);
        case 6: return launch_L<6, BF16, QK>(a, s);
        case 7: return launch_L<7, BF16, QK>(a, s);
        case 8: return launch_L<8, BF16, QK>(a, s);
        case 9: return launch_L<9, BF16, QK>(a, s);
        case 10: return launch_L<10, BF16, QK>(a, s);
        default: return hipErrorInvalidValue;
    }
}

RpbhArgs make_args(const void *X, int64_t T, int K, const int8_t *sign, const int32_t *perm,
                   uint8_t *codes, uint8_t *codes_mma, float *scale) {
    RpbhArgs a;
    a.X = X;
    a.T = T;
    a.K = K;
    a.tpt = K / kE;
    a.tpw = 1;
    a.sign = sign;
    a.perm = perm;
    a.codes = codes;
    a.codes_mma = codes_mma;
    a.mma_stages = (K + 127) / 128;
    a.grouped = 0;
    a.gsz_log2 = a.ipg_log2 = 0;
    a.ngroups = 0;
    a.scale = scale;
    for (int i = 0; i < 15; ++i) a.th[i] = 0.0f;
    a.th_sym = 0;
    return a;
}

}  // namespace

int launch_rpbh_int4(const void *X, int x_bf16, int64_t T, int K, int block, const int8_t *sign,
                     const int32_t *perm, uint8_t *codes, uint8_t *codes_mma, float *scale,
                     int asym, void *stream) {
    RpbhArgs a = make_args(X, T, K, sign, perm, codes, codes_mma, scale);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int L = ilog2(block);
    if (asym) return (int)(x_bf16 ? dispatch<true, 2>(L, a, s) : dispatch<false, 2>(L, a, s));
    return (int)(x_bf16 ? dispatch<true, 0>(L, a, s) : dispatch<false, 0>(L, a, s));
}

int launch_rpbh_lloydmax(const void *X, int x_bf16, int64_t T, int K, int block,
                         const int8_t *sign, const int32_t *perm, const float *thresholds,
                         int n_thresholds, uint8_t *codes, float *sigma, void *stream) {
    if (n_thresholds != 15) return (int)hipErrorInvalidValue;
    RpbhArgs a = make_args(X, T, K, sign, perm, codes, nullptr, sigma);
    for (int i = 0; i < 15; ++i) a.th[i] = thresholds[i];
    // ascending thresholds of a book symmetric about 0 (exact float equality)
    a.th_sym = a.th[7] == 0.0f ? 1 : 0;
    for (int i = 0; i < 15; ++i)
        if (a.th[i] != -a.th[14 - i] || (i > 0 && a.th[i] < a.th[i - 1])) a.th_sym = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int L = ilog2(block);
    return (int)(x_bf16 ? dispatch<true, 1>(L, a, s) : dispatch<false, 1>(L, a, s));
}

}  // namespace rq

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
//            and every element is written to LDS at its destination
//            coordinate's slot (the permutation as a scatter of 2- or 4-byte
//            stores, which the wave does not wait on);
//   gather   each thread reads its 32 consecutive coordinates of one block
//            (see lane_hbits) as 16-byte pieces, laid out so that adjacent
//            lanes read adjacent pieces;
//   stages   index bits 0..4 of the block in registers, bits 5 .. L - 1
//            across the block's adjacent lanes, one fused multiply-add per
//            value with the partner lane's register as a DPP operand (no LDS
//            exchange); those lanes end with their values negated, which the
//            quantizer folds into its scale;
//   stat     per-token absmax (asymmetric: min and max; for the codebook
//            also the exact integer-grid squared norm) by shuffles and one
//            LDS atomic per lane group;
//   codes    packed from registers, 16 bytes per 32 coordinates; the
//            canonical layout is stored with one 16-byte store per thread.  For the
//            GEMM's FP6 fragment layout (rq_fp6.h) a workgroup takes its
//            tokens in groups of at least four consecutive ones, keeps the
//            group's codes in LDS, and once the group is complete spreads
//            them so that the four tokens' 16-byte slots of one piece -- 64
//            contiguous bytes -- come from four adjacent lanes: whole-request
//            stores instead of sixteen-byte writes to scattered lines.
// One workgroup barrier per iteration of `tpw` tokens (two for the
// codebook): each token has two staging rows, used by alternate
// iterations.  A per-workgroup prologue reads perm and sign and builds, in
// LDS, each source element's destination slot and sign.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstring>

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

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its global loads and stores (a __syncthreads() would
// also drain the next token's prefetch and the code stores in flight).
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Layout of a block in a thread's registers.  The block's 2^L coordinates
// are split over 2^NB adjacent lanes (NB = L - 5 lane bits, none for L <= 5)
// and 32 registers: index bits 0..4 are the register index r, and the high
// bits h = index bits 5 .. L - 1 sit on the lane.  Index bit 5 + t maps to
// the lane mask m_t = 1, 2, 7, 8, 16 (t = 0 .. 4): the lane of h within the
// block is the XOR of m_t over the set bits h_t.  The two butterfly partners
// of index bit 5 + t then sit in the same register of lanes l and l ^ m_t,
// which a data-parallel-primitive operand reaches inside a row of 16 lanes
// (quad swaps for 1 and 2, the half-row mirror for 7, a rotation by 8 for 8)
// and a swizzle for 16.  Every thread thus holds 32 consecutive coordinates
// of its block, chunk 32 h .. 32 h + 31.
template <int L>
constexpr int kLaneBits = L > 5 ? L - 5 : 0;

// h of lane position l (0 .. 2^NB - 1) inside the block: the inverse of the
// mask map (only m_2 = 7 has bit 2 set; bits 0 and 1 of l mix h_0, h_1 with it)
__host__ __device__ constexpr int lane_hbits(int l) {
    const int h2 = (l >> 2) & 1;
    return (l & ~7) | (h2 << 2) | ((((l >> 1) & 1) ^ h2) << 1) | ((l & 1) ^ h2);
}

// the token-relative 32-coordinate chunk that thread tt holds
template <int L>
__device__ inline int chunk_of(int tt) {
    constexpr int NB = kLaneBits<L>;
    if constexpr (NB == 0) {
        return tt;
    } else {
        const int l = tt & ((1 << NB) - 1);
        return (tt - l) | lane_hbits(l);
    }
}

// Butterfly stages on index bits 0 .. min(L, 5) - 1, inside the registers.
template <int L>
__device__ inline void reg_stages(float (&v)[kE]) {
#pragma unroll
    for (int kb = 0; kb < (L < 5 ? L : 5); ++kb) {
#pragma unroll
        for (int r = 0; r < kE; ++r) {
            if (r & (1 << kb)) continue;
            const float lo = v[r], hi = v[r | (1 << kb)];
            v[r] = lo + hi;
            v[r | (1 << kb)] = lo - hi;
        }
    }
}

// One butterfly stage across lanes, on every register: v = partner * c + v
// with one v_fmac_f32 whose first operand is the partner lane's register
// (a DPP operand).  c = +1 on the lane that holds the lower coordinate (its
// index bit is 0), which gets fl(lo + hi) exactly as the pinned butterfly;
// c = -1 on the other lane, which gets fl(hi - lo) = -fl(lo - hi), the
// butterfly's result negated (the product by -1 is exact and the sum is
// rounded once).  The negations are tracked per lane (see lane_sign): a
// partner pair always carries the same accumulated sign, so every stage takes
// the same form.  Hazard: a DPP read needs two wait states after a VALU write
// of its register.  s_nop 1 gives the block's first instruction two, and
// instruction k of the block reads at least k + 2 wait states after anything
// written before the block; inside the block every instruction reads a
// register that no earlier instruction of the block wrote.
#define RQ_FMAC_DPP(n, ctrl) "v_fmac_f32_dpp %" #n ", %" #n ", %32 " ctrl " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define RQ_FMAC_DPP8(a, b, c, d, e, f, g, h, ctrl)                                                     \
    RQ_FMAC_DPP(a, ctrl) RQ_FMAC_DPP(b, ctrl) RQ_FMAC_DPP(c, ctrl) RQ_FMAC_DPP(d, ctrl) RQ_FMAC_DPP(e, ctrl) \
        RQ_FMAC_DPP(f, ctrl) RQ_FMAC_DPP(g, ctrl) RQ_FMAC_DPP(h, ctrl)
#define RQ_FMAC_DPP32(ctrl)                                                                          \
    "s_nop 1\n\t" RQ_FMAC_DPP8(0, 1, 2, 3, 4, 5, 6, 7, ctrl) RQ_FMAC_DPP8(8, 9, 10, 11, 12, 13, 14, 15, ctrl) \
        RQ_FMAC_DPP8(16, 17, 18, 19, 20, 21, 22, 23, ctrl) RQ_FMAC_DPP8(24, 25, 26, 27, 28, 29, 30, 31, ctrl)
#define RQ_V32                                                                                        \
    "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),     \
        "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),     \
        "+v"(v[15]), "+v"(v[16]), "+v"(v[17]), "+v"(v[18]), "+v"(v[19]), "+v"(v[20]), "+v"(v[21]),   \
        "+v"(v[22]), "+v"(v[23]), "+v"(v[24]), "+v"(v[25]), "+v"(v[26]), "+v"(v[27]), "+v"(v[28]),   \
        "+v"(v[29]), "+v"(v[30]), "+v"(v[31])
static_assert(kE == 32, "the lane stages are written for 32 registers");

template <int T>
__device__ inline void lane_stage(float (&v)[kE], float c) {
    if constexpr (T == 0) {
        asm volatile(RQ_FMAC_DPP32("quad_perm:[1,0,3,2]") : RQ_V32 : "v"(c));
    } else if constexpr (T == 1) {
        asm volatile(RQ_FMAC_DPP32("quad_perm:[2,3,0,1]") : RQ_V32 : "v"(c));
    } else if constexpr (T == 2) {
        asm volatile(RQ_FMAC_DPP32("row_half_mirror") : RQ_V32 : "v"(c));
    } else if constexpr (T == 3) {
        asm volatile(RQ_FMAC_DPP32("row_ror:8") : RQ_V32 : "v"(c));
    } else {
        // lane ^ 16 inside each 32-lane half: swizzle, bit mode (and 0x1F, xor 0x10)
#pragma unroll
        for (int r = 0; r < kE; ++r) {
            const float p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[r]), 0x401F));
            v[r] = __builtin_fmaf(p, c, v[r]);
        }
    }
}
#undef RQ_V32
#undef RQ_FMAC_DPP32
#undef RQ_FMAC_DPP8
#undef RQ_FMAC_DPP

// the stages on index bits 5 .. L - 1, in order; coef[t] = -1 on the lane
// whose h_t is set, else +1
template <int L>
__device__ inline void lane_stages(float (&v)[kE], const float (&coef)[5]) {
    constexpr int NB = kLaneBits<L>;
    static_assert(NB <= 5, "block too large");
    if constexpr (NB > 0) lane_stage<0>(v, coef[0]);
    if constexpr (NB > 1) lane_stage<1>(v, coef[1]);
    if constexpr (NB > 2) lane_stage<2>(v, coef[2]);
    if constexpr (NB > 3) lane_stage<3>(v, coef[3]);
    if constexpr (NB > 4) lane_stage<4>(v, coef[4]);
}

// After the lane stages a lane holds sign * u: -1 when an odd number of h
// bits is set (each set bit negated the lane's values once).
__device__ inline float lane_sign(int h) { return (__popc((unsigned)h) & 1) ? -1.0f : 1.0f; }

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
    float *scale;         // s or sigma [T]; asymmetric: s [T] then z [T];
                          // MXFP4: E8M0 codes uint8 [T][K/32] (or null)
    int mx_tiles;         // MXFP4: ceil(T / 32) (tiled codes_mma layout)
    float th[15];         // codebook thresholds (Lloyd-Max)
    int th_sym;           // th[7] == 0 and th[i] == -th[14 - i] exactly
    uint32_t lev[16];     // Lloyd-Max: bf16 bits of the 16 levels (codes_mma)
    float qbyte;          // byte codes: symmetric qmax (31 or 127) or asymmetric
                          // top code (63 or 255) of 6- or 8-bit codes
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
    // QK: 0 symmetric 4-bit, 1 Lloyd-Max, 2 asymmetric 4-bit, 3 MXFP4,
    //     4 symmetric 8-bit, 5 asymmetric 8-bit
    constexpr bool ASYM = QK == 2 || QK == 5;
    constexpr bool MX = QK == 3;
    constexpr bool B8 = QK == 4 || QK == 5;
    constexpr int CSH = B8 ? 0 : 1;   // code byte = coordinate >> CSH
    const float kLevels = QK == 5 ? a.qbyte : 15.0f;   // asymmetric top code
    constexpr uint32_t kCanonFlip = QK == 0 ? 0x88888888u : 0u;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // per-token statistics, three slots in rotation: iteration it reduces into
    // slot it % 3 and clears slot (it + 1) % 3, last read two barriers earlier
    __shared__ unsigned red_max[3][kMaxTpw];
    __shared__ unsigned red_min[3][kMaxTpw];   // asymmetric INT4 (keys)
    __shared__ unsigned long long red_sum[3][kMaxTpw];
    // Lloyd-Max with codes_mma: packed byte of two indices -> their two bf16 levels
    __shared__ uint32_t lev_pair[QK == 1 ? 256 : 1];
    const int K = a.K;
    const int tid = threadIdx.x;
    const int tl = tid / a.tpt;
    const int tt = tid - tl * a.tpt;
    // two staging rows per token, used by alternate iterations: the next
    // token is staged while this one is gathered, without a barrier between
    uint8_t *const xs0 = smem + (size_t)tl * K * S::XB;
    uint8_t *const xs1 = xs0 + (size_t)a.tpw * K * S::XB;
    const int cb = ((K >> CSH) + 15) & ~15;
    // code staging (MMA layout, grouped): one slot per token of the group,
    // two sets used by alternate groups
    uint8_t *const cs0 = smem + (size_t)2 * a.tpw * K * S::XB;
    // the 32-coordinate chunk this thread holds, its lane's high index bits,
    // the lane stages' coefficients and the lane's final sign
    const int qc = chunk_of<L>(tt);
    constexpr int NB = kLaneBits<L>;
    const int hb = NB ? (qc & ((1 << NB) - 1)) : 0;
    float coef[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) coef[t] = ((hb >> t) & 1) ? -1.0f : 1.0f;
    const float lsign = lane_sign(hb);

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
    if constexpr (QK == 1) {
        // (visible to every thread after the prologue's barriers)
        for (int i = tid; i < 256; i += blockDim.x) lev_pair[i] = a.lev[i & 15] | (a.lev[i >> 4] << 16);
    }

    // ---- prologue: scatter offsets, source-side sign masks ----------------
    // Thread tt owns destination coordinates j = 32 qc + r: it reads perm[j]
    // and sign[j] contiguously.  A table in the first token's staging row
    // holds one entry per source element, so that the entries covering a
    // staged 16-byte chunk are the 16 bytes at the chunk's own position: for
    // source element perm[j], the LDS offset of coordinate j in the gather
    // layout, and in the element's own sign bit (bf16 bit 15, fp32 bit 31)
    // the sign that it must carry.  An offset is below K * XB (K <= 16384):
    // bf16 offsets are even and below 32 KB, so 15 bits hold them halved;
    // fp32 offsets take 16 bits.  Only the first token's threads write the
    // table; every thread then reads its staged chunks' entries.
    //
    // Gather layout: the 16-byte piece c of chunk qc (coordinates 32 qc +
    // E c .. + E - 1, E coordinates per piece) sits at piece slot c nch + qc,
    // so piece c of all chunks is one contiguous array and the gather's
    // 16-byte reads of adjacent lanes are adjacent.
    constexpr int EPC = S::ELEMS_PER_CHUNK;
    const int nch = a.tpt;   // 32-coordinate chunks per token
    int dofs[kE];            // LDS offset of each staged element's destination
    uint32_t smask[S::WORDS];
    {
        if (tl == 0) {
#pragma unroll
            for (int r = 0; r < kE; r += 16) {
                int pj[16];
#pragma unroll
                for (int e = 0; e < 16; e += 4) {
                    const int4 p4 = *reinterpret_cast<const int4 *>(a.perm + kE * qc + r + e);
                    pj[e] = p4.x;
                    pj[e + 1] = p4.y;
                    pj[e + 2] = p4.z;
                    pj[e + 3] = p4.w;
                }
                const int4 s4 = *reinterpret_cast<const int4 *>(a.sign + kE * qc + r);
                const int w[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const bool neg = (int8_t)(w[e >> 2] >> (8 * (e & 3))) < 0;
                    const int rr = r + e;
                    const uint32_t off = 16u * (uint32_t)((rr / EPC) * nch + qc) + S::XB * (rr % EPC);
                    if constexpr (BF16)
                        *reinterpret_cast<uint16_t *>(smem + 2 * pj[e]) = (uint16_t)((off >> 1) | (neg ? 0x8000u : 0u));
                    else
                        *reinterpret_cast<uint32_t *>(smem + 4 * pj[e]) = off | (neg ? 0x80000000u : 0u);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < S::CHUNKS; ++q) {
            const uint4 m = *reinterpret_cast<const uint4 *>(smem + (size_t)16 * (tt + q * a.tpt));
            const uint32_t w[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (BF16) {
                    smask[4 * q + k] = w[k] & 0x80008000u;
                    dofs[8 * q + 2 * k] = (int)((w[k] & 0x7FFFu) << 1);
                    dofs[8 * q + 2 * k + 1] = (int)((w[k] >> 15) & 0xFFFEu);
                } else {
                    smask[4 * q + k] = w[k] & 0x80000000u;
                    dofs[4 * q + k] = (int)(w[k] & 0xFFFFu);
                }
            }
        }
        __syncthreads();
    }

    // the staged row: each element, its destination's sign applied (one XOR
    // per 32-bit word), written to its destination's slot of the gather layout
    auto stage = [&](uint8_t *xs) {
#pragma unroll
        for (int q = 0; q < S::CHUNKS; ++q) {
            const uint32_t w[4] = {pre[q].x ^ smask[4 * q], pre[q].y ^ smask[4 * q + 1],
                                   pre[q].z ^ smask[4 * q + 2], pre[q].w ^ smask[4 * q + 3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (BF16) {
                    *reinterpret_cast<uint16_t *>(xs + dofs[8 * q + 2 * k]) = (uint16_t)w[k];
                    *reinterpret_cast<uint16_t *>(xs + dofs[8 * q + 2 * k + 1]) = (uint16_t)(w[k] >> 16);
                } else {
                    *reinterpret_cast<uint32_t *>(xs + dofs[4 * q + k]) = w[k];
                }
            }
        }
    };
    if (base >= 0) {
        stage(xs0);
        const int64_t b1 = first_tok(1);
        if (b1 >= 0) fetch(b1);
    }
    if (tt == 0) {
        red_max[0][tl] = 0u;
        if constexpr (QK == 1) red_sum[0][tl] = 0ull;
        if constexpr (ASYM) red_min[0][tl] = 0xFFFFFFFFu;
    }
    __syncthreads();

    // MMA-layout codes of group g (complete in slot set `set`, LDS writes
    // ordered by a barrier): item i is (stage s, half h) = (i >> gsz_log2)
    // and token j = i % group size, so four adjacent lanes write one 64-byte
    // run.  A group (at most 16 tokens, aligned) lies inside one 32-token tile.
    auto flush = [&](int64_t g, int set) {
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
            const uint8_t *slot = cs0 + (size_t)((set << a.gsz_log2) + j) * cb;
            // chunks c0 (k-step 0) and c1 (k-step 1); those past the last
            // coordinate are not written
            const int c0 = 2 * (sh & ~1) + (sh & 1), c1 = c0 + 2;
            if (c0 >= nch) continue;
            const uint4 w0 = *reinterpret_cast<const uint4 *>(slot + 16 * c0);
            const uint4 w1 = c1 < nch ? *reinterpret_cast<const uint4 *>(slot + 16 * c1)
                                      : make_uint4(0u, 0u, 0u, 0u);
            store_pair_mma_in_tile(tile, sh >> 1, t32 + j, sh & 1, w0, w1, c1 < nch, 0u);
        }
    };
    const bool grouped = (QK == 0 || QK == 2) && a.grouped;

    // lane groups of one token for the shuffle reductions
    int grp = 64;
    while (a.tpt % grp) grp >>= 1;
    // the same runs cut to one row of 16 lanes (max / min reductions)
    const int rg = grp < 16 ? grp : 16;

    // Per iteration one barrier (B, two for the codebook).  Iteration it
    // gathers row it % 2, stages the next token into the other row (gathered
    // at it + 1, after B; restaged at it + 2, after this iteration's B, so
    // after every gather of this one), reduces into statistic slot it % 3,
    // and after B quantizes and writes the codes.
    int it = 0, rs = 0;   // rs = it % 3
    for (; base >= 0; ++it) {
        const int64_t tok = base + tl;
        const bool valid = tok < a.T;
        const int rn = rs == 2 ? 0 : rs + 1;
        uint8_t *const xg = (it & 1) ? xs1 : xs0;
        uint8_t *const cs =
            cs0 + (size_t)((((it >> a.ipg_log2) & 1) << a.gsz_log2) + (it & ipg_mask) * a.tpw + tl) * cb;
        if (tt == 0) {
            red_max[rn][tl] = 0u;
            if constexpr (QK == 1) red_sum[rn][tl] = 0ull;
            if constexpr (ASYM) red_min[rn][tl] = 0xFFFFFFFFu;
        }
        // gather: the thread's 32 coordinates, in 16-byte pieces
        float v[kE];
#pragma unroll
        for (int c = 0; c < kE / EPC; ++c) {
            const uint4 m = *reinterpret_cast<const uint4 *>(xg + (size_t)16 * (c * nch + qc));
            const uint32_t w[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (BF16) {
                    v[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
                    v[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                } else {
                    v[4 * c + k] = __uint_as_float(w[k]);
                }
            }
        }
        reg_stages<L>(v);
        const int64_t next = first_tok(it + 1);
        if (next >= 0) {
            stage((it & 1) ? xs0 : xs1);                    // next token -> LDS
            const int64_t b2 = first_tok(it + 2);
            if (b2 >= 0) fetch(b2);
        }
        // v = lsign * u from here on (coordinates 32 qc .. 32 qc + 31)
        lane_stages<L>(v, coef);
        if constexpr (ASYM) {
            float lo = v[0], hi = v[0];
#pragma unroll
            for (int r = 1; r < kE; ++r) {
                lo = fminf(lo, v[r]);
                hi = fmaxf(hi, v[r]);
            }
            if (lsign < 0.0f) {
                const float t = lo;
                lo = -hi;
                hi = -t;
            }
            const unsigned klo = run_reduce<false>(fkey(lo), rg);
            const unsigned khi = run_reduce<true>(fkey(hi), rg);
            if ((tid & (rg - 1)) == 0) {
                atomicMin(&red_min[rs][tl], klo);
                atomicMax(&red_max[rs][tl], khi);
            }
        } else if constexpr (!MX) {
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < kE; ++r) m = fmaxf(m, fabsf(v[r]));
            // m >= 0: its bits order as unsigned integers
            const unsigned km = run_reduce<true>(__float_as_uint(m), rg);
            if ((tid & (rg - 1)) == 0) atomicMax(&red_max[rs][tl], km);
        }
        lds_barrier();  // B: statistic complete, next token staged
        // the previous group is complete (its codes were written before B)
        // and the codes written from here on go to the other slot set
        if (grouped && it > 0 && (it & ipg_mask) == 0) {
            const int gl = (it - 1) >> a.ipg_log2;
            flush(vb + (int64_t)gl * gridDim.x, gl & 1);
        }
        const float amax = __uint_as_float(red_max[rs][tl]);

        uint32_t nib[kE];   // the codes: nibbles, or bytes for 8-bit codes
        // The token's scale is stored by its first thread only, so only that
        // wave divides: s = snum / sden (0 when snum = 0), or for the
        // codebook sigma = sqrt(dn / K).
        float snum = 0.0f, sden = 1.0f, zp = 0.0f;
        double dn = 0.0;
        uint32_t mxsc = 0u;  // MXFP4: E8M0 code of this thread's block
        uint32_t mxw[4];     // MXFP4: the block's 32 codes, two per byte
        if constexpr (ASYM) {
            // L = 15 or 255: s = fl32(d / L), inv = fl32(L / d),
            // z = clamp(-rne(fl32(lo inv)), 0, L), q = clamp(rne(fl32(u inv)) + z, 0, L);
            // the float sum is exact wherever the clamp does not bind
            const float lo = fkey_inv(red_min[rs][tl]);
            const float hi = fkey_inv(red_max[rs][tl]);
            const float d = hi - lo;
            if (d != 0.0f) {
                const float inv = kLevels / d;
                snum = d;
                sden = kLevels;
                // z is the integer -rne(lo inv) clamped to [0, L], as a float;
                // rne(lo inv) = -0 or +0 (a row whose minimum is at most s / 2
                // from zero) gives z = +0
                const float zr = rintf(lo * inv);
                zp = zr >= 0.0f ? 0.0f : (zr < -kLevels ? kLevels : -zr);
                // v = lsign u, so v (lsign inv) = fl32(u inv) (the sign flip is exact)
                const float sinv = lsign * inv;
#pragma unroll
                for (int r = 0; r < kE; ++r) {
                    const float t = fminf(fmaxf(rintf(v[r] * sinv) + zp, 0.0f), kLevels);
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
            const float sinv = lsign * inv;   // v = lsign u
#pragma unroll
            for (int r = 0; r < kE; ++r) {
                const float mq = v[r] * sinv;
                nib[r] = __float_as_uint(mq + 12582920.0f);   // q + 8 in bits 0..3
            }
            snum = amax;
            sden = 7.0f;
        } else if constexpr (QK == 4) {
            // q = rne(fl32(u * inv)) in [-qm, qm] (|u * inv| <= fl32(qm (1 + 2^-24))
            // rounds to at most qm); adding 1.5 * 2^23 leaves q in the low
            // mantissa bits, whose low byte is q in two's complement
            const float qm = a.qbyte;   // 127 (8-bit) or 31 (6-bit)
            const float inv = amax > 0.0f ? qm / amax : 0.0f;
            const float sinv = lsign * inv;   // v = lsign u
#pragma unroll
            for (int r = 0; r < kE; ++r) nib[r] = __float_as_uint(v[r] * sinv + 12582912.0f) & 0xFFu;
            snum = amax;
            sden = qm;
        } else if constexpr (MX) {
            // this thread's 32 coordinates are one block: e = floor(log2 max|u|) - 2
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < kE; ++r) m = fmaxf(m, fabsf(v[r]));
            int e = m > 0.0f ? ilogbf(m) - 2 : -127;
            e = e < -127 ? -127 : e;
            mxsc = (uint32_t)(e + 127);
            // 2^-e (2^-125 .. 2^127, exact), times the lane's sign: v sinv =
            // u 2^-e = a, exact but for values far below E2M1's smallest step
            // (code 0 either way), and |a| < 8.  The element's E2M1 code is
            // |a| rounded to the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}, nearest
            // with ties to even, saturating at 6, with the sign of a in bit 3
            // unless the magnitude is 0.  v_cvt_scalef32_pk_fp4_f32 (scale 1)
            // rounds two values that way into byte b of a word, low nibble
            // first (checked on the device against a software encoder of the
            // rule for every fp32 value of either sign up to 16), except that
            // a value rounding to 0 may keep its sign; that sign is cleared
            // per nibble (m + 7 sets bit 3 exactly when m != 0).
            const float sinv = lsign * ldexpf(1.0f, -e);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t w = 0u;
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * q + 0] * sinv, v[8 * q + 1] * sinv, 1.0f, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * q + 2] * sinv, v[8 * q + 3] * sinv, 1.0f, 1);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * q + 4] * sinv, v[8 * q + 5] * sinv, 1.0f, 2);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * q + 6] * sinv, v[8 * q + 7] * sinv, 1.0f, 3);
                const uint32_t mag = w & 0x77777777u;
                mxw[q] = mag | (w & (mag + 0x77777777u) & 0x88888888u);
            }
        } else {
            // exact squared norm on the grid 2^(2E - 36), E = ilogb(max |u|):
            // each term rint(u^2 2^(36 - 2E)) = rint((u 2^(18 - E))^2) (both
            // the scaling and the square are exact in fp64) is an integer
            // below 2^38, so the fp64 sums of at most 16384 of them (below
            // 2^52) are exact integers in any order
            const int E = amax > 0.0f ? ilogbf(amax) : 0;
            double sd = 0.0;
            if (amax > 0.0f) {
#pragma unroll
                for (int r = 0; r < kE; ++r) {
                    const double xs = ldexp((double)v[r], 18 - E);
                    sd += rint(xs * xs);
                }
            }
            for (int off = 1; off < grp; off <<= 1) sd += __shfl_xor(sd, off, 64);
            const unsigned long long s = (unsigned long long)sd;
            if ((tid & (grp - 1)) == 0 && s) atomicAdd(&red_sum[rs][tl], s);
            lds_barrier();  // B3
            const unsigned long long S = red_sum[rs][tl];
            if (amax > 0.0f) {
                const double d = ldexp((double)S, 2 * E - 36);
                const float g = (float)sqrt((double)K / d);
                dn = d;
                const float sg = lsign * g;   // v = lsign u: x = fl32(u g)
#pragma unroll
                for (int r = 0; r < kE; ++r) {
                    const float x = v[r] * sg;
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

        // pack: the thread's 32 codes are coordinates 32 qc .. 32 qc + 31 in
        // register order; bits 4..7 (8..31) of every code word are clear
        uint4 chunk, chunk1 = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (B8) {
            uint32_t w[8];
#pragma unroll
            for (int m = 0; m < 8; ++m)
                w[m] = nib[4 * m] | (nib[4 * m + 1] << 8) | (nib[4 * m + 2] << 16) | (nib[4 * m + 3] << 24);
            chunk = make_uint4(w[0], w[1], w[2], w[3]);
            chunk1 = make_uint4(w[4], w[5], w[6], w[7]);
        } else if constexpr (MX) {
            chunk = make_uint4(mxw[0], mxw[1], mxw[2], mxw[3]);
        } else {
            // byte m = code 2m | code 2m + 1 << 4 (one shift-or: only bits
            // 0..3 of a code word and 4..7 of the shifted one reach byte 0),
            // then byte selects: two bytes per halfword, two halfwords per word
            uint32_t by[16], hw[8], w[4];
#pragma unroll
            for (int m = 0; m < 16; ++m) by[m] = (nib[2 * m + 1] << 4) | nib[2 * m];
#pragma unroll
            for (int m = 0; m < 8; ++m) hw[m] = __builtin_amdgcn_perm(by[2 * m + 1], by[2 * m], 0x0c0c0400u);
#pragma unroll
            for (int m = 0; m < 4; ++m) w[m] = __builtin_amdgcn_perm(hw[2 * m + 1], hw[2 * m], 0x05040100u);
            chunk = make_uint4(w[0], w[1], w[2], w[3]);
            if (grouped) *reinterpret_cast<uint4 *>(cs + 16 * qc) = chunk;
        }
        if (valid) {
            if (a.codes) {
                if constexpr (B8) {
                    uint4 *dst = reinterpret_cast<uint4 *>(a.codes + tok * (int64_t)K + 32 * qc);
                    dst[0] = chunk;
                    dst[1] = chunk1;
                } else {
                    *reinterpret_cast<uint4 *>(a.codes + tok * (int64_t)(K / 2) + 16 * qc) =
                        make_uint4(chunk.x ^ kCanonFlip, chunk.y ^ kCanonFlip, chunk.z ^ kCanonFlip,
                                   chunk.w ^ kCanonFlip);
                }
            }
            if constexpr (QK == 0 || QK == 2)
                if (a.codes_mma && !grouped) store_chunk_mma(a.codes_mma, tok, a.mma_stages, qc, chunk, 0u);
            if constexpr (B8) {
                // the int8 GEMM's fragment order [t / 32][k-step][lane][16 B]: the
                // thread's 32 codes are k-step qc, lanes t % 32 and t % 32 + 32
                if (a.codes_mma) {
                    uint8_t *d = a.codes_mma + (((tok >> 5) * (K / 32) + qc) * 64 + (tok & 31)) * 16;
                    *reinterpret_cast<uint4 *>(d) = chunk;
                    *reinterpret_cast<uint4 *>(d + 512) = chunk1;
                }
            }
            if constexpr (QK == 1) {
                // the levels in bf16, in the codebook GEMM's fragment order
                // [32-token tile][16-coordinate k-step][lane][16 bytes]:
                // coordinates 16 ks + 8 h .. + 7 of token t sit in lane
                // t % 32 + 32 h of k-step ks
                if (a.codes_mma) {
                    const uint32_t wq[4] = {chunk.x, chunk.y, chunk.z, chunk.w};
                    uint8_t *tile = a.codes_mma + (tok >> 5) * (int64_t)(K / 16) * 1024 + (tok & 31) * 16;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t w = wq[c];
                        const uint4 v = make_uint4(lev_pair[w & 0xFFu], lev_pair[(w >> 8) & 0xFFu],
                                                   lev_pair[(w >> 16) & 0xFFu], lev_pair[w >> 24]);
                        *reinterpret_cast<uint4 *>(tile + (2 * qc + (c >> 1)) * 1024 + 512 * (c & 1)) = v;
                    }
                }
            }
            if constexpr (MX) {
                // E8M0 code of block qc: canonical [T][K/32], and the tiled
                // copies [tile][K/32][32][16] (codes) and
                // [stage][tile][64][2] (scales) of the scaled FP4 GEMM
                const int nch = K / kE;
                if (a.scale) reinterpret_cast<uint8_t *>(a.scale)[tok * nch + qc] = (uint8_t)mxsc;
                if (a.codes_mma) {
                    const int64_t tile = tok >> 5;
                    const int row = (int)(tok & 31);
                    *reinterpret_cast<uint4 *>(a.codes_mma + ((tile * nch + qc) * 32 + row) * 16) = chunk;
                    uint8_t *mxs = a.codes_mma + (int64_t)a.mx_tiles * nch * 512;
                    mxs[(((int64_t)(qc >> 2) * a.mx_tiles + tile) * 64 + 32 * (qc & 1) + row) * 2 +
                        ((qc >> 1) & 1)] = (uint8_t)mxsc;
                }
            } else if (tt == 0) {
                float sc;
                if constexpr (QK == 1)
                    sc = (float)sqrt(dn / (double)K);
                else
                    sc = snum != 0.0f ? snum / sden : 0.0f;
                a.scale[tok] = sc;
                if constexpr (ASYM) a.scale[a.T + tok] = zp;
            }
        }
        base = next;
        rs = rn;
    }
    if (grouped && it > 0) {
        lds_barrier();
        const int gl = (it - 1) >> a.ipg_log2;
        flush(vb + (int64_t)gl * gridDim.x, gl & 1);
    }
}

template <int L, bool BF16, int QK>
hipError_t launch_L(RpbhArgs a, hipStream_t s) {
    const int xb = BF16 ? 2 : 4;
    const size_t per_tok = (size_t)a.K * xb;
    constexpr int CSH = (QK == 4 || QK == 5) ? 0 : 1;
    const size_t slot_bytes = (size_t)((((size_t)a.K >> CSH) + 15) & ~(size_t)15);
    // the dynamic LDS a workgroup may take (160 KB less the static arrays)
    constexpr size_t kLdsMax = 159 * 1024;
    // MMA-layout codes are written per group of >= 4 consecutive tokens when
    // the group's code slots fit, else per token
    const bool grouped = (QK == 0 || QK == 2) && a.codes_mma != nullptr && 2 * per_tok + 8 * slot_bytes <= kLdsMax;
    a.grouped = grouped ? 1 : 0;
    // per-token code staging: the group's slots (grouped MMA-layout codes only)
    const size_t slot = grouped ? slot_bytes : 0;
    auto group_of = [&](int tpw) { return grouped && tpw < 4 ? 4 : tpw; };
    // two staging rows per token and two sets of group slots
    auto lds_of = [&](int tpw) { return 2 * (per_tok * tpw + slot * group_of(tpw)); };
    auto kern = rpbh_quant_kernel<L, BF16, QK>;
    // waves one SIMD holds given the kernel's registers (512 per lane); the
    // same on every gfx950 device, read once (thread-safe static init)
    static const int simd_waves = [kern] {
        hipFuncAttributes fa;
        int w = 2;
        if (hipFuncGetAttributes(&fa, (const void *)kern) == hipSuccess && fa.numRegs > 0) {
            w = 512 / ((fa.numRegs + 7) & ~7);
            w = w < 1 ? 1 : (w > 8 ? 8 : w);
        }
        return w;
    }();
    // Tokens per workgroup (<= 768 or 512 threads, <= 159 KB of LDS) and workgroups
    // per CU (as many as LDS and registers allow, or fewer).  A workgroup of
    // w waves puts ceil(w / 4) of them on some SIMD, and co-resident
    // workgroups are counted as landing on the same SIMDs (a pair of six-wave
    // workgroups at three waves per SIMD was measured not to co-reside).
    // Every workgroup stays resident and loops over groups.  Cost: the tokens
    // on the busiest CU, times a per-token time that falls with the waves
    // the CU holds, as 1 / sqrt(waves / the registers' limit) (a fit to a
    // sweep of launch shapes on the 3072-wide FLUX layer).  Ties go to more
    // waves per CU, then to the larger workgroup (fewer barriers per token).
    const int cus = device_cus();
    const int max_waves = 4 * simd_waves;
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
            const int waves = occ * wpw;
            const double cost = (double)load / std::sqrt((double)(waves < max_waves ? waves : max_waves) / max_waves);
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
    // raise the dynamic-LDS limit once per kernel and device (the call is not free)
    {
        const hipError_t e = (hipError_t)ensure_dyn_lds((const void *)kern, lds);
        if (e != hipSuccess) return e;
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
    a.mx_tiles = (int)((T + 31) / 32);
    for (int i = 0; i < 15; ++i) a.th[i] = 0.0f;
    a.th_sym = 0;
    for (int i = 0; i < 16; ++i) a.lev[i] = 0u;
    a.qbyte = 0.0f;
    return a;
}

}  // namespace

int launch_rpbh_int4(const void *X, int x_bf16, int64_t T, int K, int block, const int8_t *sign,
                     const int32_t *perm, uint8_t *codes, uint8_t *codes_mma, float *scale,
                     int asym, int a_bits, void *stream) {
    RpbhArgs a = make_args(X, T, K, sign, perm, codes, codes_mma, scale);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int L = ilog2(block);
    if (a_bits != 4) {
        // 6- or 8-bit codes, one per byte
        a.qbyte = asym ? (float)((1 << a_bits) - 1) : (float)((1 << (a_bits - 1)) - 1);
        if (asym) return (int)(x_bf16 ? dispatch<true, 5>(L, a, s) : dispatch<false, 5>(L, a, s));
        return (int)(x_bf16 ? dispatch<true, 4>(L, a, s) : dispatch<false, 4>(L, a, s));
    }
    if (asym) return (int)(x_bf16 ? dispatch<true, 2>(L, a, s) : dispatch<false, 2>(L, a, s));
    return (int)(x_bf16 ? dispatch<true, 0>(L, a, s) : dispatch<false, 0>(L, a, s));
}

int launch_rpbh_mxfp4(const void *X, int x_bf16, int64_t T, int K, int block, const int8_t *sign,
                      const int32_t *perm, uint8_t *codes, uint8_t *scales, uint8_t *codes_mma,
                      void *stream) {
    RpbhArgs a = make_args(X, T, K, sign, perm, codes, codes_mma, reinterpret_cast<float *>(scales));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int L = ilog2(block);
    return (int)(x_bf16 ? dispatch<true, 3>(L, a, s) : dispatch<false, 3>(L, a, s));
}

int launch_rpbh_lloydmax(const void *X, int x_bf16, int64_t T, int K, int block,
                         const int8_t *sign, const int32_t *perm, const float *thresholds,
                         int n_thresholds, const float *levels, uint8_t *codes, float *sigma,
                         uint8_t *codes_mma, void *stream) {
    if (n_thresholds != 15) return (int)hipErrorInvalidValue;
    RpbhArgs a = make_args(X, T, K, sign, perm, codes, codes_mma, sigma);
    for (int i = 0; i < 15; ++i) a.th[i] = thresholds[i];
    uint32_t lb[16];
    std::memcpy(lb, levels, sizeof lb);   // bf16-representable: the top halves
    for (int i = 0; i < 16; ++i) a.lev[i] = lb[i] >> 16;
    // ascending thresholds of a book symmetric about 0 (exact float equality)
    a.th_sym = a.th[7] == 0.0f ? 1 : 0;
    for (int i = 0; i < 15; ++i)
        if (a.th[i] != -a.th[14 - i] || (i > 0 && a.th[i] < a.th[i - 1])) a.th_sym = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int L = ilog2(block);
    return (int)(x_bf16 ? dispatch<true, 1>(L, a, s) : dispatch<false, 1>(L, a, s));
}

}  // namespace rq

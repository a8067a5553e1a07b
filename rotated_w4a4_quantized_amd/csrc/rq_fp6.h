// rq_fp6.h -- device helpers shared by the kernels that produce and consume
// INT4 codes in the GEMM's FP6 (E2M3) matrix-core layout.
//
// An E2M3 element (sign, 2 exponent bits with bias 1, 3 mantissa bits) whose
// 6-bit code is an unsigned u < 16 decodes to u / 8 (codes 0..7 are the
// subnormals m / 8, codes 8..15 have exponent 1 and decode to (8 + m) / 8).
// A symmetric activation code q in [-7, 7] is carried as u = q + 8: the two's-
// complement nibble with its top bit flipped.  An asymmetric (zero-point)
// code is already unsigned and is carried as itself.  Weights are carried
// sign-magnitude ((q < 0) << 5 | |q|, i.e. q / 8), so with both block scales
// at 2^3 the matrix core sums (qa + 8) qw exactly.
//
// "Codes in MMA layout" (rq_rotate_quant's codes_mma output): tokens in
// tiles of 32, and per tile one 3 KB block per 128 quantized coordinates
// (stage s, coordinates 128 s .. 128 s + 127), laid out
// [tile][stage][piece 0..2][lane 0..63][16 bytes] -- the layout of the
// weight blob's FP6 section, so that every 1 KB piece is one contiguous
// direct-to-LDS load of the GEMM.  Token t of the tile sits in lanes t and
// t + 32 (half h = 0, 1).  Half h of a token's stage holds four 24-byte
// fragments, one per (k-step ks, half h) over coordinates
// 128 s + 64 ks + 32 h + (0..31), as twelve dwords f[0..11] (ks 0: f[0..5],
// ks 1: f[6..11]); dword f[d] is dword d % 4 of the 16 bytes of lane
// t + 32 h in piece d / 4.  Within a fragment, 6-bit field e at bits
// [6 e, 6 e + 6) holds coordinate offset kFp6Order[e % 16] + 16 (e / 16)
// (to_fp6 below).
#pragma once

#include <stdint.h>

namespace rq {

constexpr int kMmaTileStageBytes = 3 * 1024;   // per 32 tokens per 128 coordinates

// 16 canonical nibble codes (a: offsets 0..7, b: offsets 8..15 of a group of
// coordinates; low nibble = even offset) -> sixteen 6-bit fields holding the
// nibble XOR flip (flip = 0x88888888: q + 8 for signed codes; 0: unsigned
// codes as they are), in three dwords.  Field e takes offset
// {0,1,3,4,6,7,9,10,12,13,15,8,2,11,5,14}[e]: with that order each field is
// a nibble of a or b shifted by 0 or 2 bits, so three masks per output dword
// do the spreading.
__device__ __forceinline__ void to_fp6(uint32_t a, uint32_t b, uint32_t &d0, uint32_t &d1,
                                       uint32_t &d2, uint32_t flip) {
    a ^= flip;
    b ^= flip;
    const uint32_t a2 = a << 2, b2 = b << 2;
    d0 = (a & 0x0F00F00Fu) | (a2 & 0xC03C03C0u);
    d1 = (a >> 30) | (b & 0xF00F00F0u) | (b2 & 0x03C03C00u);
    d2 = (a & 0x00F00F00u) | (b2 & 0x3C03C03Cu);
}

// Stores the 32 nibble codes of chunk c (coordinates 32 c .. 32 c + 31,
// sixteen bytes w, each nibble XOR flip giving the field) of token t into the
// MMA-layout buffer of S stages.
__device__ __forceinline__ void store_chunk_mma(uint8_t *mma, int64_t t, int S, int c, uint4 w,
                                                uint32_t flip) {
    uint32_t d[6];
    to_fp6(w.x, w.y, d[0], d[1], d[2], flip);
    to_fp6(w.z, w.w, d[3], d[4], d[5], flip);
    const int s = c >> 2, ks = (c >> 1) & 1, h = c & 1;
    uint8_t *blk = mma + ((t >> 5) * S + s) * (int64_t)kMmaTileStageBytes + (((int)t & 31) + 32 * h) * 16;
    if (ks == 0) {
        // dwords f[0..3] -> piece 0, f[4..5] -> first half of piece 1
        *reinterpret_cast<uint4 *>(blk) = make_uint4(d[0], d[1], d[2], d[3]);
        *reinterpret_cast<uint2 *>(blk + 1024) = make_uint2(d[4], d[5]);
    } else {
        // dwords f[6..7] -> second half of piece 1, f[8..11] -> piece 2
        *reinterpret_cast<uint2 *>(blk + 1024 + 8) = make_uint2(d[0], d[1]);
        *reinterpret_cast<uint4 *>(blk + 2048) = make_uint4(d[2], d[3], d[4], d[5]);
    }
}

// Stores the MMA-layout codes of the token at position t32 (0..31) of the
// 32-token tile whose S stage blocks start at `tile` (= mma + (t / 32) S
// kMmaTileStageBytes), for stage s and half h: the chunks c0 = 4 s + h
// (k-step 0) and c1 = 4 s + 2 + h (k-step 1), sixteen bytes each, become the
// token's three 16-byte lane slots (lane t32 + 32 h) of the stage block's
// pieces 0, 1 and 2 (only k-step 0's 24 bytes when has1 is false: chunk c1
// lies past the last coordinate).  Four consecutive tokens of one tile write
// one contiguous 64-byte run per piece.
__device__ __forceinline__ void store_pair_mma_in_tile(uint8_t *tile, int s, int t32, int h, uint4 w0,
                                                       uint4 w1, bool has1, uint32_t flip) {
    uint32_t d[12];
    to_fp6(w0.x, w0.y, d[0], d[1], d[2], flip);
    to_fp6(w0.z, w0.w, d[3], d[4], d[5], flip);
    to_fp6(w1.x, w1.y, d[6], d[7], d[8], flip);
    to_fp6(w1.z, w1.w, d[9], d[10], d[11], flip);
    uint8_t *blk = tile + s * kMmaTileStageBytes + (t32 + 32 * h) * 16;
    *reinterpret_cast<uint4 *>(blk) = make_uint4(d[0], d[1], d[2], d[3]);
    if (!has1) {
        *reinterpret_cast<uint2 *>(blk + 1024) = make_uint2(d[4], d[5]);
        return;
    }
    *reinterpret_cast<uint4 *>(blk + 1024) = make_uint4(d[4], d[5], d[6], d[7]);
    *reinterpret_cast<uint4 *>(blk + 2048) = make_uint4(d[8], d[9], d[10], d[11]);
}

}  // namespace rq

// rq_host.cpp -- host half of librq: error state, descriptor validation,
// the offline weight pack (fold + quantize + blob) and the Lloyd-Max
// codebook.  No GPU calls in this file.
//
// Compiled with -ffp-contract=off: every a*b+c below is two roundings unless
// std::fma is written out, so the fold and the quantizers are reproducible.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <string>
#include <thread>
#include <vector>

#include "rq_internal.h"

namespace rq {

static thread_local std::string g_err;

rq_status fail(rq_status st, const std::string &msg) {
    g_err = msg;
    return st;
}
void clear_error() { g_err.clear(); }

rq_status check_rotation(const rq_rotation *rot, bool need_tables) {
    if (!rot) return fail(RQ_ERR_NULL, "rotation descriptor is NULL");
    const int K = rot->K;
    if (K < 32 || K > 16384 || K % 32 != 0)
        return fail(RQ_ERR_SHAPE, "K must satisfy 32 <= K <= 16384 and K % 32 == 0, got " +
                                      std::to_string(K));
    if (rot->kind == RQ_ROT_RPBH) {
        const int b = rot->block;
        if (!is_pow2(b) || b < 2 || b > 1024)
            return fail(RQ_ERR_SHAPE, "RPBH block must be a power of two in [2, 1024], got " +
                                          std::to_string(b));
        if (K % b != 0)
            return fail(RQ_ERR_SHAPE, "RPBH block " + std::to_string(b) + " does not divide K " +
                                          std::to_string(K));
        if (rot->r != 0) return fail(RQ_ERR_SHAPE, "RPBH takes r == 0");
        if (need_tables && (!rot->sign || !rot->perm))
            return fail(RQ_ERR_NULL, "RPBH needs sign and perm tables");
    } else if (rot->kind == RQ_ROT_TRDQ) {
        const int b = rot->block;
        if (!is_pow2(b) || b < 16 || b > 256)
            return fail(RQ_ERR_SHAPE, "TRDQ block must be a power of two in [16, 256], got " +
                                          std::to_string(b));
        if (K % b != 0)
            return fail(RQ_ERR_SHAPE, "TRDQ block " + std::to_string(b) + " does not divide K " +
                                          std::to_string(K));
        if (rot->r != 0) return fail(RQ_ERR_SHAPE, "TRDQ takes r == 0");
        if (need_tables && (!rot->smooth || !rot->R || !rot->perm || !rot->R2))
            return fail(RQ_ERR_NULL, "TRDQ needs smooth, R (R1), perm and R2");
    } else if (rot->kind == RQ_ROT_DENSE) {
        if (rot->r < 0 || rot->r >= K || rot->r % 32 != 0)
            return fail(RQ_ERR_SHAPE, "DENSE r must satisfy 0 <= r < K and r % 32 == 0, got " +
                                          std::to_string(rot->r));
        if (need_tables && !rot->R) return fail(RQ_ERR_NULL, "DENSE needs the basis R");
    } else {
        return fail(RQ_ERR_UNSUPPORTED, "unknown rotation kind " + std::to_string(rot->kind));
    }
    return RQ_OK;
}

rq_status check_quant(const rq_rotation *rot, const rq_quant *q) {
    if (!q) return fail(RQ_ERR_NULL, "quantizer descriptor is NULL");
    if (q->kind == RQ_Q_INT4_SYM || q->kind == RQ_Q_INT4_ASYM) {
        if (q->a_bits != 4 && q->a_bits != 6 && q->a_bits != 8)
            return fail(RQ_ERR_UNSUPPORTED, "integer activations take a_bits 4, 6 or 8");
        if (q->w_bits != 4 && q->w_bits != 6 && q->w_bits != 8)
            return fail(RQ_ERR_UNSUPPORTED, "integer weights take w_bits 4, 6 or 8");
        if (q->a_bits == 4 && q->w_bits != 4)
            return fail(RQ_ERR_UNSUPPORTED, "4-bit activations take w_bits 4");
        if ((q->a_bits != 4 || q->kind == RQ_Q_INT4_ASYM) && rot->kind == RQ_ROT_DENSE)
            return fail(RQ_ERR_UNSUPPORTED,
                        "the dense rotation takes symmetric 4-bit activations (with top-r bf16)");
    } else if (q->kind == RQ_Q_MXFP4) {
        if (q->a_bits != 4 || q->w_bits != 4)
            return fail(RQ_ERR_UNSUPPORTED, "MXFP4 takes a_bits 4 and w_bits 4");
        if (rot->kind != RQ_ROT_RPBH)
            return fail(RQ_ERR_UNSUPPORTED, "MXFP4 is built for the RPBH rotation only");
        if (rot->K % 128 != 0)
            return fail(RQ_ERR_SHAPE, "MXFP4 needs K % 128 == 0 (whole 128-coordinate GEMM stages)");
    } else if (q->kind == RQ_Q_LLOYDMAX) {
        if (q->a_bits != 4) return fail(RQ_ERR_UNSUPPORTED, "LLOYDMAX takes a_bits 4");
        if (q->w_bits != 2 && q->w_bits != 4)
            return fail(RQ_ERR_UNSUPPORTED, "LLOYDMAX needs w_bits 2 or 4");
        if (rot->kind != RQ_ROT_RPBH)
            return fail(RQ_ERR_UNSUPPORTED, "LLOYDMAX is built for the RPBH rotation only");
        const int La = 1 << q->a_bits, Lw = 1 << q->w_bits;
        for (int i = 0; i + 1 < La; ++i)
            if (!(q->a_levels[i] < q->a_levels[i + 1]))
                return fail(RQ_ERR_SHAPE, "a_levels must be strictly ascending");
        for (int i = 0; i + 1 < Lw; ++i)
            if (!(q->w_levels[i] < q->w_levels[i + 1]))
                return fail(RQ_ERR_SHAPE, "w_levels must be strictly ascending");
        for (int i = 0; i < La; ++i) {
            uint32_t bits;
            std::memcpy(&bits, &q->a_levels[i], 4);
            if ((bits & 0xFFFFu) != 0 || !std::isfinite(q->a_levels[i]))
                return fail(RQ_ERR_SHAPE, "a_levels must be finite bf16 values");
        }
        for (int i = 0; i < Lw; ++i) {
            uint32_t bits;
            std::memcpy(&bits, &q->w_levels[i], 4);
            if ((bits & 0xFFFFu) != 0 || !std::isfinite(q->w_levels[i]))
                return fail(RQ_ERR_SHAPE, "w_levels must be finite bf16 values");
        }
    } else {
        return fail(RQ_ERR_UNSUPPORTED, "unknown quantizer kind " + std::to_string(q->kind));
    }
    return RQ_OK;
}

// ---------------------------------------------------------------------------
// weight fold (fp64) -- the transposed rotation of TR-DQ Eq.(9) applied to
// each output row of W stored [N][K]: v = w R.
// ---------------------------------------------------------------------------

// Sign/permutation gather, then the Sylvester butterflies of every block in
// ascending stage order, all in fp64.
static void fold_rpbh(const double *w, int K, int b, const int8_t *sign, const int32_t *perm,
                      double *v) {
    for (int j = 0; j < K; ++j) v[j] = sign[j] < 0 ? -w[perm[j]] : w[perm[j]];
    for (int base = 0; base < K; base += b)
        for (int h = 1; h < b; h <<= 1)
            for (int s = 0; s < b; s += 2 * h)
                for (int i = base + s; i < base + s + h; ++i) {
                    const double lo = v[i], hi = v[i + h];
                    v[i] = lo + hi;
                    v[i + h] = lo - hi;
                }
}

// TR-DQ (Eq.(9)-(10), H(W) = R2^T P^T R1^T Delta^-1 W): each weight row
// divided by the activations' smoothing multiplier, then the two block
// rotations around the zigzag gather, fp64 fma chains over i ascending.
static void fold_trdq(const double *w, int K, int b, const float *smooth, const float *R1,
                      const int32_t *perm, const float *R2, double *v) {
    std::vector<double> y(K), z(K);
    for (int j = 0; j < K; ++j) y[j] = w[j] / (double)smooth[j];
    for (int c = 0; c < K / b; ++c)
        for (int j = 0; j < b; ++j) {
            double acc = 0.0;
            for (int i = 0; i < b; ++i)
                acc = std::fma(y[c * b + i], (double)R1[((size_t)c * b + i) * b + j], acc);
            z[c * b + j] = acc;
        }
    for (int j = 0; j < K; ++j) y[j] = z[perm[j]];
    for (int c = 0; c < K / b; ++c)
        for (int j = 0; j < b; ++j) {
            double acc = 0.0;
            for (int i = 0; i < b; ++i)
                acc = std::fma(y[c * b + i], (double)R2[((size_t)c * b + i) * b + j], acc);
            v[c * b + j] = acc;
        }
}

// MXFP4 element: the E2M1 code (sign in bit 3) of the value nearest to x,
// ties to the even mantissa, magnitudes above 6 saturating.  Below 1 the
// grid is the multiples of 1/2; in [2^e, 2^(e+1)) the multiples of 2^(e-1).
static int e2m1_code(double x) {
    const double a = std::fabs(x);
    int c;
    if (a < 1.0) {
        c = (int)std::nearbyint(2.0 * a);   // 0, 1 (0.5) or 2 (1.0)
    } else {
        int e;
        std::frexp(a, &e);                  // a = f 2^e, 0.5 <= f < 1: binade 2^(e-1)
        const double step = std::ldexp(1.0, e - 2);
        const double v = std::min(6.0, std::nearbyint(a / step) * step);
        // v in {1, 1.5, 2, 3, 4, 6}: code = 2 (exponent field) + mantissa bit
        int ve;
        const double vf = std::frexp(v, &ve);   // v = vf 2^ve
        c = 2 * ve + (vf > 0.5 ? 1 : 0);        // 1 -> 2, 1.5 -> 3, 2 -> 4, 3 -> 5, 4 -> 6, 6 -> 7
    }
    if (c == 0) return 0;
    return (x < 0.0 ? 8 : 0) | c;
}

// E8M0 code of a 32-coordinate block whose largest magnitude is amax:
// e = floor(log2 amax) - 2 (E2M1's largest exponent), clamped to [-127, 127].
static int e8m0_code(double amax) {
    if (amax == 0.0) return 0;
    const int e = std::max(-127, std::min(127, std::ilogb(amax) - 2));
    return e + 127;
}

// Dense: v[j] = fp64 fma chain over k ascending of w[k] * R[k][j], from +0.
static void fold_dense(const double *w, int K, const float *R, double *v) {
    std::fill(v, v + K, 0.0);
    for (int k = 0; k < K; ++k) {
        const float *Rk = R + (size_t)k * K;
        const double wk = w[k];
        for (int j = 0; j < K; ++j) v[j] = std::fma(wk, (double)Rk[j], v[j]);
    }
}

static inline double bf16_bits_to_double(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return (double)f;
}

struct BlobLayout {
    int32_t row_bytes;
    int64_t scale_off, codes_off, wsum_off, mma_off, i8_off, mxs_off, total;
    int32_t mma_stages, mma_ntiles;
};

static inline int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

static BlobLayout blob_layout(const rq_rotation *rot, const rq_quant *q, int32_t N) {
    const int K = rot->K;
    const int r = rot->kind == RQ_ROT_DENSE ? rot->r : 0;
    const bool mx = q->kind == RQ_Q_MXFP4, lm = q->kind == RQ_Q_LLOYDMAX;
    BlobLayout L;
    // integer codes: 4-bit two per byte, 6- and 8-bit one per byte
    L.row_bytes = lm ? (q->w_bits == 4 ? K / 2 : K / 4) : (mx ? K / 2 : (q->w_bits == 4 ? K / 2 : K));
    L.scale_off = (int64_t)sizeof(rq_weight_header);
    L.codes_off = L.scale_off + round256(mx ? (int64_t)N * (K / 32) : (int64_t)N * 4);
    int64_t end = L.codes_off + round256((int64_t)N * L.row_bytes);
    L.mma_stages = L.mma_ntiles = 0;
    L.wsum_off = L.mma_off = L.i8_off = L.mxs_off = 0;
    if (mx) {
        L.mma_stages = (K + 127) / 128;
        L.mma_ntiles = (N + 31) / 32;
        L.mma_off = end;
        L.mxs_off = L.mma_off + (int64_t)L.mma_ntiles * (K / 32) * 512;
        end = L.mxs_off + round256((int64_t)L.mma_stages * L.mma_ntiles * 128);
    } else if (lm) {
        // 16-level weight books: the levels as bf16 in the codebook GEMM's
        // fragment order (2-bit books are decoded in the GEMM: cheap enough)
        if (q->w_bits != 4) {
            L.total = end;
            return L;
        }
        L.mma_ntiles = (N + 31) / 32;
        L.mma_off = end;
        end = L.mma_off + (int64_t)L.mma_ntiles * (K / 16) * 1024;
    } else {                             // integer weights
        L.wsum_off = end;
        end = L.wsum_off + round256((int64_t)N * 4);
        if (q->a_bits == 4) {            // FP6 fragments of the quantized coordinates
            L.mma_stages = (K - r + 127) / 128;
            L.mma_ntiles = (N + 31) / 32;
            L.mma_off = end;
            end = L.mma_off + (int64_t)L.mma_ntiles * L.mma_stages * 3 * 1024;
        } else {                         // int8 codes in the int8 GEMM's fragment order
            L.i8_off = end;
            end = L.i8_off + round256((int64_t)(N + 31) / 32 * 32 * K);
        }
    }
    L.total = end;
    return L;
}

// FP6 (E2M3) fragments of the GEMM's matrix cores.  A weight code q in
// [-7, 7] is stored sign-magnitude, (q < 0) << 5 | |q|, which E2M3 decodes as
// the subnormal q / 8.  Tile (nt, s) covers rows 32 nt .. 32 nt + 31 and the
// quantized coordinates 128 s .. 128 s + 127; lane l (row 32 nt + l % 32,
// half h = l / 32) holds two 24-byte fragments, for k-steps ks = 0, 1, over
// coordinates 128 s + 64 ks + 32 h + (0..31).  Within a fragment, 6-bit field
// f holds coordinate offset kFieldOrder[f % 16] + 16 (f / 16): the order in
// which the GEMM spreads activation nibbles into fields without per-element
// shifts (rq_gemm_fp6.hip).  The lane's 48 bytes go out as three 16-byte
// parts, part-major: [part][lane][16].
static const int kFieldOrder[16] = {0, 1, 3, 4, 6, 7, 9, 10, 12, 13, 15, 8, 2, 11, 5, 14};

static void pack_mma_tile(const uint8_t *codes, int32_t N, int row_bytes, int r, int Kq,
                          int nt, int s, uint8_t *tile /* 3 KB */) {
    for (int l = 0; l < 64; ++l) {
        const int n = 32 * nt + (l % 32), h = l / 32;
        uint32_t dw[12] = {0};
        for (int ks = 0; ks < 2; ++ks) {
            const int kbase = 128 * s + 64 * ks + 32 * h;
            for (int f = 0; f < 32; ++f) {
                const int k = kbase + kFieldOrder[f % 16] + 16 * (f / 16);
                int qv = 0;
                if (n < N && k < Kq) {
                    const int kk = r + k;
                    const uint8_t byte = codes[(size_t)n * row_bytes + kk / 2];
                    const int nib = (kk & 1) ? (byte >> 4) : (byte & 15);
                    qv = nib >= 8 ? nib - 16 : nib;
                }
                const uint32_t code = (qv < 0 ? 32u : 0u) | (uint32_t)(qv < 0 ? -qv : qv);
                const int w = (6 * f) / 32, o = (6 * f) % 32;   // field f at bits [6f, 6f + 6)
                dw[6 * ks + w] |= code << o;
                if (o > 26) dw[6 * ks + w + 1] |= code >> (32 - o);   // straddles two dwords
            }
        }
        for (int part = 0; part < 3; ++part)
            std::memcpy(tile + (part * 64 + l) * 16, &dw[4 * part], 16);
    }
}

}  // namespace rq

using namespace rq;

extern "C" {

int32_t rq_version(void) { return 200; }

const char *rq_last_error(void) { return g_err.c_str(); }

rq_status rq_packed_weight_bytes(const rq_rotation *rot, const rq_quant *q, int32_t N,
                                 size_t *bytes) {
    clear_error();
    rq_status st = check_rotation(rot, false);
    if (st != RQ_OK) return st;
    if ((st = check_quant(rot, q)) != RQ_OK) return st;
    if (!bytes) return fail(RQ_ERR_NULL, "bytes is NULL");
    if (N < 1 || N > (1 << 20)) return fail(RQ_ERR_SHAPE, "N must be in [1, 2^20]");
    *bytes = (size_t)blob_layout(rot, q, N).total;
    return RQ_OK;
}

rq_status rq_pack_weights(const rq_rotation *rot, const rq_quant *q, const void *W,
                          int32_t w_dtype, int32_t N, void *blob, size_t blob_bytes) {
    clear_error();
    rq_status st = check_rotation(rot, true);
    if (st != RQ_OK) return st;
    if ((st = check_quant(rot, q)) != RQ_OK) return st;
    if (!W || !blob) return fail(RQ_ERR_NULL, "W and blob must not be NULL");
    if (w_dtype != RQ_F32 && w_dtype != RQ_BF16)
        return fail(RQ_ERR_DTYPE, "W must be RQ_F32 or RQ_BF16");
    if (N < 1 || N > (1 << 20)) return fail(RQ_ERR_SHAPE, "N must be in [1, 2^20]");
    const int K = rot->K;
    if (rot->kind == RQ_ROT_RPBH || rot->kind == RQ_ROT_TRDQ) {
        std::vector<char> seen(K, 0);
        for (int j = 0; j < K; ++j) {
            const int p = rot->perm[j];
            if (p < 0 || p >= K || seen[p]) return fail(RQ_ERR_SHAPE, "perm is not a permutation");
            seen[p] = 1;
            if (rot->kind == RQ_ROT_RPBH && rot->sign[j] != 1 && rot->sign[j] != -1)
                return fail(RQ_ERR_SHAPE, "sign entries must be -1 or +1");
            if (rot->kind == RQ_ROT_TRDQ && (!std::isfinite(rot->smooth[j]) || rot->smooth[j] == 0.0f))
                return fail(RQ_ERR_SHAPE, "smooth entries must be finite and nonzero");
        }
    }
    const BlobLayout BL = blob_layout(rot, q, N);
    const int32_t rb = BL.row_bytes;
    const int64_t so = BL.scale_off, co = BL.codes_off, total = BL.total;
    if ((int64_t)blob_bytes < total)
        return fail(RQ_ERR_SHAPE, "blob_bytes " + std::to_string(blob_bytes) + " < required " +
                                      std::to_string(total));

    uint8_t *out = static_cast<uint8_t *>(blob);
    std::memset(out, 0, (size_t)total);
    rq_weight_header hdr;
    std::memset(&hdr, 0, sizeof hdr);
    hdr.magic = RQ_WEIGHT_MAGIC;
    hdr.version = RQ_WEIGHT_VERSION;
    hdr.format = q->kind;
    hdr.K = K;
    hdr.N = N;
    hdr.r = rot->kind == RQ_ROT_DENSE ? rot->r : 0;
    hdr.b_div = rot->kind == RQ_ROT_RPBH ? rot->block : 1;   // DENSE, TRDQ: orthonormal
    hdr.a_bits = q->a_bits;
    hdr.w_bits = q->w_bits;
    hdr.row_bytes = rb;
    hdr.scale_offset = so;
    hdr.codes_offset = co;
    hdr.total_bytes = total;
    hdr.wsum_offset = BL.wsum_off;
    hdr.mma_offset = BL.mma_off;
    hdr.mma_stages = BL.mma_stages;
    hdr.mma_ntiles = BL.mma_ntiles;
    hdr.i8_offset = BL.i8_off;
    hdr.mxs_offset = BL.mxs_off;
    if (q->kind == RQ_Q_LLOYDMAX) {
        std::memcpy(hdr.a_levels, q->a_levels, sizeof hdr.a_levels);
        std::memcpy(hdr.w_levels, q->w_levels, sizeof hdr.w_levels);
    }
    std::memcpy(out, &hdr, sizeof hdr);
    float *scales = reinterpret_cast<float *>(out + so);
    uint8_t *codes = out + co;

    // Lloyd-Max: midpoints of adjacent weight levels (exact for bf16 levels)
    const int Lw = q->kind == RQ_Q_LLOYDMAX ? 1 << q->w_bits : 0;
    double wth[15] = {0};
    for (int i = 0; i + 1 < Lw; ++i)
        wth[i] = ((double)q->w_levels[i] + (double)q->w_levels[i + 1]) / 2.0;

    auto work = [&](int n0, int n1) {
        std::vector<double> w(K), v(K);
        for (int n = n0; n < n1; ++n) {
            if (w_dtype == RQ_F32) {
                const float *src = static_cast<const float *>(W) + (size_t)n * K;
                for (int k = 0; k < K; ++k) w[k] = (double)src[k];
            } else {
                const uint16_t *src = static_cast<const uint16_t *>(W) + (size_t)n * K;
                for (int k = 0; k < K; ++k) w[k] = bf16_bits_to_double(src[k]);
            }
            if (rot->kind == RQ_ROT_RPBH)
                fold_rpbh(w.data(), K, rot->block, rot->sign, rot->perm, v.data());
            else if (rot->kind == RQ_ROT_TRDQ)
                fold_trdq(w.data(), K, rot->block, rot->smooth, rot->R, rot->perm, rot->R2, v.data());
            else
                fold_dense(w.data(), K, rot->R, v.data());
            uint8_t *row = codes + (size_t)n * rb;
            if (q->kind == RQ_Q_MXFP4) {
                uint8_t *e8 = out + so + (size_t)n * (K / 32);
                for (int c = 0; c < K / 32; ++c) {
                    double amax = 0.0;
                    for (int k = 32 * c; k < 32 * c + 32; ++k) amax = std::max(amax, std::fabs(v[k]));
                    const int sc = e8m0_code(amax);
                    e8[c] = (uint8_t)sc;
                    for (int k = 32 * c; k < 32 * c + 32; k += 2)
                        row[k / 2] = (uint8_t)(e2m1_code(std::ldexp(v[k], 127 - sc)) |
                                               (e2m1_code(std::ldexp(v[k + 1], 127 - sc)) << 4));
                }
            } else if (q->kind != RQ_Q_LLOYDMAX) {   // symmetric integer weights
                const int qmax = (1 << (q->w_bits - 1)) - 1;   // 7, 31, 127
                double amax = 0.0;
                for (int k = 0; k < K; ++k) amax = std::max(amax, std::fabs(v[k]));
                if (amax == 0.0) {
                    scales[n] = 0.0f;
                    continue;  // codes already zero
                }
                const double inv = (double)qmax / amax;
                for (int k = 0; k < K; k += 2) {
                    int c[2];
                    for (int e = 0; e < 2; ++e) {
                        double t = std::nearbyint(v[k + e] * inv);
                        t = std::min((double)qmax, std::max(-(double)qmax, t));
                        c[e] = (int)t;
                    }
                    if (q->w_bits != 4) {
                        row[k] = (uint8_t)(int8_t)c[0];
                        row[k + 1] = (uint8_t)(int8_t)c[1];
                    } else {
                        row[k / 2] = (uint8_t)((c[0] & 0xF) | ((c[1] & 0xF) << 4));
                    }
                }
                scales[n] = (float)(amax / (double)qmax);
            } else {
                double ss = 0.0;
                for (int k = 0; k < K; ++k) ss += v[k] * v[k];
                const double nrm = std::sqrt(ss);
                if (nrm == 0.0) {
                    scales[n] = 0.0f;
                    continue;
                }
                const double g = std::sqrt((double)K) / nrm;
                const int per_byte = 8 / q->w_bits;
                for (int k = 0; k < K; ++k) {
                    const double x = v[k] * g;
                    int idx = 0;
                    for (int i = 0; i + 1 < Lw; ++i) idx += (x > wth[i]) ? 1 : 0;
                    row[k / per_byte] |= (uint8_t)(idx << ((k % per_byte) * q->w_bits));
                }
                scales[n] = (float)(nrm / std::sqrt((double)K));
            }
        }
    };
    unsigned nt = std::max(1u, std::min(32u, std::thread::hardware_concurrency()));
    nt = std::min<unsigned>(nt, (unsigned)N);
    std::vector<std::thread> pool;
    const int chunk = (N + (int)nt - 1) / (int)nt;
    for (unsigned t = 0; t < nt; ++t) {
        const int n0 = (int)t * chunk, n1 = std::min(N, n0 + chunk);
        if (n0 < n1) pool.emplace_back(work, n0, n1);
    }
    for (auto &th : pool) th.join();
    auto parallel = [&](int count, const std::function<void(int, int)> &fn) {
        std::vector<std::thread> tp;
        const unsigned nth = std::max(1u, std::min<unsigned>(nt, (unsigned)count));
        const int ch = (count + (int)nth - 1) / (int)nth;
        for (unsigned t = 0; t < nth; ++t) {
            const int a0 = (int)t * ch, a1 = std::min(count, a0 + ch);
            if (a0 < a1) tp.emplace_back(fn, a0, a1);
        }
        for (auto &th : tp) th.join();
    };
    if (q->kind == RQ_Q_INT4_SYM || q->kind == RQ_Q_INT4_ASYM) {
        // the GEMMs' copies of the quantized coordinates [r, K): row sums, and
        // FP6 fragments (4-bit activations, see pack_mma_tile) or int8 codes
        const int r = hdr.r, Kq = K - r;
        const bool wbytes = q->w_bits != 4;
        auto wcode = [&](int n, int k) -> int {
            if (wbytes) return (int)(int8_t)codes[(size_t)n * rb + k];
            const uint8_t byte = codes[(size_t)n * rb + k / 2];
            const int nib = (k & 1) ? (byte >> 4) : (byte & 15);
            return nib >= 8 ? nib - 16 : nib;
        };
        int32_t *wsum = reinterpret_cast<int32_t *>(out + BL.wsum_off);
        for (int n = 0; n < N; ++n) {
            int32_t sum = 0;
            for (int k = r; k < K; ++k) sum += wcode(n, k);
            wsum[n] = sum;
        }
        if (q->a_bits == 4) {
            const int ntiles = BL.mma_ntiles, S = BL.mma_stages;
            parallel(ntiles, [&](int t0, int t1) {
                for (int tile = t0; tile < t1; ++tile)
                    for (int s = 0; s < S; ++s)
                        pack_mma_tile(codes, N, rb, r, Kq, tile, s,
                                      out + BL.mma_off + ((int64_t)tile * S + s) * 3 * 1024);
            });
        } else {
            // [ceil(N/32)][K/32][64 lanes][16 B]: lane l of k-step kb holds row
            // 32 tile + l % 32, coordinates 32 kb + 16 (l / 32) .. + 15
            // (rows past N stay zero)
            int8_t *i8 = reinterpret_cast<int8_t *>(out + BL.i8_off);
            const int nkb = K / 32;
            for (int n = 0; n < N; ++n)
                for (int k = 0; k < K; ++k) {
                    const size_t lane = (size_t)(n % 32) + 32 * ((k % 32) / 16);
                    i8[(((size_t)(n / 32) * nkb + k / 32) * 64 + lane) * 16 + k % 16] = (int8_t)wcode(n, k);
                }
        }
    } else if (q->kind == RQ_Q_MXFP4) {
        // tiled copies for the scaled FP4 GEMM: codes [tile][K/32][32][16],
        // scales [stage][tile][64][2] (byte ks of lane 32 h + i: row
        // 32 tile + i, coordinates 128 s + 64 ks + 32 h ..)
        const int ntiles = BL.mma_ntiles, nch = K / 32;
        const uint8_t *e8 = out + so;
        for (int tile = 0; tile < ntiles; ++tile)
            for (int c = 0; c < nch; ++c)
                for (int i = 0; i < 32; ++i) {
                    const int n = 32 * tile + i;
                    if (n >= N) continue;
                    std::memcpy(out + BL.mma_off + (((int64_t)tile * nch + c) * 32 + i) * 16,
                                codes + (size_t)n * rb + 16 * c, 16);
                    const int s = c / 4, ks = (c / 2) & 1, h = c & 1;
                    out[BL.mxs_off + (((int64_t)s * ntiles + tile) * 64 + 32 * h + i) * 2 + ks] =
                        e8[(size_t)n * nch + c];
                }
    } else if (q->kind == RQ_Q_LLOYDMAX && BL.mma_off) {
        // the levels as bf16 in the codebook GEMM's fragment order
        // [ceil(N/32)][K/16][64 lanes][8 x bf16]: lane i + 32 h of k-step c
        // holds row 32 tile + i, coordinates 16 c + 8 h .. + 7 (rows past N
        // stay zero); the levels are bf16 values, so the top halves are exact
        const int per_byte = 8 / q->w_bits, nks = K / 16;
        uint16_t lev16[16];
        for (int i = 0; i < Lw; ++i) {
            uint32_t bits;
            std::memcpy(&bits, &q->w_levels[i], 4);
            lev16[i] = (uint16_t)(bits >> 16);
        }
        uint16_t *frag = reinterpret_cast<uint16_t *>(out + BL.mma_off);
        parallel(N, [&](int n0, int n1) {
            for (int n = n0; n < n1; ++n)
                for (int k = 0; k < K; ++k) {
                    const int idx = (codes[(size_t)n * rb + k / per_byte] >> ((k % per_byte) * q->w_bits)) & (Lw - 1);
                    const size_t lane = (size_t)(n % 32) + 32 * ((k % 16) / 8);
                    frag[(((size_t)(n / 32) * nks + k / 16) * 64 + lane) * 8 + k % 8] = lev16[idx];
                }
        });
    }
    return RQ_OK;
}

static_assert(sizeof(rq_set_header) == 4864, "set header size");

rq_status rq_weight_set_bytes(const rq_rotation *rots, int32_t groups, const rq_quant *q,
                              int32_t N, size_t *bytes) {
    clear_error();
    if (!rots || !bytes) return fail(RQ_ERR_NULL, "rots and bytes must not be NULL");
    if (groups < 1 || groups > RQ_SET_MAX_GROUPS)
        return fail(RQ_ERR_SHAPE, "groups must be in [1, " + std::to_string(RQ_SET_MAX_GROUPS) + "]");
    size_t total = sizeof(rq_set_header);
    for (int g = 0; g < groups; ++g) {
        if (rots[g].K != rots[0].K) return fail(RQ_ERR_SHAPE, "the set's rotations differ in K");
        size_t b = 0;
        const rq_status st = rq_packed_weight_bytes(&rots[g], q, N, &b);
        if (st != RQ_OK) return st;
        total += (b + 255) / 256 * 256;
    }
    *bytes = total;
    return RQ_OK;
}

rq_status rq_pack_weight_set(const rq_rotation *rots, int32_t groups, const int32_t *step_group,
                             int32_t steps, const rq_quant *q, const void *W, int32_t w_dtype,
                             int32_t N, void *blob, size_t blob_bytes) {
    size_t need = 0;
    rq_status st = rq_weight_set_bytes(rots, groups, q, N, &need);
    if (st != RQ_OK) return st;
    if (!step_group || !blob || !W) return fail(RQ_ERR_NULL, "step_group, W and blob must not be NULL");
    if (steps < 1 || steps > RQ_SET_MAX_STEPS)
        return fail(RQ_ERR_SHAPE, "steps must be in [1, " + std::to_string(RQ_SET_MAX_STEPS) + "]");
    for (int t = 0; t < steps; ++t)
        if (step_group[t] < 0 || step_group[t] >= groups)
            return fail(RQ_ERR_SHAPE, "step " + std::to_string(t) + " maps outside the groups");
    if (blob_bytes < need)
        return fail(RQ_ERR_SHAPE, "blob_bytes " + std::to_string(blob_bytes) + " < required " +
                                      std::to_string(need));
    uint8_t *out = static_cast<uint8_t *>(blob);
    rq_set_header sh;
    std::memset(&sh, 0, sizeof sh);
    sh.magic = RQ_SET_MAGIC;
    sh.version = RQ_SET_VERSION;
    sh.groups = groups;
    sh.steps = steps;
    for (int t = 0; t < steps; ++t) sh.step_group[t] = step_group[t];
    size_t off = sizeof(rq_set_header);
    for (int g = 0; g < groups; ++g) {
        size_t b = 0;
        rq_packed_weight_bytes(&rots[g], q, N, &b);
        sh.member_offset[g] = (int64_t)off;
        st = rq_pack_weights(&rots[g], q, W, w_dtype, N, out + off, b);
        if (st != RQ_OK) return st;
        off += (b + 255) / 256 * 256;
    }
    std::memcpy(out, &sh, sizeof sh);
    return RQ_OK;
}

rq_status rq_weight_set_member(const void *set_host, int32_t step, int32_t *group,
                               const rq_weight_header **hdr, int64_t *offset) {
    clear_error();
    if (!set_host || !group || !hdr || !offset)
        return fail(RQ_ERR_NULL, "set, group, hdr and offset must not be NULL");
    const rq_set_header *sh = static_cast<const rq_set_header *>(set_host);
    if (sh->magic != RQ_SET_MAGIC || sh->version != RQ_SET_VERSION || sh->groups < 1 ||
        sh->groups > RQ_SET_MAX_GROUPS || sh->steps < 1 || sh->steps > RQ_SET_MAX_STEPS)
        return fail(RQ_ERR_FORMAT, "not a time-step set blob");
    if (step < 0 || step >= sh->steps)
        return fail(RQ_ERR_SHAPE, "step " + std::to_string(step) + " outside the set's " +
                                      std::to_string(sh->steps) + " steps");
    const int g = sh->step_group[step];
    if (g < 0 || g >= sh->groups) return fail(RQ_ERR_FORMAT, "set step table is corrupt");
    *group = g;
    *offset = sh->member_offset[g];
    *hdr = reinterpret_cast<const rq_weight_header *>(static_cast<const uint8_t *>(set_host) +
                                                      sh->member_offset[g]);
    return RQ_OK;
}

// Lloyd's iteration for N(0,1) in fp64, then bf16 rounding of the levels.
rq_status rq_lloydmax_gaussian(int32_t L, float *levels) {
    clear_error();
    if (!levels) return fail(RQ_ERR_NULL, "levels is NULL");
    if (L != 2 && L != 4 && L != 8 && L != 16)
        return fail(RQ_ERR_SHAPE, "L must be 2, 4, 8 or 16");
    const double inv_sqrt2 = 0.70710678118654752440;
    const double inv_sqrt2pi = 0.39894228040143267794;
    auto pdf = [&](double t) { return std::isinf(t) ? 0.0 : inv_sqrt2pi * std::exp(-0.5 * t * t); };
    // upper-tail mass Q(t) = P(Z > t) through erfc (accurate in the tails)
    auto upper = [&](double t) {
        if (std::isinf(t)) return t > 0 ? 0.0 : 1.0;
        return 0.5 * std::erfc(t * inv_sqrt2);
    };
    auto cell_mass = [&](double a, double b) {
        if (a >= 0) return upper(a) - upper(b);
        if (b <= 0) return upper(-b) - upper(-a);
        return 1.0 - upper(-a) - upper(b);
    };
    std::vector<double> c(L), t(L + 1), nc(L);
    const double span = 1.0 + 0.25 * std::log2((double)L);
    for (int i = 0; i < L; ++i) c[i] = -span + 2.0 * span * (i + 0.5) / L;
    for (int it = 0; it < 200000; ++it) {
        t[0] = -INFINITY;
        t[L] = INFINITY;
        for (int i = 1; i < L; ++i) t[i] = (c[i - 1] + c[i]) / 2.0;
        double delta = 0.0;
        for (int i = 0; i < L; ++i) {
            nc[i] = (pdf(t[i]) - pdf(t[i + 1])) / cell_mass(t[i], t[i + 1]);
            delta = std::max(delta, std::fabs(nc[i] - c[i]));
        }
        c.swap(nc);
        if (delta < 1e-15) break;
    }
    for (int i = 0; i < L; ++i) {
        // nearest bf16 (8 significant bits), ties to even, straight from fp64
        int e;
        const double m = std::frexp(c[i], &e);      // c = m 2^e, 0.5 <= |m| < 1
        const double q = std::nearbyint(m * 256.0);  // exact scaling; RNE mode
        levels[i] = (float)std::ldexp(q, e - 8);
    }
    return RQ_OK;
}

}  // extern "C"

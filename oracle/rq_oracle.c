/*
 * rq_oracle.c -- plain, slow, obviously-correct CPU oracle for the rotated
 * low-bit quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only tests/, the smoke check in __graft_entry__.py and
 * the cpu_baseline leg of bench.py load it (through oracle/oracle.py).  It
 * shares no source, header, table or helper with the HIP path.
 *
 * Sources (pages, not code):
 *   [TRDQ]  "TR-DQ: Time-Rotation Diffusion Quantization", section 3.1
 *           (Y = X.W; Eq.(1)-(3) uniform quantizer; per-token activations and
 *           per-channel weights) and section 3.2 (Eq.(8) block-diagonal
 *           rotation with 2^n x 2^n blocks; Eq.(9)-(10) computational
 *           invariance: activations rotated at runtime, the transposed
 *           rotation folded into the weights).
 *   [ORBIT] "OrbitQuant: Data-Agnostic Quantization for Image and Video
 *           Diffusion Transformers", abstract: randomized permuted
 *           block-Hadamard (RPBH) rotation, quantization in a normalized
 *           rotated basis with one Lloyd-Max codebook per input dimension,
 *           the same quantizer applied offline to weight rows with the
 *           rotation absorbed into them.
 *   [DIROTQ] "DiRotQ: Rotation-Aware Quantization for 4-bit Diffusion
 *           Transformers", abstract: activations rotated into a PCA basis at
 *           inference, the top principal subspace kept at higher precision,
 *           the rest quantized to 4 bits, the inverse rotation fused into the
 *           weights offline.
 *
 * Where the pages leave the arithmetic open, this file follows the readings
 * listed in the design notes (fp32 butterflies in ascending stage order,
 * an fp32 FMA chain for the dense basis, symmetric RNE quantization, exact
 * integer-grid norm).  Every function states the reading it implements.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (no contraction: every a*b+c below is two roundings unless fma() is
 * written out).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

/* ------------------------------------------------------------------ */
/* bf16 helpers (the input format of the DiT workloads)                 */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> fp32, exact (bf16 is the top half of an fp32). */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* fp32 -> bf16 with round-half-to-even on the dropped 16 bits (finite x).
 * Used for DiRotQ's top-r coefficients "kept at higher precision". */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, 4);
    uint32_t upper = bits >> 16;
    uint32_t lower = bits & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/* ------------------------------------------------------------------ */
/* Rotations                                                            */
/* ------------------------------------------------------------------ */

/*
 * RPBH forward on one row, fp32 arithmetic ([ORBIT] abstract; [TRDQ] Eq.(8)).
 *   1. permute and sign:  y[j] = sign[j] * x[perm[j]]            (exact)
 *   2. for every block [c*b, (c+1)*b) and h = 1, 2, 4, ..., b/2 in that
 *      order, every index i of the block whose local bit h is clear:
 *         (y[i], y[i+h]) <- (y[i] + y[i+h], y[i] - y[i+h])
 *      each + and - one IEEE fp32 round-to-nearest-even operation.
 * The result is y . BlockDiag(H_b) with the unnormalized Sylvester matrix
 * H_b[i][k] = (-1)^popcount(i & k); it equals sqrt(b) times the orthonormal
 * rotation.
 */
void orc_rpbh_row_f32(const float *x, int K, int b, const int8_t *sign,
                      const int32_t *perm, float *y)
{
    for (int j = 0; j < K; j++)
        y[j] = (float)sign[j] * x[perm[j]];
    for (int c = 0; c < K; c += b) {
        for (int h = 1; h < b; h *= 2) {
            for (int i = c; i < c + b; i++) {
                if (((i - c) & h) != 0)
                    continue;
                float lo = y[i];
                float hi = y[i + h];
                y[i] = lo + hi;
                y[i + h] = lo - hi;
            }
        }
    }
}

/* The same RPBH forward in fp64, used for the offline weight fold
 * ([TRDQ] Eq.(9): the weights receive the transposed rotation; with
 * W stored [N][K] each weight row is rotated exactly like a token). */
void orc_rpbh_row_f64(const double *x, int K, int b, const int8_t *sign,
                      const int32_t *perm, double *y)
{
    for (int j = 0; j < K; j++)
        y[j] = (double)sign[j] * x[perm[j]];
    for (int c = 0; c < K; c += b) {
        for (int h = 1; h < b; h *= 2) {
            for (int i = c; i < c + b; i++) {
                if (((i - c) & h) != 0)
                    continue;
                double lo = y[i];
                double hi = y[i + h];
                y[i] = lo + hi;
                y[i + h] = lo - hi;
            }
        }
    }
}

/*
 * Dense rotation u = x . R for one row ([DIROTQ] abstract: rotation into the
 * PCA basis at inference).  R is [K][K] row-major fp32, column j is basis
 * vector j.  Each output is one fp32 fused multiply-add chain over k
 * ascending, starting from +0:  acc = fmaf(x[k], R[k][j], acc).
 */
void orc_dense_row_f32(const float *x, const float *R, int K, float *u)
{
    for (int j = 0; j < K; j++) {
        float acc = 0.0f;
        for (int k = 0; k < K; k++)
            acc = fmaf(x[k], R[(size_t)k * K + j], acc);
        u[j] = acc;
    }
}

/* Dense fold of one weight row in fp64: v[j] = sum_k w[k] * R[k][j] as an
 * fp64 fma chain over k ascending, starting from +0. */
void orc_dense_row_f64(const double *w, const float *R, int K, double *v)
{
    for (int j = 0; j < K; j++) {
        double acc = 0.0;
        for (int k = 0; k < K; k++)
            acc = fma(w[k], (double)R[(size_t)k * K + j], acc);
        v[j] = acc;
    }
}

/* ------------------------------------------------------------------ */
/* Symmetric INT4 quantizers                                            */
/* ------------------------------------------------------------------ */

/*
 * Per-token symmetric INT4 ([TRDQ] Eq.(1)-(2) with the zero point fixed at 0
 * and the range made symmetric; per-token granularity from [TRDQ] 3.1).
 * Quantized coordinates are u[r..K-1] (r = 0 except the DiRotQ path).
 *   amax = max |u[j]|
 *   amax == 0  ->  all codes 0, scale 0
 *   else       s = fl32(amax / 7), inv = fl32(7 / amax)  (correctly rounded)
 *              q[j] = clamp(rne(fl32(u[j] * inv)), -7, 7)
 * q has K - r entries.
 */
void orc_quant_sym_row(const float *u, int K, int r, int qmax, int16_t *q, float *s_out);

void orc_quant_int4_row(const float *u, int K, int r, int8_t *q, float *s_out)
{
    int16_t *w = (int16_t *)malloc((size_t)(K - r) * sizeof(int16_t));
    orc_quant_sym_row(u, K, r, 7, w, s_out);
    for (int j = 0; j < K - r; j++)
        q[j] = (int8_t)w[j];
    free(w);
}

/*
 * Per-token symmetric b-bit quantizer of a rotated row, qmax = 2^(b-1) - 1
 * (7 for INT4, 31 for 6-bit, 127 for INT8 -- TR-DQ's W6A6, W8A8 and W4A8
 * settings), over the
 * coordinates u[r..K-1]:
 *   amax = max |u[j]|
 *   amax == 0  ->  all codes 0, scale 0
 *   else       s = fl32(amax / qmax), inv = fl32(qmax / amax)  (correctly rounded)
 *              q[j] = clamp(rne(fl32(u[j] * inv)), -qmax, qmax)
 * q has K - r entries.
 */
void orc_quant_sym_row(const float *u, int K, int r, int qmax, int16_t *q, float *s_out)
{
    float amax = 0.0f;
    for (int j = r; j < K; j++) {
        float a = fabsf(u[j]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f) {
        for (int j = r; j < K; j++)
            q[j - r] = 0;
        *s_out = 0.0f;
        return;
    }
    float fq = (float)qmax;
    float s = amax / fq;
    float inv = fq / amax;
    for (int j = r; j < K; j++) {
        float m = u[j] * inv;
        float t = rintf(m);
        if (t > fq) t = fq;
        if (t < -fq) t = -fq;
        q[j - r] = (int16_t)t;
    }
    *s_out = s;
}

void orc_quant_asym_row(const float *u, int K, int levels, uint16_t *q, float *s_out,
                        float *z_out);

/*
 * Per-token asymmetric INT4 of a rotated row ([TRDQ] section 3.1: Eq.(1)
 * X_int = clamp(round(X / s) + z, 0, 2^b - 1), Eq.(2) s = (max X - min X) /
 * (2^b - 1), Eq.(3) the zero point z), b = 4, over all K coordinates; the
 * general b-bit form is orc_quant_asym_row below.
 */
void orc_quant_int4_asym_row(const float *u, int K, uint8_t *q, float *s_out, float *z_out)
{
    uint16_t *w = (uint16_t *)malloc((size_t)K * sizeof(uint16_t));
    orc_quant_asym_row(u, K, 15, w, s_out, z_out);
    for (int j = 0; j < K; j++)
        q[j] = (uint8_t)w[j];
    free(w);
}

/*
 * Per-token asymmetric b-bit quantizer, levels = 2^b - 1 (15, 63 or 255), over
 * all K coordinates ([TRDQ] Eq.(1)-(3)).  Readings where the pages are open
 * or garbled:
 *   - Eq.(3) prints z = round(min X / s); with Eq.(1)'s "+ z" the minimum
 *     must land on code 0, so z = -round(min X / s);
 *   - z is kept in [0, levels] (it already is whenever min <= 0 <= max);
 *   - one fp32 rounding per operation, the division by s taken as a
 *     multiplication by its reciprocal computed directly:
 *       lo = min u, hi = max u, d = fl32(hi - lo)
 *       d == 0  ->  all codes 0, s = 0, z = 0
 *       else    s = fl32(d / levels), inv = fl32(levels / d)
 *               z = clamp(-rne(fl32(lo * inv)), 0, levels)   (an integer, +0 for zero)
 *               q[j] = clamp(rne(fl32(u[j] * inv)) + z, 0, levels)
 * Codes are unsigned, 0..levels.
 */
void orc_quant_asym_row(const float *u, int K, int levels, uint16_t *q, float *s_out,
                        float *z_out)
{
    float lo = u[0], hi = u[0];
    for (int j = 1; j < K; j++) {
        if (u[j] < lo) lo = u[j];
        if (u[j] > hi) hi = u[j];
    }
    float d = hi - lo;
    if (d == 0.0f) {
        for (int j = 0; j < K; j++)
            q[j] = 0;
        *s_out = 0.0f;
        *z_out = 0.0f;
        return;
    }
    float fl = (float)levels;
    float s = d / fl;
    float inv = fl / d;
    float zl = lo * inv;
    float zr = rintf(zl);
    int zi = zr > 0.0f ? 0 : (zr < -fl ? levels : -(int)zr);
    float z = (float)zi;        /* an integer in [0, levels]; +0 for zero */
    for (int j = 0; j < K; j++) {
        float m = u[j] * inv;
        float t = rintf(m) + z;   /* integers below 2^24: exact */
        if (t < 0.0f) t = 0.0f;
        if (t > fl) t = fl;
        q[j] = (uint16_t)t;
    }
    *s_out = s;
    *z_out = z;
}

/* Per-output-channel symmetric b-bit quantizer of a folded fp64 weight row
 * (all K), qmax = 7 (INT4), 31 (6-bit) or 127 (INT8):
 *   amax == 0 -> codes 0, scale 0
 *   s_w = (float)(amax / qmax), inv = qmax / amax (fp64), q = clamp(rne(v*inv)). */
void orc_quant_sym_wrow(const double *v, int K, int qmax, int16_t *q, float *s_out)
{
    double amax = 0.0;
    for (int j = 0; j < K; j++) {
        double a = fabs(v[j]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0) {
        for (int j = 0; j < K; j++)
            q[j] = 0;
        *s_out = 0.0f;
        return;
    }
    double dq = (double)qmax;
    double inv = dq / amax;
    for (int j = 0; j < K; j++) {
        double t = rint(v[j] * inv);
        if (t > dq) t = dq;
        if (t < -dq) t = -dq;
        q[j] = (int16_t)t;
    }
    *s_out = (float)(amax / dq);
}

void orc_quant_int4_wrow(const double *v, int K, int8_t *q, float *s_out)
{
    int16_t *w = (int16_t *)malloc((size_t)K * sizeof(int16_t));
    orc_quant_sym_wrow(v, K, 7, w, s_out);
    for (int j = 0; j < K; j++)
        q[j] = (int8_t)w[j];
    free(w);
}

/* ------------------------------------------------------------------ */
/* MXFP4: E2M1 elements with one E8M0 scale per 32 coordinates          */
/* ------------------------------------------------------------------ */

/*
 * The FP4 format variant ("DiRotQ" abstract, later version: the same method
 * run with NVFP4 on a Blackwell GPU).  The pages name the format and define
 * nothing more; the reading here is the OCP Microscaling (MX) v1.0 MXFP4
 * format, the one gfx950's scaled matrix cores take:
 *   element  E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit;
 *            magnitudes by 3-bit code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6
 *            (code 1 is the subnormal 0.5); the sign is bit 3
 *   block    32 consecutive coordinates share an E8M0 scale 2^e
 *            (code e + 127, e in [-127, 127])
 *   scale    e = floor(log2(max |x| of the block)) - 2  (2 = the exponent of
 *            E2M1's largest value), clamped to [-127, 127]; a block of
 *            zeros takes e = -127
 *   element  nearest E2M1 value to x / 2^e, ties to the even code (mantissa
 *            bit 0), magnitudes above 6 saturate to 6; a zero is code 0
 *            (positive) whatever the sign of x
 * The value of a block element is e2m1(code) * 2^e.
 */
static const double orc_e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code)
{
    double m = orc_e2m1_mag[code & 7];
    return (code & 8) ? -m : m;
}

/* Nearest E2M1 code to x (brute force over the eight magnitudes). */
int orc_e2m1_encode(double x)
{
    double a = fabs(x);
    int best = 0;
    double bd = a;
    for (int c = 1; c < 8; c++) {
        double d = fabs(a - orc_e2m1_mag[c]);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    if (best == 0)
        return 0;
    return (x < 0.0 ? 8 : 0) | best;
}

/* E8M0 code of the scale of a block whose largest magnitude is amax. */
int orc_mx_scale_code(double amax)
{
    if (amax == 0.0)
        return 0;
    int e = ilogb(amax) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
}

/* MXFP4 of a vector of K coordinates (K % 32 == 0), given in fp64 (the
 * fp32 activations convert exactly): codes [K/2] nibbles (low nibble = even
 * coordinate), scales [K/32] E8M0 codes.  x / 2^e is exact in fp64. */
void orc_quant_mxfp4_f64(const double *x, int K, uint8_t *codes, uint8_t *scales)
{
    for (int c = 0; c < K / 32; c++) {
        double amax = 0.0;
        for (int j = 32 * c; j < 32 * c + 32; j++)
            if (fabs(x[j]) > amax)
                amax = fabs(x[j]);
        int sc = orc_mx_scale_code(amax);
        scales[c] = (uint8_t)sc;
        for (int j = 32 * c; j < 32 * c + 32; j += 2) {
            int lo = orc_e2m1_encode(ldexp(x[j], 127 - sc));
            int hi = orc_e2m1_encode(ldexp(x[j + 1], 127 - sc));
            codes[j / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

void orc_quant_mxfp4_row(const float *u, int K, uint8_t *codes, uint8_t *scales)
{
    double *x = (double *)malloc((size_t)K * sizeof(double));
    for (int j = 0; j < K; j++)
        x[j] = (double)u[j];
    orc_quant_mxfp4_f64(x, K, codes, scales);
    free(x);
}

/* ------------------------------------------------------------------ */
/* TR-DQ runtime rotation: smoothing, block rotation, zigzag            */
/* permutation, block rotation                                          */
/* ------------------------------------------------------------------ */

/*
 * [TRDQ] Eq.(9)-(10): G(X) = (X . Delta) R1 P R2, with Delta a per-channel
 * scale (Eq.(4)-(5), SmoothQuant's migration), R1 and R2 block-diagonal
 * rotations (Eq.(8): b x b blocks) and P the zigzag permutation.  Readings:
 *   - m[K] is the per-channel multiplier the activations receive (Eq.(9)'s
 *     Delta; Eq.(4) writes the same migration as X diag(Delta)^-1), the
 *     weights receive its inverse;
 *   - R1, R2 are [K/b][b][b], block c mapping coordinates cb..cb+b-1 to
 *     themselves: z[cb + j] = sum_i y[cb + i] R1[c][i][j];
 *   - P as a gather: p[j] = z[perm[j]] (the same convention as RPBH's);
 *   - arithmetic as the dense path's: one fp32 multiply per smoothed
 *     coordinate, then per output one fp32 fused multiply-add chain over i
 *     ascending from +0, for each of the two block rotations.
 */
void orc_trdq_row_f32(const float *x, int K, int b, const float *m, const float *R1,
                      const int32_t *perm, const float *R2, float *u)
{
    float *y = (float *)malloc((size_t)K * sizeof(float));
    float *z = (float *)malloc((size_t)K * sizeof(float));
    for (int j = 0; j < K; j++)
        y[j] = x[j] * m[j];
    for (int c = 0; c < K / b; c++) {
        const float *Rc = R1 + (size_t)c * b * b;
        for (int j = 0; j < b; j++) {
            float acc = 0.0f;
            for (int i = 0; i < b; i++)
                acc = fmaf(y[c * b + i], Rc[(size_t)i * b + j], acc);
            z[c * b + j] = acc;
        }
    }
    for (int j = 0; j < K; j++)
        y[j] = z[perm[j]];
    for (int c = 0; c < K / b; c++) {
        const float *Rc = R2 + (size_t)c * b * b;
        for (int j = 0; j < b; j++) {
            float acc = 0.0f;
            for (int i = 0; i < b; i++)
                acc = fmaf(y[c * b + i], Rc[(size_t)i * b + j], acc);
            u[c * b + j] = acc;
        }
    }
    free(y);
    free(z);
}

/* The weight fold of [TRDQ] Eq.(9)-(10), H(W) = R2^T P^T R1^T Delta^-1 W:
 * with W stored [N][K], row w becomes ((w / m) R1) P R2, in fp64 (division
 * correctly rounded, fp64 fma chains over i ascending). */
void orc_trdq_row_f64(const double *w, int K, int b, const float *m, const float *R1,
                      const int32_t *perm, const float *R2, double *v)
{
    double *y = (double *)malloc((size_t)K * sizeof(double));
    double *z = (double *)malloc((size_t)K * sizeof(double));
    for (int j = 0; j < K; j++)
        y[j] = w[j] / (double)m[j];
    for (int c = 0; c < K / b; c++) {
        const float *Rc = R1 + (size_t)c * b * b;
        for (int j = 0; j < b; j++) {
            double acc = 0.0;
            for (int i = 0; i < b; i++)
                acc = fma(y[c * b + i], (double)Rc[(size_t)i * b + j], acc);
            z[c * b + j] = acc;
        }
    }
    for (int j = 0; j < K; j++)
        y[j] = z[perm[j]];
    for (int c = 0; c < K / b; c++) {
        const float *Rc = R2 + (size_t)c * b * b;
        for (int j = 0; j < b; j++) {
            double acc = 0.0;
            for (int i = 0; i < b; i++)
                acc = fma(y[c * b + i], (double)Rc[(size_t)i * b + j], acc);
            v[c * b + j] = acc;
        }
    }
    free(y);
    free(z);
}

/* Two 4-bit two's-complement codes per byte, low nibble = even index. */
void orc_pack_nibbles(const int8_t *q, int n, uint8_t *out)
{
    for (int i = 0; i < n / 2; i++)
        out[i] = (uint8_t)(((uint8_t)q[2 * i] & 0x0Fu) |
                           (((uint8_t)q[2 * i + 1] & 0x0Fu) << 4));
}

/* Four 2-bit indices per byte, lowest index in the lowest bits. */
void orc_pack_crumbs(const uint8_t *idx, int n, uint8_t *out)
{
    for (int i = 0; i < n / 4; i++)
        out[i] = (uint8_t)((idx[4 * i] & 3u) | ((idx[4 * i + 1] & 3u) << 2) |
                           ((idx[4 * i + 2] & 3u) << 4) |
                           ((idx[4 * i + 3] & 3u) << 6));
}

/* ------------------------------------------------------------------ */
/* OrbitQuant normalized-basis codebook quantizer                       */
/* ------------------------------------------------------------------ */

/*
 * Squared norm of one rotated token on an exact integer grid.
 *   M = max |u[j]|;  M == 0 -> returns 0 and *E_out = 0.
 *   E = ilogb(M)  (2^E <= M < 2^(E+1))
 *   e[j] = rne_f64(u[j]^2 * 2^(36 - 2E))   (u[j]^2 exact in fp64)
 *   S = sum e[j]  (integers below 2^38, K <= 2^14: every partial sum is
 *                  an integer below 2^53, exact in any order)
 *   d = S * 2^(2E - 36)
 * Returned: d.
 */
double orc_norm2_grid(const float *u, int K)
{
    float M = 0.0f;
    for (int j = 0; j < K; j++) {
        float a = fabsf(u[j]);
        if (a > M)
            M = a;
    }
    if (M == 0.0f)
        return 0.0;
    int E = ilogbf(M);
    double S = 0.0;
    for (int j = 0; j < K; j++) {
        double sq = (double)u[j] * (double)u[j];
        S += rint(ldexp(sq, 36 - 2 * E));
    }
    return ldexp(S, 2 * E - 36);
}

/*
 * Activation quantizer of the Lloyd-Max variant ([ORBIT] abstract: quantize
 * in a normalized, rotated basis with one fixed codebook).
 *   d = orc_norm2_grid(u);   d == 0 -> indices 0, sigma 0
 *   g = (float) sqrt(K / d)            (fp64 divide and sqrt, then to fp32)
 *   v[j] = fl32(u[j] * g)              (v = sqrt(K) u / |u|)
 *   idx[j] = #{ i in 0..L-2 : v[j] > theta[i] },
 *            theta[i] = (levels[i] + levels[i+1]) / 2  (exact: bf16 levels)
 *   sigma = (float) sqrt(d / K)
 * levels: L ascending fp32 values.
 */
void orc_quant_lloydmax_row(const float *u, int K, const float *levels, int L,
                            uint8_t *idx, float *sigma_out)
{
    double d = orc_norm2_grid(u, K);
    if (d == 0.0) {
        for (int j = 0; j < K; j++)
            idx[j] = 0;
        *sigma_out = 0.0f;
        return;
    }
    float g = (float)sqrt((double)K / d);
    for (int j = 0; j < K; j++) {
        float v = u[j] * g;
        int count = 0;
        for (int i = 0; i + 1 < L; i++) {
            float theta = (levels[i] + levels[i + 1]) / 2.0f;
            if (v > theta)
                count++;
        }
        idx[j] = (uint8_t)count;
    }
    *sigma_out = (float)sqrt(d / (double)K);
}

/*
 * Weight-row quantizer of the Lloyd-Max variant ([ORBIT] abstract: the same
 * quantizer applied to weight rows offline, rotation absorbed).  fp64:
 *   nrm = sqrt(sum_k v[k]^2)  (k ascending);  nrm == 0 -> idx 0, tau 0
 *   w_hat[k] = v[k] * (sqrt(K) / nrm)
 *   idx[k] = #{ i : w_hat[k] > (levels[i] + levels[i+1]) / 2 }
 *   tau = (float)(nrm / sqrt(K))
 */
void orc_quant_lloydmax_wrow(const double *v, int K, const float *levels, int L,
                             uint8_t *idx, float *tau_out)
{
    double ss = 0.0;
    for (int k = 0; k < K; k++)
        ss += v[k] * v[k];
    double nrm = sqrt(ss);
    if (nrm == 0.0) {
        for (int k = 0; k < K; k++)
            idx[k] = 0;
        *tau_out = 0.0f;
        return;
    }
    double scale = sqrt((double)K) / nrm;
    for (int k = 0; k < K; k++) {
        double wh = v[k] * scale;
        int count = 0;
        for (int i = 0; i + 1 < L; i++) {
            double theta = ((double)levels[i] + (double)levels[i + 1]) / 2.0;
            if (wh > theta)
                count++;
        }
        idx[k] = (uint8_t)count;
    }
    *tau_out = (float)(nrm / sqrt((double)K));
}

/* ------------------------------------------------------------------ */
/* Row drivers (OpenMP over independent rows; arithmetic per row as above) */
/* ------------------------------------------------------------------ */

/* Widen an input row (fp32 or bf16 bit patterns) to fp32, exactly. */
static void widen_row(const void *X, int xdtype, size_t row, int K, float *out)
{
    if (xdtype == 0) {
        memcpy(out, (const float *)X + row * (size_t)K, (size_t)K * 4);
    } else {
        const uint16_t *h = (const uint16_t *)X + row * (size_t)K;
        for (int k = 0; k < K; k++)
            out[k] = orc_bf16_to_f32(h[k]);
    }
}

/* A rotation as the row drivers take it. */
typedef struct {
    int kind;             /* 0: RPBH, 1: dense, 2: TR-DQ */
    int b;                /* RPBH / TR-DQ block */
    const int8_t *sign;   /* RPBH signs [K] */
    const int32_t *perm;  /* RPBH / TR-DQ permutation [K] */
    const float *R;       /* dense basis [K][K]; TR-DQ first block rotation [K/b][b][b] */
    const float *m;       /* TR-DQ per-channel multiplier [K] */
    const float *R2;      /* TR-DQ second block rotation [K/b][b][b] */
} orc_rot;

static void rotate_row_f32(const orc_rot *rot, const float *x, int K, float *u)
{
    if (rot->kind == 0)
        orc_rpbh_row_f32(x, K, rot->b, rot->sign, rot->perm, u);
    else if (rot->kind == 1)
        orc_dense_row_f32(x, rot->R, K, u);
    else
        orc_trdq_row_f32(x, K, rot->b, rot->m, rot->R, rot->perm, rot->R2, u);
}

static void rotate_row_f64(const orc_rot *rot, const double *w, int K, double *v)
{
    if (rot->kind == 0)
        orc_rpbh_row_f64(w, K, rot->b, rot->sign, rot->perm, v);
    else if (rot->kind == 1)
        orc_dense_row_f64(w, rot->R, K, v);
    else
        orc_trdq_row_f64(w, K, rot->b, rot->m, rot->R, rot->perm, rot->R2, v);
}

/*
 * Activation side of the layer for a list of rows.
 *   rot      the rotation (RPBH, dense R with top-r bf16, or TR-DQ)
 *   q_kind   0: symmetric integer, a_bits 4, 6 or 8 (qmax 7, 31, 127) ->
 *               codes [nrows][K-r] as nibbles (4) or int8 bytes (6, 8),
 *               scale[nrows]
 *            1: Lloyd-Max (levels, L=16) -> codes [nrows][K/2] nibbles of the
 *               4-bit index, scale[nrows] = sigma
 *            2: asymmetric integer, a_bits 4, 6 or 8 (r = 0; 15, 63, 255
 *               levels) -> unsigned nibbles (4) or bytes (6, 8) [nrows][K],
 *               scale[nrows] = s, zero[nrows] = z
 *            3: MXFP4 (r = 0) -> codes [nrows][K/2] E2M1 nibbles,
 *               mx_scales [nrows][K/32] E8M0 codes
 *   top: bf16 [nrows][r] (dense only), may be NULL when r == 0.
 *   u_out: optional fp32 [nrows][K] copy of the rotated rows.
 * rows: indices into X (nrows of them).  Codes pack low nibble = even index.
 */
void orc_act_rows(const void *X, int xdtype, int K, const int64_t *rows, int64_t nrows,
                  const orc_rot *rot, int r, int q_kind, int a_bits, const float *levels,
                  int L, uint8_t *codes, float *scale, float *zero, uint16_t *top,
                  uint8_t *mx_scales, float *u_out)
{
    int Kq = K - r;
    /* 4-bit codes two per byte, 6- and 8-bit codes one per byte */
    const int a_bytes = a_bits != 4;
    int row_bytes = q_kind == 3 || q_kind == 1 ? K / 2 : (a_bytes ? Kq : Kq / 2);
#pragma omp parallel
    {
        float *x = (float *)malloc((size_t)K * 4);
        float *u = (float *)malloc((size_t)K * 4);
        int16_t *q = (int16_t *)malloc((size_t)K * sizeof(int16_t));
        uint16_t *ix = (uint16_t *)malloc((size_t)K * sizeof(uint16_t));
        uint8_t *b8 = (uint8_t *)malloc((size_t)K);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; i++) {
            uint8_t *crow = codes + (size_t)i * row_bytes;
            widen_row(X, xdtype, (size_t)rows[i], K, x);
            rotate_row_f32(rot, x, K, u);
            if (u_out)
                memcpy(u_out + (size_t)i * K, u, (size_t)K * 4);
            if (q_kind == 0) {
                orc_quant_sym_row(u, K, r, (1 << (a_bits - 1)) - 1, q, &scale[i]);
                if (a_bytes) {
                    for (int j = 0; j < Kq; j++)
                        crow[j] = (uint8_t)(int8_t)q[j];
                } else {
                    for (int j = 0; j < Kq; j++)
                        b8[j] = (uint8_t)(int8_t)q[j];
                    orc_pack_nibbles((const int8_t *)b8, Kq, crow);
                }
                for (int j = 0; j < r; j++)
                    top[(size_t)i * r + j] = orc_f32_to_bf16(u[j]);
            } else if (q_kind == 2) {
                orc_quant_asym_row(u, K, (1 << a_bits) - 1, ix, &scale[i], &zero[i]);
                if (a_bytes) {
                    for (int j = 0; j < K; j++)
                        crow[j] = (uint8_t)ix[j];
                } else {
                    for (int j = 0; j < K / 2; j++)
                        crow[j] = (uint8_t)((ix[2 * j] & 0x0Fu) | ((ix[2 * j + 1] & 0x0Fu) << 4));
                }
            } else if (q_kind == 3) {
                orc_quant_mxfp4_row(u, K, crow, mx_scales + (size_t)i * (K / 32));
            } else {
                orc_quant_lloydmax_row(u, K, levels, L, b8, &scale[i]);
                for (int j = 0; j < K / 2; j++)
                    crow[j] = (uint8_t)((b8[2 * j] & 0x0Fu) | ((b8[2 * j + 1] & 0x0Fu) << 4));
            }
        }
        free(x); free(u); free(q); free(ix); free(b8);
    }
}

/*
 * Weight side (offline): fold every row of W [N][K] (fp32) with the rotation
 * in fp64, then quantize.
 *   q_kind 0, 2: symmetric integer over all K, w_bits 4, 6 or 8 (qmax 7,
 *             31, 127) -> codes [N][K/2] nibbles (4) or [N][K] int8 bytes
 *             (6, 8), scale s_w[N]; qvals
 *             (optional) [N][K] signed codes
 *   q_kind 1: Lloyd-Max (levels, L = 4 or 16) -> codes [N][K/4] crumbs
 *             (L = 4) or [N][K/2] nibbles (L = 16), scale tau[N];
 *             qvals (optional) [N][K] indices
 *   q_kind 3: MXFP4 -> codes [N][K/2] E2M1 nibbles, mx_scales [N][K/32];
 *             qvals (optional) [N][K] E2M1 codes
 */
void orc_weight_rows(const float *W, int N, int K, const orc_rot *rot, int q_kind, int w_bits,
                     const float *levels, int L, uint8_t *codes, float *scale,
                     uint8_t *mx_scales, int16_t *qvals)
{
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)K * 8);
        double *v = (double *)malloc((size_t)K * 8);
        int16_t *q = (int16_t *)malloc((size_t)K * sizeof(int16_t));
        uint8_t *b8 = (uint8_t *)malloc((size_t)K);
#pragma omp for schedule(static)
        for (int n = 0; n < N; n++) {
            for (int k = 0; k < K; k++)
                w[k] = (double)W[(size_t)n * K + k];
            rotate_row_f64(rot, w, K, v);
            if (q_kind == 0 || q_kind == 2) {
                orc_quant_sym_wrow(v, K, (1 << (w_bits - 1)) - 1, q, &scale[n]);
                for (int k = 0; k < K; k++)
                    b8[k] = (uint8_t)(int8_t)q[k];
                if (w_bits != 4)
                    memcpy(codes + (size_t)n * K, b8, (size_t)K);
                else
                    orc_pack_nibbles((const int8_t *)b8, K, codes + (size_t)n * (K / 2));
                if (qvals)
                    memcpy(qvals + (size_t)n * K, q, (size_t)K * sizeof(int16_t));
            } else if (q_kind == 3) {
                uint8_t *crow = codes + (size_t)n * (K / 2);
                orc_quant_mxfp4_f64(v, K, crow, mx_scales + (size_t)n * (K / 32));
                if (qvals)
                    for (int k = 0; k < K; k++)
                        qvals[(size_t)n * K + k] = (int16_t)((crow[k >> 1] >> ((k & 1) * 4)) & 0xF);
            } else {
                orc_quant_lloydmax_wrow(v, K, levels, L, b8, &scale[n]);
                if (L == 16)
                    orc_pack_nibbles((const int8_t *)b8, K, codes + (size_t)n * (K / 2));
                else
                    orc_pack_crumbs(b8, K, codes + (size_t)n * (K / 4));
                if (qvals)
                    for (int k = 0; k < K; k++)
                        qvals[(size_t)n * K + k] = (int16_t)b8[k];
            }
        }
        free(w); free(v); free(q); free(b8);
    }
}

/* ------------------------------------------------------------------ */
/* Integer GEMM and fp64 dequantized output                             */
/* ------------------------------------------------------------------ */

/* Sign-extend nibble i of a packed row. */
static int nib(const uint8_t *row, int i)
{
    int v = (row[i >> 1] >> ((i & 1) * 4)) & 0xF;
    return v >= 8 ? v - 16 : v;
}

/*
 * acc[p] = sum_{k < Kq} qa[t_p][k] * qw[n_p][koff + k]   in int64, for the
 * (t, n) pairs listed (t from a_rows index into codes_a, n into codes_w).
 * codes_a: [*][Kq/2] nibbles; codes_w: [N][Kw/2] nibbles.  koff = r for the
 * DiRotQ path (the INT4 activation coordinates start after the top-r ones).
 */
void orc_int_gemm_pairs(const uint8_t *codes_a, int Kq, const uint8_t *codes_w,
                        int Kw, int koff, const int64_t *ta, const int64_t *nw,
                        int64_t npairs, int64_t *acc)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++) {
        const uint8_t *ra = codes_a + (size_t)ta[p] * (Kq / 2);
        const uint8_t *rw = codes_w + (size_t)nw[p] * (Kw / 2);
        int64_t s = 0;
        for (int k = 0; k < Kq; k++)
            s += (int64_t)nib(ra, k) * (int64_t)nib(rw, koff + k);
        acc[p] = s;
    }
}

/*
 * Asymmetric activations: acc[p] = sum_{k < K} ua[t_p][k] * qw[n_p][k] in
 * int64, ua the unsigned activation codes (0..15), qw the signed weight
 * codes.  The layer output subtracts z[t] * sum_k qw[n][k] (see oracle.py).
 */
void orc_asym_gemm_pairs(const uint8_t *codes_a, int K, const uint8_t *codes_w,
                         const int64_t *ta, const int64_t *nw, int64_t npairs, int64_t *acc)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++) {
        const uint8_t *ra = codes_a + (size_t)ta[p] * (K / 2);
        const uint8_t *rw = codes_w + (size_t)nw[p] * (K / 2);
        int64_t s = 0;
        for (int k = 0; k < K; k++) {
            int ua = (ra[k >> 1] >> ((k & 1) * 4)) & 0xF;
            s += (int64_t)ua * (int64_t)nib(rw, k);
        }
        acc[p] = s;
    }
}

/* Full int64 accumulator block acc[T][N] (small shapes). */
void orc_int_gemm(const uint8_t *codes_a, int T, int Kq, const uint8_t *codes_w,
                  int N, int Kw, int koff, int64_t *acc)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        const uint8_t *ra = codes_a + (size_t)t * (Kq / 2);
        for (int n = 0; n < N; n++) {
            const uint8_t *rw = codes_w + (size_t)n * (Kw / 2);
            int64_t s = 0;
            for (int k = 0; k < Kq; k++)
                s += (int64_t)nib(ra, k) * (int64_t)nib(rw, koff + k);
            acc[(size_t)t * N + n] = s;
        }
    }
}

/*
 * Low-rank term of the DiRotQ path for listed pairs, fp64:
 *   lr[p] = sum_{j < r} bf16(top[t][j]) * qw[n][j]
 */
void orc_lowrank_pairs(const uint16_t *top, int r, const uint8_t *codes_w, int Kw,
                       const int64_t *ta, const int64_t *nw, int64_t npairs,
                       double *lr)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++) {
        const uint16_t *tr = top + (size_t)ta[p] * r;
        const uint8_t *rw = codes_w + (size_t)nw[p] * (Kw / 2);
        double s = 0.0;
        for (int j = 0; j < r; j++)
            s += (double)orc_bf16_to_f32(tr[j]) * (double)nib(rw, j);
        lr[p] = s;
    }
}

/*
 * Codebook dot product of the Lloyd-Max variant for listed pairs, fp64:
 *   dot[p] = sum_k a_lv[idx_a[t][k]] * w_lv[idx_w[n][k]]
 * codes_a: [*][K/2] nibbles (4-bit index); codes_w: [N][K/4] crumbs
 * (w_bits 2) or [N][K/2] nibbles (w_bits 4).
 */
void orc_codebook_dot_pairs(const uint8_t *codes_a, const uint8_t *codes_w, int K, int w_bits,
                            const float *a_lv, const float *w_lv,
                            const int64_t *ta, const int64_t *nw, int64_t npairs,
                            double *dot)
{
    const int per_byte = 8 / w_bits;
    const int mask = (1 << w_bits) - 1;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++) {
        const uint8_t *ra = codes_a + (size_t)ta[p] * (K / 2);
        const uint8_t *rw = codes_w + (size_t)nw[p] * (K / per_byte);
        double s = 0.0;
        for (int k = 0; k < K; k++) {
            int ia = (ra[k >> 1] >> ((k & 1) * 4)) & 0xF;
            int iw = (rw[k / per_byte] >> ((k % per_byte) * w_bits)) & mask;
            s += (double)a_lv[ia] * (double)w_lv[iw];
        }
        dot[p] = s;
    }
}

/* Code i of a row of `bits`-bit codes (4: nibbles, low nibble = even index;
 * 6 and 8: one per byte), two's complement in its container (nibble or
 * byte) when is_signed, else unsigned. */
static int code_at(const uint8_t *row, int bits, int is_signed, int i)
{
    const int cont = bits == 4 ? 4 : 8;
    int v = cont == 8 ? row[i] : (row[i >> 1] >> ((i & 1) * 4)) & 0xF;
    if (is_signed) {
        int half = 1 << (cont - 1);
        if (v >= half)
            v -= 2 * half;
    }
    return v;
}

/*
 * Integer GEMM of 4-, 6- or 8-bit codes for listed pairs, int64:
 *   acc[p] = sum_{k < Kq} a[t_p][k] * w[n_p][koff + k]
 * a: rows of Kq codes of a_bits (signed or unsigned); w: rows of Kw signed
 * codes of w_bits.  (W4A4, and the W4A8, W8A8 and W6A6 settings of the
 * "TR-DQ" page's tables.)
 */
void orc_gemm_codes_pairs(const uint8_t *codes_a, int a_bits, int a_signed, int Kq,
                          const uint8_t *codes_w, int w_bits, int Kw, int koff,
                          const int64_t *ta, const int64_t *nw, int64_t npairs, int64_t *acc)
{
    size_t arow = a_bits == 4 ? (size_t)Kq / 2 : (size_t)Kq, wrow = w_bits == 4 ? (size_t)Kw / 2 : (size_t)Kw;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++) {
        const uint8_t *ra = codes_a + (size_t)ta[p] * arow;
        const uint8_t *rw = codes_w + (size_t)nw[p] * wrow;
        int64_t s = 0;
        for (int k = 0; k < Kq; k++)
            s += (int64_t)code_at(ra, a_bits, a_signed, k) *
                 (int64_t)code_at(rw, w_bits, 1, koff + k);
        acc[p] = s;
    }
}

/*
 * MXFP4 dot products for listed pairs, fp64:
 *   dot[p] = sum_c 2^(ea[t][c] + ew[n][c]) sum_{k in block c} e2m1(a[t][k]) e2m1(w[n][k])
 * Every block's inner sum is exact in fp64 (multiples of 1/4 below 2^11).
 */
void orc_mx_dot_pairs(const uint8_t *codes_a, const uint8_t *sc_a, const uint8_t *codes_w,
                      const uint8_t *sc_w, int K, const int64_t *ta, const int64_t *nw,
                      int64_t npairs, double *dot)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++) {
        const uint8_t *ra = codes_a + (size_t)ta[p] * (K / 2);
        const uint8_t *rw = codes_w + (size_t)nw[p] * (K / 2);
        const uint8_t *sa = sc_a + (size_t)ta[p] * (K / 32);
        const uint8_t *sw = sc_w + (size_t)nw[p] * (K / 32);
        double s = 0.0;
        for (int c = 0; c < K / 32; c++) {
            double blk = 0.0;
            for (int k = 32 * c; k < 32 * c + 32; k++)
                blk += orc_e2m1_value((ra[k >> 1] >> ((k & 1) * 4)) & 0xF) *
                       orc_e2m1_value((rw[k >> 1] >> ((k & 1) * 4)) & 0xF);
            s += ldexp(blk, (int)sa[c] + (int)sw[c] - 254);
        }
        dot[p] = s;
    }
}

/* Threads OpenMP will use for the parallel regions above. */
int orc_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Set the OpenMP thread count of the parallel regions above. */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

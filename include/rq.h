/*
 * rq.h -- C ABI of librq, the MI355X (gfx950) rotated low-bit quantized
 * linear layer of diffusion-transformer inference.
 *
 * The layer (pages: "TR-DQ: Time-Rotation Diffusion Quantization",
 * section 3.1 and Eq.(8)-(9); "OrbitQuant" abstract; "DiRotQ" abstract):
 *
 *   Y = X . W^T  is evaluated as  Y ~ Q(X R) . Q(W R)^T
 *
 * where R is orthogonal, so the product is unchanged in exact arithmetic
 * (computational invariance, TR-DQ Eq.(9)).  W R is folded and quantized
 * offline (rq_pack_weights); at runtime only the forward rotation of the
 * activations, their per-token 4-bit quantization (rq_rotate_quant) and the
 * low-bit GEMM with the per-token x per-channel rescale (rq_w4a4_linear)
 * remain.  Two rotations are supported:
 *
 *   RPBH   randomized permuted block-Hadamard (OrbitQuant abstract):
 *          y[j] = sign[j] * x[perm[j]], then an unnormalized Sylvester
 *          Walsh-Hadamard transform on every contiguous block of `block`
 *          coordinates (TR-DQ Eq.(8): block-diagonal, 2^n x 2^n blocks).
 *          The unnormalized transform scales dot products by `block`; the
 *          GEMM epilogue divides it out.
 *   DENSE  an orthogonal basis R [K][K] (DiRotQ abstract: PCA basis from
 *          calibration); the first r rotated coordinates of every token are
 *          kept in bf16, the remaining K - r quantized to 4 bits.
 *
 * and two quantizers:
 *
 *   INT4_SYM   symmetric round-to-nearest-even INT4 in [-7, 7], one fp32
 *              scale per token (activations) / per output channel (weights)
 *              (TR-DQ Eq.(1)-(2) with a zero point of 0; granularity from
 *              TR-DQ section 3.1).
 *   LLOYDMAX   OrbitQuant's normalized-basis quantizer: a token is scaled to
 *              norm sqrt(K) and every coordinate is coded by the nearest of
 *              2^a_bits fixed levels (a Lloyd-Max codebook of N(0,1)); weight
 *              rows likewise with 2^w_bits levels.  The token norm sigma and
 *              the row norm tau (both divided by sqrt(K)) rescale the output.
 *
 * Conventions for every entry point:
 *   - Pointers documented "device" must be device memory of the current HIP
 *     device (torch tensors are fine); "host" pointers are CPU memory.
 *   - The caller owns and allocates every buffer; the library allocates no
 *     memory on the runtime path and keeps no state besides a thread-local
 *     error message and its loaded kernels.  Calls are re-entrant.
 *   - Runtime calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).  Inputs are read only; outputs must not alias inputs.
 *   - Every call validates its arguments before touching the GPU and returns
 *     an rq_status; nothing aborts.  rq_last_error() describes the last
 *     non-OK status of the calling thread.  Faults during kernel execution
 *     surface at the caller's next synchronization.
 *   - Token counts T may be 0 (the call returns RQ_OK and launches nothing).
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rq_status {
    RQ_OK = 0,
    RQ_ERR_NULL = -1,        /* a required pointer is NULL */
    RQ_ERR_SHAPE = -2,       /* a size violates the constraints stated below */
    RQ_ERR_DTYPE = -3,       /* unsupported dtype code */
    RQ_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
    RQ_ERR_FORMAT = -5,      /* weight header magic/version/format mismatch */
    RQ_ERR_UNSUPPORTED = -6, /* valid but unsupported combination */
    RQ_ERR_HIP = -7          /* a HIP runtime call failed (message has details) */
} rq_status;

typedef enum rq_dtype {
    RQ_F32 = 0,   /* IEEE binary32 */
    RQ_BF16 = 1,  /* bfloat16 bit patterns (uint16) */
    RQ_I32 = 2    /* raw int32 accumulators (rq_w4a4_linear output only) */
} rq_dtype;

typedef enum rq_rot_kind { RQ_ROT_RPBH = 0, RQ_ROT_DENSE = 1 } rq_rot_kind;
typedef enum rq_q_kind { RQ_Q_INT4_SYM = 0, RQ_Q_LLOYDMAX = 1, RQ_Q_INT4_ASYM = 2 } rq_q_kind;

/*
 * Rotation descriptor.  Pointer members are host pointers for
 * rq_pack_weights and device pointers for rq_rotate_quant.
 *   kind   rq_rot_kind
 *   K      input features; 32 <= K <= 16384, K % 32 == 0
 *   block  RPBH: b, a power of two, 2 <= b <= 1024, K % b == 0
 *   r      DENSE: coordinates kept in bf16, 0 <= r < K, r % 32 == 0; RPBH: 0
 *   sign   RPBH: int8 [K], each -1 or +1
 *   perm   RPBH: int32 [K], a permutation of 0..K-1 (not checked on device)
 *          (rq_rotate_quant reads both as 16-byte vectors: the device copies
 *          must be 16-byte aligned, else RQ_ERR_ALIGN)
 *   R      DENSE: fp32 [K][K] row-major, column j is basis vector j
 */
typedef struct rq_rotation {
    int32_t kind;
    int32_t K;
    int32_t block;
    int32_t r;
    const int8_t *sign;
    const int32_t *perm;
    const float *R;
} rq_rotation;

/*
 * Quantizer descriptor (plain values, no pointers).
 *   kind      rq_q_kind.  INT4_ASYM: activations per token with a zero point
 *             (TR-DQ section 3.1 Eq.(1)-(3)), weights as INT4_SYM; RPBH only
 *   a_bits    4
 *   w_bits    INT4_SYM, INT4_ASYM: 4;  LLOYDMAX: 2 or 4
 *   a_levels  LLOYDMAX: 2^a_bits strictly ascending, bf16-representable
 *   w_levels  LLOYDMAX: 2^w_bits strictly ascending, bf16-representable
 */
typedef struct rq_quant {
    int32_t kind;
    int32_t a_bits;
    int32_t w_bits;
    int32_t reserved;
    float a_levels[16];
    float w_levels[16];
} rq_quant;

#define RQ_WEIGHT_MAGIC 0x31575152u /* "RQW1" */
#define RQ_WEIGHT_VERSION 2u

/*
 * Header at the start of every packed-weight blob (256 bytes).  The blob is
 * written on the host by rq_pack_weights and copied to the device by the
 * caller unchanged; rq_w4a4_linear reads this header from host memory and
 * the rest of the blob from device memory.
 *   format        rq_q_kind of the weights
 *   K, N          input / output features
 *   r             DENSE top-r (0 otherwise)
 *   b_div         epilogue divisor: the RPBH block, 1 for DENSE
 *   row_bytes     bytes per packed weight row (K/2 for INT4, K/4 for 2-bit)
 *   scale_offset  byte offset of fp32 [N] (INT4: s_w; LLOYDMAX: tau)
 *   codes_offset  byte offset of the packed codes [N][row_bytes]
 *                 INT4: two's-complement nibbles, low nibble = even k;
 *                 LLOYDMAX 2-bit: four level indices per byte, lowest k in
 *                 the lowest bits
 *   total_bytes   size of the whole blob
 *   a_levels, w_levels  the LLOYDMAX decode levels (zeros for INT4)
 *   INT4 only, the GEMM's private copy of the codes of the quantized
 *   coordinates k in [r, K) (zeros for LLOYDMAX):
 *   wsum_offset   byte offset of int32 [N]: sum over k in [r, K) of q_w[n][k]
 *   mma_offset    byte offset of the FP6 matrix-core fragments,
 *                 [mma_ntiles][mma_stages][3][64][16] bytes: 32 output rows
 *                 by 128 coordinates per 3 KB tile, zero-padded past N and K
 *   mma_stages    ceil((K - r) / 128)
 *   mma_ntiles    ceil(N / 32)
 */
typedef struct rq_weight_header {
    uint32_t magic;
    uint32_t version;
    int32_t format;
    int32_t K;
    int32_t N;
    int32_t r;
    int32_t b_div;
    int32_t a_bits;
    int32_t w_bits;
    int32_t row_bytes;
    int64_t scale_offset;
    int64_t codes_offset;
    int64_t total_bytes;
    float a_levels[16];
    float w_levels[16];
    int64_t wsum_offset;
    int64_t mma_offset;
    int32_t mma_stages;
    int32_t mma_ntiles;
    uint8_t reserved[256 - 64 - 128 - 24];
} rq_weight_header;

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t rq_version(void);

/* Message for the last non-OK status returned on the calling thread
 * (empty string if none).  Valid until the thread's next rq_* call. */
const char *rq_last_error(void);

/*
 * Lloyd-Max levels of the standard normal ("OrbitQuant" abstract: one
 * Lloyd-Max codebook for the fixed, known marginal of a rotated,
 * normalized coordinate): Lloyd's iteration in fp64 (thresholds at the
 * midpoints of the levels, levels at the conditional means of their cells),
 * converged to 1e-15, then rounded to bf16 (nearest, ties to even).
 *   L       number of levels: 2, 4, 8 or 16
 *   levels  host fp32 [L], written ascending
 * Errors: RQ_ERR_NULL, RQ_ERR_SHAPE (L not in {2,4,8,16}).
 */
rq_status rq_lloydmax_gaussian(int32_t L, float *levels);

/*
 * Bytes of the packed-weight blob for N output features (header included).
 * Errors: as rq_pack_weights' descriptor checks.
 */
rq_status rq_packed_weight_bytes(const rq_rotation *rot, const rq_quant *q, int32_t N,
                                 size_t *bytes);

/*
 * Offline weight preparation ("DiRotQ" abstract: the inverse rotation is
 * fused into the layer weights offline; "OrbitQuant" abstract: the rotation
 * absorbed into the weights cancels inside the layer; TR-DQ Eq.(9)).
 * Untimed, host only, no GPU call.  For every output row n of W [N][K]:
 *   fold   v = w_n R in fp64 (RPBH: the same sign, permutation and
 *          ascending-stage butterflies as the activations, in fp64;
 *          DENSE: fp64 fused multiply-add chain over k ascending)
 *   INT4   amax = max |v|; s_w = (float)(amax / 7); codes
 *          clamp(rne(v * (7 / amax)), -7, 7) in fp64 (amax == 0: codes 0,
 *          s_w 0) -- symmetric per-output-channel round-to-nearest
 *   LLOYDMAX  nrm = |v| (fp64, k ascending); codes = nearest of w_levels
 *          to v * sqrt(K) / nrm (ties to the lower level); tau = nrm / sqrt(K)
 * Arguments:
 *   rot      host descriptor, host sign/perm/R
 *   q        quantizer (w_bits 4 for INT4, 2 or 4 for LLOYDMAX)
 *   W        host [N][K], dtype w_dtype (RQ_F32 or RQ_BF16)
 *   N        output features, 1 <= N <= 2^20
 *   blob     host buffer of blob_bytes >= rq_packed_weight_bytes(), written
 * Errors: RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_DTYPE, RQ_ERR_UNSUPPORTED.
 */
rq_status rq_pack_weights(const rq_rotation *rot, const rq_quant *q, const void *W,
                          int32_t w_dtype, int32_t N, void *blob, size_t blob_bytes);

/*
 * Bytes of device workspace rq_rotate_quant needs (0 for RPBH; T*K*4 for
 * DENSE, which stages the rotated tokens in fp32).
 */
rq_status rq_rotate_quant_workspace_bytes(const rq_rotation *rot, const rq_quant *q,
                                          int64_t T, size_t *bytes);

/*
 * Bytes of a codes_mma buffer for T tokens (rq_rotate_quant's optional
 * output, rq_w4a4_linear's optional input):
 * ceil(T / 32) * ceil((K - r) / 128) * 3072.
 * Errors: RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_UNSUPPORTED.
 */
rq_status rq_codes_mma_bytes(const rq_rotation *rot, int64_t T, size_t *bytes);

/*
 * Runtime activation path: rotate and quantize T tokens.
 * ("OrbitQuant" abstract: only a forward rotation of the activations
 * remains at runtime; TR-DQ section 3.2: quantization parameters are
 * computed online per token from the extremes.)
 *   RPBH:  u = the block Walsh-Hadamard transform of y, y[j] = sign[j] x[perm[j]],
 *          radix-2 butterflies (lo, hi) -> (lo + hi, lo - hi) in fp32,
 *          stages h = 1, 2, 4, ..., block/2 in that order.
 *   DENSE: u[j] = fp32 fused multiply-add chain over k ascending of
 *          x[k] * R[k][j], starting from +0.
 *   INT4_SYM: over the quantized coordinates j in [r, K):
 *          amax = max |u[j]|; s = fl32(amax / 7); inv = fl32(7 / amax)
 *          q[j] = clamp(rne(fl32(u[j] * inv)), -7, 7); amax == 0 -> 0, s = 0.
 *          DENSE also writes top[t][j] = bf16_rne(u[j]) for j < r.
 *   INT4_ASYM (RPBH): lo = min u, hi = max u, d = fl32(hi - lo);
 *          s = fl32(d / 15); inv = fl32(15 / d);
 *          z = clamp(-rne(fl32(lo * inv)), 0, 15) (an integer);
 *          q[j] = clamp(rne(fl32(u[j] * inv)) + z, 0, 15); d == 0 -> 0, s = z = 0.
 *   LLOYDMAX: d = |u|^2 on an exact integer grid (order independent),
 *          g = (float)sqrt(K / d); index[j] = number of midpoints of adjacent
 *          a_levels strictly below fl32(u[j] * g); sigma = (float)sqrt(d / K).
 * Arguments:
 *   rot     host descriptor with device sign/perm (RPBH) or R (DENSE)
 *   q       quantizer (INT4_SYM with RPBH or DENSE; INT4_ASYM and LLOYDMAX
 *           with RPBH)
 *   X       device [T][K] tokens, row-major, dtype x_dtype (RQ_F32/RQ_BF16),
 *           16-byte aligned
 *   T       tokens, 0 <= T < 2^31
 *   codes   device uint8 [T][(K - r) / 2]: INT4_SYM nibbles (two's complement,
 *           low nibble = even coordinate), INT4_ASYM unsigned nibbles, or
 *           LLOYDMAX 4-bit indices, same packing.  May be NULL for RPBH
 *           INT4 when codes_mma is given.
 *   scale   device fp32 [T]: s (INT4_SYM) or sigma (LLOYDMAX); INT4_ASYM:
 *           fp32 [2][T], s[t] then the zero point z[t]
 *   top     device bf16 [T][r] for DENSE with r > 0, else NULL
 *   codes_mma  RPBH INT4 only, optional: device buffer of
 *           rq_codes_mma_bytes() receiving the same codes in the low-bit
 *           GEMM's matrix-core layout (NULL: not written).  Tokens come in
 *           tiles of 32 and coordinates in stages of 128; the buffer is
 *           [tile][stage][piece 0..2][lane 0..63][16 bytes], 3 KB per tile
 *           and stage.  Token t of a tile owns lanes t and t + 32 (half h);
 *           its twelve dwords f[0..11] for half h of a stage are dword d % 4
 *           of its lane in piece d / 4.  f[0..5] and f[6..11] are the 192-bit
 *           fragments of coordinates 128 s + 64 ks + 32 h + (0..31) for
 *           ks = 0, 1; bits [6 e, 6 e + 6) of a fragment hold the E2M3 code
 *           u (value u / 8, top two bits clear; u = q + 8 for INT4_SYM, the
 *           unsigned code for INT4_ASYM) of coordinate offset
 *           {0,1,3,4,6,7,9,10,12,13,15,8,2,11,5,14}[e % 16] + 16 (e / 16).
 *           Bytes of tokens past T and coordinates past K - r are left
 *           unwritten.
 *   workspace, workspace_bytes  device scratch of at least
 *           rq_rotate_quant_workspace_bytes() (NULL/0 when that is 0)
 *   stream  hipStream_t
 * Errors: RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_DTYPE, RQ_ERR_ALIGN,
 *         RQ_ERR_UNSUPPORTED, RQ_ERR_HIP.
 */
rq_status rq_rotate_quant(const rq_rotation *rot, const rq_quant *q, const void *X,
                          int32_t x_dtype, int64_t T, uint8_t *codes, float *scale,
                          uint16_t *top, uint8_t *codes_mma, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Runtime low-bit GEMM with the per-token x per-channel rescale
 * (TR-DQ section 3.1: Y = X W with per-token activation and per-channel
 * weight scales; DiRotQ abstract: the top principal coefficients add a
 * higher-precision term).
 *   INT4:  acc[t][n] = sum_{k < K-r} q_a[t][k] * q_w[n][r + k]  (exact, int32);
 *          INT4_ASYM: q_a[t][k] = u_a[t][k] - z[t] (codes minus zero point)
 *          RPBH:  Y = s_a[t] s_w[n] acc / b_div
 *          DENSE: Y = s_w[n] (lr[t][n] + s_a[t] acc), with
 *                 lr = sum_{j < r} top[t][j] * q_w[n][j] (bf16 x int4 products,
 *                 fp32 accumulation)
 *   LLOYDMAX: Y = sigma[t] tau[n] / b_div * sum_k a_levels[idx_a] * w_levels[idx_w]
 *          (bf16 products, fp32 accumulation)
 *   + bias[n] when bias is not NULL.
 * INT4 weights run on the FP6 (E2M3) matrix cores: activation codes become
 * q + 8, weight codes q, both exact in E2M3, and the per-channel sum of the
 * weight codes (in the blob) removes the offset; every partial sum is an
 * integer below 2^24, so the fp32 accumulation is exact.  With
 * RQ_W4A4_MFMA=int8 in the environment the int8 matrix cores run instead
 * (codes must then be given; INT4_SYM only).
 * Arguments:
 *   hdr     host pointer to the blob's header (its first 256 bytes)
 *   blob    device copy of the whole blob, 16-byte aligned
 *   codes, scale, top  as written by rq_rotate_quant (device); the weights'
 *           format (INT4_SYM / INT4_ASYM) must match the activations' quantizer
 *   codes_mma  optional (INT4 weights with r == 0): the codes_mma output of
 *           rq_rotate_quant for the same tokens; when given it is read
 *           instead of codes (which may then be NULL)
 *   T       tokens, 0 <= T < 2^31
 *   bias    device fp32 [N] or NULL
 *   Y       device [T][N], dtype y_dtype: RQ_F32, RQ_BF16 (nearest-even), or
 *           RQ_I32 = the exact INT4 accumulators acc (INT4 formats only;
 *           the low-rank term and bias are left out)
 *   stream  hipStream_t
 * Errors: RQ_ERR_NULL, RQ_ERR_FORMAT, RQ_ERR_SHAPE, RQ_ERR_DTYPE,
 *         RQ_ERR_ALIGN, RQ_ERR_UNSUPPORTED, RQ_ERR_HIP.
 */
rq_status rq_w4a4_linear(const rq_weight_header *hdr, const void *blob, const uint8_t *codes,
                         const float *scale, const uint16_t *top, const uint8_t *codes_mma,
                         int64_t T, const float *bias, void *Y, int32_t y_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */

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
 * remain.  Three rotations are supported:
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
 *   TRDQ   TR-DQ's runtime rotation (section 3.2, Eq.(9)-(10)): a
 *          per-channel smoothing multiplier, a block rotation R1, the
 *          zigzag permutation, a block rotation R2.
 *
 * and three quantizer families:
 *
 *   INT (RQ_Q_INT4_SYM / RQ_Q_INT4_ASYM, a_bits 4, 6 or 8, w_bits 4, 6
 *        or 8; 6- and 8-bit codes are stored one per byte)
 *              round-to-nearest-even integers, one fp32 scale per token
 *              (activations, symmetric in [-qmax, qmax] or asymmetric in
 *              [0, 2^b - 1] with a zero point) and per output channel
 *              (weights, symmetric) (TR-DQ Eq.(1)-(3); granularity from
 *              TR-DQ section 3.1; its W4A8 / W8A8 settings).
 *   LLOYDMAX   OrbitQuant's normalized-basis quantizer: a token is scaled to
 *              norm sqrt(K) and every coordinate is coded by the nearest of
 *              2^a_bits fixed levels (a Lloyd-Max codebook of N(0,1)); weight
 *              rows likewise with 2^w_bits levels.  The token norm sigma and
 *              the row norm tau (both divided by sqrt(K)) rescale the output.
 *   MXFP4      the FP4 variant (DiRotQ abstract, later version: NVFP4 on a
 *              Blackwell GPU), read as OCP MX v1.0 MXFP4: E2M1 elements, one
 *              E8M0 power-of-two scale per 32 consecutive coordinates,
 *              e = floor(log2 max|x|) - 2, elements rounded to nearest with
 *              ties to even and saturated at 6 -- the format gfx950's scaled
 *              matrix cores take.
 *
 * Conventions for every entry point:
 *   - Pointers documented "device" must be device memory of the current HIP
 *     device (torch tensors are fine); "host" pointers are CPU memory.
 *   - The caller owns and allocates every buffer; the library allocates no
 *     memory on the runtime path and keeps no state besides a thread-local
 *     error message, its loaded kernels and per-device launch facts (compute-unit
 *     count, raised LDS limits) that it caches under a lock.  Host threads may
 *     call in concurrently; calls on one stream run in issue order.
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

/* Matrix cores that run an INT4 GEMM (rq_w4a4_linear_engine).
 *   AUTO  the library's choice: FP6 for INT weights with 4-bit activations,
 *         int8 for 6- and 8-bit activations, the scaled FP4 cores for MXFP4, the
 *         codebook kernel for Lloyd-Max weights
 *   FP6   E2M3 operands on v_mfma_scale_f32_32x32x64_f8f6f4: codes carried
 *         exactly, fp32 accumulation exact, twice the int8 rate
 *   INT8  v_mfma_i32_32x32x32_i8 with the nibbles widened to int8 in
 *         registers, int32 accumulation (INT4_SYM weights, canonical codes) */
typedef enum rq_engine { RQ_ENGINE_AUTO = 0, RQ_ENGINE_FP6 = 1, RQ_ENGINE_INT8 = 2 } rq_engine;

typedef enum rq_rot_kind { RQ_ROT_RPBH = 0, RQ_ROT_DENSE = 1, RQ_ROT_TRDQ = 2 } rq_rot_kind;
/* RQ_Q_INT4_SYM / RQ_Q_INT4_ASYM are the integer family at any a_bits / w_bits
 * (RQ_Q_INT_SYM / RQ_Q_INT_ASYM name the same values). */
typedef enum rq_q_kind {
    RQ_Q_INT4_SYM = 0,
    RQ_Q_LLOYDMAX = 1,
    RQ_Q_INT4_ASYM = 2,
    RQ_Q_MXFP4 = 3,
    RQ_Q_INT_SYM = 0,
    RQ_Q_INT_ASYM = 2
} rq_q_kind;

/*
 * Rotation descriptor.  Pointer members are host pointers for
 * rq_pack_weights and device pointers for rq_rotate_quant.
 *   kind   rq_rot_kind
 *   K      input features; 32 <= K <= 16384, K % 32 == 0
 *   block  RPBH: b, a power of two, 2 <= b <= 1024, K % b == 0;
 *          TRDQ: b, a power of two, 16 <= b <= 256, K % b == 0
 *   r      DENSE: coordinates kept in bf16, 0 <= r < K, r % 32 == 0; else 0
 *   sign   RPBH: int8 [K], each -1 or +1
 *   perm   RPBH: int32 [K], a permutation of 0..K-1 (not checked on device);
 *          TRDQ: the zigzag permutation as a gather, p[j] = z[perm[j]]
 *          (rq_rotate_quant reads sign and perm as 16-byte vectors: the
 *          device copies must be 16-byte aligned, else RQ_ERR_ALIGN)
 *   R      DENSE: fp32 [K][K] row-major, column j is basis vector j;
 *          TRDQ: R1, fp32 [K/b][b][b]; block c maps coordinates cb..cb+b-1:
 *          z[cb + j] = sum_i y[cb + i] R1[c][i][j]
 *   smooth TRDQ: fp32 [K], the per-channel multiplier the activations
 *          receive (y = x * smooth; TR-DQ Eq.(4)-(5): 1 / Delta); the weights
 *          are divided by it.  NULL otherwise.
 *   R2     TRDQ: fp32 [K/b][b][b], the second block rotation (as R1).
 *          NULL otherwise.
 */
typedef struct rq_rotation {
    int32_t kind;
    int32_t K;
    int32_t block;
    int32_t r;
    const int8_t *sign;
    const int32_t *perm;
    const float *R;
    const float *smooth;
    const float *R2;
} rq_rotation;

/*
 * Quantizer descriptor (plain values, no pointers).
 *   kind      rq_q_kind.  INT4_ASYM: activations per token with a zero point
 *             (TR-DQ section 3.1 Eq.(1)-(3)), weights symmetric; RPBH or TRDQ
 *   a_bits    INT kinds: 4, 6 or 8 (6, 8: RPBH or TRDQ, symmetric weights
 *             of w_bits 4, 6 or 8 -- TR-DQ's W4A8, W8A8 and W6A6 settings;
 *             4: w_bits 4);  LLOYDMAX, MXFP4: 4
 *   w_bits    INT kinds: 4, 6 or 8;  LLOYDMAX: 2 or 4;  MXFP4: 4
 *   a_levels  LLOYDMAX: 2^a_bits strictly ascending, bf16-representable
 *   w_levels  LLOYDMAX: 2^w_bits strictly ascending, bf16-representable
 * MXFP4 runs with the RPBH rotation.
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
#define RQ_WEIGHT_VERSION 5u

/*
 * Header at the start of every packed-weight blob (256 bytes).  The blob is
 * written on the host by rq_pack_weights and copied to the device by the
 * caller unchanged; rq_w4a4_linear reads this header from host memory and
 * the rest of the blob from device memory.
 *   format        rq_q_kind of the weights
 *   K, N          input / output features
 *   r             DENSE top-r (0 otherwise)
 *   b_div         epilogue divisor: the RPBH block, 1 otherwise
 *   a_bits, w_bits  as in rq_quant
 *   row_bytes     bytes per packed weight row (K/2 for 4-bit codes, K for
 *                 6- and 8-bit, K/4 for 2-bit)
 *   scale_offset  byte offset of the weight scales: fp32 [N] (INT: s_w;
 *                 LLOYDMAX: tau) or, MXFP4, the E8M0 codes uint8 [N][K/32]
 *   codes_offset  byte offset of the packed codes [N][row_bytes]
 *                 INT 4-bit: two's-complement nibbles, low nibble = even k;
 *                 INT 6- and 8-bit: int8; MXFP4: E2M1 nibbles (sign in bit 3), low
 *                 nibble = even k; LLOYDMAX 2-bit: four level indices per
 *                 byte, lowest k in the lowest bits
 *   total_bytes   size of the whole blob
 *   a_levels, w_levels  the LLOYDMAX decode levels (zeros otherwise)
 *   The GEMMs' private copies (zero when absent):
 *   wsum_offset   INT: int32 [N], sum over k in [r, K) of q_w[n][k]
 *   mma_offset    INT with a_bits 4: the FP6 matrix-core fragments of the
 *                 quantized coordinates k in [r, K),
 *                 [mma_ntiles][mma_stages][3][64][16] bytes: 32 output rows
 *                 by 128 coordinates per 3 KB tile, zero-padded past N and K;
 *                 MXFP4: the E2M1 codes tiled [mma_ntiles][K/32][32][16]:
 *                 rows in tiles of 32, each row's 16 bytes of coordinates
 *                 32 c .. 32 c + 31 (zero rows past N);
 *                 LLOYDMAX with w_bits 4: the weight levels as bf16 in the
 *                 codebook GEMM's fragment order [mma_ntiles][K/16][64][8 x
 *                 bf16]: lane i + 32 h of k-step c holds row 32 tile + i,
 *                 coordinates 16 c + 8 h .. + 7 (zero rows past N), which
 *                 the GEMM copies with direct-to-LDS loads instead of
 *                 decoding the indices (2 bytes per weight, 4x the 4-bit
 *                 codes, which stay in the blob); 2-bit weights have none
 *                 (the GEMM decodes them)
 *   mma_stages    INT, MXFP4: ceil((K - r) / 128); LLOYDMAX: 0
 *   mma_ntiles    ceil(N / 32) (0 for 2-bit LLOYDMAX weights)
 *   i8_offset     INT with a_bits 6 or 8: the int8 weight codes (the canonical
 *                 codes when w_bits is 6 or 8, their widened copy when 4) in the
 *                 int8 matrix cores' fragment order
 *                 [mma_ntiles][K/32][64 lanes][16 bytes]: lane 32 h + i of
 *                 k-step c holds coordinates 32 c + 16 h .. + 15 of row
 *                 32 tile + i (zero rows past N)
 *   mxs_offset    MXFP4: the E8M0 codes tiled [mma_stages][mma_ntiles][64][2]:
 *                 byte ks of lane 32 h + i is the scale of row 32 tile + i,
 *                 coordinates 128 s + 64 ks + 32 h .. + 31
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
    int64_t i8_offset;
    int64_t mxs_offset;
    uint8_t reserved[256 - 64 - 128 - 40];
} rq_weight_header;

/*
 * Time-step rotation sets (TR-DQ section 3.2, Eq.(10)): instead of one
 * rotation and one packed weight for every denoising step, step t selects a
 * group g = step_group[t] with its own rotation (smoothing multiplier,
 * rotations, permutation -- or any rotation kind) and its own weights folded
 * with that rotation.  A set blob is this header followed by one ordinary
 * packed-weight blob per group (memory grows with the groups).
 *   groups        G, 1 <= G <= RQ_SET_MAX_GROUPS
 *   steps         number of steps mapped, 1 <= steps <= RQ_SET_MAX_STEPS
 *   member_offset byte offset of group g's blob (256-byte aligned)
 *   step_group    group of step t, in [0, G)
 */
#define RQ_SET_MAGIC 0x53545152u /* "RQTS" */
#define RQ_SET_VERSION 1u
#define RQ_SET_MAX_GROUPS 64
#define RQ_SET_MAX_STEPS 1024
typedef struct rq_set_header {
    uint32_t magic;
    uint32_t version;
    int32_t groups;
    int32_t steps;
    int64_t member_offset[RQ_SET_MAX_GROUPS];
    int32_t step_group[RQ_SET_MAX_STEPS];
    uint8_t reserved[4864 - 16 - 8 * RQ_SET_MAX_GROUPS - 4 * RQ_SET_MAX_STEPS];
} rq_set_header;

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
 * Bytes of a time-step set blob for `groups` rotations (host descriptors;
 * all of one K and kind family accepted by rq_pack_weights) and N outputs.
 * Errors: as rq_packed_weight_bytes; RQ_ERR_SHAPE for a group count out of
 *         range or rotations of different K.
 */
rq_status rq_weight_set_bytes(const rq_rotation *rots, int32_t groups, const rq_quant *q,
                              int32_t N, size_t *bytes);

/*
 * Offline packing of a time-step set: rq_pack_weights of W for each group's
 * rotation, behind an rq_set_header holding step_group[0 .. steps).
 *   rots        host descriptors [groups]
 *   step_group  host int32 [steps], each in [0, groups)
 *   q, W, w_dtype, N  as rq_pack_weights
 *   blob        host buffer of blob_bytes >= rq_weight_set_bytes()
 * Errors: as rq_pack_weights; RQ_ERR_SHAPE for a step mapped outside the
 *         groups or counts out of range.
 */
rq_status rq_pack_weight_set(const rq_rotation *rots, int32_t groups, const int32_t *step_group,
                             int32_t steps, const rq_quant *q, const void *W, int32_t w_dtype,
                             int32_t N, void *blob, size_t blob_bytes);

/*
 * The member of a set that step `step` uses: its group (the index of the
 * rotation descriptor to pass to rq_rotate_quant), a pointer to its weight
 * header inside the host copy of the set, and the byte offset of its blob
 * (add it to the device copy's address for rq_w4a4_linear).  Host only.
 * Errors: RQ_ERR_NULL, RQ_ERR_FORMAT (not a set), RQ_ERR_SHAPE (step out of
 *         range).
 */
rq_status rq_weight_set_member(const void *set_host, int32_t step, int32_t *group,
                               const rq_weight_header **hdr, int64_t *offset);

/*
 * Bytes of device workspace rq_rotate_quant takes: 0 for RPBH; T*K*4 for
 * DENSE, which stages the rotated tokens in fp32 (required); T*K*8 + T*8
 * for TRDQ (optional: with it the two block rotations run as tiled launches
 * through fp32 buffers, each rotation matrix read once per 128 tokens; without
 * it one pass per few tokens holds the rows in LDS; the codes are the same
 * bit for bit).
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
 * Bytes of every activation buffer of T tokens under a quantizer:
 *   codes      the canonical codes: T * (K - r) / 2 (INT 4-bit), T * K (INT
 *              6- and 8-bit, one code per byte), T * K / 2 (LLOYDMAX, MXFP4)
 *   scale      T * 4 (INT symmetric, LLOYDMAX), T * 8 (INT asymmetric: s
 *              then z), T * K / 32 (MXFP4: E8M0 codes)
 *   codes_mma  the GEMM-layout copy rq_rotate_quant can write: INT with
 *              a_bits 4 (RPBH, DENSE): rq_codes_mma_bytes(); MXFP4: the tiled codes
 *              and tiled scales; LLOYDMAX (RPBH): the bf16 levels,
 *              ceil(T / 32) * (K / 16) * 1024; INT with a_bits 6 or 8 (RPBH,
 *              TRDQ): the int8 fragments, ceil(T / 32) * 32 * K (see
 *              rq_rotate_quant); 0 where none exists
 * Any output pointer may be NULL.
 * Errors: descriptor errors, RQ_ERR_SHAPE (T out of range).
 */
rq_status rq_activation_bytes(const rq_rotation *rot, const rq_quant *q, int64_t T,
                              size_t *codes, size_t *scale, size_t *codes_mma);

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
 *   TRDQ:  y[j] = fl32(x[j] * smooth[j]); z = y BlockDiag(R1) and then
 *          u = p BlockDiag(R2) with p[j] = z[perm[j]], every output one fp32
 *          fused multiply-add chain over its block's inputs ascending, from +0.
 *   INT symmetric (qmax = 2^(a_bits - 1) - 1: 7, 31 or 127), over the quantized
 *          coordinates j in [r, K):
 *          amax = max |u[j]|; s = fl32(amax / qmax); inv = fl32(qmax / amax)
 *          q[j] = clamp(rne(fl32(u[j] * inv)), -qmax, qmax); amax == 0 -> 0, s = 0.
 *          DENSE also writes top[t][j] = bf16_rne(u[j]) for j < r.
 *   INT asymmetric (L = 2^a_bits - 1: 15, 63 or 255): lo = min u, hi = max u, d = fl32(hi - lo);
 *          s = fl32(d / L); inv = fl32(L / d);
 *          z = clamp(-rne(fl32(lo * inv)), 0, L) (an integer, +0 for zero);
 *          q[j] = clamp(rne(fl32(u[j] * inv)) + z, 0, L); d == 0 -> 0, s = z = 0.
 *   LLOYDMAX: d = |u|^2 on an exact integer grid (order independent),
 *          g = (float)sqrt(K / d); index[j] = number of midpoints of adjacent
 *          a_levels strictly below fl32(u[j] * g); sigma = (float)sqrt(d / K).
 *   MXFP4: per 32 coordinates c: e = floor(log2(max |u|)) - 2 (clamped to
 *          [-127, 127]; -127 for a zero block), E8M0 code e + 127; element
 *          code = the E2M1 value nearest to u / 2^e, ties to the even code,
 *          magnitudes above 6 saturating to 6, zero always code 0.
 * Arguments:
 *   rot     host descriptor with device sign/perm (RPBH), R (DENSE) or
 *           smooth/R/perm/R2 (TRDQ)
 *   q       quantizer: INT with RPBH, TRDQ, or DENSE (symmetric, a_bits 4);
 *           LLOYDMAX and MXFP4 with RPBH
 *   X       device [T][K] tokens, row-major, dtype x_dtype (RQ_F32/RQ_BF16),
 *           16-byte aligned
 *   T       tokens, 0 <= T < 2^31
 *   codes   device uint8 [T][...] of rq_activation_bytes(): INT 4-bit
 *           nibbles (two's complement when symmetric, unsigned when
 *           asymmetric; low nibble = even coordinate), INT 6- and 8-bit
 *           bytes (int8 / uint8), LLOYDMAX 4-bit indices or MXFP4 E2M1 codes
 *           as nibbles.  May be NULL for INT 4-bit (RPBH, DENSE), INT 6- and
 *           8-bit (RPBH, TRDQ), MXFP4 and LLOYDMAX (RPBH) when codes_mma is
 *           given.
 *   scale   device: fp32 [T] s (INT symmetric) or sigma (LLOYDMAX); INT
 *           asymmetric: fp32 [2][T], s[t] then the zero point z[t]; MXFP4:
 *           uint8 [T][K/32] E8M0 codes (the pointer is read as bytes).  May
 *           be NULL for MXFP4 when codes_mma is given.
 *   top     device bf16 [T][r] for DENSE with r > 0, else NULL
 *   codes_mma  optional (NULL: not written), RPBH or DENSE:
 *           LLOYDMAX (RPBH): a device buffer of rq_activation_bytes()'s
 *           codes_mma receiving the levels a_levels[code] as bf16 in the
 *           codebook GEMM's matrix-core order [ceil(T/32)][K/16][64 lanes]
 *           [8 bf16]: coordinates 16 ks + 8 h .. 16 ks + 8 h + 7 of token t
 *           are lane t % 32 + 32 h of k-step ks of tile t / 32 (slots of
 *           tokens past T are left unwritten).
 *           INT 6- and 8-bit (RPBH, TRDQ): a device buffer of rq_activation_bytes()'s
 *           codes_mma receiving the code bytes in the int8 GEMM's fragment
 *           order [ceil(T/32)][K/32][64 lanes][16 bytes]: coordinates
 *           32 c + 16 h .. + 15 of token t are lane t % 32 + 32 h of k-step c
 *           of tile t / 32 (slots of tokens past T are left unwritten).
 *           INT 4-bit: a device buffer of rq_codes_mma_bytes() receiving the
 *           same codes in the FP6 GEMM's matrix-core layout.  Tokens come in
 *           tiles of 32 and coordinates in stages of 128; the buffer is
 *           [tile][stage][piece 0..2][lane 0..63][16 bytes], 3 KB per tile
 *           and stage (DENSE: the K - r quantized coordinates; fields of
 *           coordinates past K - r and of token slots past T are left
 *           unwritten).  Token t of a tile owns lanes t and t + 32 (half h);
 *           its twelve dwords f[0..11] for half h of a stage are dword d % 4
 *           of its lane in piece d / 4.  f[0..5] and f[6..11] are the 192-bit
 *           fragments of coordinates 128 s + 64 ks + 32 h + (0..31) for
 *           ks = 0, 1; bits [6 e, 6 e + 6) of a fragment hold the E2M3 code
 *           u (value u / 8, top two bits clear; u = q + 8 for INT4_SYM, the
 *           unsigned code for INT4_ASYM) of coordinate offset
 *           {0,1,3,4,6,7,9,10,12,13,15,8,2,11,5,14}[e % 16] + 16 (e / 16).
 *           MXFP4: a device buffer of rq_activation_bytes()'s codes_mma:
 *           the E2M1 codes tiled [ceil(T/32)][K/32][32][16 bytes] (token t
 *           of a tile, its 16 bytes of coordinates 32 c .. 32 c + 31),
 *           followed by the E8M0 codes tiled [ceil(K/128)][ceil(T/32)][64][2]
 *           (byte ks of lane 32 h + t: coordinates 128 s + 64 ks + 32 h ..).
 *           Bytes of tokens past T and coordinates past K - r are left
 *           unwritten.
 *   workspace, workspace_bytes  device scratch of at least
 *           rq_rotate_quant_workspace_bytes() (NULL/0 when that is 0; TRDQ:
 *           NULL or at least that size), 16-byte aligned
 *   stream  hipStream_t
 * Errors: RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_DTYPE, RQ_ERR_ALIGN,
 *         RQ_ERR_UNSUPPORTED, RQ_ERR_HIP.
 */
rq_status rq_rotate_quant(const rq_rotation *rot, const rq_quant *q, const void *X,
                          int32_t x_dtype, int64_t T, uint8_t *codes, float *scale,
                          uint16_t *top, uint8_t *codes_mma, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * rq_rotate_quant for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, the same kernels and the same
 * results bit for bit.  DENSE stages its fp32 rotated tokens in a scratch
 * array inside the library (one per device, 64 MiB, held from the module's
 * load until the process ends; its address is looked up once per device at
 * the first call there); RPBH uses none and TRDQ runs its workspace-free
 * one-pass form.  The call allocates nothing and
 * calls no allocating routine.  Every call on a device shares that device's
 * scratch: DENSE calls that overlap on one device (other streams, other host
 * threads) race and must be serialized by the caller.
 * Errors: as rq_rotate_quant; RQ_ERR_SHAPE when DENSE needs more than
 *         64 MiB (T * K * 4 bytes) -- use rq_rotate_quant with a workspace.
 */
rq_status rq_rotate_quant_noalloc(const rq_rotation *rot, const rq_quant *q, const void *X,
                                  int32_t x_dtype, int64_t T, uint8_t *codes, float *scale,
                                  uint16_t *top, uint8_t *codes_mma, void *stream);

/*
 * Runtime low-bit GEMM with the per-token x per-channel rescale
 * (TR-DQ section 3.1: Y = X W with per-token activation and per-channel
 * weight scales; DiRotQ abstract: the top principal coefficients add a
 * higher-precision term).
 *   INT:   acc[t][n] = sum_{k < K-r} q_a[t][k] * q_w[n][r + k]  (exact, int32);
 *          asymmetric: q_a[t][k] = u_a[t][k] - z[t] (codes minus zero point)
 *          RPBH:  Y = s_a[t] s_w[n] acc / b_div
 *          TRDQ:  Y = s_a[t] s_w[n] acc
 *          DENSE: Y = s_w[n] (lr[t][n] + s_a[t] acc), with
 *                 lr = sum_{j < r} top[t][j] * q_w[n][j] (bf16 x int4 products,
 *                 fp32 accumulation)
 *   LLOYDMAX: Y = sigma[t] tau[n] / b_div * sum_k a_levels[idx_a] * w_levels[idx_w]
 *          (bf16 products, fp32 accumulation)
 *   MXFP4: Y = 1 / b_div * sum over 32-coordinate blocks c of
 *          2^(e_a[t][c] + e_w[n][c]) sum_{k in c} e2m1(a[t][k]) e2m1(w[n][k])
 *          (exact products, fp32 accumulation in the matrix cores)
 *   + bias[n] when bias is not NULL.
 * INT weights with 4-bit activations run on the FP6 (E2M3) matrix cores:
 * activation codes become q + 8, weight codes q, both exact in E2M3, and the
 * per-channel sum of the weight codes (in the blob) removes the offset;
 * every partial sum is an integer below 2^24, so the fp32 accumulation is
 * exact.  6- and 8-bit activations run on the int8 matrix cores (int32
 * accumulation), MXFP4 on the scaled FP4 matrix cores with the E8M0 block
 * scales as the instruction's per-lane scales.
 * rq_w4a4_linear_engine() selects the matrix cores explicitly.
 * Arguments:
 *   hdr     host pointer to the blob's header (its first 256 bytes)
 *   blob    device copy of the whole blob, 16-byte aligned
 *   codes, scale, top  as written by rq_rotate_quant (device); the weights'
 *           format (kind, a_bits) must match the activations' quantizer
 *   codes_mma  optional (INT, MXFP4 or LLOYDMAX): the
 *           codes_mma output of rq_rotate_quant for the same tokens; when
 *           given it is read instead of codes (and, MXFP4, scale), which may
 *           then be NULL
 *   T       tokens, 0 <= T < 2^31
 *   bias    device fp32 [N] or NULL
 *   Y       device [T][N], dtype y_dtype: RQ_F32, RQ_BF16 (nearest-even), or
 *           RQ_I32 = the exact accumulators acc (INT formats only; the
 *           low-rank term and bias are left out)
 *   stream  hipStream_t
 * Errors: RQ_ERR_NULL, RQ_ERR_FORMAT, RQ_ERR_SHAPE, RQ_ERR_DTYPE,
 *         RQ_ERR_ALIGN, RQ_ERR_UNSUPPORTED, RQ_ERR_HIP.
 */
rq_status rq_w4a4_linear(const rq_weight_header *hdr, const void *blob, const uint8_t *codes,
                         const float *scale, const uint16_t *top, const uint8_t *codes_mma,
                         int64_t T, const float *bias, void *Y, int32_t y_dtype, void *stream);

/*
 * rq_w4a4_linear with an explicit choice of matrix cores (same passages and
 * arguments as rq_w4a4_linear, which is this call with RQ_ENGINE_AUTO).
 *   engine  rq_engine.  RQ_ENGINE_INT8 takes INT4_SYM weights with 4-bit
 *           activations (any r) and their canonical codes (codes_mma must
 *           be NULL for 4-bit activations); the accumulators and outputs equal the FP6 engine's bit
 *           for bit.  6- and 8-bit activations run on the int8 engine only (AUTO or
 *           INT8); Lloyd-Max and MXFP4 take RQ_ENGINE_AUTO only.
 * Errors: as rq_w4a4_linear; RQ_ERR_UNSUPPORTED for an engine that cannot
 *         run the blob's format or for codes_mma of 4-bit activations with
 *         RQ_ENGINE_INT8.
 */
rq_status rq_w4a4_linear_engine(const rq_weight_header *hdr, const void *blob,
                                const uint8_t *codes, const float *scale, const uint16_t *top,
                                const uint8_t *codes_mma, int64_t T, const float *bias, void *Y,
                                int32_t y_dtype, int32_t engine, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */

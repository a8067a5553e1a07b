// rq_api.cpp -- runtime entry points of librq: argument validation and
// dispatch to the gfx950 kernels.  Every check runs before any HIP call.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>

#include "rq_internal.h"

using namespace rq;

namespace {

rq_status hip_status(int err, const char *what) {
    if (err == (int)hipSuccess) return RQ_OK;
    return fail(RQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString((hipError_t)err));
}

rq_status check_header(const rq_weight_header *hdr) {
    if (!hdr) return fail(RQ_ERR_NULL, "weight header is NULL");
    if (hdr->magic != RQ_WEIGHT_MAGIC) return fail(RQ_ERR_FORMAT, "weight header magic mismatch");
    if (hdr->version != RQ_WEIGHT_VERSION)
        return fail(RQ_ERR_FORMAT, "weight header version " + std::to_string(hdr->version) +
                                       " is not " + std::to_string(RQ_WEIGHT_VERSION));
    if (hdr->format != RQ_Q_INT4_SYM && hdr->format != RQ_Q_LLOYDMAX && hdr->format != RQ_Q_INT4_ASYM)
        return fail(RQ_ERR_FORMAT, "unknown weight format");
    const bool int4 = hdr->format != RQ_Q_LLOYDMAX;
    if (hdr->K < 32 || hdr->K > 16384 || hdr->K % 32 != 0 || hdr->N < 1 || hdr->N > (1 << 20) ||
        hdr->r < 0 || hdr->r >= hdr->K || hdr->r % 32 != 0 || hdr->b_div < 1)
        return fail(RQ_ERR_FORMAT, "weight header shape fields are inconsistent");
    const int want_rb = (int4 || hdr->w_bits == 4) ? hdr->K / 2 : hdr->K / 4;
    if (hdr->row_bytes != want_rb) return fail(RQ_ERR_FORMAT, "weight header row_bytes mismatch");
    if (hdr->format == RQ_Q_LLOYDMAX && hdr->K % 64 != 0)
        return fail(RQ_ERR_SHAPE, "the codebook GEMM needs K % 64 == 0");
    if (hdr->scale_offset % 16 != 0 || hdr->codes_offset % 16 != 0)
        return fail(RQ_ERR_FORMAT, "weight header offsets are not 16-byte aligned");
    if (hdr->format == RQ_Q_INT4_ASYM && hdr->r != 0)
        return fail(RQ_ERR_FORMAT, "INT4_ASYM weights have r == 0 (RPBH)");
    if (int4) {
        if (hdr->mma_stages != (hdr->K - hdr->r + 127) / 128 || hdr->mma_ntiles != (hdr->N + 31) / 32)
            return fail(RQ_ERR_FORMAT, "weight header FP6 tile counts are inconsistent");
        if (hdr->wsum_offset % 16 != 0 || hdr->mma_offset % 16 != 0 || hdr->wsum_offset <= 0 ||
            hdr->mma_offset + (int64_t)hdr->mma_ntiles * hdr->mma_stages * 3 * 1024 > hdr->total_bytes)
            return fail(RQ_ERR_FORMAT, "weight header FP6 section offsets are inconsistent");
    }
    return RQ_OK;
}

// Which matrix cores run the INT4 GEMM: FP6 (default; exact, twice the int8
// rate on gfx950) or, with RQ_W4A4_MFMA=int8 in the environment, the int8
// kernel that widens the nibbles in registers.  Read once per process.
bool use_int8_gemm() {
    static const bool v = [] {
        const char *e = std::getenv("RQ_W4A4_MFMA");
        return e && std::strcmp(e, "int8") == 0;
    }();
    return v;
}

}  // namespace

extern "C" {

rq_status rq_rotate_quant_workspace_bytes(const rq_rotation *rot, const rq_quant *q, int64_t T,
                                          size_t *bytes) {
    clear_error();
    rq_status st = check_rotation(rot, false);
    if (st != RQ_OK) return st;
    if ((st = check_quant(rot, q)) != RQ_OK) return st;
    if (!bytes) return fail(RQ_ERR_NULL, "bytes is NULL");
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    *bytes = rot->kind == RQ_ROT_DENSE ? (size_t)T * (size_t)rot->K * sizeof(float) : 0;
    return RQ_OK;
}

rq_status rq_codes_mma_bytes(const rq_rotation *rot, int64_t T, size_t *bytes) {
    clear_error();
    rq_status st = check_rotation(rot, false);
    if (st != RQ_OK) return st;
    if (!bytes) return fail(RQ_ERR_NULL, "bytes is NULL");
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    *bytes = (size_t)mma_codes_bytes(T, rot->K - rot->r);
    return RQ_OK;
}

rq_status rq_rotate_quant(const rq_rotation *rot, const rq_quant *q, const void *X,
                          int32_t x_dtype, int64_t T, uint8_t *codes, float *scale,
                          uint16_t *top, uint8_t *codes_mma, void *workspace,
                          size_t workspace_bytes, void *stream) {
    clear_error();
    rq_status st = check_rotation(rot, true);
    if (st != RQ_OK) return st;
    if ((st = check_quant(rot, q)) != RQ_OK) return st;
    if (x_dtype != RQ_F32 && x_dtype != RQ_BF16)
        return fail(RQ_ERR_DTYPE, "X must be RQ_F32 or RQ_BF16");
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    const int K = rot->K;
    const bool dense = rot->kind == RQ_ROT_DENSE;
    const bool int4 = q->kind == RQ_Q_INT4_SYM || q->kind == RQ_Q_INT4_ASYM;
    if (codes_mma && (dense || !int4))
        return fail(RQ_ERR_UNSUPPORTED, "codes_mma is written for RPBH with INT4 only");
    if (T == 0) return RQ_OK;
    if (!X || !scale || (!codes && !codes_mma))
        return fail(RQ_ERR_NULL, "X, scale and at least one of codes / codes_mma must not be NULL");
    if (dense && !codes) return fail(RQ_ERR_NULL, "DENSE needs codes");
    if (!int4 && !codes) return fail(RQ_ERR_NULL, "LLOYDMAX needs codes");
    if (dense && rot->r > 0 && !top) return fail(RQ_ERR_NULL, "DENSE with r > 0 needs top");
    if (!aligned16(X) || (codes && !aligned16(codes)) || !aligned16(scale) ||
        (top && !aligned16(top)) || (codes_mma && !aligned16(codes_mma)))
        return fail(RQ_ERR_ALIGN, "device buffers must be 16-byte aligned");
    if (!dense && (!aligned16(rot->sign) || !aligned16(rot->perm)))
        return fail(RQ_ERR_ALIGN, "RPBH sign and perm must be 16-byte aligned");
    const int xb = x_dtype == RQ_BF16 ? 1 : 0;
    if (!dense) {
        if (int4)
            return hip_status(launch_rpbh_int4(X, xb, T, K, rot->block, rot->sign, rot->perm, codes,
                                               codes_mma, scale, q->kind == RQ_Q_INT4_ASYM ? 1 : 0,
                                               stream),
                              "rotate_quant launch");
        float th[15];
        const int La = 1 << q->a_bits;
        for (int i = 0; i + 1 < La; ++i) th[i] = (q->a_levels[i] + q->a_levels[i + 1]) / 2.0f;
        return hip_status(launch_rpbh_lloydmax(X, xb, T, K, rot->block, rot->sign, rot->perm, th,
                                               La - 1, codes, scale, stream),
                          "rotate_quant launch");
    }
    const size_t need = (size_t)T * (size_t)K * sizeof(float);
    if (!workspace || workspace_bytes < need)
        return fail(RQ_ERR_SHAPE, "DENSE needs a workspace of " + std::to_string(need) + " bytes");
    if (!aligned16(workspace)) return fail(RQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    float *U = static_cast<float *>(workspace);
    st = hip_status(launch_dense_rotate(X, xb, T, K, rot->R, U, stream), "dense rotate launch");
    if (st != RQ_OK) return st;
    return hip_status(launch_dense_quant(U, T, K, rot->r, codes, scale, top, stream),
                      "dense quant launch");
}

rq_status rq_w4a4_linear(const rq_weight_header *hdr, const void *blob, const uint8_t *codes,
                         const float *scale, const uint16_t *top, const uint8_t *codes_mma,
                         int64_t T, const float *bias, void *Y, int32_t y_dtype, void *stream) {
    clear_error();
    rq_status st = check_header(hdr);
    if (st != RQ_OK) return st;
    if (y_dtype != RQ_F32 && y_dtype != RQ_BF16 && y_dtype != RQ_I32)
        return fail(RQ_ERR_DTYPE, "Y must be RQ_F32, RQ_BF16 or RQ_I32");
    const bool int4 = hdr->format != RQ_Q_LLOYDMAX;
    const bool asym = hdr->format == RQ_Q_INT4_ASYM;
    if (y_dtype == RQ_I32 && !int4)
        return fail(RQ_ERR_UNSUPPORTED, "raw accumulators exist for INT4 weights only");
    if (codes_mma && (!int4 || hdr->r != 0))
        return fail(RQ_ERR_UNSUPPORTED, "codes_mma is read for INT4 weights with r == 0 only");
    if (asym && use_int8_gemm())
        return fail(RQ_ERR_UNSUPPORTED, "the int8 GEMM (RQ_W4A4_MFMA=int8) takes INT4_SYM only");
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    if (T == 0) return RQ_OK;
    const bool int8 = hdr->format == RQ_Q_INT4_SYM && use_int8_gemm();
    if (!blob || !scale || !Y || (!codes && !codes_mma) || (int8 && !codes))
        return fail(RQ_ERR_NULL, "blob, scale, Y and the activation codes must not be NULL");
    if (!int4 && !codes) return fail(RQ_ERR_NULL, "LLOYDMAX needs codes");
    if (hdr->r > 0 && !top) return fail(RQ_ERR_NULL, "weights with r > 0 need top");
    if (!aligned16(blob) || (codes && !aligned16(codes)) || !aligned16(scale) || !aligned16(Y) ||
        (top && !aligned16(top)) || (bias && !aligned16(bias)) ||
        (codes_mma && !aligned16(codes_mma)))
        return fail(RQ_ERR_ALIGN, "device buffers must be 16-byte aligned");
    if (int4) {
        if (int8)
            return hip_status(launch_gemm_w4a4(codes, scale, top, T, hdr, blob, bias, Y, y_dtype, stream),
                              "w4a4 int8 gemm launch");
        return hip_status(launch_gemm_fp6(codes_mma ? nullptr : codes, codes_mma, scale,
                                          asym ? scale + T : nullptr, top, T, hdr, blob, bias, Y,
                                          y_dtype, stream),
                          "w4a4 fp6 gemm launch");
    }
    return hip_status(launch_gemm_codebook(codes, scale, T, hdr, blob, bias, Y, y_dtype, stream),
                      "codebook gemm launch");
}

}  // extern "C"

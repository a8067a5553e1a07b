// rq_api.cpp -- runtime entry points of librq: argument validation and
// dispatch to the gfx950 kernels.  Every check runs before any HIP call.

#include <hip/hip_runtime.h>

#include <cmath>
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
    const int f = hdr->format;
    if (f != RQ_Q_INT4_SYM && f != RQ_Q_LLOYDMAX && f != RQ_Q_INT4_ASYM && f != RQ_Q_MXFP4)
        return fail(RQ_ERR_FORMAT, "unknown weight format");
    const bool intq = f == RQ_Q_INT4_SYM || f == RQ_Q_INT4_ASYM;
    if (hdr->K < 32 || hdr->K > 16384 || hdr->K % 32 != 0 || hdr->N < 1 || hdr->N > (1 << 20) ||
        hdr->r < 0 || hdr->r >= hdr->K || hdr->r % 32 != 0 || hdr->b_div < 1)
        return fail(RQ_ERR_FORMAT, "weight header shape fields are inconsistent");
    // 4-bit activations with 4-bit weights; 6- or 8-bit activations (one
    // code per byte) with 4-, 6- or 8-bit weights
    const bool wb_ok = hdr->w_bits == 4 || hdr->w_bits == 6 || hdr->w_bits == 8;
    if (intq && !((hdr->a_bits == 4 && hdr->w_bits == 4) ||
                  ((hdr->a_bits == 6 || hdr->a_bits == 8) && wb_ok && hdr->r == 0)))
        return fail(RQ_ERR_FORMAT, "weight header bit widths are inconsistent");
    int want_rb;
    if (f == RQ_Q_LLOYDMAX)
        want_rb = hdr->w_bits == 4 ? hdr->K / 2 : hdr->K / 4;
    else if (f == RQ_Q_MXFP4)
        want_rb = hdr->K / 2;
    else
        want_rb = hdr->w_bits == 4 ? hdr->K / 2 : hdr->K;
    if (hdr->row_bytes != want_rb) return fail(RQ_ERR_FORMAT, "weight header row_bytes mismatch");
    if (f == RQ_Q_LLOYDMAX && hdr->K % 64 != 0)
        return fail(RQ_ERR_SHAPE, "the codebook GEMM needs K % 64 == 0");
    if (f == RQ_Q_LLOYDMAX && hdr->w_bits == 4 &&
        (hdr->mma_ntiles != (hdr->N + 31) / 32 || hdr->mma_offset <= 0 || hdr->mma_offset % 16 != 0 ||
         hdr->mma_offset + (int64_t)hdr->mma_ntiles * (hdr->K / 16) * 1024 > hdr->total_bytes))
        return fail(RQ_ERR_FORMAT, "weight header bf16 fragment section is inconsistent");
    if (f == RQ_Q_LLOYDMAX && hdr->w_bits != 4 && hdr->mma_offset != 0)
        return fail(RQ_ERR_FORMAT, "2-bit Lloyd-Max weights carry no bf16 fragment section");
    if (hdr->scale_offset % 16 != 0 || hdr->codes_offset % 16 != 0)
        return fail(RQ_ERR_FORMAT, "weight header offsets are not 16-byte aligned");
    if (f == RQ_Q_INT4_ASYM && hdr->r != 0)
        return fail(RQ_ERR_FORMAT, "INT4_ASYM weights have r == 0");
    if (intq && hdr->a_bits == 4) {
        if (hdr->mma_stages != (hdr->K - hdr->r + 127) / 128 || hdr->mma_ntiles != (hdr->N + 31) / 32)
            return fail(RQ_ERR_FORMAT, "weight header FP6 tile counts are inconsistent");
        if (hdr->wsum_offset % 16 != 0 || hdr->mma_offset % 16 != 0 || hdr->wsum_offset <= 0 ||
            hdr->mma_offset + (int64_t)hdr->mma_ntiles * hdr->mma_stages * 3 * 1024 > hdr->total_bytes)
            return fail(RQ_ERR_FORMAT, "weight header FP6 section offsets are inconsistent");
    }
    if (intq && hdr->a_bits != 4) {
        if (hdr->wsum_offset <= 0 || hdr->wsum_offset % 16 != 0 || hdr->i8_offset <= 0 ||
            hdr->i8_offset % 16 != 0 ||
            hdr->i8_offset + (int64_t)(hdr->N + 31) / 32 * 32 * hdr->K > hdr->total_bytes)
            return fail(RQ_ERR_FORMAT, "weight header int8 section offsets are inconsistent");
    }
    if (f == RQ_Q_MXFP4) {
        if (hdr->K % 128 != 0) return fail(RQ_ERR_FORMAT, "MXFP4 weights need K % 128 == 0");
        if (hdr->mma_stages != hdr->K / 128 || hdr->mma_ntiles != (hdr->N + 31) / 32 ||
            hdr->mma_offset <= 0 || hdr->mma_offset % 16 != 0 || hdr->mxs_offset % 16 != 0 ||
            hdr->mxs_offset < hdr->mma_offset + (int64_t)hdr->mma_ntiles * (hdr->K / 32) * 512 ||
            hdr->mxs_offset + (int64_t)hdr->mma_stages * hdr->mma_ntiles * 128 > hdr->total_bytes)
            return fail(RQ_ERR_FORMAT, "weight header MXFP4 sections are inconsistent");
    }
    return RQ_OK;
}

// Argument checks of the runtime activation call that follow the descriptor
// checks (everything but the workspace).
rq_status validate_rotate_quant(const rq_rotation *rot, const rq_quant *q, const void *X,
                                int32_t x_dtype, int64_t T, const uint8_t *codes,
                                const float *scale, const uint16_t *top,
                                const uint8_t *codes_mma) {
    if (x_dtype != RQ_F32 && x_dtype != RQ_BF16)
        return fail(RQ_ERR_DTYPE, "X must be RQ_F32 or RQ_BF16");
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    const bool rpbh = rot->kind == RQ_ROT_RPBH;
    const bool dense = rot->kind == RQ_ROT_DENSE;
    const bool mx = q->kind == RQ_Q_MXFP4;
    const bool int4 = (q->kind == RQ_Q_INT4_SYM || q->kind == RQ_Q_INT4_ASYM) && q->a_bits == 4;
    const bool int8 = (q->kind == RQ_Q_INT4_SYM || q->kind == RQ_Q_INT4_ASYM) && q->a_bits != 4;
    const bool lm = q->kind == RQ_Q_LLOYDMAX;
    const bool trdq = rot->kind == RQ_ROT_TRDQ;
    const bool mma_ok = (rpbh && (int4 || int8 || mx || lm)) || (dense && int4) || (trdq && int8);
    if (codes_mma && !mma_ok)
        return fail(RQ_ERR_UNSUPPORTED,
                    "codes_mma is written for 4-bit integer codes (RPBH, DENSE), 6- and 8-bit integer "
                    "codes (RPBH, TRDQ), and MXFP4 or LLOYDMAX (RPBH) only");
    if (T == 0) return RQ_OK;
    if (!X || (!codes && !codes_mma) || (!scale && !(mx && codes_mma)))
        return fail(RQ_ERR_NULL, "X, scale and at least one of codes / codes_mma must not be NULL");
    if (!codes && !mma_ok)
        return fail(RQ_ERR_NULL, "this rotation and quantizer write the canonical codes: codes is NULL");
    if (dense && rot->r > 0 && !top) return fail(RQ_ERR_NULL, "DENSE with r > 0 needs top");
    if (!aligned16(X) || (codes && !aligned16(codes)) || (scale && !aligned16(scale)) ||
        (top && !aligned16(top)) || (codes_mma && !aligned16(codes_mma)))
        return fail(RQ_ERR_ALIGN, "device buffers must be 16-byte aligned");
    if (!dense && (!aligned16(rot->sign) || !aligned16(rot->perm)))
        return fail(RQ_ERR_ALIGN, "RPBH sign and perm must be 16-byte aligned");
    return RQ_OK;
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
    *bytes = rot->kind == RQ_ROT_DENSE  ? (size_t)T * (size_t)rot->K * sizeof(float)
             : rot->kind == RQ_ROT_TRDQ ? trdq_workspace_bytes(T, rot->K)
                                        : 0;
    return RQ_OK;
}

rq_status rq_activation_bytes(const rq_rotation *rot, const rq_quant *q, int64_t T,
                              size_t *codes, size_t *scale, size_t *codes_mma) {
    clear_error();
    rq_status st = check_rotation(rot, false);
    if (st != RQ_OK) return st;
    if ((st = check_quant(rot, q)) != RQ_OK) return st;
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    const int K = rot->K, Kq = K - rot->r;
    const bool intq = q->kind == RQ_Q_INT4_SYM || q->kind == RQ_Q_INT4_ASYM;
    const bool mx = q->kind == RQ_Q_MXFP4;
    if (codes) *codes = (size_t)T * (size_t)(intq ? (q->a_bits == 4 ? Kq / 2 : Kq) : K / 2);
    if (scale)
        *scale = mx ? (size_t)T * (K / 32)
                    : (size_t)T * (q->kind == RQ_Q_INT4_ASYM ? 8 : 4);
    if (codes_mma) {
        *codes_mma = 0;
        if ((rot->kind == RQ_ROT_RPBH || rot->kind == RQ_ROT_DENSE) && intq && q->a_bits == 4)
            *codes_mma = (size_t)mma_codes_bytes(T, Kq);
        else if ((rot->kind == RQ_ROT_RPBH || rot->kind == RQ_ROT_TRDQ) && intq && q->a_bits != 4)
            *codes_mma = (size_t)i8_mma_bytes(T, K);
        else if (rot->kind == RQ_ROT_RPBH && mx)
            *codes_mma = (size_t)mx_mma_bytes(T, K);
        else if (rot->kind == RQ_ROT_RPBH && q->kind == RQ_Q_LLOYDMAX)
            *codes_mma = (size_t)cb_mma_bytes(T, K);
    }
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
    if ((st = validate_rotate_quant(rot, q, X, x_dtype, T, codes, scale, top, codes_mma)) != RQ_OK)
        return st;
    if (T == 0) return RQ_OK;
    const int K = rot->K;
    const int xb = x_dtype == RQ_BF16 ? 1 : 0;
    if (rot->kind == RQ_ROT_RPBH) {
        if (q->kind == RQ_Q_MXFP4)
            return hip_status(launch_rpbh_mxfp4(X, xb, T, K, rot->block, rot->sign, rot->perm, codes,
                                                reinterpret_cast<uint8_t *>(scale), codes_mma, stream),
                              "rotate_quant launch");
        if (q->kind == RQ_Q_INT4_SYM || q->kind == RQ_Q_INT4_ASYM)
            return hip_status(launch_rpbh_int4(X, xb, T, K, rot->block, rot->sign, rot->perm, codes,
                                               codes_mma, scale, q->kind == RQ_Q_INT4_ASYM ? 1 : 0,
                                               q->a_bits, stream),
                              "rotate_quant launch");
        float th[15];
        const int La = 1 << q->a_bits;
        for (int i = 0; i + 1 < La; ++i) th[i] = (q->a_levels[i] + q->a_levels[i + 1]) / 2.0f;
        return hip_status(launch_rpbh_lloydmax(X, xb, T, K, rot->block, rot->sign, rot->perm, th,
                                               La - 1, q->a_levels, codes, scale, codes_mma, stream),
                          "rotate_quant launch");
    }
    if (rot->kind == RQ_ROT_TRDQ && workspace) {
        const size_t need = trdq_workspace_bytes(T, K);
        if (workspace_bytes < need)
            return fail(RQ_ERR_SHAPE, "TRDQ: a workspace, when given, needs " + std::to_string(need) + " bytes");
        if (!aligned16(workspace)) return fail(RQ_ERR_ALIGN, "workspace must be 16-byte aligned");
        return hip_status(launch_trdq_tiled(X, xb, T, K, rot->block, rot->smooth, rot->R, rot->perm,
                                            rot->R2, codes, codes_mma, scale,
                                            q->kind == RQ_Q_INT4_ASYM ? 1 : 0, q->a_bits, workspace,
                                            stream),
                          "rotate_quant launch");
    }
    if (rot->kind == RQ_ROT_TRDQ)
        return hip_status(launch_trdq(X, xb, T, K, rot->block, rot->smooth, rot->R, rot->perm, rot->R2,
                                      codes, codes_mma, scale, q->kind == RQ_Q_INT4_ASYM ? 1 : 0,
                                      q->a_bits, stream),
                          "rotate_quant launch");
    const size_t need = (size_t)T * (size_t)K * sizeof(float);
    if (!workspace || workspace_bytes < need)
        return fail(RQ_ERR_SHAPE, "DENSE needs a workspace of " + std::to_string(need) + " bytes");
    if (!aligned16(workspace)) return fail(RQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    float *U = static_cast<float *>(workspace);
    st = hip_status(launch_dense_rotate(X, xb, T, K, rot->R, U, stream), "dense rotate launch");
    if (st != RQ_OK) return st;
    return hip_status(launch_dense_quant(U, T, K, rot->r, codes, scale, top, codes_mma, stream),
                      "dense quant launch");
}

rq_status rq_rotate_quant_noalloc(const rq_rotation *rot, const rq_quant *q, const void *X,
                                  int32_t x_dtype, int64_t T, uint8_t *codes, float *scale,
                                  uint16_t *top, uint8_t *codes_mma, void *stream) {
    clear_error();
    rq_status st = check_rotation(rot, true);
    if (st != RQ_OK) return st;
    if ((st = check_quant(rot, q)) != RQ_OK) return st;
    if (rot->kind != RQ_ROT_DENSE)   // RPBH kernels use no scratch
        return rq_rotate_quant(rot, q, X, x_dtype, T, codes, scale, top, codes_mma, nullptr, 0,
                               stream);
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    const size_t need = (size_t)T * (size_t)rot->K * sizeof(float);
    if (need > kDenseScratchBytes)
        return fail(RQ_ERR_SHAPE, "rq_rotate_quant_noalloc: DENSE needs T * K * 4 = " +
                                      std::to_string(need) + " bytes of scratch, above its " +
                                      std::to_string(kDenseScratchBytes) +
                                      "-byte limit; use rq_rotate_quant with a workspace");
    if (T == 0) return rq_rotate_quant(rot, q, X, x_dtype, 0, codes, scale, top, codes_mma,
                                       nullptr, 0, stream);
    // every argument check runs before the scratch lookup touches the GPU
    st = validate_rotate_quant(rot, q, X, x_dtype, T, codes, scale, top, codes_mma);
    if (st != RQ_OK) return st;
    float *ws = nullptr;
    st = hip_status(dense_scratch(&ws), "scratch lookup");
    if (st != RQ_OK) return st;
    return rq_rotate_quant(rot, q, X, x_dtype, T, codes, scale, top, codes_mma, ws, need, stream);
}

rq_status rq_w4a4_linear_engine(const rq_weight_header *hdr, const void *blob,
                                const uint8_t *codes, const float *scale, const uint16_t *top,
                                const uint8_t *codes_mma, int64_t T, const float *bias, void *Y,
                                int32_t y_dtype, int32_t engine, void *stream) {
    clear_error();
    rq_status st = check_header(hdr);
    if (st != RQ_OK) return st;
    if (y_dtype != RQ_F32 && y_dtype != RQ_BF16 && y_dtype != RQ_I32)
        return fail(RQ_ERR_DTYPE, "Y must be RQ_F32, RQ_BF16 or RQ_I32");
    if (engine != RQ_ENGINE_AUTO && engine != RQ_ENGINE_FP6 && engine != RQ_ENGINE_INT8)
        return fail(RQ_ERR_UNSUPPORTED, "unknown engine " + std::to_string(engine));
    const int f = hdr->format;
    const bool intq = f == RQ_Q_INT4_SYM || f == RQ_Q_INT4_ASYM;
    const bool asym = f == RQ_Q_INT4_ASYM;
    const bool a8 = intq && hdr->a_bits != 4;   // 6- or 8-bit codes, one per byte
    const bool mx = f == RQ_Q_MXFP4;
    if (y_dtype == RQ_I32 && !intq)
        return fail(RQ_ERR_UNSUPPORTED, "raw accumulators exist for integer weights only");

    if (engine != RQ_ENGINE_AUTO && !intq)
        return fail(RQ_ERR_UNSUPPORTED, "the Lloyd-Max and MXFP4 formats have one engine (RQ_ENGINE_AUTO)");
    if (a8 && engine == RQ_ENGINE_FP6)
        return fail(RQ_ERR_UNSUPPORTED, "6- and 8-bit activations run on the int8 engine");
    const bool int8 = a8 || engine == RQ_ENGINE_INT8;
    if (int8 && !a8 && asym)
        return fail(RQ_ERR_UNSUPPORTED, "the int8 engine takes INT4_SYM weights with 4-bit activations");
    if (int8 && !a8 && codes_mma)
        return fail(RQ_ERR_UNSUPPORTED,
                    "the int8 engine reads the canonical codes of 4-bit activations (codes_mma must be NULL)");
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(RQ_ERR_SHAPE, "T out of range");
    if (T == 0) return RQ_OK;
    if (!blob || !Y) return fail(RQ_ERR_NULL, "blob and Y must not be NULL");
    if (mx) {
        if (!codes_mma)
            return fail(RQ_ERR_UNSUPPORTED, "the MXFP4 GEMM reads the tiled codes_mma of rq_rotate_quant");
    } else {
        if (!scale || (!codes && !codes_mma))
            return fail(RQ_ERR_NULL, "scale and the activation codes must not be NULL");
        if (int8 && !a8 && !codes) return fail(RQ_ERR_NULL, "this engine needs codes");
    }
    if (hdr->r > 0 && !top) return fail(RQ_ERR_NULL, "weights with r > 0 need top");
    if (!aligned16(blob) || (codes && !aligned16(codes)) || (scale && !aligned16(scale)) ||
        !aligned16(Y) || (top && !aligned16(top)) || (bias && !aligned16(bias)) ||
        (codes_mma && !aligned16(codes_mma)))
        return fail(RQ_ERR_ALIGN, "device buffers must be 16-byte aligned");
    if (mx) {
        if (y_dtype == RQ_I32) return fail(RQ_ERR_UNSUPPORTED, "MXFP4 has no integer accumulators");
        return hip_status(launch_gemm_mx(codes_mma, T, hdr, blob, bias, Y, y_dtype, stream),
                          "mxfp4 gemm launch");
    }
    if (intq) {
        if (a8)
            return hip_status(launch_gemm_i8(codes_mma ? nullptr : codes, codes_mma, scale,
                                             asym ? scale + T : nullptr, T, hdr, blob, bias, Y,
                                             y_dtype, stream),
                              "int8 gemm launch");
        if (int8)
            return hip_status(launch_gemm_w4a4(codes, scale, top, T, hdr, blob, bias, Y, y_dtype, stream),
                              "int8 gemm launch");
        return hip_status(launch_gemm_fp6(codes_mma ? nullptr : codes, codes_mma, scale,
                                          asym ? scale + T : nullptr, top, T, hdr, blob, bias, Y,
                                          y_dtype, stream),
                          "w4a4 fp6 gemm launch");
    }
    return hip_status(launch_gemm_codebook(codes, codes_mma, scale, T, hdr, blob, bias, Y, y_dtype, stream),
                      "codebook gemm launch");
}

rq_status rq_w4a4_linear(const rq_weight_header *hdr, const void *blob, const uint8_t *codes,
                         const float *scale, const uint16_t *top, const uint8_t *codes_mma,
                         int64_t T, const float *bias, void *Y, int32_t y_dtype, void *stream) {
    return rq_w4a4_linear_engine(hdr, blob, codes, scale, top, codes_mma, T, bias, Y, y_dtype,
                                 RQ_ENGINE_AUTO, stream);
}

}  // extern "C"

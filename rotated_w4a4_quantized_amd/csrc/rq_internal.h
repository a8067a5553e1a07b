// rq_internal.h -- declarations shared by librq's translation units.
#pragma once

#include <cstdint>
#include <cstddef>
#include <string>

#include "../../include/rq.h"

namespace rq {

// Thread-local error state behind rq_last_error().
rq_status fail(rq_status st, const std::string &msg);
void clear_error();

// Shape/descriptor checks shared by pack and runtime entry points.
rq_status check_rotation(const rq_rotation *rot, bool need_tables);
rq_status check_quant(const rq_rotation *rot, const rq_quant *q);

inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline int ilog2(int64_t v) { int l = 0; while ((int64_t(1) << l) < v) ++l; return l; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// bytes of codes in the GEMM's FP6 fragment layout for T tokens: 3 KB per 32
// tokens per 128 quantized coordinates
inline int64_t mma_codes_bytes(int64_t T, int Kq) {
    return ((T + 31) / 32) * (int64_t)((Kq + 127) / 128) * 3 * 1024;
}

// Kernel launchers (rq_rpbh.hip, rq_dense.hip, rq_gemm_*.hip).  Arguments are validated
// by the caller; these only launch.  They return a hipError_t as int.
// asym: per-token zero point (INT4_ASYM), written to scale[T .. 2T)
int launch_rpbh_int4(const void *X, int x_bf16, int64_t T, int K, int block,
                     const int8_t *sign, const int32_t *perm, uint8_t *codes,
                     uint8_t *codes_mma, float *scale, int asym, void *stream);
int launch_rpbh_lloydmax(const void *X, int x_bf16, int64_t T, int K, int block,
                         const int8_t *sign, const int32_t *perm, const float *thresholds,
                         int n_thresholds, uint8_t *codes, float *sigma, void *stream);
int launch_dense_rotate(const void *X, int x_bf16, int64_t T, int K, const float *R,
                        float *U, void *stream);
int launch_dense_quant(const float *U, int64_t T, int K, int r, uint8_t *codes,
                       float *scale, uint16_t *top, void *stream);
int launch_gemm_w4a4(const uint8_t *codes, const float *scale, const uint16_t *top,
                     int64_t T, const rq_weight_header *hdr, const void *blob,
                     const float *bias, void *Y, int y_dtype, void *stream);
// zero: per-token zero points of INT4_ASYM activations, or null (symmetric)
int launch_gemm_fp6(const uint8_t *codes, const uint8_t *codes_mma, const float *scale,
                    const float *zero, const uint16_t *top, int64_t T,
                    const rq_weight_header *hdr, const void *blob, const float *bias, void *Y,
                    int y_dtype, void *stream);
int launch_gemm_codebook(const uint8_t *codes, const float *sigma, int64_t T,
                         const rq_weight_header *hdr, const void *blob,
                         const float *bias, void *Y, int y_dtype, void *stream);

}  // namespace rq

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

// Launch facts of the current HIP device, cached per device and safe to call
// from several host threads: compute units, and raising a kernel's dynamic-LDS
// limit to `bytes` (once per kernel and device; a no-op up to 64 KB).  The
// second returns a hipError_t as int.
int device_cus();
int ensure_dyn_lds(const void *kernel, size_t bytes);

// Kernel launchers (rq_rpbh.hip, rq_dense.hip, rq_gemm_*.hip).  Arguments are validated
// by the caller; these only launch.  They return a hipError_t as int.
// asym: per-token zero point (INT4_ASYM), written to scale[T .. 2T)
// a_bits 4 or 8 (8: canonical codes only)
int launch_rpbh_int4(const void *X, int x_bf16, int64_t T, int K, int block,
                     const int8_t *sign, const int32_t *perm, uint8_t *codes,
                     uint8_t *codes_mma, float *scale, int asym, int a_bits, void *stream);
// MXFP4: codes [T][K/2] and E8M0 scales [T][K/32] (either may be null), and/or
// the tiled copies in codes_mma
int launch_rpbh_mxfp4(const void *X, int x_bf16, int64_t T, int K, int block,
                      const int8_t *sign, const int32_t *perm, uint8_t *codes,
                      uint8_t *scales, uint8_t *codes_mma, void *stream);
int launch_rpbh_lloydmax(const void *X, int x_bf16, int64_t T, int K, int block,
                         const int8_t *sign, const int32_t *perm, const float *thresholds,
                         int n_thresholds, const float *levels, uint8_t *codes, float *sigma,
                         uint8_t *codes_mma, void *stream);
// bytes of the Lloyd-Max activations in the codebook GEMM's bf16 fragment
// layout: [ceil(T / 32)][K / 16][64 lanes][16 bytes]
inline int64_t cb_mma_bytes(int64_t T, int K) { return (T + 31) / 32 * (int64_t)(K / 16) * 1024; }
int launch_dense_rotate(const void *X, int x_bf16, int64_t T, int K, const float *R,
                        float *U, void *stream);
// Largest fp32 staging of rq_rotate_quant_noalloc (T * K * 4 bytes, DENSE).
constexpr size_t kDenseScratchBytes = size_t(64) << 20;
// The calling thread's current device's copy of that scratch (looked up once
// per device with hipGetSymbolAddress); returns a hipError_t as int.
int dense_scratch(float **ptr);
int launch_dense_quant(const float *U, int64_t T, int K, int r, uint8_t *codes, float *scale,
                       uint16_t *top, uint8_t *codes_mma, void *stream);
// the int8-MFMA engine of the INT4_SYM GEMM (4-bit activation codes widened
// in registers; a_bits 4 only)
int launch_gemm_w4a4(const uint8_t *codes, const float *scale, const uint16_t *top, int64_t T,
                     const rq_weight_header *hdr, const void *blob, const float *bias, void *Y,
                     int y_dtype, void *stream);
// 8-bit activations on the int8 matrix cores (operands copied straight from
// the row-major int8 matrices; blob's int8 weight copy)
int launch_gemm_i8(const uint8_t *codes, const uint8_t *codes_mma, const float *scale,
                   const float *zero, int64_t T, const rq_weight_header *hdr, const void *blob,
                   const float *bias, void *Y, int y_dtype, void *stream);
// bytes of 8-bit activation codes in the int8 GEMM's fragment order:
// [ceil(T / 32)][K / 32][64 lanes][16 bytes]
inline int64_t i8_mma_bytes(int64_t T, int K) { return (T + 31) / 32 * 32 * (int64_t)K; }
// TR-DQ runtime rotation (smoothing, block rotation, zigzag gather, block
// rotation) and per-token integer quantization (a_bits 4 or 8, asym or not)
int launch_trdq(const void *X, int x_bf16, int64_t T, int K, int block, const float *smooth,
                const float *R1, const int32_t *perm, const float *R2, uint8_t *codes,
                uint8_t *codes_mma, float *scale, int asym, int a_bits, void *stream);
// TR-DQ with a workspace: two tiled block-rotation launches through fp32
// buffers and a quantize launch (bit-identical codes); the workspace holds
// Z and U, fp32 [T][K] each, then the per-token extremes, uint32 [2][T]
size_t trdq_workspace_bytes(int64_t T, int K);
int launch_trdq_tiled(const void *X, int x_bf16, int64_t T, int K, int block, const float *smooth,
                      const float *R1, const int32_t *perm, const float *R2, uint8_t *codes,
                      uint8_t *codes_mma, float *scale, int asym, int a_bits, void *workspace,
                      void *stream);
// zero: per-token zero points of INT4_ASYM activations, or null (symmetric)
int launch_gemm_fp6(const uint8_t *codes, const uint8_t *codes_mma, const float *scale,
                    const float *zero, const uint16_t *top, int64_t T,
                    const rq_weight_header *hdr, const void *blob, const float *bias, void *Y,
                    int y_dtype, void *stream);
// MXFP4 GEMM on the tiled codes and scales of rq_rotate_quant's codes_mma
int launch_gemm_mx(const uint8_t *codes_mma, int64_t T, const rq_weight_header *hdr,
                   const void *blob, const float *bias, void *Y, int y_dtype, void *stream);
// bytes of an MXFP4 codes_mma buffer: tiled codes, then tiled scales
inline int64_t mx_mma_bytes(int64_t T, int K) {
    const int64_t tiles = (T + 31) / 32;
    return tiles * (K / 32) * 512 + (int64_t)((K + 127) / 128) * tiles * 128;
}
int launch_gemm_codebook(const uint8_t *codes, const uint8_t *codes_mma, const float *sigma, int64_t T,
                         const rq_weight_header *hdr, const void *blob, const float *bias,
                         void *Y, int y_dtype, void *stream);

}  // namespace rq

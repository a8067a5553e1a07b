"""Python side of the CPU oracle for the rotated low-bit quantized linear layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__.py and by the cpu_baseline leg of bench.py, never by the
product package.  It shares no code with the HIP path; the heavy loops live
in rq_oracle.c (plain C, no contraction), loaded here with ctypes.

What each function computes is stated with the page passage it follows:

* "TR-DQ: Time-Rotation Diffusion Quantization" section 3.1 -- linear layer
  Y = X.W, uniform quantizer Eq.(1)-(3) (symmetric form, and the asymmetric
  per-token form with a zero point), per-token activation and
  per-channel weight granularity; section 3.2 Eq.(8)-(9) -- block-diagonal
  rotation, runtime rotation of X with the transposed rotation folded into W.
* "OrbitQuant" abstract -- RPBH rotation, normalized rotated basis, one
  Lloyd-Max codebook for a fixed known marginal, same quantizer on weight
  rows offline, W2A4.
* "DiRotQ" abstract -- PCA basis at inference, top principal coefficients
  kept at higher precision, inverse rotation fused into the weights.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rq_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-shared", "-fPIC", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile rq_oracle.c into liboracle.so (plain gcc, no GPU code)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        build()
        _LIB = ctypes.CDLL(_SO)
        _declare(_LIB)
    return _LIB


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def _declare(L):
    L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_f32_to_bf16.restype = ctypes.c_uint16
    L.orc_rpbh_row_f32.argtypes = [_P, _I, _I, _P, _P, _P]
    L.orc_rpbh_row_f64.argtypes = [_P, _I, _I, _P, _P, _P]
    L.orc_dense_row_f32.argtypes = [_P, _P, _I, _P]
    L.orc_dense_row_f64.argtypes = [_P, _P, _I, _P]
    L.orc_quant_int4_row.argtypes = [_P, _I, _I, _P, _P]
    L.orc_quant_int4_wrow.argtypes = [_P, _I, _P, _P]
    L.orc_quant_int4_asym_row.argtypes = [_P, _I, _P, _P, _P]
    L.orc_pack_nibbles.argtypes = [_P, _I, _P]
    L.orc_pack_crumbs.argtypes = [_P, _I, _P]
    L.orc_norm2_grid.argtypes = [_P, _I]
    L.orc_norm2_grid.restype = ctypes.c_double
    L.orc_quant_lloydmax_row.argtypes = [_P, _I, _P, _I, _P, _P]
    L.orc_quant_lloydmax_wrow.argtypes = [_P, _I, _P, _I, _P, _P]
    L.orc_quant_sym_row.argtypes = [_P, _I, _I, _I, _P, _P]
    L.orc_quant_asym_row.argtypes = [_P, _I, _I, _P, _P, _P]
    L.orc_quant_sym_wrow.argtypes = [_P, _I, _I, _P, _P]
    L.orc_e2m1_value.argtypes = [_I]
    L.orc_e2m1_value.restype = ctypes.c_double
    L.orc_e2m1_encode.argtypes = [ctypes.c_double]
    L.orc_e2m1_encode.restype = _I
    L.orc_mx_scale_code.argtypes = [ctypes.c_double]
    L.orc_mx_scale_code.restype = _I
    L.orc_quant_mxfp4_f64.argtypes = [_P, _I, _P, _P]
    L.orc_quant_mxfp4_row.argtypes = [_P, _I, _P, _P]
    L.orc_trdq_row_f32.argtypes = [_P, _I, _I, _P, _P, _P, _P, _P]
    L.orc_trdq_row_f64.argtypes = [_P, _I, _I, _P, _P, _P, _P, _P]
    L.orc_act_rows.argtypes = [_P, _I, _I, _P, _I64, _P, _I, _I, _I, _P, _I,
                               _P, _P, _P, _P, _P, _P]
    L.orc_weight_rows.argtypes = [_P, _I, _I, _P, _I, _I, _P, _I, _P, _P, _P, _P]
    L.orc_gemm_codes_pairs.argtypes = [_P, _I, _I, _I, _P, _I, _I, _I, _P, _P, _I64, _P]
    L.orc_mx_dot_pairs.argtypes = [_P, _P, _P, _P, _I, _P, _P, _I64, _P]
    L.orc_int_gemm_pairs.argtypes = [_P, _I, _P, _I, _I, _P, _P, _I64, _P]
    L.orc_asym_gemm_pairs.argtypes = [_P, _I, _P, _P, _P, _I64, _P]
    L.orc_int_gemm.argtypes = [_P, _I, _I, _P, _I, _I, _I, _P]
    L.orc_lowrank_pairs.argtypes = [_P, _I, _P, _I, _P, _P, _I64, _P]
    L.orc_codebook_dot_pairs.argtypes = [_P, _P, _I, _I, _P, _P, _P, _P, _I64, _P]
    L.orc_num_threads.restype = _I
    L.orc_set_threads.argtypes = [_I]


class _Rot(ctypes.Structure):
    """orc_rot: the rotation the row drivers apply."""
    _fields_ = [("kind", ctypes.c_int), ("b", ctypes.c_int), ("sign", _P), ("perm", _P),
                ("R", _P), ("m", _P), ("R2", _P)]


def _rot(rot_kind, b=0, sign=None, perm=None, R=None, m=None, R2=None):
    """A _Rot plus the contiguous arrays it points into (kept alive by the caller)."""
    keep = [None if sign is None else np.ascontiguousarray(sign, np.int8),
            None if perm is None else np.ascontiguousarray(perm, np.int32),
            None if R is None else np.ascontiguousarray(R, np.float32),
            None if m is None else np.ascontiguousarray(m, np.float32),
            None if R2 is None else np.ascontiguousarray(R2, np.float32)]
    return _Rot(rot_kind, b, *(_ptr(a) for a in keep)), keep


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's parallel row loops."""
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------------------
# single-row primitives (used by the pins)
# ---------------------------------------------------------------------------

def rpbh_row_f32(x, b, sign, perm):
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty_like(x)
    lib().orc_rpbh_row_f32(_ptr(x), x.size, b, _ptr(np.ascontiguousarray(sign, np.int8)),
                           _ptr(np.ascontiguousarray(perm, np.int32)), _ptr(y))
    return y


def rpbh_row_f64(x, b, sign, perm):
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty_like(x)
    lib().orc_rpbh_row_f64(_ptr(x), x.size, b, _ptr(np.ascontiguousarray(sign, np.int8)),
                           _ptr(np.ascontiguousarray(perm, np.int32)), _ptr(y))
    return y


def dense_row_f32(x, R):
    x = np.ascontiguousarray(x, np.float32)
    R = np.ascontiguousarray(R, np.float32)
    u = np.empty_like(x)
    lib().orc_dense_row_f32(_ptr(x), _ptr(R), x.size, _ptr(u))
    return u


def dense_row_f64(w, R):
    w = np.ascontiguousarray(w, np.float64)
    R = np.ascontiguousarray(R, np.float32)
    v = np.empty_like(w)
    lib().orc_dense_row_f64(_ptr(w), _ptr(R), w.size, _ptr(v))
    return v


def quant_int4_row(u, r=0):
    u = np.ascontiguousarray(u, np.float32)
    q = np.empty(u.size - r, np.int8)
    s = np.zeros(1, np.float32)
    lib().orc_quant_int4_row(_ptr(u), u.size, r, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def quant_int4_asym_row(u):
    """Asymmetric per-token INT4 (TR-DQ Eq.(1)-(3)): unsigned codes, s, z."""
    u = np.ascontiguousarray(u, np.float32)
    q = np.empty(u.size, np.uint8)
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.float32)
    lib().orc_quant_int4_asym_row(_ptr(u), u.size, _ptr(q), _ptr(s), _ptr(z))
    return q, np.float32(s[0]), np.float32(z[0])


def quant_int4_wrow(v):
    v = np.ascontiguousarray(v, np.float64)
    q = np.empty(v.size, np.int8)
    s = np.zeros(1, np.float32)
    lib().orc_quant_int4_wrow(_ptr(v), v.size, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def quant_sym_row(u, r=0, qmax=7):
    """Symmetric per-token quantizer with qmax 7 (INT4), 31 (6-bit) or 127 (INT8)."""
    u = np.ascontiguousarray(u, np.float32)
    q = np.zeros(u.size - r, np.int16)
    s = ctypes.c_float(0)
    lib().orc_quant_sym_row(_ptr(u), u.size, r, qmax, _ptr(q), ctypes.byref(s))
    return q, s.value


def quant_asym_row(u, levels=15):
    """Asymmetric per-token quantizer with 15 (4-bit), 63 (6-bit) or 255 (8-bit) levels."""
    u = np.ascontiguousarray(u, np.float32)
    q = np.zeros(u.size, np.uint16)
    s, z = ctypes.c_float(0), ctypes.c_float(0)
    lib().orc_quant_asym_row(_ptr(u), u.size, levels, _ptr(q), ctypes.byref(s), ctypes.byref(z))
    return q, s.value, z.value


def quant_sym_wrow(v, qmax=7):
    v = np.ascontiguousarray(v, np.float64)
    q = np.zeros(v.size, np.int16)
    s = ctypes.c_float(0)
    lib().orc_quant_sym_wrow(_ptr(v), v.size, qmax, _ptr(q), ctypes.byref(s))
    return q, s.value


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e2m1_encode(x: float) -> int:
    return lib().orc_e2m1_encode(float(x))


def mx_scale_code(amax: float) -> int:
    return lib().orc_mx_scale_code(float(amax))


def quant_mxfp4_row(u):
    """MXFP4 of an fp32 row: (codes [K/2] nibbles, E8M0 scale codes [K/32])."""
    u = np.ascontiguousarray(u, np.float32)
    codes = np.zeros(u.size // 2, np.uint8)
    sc = np.zeros(u.size // 32, np.uint8)
    lib().orc_quant_mxfp4_row(_ptr(u), u.size, _ptr(codes), _ptr(sc))
    return codes, sc


def quant_mxfp4_f64(x):
    x = np.ascontiguousarray(x, np.float64)
    codes = np.zeros(x.size // 2, np.uint8)
    sc = np.zeros(x.size // 32, np.uint8)
    lib().orc_quant_mxfp4_f64(_ptr(x), x.size, _ptr(codes), _ptr(sc))
    return codes, sc


def trdq_row_f32(x, b, m, R1, perm, R2):
    x = np.ascontiguousarray(x, np.float32)
    u = np.empty_like(x)
    keep = [np.ascontiguousarray(a, t) for a, t in ((m, np.float32), (R1, np.float32),
                                                     (perm, np.int32), (R2, np.float32))]
    lib().orc_trdq_row_f32(_ptr(x), x.size, b, *(_ptr(a) for a in keep), _ptr(u))
    return u


def trdq_row_f64(w, b, m, R1, perm, R2):
    w = np.ascontiguousarray(w, np.float64)
    v = np.empty_like(w)
    keep = [np.ascontiguousarray(a, t) for a, t in ((m, np.float32), (R1, np.float32),
                                                     (perm, np.int32), (R2, np.float32))]
    lib().orc_trdq_row_f64(_ptr(w), w.size, b, *(_ptr(a) for a in keep), _ptr(v))
    return v


def pack_nibbles(q):
    q = np.ascontiguousarray(q, np.int8)
    out = np.empty(q.size // 2, np.uint8)
    lib().orc_pack_nibbles(_ptr(q), q.size, _ptr(out))
    return out


def pack_crumbs(idx):
    idx = np.ascontiguousarray(idx, np.uint8)
    out = np.empty(idx.size // 4, np.uint8)
    lib().orc_pack_crumbs(_ptr(idx), idx.size, _ptr(out))
    return out


def norm2_grid(u):
    u = np.ascontiguousarray(u, np.float32)
    return lib().orc_norm2_grid(_ptr(u), u.size)


def quant_lloydmax_row(u, levels):
    u = np.ascontiguousarray(u, np.float32)
    lv = np.ascontiguousarray(levels, np.float32)
    idx = np.empty(u.size, np.uint8)
    s = np.zeros(1, np.float32)
    lib().orc_quant_lloydmax_row(_ptr(u), u.size, _ptr(lv), lv.size, _ptr(idx), _ptr(s))
    return idx, np.float32(s[0])


def quant_lloydmax_wrow(v, levels):
    v = np.ascontiguousarray(v, np.float64)
    lv = np.ascontiguousarray(levels, np.float32)
    idx = np.empty(v.size, np.uint8)
    s = np.zeros(1, np.float32)
    lib().orc_quant_lloydmax_wrow(_ptr(v), v.size, _ptr(lv), lv.size, _ptr(idx), _ptr(s))
    return idx, np.float32(s[0])


def f32_to_bf16(x):
    return np.array([lib().orc_f32_to_bf16(float(v)) for v in np.ravel(x)], np.uint16)


def unpack_nibbles(packed, n):
    """Signed 4-bit codes from packed bytes (low nibble = even index)."""
    p = np.ascontiguousarray(packed, np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out).astype(np.int8)
    return out[..., :n]


def unpack_crumbs(packed, n):
    p = np.ascontiguousarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 4,), np.uint8)
    for i in range(4):
        out[..., i::4] = (p >> (2 * i)) & 3
    return out[..., :n]


# ---------------------------------------------------------------------------
# Lloyd-Max codebook for the standard normal ("OrbitQuant" abstract: one
# Lloyd-Max codebook for the fixed, known marginal of a rotated coordinate)
# ---------------------------------------------------------------------------

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(t):
    return 0.0 if math.isinf(t) else _INV_SQRT_2PI * math.exp(-0.5 * t * t)


def _mass(a, b):
    """P(a < Z < b) for Z ~ N(0,1), computed without cancellation in the tails."""
    if a >= 0:
        return 0.5 * (math.erfc(a / _SQRT2) - (0.0 if math.isinf(b) else math.erfc(b / _SQRT2)))
    if b <= 0:
        return 0.5 * (math.erfc(-b / _SQRT2) - (0.0 if math.isinf(a) else math.erfc(-a / _SQRT2)))
    return 1.0 - _mass(-math.inf, a) - _mass(b, math.inf)


def lloyd_max_gaussian(L: int, tol: float = 1e-15, max_iter: int = 200000):
    """Lloyd's iteration in fp64 on the N(0,1) density.

    Alternates the two optimality conditions of a minimum-MSE scalar
    quantizer: thresholds are midpoints of adjacent levels, levels are the
    conditional means of their cells, (phi(t_i) - phi(t_i+1)) / P(cell).
    Starts from symmetric uniform levels on [-2.5, 2.5] (scaled by L) and stops
    when no level moves by more than tol.  Returns (levels, thresholds) fp64.
    """
    span = 1.0 + 0.25 * math.log2(L)
    lv = [(-span + 2.0 * span * (i + 0.5) / L) for i in range(L)]
    for _ in range(max_iter):
        th = [-math.inf] + [(lv[i] + lv[i + 1]) / 2.0 for i in range(L - 1)] + [math.inf]
        new = [(_phi(th[i]) - _phi(th[i + 1])) / _mass(th[i], th[i + 1]) for i in range(L)]
        delta = max(abs(a - b) for a, b in zip(new, lv))
        lv = new
        if delta < tol:
            break
    th = [(lv[i] + lv[i + 1]) / 2.0 for i in range(L - 1)]
    return np.array(lv, np.float64), np.array(th, np.float64)


def round_to_bf16(x: float) -> float:
    """Round an fp64 value to the nearest bf16 value (8 significant bits),
    ties to even, in one step (normal range)."""
    if x == 0.0:
        return 0.0
    m, e = math.frexp(x)             # x = m * 2^e, 0.5 <= |m| < 1
    q = Fraction(m) * 256            # exact
    rq = round(q)                    # Fraction.__round__: half to even
    return float(Fraction(rq) * Fraction(2) ** (e - 8))


def codebook_bf16(L: int) -> np.ndarray:
    """The decode levels: Lloyd-Max levels for N(0,1) rounded to bf16, fp32."""
    lv, _ = lloyd_max_gaussian(L)
    return np.array([round_to_bf16(v) for v in lv], np.float32)


# ---------------------------------------------------------------------------
# layer-level drivers
# ---------------------------------------------------------------------------

def act_rows(X, xdtype, K, rows, *, rot_kind, b=0, sign=None, perm=None, R=None,
             m=None, R2=None, r=0, q_kind=0, a_bits=4, levels=None, want_u=False):
    """Activation side for the listed rows of X (see orc_act_rows).

    X: np.float32 [T][K] (xdtype 0) or np.uint16 bf16 bits [T][K] (xdtype 1).
    rot_kind 0 RPBH (b, sign, perm), 1 dense (R, r), 2 TR-DQ (b, m, R = the
    first block rotation, perm, R2).  q_kind 0 symmetric integer, 1
    Lloyd-Max, 2 asymmetric integer (also returns the zero points), 3 MXFP4
    (also returns the E8M0 block scales); a_bits 4, 6 or 8 for the integer
    kinds (4-bit codes two per byte, 6- and 8-bit codes one per byte).
    Returns dict(codes, scale, zero, top, u, mx_scales)."""
    rows = np.ascontiguousarray(rows, np.int64)
    n = rows.size
    X = np.ascontiguousarray(X)
    Kq = K - r
    if q_kind in (1, 3):
        ncode = K // 2
    else:
        ncode = Kq // 2 if a_bits == 4 else Kq
    codes = np.zeros((n, ncode), np.uint8)
    scale = np.zeros(n, np.float32)
    zero = np.zeros(n, np.float32) if q_kind == 2 else None
    top = np.zeros((n, r), np.uint16) if r > 0 else None
    mx = np.zeros((n, K // 32), np.uint8) if q_kind == 3 else None
    u = np.zeros((n, K), np.float32) if want_u else None
    lv = None if levels is None else np.ascontiguousarray(levels, np.float32)
    rot, keep = _rot(rot_kind, b, sign, perm, R, m, R2)
    lib().orc_act_rows(_ptr(X), xdtype, K, _ptr(rows), n, ctypes.byref(rot), r, q_kind, a_bits,
                       _ptr(lv), 0 if lv is None else lv.size, _ptr(codes), _ptr(scale),
                       _ptr(zero), _ptr(top), _ptr(mx), _ptr(u))
    del keep
    return dict(codes=codes, scale=scale, zero=zero, top=top, u=u, mx_scales=mx)


def weight_rows(W, *, rot_kind, b=0, sign=None, perm=None, R=None, m=None, R2=None, q_kind=0,
                w_bits=4, levels=None):
    """Offline weight side: fold every row of W [N][K] (fp32) in fp64 and
    quantize (see orc_weight_rows).  Returns dict(codes, scale, q, mx_scales)."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    if q_kind == 1:
        # 16-level codebooks: nibbles; 4-level codebooks: crumbs
        ncode = K // 2 if len(levels) == 16 else K // 4
    elif q_kind == 3:
        ncode = K // 2
    else:
        ncode = K // 2 if w_bits == 4 else K
    codes = np.zeros((N, ncode), np.uint8)
    scale = np.zeros(N, np.float32)
    mx = np.zeros((N, K // 32), np.uint8) if q_kind == 3 else None
    q = np.zeros((N, K), np.int16)
    lv = None if levels is None else np.ascontiguousarray(levels, np.float32)
    rot, keep = _rot(rot_kind, b, sign, perm, R, m, R2)
    lib().orc_weight_rows(_ptr(W), N, K, ctypes.byref(rot), q_kind, w_bits, _ptr(lv),
                          0 if lv is None else lv.size, _ptr(codes), _ptr(scale), _ptr(mx), _ptr(q))
    del keep
    return dict(codes=codes, scale=scale, q=q, mx_scales=mx)


def int_gemm(codes_a, Kq, codes_w, Kw, koff=0):
    """acc[t][n] = sum_k qa[t][k] qw[n][koff+k], int64 (small shapes)."""
    codes_a = np.ascontiguousarray(codes_a, np.uint8)
    codes_w = np.ascontiguousarray(codes_w, np.uint8)
    T, N = codes_a.shape[0], codes_w.shape[0]
    acc = np.zeros((T, N), np.int64)
    lib().orc_int_gemm(_ptr(codes_a), T, Kq, _ptr(codes_w), N, Kw, koff, _ptr(acc))
    return acc


def int_gemm_pairs(codes_a, Kq, codes_w, Kw, ta, nw, koff=0):
    ta = np.ascontiguousarray(ta, np.int64)
    nw = np.ascontiguousarray(nw, np.int64)
    acc = np.zeros(ta.size, np.int64)
    lib().orc_int_gemm_pairs(_ptr(np.ascontiguousarray(codes_a, np.uint8)), Kq,
                             _ptr(np.ascontiguousarray(codes_w, np.uint8)), Kw, koff,
                             _ptr(ta), _ptr(nw), ta.size, _ptr(acc))
    return acc


def asym_gemm_pairs(codes_a, codes_w, K, ta, nw):
    """acc[p] = sum_k ua[t_p][k] qw[n_p][k] (unsigned activation codes)."""
    ta = np.ascontiguousarray(ta, np.int64)
    nw = np.ascontiguousarray(nw, np.int64)
    acc = np.zeros(ta.size, np.int64)
    lib().orc_asym_gemm_pairs(_ptr(np.ascontiguousarray(codes_a, np.uint8)), K,
                              _ptr(np.ascontiguousarray(codes_w, np.uint8)),
                              _ptr(ta), _ptr(nw), ta.size, _ptr(acc))
    return acc


def gemm_codes_pairs(codes_a, a_bits, a_signed, Kq, codes_w, w_bits, Kw, ta, nw, koff=0):
    """acc[p] = sum_k a[t_p][k] w[n_p][koff + k] for 4-, 6- or 8-bit codes
    (6-bit codes one per byte), int64."""
    ta = np.ascontiguousarray(ta, np.int64)
    nw = np.ascontiguousarray(nw, np.int64)
    acc = np.zeros(ta.size, np.int64)
    lib().orc_gemm_codes_pairs(_ptr(np.ascontiguousarray(codes_a, np.uint8)), a_bits,
                               1 if a_signed else 0, Kq,
                               _ptr(np.ascontiguousarray(codes_w, np.uint8)), w_bits, Kw, koff,
                               _ptr(ta), _ptr(nw), ta.size, _ptr(acc))
    return acc


def mx_dot_pairs(codes_a, sc_a, codes_w, sc_w, K, ta, nw):
    """fp64 MXFP4 dot products for listed pairs (see orc_mx_dot_pairs)."""
    ta = np.ascontiguousarray(ta, np.int64)
    nw = np.ascontiguousarray(nw, np.int64)
    dot = np.zeros(ta.size, np.float64)
    lib().orc_mx_dot_pairs(_ptr(np.ascontiguousarray(codes_a, np.uint8)),
                           _ptr(np.ascontiguousarray(sc_a, np.uint8)),
                           _ptr(np.ascontiguousarray(codes_w, np.uint8)),
                           _ptr(np.ascontiguousarray(sc_w, np.uint8)), K,
                           _ptr(ta), _ptr(nw), ta.size, _ptr(dot))
    return dot


def lowrank_pairs(top, r, codes_w, Kw, ta, nw):
    ta = np.ascontiguousarray(ta, np.int64)
    nw = np.ascontiguousarray(nw, np.int64)
    lr = np.zeros(ta.size, np.float64)
    lib().orc_lowrank_pairs(_ptr(np.ascontiguousarray(top, np.uint16)), r,
                            _ptr(np.ascontiguousarray(codes_w, np.uint8)), Kw,
                            _ptr(ta), _ptr(nw), ta.size, _ptr(lr))
    return lr


def codebook_dot_pairs(codes_a, codes_w, K, a_lv, w_lv, ta, nw):
    """fp64 sum_k a_lv[ia] w_lv[iw] for listed pairs; the weight index width
    (2 or 4 bits) follows the size of w_lv (4 or 16 levels)."""
    ta = np.ascontiguousarray(ta, np.int64)
    nw = np.ascontiguousarray(nw, np.int64)
    dot = np.zeros(ta.size, np.float64)
    w_bits = {4: 2, 16: 4}[len(w_lv)]
    lib().orc_codebook_dot_pairs(_ptr(np.ascontiguousarray(codes_a, np.uint8)),
                                 _ptr(np.ascontiguousarray(codes_w, np.uint8)), K, w_bits,
                                 _ptr(np.ascontiguousarray(a_lv, np.float32)),
                                 _ptr(np.ascontiguousarray(w_lv, np.float32)),
                                 _ptr(ta), _ptr(nw), ta.size, _ptr(dot))
    return dot


def yhat_int4(s_a, s_w, acc, b_eff, lr=None):
    """fp64 dequantized output of the INT4 paths ([TRDQ] 3.1, per-token x
    per-channel scales):  RPBH:  s_a s_w acc / b;  dense: s_w (lr + s_a acc)."""
    s_a = np.asarray(s_a, np.float64)
    s_w = np.asarray(s_w, np.float64)
    acc = np.asarray(acc, np.float64)
    if lr is None:
        return s_a * s_w * acc / float(b_eff)
    return s_w * (np.asarray(lr, np.float64) + s_a * acc) / float(b_eff)


def yhat_int4_asym(s_a, z_a, s_w, acc_u, wsum, b):
    """fp64 output with asymmetric activations ([TRDQ] 3.1: X ~ s (X_int - z)):
    s_a s_w (sum_k ua qw - z sum_k qw) / b."""
    return (np.asarray(s_a, np.float64) * np.asarray(s_w, np.float64) *
            (np.asarray(acc_u, np.float64) -
             np.asarray(z_a, np.float64) * np.asarray(wsum, np.float64)) / float(b))


def yhat_codebook(sigma, tau, dot, b):
    """fp64 output of the Lloyd-Max path: sigma tau / b * codebook dot."""
    return (np.asarray(sigma, np.float64) * np.asarray(tau, np.float64) *
            np.asarray(dot, np.float64) / float(b))


def yhat_mx(dot, b):
    """fp64 output of the MXFP4 path: the block-scaled dot product / b (the
    unnormalized block Hadamard scales dot products by b)."""
    return np.asarray(dot, np.float64) / float(b)

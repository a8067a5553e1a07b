"""Thin ctypes binding of librq (include/rq.h): argument marshalling only.

Every computation runs inside librq's gfx950 kernels (or, for the offline
weight pack, in librq's host code).  This module converts numpy / torch
arguments into the C structs and raw pointers of the C ABI, passes the
current HIP stream, and raises RQError on any non-OK status.  There is no
fallback: if librq.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librq.so")

RQ_OK = 0
RQ_F32, RQ_BF16, RQ_I32 = 0, 1, 2
RQ_ROT_RPBH, RQ_ROT_DENSE, RQ_ROT_TRDQ = 0, 1, 2
RQ_Q_INT4_SYM, RQ_Q_LLOYDMAX, RQ_Q_INT4_ASYM, RQ_Q_MXFP4 = 0, 1, 2, 3
RQ_ENGINE_AUTO, RQ_ENGINE_FP6, RQ_ENGINE_INT8 = 0, 1, 2
ENGINES = {"auto": RQ_ENGINE_AUTO, "fp6": RQ_ENGINE_FP6, "int8": RQ_ENGINE_INT8}
RQ_WEIGHT_MAGIC = 0x31575152
STATUS_NAMES = {0: "RQ_OK", -1: "RQ_ERR_NULL", -2: "RQ_ERR_SHAPE", -3: "RQ_ERR_DTYPE",
                -4: "RQ_ERR_ALIGN", -5: "RQ_ERR_FORMAT", -6: "RQ_ERR_UNSUPPORTED",
                -7: "RQ_ERR_HIP"}


class RQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class c_rotation(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("K", ctypes.c_int32), ("block", ctypes.c_int32),
                ("r", ctypes.c_int32), ("sign", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("R", ctypes.c_void_p), ("smooth", ctypes.c_void_p), ("R2", ctypes.c_void_p)]


class c_quant(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("a_bits", ctypes.c_int32), ("w_bits", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("a_levels", ctypes.c_float * 16),
                ("w_levels", ctypes.c_float * 16)]


class c_weight_header(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("format", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32),
                ("r", ctypes.c_int32), ("b_div", ctypes.c_int32), ("a_bits", ctypes.c_int32),
                ("w_bits", ctypes.c_int32), ("row_bytes", ctypes.c_int32),
                ("scale_offset", ctypes.c_int64), ("codes_offset", ctypes.c_int64),
                ("total_bytes", ctypes.c_int64), ("a_levels", ctypes.c_float * 16),
                ("w_levels", ctypes.c_float * 16), ("wsum_offset", ctypes.c_int64),
                ("mma_offset", ctypes.c_int64), ("mma_stages", ctypes.c_int32),
                ("mma_ntiles", ctypes.c_int32), ("i8_offset", ctypes.c_int64),
                ("mxs_offset", ctypes.c_int64), ("reserved", ctypes.c_uint8 * 24)]


assert ctypes.sizeof(c_weight_header) == 256


class c_set_header(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("groups", ctypes.c_int32), ("steps", ctypes.c_int32),
                ("member_offset", ctypes.c_int64 * 64), ("step_group", ctypes.c_int32 * 1024),
                ("reserved", ctypes.c_uint8 * (4864 - 16 - 8 * 64 - 4 * 1024))]


assert ctypes.sizeof(c_set_header) == 4864

# every symbol include/rq.h declares
EXPORTS = ("rq_version", "rq_last_error", "rq_lloydmax_gaussian", "rq_packed_weight_bytes",
           "rq_pack_weights", "rq_rotate_quant_workspace_bytes", "rq_codes_mma_bytes",
           "rq_rotate_quant", "rq_w4a4_linear", "rq_w4a4_linear_engine",
           "rq_rotate_quant_noalloc", "rq_activation_bytes", "rq_weight_set_bytes",
           "rq_pack_weight_set", "rq_weight_set_member")

_lib = None


def load() -> ctypes.CDLL:
    """Load librq.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with `python -m rotated_w4a4_quantized_amd.build` "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.rq_version.restype = I32
    L.rq_last_error.restype = ctypes.c_char_p
    L.rq_lloydmax_gaussian.argtypes = [I32, P]
    L.rq_packed_weight_bytes.argtypes = [P, P, I32, ctypes.POINTER(SZ)]
    L.rq_pack_weights.argtypes = [P, P, P, I32, I32, P, SZ]
    L.rq_rotate_quant_workspace_bytes.argtypes = [P, P, I64, ctypes.POINTER(SZ)]
    L.rq_codes_mma_bytes.argtypes = [P, I64, ctypes.POINTER(SZ)]
    L.rq_rotate_quant.argtypes = [P, P, P, I32, I64, P, P, P, P, P, SZ, P]
    L.rq_w4a4_linear.argtypes = [P, P, P, P, P, P, I64, P, P, I32, P]
    L.rq_w4a4_linear_engine.argtypes = [P, P, P, P, P, P, I64, P, P, I32, I32, P]
    L.rq_rotate_quant_noalloc.argtypes = [P, P, P, I32, I64, P, P, P, P, P]
    L.rq_activation_bytes.argtypes = [P, P, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ),
                                      ctypes.POINTER(SZ)]
    L.rq_weight_set_bytes.argtypes = [P, I32, P, I32, ctypes.POINTER(SZ)]
    L.rq_pack_weight_set.argtypes = [P, I32, P, I32, P, P, I32, I32, P, SZ]
    L.rq_weight_set_member.argtypes = [P, I32, ctypes.POINTER(I32), ctypes.POINTER(P),
                                       ctypes.POINTER(I64)]
    for name in ("rq_lloydmax_gaussian", "rq_packed_weight_bytes", "rq_pack_weights",
                 "rq_rotate_quant_workspace_bytes", "rq_codes_mma_bytes", "rq_rotate_quant",
                 "rq_w4a4_linear", "rq_w4a4_linear_engine", "rq_rotate_quant_noalloc",
                 "rq_activation_bytes", "rq_weight_set_bytes", "rq_pack_weight_set",
                 "rq_weight_set_member"):
        getattr(L, name).restype = I32
    _lib = L
    return L


def _check(status: int):
    if status != RQ_OK:
        raise RQError(status, load().rq_last_error().decode())


def _np_ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _t_ptr(t):
    if t is None:
        return None
    assert t.is_contiguous(), "device buffers must be contiguous"
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

@dataclass
class Rotation:
    """Host description of a rotation (numpy arrays)."""
    kind: int
    K: int
    block: int = 0
    r: int = 0
    sign: Optional[np.ndarray] = None
    perm: Optional[np.ndarray] = None
    R: Optional[np.ndarray] = None
    smooth: Optional[np.ndarray] = None
    R2: Optional[np.ndarray] = None

    @staticmethod
    def rpbh(sign, perm, block):
        sign = np.ascontiguousarray(sign, np.int8)
        perm = np.ascontiguousarray(perm, np.int32)
        return Rotation(RQ_ROT_RPBH, int(sign.size), int(block), 0, sign, perm, None)

    @staticmethod
    def dense(R, r):
        R = np.ascontiguousarray(R, np.float32)
        return Rotation(RQ_ROT_DENSE, int(R.shape[0]), 0, int(r), None, None, R)

    @staticmethod
    def trdq(smooth, R1, perm, R2, block):
        """TR-DQ: smoothing multiplier [K], block rotations R1, R2 [K/b][b][b],
        zigzag permutation [K] (a gather)."""
        smooth = np.ascontiguousarray(smooth, np.float32)
        return Rotation(RQ_ROT_TRDQ, int(smooth.size), int(block), 0, None,
                        np.ascontiguousarray(perm, np.int32), np.ascontiguousarray(R1, np.float32),
                        smooth, np.ascontiguousarray(R2, np.float32))

    def c_host(self) -> c_rotation:
        ptr = (lambda a: None if a is None else a.ctypes.data)
        return c_rotation(self.kind, self.K, self.block, self.r, ptr(self.sign), ptr(self.perm),
                          ptr(self.R), ptr(self.smooth), ptr(self.R2))

    def to_device(self, device="cuda") -> "DeviceRotation":
        import torch
        d = DeviceRotation(self)
        for name in ("sign", "perm", "R", "smooth", "R2"):
            a = getattr(self, name)
            if a is not None:
                setattr(d, name, torch.from_numpy(a).to(device))
        return d


@dataclass
class DeviceRotation:
    host: Rotation
    sign: object = None
    perm: object = None
    R: object = None
    smooth: object = None
    R2: object = None

    def c_dev(self) -> c_rotation:
        h = self.host
        ptr = (lambda t: None if t is None else t.data_ptr())
        return c_rotation(h.kind, h.K, h.block, h.r, ptr(self.sign), ptr(self.perm), ptr(self.R),
                          ptr(self.smooth), ptr(self.R2))


@dataclass
class Quant:
    kind: int = RQ_Q_INT4_SYM
    a_bits: int = 4
    w_bits: int = 4
    a_levels: Optional[np.ndarray] = None
    w_levels: Optional[np.ndarray] = None

    @staticmethod
    def int4():
        return Quant(RQ_Q_INT4_SYM, 4, 4)

    @staticmethod
    def int4_asym():
        """Asymmetric per-token INT4 activations (zero point), INT4 weights."""
        return Quant(RQ_Q_INT4_ASYM, 4, 4)

    @staticmethod
    def integer(a_bits, w_bits, asym=False):
        """Integer activations of a_bits (4, 6 or 8, zero point if asym) and
        symmetric weights of w_bits (W4A4, W4A8, W8A8, W6A6); 6- and 8-bit
        codes are stored one per byte."""
        return Quant(RQ_Q_INT4_ASYM if asym else RQ_Q_INT4_SYM, a_bits, w_bits)

    @staticmethod
    def mxfp4():
        """MXFP4: E2M1 elements, one E8M0 scale per 32 coordinates."""
        return Quant(RQ_Q_MXFP4, 4, 4)

    @property
    def scale_rows(self) -> int:
        """Rows of the fp32 scale output per token set: 2 (s, z) for INT4_ASYM."""
        return 2 if self.kind == RQ_Q_INT4_ASYM else 1

    @staticmethod
    def lloydmax(a_levels, w_levels):
        a = np.ascontiguousarray(a_levels, np.float32)
        w = np.ascontiguousarray(w_levels, np.float32)
        return Quant(RQ_Q_LLOYDMAX, 4, int(np.log2(w.size)), a, w)

    def c(self) -> c_quant:
        q = c_quant(self.kind, self.a_bits, self.w_bits, 0)
        if self.a_levels is not None:
            for i, v in enumerate(self.a_levels):
                q.a_levels[i] = float(v)
        if self.w_levels is not None:
            for i, v in enumerate(self.w_levels):
                q.w_levels[i] = float(v)
        return q


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def version() -> int:
    return load().rq_version()


def lloydmax_gaussian(L: int) -> np.ndarray:
    out = np.zeros(L, np.float32)
    _check(load().rq_lloydmax_gaussian(L, _np_ptr(out)))
    return out


def packed_weight_bytes(rot: Rotation, q: Quant, N: int) -> int:
    n = ctypes.c_size_t(0)
    cr, cq = rot.c_host(), q.c()
    _check(load().rq_packed_weight_bytes(ctypes.byref(cr), ctypes.byref(cq), N, ctypes.byref(n)))
    return n.value


@dataclass
class PackedWeights:
    blob: np.ndarray                      # uint8, host
    header: c_weight_header = field(default=None)

    @property
    def N(self):
        return self.header.N

    @property
    def K(self):
        return self.header.K

    def scales(self) -> np.ndarray:
        h = self.header
        return self.blob[h.scale_offset:h.scale_offset + 4 * h.N].view(np.float32)

    def codes(self) -> np.ndarray:
        h = self.header
        return self.blob[h.codes_offset:h.codes_offset + h.N * h.row_bytes].reshape(h.N, h.row_bytes)

    def wsum(self) -> np.ndarray:
        """INT4: per-channel sums of the quantized weight codes (int32 [N])."""
        h = self.header
        return self.blob[h.wsum_offset:h.wsum_offset + 4 * h.N].view(np.int32)

    def mx_scales(self) -> np.ndarray:
        """MXFP4: the E8M0 codes, uint8 [N][K/32]."""
        h = self.header
        return self.blob[h.scale_offset:h.scale_offset + h.N * (h.K // 32)].reshape(h.N, h.K // 32)

    def i8_codes(self) -> np.ndarray:
        """INT with 8-bit activations: the int8 weight codes [N][K], read back
        from the blob's fragment order [N/32][K/32][64 lanes][16 bytes] (lane
        l: row 32 tile + l % 32, coordinates 32 kb + 16 (l / 32) .. + 15)."""
        h = self.header
        tiles = -(-h.N // 32)
        raw = self.blob[h.i8_offset:h.i8_offset + tiles * 32 * h.K].view(np.int8)
        v = raw.reshape(tiles, h.K // 32, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(tiles * 32, h.K)
        return v[:h.N]

    def mma_tiles(self) -> np.ndarray:
        """INT4: the GEMM's FP6 fragments, uint8 [ntiles][stages][3][64][16]."""
        h = self.header
        n = h.mma_ntiles * h.mma_stages * 3 * 1024
        return self.blob[h.mma_offset:h.mma_offset + n].reshape(h.mma_ntiles, h.mma_stages, 3, 64, 16)

    def to_device(self, device="cuda") -> "DeviceWeights":
        import torch
        return DeviceWeights(self.header, torch.from_numpy(self.blob).to(device))


@dataclass
class DeviceWeights:
    header: c_weight_header
    blob: object                          # torch uint8 tensor on the GPU

    @property
    def N(self):
        return self.header.N


def pack_weights(rot: Rotation, q: Quant, W: np.ndarray) -> PackedWeights:
    """Offline fold + quantize + pack (librq host code)."""
    if W.dtype == np.float32:
        wdt = RQ_F32
    elif W.dtype == np.uint16:
        wdt = RQ_BF16
    else:
        raise TypeError("W must be float32 or bf16 bit patterns (uint16)")
    W = np.ascontiguousarray(W)
    N = int(W.shape[0])
    nbytes = packed_weight_bytes(rot, q, N)
    blob = np.zeros(nbytes, np.uint8)
    cr, cq = rot.c_host(), q.c()
    _check(load().rq_pack_weights(ctypes.byref(cr), ctypes.byref(cq), _np_ptr(W), wdt, N,
                                  _np_ptr(blob), nbytes))
    hdr = c_weight_header.from_buffer_copy(blob[:256].tobytes())
    return PackedWeights(blob, hdr)


class WeightSet:
    """A time-step set (host blob): per group the weights folded with that
    group's rotation, and the step -> group table."""

    def __init__(self, blob: np.ndarray):
        self.blob = blob
        self.device_blob = None

    def member(self, step: int):
        """(group, header, byte offset) of the blob that step uses."""
        g = ctypes.c_int32(0)
        h = ctypes.c_void_p(0)
        off = ctypes.c_int64(0)
        _check(load().rq_weight_set_member(_np_ptr(self.blob), step, ctypes.byref(g),
                                           ctypes.byref(h), ctypes.byref(off)))
        hdr = c_weight_header.from_buffer_copy(self.blob[off.value:off.value + 256].tobytes())
        return g.value, hdr, off.value

    def to_device(self, device="cuda"):
        import torch
        self.device_blob = torch.from_numpy(self.blob).to(device)
        return self

    def device_member(self, step: int) -> "DeviceWeights":
        """The DeviceWeights of the step's member: a view into the device set."""
        g, hdr, off = self.member(step)
        return DeviceWeights(hdr, self.device_blob[off:off + hdr.total_bytes])


def pack_weight_set(rots, step_group, q: Quant, W: np.ndarray) -> WeightSet:
    """Offline packing of a time-step set (rq_pack_weight_set)."""
    W = np.ascontiguousarray(W, np.float32)
    N = int(W.shape[0])
    arr = (c_rotation * len(rots))(*[r.c_host() for r in rots])
    cq = q.c()
    n = ctypes.c_size_t(0)
    _check(load().rq_weight_set_bytes(arr, len(rots), ctypes.byref(cq), N, ctypes.byref(n)))
    blob = np.zeros(n.value, np.uint8)
    sg = np.ascontiguousarray(step_group, np.int32)
    _check(load().rq_pack_weight_set(arr, len(rots), _np_ptr(sg), sg.size, ctypes.byref(cq),
                                     _np_ptr(W), RQ_F32, N, _np_ptr(blob), n.value))
    return WeightSet(blob)


def rotate_quant_workspace_bytes(rot: Rotation, q: Quant, T: int) -> int:
    n = ctypes.c_size_t(0)
    cr, cq = rot.c_host(), q.c()
    _check(load().rq_rotate_quant_workspace_bytes(ctypes.byref(cr), ctypes.byref(cq), T,
                                                  ctypes.byref(n)))
    return n.value


def activation_bytes(rot: Rotation, q: Quant, T: int):
    """(codes, scale, codes_mma) byte counts of the activation buffers."""
    c, sc, m = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    cr, cq = rot.c_host(), q.c()
    _check(load().rq_activation_bytes(ctypes.byref(cr), ctypes.byref(cq), T, ctypes.byref(c),
                                      ctypes.byref(sc), ctypes.byref(m)))
    return c.value, sc.value, m.value


def dtype_code(t) -> int:
    import torch
    return {torch.float32: RQ_F32, torch.bfloat16: RQ_BF16, torch.int16: RQ_BF16,
            torch.uint16: RQ_BF16, torch.int32: RQ_I32}[t.dtype]


def codes_mma_bytes(rot: Rotation, T: int) -> int:
    n = ctypes.c_size_t(0)
    cr = rot.c_host()
    _check(load().rq_codes_mma_bytes(ctypes.byref(cr), T, ctypes.byref(n)))
    return n.value


def rotate_quant(drot: DeviceRotation, q: Quant, X, codes, scale, top=None, workspace=None,
                 stream=None, codes_mma=None):
    """Launch the activation kernels on `stream` (default: torch's current).
    codes and/or codes_mma (the GEMM's matrix-core layout of this format:
    FP6 fragments for INT 4-bit, int8 fragments for INT 8-bit, tiled codes
    and scales for MXFP4, bf16 level fragments for Lloyd-Max) receive the
    codes; scale holds T floats, or 2T (s then z) for INT4_ASYM."""
    cr, cq = drot.c_dev(), q.c()
    T = int(X.shape[0])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    # (MXFP4: scale is a uint8 tensor of E8M0 codes, passed as a pointer)
    _check(load().rq_rotate_quant(ctypes.byref(cr), ctypes.byref(cq), _t_ptr(X), dtype_code(X), T,
                                  _t_ptr(codes), _t_ptr(scale), _t_ptr(top), _t_ptr(codes_mma),
                                  _t_ptr(workspace), ws_bytes, _stream(stream)))


def rotate_quant_noalloc(drot: DeviceRotation, q: Quant, X, codes, scale, top=None, stream=None,
                         codes_mma=None):
    """rq_rotate_quant_noalloc: rotate_quant without a workspace (the library's
    per-device scratch serves DENSE)."""
    cr, cq = drot.c_dev(), q.c()
    T = int(X.shape[0])
    _check(load().rq_rotate_quant_noalloc(ctypes.byref(cr), ctypes.byref(cq), _t_ptr(X),
                                          dtype_code(X), T, _t_ptr(codes), _t_ptr(scale),
                                          _t_ptr(top), _t_ptr(codes_mma), _stream(stream)))


def w4a4_linear(dw: DeviceWeights, codes, scale, Y, top=None, bias=None, T=None, stream=None,
                codes_mma=None, engine="auto"):
    """Launch the low-bit GEMM; Y dtype picks the output (f32, bf16, raw int32).
    When codes_mma is given it is read instead of codes (which may be None).
    engine: "auto" (rq_w4a4_linear), or "fp6" / "int8" (rq_w4a4_linear_engine)."""
    if T is None:
        if codes is None:
            raise ValueError("T must be given when codes is None")
        T = int(codes.shape[0])
    args = (ctypes.byref(dw.header), _t_ptr(dw.blob), _t_ptr(codes), _t_ptr(scale), _t_ptr(top),
            _t_ptr(codes_mma), T, _t_ptr(bias), _t_ptr(Y), dtype_code(Y))
    if engine == "auto":
        _check(load().rq_w4a4_linear(*args, _stream(stream)))
    else:
        _check(load().rq_w4a4_linear_engine(*args, ENGINES[engine], _stream(stream)))

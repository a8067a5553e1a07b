"""Seeded synthetic inputs for the rotated low-bit linear layer.

This module only draws inputs: activations shaped like diffusion-transformer
tokens, weights, the random signs and permutation of the RPBH rotation, the
dense PCA basis of the DiRotQ path and its calibration sample.  It holds none
of the layer's arithmetic (no rotation, quantization or GEMM), so the product
path and the CPU oracle can both take their inputs from it.

Workloads (token counts include the two classifier-free-guidance branches
stacked into one batch):

  tiny   256 x 1152 -> 1152, fp32 input, RPBH block 128, INT4
  pixart 8192 x 1152 -> 4608, bf16, dense PCA basis, top 32 kept bf16, INT4
  flux_up   9216 x 3072 -> 12288, bf16, RPBH block 256, INT4
  flux_down 9216 x 12288 -> 3072, bf16 (GELU-shaped), RPBH block 512, INT4
  video  32760 x 1536 -> 8960, bf16, RPBH block 256, Lloyd-Max A4 / W2

and variants of the FLUX up-projection for the other formats: MXFP4
(E2M1 + E8M0 per 32), INT8 activations (W4A8, W8A8), and TR-DQ's runtime
rotation (smoothing, block rotation, zigzag permutation, block rotation).

Random streams: numpy PCG64 seeded from SeedSequence(1000 + i) for workload
i, with spawned child streams for X, W, sign, perm and the calibration
sample, so every tensor is reproducible on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    K: int
    N: int
    rot: str            # "rpbh" | "dense" | "trdq"
    block: int          # RPBH / TR-DQ block (0 for dense)
    r: int              # top-r kept in bf16 (dense only)
    quant: str          # "int4" | "int4_asym" | "lloydmax" | "mxfp4"; int4* with a_bits 6 or 8 = 6- or 8-bit activations
    xdtype: str         # "f32" | "bf16"
    ydtype: str         # "f32" | "bf16"
    x_kind: str         # distribution recipe of X
    a_bits: int = 4
    w_bits: int = 4

    @property
    def Kq(self) -> int:
        return self.K - self.r

    @property
    def b_eff(self) -> int:
        return self.block if self.rot == "rpbh" else 1

    @property
    def code_bytes(self) -> int:
        """Bytes of activation codes per token at the method's minimal
        encoding (the canonical layout stores 6-bit codes one per byte)."""
        return self.Kq * self.a_bits // 8

    def ops(self) -> int:
        """Algorithmic GEMM operations 2*T*Kq*N (multiply-add counted as 2)."""
        return 2 * self.T * self.Kq * self.N

    def with_shape(self, T=None, K=None, N=None, block=None, w_bits=None, a_bits=None) -> "Workload":
        return replace(self, T=self.T if T is None else T, K=self.K if K is None else K,
                       N=self.N if N is None else N,
                       block=self.block if block is None else block,
                       w_bits=self.w_bits if w_bits is None else w_bits,
                       a_bits=self.a_bits if a_bits is None else a_bits)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 256, 1152, 1152, "rpbh", 128, 0, "int4", "f32", "f32",
                     "gauss_outlier8x50"),
    "pixart": Workload("pixart", 1, 8192, 1152, 4608, "dense", 0, 32, "int4", "bf16", "bf16",
                       "gauss_t4rows_outlier16x30"),
    "flux_up": Workload("flux_up", 2, 9216, 3072, 12288, "rpbh", 256, 0, "int4", "bf16", "bf16",
                        "gauss_outlier16x30"),
    "flux_down": Workload("flux_down", 3, 9216, 12288, 3072, "rpbh", 512, 0, "int4", "bf16",
                          "bf16", "gelu"),
    # the FLUX layers with asymmetric per-token activations (zero point): same
    # seeds, so the same X, W and rotation as flux_up / flux_down
    "flux_up_asym": Workload("flux_up_asym", 2, 9216, 3072, 12288, "rpbh", 256, 0, "int4_asym",
                             "bf16", "bf16", "gauss_outlier16x30"),
    "flux_down_asym": Workload("flux_down_asym", 3, 9216, 12288, 3072, "rpbh", 512, 0, "int4_asym",
                               "bf16", "bf16", "gelu"),
    "video": Workload("video", 4, 32760, 1536, 8960, "rpbh", 256, 0, "lloydmax", "bf16", "bf16",
                      "gauss", a_bits=4, w_bits=2),
    # OrbitQuant's W4A4 setting on the same layer (same seeds as video): a
    # 16-level weight book instead of the 4-level one
    "video_w4": Workload("video_w4", 4, 32760, 1536, 8960, "rpbh", 256, 0, "lloydmax", "bf16", "bf16",
                         "gauss", a_bits=4, w_bits=4),
    # the FP4 format variant (MXFP4: E2M1 elements, one E8M0 scale per 32
    # coordinates) on the FLUX layers, same seeds as flux_up / flux_down
    "flux_up_mxfp4": Workload("flux_up_mxfp4", 2, 9216, 3072, 12288, "rpbh", 256, 0, "mxfp4",
                              "bf16", "bf16", "gauss_outlier16x30"),
    "flux_down_mxfp4": Workload("flux_down_mxfp4", 3, 9216, 12288, 3072, "rpbh", 512, 0, "mxfp4",
                                "bf16", "bf16", "gelu"),
    # INT8 activations (TR-DQ's W4A8 and W8A8 settings) on the FLUX up-projection
    "flux_up_w4a8": Workload("flux_up_w4a8", 2, 9216, 3072, 12288, "rpbh", 256, 0, "int4", "bf16",
                             "bf16", "gauss_outlier16x30", a_bits=8, w_bits=4),
    "flux_up_w8a8": Workload("flux_up_w8a8", 2, 9216, 3072, 12288, "rpbh", 256, 0, "int4", "bf16",
                             "bf16", "gauss_outlier16x30", a_bits=8, w_bits=8),
    # TR-DQ's runtime rotation (smoothing, block rotation 128, zigzag
    # permutation, block rotation 128) with its W4A8 setting
    "flux_up_trdq": Workload("flux_up_trdq", 2, 9216, 3072, 12288, "trdq", 128, 0, "int4", "bf16",
                             "bf16", "gauss_outlier16x30", a_bits=8, w_bits=4),
    # TR-DQ's W6A6 setting: 6-bit codes (one per byte) on the int8 matrix
    # cores, with TR-DQ's rotation and with RPBH
    "flux_up_trdq_w6a6": Workload("flux_up_trdq_w6a6", 2, 9216, 3072, 12288, "trdq", 128, 0, "int4",
                                  "bf16", "bf16", "gauss_outlier16x30", a_bits=6, w_bits=6),
    "flux_up_w6a6": Workload("flux_up_w6a6", 2, 9216, 3072, 12288, "rpbh", 256, 0, "int4", "bf16",
                             "bf16", "gauss_outlier16x30", a_bits=6, w_bits=6),
}


def _streams(w: Workload, seed_offset: int = 0):
    ss = np.random.SeedSequence(1000 + w.index + seed_offset)
    kids = ss.spawn(6)
    names = ("x", "w", "sign", "perm", "calib", "extra")
    return {n: np.random.Generator(np.random.PCG64(k)) for n, k in zip(names, kids)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the bit patterns
    as uint16.  Only used to produce bf16 inputs."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + up.astype(np.uint64)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _gelu_erf(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def _draw_x(w: Workload, g: np.random.Generator, T: int, K: int, outlier_cols=None):
    """fp32 activations [T][K] for the workload's recipe."""
    kind = w.x_kind
    if kind == "gelu":
        z = g.standard_normal((T, K), dtype=np.float32)
        return _gelu_erf(z.astype(np.float64)).astype(np.float32)
    x = g.standard_normal((T, K), dtype=np.float32)
    if kind.startswith("gauss_t4rows"):
        # a random eighth of the rows are heavy-tailed Student-t (df = 4)
        nt = T // 8
        rows = g.choice(T, size=nt, replace=False) if nt > 0 else np.zeros(0, np.int64)
        x[rows] = g.standard_t(4.0, size=(nt, K)).astype(np.float32)
    if "outlier" in kind:
        spec = kind.split("outlier")[1]           # e.g. "16x30"
        cnt, mag = (int(v) for v in spec.split("x"))
        cnt = min(cnt, K)
        cols = outlier_cols if outlier_cols is not None else g.choice(K, size=cnt, replace=False)
        x[:, cols] *= np.float32(mag)
    return x


def make_inputs(w: Workload, seed_offset: int = 0, W=None) -> dict:
    """All inputs of one workload instance.

    Returns dict with:
      X     np.float32 [T][K] (fp32 workloads) or np.uint16 bf16 bits [T][K]
      Xf    np.float32 [T][K]: X widened to fp32 (for reporting only)
      W     np.float32 [N][K] ~ N(0, 0.02^2)
      sign  np.int8 [K] in {-1, +1}          (RPBH)
      perm  np.int32 [K], a uniform permutation (RPBH)
      R     np.float32 [K][K] dense PCA basis (dense), columns by descending
            variance of a separate 4096-row calibration sample
    """
    s = _streams(w, seed_offset)
    T, K, N = w.T, w.K, w.N
    # outlier channels are a property of the layer: the calibration sample of
    # the dense path shares them with the runtime tokens
    cols = None
    if "outlier" in w.x_kind:
        spec = w.x_kind.split("outlier")[1]
        cnt = min(int(spec.split("x")[0]), K)
        cols = s["extra"].choice(K, size=cnt, replace=False)
    xf = _draw_x(w, s["x"], T, K, cols)
    out = {"workload": w}
    if w.xdtype == "bf16":
        out["X"] = f32_to_bf16_bits(xf)
        out["Xf"] = bf16_bits_to_f32(out["X"])
    else:
        out["X"] = xf
        out["Xf"] = xf
    out["W"] = (s["w"].standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    if W is not None:   # a given layer (time-step sets: one W, several rotations)
        out["W"] = np.ascontiguousarray(W, np.float32)
    if w.rot == "rpbh":
        out["sign"] = np.where(s["sign"].integers(0, 2, size=K) == 1, 1, -1).astype(np.int8)
        out["perm"] = s["perm"].permutation(K).astype(np.int32)
        out["R"] = None
    elif w.rot == "trdq":
        calib = _draw_x(w, s["calib"], 1024, K, cols)
        if w.xdtype == "bf16":
            calib = bf16_bits_to_f32(f32_to_bf16_bits(calib))
        out.update(trdq_rotation(calib, out["W"], w.block, s["perm"]))
        out["sign"] = None
    else:
        out["sign"] = None
        out["perm"] = None
        out["R"] = pca_basis(_draw_x(w, s["calib"], 4096, K, cols))
    return out


def pca_basis(calib: np.ndarray) -> np.ndarray:
    """Dense orthogonal basis from a calibration sample (stand-in for the
    calibration step that produces the rotation): eigenvectors of the centered
    covariance, fp64, ordered by descending eigenvalue (ties by index), each
    column's largest-magnitude entry made positive, stored as fp32 [K][K]
    with column j = component j."""
    c = calib.astype(np.float64)
    c = c - c.mean(axis=0, keepdims=True)
    cov = c.T @ c / max(1, c.shape[0] - 1)
    evals, evecs = np.linalg.eigh(cov)
    order = np.lexsort((np.arange(evals.size), -evals))
    V = evecs[:, order]
    idx = np.argmax(np.abs(V), axis=0)
    sgn = np.sign(V[idx, np.arange(V.shape[1])])
    sgn[sgn == 0] = 1.0
    return np.ascontiguousarray((V * sgn).astype(np.float32))


def random_rpbh(K: int, seed: int):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    sign = np.where(g.integers(0, 2, size=K) == 1, 1, -1).astype(np.int8)
    perm = g.permutation(K).astype(np.int32)
    return sign, perm


# ---------------------------------------------------------------------------
# TR-DQ's runtime rotation, built from a calibration sample (harness only:
# the library takes the smoothing vector, the two block rotations and the
# permutation as inputs, like the dense path's PCA basis)
# ---------------------------------------------------------------------------

def smoothing_multiplier(calib: np.ndarray, W: np.ndarray, alpha: float = 0.5) -> np.ndarray:
    """Per-channel multiplier m = 1 / Delta of the SmoothQuant-style migration
    ("TR-DQ" Eq.(4)-(5)): Delta_j = max|X_j|^alpha / max|W_j|^(1 - alpha), the
    activations divided by Delta and the weights multiplied by it.  W is
    [N][K], so W_j is column j.  fp64, stored fp32."""
    ax = np.max(np.abs(calib.astype(np.float64)), axis=0)
    aw = np.max(np.abs(W.astype(np.float64)), axis=0)
    ax = np.where(ax > 0, ax, 1.0)
    aw = np.where(aw > 0, aw, 1.0)
    delta = ax ** alpha / aw ** (1.0 - alpha)
    return (1.0 / delta).astype(np.float32)


def _uniform_first_row_orthogonal(b: int, g: np.random.Generator) -> np.ndarray:
    """A random b x b orthogonal matrix whose first row is uniform (every
    entry 1 / sqrt(b)), fp64: QR of a Gaussian matrix whose first column is
    all ones, transposed."""
    A = g.standard_normal((b, b))
    A[:, 0] = 1.0
    Q, Rr = np.linalg.qr(A)
    Q = Q * np.sign(np.diag(Rr))[None, :]
    return Q.T


def greedy_block_rotation(Xb: np.ndarray, g: np.random.Generator, steps: int = 4) -> np.ndarray:
    """One block of TR-DQ's rotation ("TR-DQ" Eq.(6)-(7)): R^k = C1 Q C2,
    where C1 swaps column 0 with the column holding the largest |value| of
    the current activations, Q is a random orthogonal matrix with a uniform
    first row, and C2 swaps the two columns back; R = R^1 ... R^n with n the
    step count that minimizes the largest |value|.  fp64."""
    b = Xb.shape[1]
    R = np.eye(b)
    cur = Xb.astype(np.float64)
    best, best_R = np.max(np.abs(cur)), R.copy()
    for _ in range(steps):
        col = int(np.argmax(np.max(np.abs(cur), axis=0)))
        C = np.eye(b)
        C[[0, col]] = C[[col, 0]]
        Rk = C @ _uniform_first_row_orthogonal(b, g) @ C
        R = R @ Rk
        cur = cur @ Rk
        m = np.max(np.abs(cur))
        if m < best:
            best, best_R = m, R.copy()
    return best_R


def zigzag_permutation(chan_max: np.ndarray, b: int) -> np.ndarray:
    """TR-DQ's zigzag permutation (section 3.2): channels ranked by
    descending largest |activation| are dealt to blocks 0, 1, ..., nb - 1,
    then nb - 1, ..., 0, and so on, each block filling its slots in arrival
    order.  Returned as a gather: p[j] = z[perm[j]]."""
    K = chan_max.size
    nb = K // b
    order = np.lexsort((np.arange(K), -chan_max.astype(np.float64)))
    fill = np.zeros(nb, np.int64)
    perm = np.zeros(K, np.int32)
    for rank, ch in enumerate(order):
        lap, pos = divmod(rank, nb)
        blk = pos if lap % 2 == 0 else nb - 1 - pos
        perm[blk * b + fill[blk]] = ch
        fill[blk] += 1
    return perm


def trdq_rotation(calib: np.ndarray, W: np.ndarray, b: int, g: np.random.Generator) -> dict:
    """Smoothing multiplier m [K], block rotations R1, R2 [K/b][b][b] (fp32)
    and the zigzag permutation [K] for one layer, from a calibration sample
    [Tc][K] (fp32): m from Eq.(5); R1 block by block on the smoothed sample;
    the zigzag order from the channel maxima after R1; R2 block by block on
    the permuted sample."""
    K = calib.shape[1]
    nb = K // b
    m = smoothing_multiplier(calib, W)
    y = calib.astype(np.float64) * m.astype(np.float64)[None, :]
    R1 = np.stack([greedy_block_rotation(y[:, c * b:(c + 1) * b], g) for c in range(nb)])
    R1 = R1.astype(np.float32)
    z = np.concatenate([y[:, c * b:(c + 1) * b] @ R1[c].astype(np.float64) for c in range(nb)], axis=1)
    perm = zigzag_permutation(np.max(np.abs(z), axis=0), b)
    p = z[:, perm]
    R2 = np.stack([greedy_block_rotation(p[:, c * b:(c + 1) * b], g) for c in range(nb)])
    return {"m": m, "R1": R1, "perm": perm, "R2": R2.astype(np.float32), "R": None}


def make_timestep_inputs(w: Workload, groups: int) -> list:
    """One layer seen at `groups` groups of denoising steps ("TR-DQ" Eq.(10)):
    the weights are the layer's, fixed; the activations -- their outlier
    channels and calibration statistics -- and so the rotation differ per
    group.  Returns one make_inputs dict per group, all with the same W."""
    W = make_inputs(w)["W"]
    return [make_inputs(w, seed_offset=50 + g, W=W) for g in range(groups)]

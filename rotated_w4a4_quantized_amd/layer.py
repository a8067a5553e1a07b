"""Device-side convenience for one layer instance: the rotation and packed
weights uploaded once, the activation/code/scale/output buffers allocated
once, and the two runtime calls of the C ABI.  Marshalling only -- every
computation runs in librq.
"""
from __future__ import annotations

import numpy as np

from . import rq


def torch_mod():
    import torch
    return torch


def device_x(inp, device):
    torch = torch_mod()
    X = inp["X"]
    if X.dtype == np.uint16:
        return torch.from_numpy(X.view(np.int16)).to(device)
    return torch.from_numpy(X).to(device)


def rotation_for(w, inp) -> rq.Rotation:
    if w.rot == "rpbh":
        return rq.Rotation.rpbh(inp["sign"], inp["perm"], w.block)
    if w.rot == "trdq":
        return rq.Rotation.trdq(inp["m"], inp["R1"], inp["perm"], inp["R2"], w.block)
    return rq.Rotation.dense(inp["R"], w.r)


def quant_for(w) -> rq.Quant:
    if w.quant in ("int4", "int4_asym"):
        return rq.Quant.integer(w.a_bits, w.w_bits, asym=w.quant == "int4_asym")
    if w.quant == "mxfp4":
        return rq.Quant.mxfp4()
    return rq.Quant.lloydmax(rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(1 << w.w_bits))


def mma_capable(w) -> bool:
    """Whether rq_rotate_quant can hand this workload's GEMM its codes in the
    matrix-core layout: 4-bit integer codes under RPBH or DENSE, 6- and 8-bit
    integer codes under RPBH or TR-DQ, and MXFP4 and Lloyd-Max codes (as their
    bf16 levels) under RPBH."""
    intq = w.quant in ("int4", "int4_asym")
    int4, int8 = intq and w.a_bits == 4, intq and w.a_bits in (6, 8)
    return ((w.rot in ("rpbh", "dense") and int4) or (w.rot in ("rpbh", "trdq") and int8) or
            (w.rot == "rpbh" and w.quant in ("mxfp4", "lloydmax")))


class QuantLinear:
    """Device state of one layer instance (w: a datagen.Workload, inp: its
    inputs): rotation, packed weights, buffers.

    codes: which activation-code layouts rq_rotate_quant writes and
    rq_w4a4_linear reads -- "canonical" (nibbles or bytes), "mma" (the GEMM's
    matrix-core layout only; see mma_capable)
    or "both" (writes both, the GEMM reads the MMA copy).  MXFP4 layers
    always write the MMA copy, which their GEMM reads."""

    def __init__(self, w, inp: dict, device="cuda", y_dtype=None, codes="canonical"):
        torch = torch_mod()
        self.w, self.inp, self.device = w, inp, device
        self.rot = rotation_for(w, inp)
        self.q = quant_for(w)
        self.packed = rq.pack_weights(self.rot, self.q, inp["W"])
        self.dw = self.packed.to_device(device)
        self.drot = self.rot.to_device(device)
        self.X = device_x(inp, device)
        T = w.T
        if codes not in ("canonical", "mma", "both") or (codes != "canonical" and not mma_capable(w)):
            raise ValueError(f"codes={codes!r} is not available for {w.name}")
        if w.quant == "mxfp4" and codes == "canonical":
            codes = "both"
        ncode, nscale, nmma = rq.activation_bytes(self.rot, self.q, T)
        self.codes = (torch.empty((T, ncode // max(T, 1)), dtype=torch.uint8, device=device)
                      if codes != "mma" else None)
        self.codes_mma = None
        if codes != "canonical":
            self.codes_mma = torch.empty((max(nmma, 16),), dtype=torch.uint8, device=device)
        if w.quant == "mxfp4":   # E8M0 codes [T][K/32]
            self.scale = (torch.empty((T, w.K // 32), dtype=torch.uint8, device=device)
                          if codes != "mma" else None)
        else:                    # fp32 s [T] (and z [T] for asymmetric codes)
            self.scale = torch.empty((self.q.scale_rows * T,), dtype=torch.float32, device=device)
        self.top = torch.empty((T, w.r), dtype=torch.int16, device=device) if w.r else None
        wsb = rq.rotate_quant_workspace_bytes(self.rot, self.q, T)
        self.ws = torch.empty((max(wsb, 16) // 4,), dtype=torch.float32, device=device) if wsb else None
        ydt = {"f32": torch.float32, "bf16": torch.bfloat16}[y_dtype or w.ydtype]
        self.Y = torch.empty((T, w.N), dtype=ydt, device=device)

    def rotate_quant(self, stream=None):
        rq.rotate_quant(self.drot, self.q, self.X, self.codes, self.scale, self.top, self.ws,
                        stream=stream, codes_mma=self.codes_mma)

    def linear(self, Y=None, stream=None, use_mma=True, engine="auto"):
        rq.w4a4_linear(self.dw, self.codes, self.scale, self.Y if Y is None else Y, top=self.top,
                       stream=stream, T=self.w.T,
                       codes_mma=self.codes_mma if use_mma else None, engine=engine)

    def run(self):
        self.rotate_quant()
        self.linear()

    def raw_acc(self, use_mma=True, engine="auto"):
        torch = torch_mod()
        acc = torch.empty((self.w.T, self.w.N), dtype=torch.int32, device=self.device)
        self.linear(acc, use_mma=use_mma, engine=engine)
        return acc



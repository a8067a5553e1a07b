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
    return rq.Rotation.dense(inp["R"], w.r)


def quant_for(w) -> rq.Quant:
    if w.quant == "int4":
        return rq.Quant.int4()
    if w.quant == "int4_asym":
        return rq.Quant.int4_asym()
    return rq.Quant.lloydmax(rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(1 << w.w_bits))


class QuantLinear:
    """Device state of one layer instance (w: a datagen.Workload, inp: its
    inputs): rotation, packed weights, buffers.

    codes: which activation-code layouts rq_rotate_quant writes and
    rq_w4a4_linear reads -- "canonical" (nibbles), "mma" (the GEMM's FP6
    fragment layout only; RPBH INT4 layers) or "both" (writes both, the GEMM
    reads the MMA copy)."""

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
        ncode = (w.Kq // 2)
        mma_ok = w.rot == "rpbh" and w.quant in ("int4", "int4_asym")
        if codes not in ("canonical", "mma", "both") or (codes != "canonical" and not mma_ok):
            raise ValueError(f"codes={codes!r} is not available for {w.name}")
        self.codes = (torch.empty((T, ncode), dtype=torch.uint8, device=device)
                      if codes != "mma" else None)
        self.codes_mma = None
        if codes != "canonical":
            nb = rq.codes_mma_bytes(self.rot, T)
            self.codes_mma = torch.empty((max(nb, 16),), dtype=torch.uint8, device=device)
        # INT4_ASYM: s [T] then the zero points [T]
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



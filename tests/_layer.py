"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and compare them.

Comparison rules (the oracle is the fp64 value of the same codes/scales):
* codes, packed nibbles, scales, sigma, int32 accumulators: bit-exact;
* fp32 output: max |Y - Yhat| / max(|Yhat|, 1e-2 * rms(Yhat)) <= 1e-3;
* bf16 output: within 1 bf16 ulp of the nearest-even rounding of Yhat, or
  within 1e-5 * rms(Yhat) for entries that are tiny next to the rest.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as orc
from rotated_w4a4_quantized_amd import datagen, rq  # noqa: F401
from rotated_w4a4_quantized_amd.layer import (QuantLinear as GpuLayer, device_x,  # noqa: F401
                                              quant_for, rotation_for, torch_mod)

REL_TOL = 1e-3


def oracle_act(w, inp, rows=None):
    rows = np.arange(w.T) if rows is None else np.asarray(rows)
    xd = 0 if w.xdtype == "f32" else 1
    if w.rot == "rpbh":
        if w.quant == "int4":
            return orc.act_rows(inp["X"], xd, w.K, rows, rot_kind=0, b=w.block, sign=inp["sign"],
                                perm=inp["perm"])
        return orc.act_rows(inp["X"], xd, w.K, rows, rot_kind=0, b=w.block, sign=inp["sign"],
                            perm=inp["perm"], q_kind=1, levels=orc.codebook_bf16(16))
    return orc.act_rows(inp["X"], xd, w.K, rows, rot_kind=1, R=inp["R"], r=w.r)


def oracle_weights(w, inp):
    if w.rot == "rpbh":
        if w.quant == "int4":
            return orc.weight_rows(inp["W"], rot_kind=0, b=w.block, sign=inp["sign"], perm=inp["perm"])
        return orc.weight_rows(inp["W"], rot_kind=0, b=w.block, sign=inp["sign"], perm=inp["perm"],
                               q_kind=1, levels=orc.codebook_bf16(1 << w.w_bits))
    return orc.weight_rows(inp["W"], rot_kind=1, R=inp["R"])


def oracle_yhat_pairs(w, act, wts, ta, nw, act_rows=None):
    """fp64 Yhat at (ta[p], nw[p]); act holds the oracle activation of rows
    act_rows (default: all rows, act index == token)."""
    ia = ta if act_rows is None else np.searchsorted(act_rows, ta)
    if w.quant == "lloydmax":
        dot = orc.codebook_dot_pairs(act["codes"], wts["codes"], w.K, orc.codebook_bf16(16),
                                     orc.codebook_bf16(1 << w.w_bits), ia, nw)
        return orc.yhat_codebook(act["scale"][ia], wts["scale"][nw], dot, w.block)
    acc = orc.int_gemm_pairs(act["codes"], w.Kq, wts["codes"], w.K, ia, nw, koff=w.r)
    lr = None
    if w.r:
        lr = orc.lowrank_pairs(act["top"], w.r, wts["codes"], w.K, ia, nw)
    return orc.yhat_int4(act["scale"][ia], wts["scale"][nw], acc, w.b_eff, lr=lr)


def rel_err(y, yhat):
    y = np.asarray(y, np.float64)
    yhat = np.asarray(yhat, np.float64)
    rms = np.sqrt(np.mean(yhat ** 2)) if yhat.size else 0.0
    den = np.maximum(np.abs(yhat), 1e-2 * rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y - yhat) / den)) if y.size else 0.0


def _ordered(bits16):
    b = bits16.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_check(y_bits, yhat):
    """(max bf16 ulp distance, pass) for a bf16 output against fp64 Yhat."""
    yhat = np.asarray(yhat, np.float64)
    ref = datagen.f32_to_bf16_bits(yhat.astype(np.float32))
    # fp32 rounding of yhat first can only matter at exact bf16 ties; allow it
    dist = np.abs(_ordered(np.asarray(y_bits, np.uint16)) - _ordered(ref))
    rms = np.sqrt(np.mean(yhat ** 2)) if yhat.size else 0.0
    tiny = np.abs(datagen.bf16_bits_to_f32(np.asarray(y_bits, np.uint16)).astype(np.float64) - yhat) \
        <= 1e-5 * rms
    ok = (dist <= 1) | tiny
    return int(dist.max()) if dist.size else 0, bool(ok.all())


def to_np_bf16_bits(t):
    torch = torch_mod()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)

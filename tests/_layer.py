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


def _rot_args(w, inp):
    if w.rot == "rpbh":
        return dict(rot_kind=0, b=w.block, sign=inp["sign"], perm=inp["perm"])
    if w.rot == "trdq":
        return dict(rot_kind=2, b=w.block, m=inp["m"], R=inp["R1"], perm=inp["perm"], R2=inp["R2"])
    return dict(rot_kind=1, R=inp["R"])


def oracle_act(w, inp, rows=None):
    rows = np.arange(w.T) if rows is None else np.asarray(rows)
    xd = 0 if w.xdtype == "f32" else 1
    ra = _rot_args(w, inp)
    if w.quant == "int4":
        return orc.act_rows(inp["X"], xd, w.K, rows, r=w.r, a_bits=w.a_bits, **ra)
    if w.quant == "int4_asym":
        return orc.act_rows(inp["X"], xd, w.K, rows, q_kind=2, a_bits=w.a_bits, **ra)
    if w.quant == "mxfp4":
        return orc.act_rows(inp["X"], xd, w.K, rows, q_kind=3, **ra)
    return orc.act_rows(inp["X"], xd, w.K, rows, q_kind=1, levels=orc.codebook_bf16(16), **ra)


def oracle_weights(w, inp):
    ra = _rot_args(w, inp)
    if w.quant in ("int4", "int4_asym"):   # integer weights are symmetric either way
        return orc.weight_rows(inp["W"], w_bits=w.w_bits, **ra)
    if w.quant == "mxfp4":
        return orc.weight_rows(inp["W"], q_kind=3, **ra)
    return orc.weight_rows(inp["W"], q_kind=1, levels=orc.codebook_bf16(1 << w.w_bits), **ra)


def _acc_pairs(w, act, wts, ia, nw):
    """Exact integer accumulators sum_k code_a code_w at pairs (codes as stored:
    asymmetric activation codes unsigned)."""
    return orc.gemm_codes_pairs(act["codes"], w.a_bits, w.quant == "int4", w.Kq, wts["codes"],
                                w.w_bits, w.K, ia, nw, koff=w.r)


def oracle_yhat_pairs(w, act, wts, ta, nw, act_rows=None):
    """fp64 Yhat at (ta[p], nw[p]); act holds the oracle activation of rows
    act_rows (default: all rows, act index == token)."""
    ia = ta if act_rows is None else np.searchsorted(act_rows, ta)
    if w.quant == "lloydmax":
        dot = orc.codebook_dot_pairs(act["codes"], wts["codes"], w.K, orc.codebook_bf16(16),
                                     orc.codebook_bf16(1 << w.w_bits), ia, nw)
        return orc.yhat_codebook(act["scale"][ia], wts["scale"][nw], dot, w.block)
    if w.quant == "mxfp4":
        dot = orc.mx_dot_pairs(act["codes"], act["mx_scales"], wts["codes"], wts["mx_scales"], w.K,
                               ia, nw)
        return orc.yhat_mx(dot, w.b_eff)
    if w.quant == "int4_asym":
        acc_u = _acc_pairs(w, act, wts, ia, nw)
        wsum = wts["q"].astype(np.int64).sum(axis=1)
        return orc.yhat_int4_asym(act["scale"][ia], act["zero"][ia], wts["scale"][nw], acc_u,
                                  wsum[nw], w.b_eff)
    acc = _acc_pairs(w, act, wts, ia, nw)
    lr = None
    if w.r:
        lr = orc.lowrank_pairs(act["top"], w.r, wts["codes"], w.K, ia, nw)
    return orc.yhat_int4(act["scale"][ia], wts["scale"][nw], acc, w.b_eff, lr=lr)


def oracle_raw_acc(w, act, wts):
    """Exact int64 accumulators [T][N] that RQ_I32 output returns:
    sum_k q_a q_w, with q_a = u - z for asymmetric activations."""
    T, N = act["codes"].shape[0], wts["codes"].shape[0]
    ta, nw = np.meshgrid(np.arange(T), np.arange(N), indexing="ij")
    acc = _acc_pairs(w, act, wts, ta.ravel(), nw.ravel()).reshape(T, N)
    if w.quant == "int4_asym":
        wsum = wts["q"].astype(np.int64).sum(axis=1)
        return acc - act["zero"].astype(np.int64)[:, None] * wsum[None, :]
    return acc


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


FP6_ORDER = np.array([0, 1, 3, 4, 6, 7, 9, 10, 12, 13, 15, 8, 2, 11, 5, 14])


def decode_codes_mma(buf, T, Kq):
    """INT4 codes [T][Kq] (int16) from rq_rotate_quant's codes_mma output, read
    as rq.h documents it: [token tile of 32][stage of 128 coordinates]
    [piece 0..2][lane 0..63][16 bytes]; token t of a tile owns lanes t and
    t + 32 (half h); its dwords f[0..11] of half h are dword d % 4 of its lane
    in piece d // 4; k-step ks is f[6 ks .. 6 ks + 5], 6-bit field e holding
    (q + 8) for coordinate 128 s + 64 ks + 32 h + order[e % 16] + 16 (e // 16).
    Also returns whether every field of a real coordinate (token below T,
    coordinate below Kq) had its two top bits clear."""
    S = -(-Kq // 128)
    NT = -(-T // 32)
    buf = np.ascontiguousarray(buf, np.uint8)[:NT * S * 3 * 1024]
    blk = buf.view(np.uint32).reshape(NT, S, 3, 2, 32, 4)        # [tile][s][piece][h][t][dword]
    f = blk.transpose(0, 4, 1, 3, 2, 5).reshape(NT * 32, S, 2, 12).astype(np.uint64)  # [tok][s][h][f]
    Tp = NT * 32
    q = np.zeros((Tp, S, 2, 2, 32), np.int16)   # [tok][s][ks][h][field]
    top = np.zeros((Tp, S, 2, 2, 32), bool)
    for ks in range(2):
        d = f[:, :, :, 6 * ks:6 * ks + 6]
        for e in range(32):
            w, off = divmod(6 * e, 32)
            v = d[..., w] >> np.uint64(off)
            if off > 26:
                v = v | (d[..., w + 1] << np.uint64(32 - off))
            v = (v & np.uint64(63)).astype(np.int16)
            top[:, :, ks, :, e] = (v & 48) != 0
            q[:, :, ks, :, e] = (v & 15) - 8
    k_of = np.zeros((2, 2, 32), np.int64)
    for ks in range(2):
        for h in range(2):
            for e in range(32):
                k_of[ks, h, e] = 64 * ks + 32 * h + FP6_ORDER[e % 16] + 16 * (e // 16)
    out = np.zeros((Tp, S * 128), np.int16)
    tops = np.zeros((Tp, S * 128), bool)
    for s_ in range(S):
        out[:, 128 * s_ + k_of.reshape(-1)] = q[:, s_].reshape(Tp, -1)
        tops[:, 128 * s_ + k_of.reshape(-1)] = top[:, s_].reshape(Tp, -1)
    # only real tokens and coordinates are ever written
    return out[:T, :Kq], not tops[:T, :Kq].any()


def unpack_nibbles(codes):
    """Canonical unsigned nibbles [T][K/2] -> indices [T][K] (low nibble first)."""
    codes = np.asarray(codes, np.uint8)
    return np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[0], -1).astype(np.int64)


def unpack_codes(codes):
    """Canonical nibbles [T][Kq/2] -> INT4 codes [T][Kq]."""
    codes = np.asarray(codes, np.uint8)
    lo = (codes & 15).astype(np.int16)
    hi = (codes >> 4).astype(np.int16)
    q = np.stack([lo, hi], -1).reshape(codes.shape[0], -1)
    return np.where(q >= 8, q - 16, q)


def decode_cb_mma(buf, T, K):
    """bf16 bits [T][K] from the Lloyd-Max codes_mma output, read as rq.h
    documents it: [32-token tile][16-coordinate k-step][lane 0..63][8 bf16];
    coordinate 16 ks + 8 h + e of token t is element e of lane t % 32 + 32 h."""
    tiles = -(-T // 32)
    v = np.ascontiguousarray(buf, np.uint8)[:tiles * (K // 16) * 1024].view(np.uint16)
    v = v.reshape(tiles, K // 16, 2, 32, 8)            # [tile][ks][h][t32][e]
    v = v.transpose(0, 3, 1, 2, 4).reshape(tiles * 32, K)
    return v[:T]


def decode_i8_mma(buf, T, K):
    """uint8 codes [T][K] from the 8-bit codes_mma output, read as rq.h
    documents it: [32-token tile][32-coordinate k-step][lane 0..63][16 bytes];
    coordinate 32 kb + 16 h + e of token t is byte e of lane t % 32 + 32 h."""
    tiles = -(-T // 32)
    v = np.ascontiguousarray(buf, np.uint8)[:tiles * 32 * K]
    v = v.reshape(tiles, K // 32, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(tiles * 32, K)
    return v[:T]

"""C-ABI checks that need no GPU: librq loads, exports every symbol that
include/rq.h declares, rejects bad arguments before touching the GPU, and its
host-side weight pack (fold in fp64 + quantize + pack) and Lloyd-Max codebook
match the oracle bit for bit.

Weight pack: "DiRotQ" abstract (inverse rotation fused into the weights
offline), "OrbitQuant" abstract (rotation absorbed into the weight rows,
same normalized-basis quantizer), "TR-DQ" Eq.(9) and section 3.1
(per-output-channel weight quantization).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import oracle as orc
from rotated_w4a4_quantized_amd import datagen, rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "rq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = rq.load()
    declared = header_functions()
    assert declared, "no declarations parsed"
    assert sorted(rq.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name
    assert rq.version() >= 100


def test_struct_sizes_match_header(tmp_path):
    """The binding's ctypes structs lay out exactly as the C compiler lays out
    include/rq.h's (sizes and every field offset, from a compiled probe)."""
    assert ctypes.sizeof(rq.c_weight_header) == 256
    structs = {"rq_rotation": rq.c_rotation, "rq_quant": rq.c_quant,
               "rq_weight_header": rq.c_weight_header, "rq_set_header": rq.c_set_header}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "rq.h"', 'int main(void) {']
    for cname, ct in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in ct._fields_:
            lines.append(f'printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    import subprocess
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)]).decode().splitlines())
    for cname, ct in structs.items():
        assert int(got[cname]) == ctypes.sizeof(ct), cname
        for fname, _ in ct._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(ct, fname).offset, (cname, fname)


def _status(fn, *args):
    return fn(*args)


def _rq_call(rot: rq.c_rotation, q: rq.c_quant, X=1 << 20, xdt=rq.RQ_BF16, T=4, codes=1 << 20,
             scale=1 << 20, top=None, ws=None, wsb=0, mma=None):
    L = rq.load()
    return L.rq_rotate_quant(ctypes.byref(rot), ctypes.byref(q), ctypes.c_void_p(X), xdt, T,
                             None if codes is None else ctypes.c_void_p(codes),
                             ctypes.c_void_p(scale),
                             None if top is None else ctypes.c_void_p(top),
                             None if mma is None else ctypes.c_void_p(mma),
                             None if ws is None else ctypes.c_void_p(ws), wsb, None)


def _rpbh(K=256, b=64):
    # pointer values only: every call below is rejected (or returns for T == 0)
    # before any pointer is dereferenced or any HIP call is made
    return rq.c_rotation(rq.RQ_ROT_RPBH, K, b, 0, 1 << 20, 1 << 21, None, None, None)


def test_rotate_quant_validation_errors():
    q = rq.Quant.int4().c()
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 100, 4, 0, 1 << 20, 1 << 21, None), q) == -2
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 256, 48, 0, 1 << 20, 1 << 21, None), q) == -2
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 256, 512, 0, 1 << 20, 1 << 21, None), q) == -2
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 32768, 64, 0, 1 << 20, 1 << 21, None), q) == -2
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 256, 64, 0, None, 1 << 21, None), q) == -1
    assert _rq_call(rq.c_rotation(7, 256, 64, 0, 1 << 20, 1 << 21, None), q) == -6
    assert _rq_call(_rpbh(), q, xdt=5) == -3
    assert _rq_call(_rpbh(), q, T=-1) == -2
    assert _rq_call(_rpbh(), q, X=0) == -1
    assert _rq_call(_rpbh(), q, codes=(1 << 20) + 8) == -4
    assert "aligned" in rq.load().rq_last_error().decode()
    # the kernel reads sign and perm as 16-byte vectors
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 256, 64, 0, (1 << 20) + 4, 1 << 21, None), q) == -4
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 256, 64, 0, 1 << 20, (1 << 21) + 4, None), q) == -4
    assert "sign and perm" in rq.load().rq_last_error().decode()
    # dense: r must be a multiple of 32 below K; workspace required; top required
    dense = rq.c_rotation(rq.RQ_ROT_DENSE, 256, 0, 16, None, None, 1 << 22)
    assert _rq_call(dense, q) == -2
    dense = rq.c_rotation(rq.RQ_ROT_DENSE, 256, 0, 32, None, None, 1 << 22)
    assert _rq_call(dense, q, top=None) == -1
    assert _rq_call(dense, q, top=1 << 23, ws=None) == -2
    # a bad quantizer
    bad = rq.Quant(kind=rq.RQ_Q_INT4_SYM, a_bits=4, w_bits=2).c()
    assert _rq_call(_rpbh(), bad) == -6
    lm = rq.Quant.lloydmax(np.arange(16, dtype=np.float32)[::-1], np.arange(4, dtype=np.float32)).c()
    assert _rq_call(_rpbh(), lm) == -2      # levels not ascending
    lm = rq.Quant.lloydmax(np.linspace(-2, 2, 16).astype(np.float32), np.arange(4, dtype=np.float32)).c()
    assert _rq_call(_rpbh(), lm) == -2      # levels not bf16-representable
    # the MMA-layout copy of the codes: INT4 under RPBH or DENSE, aligned, one
    # of the two outputs
    assert _rq_call(_rpbh(), q, codes=None, mma=None) == -1
    assert _rq_call(_rpbh(), q, codes=None, mma=(1 << 22) + 8) == -4
    dense = rq.c_rotation(rq.RQ_ROT_DENSE, 256, 0, 32, None, None, 1 << 22)
    assert _rq_call(dense, q, top=1 << 23, ws=1 << 24, wsb=1 << 30, codes=None, mma=None) == -1
    assert _rq_call(dense, q, top=1 << 23, ws=1 << 24, wsb=1 << 30, codes=None,
                    mma=(1 << 22) + 8) == -4
    lm = rq.Quant.lloydmax(rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(4)).c()
    assert _rq_call(_rpbh(), lm, codes=None, mma=None) == -1
    assert _rq_call(_rpbh(), lm, codes=None, mma=(1 << 22) + 8) == -4
    td = rq.c_rotation(rq.RQ_ROT_TRDQ, 256, 64, 0, None, 1 << 21, 1 << 22, 1 << 23, 1 << 24)
    assert _rq_call(td, q, mma=1 << 22) == -6


def test_codes_mma_bytes():
    def nbytes(rot, T):
        n = ctypes.c_size_t(0)
        assert rq.load().rq_codes_mma_bytes(ctypes.byref(rot), T, ctypes.byref(n)) == 0
        return n.value
    # 3 KB per 32 tokens per 128 quantized coordinates
    assert nbytes(_rpbh(256, 64), 4) == 1 * 2 * 3072
    assert nbytes(_rpbh(96, 32), 33) == 2 * 1 * 3072
    assert nbytes(_rpbh(12288, 512), 64) == 2 * 96 * 3072
    assert nbytes(rq.c_rotation(rq.RQ_ROT_DENSE, 1152, 0, 32, None, None, 1 << 22), 5) == 1 * 9 * 3072
    assert nbytes(_rpbh(256, 64), 0) == 0
    n = ctypes.c_size_t(0)
    assert rq.load().rq_codes_mma_bytes(ctypes.byref(_rpbh(100, 4)), 1, ctypes.byref(n)) == -2


def test_empty_token_batch_is_a_no_op():
    # T == 0 returns before any pointer is read or any kernel launched
    assert _rq_call(_rpbh(), rq.Quant.int4().c(), T=0, X=0, codes=0, scale=0) == 0
    hdr = _small_header()
    L = rq.load()
    assert L.rq_w4a4_linear(ctypes.byref(hdr), None, None, None, None, None, 0, None, None,
                            rq.RQ_F32, None) == 0


def _small_header():
    w = datagen.WORKLOADS["tiny"].with_shape(T=8, K=256, N=64, block=64)
    inp = datagen.make_inputs(w)
    pw = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 64), rq.Quant.int4(), inp["W"])
    return pw.header


def test_linear_validation_errors():
    L = rq.load()
    hdr = _small_header()
    def args(h, ydt=rq.RQ_F32, Y=1 << 24, codes=1 << 21, mma=None):
        return (ctypes.byref(h), ctypes.c_void_p(1 << 20),
                None if codes is None else ctypes.c_void_p(codes), ctypes.c_void_p(1 << 22),
                None, None if mma is None else ctypes.c_void_p(mma), 4, None, ctypes.c_void_p(Y),
                ydt, None)
    bad = rq.c_weight_header.from_buffer_copy(bytes(hdr))
    bad.magic = 0
    assert L.rq_w4a4_linear(*args(bad)) == -5
    bad = rq.c_weight_header.from_buffer_copy(bytes(hdr))
    bad.version = 9
    assert L.rq_w4a4_linear(*args(bad)) == -5
    bad = rq.c_weight_header.from_buffer_copy(bytes(hdr))
    bad.row_bytes += 1
    assert L.rq_w4a4_linear(*args(bad)) == -5
    assert L.rq_w4a4_linear(*args(hdr, ydt=9)) == -3
    assert L.rq_w4a4_linear(*args(hdr, Y=(1 << 24) + 4)) == -4
    assert L.rq_w4a4_linear(None, None, None, None, None, None, 1, None, None, 0, None) == -1
    assert L.rq_w4a4_linear(*args(hdr, codes=None)) == -1
    assert L.rq_w4a4_linear(*args(hdr, codes=None, mma=(1 << 23) + 4)) == -4
    # 8-bit activations read their int8 fragment copy and the codebook format
    # its bf16 level fragments, both 16-byte aligned
    w = datagen.WORKLOADS["flux_up_w4a8"].with_shape(T=4, K=256, N=40, block=64)
    inp = datagen.make_inputs(w)
    h8 = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 64), rq.Quant.integer(8, 4),
                         inp["W"]).header
    assert L.rq_w4a4_linear(*args(h8, mma=(1 << 23) + 4)) == -4
    w = datagen.WORKLOADS["video"].with_shape(T=4, K=256, N=40)
    inp = datagen.make_inputs(w)
    lh = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 256),
                         rq.Quant.lloydmax(rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(4)),
                         inp["W"]).header
    assert L.rq_w4a4_linear(*args(lh, mma=(1 << 23) + 4)) == -4
    assert L.rq_w4a4_linear(*args(lh, codes=None)) == -1


def test_engine_validation_errors():
    """rq_w4a4_linear_engine rejects what its engine cannot run, before any
    GPU call."""
    L = rq.load()
    hdr = _small_header()

    def call(h, engine, codes=1 << 21, mma=None):
        return L.rq_w4a4_linear_engine(ctypes.byref(h), ctypes.c_void_p(1 << 20),
                                       None if codes is None else ctypes.c_void_p(codes),
                                       ctypes.c_void_p(1 << 22), None,
                                       None if mma is None else ctypes.c_void_p(mma), 4, None,
                                       ctypes.c_void_p(1 << 24), rq.RQ_F32, engine, None)
    assert call(hdr, 7) == -6                                  # unknown engine
    assert call(hdr, rq.RQ_ENGINE_INT8, mma=1 << 23) == -6     # int8 reads canonical codes
    assert call(hdr, rq.RQ_ENGINE_INT8, codes=None) == -1
    w = datagen.WORKLOADS["flux_up_asym"].with_shape(T=4, K=256, N=40, block=64)
    inp = datagen.make_inputs(w)
    ah = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 64), rq.Quant.int4_asym(),
                         inp["W"]).header
    assert call(ah, rq.RQ_ENGINE_INT8) == -6                   # int8 engine: INT4_SYM only
    w = datagen.WORKLOADS["video"].with_shape(T=4, K=256, N=40)
    inp = datagen.make_inputs(w)
    lh = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 256),
                         rq.Quant.lloydmax(rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(4)),
                         inp["W"]).header
    assert call(lh, rq.RQ_ENGINE_FP6) == -6                    # codebook: AUTO only
    assert call(hdr, rq.RQ_ENGINE_INT8, codes=None) == -1
    # T == 0 is a no-op for every engine
    for e in (rq.RQ_ENGINE_AUTO, rq.RQ_ENGINE_FP6, rq.RQ_ENGINE_INT8):
        assert L.rq_w4a4_linear_engine(ctypes.byref(hdr), None, None, None, None, None, 0, None,
                                       None, rq.RQ_F32, e, None) == 0


def test_lloydmax_codebook_matches_oracle():
    for L in (2, 4, 8, 16):
        assert np.array_equal(rq.lloydmax_gaussian(L), orc.codebook_bf16(L)), L
    with pytest.raises(rq.RQError):
        rq.lloydmax_gaussian(5)


def _oracle_weights(w, inp, q_kind=0, levels=None):
    if w.rot == "rpbh":
        return orc.weight_rows(inp["W"], rot_kind=0, b=w.block, sign=inp["sign"], perm=inp["perm"],
                               q_kind=q_kind, levels=levels)
    return orc.weight_rows(inp["W"], rot_kind=1, R=inp["R"], q_kind=q_kind, levels=levels)


@pytest.mark.parametrize("name,shape", [("tiny", dict(N=96)),
                                        ("flux_up", dict(K=1024, N=70, block=256)),
                                        ("flux_down", dict(K=2048, N=33, block=512)),
                                        ("pixart", dict(K=256, N=40)),
                                        ("tiny", dict(K=64, N=10, block=2))])
def test_pack_int4_matches_oracle(name, shape):
    w = datagen.WORKLOADS[name].with_shape(T=4, **shape)
    inp = datagen.make_inputs(w)
    rot = (rq.Rotation.rpbh(inp["sign"], inp["perm"], w.block) if w.rot == "rpbh"
           else rq.Rotation.dense(inp["R"], w.r))
    pw = rq.pack_weights(rot, rq.Quant.int4(), inp["W"])
    ref = _oracle_weights(w, inp)
    assert np.array_equal(pw.codes(), ref["codes"])
    assert np.array_equal(pw.scales().view(np.uint32), ref["scale"].view(np.uint32))
    h = pw.header
    assert (h.magic, h.K, h.N, h.r, h.b_div, h.row_bytes) == (
        rq.RQ_WEIGHT_MAGIC, w.K, w.N, w.r, w.b_eff, w.K // 2)


# E2M3 (OCP MX FP6): sign, 2 exponent bits with bias 1, 3 mantissa bits
def _e2m3_value(code):
    code = np.asarray(code, np.int64)
    sgn = np.where(code & 32, -1.0, 1.0)
    e, m = (code >> 3) & 3, code & 7
    mag = np.where(e == 0, m / 8.0, np.ldexp(1.0 + m / 8.0, (e - 1).astype(np.int32)))
    return sgn * mag


def _decode_fp6_fragments(tiles, N, Kq):
    """Rebuild q_w[n][k] (k over the quantized coordinates) from the GEMM's
    FP6 fragments as rq.h documents them: tile (nt, s), lane l -> row
    32 nt + l % 32, half h = l // 32; 48 bytes = [part][16], fragment ks at
    bytes 24 ks; field f at bits 6 f holds coordinate
    128 s + 64 ks + 32 h + order[f % 16] + 16 (f // 16), scaled by 2^3."""
    order = [0, 1, 3, 4, 6, 7, 9, 10, 12, 13, 15, 8, 2, 11, 5, 14]
    nt_, S = tiles.shape[:2]
    out = np.zeros((nt_ * 32, S * 128), np.int64)
    lane_bytes = tiles.transpose(0, 1, 3, 2, 4).reshape(nt_, S, 64, 48)
    for ks in range(2):
        frag = lane_bytes[..., 24 * ks:24 * ks + 24].astype(np.uint64)
        bits = np.zeros(frag.shape[:-1], dtype=object)
        for b in range(24):
            bits = bits + (frag[..., b].astype(object) << (8 * b))
        for f in range(32):
            code = np.vectorize(lambda v: (v >> (6 * f)) & 63, otypes=[np.int64])(bits)
            val = _e2m3_value(code) * 8
            assert np.all(val == np.round(val))
            k_in = order[f % 16] + 16 * (f // 16)
            for l in range(64):
                rows = 32 * np.arange(nt_) + l % 32
                ks_ = 128 * np.arange(S) + 64 * ks + 32 * (l // 32) + k_in
                out[np.ix_(rows, ks_)] = val[:, :, l].astype(np.int64)
    return out[:N, :Kq], out


def _unpack_nibbles(codes):
    lo = (codes & 15).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    q = np.stack([lo, hi], -1).reshape(codes.shape[0], -1)
    return np.where(q >= 8, q - 16, q)


@pytest.mark.parametrize("name,shape", [("tiny", dict(K=256, N=40, block=64)),
                                        ("pixart", dict(K=224, N=33)),
                                        ("flux_up", dict(K=160, N=70, block=32))])
def test_pack_int4_fp6_fragments(name, shape):
    w = datagen.WORKLOADS[name].with_shape(T=4, **shape)
    inp = datagen.make_inputs(w)
    rot = (rq.Rotation.rpbh(inp["sign"], inp["perm"], w.block) if w.rot == "rpbh"
           else rq.Rotation.dense(inp["R"], w.r))
    pw = rq.pack_weights(rot, rq.Quant.int4(), inp["W"])
    h = pw.header
    Kq = w.K - w.r
    assert h.mma_stages == -(-Kq // 128) and h.mma_ntiles == -(-w.N // 32)
    qw = _unpack_nibbles(_oracle_weights(w, inp)["codes"])[:, w.r:]
    got, padded = _decode_fp6_fragments(pw.mma_tiles(), w.N, Kq)
    assert np.array_equal(got, qw)
    assert not padded[w.N:].any() and not padded[:, Kq:].any()   # zero padding
    assert np.array_equal(pw.wsum(), qw.sum(axis=1))


def test_pack_bf16_weights_and_zero_rows():
    w = datagen.WORKLOADS["flux_up"].with_shape(T=4, K=512, N=16, block=128)
    inp = datagen.make_inputs(w)
    Wb = datagen.f32_to_bf16_bits(inp["W"])
    Wb[3] = 0
    inp2 = dict(inp, W=datagen.bf16_bits_to_f32(Wb))
    pw = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 128), rq.Quant.int4(), Wb)
    ref = _oracle_weights(w, inp2)
    assert np.array_equal(pw.codes(), ref["codes"])
    assert np.array_equal(pw.scales(), ref["scale"])
    assert pw.scales()[3] == 0 and not pw.codes()[3].any()


def test_pack_lloydmax_matches_oracle():
    w = datagen.WORKLOADS["video"].with_shape(T=4, K=512, N=24, block=256)
    inp = datagen.make_inputs(w)
    a_lv, w_lv = rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(4)
    pw = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 256),
                         rq.Quant.lloydmax(a_lv, w_lv), inp["W"])
    ref = _oracle_weights(w, inp, q_kind=1, levels=orc.codebook_bf16(4))
    assert np.array_equal(pw.codes(), ref["codes"])
    assert np.array_equal(pw.scales(), ref["scale"])
    assert pw.header.row_bytes == w.K // 4 and pw.header.b_div == 256
    assert np.array_equal(np.array(pw.header.a_levels[:16], np.float32), a_lv)


def test_pack_lloydmax_16_level_weights_matches_oracle():
    # OrbitQuant W4A4: a 16-level weight book, 4-bit indices (nibbles)
    w = datagen.WORKLOADS["video"].with_shape(T=4, K=512, N=24, block=256, w_bits=4)
    inp = datagen.make_inputs(w)
    a_lv, w_lv = rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(16)
    pw = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 256),
                         rq.Quant.lloydmax(a_lv, w_lv), inp["W"])
    ref = _oracle_weights(w, inp, q_kind=1, levels=orc.codebook_bf16(16))
    assert pw.header.row_bytes == w.K // 2 and pw.header.w_bits == 4
    assert np.array_equal(pw.codes(), ref["codes"])
    assert np.array_equal(pw.scales(), ref["scale"])


@pytest.mark.parametrize("w_bits,N", [(4, 24), (4, 40)])
def test_pack_lloydmax_bf16_fragments(w_bits, N):
    """The codebook GEMM's copy of 16-level weights: the level of every
    oracle index as bf16, in the fragment order [N/32][K/16][64 lanes][8]
    (lane i + 32 h of k-step c: row 32 tile + i, coordinates 16 c + 8 h ..),
    rows past N zero.  2-bit weights have no copy."""
    w = datagen.WORKLOADS["video"].with_shape(T=4, K=512, N=N, block=256, w_bits=w_bits)
    inp = datagen.make_inputs(w)
    a_lv, w_lv = rq.lloydmax_gaussian(16), rq.lloydmax_gaussian(1 << w_bits)
    pw = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 256),
                         rq.Quant.lloydmax(a_lv, w_lv), inp["W"])
    ref = _oracle_weights(w, inp, q_kind=1, levels=orc.codebook_bf16(1 << w_bits))
    per = 8 // w_bits
    packed = ref["codes"].astype(np.int64)
    idx = np.stack([(packed >> (w_bits * j)) & ((1 << w_bits) - 1) for j in range(per)], axis=2)
    idx = idx.reshape(N, w.K)
    want = (w_lv.view(np.uint32) >> 16).astype(np.uint16)[idx]
    h = pw.header
    nt = -(-N // 32)
    assert h.mma_ntiles == nt and h.mma_stages == 0 and h.mma_offset % 256 == 0
    frag = pw.blob[h.mma_offset:h.mma_offset + nt * (w.K // 16) * 1024].view(np.uint16)
    frag = frag.reshape(nt, w.K // 16, 2, 32, 8)                  # [tile][c][h][i][e]
    rows = frag.transpose(0, 3, 1, 2, 4).reshape(nt * 32, w.K)    # k = 16 c + 8 h + e
    assert np.array_equal(rows[:N], want)
    assert not rows[N:].any()
    w2 = datagen.WORKLOADS["video"].with_shape(T=4, K=512, N=N, block=256)
    p2 = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 256),
                         rq.Quant.lloydmax(a_lv, rq.lloydmax_gaussian(4)), datagen.make_inputs(w2)["W"])
    assert p2.header.mma_offset == 0 and p2.header.mma_ntiles == 0


def test_pack_rejects_bad_tables():
    sign, perm = datagen.random_rpbh(256, 1)
    perm = perm.copy()
    perm[0] = perm[1]
    W = np.zeros((4, 256), np.float32)
    with pytest.raises(rq.RQError, match="permutation"):
        rq.pack_weights(rq.Rotation.rpbh(sign, perm, 64), rq.Quant.int4(), W)
    sign2 = sign.copy()
    sign2[5] = 0
    with pytest.raises(rq.RQError, match="sign"):
        rq.pack_weights(rq.Rotation.rpbh(sign2, np.arange(256, dtype=np.int32), 64), rq.Quant.int4(), W)
    with pytest.raises(TypeError):
        rq.pack_weights(rq.Rotation.rpbh(sign, np.arange(256, dtype=np.int32), 64), rq.Quant.int4(),
                        W.astype(np.float64))


def test_int4_asym_descriptor_and_blob():
    # asymmetric activations take the RPBH rotation only; their weights are the
    # symmetric INT4 weights, tagged with the activation quantizer
    qa = rq.Quant.int4_asym().c()
    dense = rq.c_rotation(rq.RQ_ROT_DENSE, 256, 0, 32, None, None, 1 << 22)
    assert _rq_call(dense, qa, top=1 << 23, ws=1 << 24, wsb=1 << 30) == -6
    assert _rq_call(_rpbh(), qa, T=0, X=0, codes=0, scale=0) == 0
    assert _rq_call(_rpbh(), qa, codes=None, mma=None) == -1
    w = datagen.WORKLOADS["flux_up_asym"].with_shape(T=4, K=512, N=40, block=128)
    inp = datagen.make_inputs(w)
    rot = rq.Rotation.rpbh(inp["sign"], inp["perm"], w.block)
    pa = rq.pack_weights(rot, rq.Quant.int4_asym(), inp["W"])
    ps = rq.pack_weights(rot, rq.Quant.int4(), inp["W"])
    assert pa.header.format == rq.RQ_Q_INT4_ASYM and ps.header.format == rq.RQ_Q_INT4_SYM
    assert np.array_equal(pa.codes(), ps.codes()) and np.array_equal(pa.scales(), ps.scales())
    assert np.array_equal(pa.wsum(), ps.wsum()) and np.array_equal(pa.mma_tiles(), ps.mma_tiles())
    n = ctypes.c_size_t(0)
    rd = rq.Rotation.dense(np.eye(512, dtype=np.float32), 0)
    assert rq.load().rq_packed_weight_bytes(ctypes.byref(rd.c_host()), ctypes.byref(qa), 40,
                                            ctypes.byref(n)) == -6


# ---------------------------------------------------------------------------
# the further formats: MXFP4, 8-bit integer weights, the TR-DQ fold
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,shape", [("flux_up_mxfp4", dict(K=1024, N=70)),
                                        ("flux_down_mxfp4", dict(K=2048, N=33)),
                                        ("tiny", dict(K=256, N=40, block=64))])
def test_pack_mxfp4_matches_oracle(name, shape):
    """Weight fold + MXFP4 (E2M1 codes, E8M0 block scales) equal the oracle
    bit for bit; the GEMM's tiled copies hold the same codes and scales."""
    w = datagen.WORKLOADS[name].with_shape(T=4, **shape)
    inp = datagen.make_inputs(w)
    pw = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], w.block), rq.Quant.mxfp4(),
                         inp["W"])
    ref = orc.weight_rows(inp["W"], rot_kind=0, b=w.block, sign=inp["sign"], perm=inp["perm"],
                          q_kind=3)
    assert np.array_equal(pw.codes(), ref["codes"])
    assert np.array_equal(pw.mx_scales(), ref["mx_scales"])
    h = pw.header
    assert (h.format, h.b_div, h.row_bytes, h.mma_stages, h.mma_ntiles) == (
        rq.RQ_Q_MXFP4, w.block, w.K // 2, w.K // 128, -(-w.N // 32))
    nch = w.K // 32
    tiles = pw.blob[h.mma_offset:h.mma_offset + h.mma_ntiles * nch * 512].reshape(h.mma_ntiles, nch, 32, 16)
    codes = tiles.transpose(0, 2, 1, 3).reshape(h.mma_ntiles * 32, nch * 16)[:w.N]
    assert np.array_equal(codes, ref["codes"])
    sc = pw.blob[h.mxs_offset:h.mxs_offset + h.mma_stages * h.mma_ntiles * 128]
    sc = sc.reshape(h.mma_stages, h.mma_ntiles, 2, 32, 2)           # [s][tile][h][row][ks]
    full = sc.transpose(1, 3, 0, 4, 2).reshape(h.mma_ntiles * 32, nch)   # chunk 4 s + 2 ks + h
    assert np.array_equal(full[:w.N], ref["mx_scales"])


@pytest.mark.parametrize("name,shape", [("flux_up_w4a8", dict(K=512, N=40)),
                                        ("flux_up_w8a8", dict(K=512, N=40)),
                                        ("flux_up_trdq", dict(K=512, N=40)),
                                        ("flux_up_trdq", dict(K=256, N=24, w_bits=8)),
                                        ("flux_up_w6a6", dict(K=512, N=40)),
                                        ("flux_up_trdq_w6a6", dict(K=256, N=24)),
                                        ("flux_up_w6a6", dict(K=256, N=40, w_bits=4))])
def test_pack_int8_paths_match_oracle(name, shape):
    """8- and 6-bit weights (one code per byte) and the int8 copy of 4-bit
    weights that the int8 GEMM reads; the TR-DQ fold (smoothing, R1, zigzag,
    R2 in fp64)."""
    w = datagen.WORKLOADS[name].with_shape(T=4, **shape)
    inp = datagen.make_inputs(w)
    from rotated_w4a4_quantized_amd.layer import quant_for, rotation_for
    pw = rq.pack_weights(rotation_for(w, inp), quant_for(w), inp["W"])
    from tests import _layer as H
    ref = H.oracle_weights(w, inp)
    assert np.array_equal(pw.codes(), ref["codes"])
    assert np.array_equal(pw.scales().view(np.uint32), ref["scale"].view(np.uint32))
    h = pw.header
    assert (h.a_bits, h.w_bits, h.b_div) == (w.a_bits, w.w_bits, w.b_eff)
    assert np.array_equal(pw.i8_codes().astype(np.int16), ref["q"])
    assert np.array_equal(pw.wsum(), ref["q"].astype(np.int64).sum(axis=1))


def test_new_format_validation_errors():
    L = rq.load()
    K = 256
    mx = rq.Quant.mxfp4().c()
    # MXFP4 needs K % 128 == 0 and the RPBH rotation
    assert _rq_call(rq.c_rotation(rq.RQ_ROT_RPBH, 160, 32, 0, 1 << 20, 1 << 21, None), mx) == -2
    dense = rq.c_rotation(rq.RQ_ROT_DENSE, K, 0, 0, None, None, 1 << 22)
    assert _rq_call(dense, mx) == -6
    # 6- and 8-bit activations: not with the dense path; a_bits / w_bits values
    assert _rq_call(dense, rq.Quant.integer(8, 4).c()) == -6
    assert _rq_call(dense, rq.Quant.integer(6, 6).c()) == -6
    assert _rq_call(_rpbh(), rq.c_quant(0, 5, 4, 0)) == -6
    assert _rq_call(_rpbh(), rq.c_quant(0, 6, 7, 0)) == -6
    assert _rq_call(_rpbh(), rq.c_quant(0, 4, 8, 0)) == -6
    assert _rq_call(_rpbh(), rq.c_quant(0, 4, 6, 0)) == -6
    # TR-DQ: block range, tables
    td = rq.c_rotation(rq.RQ_ROT_TRDQ, K, 8, 0, None, 1 << 21, 1 << 22, 1 << 23, 1 << 24)
    assert _rq_call(td, rq.Quant.integer(8, 4).c()) == -2
    td = rq.c_rotation(rq.RQ_ROT_TRDQ, K, 64, 0, None, 1 << 21, 1 << 22, None, 1 << 24)
    assert _rq_call(td, rq.Quant.integer(8, 4).c()) == -1
    td = rq.c_rotation(rq.RQ_ROT_TRDQ, K, 64, 0, None, 1 << 21, 1 << 22, 1 << 23, 1 << 24)
    assert _rq_call(td, mx) == -6
    # activation sizes
    rot = rq.Rotation.rpbh(np.ones(K, np.int8), np.arange(K, dtype=np.int32), 64)
    assert rq.activation_bytes(rot, rq.Quant.mxfp4(), 40) == (40 * K // 2, 40 * K // 32,
                                                             2 * (K // 32) * 512 + (K // 128) * 2 * 128)
    assert rq.activation_bytes(rot, rq.Quant.integer(8, 4, asym=True), 40) == (40 * K, 80 * 4, 64 * K)
    # 6-bit codes one per byte
    assert rq.activation_bytes(rot, rq.Quant.integer(6, 6), 40) == (40 * K, 40 * 4, 64 * K)
    # the MXFP4 GEMM reads the tiled codes: canonical codes alone are refused
    w = datagen.WORKLOADS["flux_up_mxfp4"].with_shape(T=4, K=K, N=40, block=64)
    inp = datagen.make_inputs(w)
    h = rq.pack_weights(rq.Rotation.rpbh(inp["sign"], inp["perm"], 64), rq.Quant.mxfp4(), inp["W"]).header
    assert L.rq_w4a4_linear(ctypes.byref(h), ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21),
                            ctypes.c_void_p(1 << 22), None, None, 4, None, ctypes.c_void_p(1 << 24),
                            rq.RQ_F32, None) == -6
    assert L.rq_w4a4_linear(ctypes.byref(h), ctypes.c_void_p(1 << 20), None, None, None,
                            ctypes.c_void_p(1 << 23), 4, None, ctypes.c_void_p(1 << 24),
                            rq.RQ_I32, None) == -6


def test_weight_set_members():
    """Time-step sets ("TR-DQ" Eq.(10)): each group's member is exactly
    rq_pack_weights with that group's rotation; steps map to their group."""
    w = datagen.WORKLOADS["flux_up_trdq"].with_shape(T=4, K=256, N=40, block=64)
    ins = datagen.make_timestep_inputs(w, 3)
    assert all(np.array_equal(i["W"], ins[0]["W"]) for i in ins)
    assert not np.array_equal(ins[0]["perm"], ins[1]["perm"])
    from rotated_w4a4_quantized_amd.layer import quant_for, rotation_for
    rots = [rotation_for(w, i) for i in ins]
    steps = [0, 0, 1, 1, 1, 2, 2, 0]
    ws = rq.pack_weight_set(rots, steps, quant_for(w), ins[0]["W"])
    for t, g_want in enumerate(steps):
        g, hdr, off = ws.member(t)
        assert g == g_want and off % 256 == 0
        one = rq.pack_weights(rots[g], quant_for(w), ins[0]["W"])
        assert np.array_equal(ws.blob[off:off + one.blob.size], one.blob)
    with pytest.raises(rq.RQError) as e:
        ws.member(len(steps))
    assert e.value.status == -2
    bad = rq.WeightSet(np.zeros(8192, np.uint8))
    with pytest.raises(rq.RQError) as e:
        bad.member(0)
    assert e.value.status == -5
    with pytest.raises(rq.RQError):
        rq.pack_weight_set(rots, [0, 3], quant_for(w), ins[0]["W"])   # step maps past the groups

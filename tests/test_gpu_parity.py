"""GPU parity: the HIP path (through the C ABI) against the oracle, on the
same seeded inputs.  Integer results bit-exact, floats within the stated
tolerance (tests/_layer.py).

Small shapes span several 128 x 128 GEMM tiles with ragged token and output
tails; the full workloads (tiny 256x1152->1152 fp32, pixart 8192x1152->4608
dense, flux_up 9216x3072->12288, flux_down 9216x12288->3072, video
32760x1536->8960 Lloyd-Max W2A4) run in the launch configuration bench.py
times, with every code and scale compared and the outputs compared at
sampled (token, channel) pairs.
"""
import dataclasses
import sys

import numpy as np
import pytest

from rotated_w4a4_quantized_amd import datagen
from tests import _layer as H
from rotated_w4a4_quantized_amd.layer import mma_capable

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def mma_mode(w):
    """Layer mode for the parity runs: layers whose codes have a matrix-core
    layout (4-bit integer codes under RPBH or DENSE, MXFP4) write both code
    layouts and the GEMM reads the MMA copy."""
    return "both" if mma_capable(w) else "canonical"


def check_act_mx(w, L, act, rows=None):
    """MXFP4: canonical E2M1 codes and E8M0 scales, and the tiled copies the
    GEMM reads, bit for bit."""
    codes = L.codes.cpu().numpy()
    sc = L.scale.cpu().numpy()
    nch = w.K // 32
    tiles = -(-w.T // 32)
    buf = L.codes_mma.cpu().numpy()
    tc = buf[:tiles * nch * 512].reshape(tiles, nch, 32, 16).transpose(0, 2, 1, 3)
    tc = tc.reshape(tiles * 32, nch * 16)[:w.T]
    S = w.K // 128
    ts = buf[tiles * nch * 512:tiles * nch * 512 + S * tiles * 128].reshape(S, tiles, 2, 32, 2)
    ts = ts.transpose(1, 3, 0, 4, 2).reshape(tiles * 32, nch)[:w.T]
    if rows is not None:
        codes, sc, tc, ts = codes[rows], sc[rows], tc[rows], ts[rows]
    for name, got in (("codes", codes), ("tiled codes", tc)):
        bad = np.nonzero(np.any(got != act["codes"], axis=1))[0]
        assert bad.size == 0, f"MXFP4 {name} differ in {bad.size} tokens, first {bad[:5]}"
    for name, got in (("scales", sc), ("tiled scales", ts)):
        bad = np.nonzero(np.any(got != act["mx_scales"], axis=1))[0]
        assert bad.size == 0, f"MXFP4 {name} differ in {bad.size} tokens, first {bad[:5]}"


def check_act(w, L, act, rows=None):
    if w.quant == "mxfp4":
        return check_act_mx(w, L, act, rows)
    codes = L.codes.cpu().numpy()
    scale = L.scale.cpu().numpy()
    asym = w.quant == "int4_asym"
    if asym:   # s [T] then the zero points [T]
        zero = scale[w.T:]
        scale = scale[:w.T]
        if rows is not None:
            zero = zero[rows]
        assert np.array_equal(zero.view(np.uint32), act["zero"].view(np.uint32)), \
            f"zero point mismatch in {int(np.sum(zero != act['zero']))} tokens"
    if rows is not None:
        codes, scale = codes[rows], scale[rows]
    assert np.array_equal(scale.view(np.uint32), act["scale"].view(np.uint32)), \
        f"scale mismatch in {int(np.sum(scale != act['scale']))} tokens"
    bad = np.nonzero(np.any(codes != act["codes"], axis=1))[0]
    assert bad.size == 0, f"codes differ in {bad.size} tokens, first {bad[:5]}"
    if L.codes_mma is not None and w.quant in ("int4", "int4_asym") and w.a_bits == 4:
        dec, top_clear = H.decode_codes_mma(L.codes_mma.cpu().numpy(), w.T, w.Kq)
        if rows is not None:
            dec = dec[rows]
        assert top_clear, "a codes_mma field has its top bits set"
        ref = H.unpack_codes(act["codes"])
        if asym:   # fields hold the unsigned codes: decoded as u - 8
            ref = (ref & 15) - 8
        bad = np.nonzero(np.any(dec != ref, axis=1))[0]
        assert bad.size == 0, f"codes_mma differs in {bad.size} tokens, first {bad[:5]}"
    if w.quant in ("int4", "int4_asym") and w.a_bits in (6, 8) and L.codes_mma is not None:
        # the same bytes in the int8 GEMM's fragment order
        dec = H.decode_i8_mma(L.codes_mma.cpu().numpy(), w.T, w.K)
        if rows is not None:
            dec = dec[rows]
        bad = np.nonzero(np.any(dec != np.asarray(act["codes"], np.uint8), axis=1))[0]
        assert bad.size == 0, f"int8 fragment codes differ in {bad.size} tokens, first {bad[:5]}"
    if w.quant == "lloydmax" and L.codes_mma is not None:
        # the bf16 levels of the codes, in the codebook GEMM's fragment order
        dec = H.decode_cb_mma(L.codes_mma.cpu().numpy(), w.T, w.K)
        if rows is not None:
            dec = dec[rows]
        lev = datagen.f32_to_bf16_bits(H.orc.codebook_bf16(16).astype(np.float32))
        ref = lev[H.unpack_nibbles(act["codes"])]
        bad = np.nonzero(np.any(dec != ref, axis=1))[0]
        assert bad.size == 0, f"bf16 level fragments differ in {bad.size} tokens, first {bad[:5]}"
    if w.r:
        top = L.top.cpu().numpy().view(np.uint16)
        if rows is not None:
            top = top[rows]
        assert np.array_equal(top, act["top"])


SMALL = [
    # MXFP4 (E2M1 + E8M0 per 32), 8-bit activations (W4A8, W8A8, asymmetric),
    # and the TR-DQ rotation
    ("flux_up_mxfp4", dict(T=257, K=3072, N=384)),
    ("flux_down_mxfp4", dict(T=131, K=12288, N=136)),
    ("flux_up_mxfp4", dict(T=40, K=256, N=300, block=64)),
    ("flux_up_mxfp4", dict(T=70, K=1024, N=128, block=1024)),
    ("flux_up_mxfp4", dict(T=33, K=128, N=40, block=2)),
    ("flux_up_mxfp4", dict(T=65, K=512, N=64, block=32)),
    ("flux_up_w4a8", dict(T=257, K=3072, N=384)),
    ("flux_up_w8a8", dict(T=257, K=3072, N=384)),
    ("flux_up_w4a8", dict(T=33, K=96, N=40, block=2)),
    ("flux_up_w8a8", dict(T=45, K=64, N=48, block=64)),
    ("flux_up_trdq", dict(T=70, K=1024, N=136)),
    ("flux_up_trdq", dict(T=33, K=512, N=40, block=16)),
    ("flux_up_trdq", dict(T=20, K=8192, N=64, block=256)),
    ("flux_up_trdq", dict(T=9, K=16384, N=40, block=64)),

    ("tiny", dict(T=300, N=200)),
    ("tiny", dict(T=1, N=130, K=256, block=256)),
    ("flux_up", dict(T=257, K=3072, N=384)),
    ("flux_down", dict(T=131, K=12288, N=136)),
    ("video", dict(T=190, N=264)),
    ("pixart", dict(T=200, N=170)),
    # dense rotation tiles with ragged column and token edges
    ("pixart", dict(T=77, K=160, N=40)),
    ("pixart", dict(T=260, K=416, N=96)),
    ("tiny", dict(T=70, K=1024, N=128, block=1024)),
    ("tiny", dict(T=65, K=96, N=40, block=2)),
    ("tiny", dict(T=33, K=32, N=7, block=8)),
    ("flux_up", dict(T=40, K=16384, N=64, block=512)),
    # fp32 input at the largest K: a group of four tokens' code slots fits in
    # LDS beside the row at block 512; at block 64 (more padding) it does
    # not, and the MMA codes are stored per token
    ("tiny", dict(T=37, K=16384, N=64, block=512)),
    ("tiny", dict(T=37, K=16384, N=64, block=64)),
    # asymmetric per-token activations (zero point)
    ("flux_up_asym", dict(T=257, K=3072, N=384)),
    ("flux_down_asym", dict(T=131, K=12288, N=136)),
    ("flux_up_asym", dict(T=33, K=96, N=40, block=2)),
    # OrbitQuant W4A4: a 16-level weight book
    ("video_w4", dict(T=190, N=264)),
    # two and six threads per token: per-token reductions over runs of two lanes
    ("tiny", dict(T=45, K=64, N=48, block=64)),
    ("tiny", dict(T=21, K=192, N=40, block=64)),
    ("flux_up_asym", dict(T=33, K=64, N=40, block=64)),
    # the block's high index bits across 16 and 32 lanes (the lane stages'
    # last mask is a swizzle at block 1024) under every quantizer that folds
    # the lanes' sign: zero point, codebook, 8-bit codes
    ("flux_up_asym", dict(T=70, K=2048, N=96, block=1024)),
    ("video", dict(T=70, K=2048, N=96, block=1024)),
    ("video_w4", dict(T=45, K=1024, N=64, block=512)),
    ("flux_up_w8a8", dict(T=70, K=2048, N=96, block=1024)),
    ("flux_up_w4a8", dict(T=33, K=1024, N=40, block=512)),
    # TR-DQ's W6A6 setting: 6-bit codes one per byte, int8 matrix cores
    ("flux_up_w6a6", dict(T=257, K=3072, N=384)),
    ("flux_up_w6a6", dict(T=33, K=96, N=40, block=2)),
    ("flux_up_w6a6", dict(T=70, K=2048, N=96, block=1024)),
    ("flux_up_trdq_w6a6", dict(T=70, K=1024, N=136)),
    ("flux_up_trdq_w6a6", dict(T=9, K=16384, N=40, block=64)),
    ("flux_up_w6a6", dict(T=1, K=64, N=7, block=64)),
    ("flux_up_w6a6", dict(T=5, K=16384, N=40, block=512)),
]


@pytest.mark.parametrize("name,shape", SMALL, ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in s.items())}"
                                                   for n, s in SMALL])
def test_small_full_parity(name, shape):
    w = datagen.WORKLOADS[name].with_shape(**shape)
    say(f"[parity small] {w}")
    small_parity(w, datagen.make_inputs(w))


# Asymmetric byte codes under RPBH: 8-bit (255 levels) and 6-bit (63 levels,
# TR-DQ's W6A6), against the oracle like the small cases.
BYTE_ASYM = [(8, dict(T=70, K=1024, N=64)), (6, dict(T=70, K=1024, N=64)),
             (6, dict(T=33, K=2048, N=40, block=1024))]


@pytest.mark.parametrize("bits,shape", BYTE_ASYM,
                         ids=[f"a{b}-{'-'.join(f'{k}{v}' for k, v in s.items())}" for b, s in BYTE_ASYM])
def test_asym_byte_codes_parity(bits, shape):
    w = dataclasses.replace(datagen.WORKLOADS["flux_up_w6a6"].with_shape(a_bits=bits, w_bits=bits, **shape),
                            quant="int4_asym")
    say(f"[parity asym bytes] {w}")
    small_parity(w, datagen.make_inputs(w))


def small_parity(w, inp):
    """Every code, scale, accumulator and output of one small layer against
    the oracle (both code layouts for RPBH INT4, both output dtypes)."""
    L = H.GpuLayer(w, inp, y_dtype="f32", codes=mma_mode(w))
    L.run()
    torch.cuda.synchronize()
    act = H.oracle_act(w, inp)
    check_act(w, L, act)
    wts = H.oracle_weights(w, inp)
    assert np.array_equal(L.packed.codes(), wts["codes"])
    ta, nw = np.meshgrid(np.arange(w.T), np.arange(w.N), indexing="ij")
    ta, nw = ta.ravel(), nw.ravel()
    yhat = H.oracle_yhat_pairs(w, act, wts, ta, nw)
    y = L.Y.cpu().numpy().ravel()
    err = H.rel_err(y, yhat)
    say(f"  fp32 output max floored rel err {err:.3e}")
    assert err <= H.REL_TOL
    if w.quant == "lloydmax" and L.codes_mma is not None and L.codes is not None:
        # the same GEMM decoding the canonical indices itself
        Yc = torch.empty((w.T, w.N), dtype=torch.float32, device="cuda")
        L.linear(Yc, use_mma=False)
        err = H.rel_err(Yc.cpu().numpy().ravel(), yhat)
        say(f"  fp32 output (index-decoding GEMM) max floored rel err {err:.3e}")
        assert err <= H.REL_TOL
    if w.quant in ("int4", "int4_asym"):
        ref = H.oracle_raw_acc(w, act, wts)
        acc = L.raw_acc().cpu().numpy().astype(np.int64)
        assert np.array_equal(acc, ref)
        if L.codes_mma is not None and L.codes is not None:
            # the same accumulators from the canonical codes (converted in the GEMM)
            acc = L.raw_acc(use_mma=False).cpu().numpy().astype(np.int64)
            assert np.array_equal(acc, ref)
            Yc = torch.empty((w.T, w.N), dtype=torch.float32, device="cuda")
            L.linear(Yc, use_mma=False)
            err = H.rel_err(Yc.cpu().numpy().ravel(), yhat)
            say(f"  fp32 output (canonical-code GEMM) max floored rel err {err:.3e}")
            assert err <= H.REL_TOL
    # bf16 output of the same kernels
    Yb = torch.empty((w.T, w.N), dtype=torch.bfloat16, device="cuda")
    L.linear(Yb)
    dist, ok = H.bf16_check(H.to_np_bf16_bits(Yb).ravel(), yhat)
    say(f"  bf16 output max ulp distance {dist}")
    assert ok


FULL = ["tiny", "flux_up", "flux_down", "video", "pixart", "flux_up_asym", "flux_down_asym", "video_w4",
        "flux_up_mxfp4", "flux_down_mxfp4", "flux_up_w4a8", "flux_up_w8a8", "flux_up_trdq",
        "flux_up_w6a6", "flux_up_trdq_w6a6"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_parity(name):
    w = datagen.WORKLOADS[name]
    say(f"[parity full] {w}")
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, codes=mma_mode(w))
    L.run()
    torch.cuda.synchronize()
    g = np.random.default_rng(7)
    # every token's codes and scales, for every rotation (the dense and
    # TR-DQ oracles, fp32 chains per coordinate, take a few seconds here)
    rows = None
    act = H.oracle_act(w, inp, rows)
    check_act(w, L, act, rows)
    wts = H.oracle_weights(w, inp)
    assert np.array_equal(L.packed.codes(), wts["codes"])
    # outputs at sampled pairs: 8192 random pairs plus two whole tokens and
    # two whole channels
    tok_pool = np.arange(w.T) if rows is None else rows
    ta = g.choice(tok_pool, 8192)
    nw = g.integers(0, w.N, 8192)
    t2 = np.repeat(tok_pool[[0, -1]], w.N)
    n2 = np.tile(np.arange(w.N), 2)
    n3 = np.repeat(np.array([0, w.N - 1]), tok_pool.size)
    t3 = np.tile(tok_pool, 2)
    ta = np.concatenate([ta, t2, t3])
    nw = np.concatenate([nw, n2, n3])
    yhat = H.oracle_yhat_pairs(w, act, wts, ta, nw, act_rows=rows)
    Y = L.Y
    idx = torch.from_numpy(ta).to("cuda") * w.N + torch.from_numpy(nw).to("cuda")
    ys = Y.view(-1)[idx]
    if w.quant == "int4" and w.r == 0:
        # the exact int32 accumulators of the same launch configuration at
        # the sampled pairs
        acc = L.raw_acc().view(-1)[idx].cpu().numpy().astype(np.int64)
        ia = ta if rows is None else np.searchsorted(rows, ta)
        ref = H._acc_pairs(w, act, wts, ia, nw)
        assert np.array_equal(acc, ref), f"accumulators differ at {int(np.sum(acc != ref))} pairs"
        say(f"  int32 accumulators bit-exact at {ta.size} pairs")
    if w.ydtype == "f32":
        err = H.rel_err(ys.cpu().numpy(), yhat)
        say(f"  fp32 max floored rel err {err:.3e}")
        assert err <= H.REL_TOL
    else:
        dist, ok = H.bf16_check(H.to_np_bf16_bits(ys), yhat)
        say(f"  bf16 max ulp distance {dist}")
        assert ok
        # and the fp32-output run of the same kernels meets the 1e-3 bound
        Yf = torch.empty((w.T, w.N), dtype=torch.float32, device="cuda")
        L.linear(Yf)
        err = H.rel_err(Yf.view(-1)[idx].cpu().numpy(), yhat)
        say(f"  fp32 max floored rel err {err:.3e}")
        assert err <= H.REL_TOL


def test_zero_tokens_and_determinism():
    w = datagen.WORKLOADS["flux_up"].with_shape(T=300, K=3072, N=256)
    inp = datagen.make_inputs(w)
    Xz = inp["X"].copy()
    Xz[[0, 17, 299]] = 0
    inp = dict(inp, X=Xz, Xf=datagen.bf16_bits_to_f32(Xz))
    L = H.GpuLayer(w, inp, y_dtype="f32")
    L.run()
    c1, s1, y1 = L.codes.clone(), L.scale.clone(), L.Y.clone()
    L.run()
    torch.cuda.synchronize()
    assert torch.equal(c1, L.codes) and torch.equal(s1, L.scale) and torch.equal(y1, L.Y)
    for t in (0, 17, 299):
        assert float(L.scale[t]) == 0.0 and int(L.codes[t].abs().sum()) == 0
        assert float(L.Y[t].abs().max()) == 0.0


def test_outputs_stay_in_bounds():
    # guard bands after every output buffer must be untouched
    w = datagen.WORKLOADS["tiny"].with_shape(T=77, N=150)
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, y_dtype="f32")
    G = 4096
    codes = torch.full((w.T * w.K // 2 + G,), 0xA5, dtype=torch.uint8, device="cuda")
    scale = torch.full((w.T + G,), 7.5, dtype=torch.float32, device="cuda")
    Y = torch.full((w.T * w.N + G,), 3.25, dtype=torch.float32, device="cuda")
    L.codes = codes[: w.T * w.K // 2].view(w.T, w.K // 2)
    L.scale = scale[: w.T]
    L.rotate_quant()
    L.linear(Y[: w.T * w.N].view(w.T, w.N))
    torch.cuda.synchronize()
    assert bool((codes[w.T * w.K // 2:] == 0xA5).all())
    assert bool((scale[w.T:] == 7.5).all())
    assert bool((Y[w.T * w.N:] == 3.25).all())
    # the MMA-layout codes and the GEMM that reads them (K = 1152: a ragged
    # last 128-coordinate block)
    M = H.GpuLayer(w, inp, y_dtype="f32", codes="mma")
    nb = M.codes_mma.numel()
    mma = torch.full((nb + G,), 0x5A, dtype=torch.uint8, device="cuda")
    Y2 = torch.full((w.T * w.N + G,), 3.25, dtype=torch.float32, device="cuda")
    M.codes_mma = mma[:nb]
    M.rotate_quant()
    M.linear(Y2[: w.T * w.N].view(w.T, w.N))
    torch.cuda.synchronize()
    assert bool((mma[nb:] == 0x5A).all())
    assert bool((Y2[w.T * w.N:] == 3.25).all())
    assert torch.equal(Y2[: w.T * w.N], Y[: w.T * w.N])


def test_runs_on_a_side_stream():
    w = datagen.WORKLOADS["tiny"].with_shape(T=128, N=128)
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, y_dtype="f32")
    L.run()
    ref = L.Y.clone()
    L.Y.zero_()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.run()
    s.synchronize()
    assert torch.equal(ref, L.Y)


CODES_ONLY = [
    ("flux_down", dict(T=300, K=2048, N=520, block=512)),
    ("pixart", dict(T=300, K=1152, N=520)),
    ("flux_up_w4a8", dict(T=300, K=1024, N=520, block=256)),
    ("flux_up_w8a8", dict(T=300, K=1024, N=520, block=256)),
    ("flux_up_trdq", dict(T=300, K=1024, N=520, block=128)),
    # enough 256 x 256 output tiles (9 x 17) that the canonical-code GEMM
    # takes its 256 x 256 kernel rather than 128 x 128 tiles; ragged edges
    ("flux_up", dict(T=2200, K=1024, N=4100, block=256)),
]


@pytest.mark.parametrize("name,shape", CODES_ONLY,
                         ids=[f"{n}-T{s['T']}-N{s['N']}" for n, s in CODES_ONLY])
def test_mma_codes_only_path(name, shape):
    # the bench configuration: rq_rotate_quant writes only the MMA-layout
    # codes (canonical codes NULL) and the GEMM reads them; compared with a
    # canonical-code run
    w = datagen.WORKLOADS[name].with_shape(**shape)
    say(f"[codes only] {w}")
    inp = datagen.make_inputs(w)
    A = H.GpuLayer(w, inp, y_dtype="f32", codes="mma")
    B = H.GpuLayer(w, inp, y_dtype="f32", codes="canonical")
    A.run()
    B.run()
    accA = A.raw_acc().cpu().numpy()
    accB = B.raw_acc().cpu().numpy()
    torch.cuda.synchronize()
    assert A.codes is None and np.array_equal(accA, accB)
    assert torch.equal(A.scale, B.scale)
    if w.r == 0:
        assert torch.equal(A.Y, B.Y)
    else:
        # the MMA-layout GEMM adds the bf16 low-rank term on the matrix cores,
        # the canonical-code GEMM with fp32 FMAs: the same exact products
        # summed in another order
        assert torch.equal(A.top, B.top)
        d = (A.Y - B.Y).abs().max().item()
        assert d <= 1e-5 * B.Y.abs().max().item(), d



def test_mma_bf16_output_matches_converting_kernel():
    # Full 256 x 256 tiles of the MMA-layout GEMM round bf16 outputs with the
    # hardware conversion; the converting kernel rounds in software (nearest
    # even).  Same accumulators and the same fp32 operations, so the bits
    # must agree -- full tiles and the ragged edge alike.
    w = datagen.WORKLOADS["flux_up"].with_shape(T=600, K=1024, N=800, block=256)
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, codes="both")
    assert L.Y.dtype == torch.bfloat16
    L.rotate_quant()
    Ya = torch.empty_like(L.Y)
    Yb = torch.empty_like(L.Y)
    L.linear(Ya, use_mma=True)
    L.linear(Yb, use_mma=False)
    torch.cuda.synchronize()
    assert torch.equal(Ya.view(torch.int16), Yb.view(torch.int16))


# The codebook GEMM at mid-size shapes (many tiles, ragged token and channel
# edges, another K), against the oracle at sampled pairs plus the first and
# last token rows and channel columns.
CODEBOOK_BIG = [
    ("video", dict(T=4000, N=4100)),
    ("video", dict(T=4104, N=4000, K=1024)),
    ("video_w4", dict(T=4000, N=4100)),
]


def test_codebook_asymmetric_activation_book():
    """An activation book that is not symmetric about 0 (the Lloyd-Max levels
    shifted by 1/16, rounded to bf16) takes the general fifteen-threshold
    index count in rq_rotate_quant; codes and sigma match the oracle given the
    same levels bit for bit."""
    from oracle import oracle as orc
    w = datagen.WORKLOADS["video"].with_shape(T=190, N=264)
    say(f"[codebook asymmetric book] {w}")
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, y_dtype="f32")
    lv = np.array([orc.round_to_bf16(float(v) + 0.0625) for v in orc.codebook_bf16(16)], np.float32)
    assert np.all(np.diff(lv) > 0) and (lv[7] + lv[8]) != 0.0
    L.q = H.rq.Quant.lloydmax(lv, H.rq.lloydmax_gaussian(4))
    L.rotate_quant()
    torch.cuda.synchronize()
    act = orc.act_rows(inp["X"], 1, w.K, np.arange(w.T), rot_kind=0, b=w.block, sign=inp["sign"],
                       perm=inp["perm"], q_kind=1, levels=lv)
    check_act(w, L, act)
    # both ends of the book are in use (indices are unsigned nibbles)
    nib = np.concatenate([act["codes"] & 15, act["codes"] >> 4])
    assert nib.min() == 0 and nib.max() == 15


@pytest.mark.parametrize("name,shape", CODEBOOK_BIG,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in s.items())}" for n, s in CODEBOOK_BIG])
def test_codebook_mid_size(name, shape):
    w = datagen.WORKLOADS[name].with_shape(**shape)
    say(f"[codebook mid] {w}")
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, y_dtype="f32")
    L.run()
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([g.choice(w.T, 256, replace=False), [0, w.T - 1]]))
    act = H.oracle_act(w, inp, rows)
    wts = H.oracle_weights(w, inp)
    assert np.array_equal(L.packed.codes(), wts["codes"])
    ta = np.concatenate([g.choice(rows, 8192), np.repeat(rows[[0, -1]], w.N), np.repeat(rows, 2)])
    nw = np.concatenate([g.integers(0, w.N, 8192), np.tile(np.arange(w.N), 2),
                         np.tile(np.array([0, w.N - 1]), rows.size)])
    yhat = H.oracle_yhat_pairs(w, act, wts, ta, nw, act_rows=rows)
    idx = torch.from_numpy(ta).to("cuda") * w.N + torch.from_numpy(nw).to("cuda")
    err = H.rel_err(L.Y.view(-1)[idx].cpu().numpy(), yhat)
    say(f"  fp32 max floored rel err {err:.3e}")
    assert err <= H.REL_TOL
    Yb = torch.empty((w.T, w.N), dtype=torch.bfloat16, device="cuda")
    L.linear(Yb)
    dist, ok = H.bf16_check(H.to_np_bf16_bits(Yb.view(-1)[idx]), yhat)
    say(f"  bf16 max ulp distance {dist}")
    assert ok


def test_asym_nonnegative_rows():
    """Asymmetric activations whose rotated row has a non-negative minimum:
    rne(min / s) is +0 or positive, and the zero point must be +0.0 exactly
    (bits 0), as the oracle stores it.  K = block, identity permutation and
    +1 signs, so x = a e0 + c e1 rotates to u = (a + c, a - c, a + c, ...);
    with 0 < c < a every coordinate is positive.  Also: rows whose minimum
    is a tiny positive or negative number, a constant rotated row (x = e0,
    d = 0) and ordinary Gaussian rows."""
    base = datagen.WORKLOADS["flux_up_asym"].with_shape(T=96, K=256, N=72, block=256)
    inp = datagen.make_inputs(base)
    X = np.zeros((base.T, base.K), np.float32)
    pairs = [(1.0, 0.97), (1.0, 0.999), (2.0, 1.5), (3.0, 0.5), (1.0, 1.0 - 2.0 ** -10),
             (0.75, 0.25), (1.0, 1.001), (1.0, 1.02), (0.5, 0.5)]
    for i, (a, c) in enumerate(pairs):
        X[i, 0], X[i, 1] = a, c
    X[len(pairs), 0] = 1.0                    # constant rotated row: d = 0
    g = np.random.default_rng(11)
    X[len(pairs) + 1:] = g.standard_normal((base.T - len(pairs) - 1, base.K)).astype(np.float32)
    xb = datagen.f32_to_bf16_bits(X)
    inp = dict(inp, X=xb, Xf=datagen.bf16_bits_to_f32(xb),
               sign=np.ones(base.K, np.int8), perm=np.arange(base.K, dtype=np.int32))
    act = H.oracle_act(base, inp)
    z = act["zero"][:len(pairs)]
    assert np.any(z.view(np.uint32) == 0), "no row reaches the +0 zero point"
    say(f"[asym non-negative rows] zero points {z.tolist()}")
    small_parity(base, inp)


# The int8-MFMA engine (rq_w4a4_linear_engine, RQ_ENGINE_INT8) on canonical
# codes: exact accumulators against the oracle, outputs within tolerance and
# equal to the FP6 engine's bit for bit (same accumulators, same fp32
# epilogue operations).
INT8_ENGINE = [
    ("tiny", dict(T=300, N=200)),
    ("flux_up", dict(T=257, K=3072, N=384)),
    ("flux_down", dict(T=131, K=12288, N=136)),
    ("pixart", dict(T=200, N=170)),
    # dense rotation tiles with ragged column and token edges
    ("pixart", dict(T=77, K=160, N=40)),
    ("pixart", dict(T=260, K=416, N=96)),
    ("tiny", dict(T=65, K=96, N=40, block=2)),
    ("flux_up", dict(T=600, K=1024, N=800, block=256)),
]


@pytest.mark.parametrize("name,shape", INT8_ENGINE,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in s.items())}" for n, s in INT8_ENGINE])
def test_int8_engine_parity(name, shape):
    w = datagen.WORKLOADS[name].with_shape(**shape)
    say(f"[int8 engine] {w}")
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, y_dtype="f32")
    L.rotate_quant()
    torch.cuda.synchronize()
    act = H.oracle_act(w, inp)
    wts = H.oracle_weights(w, inp)
    acc = L.raw_acc(engine="int8").cpu().numpy().astype(np.int64)
    assert np.array_equal(acc, H.oracle_raw_acc(w, act, wts))
    Yi = torch.empty((w.T, w.N), dtype=torch.float32, device="cuda")
    L.linear(Yi, engine="int8")
    ta, nw = np.meshgrid(np.arange(w.T), np.arange(w.N), indexing="ij")
    yhat = H.oracle_yhat_pairs(w, act, wts, ta.ravel(), nw.ravel())
    err = H.rel_err(Yi.cpu().numpy().ravel(), yhat)
    say(f"  fp32 max floored rel err {err:.3e}")
    assert err <= H.REL_TOL
    Yf = torch.empty_like(Yi)
    L.linear(Yf, engine="fp6")
    assert torch.equal(Yi, Yf)
    Bi = torch.empty((w.T, w.N), dtype=torch.bfloat16, device="cuda")
    Bf = torch.empty_like(Bi)
    L.linear(Bi, engine="int8")
    L.linear(Bf, engine="fp6")
    torch.cuda.synchronize()
    assert torch.equal(Bi.view(torch.int16), Bf.view(torch.int16))


@pytest.mark.parametrize("name", ["flux_up", "flux_down"])
def test_int8_engine_full_workload(name):
    """The int8 engine at the full FLUX shapes (the bench's --engine int8
    configuration): accumulators at sampled pairs against the oracle, and
    the bf16 output equal to the FP6 engine's bit for bit."""
    w = datagen.WORKLOADS[name]
    say(f"[int8 engine full] {w}")
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp)
    L.rotate_quant()
    Bi = torch.empty((w.T, w.N), dtype=torch.bfloat16, device="cuda")
    L.linear(Bi, engine="int8")
    L.linear(engine="fp6")
    torch.cuda.synchronize()
    assert torch.equal(Bi.view(torch.int16), L.Y.view(torch.int16))
    g = np.random.default_rng(3)
    ta = g.integers(0, w.T, 4096)
    nw = g.integers(0, w.N, 4096)
    rows = np.unique(ta)
    act = H.oracle_act(w, inp, rows)
    wts = H.oracle_weights(w, inp)
    idx = torch.from_numpy(ta).to("cuda") * w.N + torch.from_numpy(nw).to("cuda")
    acc = L.raw_acc(engine="int8").view(-1)[idx].cpu().numpy().astype(np.int64)
    ref = H.orc.int_gemm_pairs(act["codes"], w.Kq, wts["codes"], w.K, np.searchsorted(rows, ta), nw)
    assert np.array_equal(acc, ref)


@pytest.mark.parametrize("name,shape", [("flux_up_trdq", dict(T=70, K=1024, N=136)),
                                        ("flux_up", dict(T=100, K=1024, N=200, block=256))])
def test_timestep_set_parity(name, shape):
    """Time-step rotation sets ("TR-DQ" Eq.(10)): eight denoising steps in
    three groups, each group with its own rotation and its own folded
    weights (one layer W).  Every step's codes and outputs match the oracle
    with that step's rotation; the wrong group's weights would not."""
    w = datagen.WORKLOADS[name].with_shape(**shape)
    ins = datagen.make_timestep_inputs(w, 3)
    rots = [H.rotation_for(w, i) for i in ins]
    q = H.quant_for(w)
    steps = [0, 0, 1, 1, 1, 2, 2, 0]
    ws = H.rq.pack_weight_set(rots, steps, q, ins[0]["W"]).to_device("cuda")
    drots = [r.to_device("cuda") for r in rots]
    for t, g in enumerate(steps):
        inp = ins[g]
        say(f"[timestep set] {w.name} step {t} group {g}")
        L = H.GpuLayer(w, inp, y_dtype="f32")
        L.drot = drots[g]
        L.dw = ws.device_member(t)
        L.run()
        torch.cuda.synchronize()
        act = H.oracle_act(w, inp)
        check_act(w, L, act)
        wts = H.oracle_weights(w, inp)
        ta, nw = np.meshgrid(np.arange(w.T), np.arange(w.N), indexing="ij")
        yhat = H.oracle_yhat_pairs(w, act, wts, ta.ravel(), nw.ravel())
        err = H.rel_err(L.Y.cpu().numpy().ravel(), yhat)
        assert err <= H.REL_TOL, (t, err)
        if t == 2:   # another group's member does not reproduce this step
            L.dw = ws.device_member(0)
            L.linear()
            assert H.rel_err(L.Y.cpu().numpy().ravel(), yhat) > 1e-2


# TR-DQ's rotation with a workspace (tiled launches through fp32 buffers) and
# without (one pass, rows in LDS): the same codes and scales bit for bit, and
# the oracle's; symmetric and asymmetric, 4- and 8-bit, blocks 16 .. 256,
# ragged token counts
TRDQ_FORMS = [
    ("flux_up_trdq", dict(T=300, K=1024, N=40), "int4"),
    ("flux_up_trdq", dict(T=129, K=512, N=40, block=16, a_bits=4), "int4"),
    ("flux_up_trdq", dict(T=70, K=2048, N=40, block=32), "int4_asym"),
    ("flux_up_trdq", dict(T=257, K=1024, N=40, block=64, a_bits=4), "int4_asym"),
    ("flux_up_trdq", dict(T=9, K=16384, N=40, block=256), "int4"),
    ("flux_up_trdq_w6a6", dict(T=129, K=512, N=40, block=16), "int4"),
    ("flux_up_trdq_w6a6", dict(T=70, K=2048, N=40, block=32), "int4_asym"),
]


@pytest.mark.parametrize("name,shape,quant", TRDQ_FORMS,
                         ids=[f"{n}-{q}-{'-'.join(f'{k}{v}' for k, v in s.items())}" for n, s, q in TRDQ_FORMS])
def test_trdq_tiled_matches_one_pass(name, shape, quant):
    w = dataclasses.replace(datagen.WORKLOADS[name].with_shape(**shape), quant=quant)
    say(f"[trdq forms] {w}")
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, y_dtype="f32")
    assert L.ws is not None, "TR-DQ takes a workspace"
    L.rotate_quant()
    torch.cuda.synchronize()
    c_tiled, s_tiled = L.codes.clone(), L.scale.clone()
    check_act(w, L, H.oracle_act(w, inp))
    L.codes.fill_(0xA5)
    L.scale.fill_(-1.0)
    L.ws = None
    L.rotate_quant()
    torch.cuda.synchronize()
    assert torch.equal(L.codes, c_tiled), "one-pass and tiled codes differ"
    assert torch.equal(L.scale.view(torch.int32), s_tiled.view(torch.int32)), "scales differ"


def test_mxfp4_rounding_boundaries():
    """MXFP4 codes at the E2M1 grid's ties (to the even code), just off
    them, at saturation, and for values of either sign that round to zero
    (code 0, no sign): block 2, identity permutation, +1 signs, so each pair
    x0 = x1 = v / 2 rotates exactly to u = (v, 0).  Every 32-coordinate block
    holds +-6 2^k first, so its E8M0 exponent is k; rows use k = -3 .. 3."""
    w = datagen.WORKLOADS["flux_up_mxfp4"].with_shape(T=56, K=128, N=64, block=2)
    inp = datagen.make_inputs(w)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [0.0, 6.0, 7.0, 7.5, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]
    for t in ties:
        d = 2.0 ** (np.floor(np.log2(t)) - 5)
        vals += [t, t - d, t + d]
    vals += [1.0 / 128, 1.0 / 16, 0.2421875]          # round to 0
    vals = np.array(vals + [-v for v in vals], dtype=np.float64)
    u = np.zeros((w.T, w.K // 2))
    for t in range(w.T):
        k = t % 7 - 3
        row = np.roll(vals, t)[: w.K // 2]
        row[::16] = 6.0 if t % 2 == 0 else -6.0       # block maxima (16 pairs = 32 coordinates)
        u[t] = row * 2.0 ** k
    x = np.repeat(u / 2, 2, axis=1).astype(np.float32)
    assert np.array_equal(datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(x)), x)
    inp["X"] = datagen.f32_to_bf16_bits(x)
    inp["sign"] = np.ones(w.K, dtype=np.int8)
    inp["perm"] = np.arange(w.K, dtype=np.int32)
    say(f"[mxfp4 boundaries] {w}")
    L = H.GpuLayer(w, inp, codes="both")
    L.rotate_quant()
    torch.cuda.synchronize()
    act = H.oracle_act(w, inp)
    check_act(w, L, act)

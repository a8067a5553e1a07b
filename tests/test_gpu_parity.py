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
import sys

import numpy as np
import pytest

from rotated_w4a4_quantized_amd import datagen
from tests import _layer as H

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
    """Layer mode for the parity runs: RPBH INT4 layers write both code
    layouts and the GEMM reads the MMA copy."""
    return "both" if (w.rot == "rpbh" and w.quant in ("int4", "int4_asym")) else "canonical"


def check_act(w, L, act, rows=None):
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
    if L.codes_mma is not None:
        dec, top_clear = H.decode_codes_mma(L.codes_mma.cpu().numpy(), w.T, w.Kq)
        if rows is not None:
            dec = dec[rows]
        assert top_clear, "a codes_mma field has its top bits set"
        ref = H.unpack_codes(act["codes"])
        if asym:   # fields hold the unsigned codes: decoded as u - 8
            ref = (ref & 15) - 8
        bad = np.nonzero(np.any(dec != ref, axis=1))[0]
        assert bad.size == 0, f"codes_mma differs in {bad.size} tokens, first {bad[:5]}"
    if w.r:
        top = L.top.cpu().numpy().view(np.uint16)
        if rows is not None:
            top = top[rows]
        assert np.array_equal(top, act["top"])


SMALL = [
    ("tiny", dict(T=300, N=200)),
    ("tiny", dict(T=1, N=130, K=256, block=256)),
    ("flux_up", dict(T=257, K=3072, N=384)),
    ("flux_down", dict(T=131, K=12288, N=136)),
    ("video", dict(T=190, N=264)),
    ("pixart", dict(T=200, N=170)),
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
]


@pytest.mark.parametrize("name,shape", SMALL, ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in s.items())}"
                                                   for n, s in SMALL])
def test_small_full_parity(name, shape):
    w = datagen.WORKLOADS[name].with_shape(**shape)
    say(f"[parity small] {w}")
    inp = datagen.make_inputs(w)
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
    if w.quant in ("int4", "int4_asym"):
        ref = H.oracle_raw_acc(w, act, wts)
        acc = L.raw_acc().cpu().numpy().astype(np.int64)
        assert np.array_equal(acc, ref)
        if L.codes_mma is not None:
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


FULL = ["tiny", "flux_up", "flux_down", "video", "pixart", "flux_up_asym", "flux_down_asym", "video_w4"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_parity(name):
    w = datagen.WORKLOADS[name]
    say(f"[parity full] {w}")
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp, codes=mma_mode(w))
    L.run()
    torch.cuda.synchronize()
    g = np.random.default_rng(7)
    # every code and scale for the RPBH paths; a token sample for the dense
    # path, whose oracle rotation is a K x K fp32 chain per token
    rows = None if w.rot == "rpbh" else np.sort(g.choice(w.T, 512, replace=False))
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


def test_mma_codes_only_path():
    # the bench configuration: rq_rotate_quant writes only the MMA-layout
    # codes and the GEMM reads them; compared with a canonical-code run
    w = datagen.WORKLOADS["flux_down"].with_shape(T=300, K=2048, N=520, block=512)
    inp = datagen.make_inputs(w)
    A = H.GpuLayer(w, inp, y_dtype="f32", codes="mma")
    B = H.GpuLayer(w, inp, y_dtype="f32", codes="canonical")
    A.run()
    B.run()
    accA = A.raw_acc().cpu().numpy()
    accB = B.raw_acc().cpu().numpy()
    torch.cuda.synchronize()
    assert A.codes is None and np.array_equal(accA, accB)
    assert torch.equal(A.scale, B.scale) and torch.equal(A.Y, B.Y)



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

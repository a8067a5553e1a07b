"""Pins of the oracle's further formats and rotation, against what their
definitions fix independently of the oracle's code:

* MXFP4 (the FP4 variant: "DiRotQ" abstract, later version, NVFP4 on a
  Blackwell GPU; read as OCP MX v1.0 MXFP4, the format gfx950's scaled matrix
  cores take): E2M1 values derived from the bit fields, element rounding
  against IEEE round-to-nearest-even through numpy, block scales from their
  defining inequality, block-scaled dot products in exact rationals;
* 8-bit integer quantizers ("TR-DQ" section 3.1 Eq.(1)-(3) with b = 8, the
  W8A8 / W4A8 settings of its tables): brute-force nearest level, exact
  rational scales, and agreement with the pinned INT4 quantizers at b = 4;
* TR-DQ's runtime rotation (section 3.2 Eq.(8)-(10)): the fold invariant with
  exactly orthogonal blocks, the fp64 rotation against library matmuls, the
  fp32 chain order (hand-derived golden), and the zigzag permutation.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc
from rotated_w4a4_quantized_amd import datagen
from tests._golden import rows


# ---------------------------------------------------------------------------
# MXFP4
# ---------------------------------------------------------------------------

def e2m1_from_bits(code):
    """E2M1 value from its fields: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0.m x 2^0)."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * 0.5 * m
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


def test_e2m1_values_from_bit_fields():
    for c in range(16):
        assert orc.e2m1_value(c) == e2m1_from_bits(c), c
    # the positive magnitudes are ascending and the largest is 6 = 1.5 * 2^2
    mags = [e2m1_from_bits(c) for c in range(8)]
    assert mags == sorted(mags) and mags[-1] == 6.0


def rne_e2m1_numpy(x):
    """Nearest E2M1 value by IEEE rounding (numpy rint is round-half-even):
    below 1 the grid is multiples of 1/2; in [2^e, 2^(e+1)) (e = 0, 1, 2) it
    is multiples of 2^(e-1); magnitudes above 6 saturate."""
    a = abs(float(x))
    if a < 1.0:
        v = float(np.rint(a * 2.0)) / 2.0
    else:
        e = int(np.floor(np.log2(a)))
        step = 2.0 ** (e - 1)
        v = float(np.rint(a / step)) * step
    v = min(v, 6.0)
    return -v if (x < 0 and v != 0) else v


def test_e2m1_encode_matches_ieee_rounding():
    g = np.random.default_rng(0)
    xs = list(g.uniform(-8, 8, 4000)) + list(g.uniform(-1, 1, 2000))
    # every midpoint between adjacent magnitudes (ties), each value, a hair
    # either side, and saturation
    mags = [e2m1_from_bits(c) for c in range(8)]
    for a, b in zip(mags, mags[1:]):
        mid = (a + b) / 2
        xs += [mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, 9), a, -a, b]
    xs += [6.0, 6.5, 7.0, 7.999, 100.0, -7.0, 0.0, -0.0, 1e-30, -1e-30]
    for x in xs:
        c = orc.e2m1_encode(x)
        assert orc.e2m1_value(c) == rne_e2m1_numpy(x), (x, c)
        if orc.e2m1_value(c) == 0.0:
            assert c == 0, (x, c)           # zero is the positive code


@pytest.mark.parametrize("seed", range(4))
def test_mx_block_scale_inequality(seed):
    """The block exponent e is the one with 4 <= amax / 2^e < 8 (the largest
    element lands in E2M1's top binade [4, 6] or saturates), clamped at -127."""
    g = np.random.default_rng(seed)
    for amax in np.concatenate([np.exp(g.uniform(-60, 60, 500)), 2.0 ** np.arange(-40, 41)]):
        code = orc.mx_scale_code(float(amax))
        e = code - 127
        r = Fraction(float(amax)) / Fraction(2) ** e
        assert 4 <= r < 8, (amax, e)
    assert orc.mx_scale_code(0.0) == 0
    assert orc.mx_scale_code(2.0 ** -140) == 0       # clamped to 2^-127


def test_mxfp4_row_quantization():
    g = np.random.default_rng(3)
    K = 256
    u = (g.standard_normal(K) * np.exp(g.uniform(-3, 3, K))).astype(np.float32)
    u[32:64] = 0.0                                   # an all-zero block
    u[64] = np.float32(7.9)                          # saturating block element
    u[65:96] = np.float32(0.001)
    codes, sc = orc.quant_mxfp4_row(u)
    assert sc[1] == 0 and not codes[16:32].any()
    for c in range(K // 32):
        blk = u[32 * c:32 * c + 32].astype(np.float64)
        e = int(sc[c]) - 127
        if blk.any():
            assert e == orc.mx_scale_code(float(np.max(np.abs(blk)))) - 127
        for j in range(32):
            k = 32 * c + j
            code = (codes[k // 2] >> (4 * (k % 2))) & 15
            assert orc.e2m1_value(code) * 2.0 ** e == rne_e2m1_numpy(blk[j] / 2.0 ** e) * 2.0 ** e
    # dequantization error: within half a grid step, except saturation
    deq = np.array([orc.e2m1_value((codes[k // 2] >> (4 * (k % 2))) & 15) * 2.0 ** (int(sc[k // 32]) - 127)
                    for k in range(K)])
    for k in range(K):
        e = int(sc[k // 32]) - 127
        a = abs(float(u[k])) / 2.0 ** e
        step = 0.5 if a < 2 else (1.0 if a < 4 else 2.0)
        if a <= 6.0:
            assert abs(deq[k] - float(u[k])) <= step / 2 * 2.0 ** e
        else:
            assert deq[k] == 6.0 * 2.0 ** e * np.sign(u[k])


def test_mxfp4_f32_row_equals_f64_path():
    g = np.random.default_rng(4)
    u = (g.standard_normal(512) * 30).astype(np.float32)
    assert all(np.array_equal(a, b) for a, b in zip(orc.quant_mxfp4_row(u),
                                                     orc.quant_mxfp4_f64(u.astype(np.float64))))


def test_mx_dot_against_exact_rationals():
    g = np.random.default_rng(5)
    K, T, N = 128, 5, 6
    A = (g.standard_normal((T, K)) * np.exp(g.uniform(-4, 4, (T, K)))).astype(np.float32)
    W = g.standard_normal((N, K)) * 0.02
    act = [orc.quant_mxfp4_row(a) for a in A]
    wts = [orc.quant_mxfp4_f64(w) for w in W]
    ca = np.stack([c for c, _ in act]); sa = np.stack([s for _, s in act])
    cw = np.stack([c for c, _ in wts]); sw = np.stack([s for _, s in wts])
    ta, nw = np.meshgrid(np.arange(T), np.arange(N), indexing="ij")
    dot = orc.mx_dot_pairs(ca, sa, cw, sw, K, ta.ravel(), nw.ravel())

    def val(codes, sc, k):
        c = (int(codes[k // 2]) >> (4 * (k % 2))) & 15
        return Fraction(e2m1_from_bits(c)) * Fraction(2) ** (int(sc[k // 32]) - 127)

    for p, (t, n) in enumerate(zip(ta.ravel(), nw.ravel())):
        exact = sum(val(ca[t], sa[t], k) * val(cw[n], sw[n], k) for k in range(K))
        assert abs(Fraction(dot[p]) - exact) <= abs(exact) * Fraction(1, 2 ** 50), (t, n)
    assert np.array_equal(orc.yhat_mx(dot, 256), dot / 256)


# ---------------------------------------------------------------------------
# 8-bit integer quantizers and GEMM
# ---------------------------------------------------------------------------

def rne_argmin(m, lo, hi):
    """Brute force: the integer level in [lo, hi] nearest to m, ties to even."""
    best = None
    for k in range(lo, hi + 1):
        d = abs(Fraction(float(m)) - k)
        if best is None or d < best[0] or (d == best[0] and k % 2 == 0):
            best = (d, k)
    return best[1]


def is_nearest_f32(s, exact):
    s = np.float32(s)
    dn, up = np.nextafter(s, np.float32(-np.inf)), np.nextafter(s, np.float32(np.inf))
    d = abs(Fraction(float(s)) - exact)
    return d <= abs(Fraction(float(dn)) - exact) and d <= abs(Fraction(float(up)) - exact)


@pytest.mark.parametrize("qmax", [31, 127])
@pytest.mark.parametrize("seed", range(4))
def test_int8_activation_brute_force(seed, qmax):
    # qmax 127: 8-bit codes (W8A8, W4A8); 31: 6-bit codes (W6A6)
    g = np.random.default_rng(10 + seed)
    K = 64
    u = (g.standard_normal(K) * g.choice([1e-3, 1.0, 37.0])).astype(np.float32)
    q, s = orc.quant_sym_row(u, qmax=qmax)
    amax = Fraction(float(np.max(np.abs(u))))
    assert is_nearest_f32(s, amax / qmax)
    inv = np.float32(qmax) / np.float32(float(amax))
    assert is_nearest_f32(inv, Fraction(qmax) / amax)
    for j in range(K):
        assert q[j] == rne_argmin(np.float32(u[j]) * inv, -qmax, qmax), j
    assert abs(int(q[int(np.argmax(np.abs(u)))])) == qmax


def test_sym_quantizer_reduces_to_int4():
    g = np.random.default_rng(20)
    for r in (0, 32):
        u = (g.standard_normal(160) * 3).astype(np.float32)
        q8, s8 = orc.quant_sym_row(u, r=r, qmax=7)
        q4, s4 = orc.quant_int4_row(u, r=r)
        assert np.array_equal(q8, q4.astype(np.int16)) and s8 == s4
        q, s, z = orc.quant_asym_row(u, levels=15)
        qa, sa, za = orc.quant_int4_asym_row(u)
        assert np.array_equal(q, qa.astype(np.uint16)) and (s, z) == (sa, za)
    v = g.standard_normal(96)
    qw, sw = orc.quant_sym_wrow(v, qmax=7)
    q4, s4 = orc.quant_int4_wrow(v)
    assert np.array_equal(qw, q4.astype(np.int16)) and sw == s4


@pytest.mark.parametrize("levels", [63, 255])
@pytest.mark.parametrize("seed", range(3))
def test_asym8_activation_brute_force(seed, levels):
    # 255 levels: 8-bit codes; 63: 6-bit codes
    g = np.random.default_rng(30 + seed)
    K = 64
    u = (g.standard_normal(K) + g.choice([0.0, 2.5])).astype(np.float32)
    q, s, z = orc.quant_asym_row(u, levels=levels)
    lo, hi = np.float32(u.min()), np.float32(u.max())
    d = np.float32(hi - lo)
    assert is_nearest_f32(s, Fraction(float(d)) / levels)
    inv = np.float32(levels) / d
    zi = -round(Fraction(float(np.float32(lo * inv))))      # Fraction rounds half to even
    assert z == float(min(max(zi, 0), levels)) and np.float32(z).view(np.uint32) == np.float32(abs(z)).view(np.uint32)
    for j in range(K):
        ref = min(max(round(Fraction(float(np.float32(u[j]) * inv))) + int(z), 0), levels)
        assert q[j] == ref, j
    assert q.min() == 0 if zi >= 0 else True


@pytest.mark.parametrize("qmax", [31, 127])
def test_int8_weight_row_brute_force(qmax):
    g = np.random.default_rng(40)
    v = g.standard_normal(80) * 0.05
    q, s = orc.quant_sym_wrow(v, qmax=qmax)
    amax = float(np.max(np.abs(v)))
    assert s == np.float32(amax / qmax)
    inv = qmax / amax
    for j in range(v.size):
        assert q[j] == rne_argmin(v[j] * inv, -qmax, qmax)


def test_gemm_codes_against_numpy():
    g = np.random.default_rng(50)
    T, N, K = 7, 9, 96
    qa8 = g.integers(-127, 128, (T, K))
    ua8 = g.integers(0, 256, (T, K))
    qa6 = g.integers(-31, 32, (T, K))
    ua6 = g.integers(0, 64, (T, K))
    qa4 = g.integers(-7, 8, (T, K))
    qw8 = g.integers(-127, 128, (N, K))
    qw6 = g.integers(-31, 32, (N, K))
    qw4 = g.integers(-7, 8, (N, K))
    ta, nw = np.meshgrid(np.arange(T), np.arange(N), indexing="ij")
    ta, nw = ta.ravel(), nw.ravel()

    def nib(q):
        q = (q & 15).astype(np.uint8)
        return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)

    # 6-bit codes sit one per byte, two's complement in the byte when signed
    cases = [(qa8.astype(np.int8).view(np.uint8), 8, True, qa8),
             (ua8.astype(np.uint8), 8, False, ua8),
             (qa6.astype(np.int8).view(np.uint8), 6, True, qa6),
             (ua6.astype(np.uint8), 6, False, ua6),
             (nib(qa4), 4, True, qa4)]
    for ca, ab, sg, qa in cases:
        for cw, wb, qw in ((qw8.astype(np.int8).view(np.uint8), 8, qw8),
                           (qw6.astype(np.int8).view(np.uint8), 6, qw6), (nib(qw4), 4, qw4)):
            acc = orc.gemm_codes_pairs(ca, ab, sg, K, cw, wb, K, ta, nw)
            assert np.array_equal(acc, (qa @ qw.T).ravel())


# ---------------------------------------------------------------------------
# TR-DQ rotation
# ---------------------------------------------------------------------------

def block_diag(Rb):
    nb, b, _ = Rb.shape
    M = np.zeros((nb * b, nb * b))
    for c in range(nb):
        M[c * b:(c + 1) * b, c * b:(c + 1) * b] = Rb[c]
    return M


def perm_matrix(perm):
    K = perm.size
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0      # (z P)[j] = z[perm[j]]
    return P


def signed_perm_blocks(nb, b, g):
    out = np.zeros((nb, b, b), np.float32)
    for c in range(nb):
        out[c][np.arange(b), g.permutation(b)] = g.choice([-1.0, 1.0], b)
    return out


def test_trdq_fold_invariant_exact():
    """With exactly orthogonal blocks (signed permutations), power-of-two
    smoothing and integer data, u . v = x . w exactly (Eq.(9):
    (X Delta R1 P R2)(R2^T P^T R1^T Delta^-1 W) = X W)."""
    g = np.random.default_rng(60)
    K, b = 64, 16
    R1 = signed_perm_blocks(K // b, b, g)
    R2 = signed_perm_blocks(K // b, b, g)
    perm = g.permutation(K).astype(np.int32)
    m = (2.0 ** g.integers(-3, 4, K)).astype(np.float32)
    for _ in range(10):
        x = g.integers(-20, 21, K).astype(np.float32)
        w = g.integers(-20, 21, K).astype(np.float64)
        u = orc.trdq_row_f32(x, b, m, R1, perm, R2)
        v = orc.trdq_row_f64(w, b, m, R1, perm, R2)
        assert Fraction(float(np.dot(u.astype(np.float64), v))) == Fraction(int(np.dot(x.astype(np.int64), w.astype(np.int64))))


def test_trdq_rotation_against_library_matmul():
    w_ = datagen.WORKLOADS["flux_up_trdq"].with_shape(T=8, K=512, N=16)
    inp = datagen.make_inputs(w_)
    b = w_.block
    M = block_diag(inp["R1"].astype(np.float64)) @ perm_matrix(inp["perm"]) @ \
        block_diag(inp["R2"].astype(np.float64))
    g = np.random.default_rng(61)
    for _ in range(4):
        w = g.standard_normal(w_.K) * 0.02
        v = orc.trdq_row_f64(w, b, inp["m"], inp["R1"], inp["perm"], inp["R2"])
        ref = (w / inp["m"].astype(np.float64)) @ M
        assert np.max(np.abs(v - ref)) <= 1e-12 * np.max(np.abs(ref))
        x = inp["Xf"][_]
        u = orc.trdq_row_f32(x, b, inp["m"], inp["R1"], inp["perm"], inp["R2"])
        refx = (x.astype(np.float64) * inp["m"].astype(np.float64)) @ M
        # two fp32 chains of b terms: well inside 2 b 2^-24 of the magnitudes summed
        bound = 2 * b * 2.0 ** -24 * (np.abs(x * inp["m"]) @ np.abs(M)).max() * 4
        assert np.max(np.abs(u - refx)) <= bound
    # the blocks are orthogonal to fp32 rounding, so the fold keeps x . w
    x = inp["Xf"][0].astype(np.float64)
    w = g.standard_normal(w_.K)
    u = orc.trdq_row_f64(x * inp["m"].astype(np.float64) ** 2, b, inp["m"], inp["R1"], inp["perm"], inp["R2"])
    v = orc.trdq_row_f64(w, b, inp["m"], inp["R1"], inp["perm"], inp["R2"])
    assert abs(np.dot(u, v) - np.dot(x, w)) <= 1e-5 * np.linalg.norm(x) * np.linalg.norm(w)


def test_trdq_chain_order_golden():
    for b, xs, ms, u0 in rows("trdq_chain_order.txt"):
        b = int(b)
        x = np.array([float(t) for t in xs.split()], np.float32)
        m = np.array([float(t) for t in ms.split()], np.float32)
        R1 = np.zeros((1, b, b), np.float32)
        R1[0, :, 0] = 1.0
        R2 = np.eye(b, dtype=np.float32)[None]
        u = orc.trdq_row_f32(x, b, m, R1, np.arange(b, dtype=np.int32), R2)
        assert u[0] == np.float32(float(u0)), (u[0], u0)


def test_zigzag_permutation():
    b, nb = 4, 3
    cm = np.array([9, 1, 5, 12, 3, 7, 11, 2, 8, 4, 10, 6], float)   # ranks by value
    perm = datagen.zigzag_permutation(cm, b)
    # descending order of channels: 3(12) 6(11) 10(10) 0(9) 8(8) 5(7) 11(6) 2(5) 9(4) 4(3) 7(2) 1(1)
    # dealt 0 1 2 | 2 1 0 | 0 1 2 | 2 1 0
    assert perm.tolist() == [3, 5, 11, 1, 6, 8, 2, 7, 10, 0, 9, 4]
    assert sorted(perm.tolist()) == list(range(12))

"""Pins of the oracle's quantizers, packing and integer GEMM.

Quantizer: "TR-DQ" section 3.1, Eq.(1)-(2) (nearest rounding onto 2^b levels
with a scale from the extremes), made symmetric with a zero point of 0;
per-token activations, per-output-channel weights.  Codebook quantizer and
normalized basis: "OrbitQuant" abstract.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc
from tests._golden import rows


def f32(v):
    return np.float32(v)


def rne_argmin(m, lo=-7, hi=7):
    """Brute force: the integer level in [lo, hi] nearest to m, ties to even."""
    best = None
    for k in range(lo, hi + 1):
        d = abs(Fraction(float(m)) - k)
        if best is None or d < best[0] or (d == best[0] and k % 2 == 0):
            best = (d, k)
    return best[1]


def is_nearest_f32(s, exact):
    """s is an fp32 value nearest to the rational `exact` (ties either way)."""
    s = np.float32(s)
    dn = np.nextafter(s, np.float32(-np.inf))
    up = np.nextafter(s, np.float32(np.inf))
    d = abs(Fraction(float(s)) - exact)
    return d <= abs(Fraction(float(dn)) - exact) and d <= abs(Fraction(float(up)) - exact)


@pytest.mark.parametrize("seed", range(6))
def test_int4_activation_brute_force(seed):
    g = np.random.default_rng(seed)
    K = 96
    u = (g.standard_normal(K) * g.choice([1e-3, 1.0, 37.0])).astype(np.float32)
    if seed == 5:   # plant exact ties: levels k + 1/2 after scaling by inv
        u[:8] = np.float32(u[0])
    q, s = orc.quant_int4_row(u)
    amax = Fraction(float(np.max(np.abs(u))))
    assert is_nearest_f32(s, amax / 7)
    inv = np.float32(7.0) / np.float32(float(amax))   # numpy fp32 divide: correctly rounded
    assert is_nearest_f32(inv, Fraction(7) / amax)
    for j in range(K):
        m = np.float32(u[j]) * inv                      # one fp32 product
        assert q[j] == rne_argmin(m), (j, u[j], m, q[j])
    # the largest element lands on +-7
    j = int(np.argmax(np.abs(u)))
    assert abs(int(q[j])) == 7


def test_int4_ties_to_even():
    # u = [7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5]: amax 7, inv = 1 exactly
    u = np.array([7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5], np.float32)
    q, s = orc.quant_int4_row(u)
    assert s == np.float32(1.0)
    assert list(q) == [7, 0, 2, 2, 0, -2, -2, 4]


def test_int4_zero_row_and_topr():
    q, s = orc.quant_int4_row(np.zeros(64, np.float32))
    assert s == 0 and not q.any()
    # top-r coordinates are excluded from the range and the codes
    u = np.zeros(64, np.float32)
    u[:4] = 1000.0
    u[4] = 7.0
    u[5] = -3.0
    q, s = orc.quant_int4_row(u, r=4)
    assert q.size == 60 and s == np.float32(1.0) and q[0] == 7 and q[1] == -3


@pytest.mark.parametrize("seed", range(4))
def test_int4_weight_brute_force(seed):
    g = np.random.default_rng(100 + seed)
    v = g.standard_normal(80) * 0.3
    q, s = orc.quant_int4_wrow(v)
    amax = Fraction(float(np.max(np.abs(v))))
    # s_w is the fp32 rounding of the fp64 quotient amax / 7
    assert s == np.float32(float(amax) / 7.0)
    inv = 7.0 / float(amax)
    for j in range(v.size):
        assert q[j] == rne_argmin(v[j] * inv)


def test_pack_golden_and_round_trip():
    for codes, hexes in rows("pack_nibbles.txt"):
        q = np.array([int(c) for c in codes.split()], np.int8)
        want = np.array([int(h, 16) for h in hexes.split()], np.uint8)
        got = orc.pack_nibbles(q)
        assert np.array_equal(got, want)
        assert np.array_equal(orc.unpack_nibbles(got, q.size), q)
    g = np.random.default_rng(0)
    q = g.integers(-8, 8, 1000).astype(np.int8)
    assert np.array_equal(orc.unpack_nibbles(orc.pack_nibbles(q), 1000), q)
    idx = g.integers(0, 4, 1000).astype(np.uint8)
    assert np.array_equal(orc.unpack_crumbs(orc.pack_crumbs(idx), 1000), idx)
    assert orc.pack_crumbs(np.array([1, 2, 3, 0], np.uint8))[0] == 0b00111001


def test_int_gemm_matches_library_matmul():
    g = np.random.default_rng(1)
    T, N, K = 37, 29, 96
    qa = g.integers(-7, 8, (T, K)).astype(np.int8)
    qw = g.integers(-7, 8, (N, K + 32)).astype(np.int8)
    pa = np.stack([orc.pack_nibbles(r) for r in qa])
    pw = np.stack([orc.pack_nibbles(r) for r in qw])
    for koff in (0, 32):
        acc = orc.int_gemm(pa, K, pw, K + 32, koff)
        ref = qa.astype(np.int64) @ qw[:, koff:koff + K].astype(np.int64).T
        assert np.array_equal(acc, ref)
        ta = g.integers(0, T, 50)
        nw = g.integers(0, N, 50)
        assert np.array_equal(orc.int_gemm_pairs(pa, K, pw, K + 32, ta, nw, koff), ref[ta, nw])
    # bound that makes int32 accumulation safe: |acc| <= 49 K
    assert np.abs(orc.int_gemm(np.full((1, K // 2), 0x99, np.uint8), K,
                               np.full((1, K // 2), 0x99, np.uint8), K)).max() == 49 * K


def test_bf16_rounding_of_top_coefficients():
    # bf16 keeps the top 16 bits with round-half-to-even on the rest
    cases = {1.0: 0x3F80, 1.00390625: 0x3F80, 1.01171875: 0x3F82, -2.5: 0xC020,
             3.0e38: 0x7F62, 1.0078125: 0x3F81}
    for v, h in cases.items():
        assert orc.f32_to_bf16(np.float32(v))[0] == h, v
    # half-way points go to the even neighbour
    assert orc.f32_to_bf16(np.float32(1.0 + 2 ** -8))[0] == 0x3F80
    assert orc.f32_to_bf16(np.float32(1.0 + 3 * 2 ** -8))[0] == 0x3F82


def _exact_sq_sum(u):
    return sum(Fraction(float(x)) ** 2 for x in u)


@pytest.mark.parametrize("seed", range(4))
def test_norm_grid_exact_bound_and_order_free(seed):
    g = np.random.default_rng(seed)
    K = 512
    u = (g.standard_normal(K) * (10.0 ** g.uniform(-3, 3))).astype(np.float32)
    d = orc.norm2_grid(u)
    M = float(np.max(np.abs(u)))
    E = int(np.floor(np.log2(M)))
    while 2.0 ** E > M:
        E -= 1
    while 2.0 ** (E + 1) <= M:
        E += 1
    exact = _exact_sq_sum(u)
    # each of the K grid roundings is at most half a grid step 2^(2E-36)
    assert abs(Fraction(d) - exact) <= K * Fraction(2) ** (2 * E - 36) / 2
    # d is a multiple of the grid step, hence order-free
    for _ in range(3):
        assert orc.norm2_grid(g.permutation(u)) == d


def test_norm_grid_zero_row():
    assert orc.norm2_grid(np.zeros(16, np.float32)) == 0.0
    idx, sig = orc.quant_lloydmax_row(np.zeros(16, np.float32), orc.codebook_bf16(16))
    assert sig == 0 and not idx.any()


def _nearest_level(v, levels):
    """Brute force: index of the nearest level, ties to the lower index."""
    best = None
    for i, c in enumerate(levels):
        d = abs(Fraction(float(v)) - Fraction(float(c)))
        if best is None or d < best[0]:
            best = (d, i)
    return best[1]


@pytest.mark.parametrize("seed", range(3))
def test_codebook_activation_brute_force(seed):
    g = np.random.default_rng(seed)
    K = 256
    levels = orc.codebook_bf16(16)
    u = (g.standard_normal(K) * 3.0).astype(np.float32)
    idx, sigma = orc.quant_lloydmax_row(u, levels)
    d = orc.norm2_grid(u)
    # the normalizing gain: fp32 rounding of the fp64 value sqrt(K / d)
    gain = np.float32(np.sqrt(K / d))
    for j in range(K):
        v = np.float32(u[j]) * gain
        assert idx[j] == _nearest_level(v, levels)
    assert sigma == np.float32(np.sqrt(d / K))
    # sigma * gain ~ 1 and the normalized vector has squared norm ~ K
    vv = (u * gain).astype(np.float64)
    assert abs(vv @ vv / K - 1.0) < 1e-6


def test_codebook_ties_go_to_lower_level():
    levels = np.array([-1.5, -0.5, 0.5, 1.5], np.float32)
    # K = 4, u chosen so the gain is exactly 1: |u|^2 = 4
    u = np.array([1.0, -1.0, 1.0, -1.0], np.float32)
    idx, sigma = orc.quant_lloydmax_row(u, levels)
    # v = +-1 is exactly the midpoint of (0.5, 1.5) / (-1.5, -0.5): lower index
    assert list(idx) == [2, 0, 2, 0] and sigma == np.float32(1.0)
    u = np.array([2.0, 0.0, 0.0, 0.0], np.float32)     # |u|^2 = 4, v = 2, 0, 0, 0
    idx, _ = orc.quant_lloydmax_row(u, levels)
    assert list(idx) == [3, 1, 1, 1]                   # 0 is the midpoint of (-0.5, 0.5)


@pytest.mark.parametrize("L", [4, 16])
def test_codebook_weight_row(L):
    g = np.random.default_rng(9)
    K = 128
    levels = orc.codebook_bf16(L)
    v = g.standard_normal(K) * 0.05
    idx, tau = orc.quant_lloydmax_wrow(v, levels)
    nrm = np.sqrt(np.sum(v * v))
    wh = v * (np.sqrt(K) / nrm)
    assert all(idx[k] == _nearest_level(wh[k], levels) for k in range(K))
    assert abs(float(tau) - nrm / np.sqrt(K)) <= 1e-7 * nrm / np.sqrt(K)


# ---------------------------------------------------------------------------
# asymmetric per-token INT4 ("TR-DQ" section 3.1, Eq.(1)-(3): codes
# clamp(round(X / s) + z, 0, 15), s = (max - min) / 15, zero point z; the
# sign of Eq.(3) read so that the minimum lands on code 0)
# ---------------------------------------------------------------------------

def asym_brute(u):
    """Independent check of one row: s and 1/s correctly rounded from the fp32
    range, z the nearest integer to -min/s (clamped to [0, 15]), every code
    the level k in [0, 15] nearest to fl32(u inv) + z by exhaustive search
    (ties to k - z even, i.e. nearest-even on the unshifted value)."""
    lo, hi = np.float32(np.min(u)), np.float32(np.max(u))
    d = np.float32(hi - lo)
    inv = np.float32(15.0) / d
    zl = np.float32(lo * inv)
    f = Fraction(float(zl))
    k0 = f.numerator // f.denominator                    # floor
    k = k0 if (f - k0 < Fraction(1, 2) or (f - k0 == Fraction(1, 2) and k0 % 2 == 0)) else k0 + 1
    z = min(max(-k, 0), 15)
    codes = []
    for x in u:
        m = np.float32(np.float32(x) * inv)
        best = None
        for k in range(16):
            dist = abs(Fraction(float(m)) + z - k)
            if best is None or dist < best[0] or (dist == best[0] and (k - z) % 2 == 0):
                best = (dist, k)
        codes.append(best[1])
    return np.array(codes), d, z


@pytest.mark.parametrize("seed", range(5))
def test_int4_asym_brute_force(seed):
    g = np.random.default_rng(100 + seed)
    K = 64
    u = (g.standard_normal(K) * g.choice([1e-3, 1.0, 23.0]) + (0.3 if seed == 3 else 0.0)).astype(np.float32)
    if seed == 4:   # plant values that scale to exact half-levels
        u[0], u[1] = np.float32(-1.0), np.float32(2.0)
        u[2:8] = np.float32(0.5)
    q, s, z = orc.quant_int4_asym_row(u)
    ref, d, zref = asym_brute(u)
    assert is_nearest_f32(s, Fraction(float(d)) / 15)
    assert z == zref
    assert np.array_equal(q.astype(np.int64), ref)


def test_int4_asym_hand_example():
    # u = [-1, 0, 0.5, 2]: range 3, s = 0.2, 1/s = 5, z = -round(-5) = 5;
    # levels round([-5, 0, 2.5, 10]) + 5 = [0, 5, 7 (2.5 -> 2, even), 15]
    q, s, z = orc.quant_int4_asym_row(np.array([-1.0, 0.0, 0.5, 2.0], np.float32))
    assert list(q) == [0, 5, 7, 15]
    assert z == 5.0 and s == np.float32(3.0) / np.float32(15.0)


@pytest.mark.parametrize("seed", range(4))
def test_int4_asym_extremes_and_error_bound(seed):
    g = np.random.default_rng(200 + seed)
    u = (g.standard_normal(4096) * 3.0).astype(np.float32)
    q, s, z = orc.quant_int4_asym_row(u)
    assert q.min() >= 0 and q.max() <= 15
    assert q[np.argmin(u)] == 0          # min X lands on code 0 (0 is inside [min, max])
    assert q[np.argmax(u)] >= 14          # max X on the top level (or one below at a tie)
    err = np.abs(s * (q.astype(np.float64) - z) - u.astype(np.float64))
    # nearest rounding: half a step, plus fp32 error of u * inv; the clamped
    # top code may be one step off
    bound = 0.5 * float(s) + 4e-7 * float(np.max(np.abs(u)))
    assert np.mean(err <= bound) > 0.999
    assert np.all(err <= 1.0001 * float(s))


def test_int4_asym_degenerate_rows():
    for u in (np.zeros(32, np.float32), np.full(32, 2.5, np.float32)):
        q, s, z = orc.quant_int4_asym_row(u)
        assert not q.any() and s == 0 and z == 0
    # all-positive row: the zero point clamps to 0 and codes still span [0, 15]
    u = np.linspace(1.0, 4.0, 64, dtype=np.float32)
    q, s, z = orc.quant_int4_asym_row(u)
    assert z == 0 and q.max() == 15


def test_asym_gemm_and_output_identity():
    g = np.random.default_rng(7)
    T, N, K, b = 5, 6, 64, 32
    ua = g.integers(0, 16, (T, K))
    qw = g.integers(-7, 8, (N, K))
    pa = orc.pack_nibbles((ua - 16 * (ua >= 8)).astype(np.int8))
    pw = orc.pack_nibbles(qw.astype(np.int8))
    ta, nw = np.repeat(np.arange(T), N), np.tile(np.arange(N), T)
    acc = orc.asym_gemm_pairs(pa.reshape(T, K // 2), pw.reshape(N, K // 2), K, ta, nw)
    assert np.array_equal(acc.reshape(T, N), ua @ qw.T)
    s_a, z_a = g.random(T).astype(np.float32), g.integers(0, 16, T).astype(np.float32)
    s_w = g.random(N).astype(np.float32)
    y = orc.yhat_int4_asym(s_a[ta], z_a[ta], s_w[nw], acc, qw.sum(1)[nw], b)
    direct = ((s_a[:, None] * (ua - z_a[:, None])) @ (s_w[:, None] * qw).T) / b
    assert np.allclose(y.reshape(T, N), direct, rtol=1e-12, atol=1e-12)


def test_codebook_weight_book_of_16_levels_packs_nibbles():
    # a 16-level weight book (OrbitQuant's W4A4 setting) stores one 4-bit
    # index per coordinate, two per byte, low nibble = even coordinate; the
    # codebook dot product reads it back: checked against a direct sum over
    # the nearest-level indices of each row
    g = np.random.default_rng(21)
    N, K = 6, 64
    W = g.standard_normal((N, K)).astype(np.float32)
    sign = np.ones(K, np.int8)
    perm = np.arange(K, dtype=np.int32)
    lv16 = orc.codebook_bf16(16)
    out = orc.weight_rows(W, rot_kind=0, b=2, sign=sign, perm=perm, q_kind=1, levels=lv16)
    assert out["codes"].shape == (N, K // 2)
    idx = out["q"].astype(np.int64)
    assert idx.min() >= 0 and idx.max() <= 15
    assert np.array_equal(out["codes"], (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8))
    # activations: one row of 4-bit indices
    ia = g.integers(0, 16, (3, K))
    codes_a = (ia[:, 0::2] | (ia[:, 1::2] << 4)).astype(np.uint8)
    a_lv = orc.codebook_bf16(16)
    ta, nw = np.meshgrid(np.arange(3), np.arange(N), indexing="ij")
    dot = orc.codebook_dot_pairs(codes_a, out["codes"], K, a_lv, lv16, ta.ravel(), nw.ravel())
    ref = [sum(float(a_lv[ia[t, k]]) * float(lv16[idx[n, k]]) for k in range(K))
           for t, n in zip(ta.ravel(), nw.ravel())]
    assert np.allclose(dot, ref, rtol=0, atol=1e-12)

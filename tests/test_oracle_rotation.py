"""Pins of the oracle's rotations against what the pages and mathematics fix.

RPBH: "OrbitQuant" abstract (randomized permuted block-Hadamard rotation);
block structure: "TR-DQ" section 3.2, Eq.(8) (2^n x 2^n blocks, C_in / 2^n of
them); orthogonality and the fold: "TR-DQ" Eq.(9) and the OrbitQuant abstract
(the rotation absorbed into the weights cancels inside the layer).
Dense PCA basis: "DiRotQ" abstract.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from tests._golden import rows


def sylvester(b):
    i = np.arange(b)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def test_sylvester_h4_golden():
    H = np.array([[int(v) for v in r[0].split()] for r in rows("sylvester_h4.txt")], np.int64)
    assert np.array_equal(H, sylvester(4))


@pytest.mark.parametrize("b", [2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_hadamard_orthogonal_exact(b):
    H = sylvester(b)
    assert np.array_equal(H @ H.T, b * np.eye(b, dtype=np.int64))


@pytest.mark.parametrize("b", [2, 4, 8, 32, 128, 512])
def test_fwht_equals_explicit_matrix_on_integers(b):
    # small integers: every partial sum is an integer below 2^24, so fp32 is
    # exact and the butterfly network must reproduce x . H_b bit for bit
    g = np.random.default_rng(b)
    K = 3 * b
    x = g.integers(-1000, 1001, size=K).astype(np.float32)
    y = orc.rpbh_row_f32(x, b, np.ones(K, np.int8), np.arange(K, dtype=np.int32))
    H = sylvester(b)
    ref = np.concatenate([x[c:c + b].astype(np.int64) @ H for c in range(0, K, b)])
    assert np.array_equal(y.astype(np.int64), ref)
    assert np.array_equal(y, ref.astype(np.float32))


def test_fwht_stage_order_golden():
    for b, xs, ys in rows("fwht_stage_order.txt"):
        b = int(b)
        x = np.array([float(v) for v in xs.split()], np.float32)
        want = np.array([float(v) for v in ys.split()], np.float32)
        got = orc.rpbh_row_f32(x, b, np.ones(x.size, np.int8), np.arange(x.size, dtype=np.int32))
        assert np.array_equal(got, want), (got, want)


@pytest.mark.parametrize("b", [128, 256, 512])
def test_fwht_fp32_within_error_bound(b):
    # each output is log2(b) levels of fp32 additions of partial sums:
    # |err| <= log2(b) * 2^-24 * sum_j |y_j| (first-order bound)
    g = np.random.default_rng(7 + b)
    K = 2 * b
    x = g.standard_normal(K).astype(np.float32)
    sign = np.where(g.integers(0, 2, K) == 1, 1, -1).astype(np.int8)
    perm = g.permutation(K).astype(np.int32)
    y32 = orc.rpbh_row_f32(x, b, sign, perm)
    ys = sign.astype(np.float64) * x.astype(np.float64)[perm]
    H = sylvester(b).astype(np.float64)
    exact = np.concatenate([ys[c:c + b] @ H for c in range(0, K, b)])
    l1 = np.concatenate([np.full(b, np.abs(ys[c:c + b]).sum()) for c in range(0, K, b)])
    bound = np.log2(b) * 2.0 ** -24 * l1 * 1.0001
    assert np.all(np.abs(y32.astype(np.float64) - exact) <= bound)


@pytest.mark.parametrize("b,m", [(128, 3), (256, 2), (512, 2)])
def test_rpbh_matrix_orthogonal(b, m):
    # the matrix of the oracle's fp64 RPBH (rows = images of the unit vectors)
    # times its transpose is b * I exactly: a permutation, a sign flip and a
    # Sylvester block are each orthogonal up to the factor b
    K = b * m
    sign, perm = np.where(np.random.default_rng(b).integers(0, 2, K) == 1, 1, -1).astype(np.int8), \
        np.random.default_rng(b + 1).permutation(K).astype(np.int32)
    M = np.stack([orc.rpbh_row_f64(np.eye(K)[i], b, sign, perm) for i in range(K)])
    assert np.array_equal(M @ M.T, b * np.eye(K))
    # and every row has entries +-1 only, inside exactly one block
    assert np.all(np.abs(M).sum(axis=1) == b)


def test_rpbh_permutation_and_sign_semantics():
    # y[j] = sign[j] * x[perm[j]] before the butterflies; with b = 2 the block
    # transform of a pair (p, q) is (p + q, p - q)
    x = np.array([10, 20, 30, 40], np.float32)
    perm = np.array([3, 0, 2, 1], np.int32)
    sign = np.array([1, -1, 1, -1], np.int8)
    y = orc.rpbh_row_f32(x, 2, sign, perm)
    pre = np.array([40, -10, 30, -20], np.float32)
    assert np.array_equal(y, np.array([pre[0] + pre[1], pre[0] - pre[1],
                                       pre[2] + pre[3], pre[2] - pre[3]], np.float32))


def test_rpbh_one_hot_block_pattern():
    # a one-hot token lands, after sign and permutation, in one block, where
    # the Hadamard spreads it evenly: all |u| equal inside that block, zero
    # elsewhere
    b, K = 64, 256
    sign, perm = np.ones(K, np.int8), np.random.default_rng(3).permutation(K).astype(np.int32)
    x = np.zeros(K, np.float32)
    x[17] = 3.0
    u = orc.rpbh_row_f32(x, b, sign, perm)
    j = int(np.where(perm == 17)[0][0])
    c = (j // b) * b
    assert np.all(np.abs(u[c:c + b]) == 3.0)
    assert np.count_nonzero(u) == b


@pytest.mark.parametrize("b", [128, 256])
def test_fold_invariant_rpbh(b):
    # TR-DQ Eq.(9): (x R)(R^T w) = x w.  With the unnormalized block
    # Hadamard the rotated dot product is b * (x . w); exact on integers,
    # 1e-12 relative on Gaussians (fp64)
    K = 4 * b
    g = np.random.default_rng(b)
    sign = np.where(g.integers(0, 2, K) == 1, 1, -1).astype(np.int8)
    perm = g.permutation(K).astype(np.int32)
    xi = g.integers(-50, 51, K).astype(np.float64)
    wi = g.integers(-50, 51, K).astype(np.float64)
    assert orc.rpbh_row_f64(xi, b, sign, perm) @ orc.rpbh_row_f64(wi, b, sign, perm) == b * (xi @ wi)
    x = g.standard_normal(K)
    w = g.standard_normal(K)
    lhs = orc.rpbh_row_f64(x, b, sign, perm) @ orc.rpbh_row_f64(w, b, sign, perm)
    assert abs(lhs - b * (x @ w)) <= 1e-12 * b * np.abs(x) @ np.abs(w)


def test_fold_invariant_dense():
    # an fp64-orthogonal basis rounded to fp32: (x R)(w R)^T equals
    # x (R R^T) w^T (evaluated with a library matmul) to fp64 accuracy, and
    # R R^T is the identity to fp32 accuracy
    K = 96
    g = np.random.default_rng(11)
    Q, _ = np.linalg.qr(g.standard_normal((K, K)))
    R = Q.astype(np.float32)
    x = g.standard_normal(K)
    w = g.standard_normal(K)
    xr = orc.dense_row_f64(x, R)
    wr = orc.dense_row_f64(w, R)
    R64 = R.astype(np.float64)
    assert abs(xr @ wr - x @ (R64 @ R64.T) @ w) <= 1e-12 * np.abs(x) @ np.abs(w) * K
    assert np.max(np.abs(R64 @ R64.T - np.eye(K))) < 1e-6
    assert abs(xr @ wr - x @ w) < 1e-5 * np.abs(x) @ np.abs(w)


def test_dense_chain_golden():
    for K, xs, Rs, us in rows("dense_chain_order.txt"):
        K = int(K)
        x = np.array([float(v) for v in xs.split()], np.float32)
        R = np.array([float(v) for v in Rs.split()], np.float32).reshape(K, K)
        want = np.array([float(v) for v in us.split()], np.float32)
        assert np.array_equal(orc.dense_row_f32(x, R), want)


def test_dense_special_cases():
    K = 64
    g = np.random.default_rng(5)
    x = g.standard_normal(K).astype(np.float32)
    assert np.array_equal(orc.dense_row_f32(x, np.eye(K, dtype=np.float32)), x)
    p = g.permutation(K)
    P = np.eye(K, dtype=np.float32)[:, p]          # column j = e_{p[j]}
    assert np.array_equal(orc.dense_row_f32(x, P), x[p])
    # fp32 chain within K * 2^-24 * sum |x_k R_kj| of the exact product
    R = g.standard_normal((K, K)).astype(np.float32)
    exact = x.astype(np.float64) @ R.astype(np.float64)
    bound = K * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(R.astype(np.float64)))
    assert np.all(np.abs(orc.dense_row_f32(x, R) - exact) <= bound)

"""Pins of the lattice-encoder oracle (oracle/lq_codebook.py) to facts fixed
outside it: the Gaussian-source table of the LiftQuant notes, closed forms,
a textbook quantiser, and brute force written as plain loops."""
import itertools
import math
import os

import numpy as np
import pytest

from oracle import lq_codebook as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _haar(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))[None, :]


def _table_rows():
    with open(os.path.join(GOLDEN, "info_mse.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, bits, mse, info = line.split()
            yield code, float(mse), float(info)


def test_info_matches_gaussian_table():
    """Info = -1/2 log2(MSE) reproduces the table's Info column from its MSE
    column within the printed rounding (MSE to 3 decimals, Info to 2); the
    LQ-32/16 row is 0.01 off as printed."""
    rows = list(_table_rows())
    assert len(rows) == 8
    for code, mse, info in rows:
        lo, hi = C.info_bits(mse + 0.0005), C.info_bits(mse - 0.0005)
        if code == "LQ-32/16":
            assert abs(C.info_bits(mse) - info) < 0.015
        else:
            assert lo - 0.005 <= info <= hi + 0.005, (code, lo, hi, info)


def test_exhaustive_identity_is_sign():
    """D = d, M = I: the nearest point of {+-1}^d to w is sign(w); at w_j = 0
    both signs tie and the smallest index (sign -1) wins."""
    rng = np.random.default_rng(1)
    W = rng.standard_normal((50, 5))
    W[0, 2] = 0.0
    codes, err, _ = C.encode_exhaustive(W, np.eye(5))
    want = np.where(W > 0, 1, -1)
    np.testing.assert_array_equal(codes, want)
    np.testing.assert_allclose(err, ((W - want) ** 2).sum(1), rtol=1e-14)


def test_exhaustive_one_bit_gaussian_quantiser():
    """D = d = 1, M = [m]: err = (|w| - m)^2; with m = E|w| = sqrt(2/pi) the
    mean over a unit Gaussian is the textbook one-bit distortion 1 - 2/pi."""
    rng = np.random.default_rng(2)
    w = rng.standard_normal(400_000)
    m = math.sqrt(2 / math.pi)
    codes, err, _ = C.encode_exhaustive(w[:, None], np.array([[m]]))
    np.testing.assert_allclose(err, (np.abs(w) - m) ** 2, rtol=1e-12, atol=1e-15)
    sigma = np.std((np.abs(w) - m) ** 2) / math.sqrt(w.size)
    assert abs(err.mean() - (1 - 2 / math.pi)) < 4 * sigma


def test_exhaustive_matches_loop_brute_force():
    """Tiny lattices: the vectorised enumeration agrees with plain loops over
    every sign vector (no numpy in the inner computation)."""
    rng = np.random.default_rng(3)
    d, D = 3, 6
    M = rng.standard_normal((d, D))
    W = rng.standard_normal((20, d))
    codes, err, _ = C.encode_exhaustive(W, M)
    for g in range(W.shape[0]):
        best = None
        for y in itertools.product((-1, 1), repeat=D):
            e = 0.0
            for r in range(d):
                acc = W[g, r]
                for j in range(D):
                    acc -= M[r, j] * y[j]
                e += acc * acc
            if best is None or e < best[0]:
                best = (e, y)
        assert tuple(codes[g]) == best[1]
        assert abs(err[g] - best[0]) <= 1e-12 * max(1.0, best[0])


def test_exhaustive_unused_columns_tie_to_first_index():
    """M = [I | 0]: the last D - d signs do not move the point; every choice
    ties and the smallest index (those signs -1) wins."""
    rng = np.random.default_rng(4)
    d, D = 3, 5
    M = np.hstack([np.eye(d), np.zeros((d, D - d))])
    W = rng.standard_normal((10, d))
    codes, err, t = C.encode_exhaustive(W, M)
    np.testing.assert_array_equal(codes[:, :d], np.where(W >= 0, 1, -1))
    assert (codes[:, d:] == -1).all()
    assert (t < (1 << d)).all()


def test_search_square_is_sign_of_solve():
    """D = d: no auxiliary signs, one candidate, y = sign(M^-1 w)."""
    rng = np.random.default_rng(5)
    d = 6
    M = rng.standard_normal((d, d)) + 2 * np.eye(d)
    W = rng.standard_normal((30, d))
    codes, err, t = C.encode_search(W, M, np.zeros((0, d)))
    want = np.where(np.linalg.solve(M, W.T).T >= 0, 1, -1)
    np.testing.assert_array_equal(codes, want)
    assert (t == 0).all()


def test_search_with_coordinate_completion_on_separable_M():
    """M = [I | 0] completed by A = [0 | I]: every candidate is (sign(w), v),
    all tie, v = all -1 (index 0) wins, and the error is the true minimum."""
    rng = np.random.default_rng(6)
    d, D = 4, 7
    M = np.hstack([np.eye(d), np.zeros((d, D - d))])
    A = np.hstack([np.zeros((D - d, d)), np.eye(D - d)])
    W = rng.standard_normal((25, d))
    codes, err, t = C.encode_search(W, M, A)
    np.testing.assert_array_equal(codes[:, :d], np.where(W >= 0, 1, -1))
    assert (codes[:, d:] == -1).all() and (t == 0).all()
    _, e_ex, _ = C.encode_exhaustive(W, M)
    np.testing.assert_allclose(err, e_ex, rtol=1e-14)


def test_search_matches_loop_over_candidates():
    """Tiny case with a random completion: plain loops over v in index order,
    each candidate from a linear solve of [M; A] x = [w; v] (not the stored
    inverse), pick the same code."""
    rng = np.random.default_rng(7)
    d, D = 3, 7
    M = rng.standard_normal((d, D))
    A = rng.standard_normal((D - d, D))
    S = np.vstack([M, A])
    W = rng.standard_normal((15, d))
    codes, err, t = C.encode_search(W, M, A)
    for g in range(W.shape[0]):
        best = None
        for ti in range(1 << (D - d)):
            v = [1.0 if (ti >> j) & 1 else -1.0 for j in range(D - d)]
            x = np.linalg.solve(S, np.concatenate([W[g], v]))
            y = [1 if xj >= 0 else -1 for xj in x]
            e = sum((W[g, r] - sum(M[r, j] * y[j] for j in range(D))) ** 2 for r in range(d))
            if best is None or e < best[0]:
                best = (e, ti, y)
        assert t[g] == best[1] and list(codes[g]) == best[2]
        assert abs(err[g] - best[0]) <= 1e-12 * max(1.0, best[0])


def test_search_never_beats_exhaustive_and_is_close():
    """The search picks a lattice point, so its error is never below the
    exhaustive minimum; from the orthogonal start it reaches the minimum for
    most Gaussian groups (the quality the notes claim for the start)."""
    rng = np.random.default_rng(8)
    d, D = 4, 10
    Q = _haar(rng, D)
    M, A = Q[:d], Q[d:]
    W = rng.standard_normal((400, d))
    _, e_s, _ = C.encode_search(W, M, A)
    _, e_x, _ = C.encode_exhaustive(W, M)
    assert (e_s >= e_x - 1e-12).all()
    assert np.mean(np.isclose(e_s, e_x)) > 0.6
    assert e_s.mean() < 1.2 * e_x.mean()


def test_orthogonal_completion_is_pseudo_inverse_start_plus_auxiliary():
    """With [M; A] orthogonal, [M; A]^-1 [w; v] = M^+ w + A^T v: the reading's
    candidate is the pseudo-inverse start plus an auxiliary part."""
    rng = np.random.default_rng(9)
    d, D = 5, 12
    Q = _haar(rng, D)
    M, A = Q[:d], Q[d:]
    B = C.search_matrix(M, A)
    np.testing.assert_allclose(B[:, :d], np.linalg.pinv(M), atol=1e-12)
    np.testing.assert_allclose(B[:, d:], A.T, atol=1e-12)


def test_float32_decisions_agree_with_float64():
    """Float32 evaluation (the precision a float32 kernel decides in) picks
    the float64 code for almost every group; where not, the two errors are a
    near-tie."""
    rng = np.random.default_rng(10)
    d, D = 8, 16
    Q = _haar(rng, D)
    M, A = Q[:d], Q[d:]
    W = rng.standard_normal((500, d))
    c64, e64, _ = C.encode_search(W, M, A)
    c32, e32, _ = C.encode_search(W, M, A, dtype=np.float32)
    same = (c64 == c32).all(axis=1)
    assert same.mean() > 0.99
    e32_64 = C.group_errors(W, M, c32)
    assert np.all(e32_64 <= e64 * (1 + 1e-5) + 1e-6)


def test_codebook_mse_and_sign_table():
    """sign_table order (bit j of t -> sign j) and the per-weight MSE."""
    T = C.sign_table(3)
    np.testing.assert_array_equal(T[0], [-1, -1, -1])
    np.testing.assert_array_equal(T[1], [1, -1, -1])
    np.testing.assert_array_equal(T[6], [-1, 1, 1])
    W = np.array([[1.0, 2.0]])
    M = np.eye(2)
    assert C.codebook_mse(W, M, np.array([[1, 1]])) == pytest.approx(0.5)


# ------------------------------------------------------------ learning M

def test_softmin_gradient_matches_finite_differences():
    """The derived gradient against central differences of the loss."""
    rng = np.random.default_rng(20)
    d, D, N, T = 2, 5, 9, 10.0
    M = rng.standard_normal((d, D)) * 0.5
    W = rng.standard_normal((N, d))
    _, g, _ = C.softmin_objective(W, M, T)
    h = 1e-6
    fd = np.zeros_like(M)
    for r in range(d):
        for j in range(D):
            Mp, Mm = M.copy(), M.copy()
            Mp[r, j] += h
            Mm[r, j] -= h
            fd[r, j] = (C.softmin_objective(W, Mp, T)[0] - C.softmin_objective(W, Mm, T)[0]) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_softmin_hard_limit_is_nearest_point_error():
    """Large T: the soft code is the nearest code, so the loss is the mean
    exhaustive nearest-point error."""
    rng = np.random.default_rng(21)
    d, D = 3, 7
    M = _haar(rng, D)[:d]
    W = rng.standard_normal((40, d))
    loss, _, yh = C.softmin_objective(W, M, 1e6)
    codes, err, _ = C.encode_exhaustive(W, M)
    np.testing.assert_allclose(yh, codes, atol=1e-9)
    assert abs(loss - err.mean()) < 1e-9


def test_softmin_zero_temperature_is_uniform():
    """T = 0: every code weighs 2^-D, the soft code is the mean of all sign
    vectors (zero), the loss is mean ||w||^2 and the gradient vanishes."""
    rng = np.random.default_rng(22)
    M = rng.standard_normal((3, 6))
    W = rng.standard_normal((11, 3))
    loss, g, yh = C.softmin_objective(W, M, 0.0)
    assert abs(loss - (W * W).sum(1).mean()) < 1e-12
    np.testing.assert_allclose(yh, 0, atol=1e-15)
    np.testing.assert_allclose(g, 0, atol=1e-12)


def test_softmin_one_dimensional_closed_form():
    """D = d = 1, M = [m]: y_hat = tanh(2 T m w), loss = mean (w - m y_hat)^2,
    d loss / d m = mean 2 (w - m y_hat)(-y_hat - m (1 - y_hat^2) 2 T w)."""
    rng = np.random.default_rng(23)
    w = rng.standard_normal(50)
    m, T = 0.8, 10.0
    loss, g, yh = C.softmin_objective(w[:, None], np.array([[m]]), T)
    th = np.tanh(2 * T * m * w)
    np.testing.assert_allclose(yh[:, 0], th, rtol=1e-12, atol=1e-15)
    assert abs(loss - np.mean((w - m * th) ** 2)) < 1e-12
    dm = np.mean(2 * (w - m * th) * (-th - m * (1 - th ** 2) * 2 * T * w))
    assert abs(g[0, 0] - dm) < 1e-10


def test_softmin_column_sign_flip_and_permutation():
    """The code set is closed under flipping a sign and permuting signs, so
    flipping column j of M (or permuting columns) leaves the loss unchanged
    and flips (permutes) the gradient the same way."""
    rng = np.random.default_rng(24)
    d, D = 3, 6
    M = rng.standard_normal((d, D))
    W = rng.standard_normal((20, d))
    loss, g, _ = C.softmin_objective(W, M, 10.0)
    Mf = M.copy()
    Mf[:, 2] *= -1
    lf, gf, _ = C.softmin_objective(W, Mf, 10.0)
    assert abs(lf - loss) < 1e-12
    gexp = g.copy()
    gexp[:, 2] *= -1
    np.testing.assert_allclose(gf, gexp, rtol=1e-10, atol=1e-12)
    perm = rng.permutation(D)
    lp, gp, _ = C.softmin_objective(W, M[:, perm], 10.0)
    assert abs(lp - loss) < 1e-12
    np.testing.assert_allclose(gp, g[:, perm], rtol=1e-10, atol=1e-12)


def test_adam_first_step_is_signed_learning_rate():
    """Step 1: bias correction makes m_hat = g and v_hat = g^2, so the update
    is -lr g / (|g| + eps)."""
    g = np.array([[0.5, -2.0], [1e-3, 0.0]])
    M0 = np.zeros_like(g)
    M1, m1, m2 = C.adam_step(M0, g, np.zeros_like(g), np.zeros_like(g), 1, lr=0.01)
    np.testing.assert_allclose(M1, -0.01 * g / (np.abs(g) + 1e-8), rtol=1e-12)
    np.testing.assert_allclose(m1, 0.1 * g)
    np.testing.assert_allclose(m2, 0.001 * g * g)


def test_learning_lowers_the_objective_and_the_codebook_error():
    """From the orthogonal initialisation, Adam on the soft objective lowers
    it and the hard nearest-point error of the learned M."""
    rng = np.random.default_rng(25)
    d, D = 4, 8
    M0 = _haar(rng, D)[:d]
    batches = [rng.standard_normal((256, d)) for _ in range(30)]
    M, losses = C.learn_m(batches, M0, 10.0, 0.01)
    assert np.mean(losses[-5:]) < losses[0]
    Wt = np.random.default_rng(26).standard_normal((4000, d))
    _, e0, _ = C.encode_exhaustive(Wt, M0)
    _, e1, _ = C.encode_exhaustive(Wt, M)
    assert e1.mean() < e0.mean()

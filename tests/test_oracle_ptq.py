"""Pins of the PTQ initialisation oracle (CPU only).

The oracle (oracle/lcvq_oracle.cpp through oracle/coracle.py) implements decoupleQ's
alternation (section 3.3) for a per-tensor LC code (A = s I, B = b 1), with the integer
step written through H = U D U^T. Each test checks it against something else:
  * the integer step against decoupleQ's literal statement of it -- round and clip
    element j, re-solve the rest by eq. (11)'s minimiser with a linear solve at every
    step (numpy, lcvq_oracle.ptq_sweep_literal);
  * with a diagonal H, against brute force over all 4^K codes of a row, and against
    decoupleQ eq. (3) (per-tensor round-to-nearest) on exactly representable inputs;
  * the (s, b) step against a least-squares solve by another route (a Cholesky factor
    of H and numpy's lstsq on the stacked residuals);
  * the objective against eq. (5)'s form through X (not H), and H against X^T X;
  * the factorisation against U diag(D) U^T = H and a reversed Cholesky from numpy;
  * the objective identity g = s^2 / 2 sum D_k (t_k - c_k)^2 and the sums of the normal
    equations written through U (the form the GPU sweep accumulates);
  * the alternation: the objective never increases, step after step.
"""

import itertools

import numpy as np
import pytest

from oracle import coracle as C
from oracle import lcvq_oracle as O


def spd(rng, K, M=None):
    X = rng.normal(size=(M or 2 * K, K))
    return X, C.hessian(X)


def away_from_ties(t, margin=1e-6):
    f = np.abs(t - np.floor(t) - 0.5)
    return bool(np.all(f > margin))


# ---------------------------------------------------------------- H and its factorisation
def test_hessian_is_xtx():
    rng = np.random.default_rng(1)
    X = rng.normal(size=(37, 23))
    H = C.hessian(X)
    np.testing.assert_allclose(H, X.T @ X, rtol=1e-12, atol=1e-12)
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("K", [1, 5, 32, 100])
def test_udu_reconstructs_and_matches_reversed_cholesky(K):
    rng = np.random.default_rng(K)
    _, H = spd(rng, K)
    Hd = C.damp(H, 0.01)
    assert np.allclose(np.diag(Hd) - np.diag(H), 0.01 * np.trace(H) / K)
    U, D = C.udu(Hd)
    assert np.all(D > 0)
    assert np.array_equal(np.diag(U), np.ones(K))
    assert np.all(np.tril(U, -1) == 0)
    np.testing.assert_allclose(U @ np.diag(D) @ U.T, Hd, rtol=1e-11, atol=1e-9 * np.abs(Hd).max())
    # another route: lower Cholesky of the index-reversed matrix, reversed back
    J = np.eye(K)[::-1]
    L = np.linalg.cholesky(J @ Hd @ J)
    V = J @ L @ J                                     # upper, Hd = V V^T
    np.testing.assert_allclose(U, V / np.diag(V)[None, :], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(D, np.diag(V) ** 2, rtol=1e-10)


def test_udu_rejects_indefinite():
    with pytest.raises(ValueError):
        C.udu(np.array([[1.0, 2.0], [2.0, 1.0]]))


# ---------------------------------------------------------------- the integer step
@pytest.mark.parametrize("K", [3, 8, 12])
def test_sweep_equals_literal_eq11(K):
    """The U-feedback form and decoupleQ's literal per-step minimisation give the same codes."""
    rng = np.random.default_rng(100 + K)
    done = 0
    for trial in range(6):
        _, H = spd(rng, K, M=K + 3)
        Hd = C.damp(H, 0.05)
        U, _ = C.udu(Hd)
        W0 = rng.normal(size=(8, K)) * 0.7
        s, b = rng.uniform(0.2, 0.6) * rng.choice([-1, 1]), rng.normal() * 0.3
        c, t = C.ptq_sweep(W0, U, s, b, want_t=True)
        if not away_from_ties(t):
            continue
        assert np.array_equal(c, O.ptq_sweep_literal(W0, Hd, s, b)), trial
        done += 1
    assert done >= 4


def test_targets_follow_the_given_codes():
    """ptq_targets driven by the sweep's own codes returns the sweep's own t; driven by
    other codes, each t_k depends only on the codes before k."""
    rng = np.random.default_rng(12)
    K, N = 40, 6
    _, H = spd(rng, K)
    U, _ = C.udu(C.damp(H, 0.01))
    W0 = rng.normal(size=(N, K)) * 0.3
    c, t = C.ptq_sweep(W0, U, 0.2, -0.3, want_t=True)
    assert np.array_equal(C.ptq_targets(W0, U, 0.2, -0.3, c), t)
    c2 = c.copy()
    c2[:, 20] = (c2[:, 20] + 1) % 4
    t2 = C.ptq_targets(W0, U, 0.2, -0.3, c2)
    assert np.array_equal(t2[:, :21], t[:, :21]) and not np.array_equal(t2[:, 21:], t[:, 21:])


@pytest.mark.parametrize("K", [1, 4, 6])
def test_diagonal_H_sweep_is_brute_force_optimum(K):
    """With a diagonal H the objective separates per element: the sweep (no feedback)
    must reach the exact minimum over all 4^K codes of every row."""
    rng = np.random.default_rng(7 + K)
    Hd = np.diag(rng.uniform(0.5, 3.0, size=K))
    U, D = C.udu(Hd)
    assert np.allclose(U, np.eye(K))
    W0 = rng.normal(size=(10, K))
    s, b = 0.45, -0.8
    c = C.ptq_sweep(W0, U, s, b)
    allc = np.array(list(itertools.product(range(4), repeat=K)), dtype=np.float64)
    for n in range(W0.shape[0]):
        R = s * allc + b - W0[n]
        g = 0.5 * np.einsum("ck,k,ck->c", R, np.diag(Hd), R)
        best = allc[int(np.argmin(g))]
        assert np.array_equal(c[n].astype(np.float64), best), n


def test_diagonal_H_is_decoupleq_round_to_nearest():
    """decoupleQ eq. (3)/(4) per tensor with alpha = -2, beta = 1: the integer part is the
    LC code minus 2, on inputs where every intermediate is exact."""
    rng = np.random.default_rng(3)
    K = 64
    s = 2.0 ** -4
    zero = 3 * s
    b = zero - 2 * s
    W0 = rng.integers(-96, 96, size=(16, K)) / 64.0 * s + zero   # a 2^-6 s grid
    U = np.eye(K)
    c = C.ptq_sweep(W0, U, s, b)
    q, wt = O.decoupleq_quant(W0, s, zero)
    assert np.array_equal(c.astype(np.int64), q.astype(np.int64) + 2)
    assert np.array_equal(s * c + b, wt)


def test_objective_identity_through_U():
    """g(c; s, b) = s^2 / 2 sum_n sum_k D_k (t_nk - c_nk)^2 for the sweep's own output, and
    the normal equations' sums written through a = U^T c, e = U^T 1, q = U^T w0 equal the
    sums over H (the form the GPU sweep accumulates)."""
    rng = np.random.default_rng(11)
    K, N = 24, 9
    _, H = spd(rng, K)
    Hd = C.damp(H, 0.01)
    U, D = C.udu(Hd)
    W0 = rng.normal(size=(N, K)) * 0.3
    s, b = 0.21, -0.33
    c, t = C.ptq_sweep(W0, U, s, b, want_t=True)
    g = C.ptq_objective(W0, c, Hd, s, b)
    assert np.isclose(g, 0.5 * s * s * np.sum(D * (t - c) ** 2), rtol=1e-11)
    cf = c.astype(np.float64)
    a = cf @ U                                       # rows: (U^T c_n)^T
    e = np.ones(K) @ U
    q = W0 @ U
    S1, S2, T1 = np.sum(D * a * a), np.sum(D * a * e), np.sum(D * a * q)
    S3, T2, Wq = N * np.sum(D * e * e), np.sum(D * e * q), np.sum(D * q * q)
    h1 = Hd @ np.ones(K)
    np.testing.assert_allclose(S1, np.einsum("nk,kj,nj->", cf, Hd, cf), rtol=1e-10)
    np.testing.assert_allclose(S2, np.sum(cf @ h1), rtol=1e-10)
    np.testing.assert_allclose(T1, np.einsum("nk,kj,nj->", cf, Hd, W0), rtol=1e-10)
    np.testing.assert_allclose(S3, N * np.sum(h1), rtol=1e-10)
    np.testing.assert_allclose(T2, np.sum(W0 @ h1), rtol=1e-10)
    g2 = 0.5 * (s * s * S1 + 2 * s * b * S2 - 2 * s * T1 + b * b * S3 - 2 * b * T2 + Wq)
    np.testing.assert_allclose(g, g2, rtol=1e-10)


# ---------------------------------------------------------------- the (s, b) step
def test_sb_step_is_least_squares_by_another_route():
    rng = np.random.default_rng(5)
    K, N = 16, 12
    _, H = spd(rng, K)
    Hd = C.damp(H, 0.01)
    W0 = rng.normal(size=(N, K)) * 0.1
    c = rng.integers(0, 4, size=(N, K)).astype(np.uint8)
    s, b, sing = C.ptq_solve_sb(W0, c, Hd)
    assert not sing
    R = np.linalg.cholesky(Hd).T                      # Hd = R^T R
    Acol = np.concatenate([R @ c[n].astype(np.float64) for n in range(N)])
    Bcol = np.concatenate([R @ np.ones(K) for _ in range(N)])
    rhs = np.concatenate([R @ W0[n] for n in range(N)])
    sol, *_ = np.linalg.lstsq(np.stack([Acol, Bcol], axis=1), rhs, rcond=None)
    np.testing.assert_allclose([s, b], sol, rtol=1e-9, atol=1e-12)
    g0 = C.ptq_objective(W0, c, Hd, s, b)
    for ds, db in [(1e-3, 0), (-1e-3, 0), (0, 1e-3), (0, -1e-3)]:
        assert C.ptq_objective(W0, c, Hd, s + ds, b + db) > g0


def test_sb_step_singular_codes_keep_sb():
    """All codes equal: s and b are not separable; the step keeps them."""
    rng = np.random.default_rng(6)
    K, N = 8, 4
    _, H = spd(rng, K)
    W0 = rng.normal(size=(N, K))
    c = np.full((N, K), 2, np.uint8)
    s, b, sing = C.ptq_solve_sb(W0, c, C.damp(H, 0.01), 0.7, -0.1)
    assert sing and (s, b) == (0.7, -0.1)


# ---------------------------------------------------------------- objective, alternation
def test_objective_is_eq5_through_X():
    """g with damp = 0 is 1/2 ||X W~^T - X W0^T||_F^2, the layer-output error of eq. (5)."""
    rng = np.random.default_rng(8)
    K, N, M = 20, 7, 50
    X = rng.normal(size=(M, K))
    H = C.hessian(X)
    W0 = rng.normal(size=(N, K)) * 0.2
    c = rng.integers(0, 4, size=(N, K)).astype(np.uint8)
    s, b = 0.17, -0.2
    Wt = s * c + b
    want = 0.5 * np.sum((X @ Wt.T - X @ W0.T) ** 2)
    assert np.isclose(C.ptq_objective(W0, c, H, s, b), want, rtol=1e-11)
    assert np.isclose(O.ptq_objective(W0, c, H, s, b), want, rtol=1e-11)


@pytest.mark.parametrize("K,N,M", [(16, 10, 40), (64, 24, 48), (96, 8, 300)])
def test_alternation_never_increases_objective(K, N, M):
    rng = np.random.default_rng(K + N)
    X = rng.normal(size=(M, K))
    X[:, :3] *= 6.0                                   # a few outlier input channels
    H = C.hessian(X)
    W0 = rng.normal(size=(N, K)) * 0.02
    r = C.ptq_init(W0, H, 0.01, 5)
    obj = r["obj"]
    assert np.all(np.diff(obj) <= 1e-12 * obj[0]), obj
    Hd = C.damp(H, 0.01)
    assert np.isclose(obj[-1], C.ptq_objective(W0, r["codes"], Hd, r["s"], r["b"]), rtol=1e-12)
    # the result beats round-to-nearest on the initial grid over the weight's range
    s0, b0 = (W0.max() - W0.min()) / 3, W0.min()
    rtn = np.clip(np.rint((W0 - b0) / s0), 0, 3).astype(np.uint8)
    assert obj[-1] < C.ptq_objective(W0, rtn, Hd, s0, b0)

"""Pins of the CPU oracles against things other than themselves.

Each test checks an oracle function against a fact the pages or the mathematics fix:
hand-worked values, brute-force search, the decoupleQ scalar special case, closed
forms computed by a different route, exact finite differences, and torch autograd on
the literal formula. All run on the CPU, once for each oracle: the plain C++ loops
(oracle/lcvq_oracle.cpp through oracle/coracle.py, the oracle of record) and the numpy
one (oracle/lcvq_oracle.py, a second opinion that uses library matmuls as steps).
Helpers that are routes of their own (brute-force codeword search, the decoupleQ
eq. (3)/(4) routine, the smooth-rounding curve) come from the numpy module in both.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import coracle
from oracle import lcvq_oracle as H


@pytest.fixture(params=["cxx", "numpy"], scope="module")
def O(request):
    if request.param == "cxx":
        coracle.lib()
        return coracle
    return H


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- hand-worked values
def test_hand_example_d2(O, golden_dir):
    g = _load(golden_dir, "hand_example_d2.json")
    d = g["d"]
    A, B = np.array(g["A"]), np.array(g["B"])
    Wp = np.array(g["Wp"], dtype=np.float32)
    X, dY = np.array(g["X"]), np.array(g["dY"])
    e = g["expect"]
    f = O.linear_fwd(X, Wp, A, B, d)
    assert f["z"].tolist() == e["z"]
    assert f["m"].tolist() == e["mask"]
    np.testing.assert_allclose(f["What"], e["What"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(f["Y"], e["Y"], rtol=0, atol=1e-12)
    b = O.linear_bwd(dY, X, f["z"], f["m"], A, B, d)
    np.testing.assert_allclose(b["dX"], e["dX"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["dWp"], e["dWp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["dA"], e["dA"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["dB"], e["dB"], rtol=0, atol=1e-12)


def test_quantize_edge_values(O, golden_dir):
    g = _load(golden_dir, "quantize_edge_values.json")
    wp = np.array([float(v) for v in g["wp"]], dtype=np.float32)
    z, m = O.quantize(wp)
    assert z.tolist() == g["z"]
    assert m.tolist() == g["mask"]


def test_quantize_matches_torch_round_clamp(O):
    # torch.round is round-half-to-even; an independent route to the same codes.
    gen = torch.Generator().manual_seed(3)
    wp = (torch.rand(4096, generator=gen) * 7 - 2).float()
    ties = torch.tensor([-0.5, 0.5, 1.5, 2.5, 3.5, -1.5, 4.5])
    wp = torch.cat([wp, ties])
    z, m = O.quantize(wp.numpy())
    r = torch.round(wp)
    assert np.array_equal(z, torch.clamp(r, 0, 3).to(torch.uint8).numpy())
    assert np.array_equal(m, ((r >= 0) & (r <= 3)).to(torch.uint8).numpy())


# ---------------------------------------------------------------- packing
def test_pack_worked_example(O):
    # codes [1, 2, 3, 0] -> 1 | 2<<2 | 3<<4 | 0<<6 = 0x39
    assert O.pack2b(np.array([[1, 2, 3, 0]], dtype=np.uint8)).tolist() == [[0x39]]
    # mask bits [1,0,1,1,0,0,0,1] -> 1 + 4 + 8 + 128 = 0x8D
    assert O.pack_mask(np.array([[1, 0, 1, 1, 0, 0, 0, 1]], dtype=np.uint8)).tolist() == [[0x8D]]


def test_pack_roundtrips(O):
    allbytes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(O.pack2b(O.unpack2b(allbytes, 1024)), allbytes)
    assert np.array_equal(O.pack_mask(O.unpack_mask(allbytes, 2048)), allbytes)
    rng = np.random.default_rng(5)
    z = rng.integers(0, 4, size=(7, 64), dtype=np.uint8)
    assert np.array_equal(O.unpack2b(O.pack2b(z), 64), z)
    m = rng.integers(0, 2, size=(7, 64), dtype=np.uint8)
    assert np.array_equal(O.unpack_mask(O.pack_mask(m), 64), m)
    # each code lands in its own bit field
    for t in range(4):
        for c in range(4):
            z = np.zeros((1, 4), dtype=np.uint8)
            z[0, t] = c
            assert int(O.pack2b(z)[0, 0]) == c << (2 * t)


# ---------------------------------------------------------------- brute force
def _away_from_ties(rng, n, d):
    w = rng.uniform(-1.2, 4.2, size=(n, d))
    frac = np.abs(w - np.floor(w) - 0.5)
    w[frac < 0.02] += 0.1
    return w.astype(np.float32)


@pytest.mark.parametrize("d", [2, 4, 8])
def test_round_clamp_is_nearest_codeword_for_orthogonal_columns(O, d):
    """Nearest-codeword search over all 4^d codes equals round/clamp when A has
    orthogonal columns (the distance then separates per coordinate)."""
    rng = np.random.default_rng(11 + d)
    n = 60 if d < 8 else 12
    W = _away_from_ties(rng, n, d)
    for case in range(3):
        if case == 0:
            A = np.diag(rng.uniform(0.2, 2.0, size=d) * rng.choice([-1, 1], size=d))
        else:
            Q, _ = np.linalg.qr(rng.normal(size=(d, d)))
            A = Q @ np.diag(rng.uniform(0.3, 3.0, size=d))
        B = rng.normal(size=d)
        z, _ = O.quantize(W)
        for r in range(n):
            assert np.array_equal(H.nearest_codeword(W[r], A, B), z[r]), (case, r)


def test_general_A_is_not_nearest_codeword(O):
    """For a general A the two rules differ (so LC-VQ is not nearest-codeword VQ):
    the brute force must find a strictly closer codeword on some inputs."""
    rng = np.random.default_rng(1)
    d = 4
    A = rng.normal(size=(d, d))
    B = np.zeros(d)
    W = _away_from_ties(rng, 200, d)
    z, _ = O.quantize(W)
    differ = 0
    for r in range(200):
        zb = H.nearest_codeword(W[r], A, B)
        if not np.array_equal(zb, z[r]):
            t = A @ W[r].astype(np.float64)
            db = np.sum((A @ zb - t) ** 2)
            dz = np.sum((A @ z[r] - t) ** 2)
            assert db < dz
            differ += 1
    assert differ > 0


# ---------------------------------------------------------------- decoupleQ special case
def test_diagonal_A_is_decoupleq_uniform_quantization(O):
    """A = s I, B = b 1 reduces LC-VQ to per-tensor uniform 2-bit quantization,
    decoupleQ eq. (3)/(4) with alpha=-2, beta=1, after the code offset z = W^ + 2."""
    rng = np.random.default_rng(2)
    d = 8
    for s_exp, k in [(-5, 3), (-2, -1), (1, 0), (-7, 17)]:
        s = 2.0 ** s_exp
        zero = k * s
        wp = (rng.integers(-4 * 65536, 8 * 65536, size=(16, 64)) / 65536.0).astype(np.float32)
        W0 = s * (wp.astype(np.float64) - 2.0 + k)
        q, wt = H.decoupleq_quant(W0, s, zero)
        z, m = O.quantize(wp)
        assert np.array_equal(z.astype(np.int64), q.astype(np.int64) + 2)
        b = zero - 2 * s
        w = O.reconstruct(z, s * np.eye(d), b * np.ones(d), d)
        assert np.array_equal(w, wt)
        # and the mask is "the clip did nothing"
        r = np.rint((W0 - zero) / s)
        assert np.array_equal(m.astype(bool), (r >= -2) & (r <= 1))


# ---------------------------------------------------------------- closed forms by another route
def _layer(seed, M=5, N=12, K=48, d=8, lo=-2.0, hi=5.0):
    rng = np.random.default_rng(seed)
    wp = rng.uniform(lo, hi, size=(N, K)).astype(np.float32)
    A = rng.normal(size=(d, d))
    B = rng.normal(size=d)
    X = rng.normal(size=(M, K))
    dY = rng.normal(size=(M, N))
    return wp, A, B, X, dY


@pytest.mark.parametrize("d", [4, 8, 16])
def test_fold_identities(O, d):
    """Y = X' Z^T + beta 1^T with X' = X (I kron A), beta = X (1 kron B); and
    dX = (dY Z)(I kron A^T) + (dY 1)(1 kron B)^T; dB = sum_g (r^T X)_g, r = dY 1."""
    wp, A, B, X, dY = _layer(7 + d, d=d, K=64)
    f = O.linear_fwd(X, wp, A, B, d)
    b = O.linear_bwd(dY, X, f["z"], f["m"], A, B, d)
    M, K = X.shape
    Z = f["z"].astype(np.float64)
    IA = np.kron(np.eye(K // d), A)                # block diagonal, blocks A
    Xp = X @ IA
    beta = X @ np.tile(B, K // d)
    np.testing.assert_allclose(f["Y"], Xp @ Z.T + beta[:, None], rtol=1e-12, atol=1e-10)
    r = dY.sum(axis=1)
    dX2 = (dY @ Z) @ IA.T + np.outer(r, np.tile(B, K // d))
    np.testing.assert_allclose(b["dX"], dX2, rtol=1e-12, atol=1e-10)
    dB2 = (r @ X).reshape(K // d, d).sum(axis=0)
    np.testing.assert_allclose(b["dB"], dB2, rtol=1e-12, atol=1e-10)


def test_gemv_matches_forward(O):
    wp, A, B, X, _ = _layer(31, M=3, N=16, K=64, d=8)
    f = O.linear_fwd(X, wp, A, B, 8)
    np.testing.assert_allclose(O.gemv2b(X, f["packed"], A, B, 8), f["Y"], rtol=1e-13, atol=1e-12)


# ---------------------------------------------------------------- exact finite differences
@pytest.mark.parametrize("d", [2, 8])
def test_finite_differences_exact(O, d):
    """L = <dY, X What^T> is affine in A, B, X and in the (continuous) codes, so a
    central difference with a unit step is exact up to rounding. The STE gradient of Wp
    is the code gradient where the mask is 1 and zero elsewhere."""
    wp, A, B, X, dY = _layer(100 + d, M=3, N=4, K=16, d=d)
    z, m = O.quantize(wp)
    b = O.linear_bwd(dY, X, z, m, A, B, d)

    def L(A_, B_, X_, zc):
        n, k = zc.shape
        w = (zc.reshape(n, k // d, d) @ np.asarray(A_).T + B_).reshape(n, k)
        return float(np.sum(dY * (X_ @ w.T)))

    zf = z.astype(np.float64)
    h = 1.0
    for i in range(d):
        for j in range(d):
            E = np.zeros((d, d))
            E[i, j] = h
            fd = (L(A + E, B, X, zf) - L(A - E, B, X, zf)) / (2 * h)
            assert math.isclose(fd, b["dA"][i, j], rel_tol=1e-12, abs_tol=1e-10)
        e = np.zeros(d)
        e[i] = h
        fd = (L(A, B + e, X, zf) - L(A, B - e, X, zf)) / (2 * h)
        assert math.isclose(fd, b["dB"][i], rel_tol=1e-12, abs_tol=1e-10)
    for (r, c) in [(0, 0), (1, 5), (2, 15)]:
        E = np.zeros_like(X)
        E[r, c] = h
        fd = (L(A, B, X + E, zf) - L(A, B, X - E, zf)) / (2 * h)
        assert math.isclose(fd, b["dX"][r, c], rel_tol=1e-12, abs_tol=1e-10)
    n, k = z.shape
    for r in range(n):
        for c in range(k):
            E = np.zeros((n, k))
            E[r, c] = h
            fd = (L(A, B, X, zf + E) - L(A, B, X, zf - E)) / (2 * h)
            want = fd if m[r, c] else 0.0
            assert math.isclose(want, b["dWp"][r, c], rel_tol=1e-12, abs_tol=1e-10)


# ---------------------------------------------------------------- third opinion: torch autograd
@pytest.mark.parametrize("d", [4, 8, 16])
def test_torch_autograd_literal_formula(O, d):
    """PyTorch CPU float64 autograd of clamp(Wp + (round(Wp) - Wp).detach(), 0, 3),
    decoded by A z + B and multiplied by X, gives the same forward and gradients."""
    wp, A, B, X, dY = _layer(200 + d, M=4, N=8, K=64, d=d)
    f = O.linear_fwd(X, wp, A, B, d)
    b = O.linear_bwd(dY, X, f["z"], f["m"], A, B, d)
    Wt = torch.tensor(wp.astype(np.float64), requires_grad=True)
    At = torch.tensor(A, requires_grad=True)
    Bt = torch.tensor(B, requires_grad=True)
    Xt = torch.tensor(X, requires_grad=True)
    zs = Wt + (torch.round(Wt) - Wt).detach()
    zc = torch.clamp(zs, 0, 3)
    n, k = wp.shape
    w = (zc.view(n, k // d, d) @ At.T + Bt).view(n, k)
    Y = Xt @ w.T
    (Y * torch.tensor(dY)).sum().backward()
    np.testing.assert_allclose(Y.detach().numpy(), f["Y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Xt.grad.numpy(), b["dX"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Wt.grad.numpy(), b["dWp"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(At.grad.numpy(), b["dA"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Bt.grad.numpy(), b["dB"], rtol=1e-12, atol=1e-12)


def test_mask_zero_outside_clamp_range(O):
    wp = np.array([[-0.51, -0.5, 3.49, 3.5, 10.0, -3.0, 1.0, 2.0]], dtype=np.float32)
    z, m = O.quantize(wp)
    assert m.tolist() == [[0, 1, 1, 0, 0, 0, 1, 1]]
    A, B = np.eye(8), np.zeros(8)
    b = O.linear_bwd(np.ones((1, 1)), np.ones((1, 8)), z, m, A, B, 8)
    assert b["dWp"].tolist() == [[0, 1, 1, 0, 0, 0, 1, 1]]


# ---------------------------------------------------------------- DGE curve (own family)
# The pages fix no DGE curve, so these pins check the oracle's family against its own
# definition by other routes: derivative by finite differences, its limits, and torch
# autograd through the literal smooth-rounding formula.
@pytest.mark.parametrize("alpha", [0.5, 4.0, 12.0])
def test_dge_slope_is_derivative_of_curve(O, alpha):
    w = np.random.default_rng(5).uniform(-1.0, 4.0, 2000)
    h = 1e-6
    fd = (H.dge_curve(w + h, alpha) - H.dge_curve(w - h, alpha)) / (2 * h)
    np.testing.assert_allclose(O.dge_slope(w, alpha), fd, rtol=1e-6, atol=1e-6)


def test_dge_curve_limits_and_fixed_points(O):
    ints = np.arange(-2.0, 6.0)
    np.testing.assert_allclose(H.dge_curve(ints, 7.0), ints, atol=1e-14)
    np.testing.assert_allclose(H.dge_curve(ints + 0.5, 7.0), ints + 0.5, atol=1e-14)
    w = np.random.default_rng(6).uniform(-1.0, 4.0, 1000)
    # alpha -> 0: the straight-through estimator (identity curve, slope 1)
    np.testing.assert_allclose(H.dge_curve(w, 1e-6), w, atol=1e-9)
    np.testing.assert_allclose(O.dge_slope(w, 1e-6), 1.0, atol=1e-9)
    # alpha -> infinity: rounding, away from the half-integers
    far = w[np.abs(w - np.floor(w) - 0.5) > 0.1]
    np.testing.assert_allclose(H.dge_curve(far, 200.0), np.rint(far), atol=1e-12)
    # monotone, and the slope integrates to 1 over a cell
    x = np.linspace(0.0, 1.0, 200001)
    assert np.all(np.diff(H.dge_curve(x, 9.0)) > 0)
    assert abs(np.trapezoid(O.dge_slope(x, 9.0), x) - 1.0) < 1e-8
    assert np.all(O.dge_slope(np.array([np.nan, np.inf, -np.inf]), 3.0) == 0.0)


@pytest.mark.parametrize("d", [4, 8])
def test_dge_backward_matches_torch_autograd(O, d):
    """Forward rounds; the backward differentiates the smooth curve (value of round,
    gradient of s): zs = s(Wp) + (round(Wp) - s(Wp)).detach(), then clamp and decode."""
    alpha = 6.0
    wp, A, B, X, dY = _layer(300 + d, M=4, N=8, K=64, d=d)
    wp = (wp * 1.6 - 1.0).astype(np.float32)                  # some clamped proxies too
    f = O.linear_fwd(X, wp, A, B, d)
    b = O.linear_bwd(dY, X, f["z"], f["m"], A, B, d, wp=wp, dge_alpha=alpha)
    Wt = torch.tensor(wp.astype(np.float64), requires_grad=True)
    fl = torch.floor(Wt).detach()
    s = fl + 0.5 + torch.tanh(alpha * (Wt - fl - 0.5)) / (2 * math.tanh(alpha / 2))
    zs = s + (torch.round(Wt) - s).detach()
    zc = torch.clamp(zs, 0, 3)
    n, k = wp.shape
    At = torch.tensor(A)
    Bt = torch.tensor(B)
    w = (zc.view(n, k // d, d) @ At.T + Bt).view(n, k)
    Y = torch.tensor(X) @ w.T
    (Y * torch.tensor(dY)).sum().backward()
    np.testing.assert_allclose(Y.detach().numpy(), f["Y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Wt.grad.numpy(), b["dWp"], rtol=1e-10, atol=1e-12)
    assert np.count_nonzero(f["m"] == 0) > 0

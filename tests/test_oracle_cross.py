"""The two CPU oracles against each other, element by element (CPU only).

The plain C++ oracle (the oracle of record) and the numpy oracle are written
independently from the same definitions; both are pinned by test_oracle_pins.py. Here
they must agree to float64 rounding on random layers with ragged shapes, every vector
length, masks and non-finite proxies, the DGE option, the decode product, and the
row-subset entry points that the large GPU tests use for sampled outputs.
"""

import numpy as np
import pytest

from oracle import coracle as C
from oracle import lcvq_oracle as O

RTOL = 1e-12


def close(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() <= RTOL * scale


def layer(seed, M, N, K, d):
    rng = np.random.default_rng(seed)
    wp = rng.uniform(-2.0, 5.0, size=(N, K)).astype(np.float32)
    wp.reshape(-1)[:6] = [np.nan, np.inf, -np.inf, 0.5, 2.5, -0.5]
    A = rng.normal(size=(d, d))
    B = rng.normal(size=d)
    X = rng.normal(size=(M, K)).astype(np.float32).astype(np.float64)
    dY = rng.normal(size=(M, N)).astype(np.float32).astype(np.float64)
    return wp, A, B, X, dY


@pytest.mark.parametrize("d", [2, 4, 8, 16])
@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (37, 48, 96), (130, 200, 160)])
def test_layer_agrees(M, N, K, d):
    if K % d:
        pytest.skip("K not a multiple of d")
    wp, A, B, X, dY = layer(M * 1000 + N + K + d, M, N, K, d)
    fc, fn = C.linear_fwd(X, wp, A, B, d), O.linear_fwd(X, wp, A, B, d)
    for k in ("z", "m", "packed", "maskbits"):
        assert np.array_equal(fc[k], fn[k]), k
    assert close(fc["What"], fn["What"]) and close(fc["Y"], fn["Y"])
    bc = C.linear_bwd(dY, X, fc["z"], fc["m"], A, B, d)
    bn = O.linear_bwd(dY, X, fn["z"], fn["m"], A, B, d)
    for k in ("dX", "dWp", "dA", "dB"):
        assert close(bc[k], bn[k]), k
    alpha = 5.0
    gc = C.linear_bwd(dY, X, fc["z"], fc["m"], A, B, d, wp=wp, dge_alpha=alpha)
    gn = O.linear_bwd(dY, X, fn["z"], fn["m"], A, B, d, wp=wp, dge_alpha=alpha)
    for k in ("dX", "dWp", "dA", "dB"):
        assert close(gc[k], gn[k]), ("dge", k)


def test_row_subsets():
    """Rows selected from X, dY and the weight give those rows of the full results; dA
    and dB over a subset of weight rows are the backward of those rows alone."""
    M, N, K, d = 50, 64, 96, 8
    wp, A, B, X, dY = layer(9, M, N, K, d)
    f = C.linear_fwd(X, wp, A, B, d)
    b = C.linear_bwd(dY, X, f["z"], f["m"], A, B, d)
    rm = np.array([0, 7, 49, 23])
    rn = np.array([63, 0, 5, 31, 32])
    fs = C.linear_fwd(X, wp, A, B, d, rows=rm)
    assert np.array_equal(fs["Y"], f["Y"][rm])
    bs = C.linear_bwd(dY, X, f["z"], f["m"], A, B, d, dx_rows=rm, dw_rows=rn)
    assert np.array_equal(bs["dX"], b["dX"][rm])
    assert np.array_equal(bs["dWp"], b["dWp"][rn])
    sub = O.linear_bwd(dY[:, rn], X, f["z"][rn], f["m"][rn], A, B, d)
    assert close(bs["dA"], sub["dA"]) and close(bs["dB"], sub["dB"])
    pk = f["packed"]
    Y = C.gemv2b(X[:3], pk, A, B, d)
    assert close(Y, O.gemv2b(X[:3], pk, A, B, d))
    assert np.array_equal(C.gemv2b(X[:3], pk, A, B, d, rows=rn), Y[:, rn])


def test_results_independent_of_thread_count():
    """Every sum runs in a fixed order, whatever the OpenMP split: the full backward equals
    the concatenation of single-row calls bit for bit."""
    M, N, K, d = 40, 24, 64, 4
    wp, A, B, X, dY = layer(3, M, N, K, d)
    f = C.linear_fwd(X, wp, A, B, d)
    b = C.linear_bwd(dY, X, f["z"], f["m"], A, B, d)
    rows = [C.linear_bwd(dY, X, f["z"], f["m"], A, B, d, dx_rows=[r], dw_rows=[r])
            for r in range(N)]
    assert np.array_equal(np.concatenate([r["dWp"] for r in rows]), b["dWp"])
    assert np.array_equal(np.concatenate([r["dX"] for r in rows]), b["dX"][:N])
    dA = np.zeros((d, d))
    dB = np.zeros(d)
    for r in rows:                       # the library adds row sums in row order
        dA = dA + r["dA"]
        dB = dB + r["dB"]
    assert np.array_equal(dA, b["dA"]) and np.array_equal(dB, b["dB"])

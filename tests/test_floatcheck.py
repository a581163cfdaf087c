"""The float parity check rejects local defects that a tensor-wide norm lets through.

CPU only. A realistic stand-in for a GPU result is built from the oracle: the same layer
computed by torch on the CPU with bf16 operands (float32 accumulation), output rounded
to bf16, which carries the same kind of rounding error as the matrix-core products.
It must pass. Then one defect at a time is planted in a copy of it -- a wrong 32 x 32
block (another tile's values, zeros, a 5% scale), one wrong element, a NaN, a ragged
tail left unwritten -- and the check must reject each, while the tensor-wide relative
Frobenius norm alone (the previous contract) accepts most of them.
"""

import numpy as np
import pytest
import torch

from floatcheck import errors, ok, stratified
from oracle import coracle as C

TOL = 1e-2


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(42)
    M, N, K, d = 200, 1000, 512, 8
    wp = rng.uniform(-0.5, 3.5, size=(N, K)).astype(np.float32)
    A = 0.02 * np.eye(d) + 0.002 * rng.normal(size=(d, d)) * (1 - np.eye(d))
    B = 0.01 * rng.normal(size=d)
    X = torch.randn(M, K, generator=torch.Generator().manual_seed(1)).bfloat16()
    f = C.linear_fwd(X.double().numpy(), wp, A, B, d)
    W16 = torch.from_numpy(f["What"]).bfloat16()
    gpu_like = (X.float() @ W16.float().T).bfloat16().double().numpy()
    return f["Y"], gpu_like


def test_realistic_result_passes(case):
    ref, g = case
    e = errors(g, ref)
    assert ok(e, TOL), e
    assert e["tensor"] < 5e-3


@pytest.mark.parametrize("defect", ["other_tile", "zero_block", "scale_block", "one_element",
                                    "nan", "tail_unwritten", "column_strip"])
def test_planted_defect_is_rejected(case, defect):
    ref, g = case
    bad = g.copy()
    if defect == "other_tile":          # a tile-index mix-up: block (64, 96) holds (0, 0)
        bad[64:96, 96:128] = g[0:32, 0:32]
    elif defect == "zero_block":
        bad[128:160, 512:544] = 0.0
    elif defect == "scale_block":        # a 5% error on one block (say, a wrong row term)
        bad[32:64, 32:64] *= 1.05
    elif defect == "one_element":
        bad[17, 333] = 0.0 if abs(g[17, 333]) > 0.5 else g[17, 333] + 1.0
    elif defect == "nan":
        bad[5, 5] = np.nan
    elif defect == "tail_unwritten":     # last 8 columns of the ragged tail never stored
        bad[:, -8:] = 0.0
    elif defect == "column_strip":       # one 32-column strip of a single row block
        bad[96:128, 992:1000] *= -1.0
    assert not ok(errors(bad, ref), TOL), defect


def test_tensor_norm_alone_misses_block_defects(case):
    """The reason for the block and element checks: these defects pass the tensor-wide
    contract on a 200 x 1000 result, and would on a larger one all the more."""
    ref, g = case
    missed = 0
    for sl, fn in [((slice(64, 96), slice(96, 128)), lambda b: b * 1.05),
                   ((slice(17, 18), slice(333, 334)), lambda b: b * 0.0),
                   ((slice(128, 160), slice(512, 544)), lambda b: b * 1.1)]:
        bad = g.copy()
        bad[sl] = fn(bad[sl])
        e = errors(bad, ref)
        missed += e["tensor"] <= TOL
        assert not ok(e, TOL)
    assert missed == 3


def test_zero_reference_needs_exact_zero():
    z = np.zeros((40, 40))
    assert ok(errors(z, z), TOL)
    w = z.copy()
    w[3, 3] = 1e-30
    assert not ok(errors(w, z), TOL)


def test_stratified_rows_cover_every_band():
    for n in (1024, 8192, 14336, 300, 64):
        rows = stratified(n, seed=n)
        assert len(set(rows.tolist())) == len(rows) and rows.min() >= 0 and rows.max() < n
        bands = set((rows // 256).tolist())
        assert bands == set(range((n + 255) // 256)), n
        assert len(rows) >= min(64, n)

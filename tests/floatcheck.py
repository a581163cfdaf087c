"""Float parity checks used by every GPU test (pinned by tests/test_floatcheck.py).

A floating-point result passes against its float64 oracle value when all three hold, tol
being the contract's bound (1e-2 for bf16-input, float32-accumulate products and
gradients; 1e-5 for the float32 decoded weights):

  1. tensor:  ||gpu - ref||_F / ||ref||_F <= tol            (the contract itself);
  2. block:   the same ratio on every 32 x 32 block <= tol, each block's reference norm
              floored at 1e-3 of the norm a block of that size has at the tensor's RMS,
              so that one wrong MFMA block, epilogue tile or ragged tail cannot hide in
              the norm of a large tensor;
  3. element: |gpu - ref| <= tol * (|ref| + 4 rms(ref)) for every element, so that one
              wrong element cannot hide in its block.

Non-finite GPU values fail. A reference that is exactly zero everywhere (a zero decode
matrix) must be matched exactly.
"""

import numpy as np

BLOCK = 32
FLOOR = 1e-3
ELEM_RMS = 4.0


def _as2d(a):
    a = np.asarray(a, dtype=np.float64)
    if a.ndim == 0:
        return a.reshape(1, 1)
    if a.ndim == 1:
        return a.reshape(1, -1)
    return a.reshape(-1, a.shape[-1])


def _block_sums(x, block):
    R, C = x.shape
    xp = np.pad(x, ((0, -R % block), (0, -C % block)))
    return xp.reshape(xp.shape[0] // block, block, xp.shape[1] // block, block).sum(axis=(1, 3))


def errors(gpu, ref, block=BLOCK):
    """The three figures of merit (each must be <= tol), plus where the worst block is."""
    g, r = _as2d(gpu), _as2d(ref)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if not np.all(np.isfinite(g)):
        return {"tensor": np.inf, "block": np.inf, "elem": np.inf, "worst_block": None,
                "nonfinite": int(np.count_nonzero(~np.isfinite(g)))}
    e = g - r
    rn = float(np.sqrt(np.sum(r * r)))
    en = float(np.sqrt(np.sum(e * e)))
    if rn == 0.0:
        z = 0.0 if en == 0.0 else np.inf
        return {"tensor": z, "block": z, "elem": z, "worst_block": None}
    rms = rn / np.sqrt(r.size)
    E2 = _block_sums(e * e, block)
    R2 = _block_sums(r * r, block)
    cnt = _block_sums(np.ones_like(r), block)
    den = np.maximum(np.sqrt(R2), FLOOR * rms * np.sqrt(cnt))
    blk = np.sqrt(E2) / den
    wb = np.unravel_index(int(np.argmax(blk)), blk.shape)
    elem = float(np.max(np.abs(e) / (np.abs(r) + ELEM_RMS * rms)))
    return {"tensor": en / rn, "block": float(blk.max()), "elem": elem,
            "worst_block": (int(wb[0]) * block, int(wb[1]) * block)}


def ok(errs, tol):
    return errs["tensor"] <= tol and errs["block"] <= tol and errs["elem"] <= tol


def check(gpu, ref, tol, label=""):
    """Raises AssertionError naming the failing figure; returns the figures."""
    errs = errors(gpu, ref)
    assert ok(errs, tol), f"{label}: {errs} (tol {tol})"
    return errs


def fmt(errs):
    return "/".join(f"{errs[k]:.1e}" for k in ("tensor", "block", "elem"))


def stratified(n, seed, band=256, total=64):
    """Sorted distinct indices in [0, n): one from every band of `band` consecutive
    indices, then more at random until `total` (or n) are drawn."""
    g = np.random.default_rng(seed)
    picks = {int(b + g.integers(0, min(band, n - b))) for b in range(0, n, band)}
    want = min(n, max(total, len(picks)))
    while len(picks) < want:
        picks.add(int(g.integers(0, n)))
    return np.array(sorted(picks), dtype=np.int64)

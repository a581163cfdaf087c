"""CPU oracle for the LC-VQ hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of the entry module and the CPU-baseline leg of
the benchmark may import this module. The GPU library never calls it, and it shares
no code, tables or constants with the HIP kernels.

Everything is written straight from the definitions, in float64 unless a step is an
integer decision. Sources (titles of the pages the method is described on):

* [LCQAT-M1]  "LC-QAT: Data-Efficient 2-Bit QAT for LLMs via Linear-Constrained Vector
  Quantization", technical summary, Methodology 1 (linear-constrained parametrization):
  a codeword is c = A z + B with z in {0,1,2,3}^d, and A (d x d) and B (d) are floats
  shared across one weight matrix; selecting z is rounding and clamping followed by the
  linear map, so the forward is lookup-free and gradients pass through the map.
* [LCQAT-M3]  same page, Methodology 3 (training pipeline): the forward rounds and clamps
  the proxy weights Wp into integer weights Wz and decodes them with A Wz + B before the
  matmul; the backward needs a gradient estimator through the rounding (the page names
  the straight-through estimator as the standard choice).
* [DQ-3.1]    "decoupleQ" (Chinese translation), section 3.1, eq. (3) and (4): scalar
  uniform quantization W^ = clip(round((W0 - z)/s), alpha, beta), W~ = W^ * s + z, with
  alpha = -2, beta = 1 for 2 bits.

Layout conventions (readings of what the pages leave open):
* a weight matrix is W[N, K] (N outputs, K inputs, as torch.nn.Linear stores it) and the
  layer computes Y = X W^T;
* the d-vectors run along K: vector (n, g) is W[n, g*d:(g+1)*d];
* A multiplies z as a column vector: What_i = B_i + sum_j A[i, j] z_j;
* rounding is round-half-to-even (numpy.rint);
* the straight-through mask is 1 exactly where the clamp did nothing, i.e. where
  0 <= rint(Wp) <= 3 (the literal autograd of clamp(round_ste(Wp), 0, 3));
* NaN proxies give code 0 and mask 0; +inf gives code 3 and mask 0; -inf gives code 0
  and mask 0.
* packing is little-endian: code k = 4b + t sits in bits [2t, 2t+1] of byte b, and mask
  bit k = 8c + t sits in bit t of mask byte c.

Parity of every function here is pinned by tests/test_oracle_pins.py (brute force,
special cases, closed forms, exact finite differences, a hand-worked example), except
dge_curve / dge_slope: parity unpinned against the pages, which give no DGE curve; they
are pinned only against their own definition (finite differences, limits, autograd).
"""

import numpy as np

__all__ = [
    "quantize", "pack2b", "unpack2b", "pack_mask", "unpack_mask", "reconstruct",
    "linear_fwd", "linear_bwd", "gemv2b", "nearest_codeword", "decoupleq_quant",
    "dge_curve", "dge_slope", "ptq_objective", "ptq_sweep_literal",
]


def quantize(wp):
    """Round and clamp proxy weights into 2-bit codes and the straight-through mask.

    [LCQAT-M1], [LCQAT-M3]: z = clamp(round(Wp), 0, 3). Returns (z uint8, m uint8) of
    the input's shape. The decision is taken on the float32 value itself (every float32
    is exact in float64, so rint gives the same integer in either precision).
    """
    w = np.asarray(wp, dtype=np.float32).astype(np.float64)
    r = np.rint(w)                                     # half to even
    finite = np.isfinite(r)
    m = finite & (r >= 0.0) & (r <= 3.0)
    z = np.zeros(w.shape, dtype=np.uint8)
    z[finite] = np.clip(r[finite], 0.0, 3.0).astype(np.uint8)
    z[np.isposinf(w)] = 3
    return z, m.astype(np.uint8)


def pack2b(z):
    """Four 2-bit codes per byte, little-endian along the last axis (K % 4 == 0)."""
    z = np.asarray(z, dtype=np.uint8)
    if z.shape[-1] % 4:
        raise ValueError("last dimension must be a multiple of 4")
    q = z.reshape(z.shape[:-1] + (z.shape[-1] // 4, 4)).astype(np.uint32)
    out = q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)
    return out.astype(np.uint8)


def unpack2b(packed, k):
    """Inverse of pack2b: bytes [..., k/4] -> codes [..., k]."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.uint32)
    if p.shape[-1] * 4 != k:
        raise ValueError("packed width does not match k")
    parts = [(p >> (2 * t)) & 3 for t in range(4)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (k,)).astype(np.uint8)


def pack_mask(m):
    """Eight mask bits per byte, little-endian along the last axis (K % 8 == 0)."""
    m = np.asarray(m, dtype=np.uint8)
    if m.shape[-1] % 8:
        raise ValueError("last dimension must be a multiple of 8")
    q = m.reshape(m.shape[:-1] + (m.shape[-1] // 8, 8)).astype(np.uint32)
    out = np.zeros(q.shape[:-1], dtype=np.uint32)
    for t in range(8):
        out |= (q[..., t] & 1) << t
    return out.astype(np.uint8)


def unpack_mask(bits, k):
    b = np.asarray(bits, dtype=np.uint8).astype(np.uint32)
    parts = [(b >> t) & 1 for t in range(8)]
    return np.stack(parts, axis=-1).reshape(b.shape[:-1] + (k,)).astype(np.uint8)


def reconstruct(z, A, B, d):
    """Decoded weights: What[n, g*d + i] = B[i] + sum_j A[i, j] * z[n, g*d + j].

    [LCQAT-M1] c = A z + B, applied to every d-vector along the input dimension.
    """
    z = np.asarray(z)
    n, k = z.shape
    if k % d:
        raise ValueError("K must be a multiple of d")
    A = np.asarray(A, dtype=np.float64).reshape(d, d)
    B = np.asarray(B, dtype=np.float64).reshape(d)
    zv = z.astype(np.float64).reshape(n, k // d, d)
    w = np.einsum("ij,ngj->ngi", A, zv) + B
    return w.reshape(n, k)


def linear_fwd(X, wp, A, B, d):
    """One forward of an LC-VQ linear layer, [LCQAT-M3].

    Returns a dict with z, m, What (float64) and Y = X What^T (float64), plus the
    packed codes and mask bytes when K is a multiple of 8. X is taken at the exact
    values given (the caller passes the bf16 or float32 values the GPU saw).
    """
    z, m = quantize(wp)
    w = reconstruct(z, A, B, d)
    Y = np.asarray(X, dtype=np.float64) @ w.T
    out = {"z": z, "m": m, "What": w, "Y": Y}
    if z.shape[1] % 8 == 0:
        out["packed"] = pack2b(z)
        out["maskbits"] = pack_mask(m)
    return out


def dge_curve(w, alpha):
    """Smooth stand-in for rounding used by the DGE backward.

    [LCQAT-M3] says only that LC-QAT's differentiable gradient estimator (DGE)
    approximates the discretization with a smooth, differentiable curve and uses its
    gradient instead of the straight-through one; the curve itself is not given. The
    family used here (this implementation's reading, parity unpinned against the pages):
      s(w) = floor(w) + 1/2 + tanh(alpha (f - 1/2)) / (2 tanh(alpha / 2)),  f = w - floor(w)
    It passes through every integer, is steepest at the half-integers where rounding
    jumps, tends to s(w) = w (the straight-through estimator) as alpha -> 0 and to
    rounding as alpha -> infinity.
    """
    w = np.asarray(w, dtype=np.float64)
    n = np.floor(w)
    f = w - n
    return n + 0.5 + np.tanh(alpha * (f - 0.5)) / (2.0 * np.tanh(alpha / 2.0))


def dge_slope(w, alpha):
    """Derivative of dge_curve: alpha (1 - tanh^2(alpha (f - 1/2))) / (2 tanh(alpha / 2)).
    Zero for non-finite w (those weights are masked by the clamp anyway)."""
    w = np.asarray(w, dtype=np.float64)
    out = np.zeros(w.shape)
    fin = np.isfinite(w)
    f = w[fin] - np.floor(w[fin])
    t = np.tanh(alpha * (f - 0.5))
    out[fin] = alpha * (1.0 - t * t) / (2.0 * np.tanh(alpha / 2.0))
    return out


def linear_bwd(dY, X, z, m, A, B, d, wp=None, dge_alpha=None):
    """Straight-through backward of Y = X What(z, A, B)^T.

    Standard backpropagation through the linear decode [LCQAT-M1]; the rounding is
    passed straight through, masked where the clamp was active [LCQAT-M3]:
      dX  = dY What
      G   = dY^T X                         (gradient w.r.t. What, never returned)
      dWp[n, g*d + j] = m[n, g*d + j] * sum_i A[i, j] G[n, g*d + i]
      dA[i, j] = sum over vectors (n, g) of G[n, g*d + i] * z[n, g*d + j]
      dB[i]    = sum over vectors (n, g) of G[n, g*d + i]
    With dge_alpha (and the proxies wp) the rounding's gradient is dge_slope(wp) instead
    of 1, still masked by the clamp: dWp is multiplied elementwise by dge_slope(wp).
    """
    dY = np.asarray(dY, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64).reshape(d, d)
    n, k = z.shape
    w = reconstruct(z, A, B, d)
    dX = dY @ w
    G = dY.T @ X
    gv = G.reshape(n, k // d, d)
    zv = z.astype(np.float64).reshape(n, k // d, d)
    dW_hat_to_wp = np.einsum("ij,ngi->ngj", A, gv).reshape(n, k)
    dWp = dW_hat_to_wp * np.asarray(m, dtype=np.float64)
    if dge_alpha is not None:
        dWp = dWp * dge_slope(np.asarray(wp, dtype=np.float32), dge_alpha)
    dA = np.einsum("ngi,ngj->ij", gv, zv)
    dB = gv.sum(axis=(0, 1))
    return {"dX": dX, "dWp": dWp, "dA": dA, "dB": dB}


def gemv2b(X, packed, A, B, d):
    """Decode-time product Y = X What^T from packed codes and (fp16-widened) A, B.

    The deployed artefact is the integer part plus the float part, and one linear
    transform turns it back into weights (decoupleQ, section 3.2; [LCQAT-M3]).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    k = packed.shape[1] * 4
    z = unpack2b(packed, k)
    w = reconstruct(z, A, B, d)
    return np.asarray(X, dtype=np.float64) @ w.T


def nearest_codeword(w, A, B):
    """Brute-force nearest codeword of one d-vector w over all 4^d codes z.

    The search that vector quantization performs and that LC-VQ replaces
    ([LCQAT-M1]): argmin_z || (A z + B) - (A w + B) ||. Ties resolve to the first
    code in lexicographic order. Test use only (d <= 8).
    """
    A = np.asarray(A, dtype=np.float64)
    d = A.shape[0]
    grid = np.array(np.meshgrid(*([np.arange(4)] * d), indexing="ij"))
    codes = grid.reshape(d, -1).T.astype(np.float64)       # [4^d, d], lexicographic
    target = A @ np.asarray(w, dtype=np.float64) + np.asarray(B, dtype=np.float64)
    cw = codes @ A.T + np.asarray(B, dtype=np.float64)
    dist = ((cw - target) ** 2).sum(axis=1)
    return codes[int(np.argmin(dist))].astype(np.uint8)


def decoupleq_quant(W0, s, zero, alpha=-2, beta=1):
    """Scalar uniform quantization, [DQ-3.1] eq. (3) and (4).

    Returns (integer part W^, dequantized W~). Written independently of quantize()
    so that the per-tensor special case A = s I, B = b 1 can be checked against it.
    """
    W0 = np.asarray(W0, dtype=np.float64)
    q = np.clip(np.rint((W0 - zero) / s), alpha, beta)
    return q, q * s + zero


def ptq_objective(W0, c, Hd, s, b):
    """[DQ-3.1] eq. (5)/(7) per output row, summed: 1/2 sum_n r_n^T Hd r_n with
    r_n = s c_n + b - w0_n (the decoded weight's error; LC codes c = W^ + 2)."""
    R = s * np.asarray(c, np.float64) + b - np.asarray(W0, np.float64)
    return 0.5 * float(np.sum((R @ np.asarray(Hd, np.float64)) * R))


def ptq_sweep_literal(W0, Hd, s, b):
    """decoupleQ section 3.3's integer step taken literally, for small K only: element j
    is rounded and clipped to {0..3} from the current continuous solution, then the
    elements after j are re-solved by the unconstrained minimiser of the objective with
    elements 0..j fixed (eq. (11)), by a linear solve at every step."""
    W0 = np.asarray(W0, np.float64)
    Hd = np.asarray(Hd, np.float64)
    N, K = W0.shape
    out = np.zeros((N, K), np.uint8)
    for n in range(N):
        v = (W0[n] - b) / s                 # minimiser with nothing fixed: s c + b = w0
        x = v.copy()
        c = np.zeros(K)
        for j in range(K):
            c[j] = np.clip(np.rint(x[j]), 0, 3)
            if j + 1 < K:
                P, F = slice(0, j + 1), slice(j + 1, K)
                d_p = c[P] - v[P]
                x[F] = v[F] - np.linalg.solve(Hd[F, F], Hd[F, P] @ d_p)
        out[n] = c.astype(np.uint8)
    return out

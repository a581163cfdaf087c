"""Python face of the plain C++ oracle (oracle/lcvq_oracle.cpp) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of the entry module and the CPU-baseline leg of the
benchmark may import this module. It loads oracle/liblcvq_oracle.so (built by
oracle/build_oracle.py, which the entry module's build() runs) and exposes the same
functions, with the same arguments and results, as the numpy oracle in lcvq_oracle.py,
so that every pin can be run against both. Arithmetic happens in the C++ library only;
this file converts arrays and allocates results.

Extra arguments over the numpy oracle: `rows` selects output rows (rows of X for the
forward and dX, rows of the weight for dWp and the decode product), so that samples of
a large layer cost only their own rows. dA and dB are then sums over the vectors of the
selected weight rows.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblcvq_oracle.so")
_lib = None

__all__ = ["quantize", "pack2b", "unpack2b", "pack_mask", "unpack_mask", "reconstruct",
           "linear_fwd", "linear_bwd", "gemv2b", "dge_slope", "threads", "lib",
           "hessian", "damp", "udu", "ptq_objective", "ptq_sweep", "ptq_solve_sb", "ptq_init",
           "ptq_targets"]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python oracle/build_oracle.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sigs = {
            "oc_threads": ([], i32),
            "oc_quantize": ([vp, i64, vp, vp], None),
            "oc_pack2b": ([vp, i64, i64, vp], None),
            "oc_unpack2b": ([vp, i64, i64, vp], None),
            "oc_pack_mask": ([vp, i64, i64, vp], None),
            "oc_unpack_mask": ([vp, i64, i64, vp], None),
            "oc_reconstruct": ([vp, i64, i64, i32, vp, vp, vp], None),
            "oc_forward": ([vp, i64, i64, vp, i64, vp, i64, vp], None),
            "oc_backward_dx": ([vp, i64, i64, vp, i64, vp, i64, vp], None),
            "oc_backward_dw": ([vp, vp, i64, i64, i64, i32, vp, vp, vp, vp, f64, vp, i64, vp,
                                vp, vp], None),
            "oc_dge_slope": ([vp, i64, f64, vp], None),
            "oc_gemv2b": ([vp, i64, i64, vp, i64, i32, vp, vp, vp, i64, vp], None),
            "oc_hessian": ([vp, i64, i64, vp], None),
            "oc_damp": ([vp, i64, f64, vp], None),
            "oc_udu": ([vp, i64, vp, vp], i32),
            "oc_ptq_objective": ([vp, vp, i64, i64, vp, f64, f64], f64),
            "oc_ptq_sweep": ([vp, i64, i64, vp, f64, f64, vp, vp], None),
            "oc_ptq_solve_sb": ([vp, vp, i64, i64, vp, vp, vp], i32),
            "oc_ptq_targets": ([vp, i64, i64, vp, f64, f64, vp, vp], None),
            "oc_ptq_init": ([vp, i64, i64, vp, f64, i32, vp, vp, vp, vp], i32),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def threads():
    """OpenMP threads the oracle runs on."""
    return int(lib().oc_threads())


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _rows(rows):
    if rows is None:
        return None, 0
    r = _c(rows, np.int64)
    return r, r.size


def quantize(wp):
    w = _c(wp, np.float32)
    z = np.empty(w.shape, np.uint8)
    m = np.empty(w.shape, np.uint8)
    lib().oc_quantize(_p(w), w.size, _p(z), _p(m))
    return z, m


def _rowsk(a):
    a = np.asarray(a)
    return (1, a.shape[0]) if a.ndim == 1 else (int(np.prod(a.shape[:-1])), a.shape[-1])


def pack2b(z):
    z = _c(z, np.uint8)
    if z.shape[-1] % 4:
        raise ValueError("last dimension must be a multiple of 4")
    r, k = _rowsk(z)
    out = np.empty(z.shape[:-1] + (k // 4,), np.uint8)
    lib().oc_pack2b(_p(z), r, k, _p(out))
    return out


def unpack2b(packed, k):
    p = _c(packed, np.uint8)
    if p.shape[-1] * 4 != k:
        raise ValueError("packed width does not match k")
    r, _ = _rowsk(p)
    out = np.empty(p.shape[:-1] + (k,), np.uint8)
    lib().oc_unpack2b(_p(p), r, k, _p(out))
    return out


def pack_mask(m):
    m = _c(m, np.uint8)
    if m.shape[-1] % 8:
        raise ValueError("last dimension must be a multiple of 8")
    r, k = _rowsk(m)
    out = np.empty(m.shape[:-1] + (k // 8,), np.uint8)
    lib().oc_pack_mask(_p(m), r, k, _p(out))
    return out


def unpack_mask(bits, k):
    b = _c(bits, np.uint8)
    r, _ = _rowsk(b)
    out = np.empty(b.shape[:-1] + (k,), np.uint8)
    lib().oc_unpack_mask(_p(b), r, k, _p(out))
    return out


def reconstruct(z, A, B, d):
    z = _c(z, np.uint8)
    n, k = z.shape
    if k % d:
        raise ValueError("K must be a multiple of d")
    Ac, Bc = _c(np.asarray(A).reshape(d, d), np.float64), _c(np.asarray(B).reshape(d), np.float64)
    w = np.empty((n, k), np.float64)
    lib().oc_reconstruct(_p(z), n, k, d, _p(Ac), _p(Bc), _p(w))
    return w


def linear_fwd(X, wp, A, B, d, rows=None):
    """As lcvq_oracle.linear_fwd; with `rows`, Y holds only those rows of X."""
    z, m = quantize(wp)
    w = reconstruct(z, A, B, d)
    Xc = _c(X, np.float64)
    M, K = Xc.shape
    r, nr = _rows(rows)
    Y = np.empty((nr if r is not None else M, w.shape[0]), np.float64)
    lib().oc_forward(_p(Xc), M, K, _p(w), w.shape[0], _p(r), nr, _p(Y))
    out = {"z": z, "m": m, "What": w, "Y": Y}
    if z.shape[1] % 8 == 0:
        out["packed"] = pack2b(z)
        out["maskbits"] = pack_mask(m)
    return out


def dge_slope(w, alpha):
    w = _c(w, np.float64)
    out = np.empty(w.shape, np.float64)
    lib().oc_dge_slope(_p(w), w.size, float(alpha), _p(out))
    return out


def linear_bwd(dY, X, z, m, A, B, d, wp=None, dge_alpha=None, dx_rows=None, dw_rows=None,
               want_dx=True):
    """As lcvq_oracle.linear_bwd. dx_rows selects rows of dX (rows of dY); dw_rows selects
    weight rows for dWp, and dA, dB are then sums over those rows' vectors."""
    dYc, Xc = _c(dY, np.float64), _c(X, np.float64)
    z, m = _c(z, np.uint8), _c(m, np.uint8)
    M, N = dYc.shape
    K = Xc.shape[1]
    Ac, Bc = _c(np.asarray(A).reshape(d, d), np.float64), _c(np.asarray(B).reshape(d), np.float64)
    out = {}
    if want_dx:
        w = reconstruct(z, Ac, Bc, d)
        r, nr = _rows(dx_rows)
        dX = np.empty((nr if r is not None else M, K), np.float64)
        lib().oc_backward_dx(_p(dYc), M, N, _p(w), K, _p(r), nr, _p(dX))
        out["dX"] = dX
    r, nr = _rows(dw_rows)
    dWp = np.empty((nr if r is not None else N, K), np.float64)
    dA = np.empty((d, d), np.float64)
    dB = np.empty((d,), np.float64)
    wpc = None if dge_alpha is None else _c(wp, np.float32)
    lib().oc_backward_dw(_p(dYc), _p(Xc), M, N, K, d, _p(z), _p(m), _p(Ac), _p(wpc),
                         float(dge_alpha or 0.0), _p(r), nr, _p(dWp), _p(dA), _p(dB))
    out.update({"dWp": dWp, "dA": dA, "dB": dB})
    return out


def gemv2b(X, packed, A, B, d, rows=None):
    """As lcvq_oracle.gemv2b; with `rows`, Y holds only those weight rows (columns of Y)."""
    Xc = _c(X, np.float64)
    pk = _c(packed, np.uint8)
    M, K = Xc.shape
    N = pk.shape[0]
    Ac, Bc = _c(np.asarray(A).reshape(d, d), np.float64), _c(np.asarray(B).reshape(d), np.float64)
    r, nr = _rows(rows)
    Y = np.empty((M, nr if r is not None else N), np.float64)
    lib().oc_gemv2b(_p(Xc), M, K, _p(pk), N, d, _p(Ac), _p(Bc), _p(r), nr, _p(Y))
    return Y


# ---------------------------------------------------------------- PTQ initialisation
def hessian(X):
    """H = X^T X for calibration activations X [M, K]."""
    Xc = _c(X, np.float64)
    M, K = Xc.shape
    H = np.empty((K, K), np.float64)
    lib().oc_hessian(_p(Xc), M, K, _p(H))
    return H


def damp(H, dmp):
    """H + dmp * mean(diag(H)) I."""
    Hc = _c(H, np.float64)
    out = np.empty_like(Hc)
    lib().oc_damp(_p(Hc), Hc.shape[0], float(dmp), _p(out))
    return out


def udu(Hd):
    """(U, D) with Hd = U diag(D) U^T, U unit upper triangular."""
    Hc = _c(Hd, np.float64)
    K = Hc.shape[0]
    U = np.empty((K, K), np.float64)
    D = np.empty(K, np.float64)
    bad = lib().oc_udu(_p(Hc), K, _p(U), _p(D))
    if bad:
        raise ValueError(f"matrix not positive definite (pivot {bad - 1})")
    return U, D


def ptq_objective(W0, c, Hd, s, b):
    W = _c(W0, np.float64)
    cc = _c(c, np.uint8)
    Hc = _c(Hd, np.float64)
    N, K = W.shape
    return float(lib().oc_ptq_objective(_p(W), _p(cc), N, K, _p(Hc), float(s), float(b)))


def ptq_sweep(W0, U, s, b, want_t=False):
    """The integer step for fixed (s, b): codes [N, K] (and the continuous targets t)."""
    W = _c(W0, np.float64)
    Uc = _c(U, np.float64)
    N, K = W.shape
    c = np.empty((N, K), np.uint8)
    t = np.empty((N, K), np.float64) if want_t else None
    lib().oc_ptq_sweep(_p(W), N, K, _p(Uc), float(s), float(b), _p(c), _p(t))
    return (c, t) if want_t else c


def ptq_targets(W0, U, s, b, c):
    """The values t the integer step rounds, driven by the given codes c (teacher forcing)."""
    W = _c(W0, np.float64)
    Uc = _c(U, np.float64)
    cc = _c(c, np.uint8)
    N, K = W.shape
    t = np.empty((N, K), np.float64)
    lib().oc_ptq_targets(_p(W), N, K, _p(Uc), float(s), float(b), _p(cc), _p(t))
    return t


def ptq_solve_sb(W0, c, Hd, s=1.0, b=0.0):
    """The (s, b) step for fixed codes; returns (s, b, singular)."""
    W = _c(W0, np.float64)
    cc = _c(c, np.uint8)
    Hc = _c(Hd, np.float64)
    N, K = W.shape
    sv = ctypes.c_double(s)
    bv = ctypes.c_double(b)
    sing = lib().oc_ptq_solve_sb(_p(W), _p(cc), N, K, _p(Hc), ctypes.byref(sv), ctypes.byref(bv))
    return sv.value, bv.value, bool(sing)


def ptq_init(W0, H, dmp, iters):
    """The whole initialisation from H = X^T X: returns codes [N, K], s, b and the
    objective after each of the 2 * iters steps."""
    W = _c(W0, np.float64)
    Hc = _c(H, np.float64)
    N, K = W.shape
    c = np.empty((N, K), np.uint8)
    sv, bv = ctypes.c_double(0.0), ctypes.c_double(0.0)
    obj = np.empty(2 * iters, np.float64)
    bad = lib().oc_ptq_init(_p(W), N, K, _p(Hc), float(dmp), int(iters), _p(c),
                            ctypes.byref(sv), ctypes.byref(bv), _p(obj))
    if bad:
        raise ValueError(f"damped H not positive definite (pivot {bad - 1})")
    return {"codes": c, "s": sv.value, "b": bv.value, "obj": obj}

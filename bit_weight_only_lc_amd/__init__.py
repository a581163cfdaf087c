"""Python binding of liblcvq.so, the LC-VQ hot path on MI355X (gfx950).

Argument marshalling only: every function here checks tensor dtypes, devices and
contiguity, then passes raw device pointers and the current HIP stream to the C ABI
declared in include/lcvq.h. All arithmetic runs in the library's HIP kernels; if the
library is missing the import of any entry point raises.

Names follow the C ABI (lcvq_quantize, lcvq_pack2b, lcvq_unpack2b, lcvq_linear_fwd,
lcvq_linear_bwd, lcvq_linear_bwd_dge, lcvq_gemv2b, lcvq_gemv2b_noalloc,
lcvq_gemv2b_batched, lcvq_hessian, lcvq_ptq_init and the *_workspace_size helpers).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblcvq.so")

LCVQ_F32, LCVQ_BF16 = 0, 1
_STATUS = {0: "LCVQ_OK", 1: "LCVQ_ERR_NULL", 2: "LCVQ_ERR_SHAPE", 3: "LCVQ_ERR_D",
           4: "LCVQ_ERR_DTYPE", 5: "LCVQ_ERR_ALIGN", 6: "LCVQ_ERR_WORKSPACE", 7: "LCVQ_ERR_HIP",
           8: "LCVQ_ERR_VALUE", 9: "LCVQ_ERR_SCRATCH"}

_lib = None


class GemvMatrix(ctypes.Structure):
    """lcvq_gemv2b_matrix: one matrix of a batched decode product."""
    _fields_ = [("packed", ctypes.c_void_p), ("A16", ctypes.c_void_p), ("B16", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("N", ctypes.c_int64), ("layout", ctypes.c_int32)]


class LcvqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} "
                         f"({lib().lcvq_status_string(status).decode()})")


def lib():
    """The loaded liblcvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m bit_weight_only_lc_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        f32 = ctypes.c_float
        L.lcvq_status_string.restype = ctypes.c_char_p
        L.lcvq_status_string.argtypes = [i32]
        sigs = {
            "lcvq_quantize": [vp, i64, i64, vp, vp, vp, vp],
            "lcvq_pack2b": [vp, i64, i64, vp, vp],
            "lcvq_unpack2b": [vp, i64, i64, vp, vp],
            "lcvq_linear_fwd": [vp, i32, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                sz, vp],
            "lcvq_linear_bwd": [vp, vp, i32, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp,
                                vp, vp, sz, vp],
            "lcvq_linear_bwd_dge": [vp, vp, i32, i64, i64, i64, i32, vp, vp, vp, f32, vp, vp,
                                    vp, vp, vp, vp, vp, sz, vp],
            "lcvq_gemv2b": [vp, i64, i64, i64, i32, vp, vp, vp, vp, vp, sz, vp],
            "lcvq_gemv2b_shuffled": [vp, i64, i64, i64, i32, vp, vp, vp, vp, vp, sz, vp],
            "lcvq_gemv2b_shuffle": [vp, i64, i64, vp, vp],
            "lcvq_gemv2b_noalloc": [vp, i64, i64, i64, i32, vp, vp, vp, vp, vp],
            "lcvq_hessian": [vp, i64, i64, vp, vp],
            "lcvq_read_probe": [vp, i64, vp, vp],
            "lcvq_mfma_probe": [i64, vp, vp],
            "lcvq_ptq_init": [vp, vp, i64, i64, f32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
        }
        for name, args in sigs.items():
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = args
        for name in ("lcvq_linear_fwd_workspace_size", "lcvq_linear_bwd_workspace_size"):
            f = getattr(L, name)
            f.restype = sz
            f.argtypes = [i64, i64, i64, i32]
        L.lcvq_gemv2b_batched.restype = i32
        L.lcvq_gemv2b_batched.argtypes = [vp, i64, i64, i32, ctypes.POINTER(GemvMatrix), i32,
                                          vp, sz, vp]
        L.lcvq_ptq_workspace_size.restype = sz
        L.lcvq_ptq_workspace_size.argtypes = [i64, i64]
        L.lcvq_gemv2b_workspace_size.restype = sz
        L.lcvq_gemv2b_workspace_size.argtypes = [i64, i64, i64, i32]
        L.lcvq_profile_next.restype = i32
        L.lcvq_profile_next.argtypes = [i32, vp, vp]
        _lib = L
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ok(status, where):
    if status != 0:
        raise LcvqError(status, where)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return LCVQ_BF16
    if t.dtype == torch.float32:
        return LCVQ_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {t.dtype}")


# ------------------------------------------------------------------ workspace sizes
def lcvq_linear_fwd_workspace_size(M, N, K, d):
    return int(lib().lcvq_linear_fwd_workspace_size(M, N, K, d))


def lcvq_linear_bwd_workspace_size(M, N, K, d):
    return int(lib().lcvq_linear_bwd_workspace_size(M, N, K, d))


def lcvq_gemv2b_workspace_size(M, N, K, d):
    return int(lib().lcvq_gemv2b_workspace_size(M, N, K, d))


# ------------------------------------------------------------------ entry points
def lcvq_quantize(Wp, z_u8=None, packed=None, mask=None):
    _check(Wp, "Wp", torch.float32)
    dev = Wp.device
    for t, n in ((z_u8, "z_u8"), (packed, "packed"), (mask, "mask")):
        _check(t, n, torch.uint8, dev)
    N, K = Wp.shape
    _ok(lib().lcvq_quantize(_p(Wp), N, K, _p(z_u8), _p(packed), _p(mask), _stream(dev)),
        "lcvq_quantize")


def lcvq_pack2b(z_u8, packed):
    _check(z_u8, "z_u8", torch.uint8)
    _check(packed, "packed", torch.uint8, z_u8.device)
    N, K = z_u8.shape
    _ok(lib().lcvq_pack2b(_p(z_u8), N, K, _p(packed), _stream(z_u8.device)), "lcvq_pack2b")


def lcvq_unpack2b(packed, z_u8):
    _check(packed, "packed", torch.uint8)
    _check(z_u8, "z_u8", torch.uint8, packed.device)
    N, K = z_u8.shape
    _ok(lib().lcvq_unpack2b(_p(packed), N, K, _p(z_u8), _stream(packed.device)),
        "lcvq_unpack2b")


def lcvq_linear_fwd(X, Wp, A, B, d, Y, packed_out, mask_out, What_out=None, workspace=None):
    _check(X, "X", (torch.bfloat16, torch.float32))
    dev = X.device
    _check(Wp, "Wp", torch.float32, dev)
    _check(A, "A", torch.float32, dev)
    _check(B, "B", torch.float32, dev)
    _check(Y, "Y", X.dtype, dev)
    _check(packed_out, "packed_out", torch.uint8, dev)
    _check(mask_out, "mask_out", torch.uint8, dev)
    _check(What_out, "What_out", torch.float32, dev)
    M, K = X.shape
    N = Wp.shape[0]
    if workspace is None:
        workspace = torch.empty(max(lcvq_linear_fwd_workspace_size(M, N, K, d), 1),
                                dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, dev)
    _ok(lib().lcvq_linear_fwd(_p(X), _dt(X), M, N, K, d, _p(Wp), _p(A), _p(B), _p(Y),
                              _p(packed_out), _p(mask_out), _p(What_out), _p(workspace),
                              workspace.numel(), _stream(dev)), "lcvq_linear_fwd")


def lcvq_linear_bwd(dY, X, packed, mask, A, B, d, dX, dWp, dA, dB, workspace=None):
    _check(dY, "dY", (torch.bfloat16, torch.float32))
    dev = dY.device
    _check(X, "X", dY.dtype, dev)
    _check(packed, "packed", torch.uint8, dev)
    _check(mask, "mask", torch.uint8, dev)
    _check(A, "A", torch.float32, dev)
    _check(B, "B", torch.float32, dev)
    _check(dX, "dX", dY.dtype, dev)
    _check(dWp, "dWp", torch.float32, dev)
    _check(dA, "dA", torch.float32, dev)
    _check(dB, "dB", torch.float32, dev)
    M, N = dY.shape
    K = X.shape[1]
    if workspace is None:
        workspace = torch.empty(max(lcvq_linear_bwd_workspace_size(M, N, K, d), 1),
                                dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, dev)
    _ok(lib().lcvq_linear_bwd(_p(dY), _p(X), _dt(dY), M, N, K, d, _p(packed), _p(mask),
                              _p(A), _p(B), _p(dX), _p(dWp), _p(dA), _p(dB), _p(workspace),
                              workspace.numel(), _stream(dev)), "lcvq_linear_bwd")


def lcvq_linear_bwd_dge(dY, X, packed, mask, Wp, alpha, A, B, d, dX, dWp, dA, dB,
                        workspace=None):
    _check(dY, "dY", (torch.bfloat16, torch.float32))
    dev = dY.device
    _check(X, "X", dY.dtype, dev)
    _check(packed, "packed", torch.uint8, dev)
    _check(mask, "mask", torch.uint8, dev)
    _check(Wp, "Wp", torch.float32, dev)
    _check(A, "A", torch.float32, dev)
    _check(B, "B", torch.float32, dev)
    _check(dX, "dX", dY.dtype, dev)
    _check(dWp, "dWp", torch.float32, dev)
    _check(dA, "dA", torch.float32, dev)
    _check(dB, "dB", torch.float32, dev)
    M, N = dY.shape
    K = X.shape[1]
    if workspace is None:
        workspace = torch.empty(max(lcvq_linear_bwd_workspace_size(M, N, K, d), 1),
                                dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, dev)
    _ok(lib().lcvq_linear_bwd_dge(_p(dY), _p(X), _dt(dY), M, N, K, d, _p(packed), _p(mask),
                                  _p(Wp), float(alpha), _p(A), _p(B), _p(dX), _p(dWp), _p(dA),
                                  _p(dB), _p(workspace), workspace.numel(), _stream(dev)),
        "lcvq_linear_bwd_dge")


def lcvq_gemv2b(X, packed, A16, B16, d, Y, workspace=None):
    _gemv2b("lcvq_gemv2b", X, packed, A16, B16, d, Y, workspace)


def lcvq_gemv2b_noalloc(X, packed, A16, B16, d, Y):
    """lcvq_gemv2b on the library's fixed scratch: no workspace, nothing allocated."""
    _check(X, "X", torch.bfloat16)
    dev = X.device
    _check(packed, "packed", torch.uint8, dev)
    _check(A16, "A16", torch.float16, dev)
    _check(B16, "B16", torch.float16, dev)
    _check(Y, "Y", torch.bfloat16, dev)
    M, K = X.shape
    N = packed.shape[0]
    _ok(lib().lcvq_gemv2b_noalloc(_p(X), M, N, K, d, _p(packed), _p(A16), _p(B16), _p(Y),
                                  _stream(dev)), "lcvq_gemv2b_noalloc")


def lcvq_gemv2b_shuffled(X, codes, A16, B16, d, Y, workspace=None):
    """codes: the decode layout written by lcvq_gemv2b_shuffle, held as uint8 [N, K/4]."""
    _gemv2b("lcvq_gemv2b_shuffled", X, codes, A16, B16, d, Y, workspace)


def lcvq_gemv2b_shuffle(packed, codes):
    dev = packed.device
    _check(packed, "packed", torch.uint8, dev)
    _check(codes, "codes", torch.uint8, dev)
    if codes.shape != packed.shape:
        raise ValueError("codes must have the shape of packed")
    N, K4 = packed.shape
    _ok(lib().lcvq_gemv2b_shuffle(_p(packed), N, K4 * 4, _p(codes), _stream(dev)),
        "lcvq_gemv2b_shuffle")


def _gemv2b(name, X, packed, A16, B16, d, Y, workspace):
    _check(X, "X", torch.bfloat16)
    dev = X.device
    _check(packed, "packed", torch.uint8, dev)
    _check(A16, "A16", torch.float16, dev)
    _check(B16, "B16", torch.float16, dev)
    _check(Y, "Y", torch.bfloat16, dev)
    M, K = X.shape
    N = packed.shape[0]
    if workspace is None:
        workspace = torch.empty(max(lcvq_gemv2b_workspace_size(M, N, K, d), 1),
                                dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, dev)
    _ok(getattr(lib(), name)(_p(X), M, N, K, d, _p(packed), _p(A16), _p(B16), _p(Y),
                             _p(workspace), workspace.numel(), _stream(dev)), name)


def lcvq_gemv2b_batched(X, mats, d, workspace=None):
    """mats: list of (packed, A16, B16, Y) or (packed, A16, B16, Y, layout) sharing the
    input X; layout 1 means codes in the decode layout of lcvq_gemv2b_shuffle."""
    _check(X, "X", torch.bfloat16)
    dev = X.device
    M, K = X.shape
    arr = (GemvMatrix * max(len(mats), 1))()
    nmax = 16
    for i, m in enumerate(mats):
        pk, a16, b16, y = m[:4]
        layout = m[4] if len(m) > 4 else 0
        _check(pk, "packed", torch.uint8, dev)
        _check(a16, "A16", torch.float16, dev)
        _check(b16, "B16", torch.float16, dev)
        _check(y, "Y", torch.bfloat16, dev)
        arr[i] = GemvMatrix(pk.data_ptr(), a16.data_ptr(), b16.data_ptr(), y.data_ptr(),
                            pk.shape[0], int(layout))
        nmax = max(nmax, pk.shape[0])
    if workspace is None:
        workspace = torch.empty(max(lcvq_gemv2b_workspace_size(M, nmax, K, d), 1),
                                dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, dev)
    _ok(lib().lcvq_gemv2b_batched(_p(X), M, K, d, arr, len(mats), _p(workspace),
                                  workspace.numel(), _stream(dev)), "lcvq_gemv2b_batched")


def lcvq_mfma_probe(iters, sink):
    """Measurement helper: iters * 2^29 flops of bf16 MFMA issue into sink (int32 [1024])."""
    _check(sink, "sink", torch.int32)
    _ok(lib().lcvq_mfma_probe(int(iters), _p(sink), _stream(sink.device)), "lcvq_mfma_probe")


def lcvq_read_probe(buf, sink):
    """Measurement helper: stream buf once (uint8 device tensor) into sink (int32 [1024])."""
    _check(buf, "buf", torch.uint8)
    _check(sink, "sink", torch.int32, buf.device)
    _ok(lib().lcvq_read_probe(_p(buf), buf.numel(), _p(sink), _stream(buf.device)),
        "lcvq_read_probe")


def lcvq_hessian(X, H):
    """H = X^T X (X bf16 [M, K], H float32 [K, K])."""
    _check(X, "X", torch.bfloat16)
    _check(H, "H", torch.float32, X.device)
    M, K = X.shape
    _ok(lib().lcvq_hessian(_p(X), M, K, _p(H), _stream(X.device)), "lcvq_hessian")


def lcvq_ptq_workspace_size(N, K):
    return int(lib().lcvq_ptq_workspace_size(N, K))


def lcvq_ptq_init(H, W0, damp, iters, packed_out, sb_out, obj_out=None, U_out=None,
                  D_out=None, workspace=None):
    _check(H, "H", torch.float32)
    dev = H.device
    _check(W0, "W0", torch.float32, dev)
    _check(packed_out, "packed_out", torch.uint8, dev)
    _check(sb_out, "sb_out", torch.float32, dev)
    for t, n in ((obj_out, "obj_out"), (U_out, "U_out"), (D_out, "D_out")):
        _check(t, n, torch.float32, dev)
    N, K = W0.shape
    if workspace is None:
        workspace = torch.empty(max(lcvq_ptq_workspace_size(N, K), 1), dtype=torch.uint8,
                                device=dev)
    _check(workspace, "workspace", torch.uint8, dev)
    _ok(lib().lcvq_ptq_init(_p(H), _p(W0), N, K, float(damp), int(iters), _p(packed_out),
                            _p(sb_out), _p(obj_out), _p(U_out), _p(D_out), _p(workspace),
                            workspace.numel(), _stream(dev)), "lcvq_ptq_init")


def ptq_init(X, W0, damp=0.01, iters=4, want_ud=False):
    """Allocating helper: H = X^T X, then the initialisation. Returns a dict with H, the
    packed codes, s, b, the objective history (and U, D with want_ud)."""
    dev = X.device
    M, K = X.shape
    N = W0.shape[0]
    H = torch.empty((K, K), dtype=torch.float32, device=dev)
    lcvq_hessian(X, H)
    out = {"H": H,
           "packed": torch.empty((N, K // 4), dtype=torch.uint8, device=dev),
           "sb": torch.empty(2, dtype=torch.float32, device=dev),
           "obj": torch.empty(2 * iters, dtype=torch.float32, device=dev),
           "U": torch.empty((K, K), dtype=torch.float32, device=dev) if want_ud else None,
           "D": torch.empty(K, dtype=torch.float32, device=dev) if want_ud else None}
    lcvq_ptq_init(H, W0, damp, iters, out["packed"], out["sb"], out["obj"], out["U"], out["D"])
    return out


# ------------------------------------------------------------------ allocating helpers
def linear_fwd(X, Wp, A, B, d, want_what=False):
    """Allocates the outputs of lcvq_linear_fwd and returns them in a dict."""
    M, K = X.shape
    N = Wp.shape[0]
    dev = X.device
    out = {
        "Y": torch.empty((M, N), dtype=X.dtype, device=dev),
        "packed": torch.empty((N, K // 4), dtype=torch.uint8, device=dev),
        "mask": torch.empty((N, K // 8), dtype=torch.uint8, device=dev),
        "What": torch.empty((N, K), dtype=torch.float32, device=dev) if want_what else None,
    }
    lcvq_linear_fwd(X, Wp, A, B, d, out["Y"], out["packed"], out["mask"], out["What"])
    return out


def linear_bwd(dY, X, packed, mask, A, B, d, want_dx=True, dge_wp=None, dge_alpha=None):
    """Allocates the outputs of lcvq_linear_bwd (or, with dge_wp and dge_alpha, of
    lcvq_linear_bwd_dge) and returns them in a dict."""
    M, N = dY.shape
    K = X.shape[1]
    dev = dY.device
    out = {
        "dX": torch.empty((M, K), dtype=dY.dtype, device=dev) if want_dx else None,
        "dWp": torch.empty((N, K), dtype=torch.float32, device=dev),
        "dA": torch.empty((d, d), dtype=torch.float32, device=dev),
        "dB": torch.empty((d,), dtype=torch.float32, device=dev),
    }
    if dge_alpha is None:
        lcvq_linear_bwd(dY, X, packed, mask, A, B, d, out["dX"], out["dWp"], out["dA"],
                        out["dB"])
    else:
        lcvq_linear_bwd_dge(dY, X, packed, mask, dge_wp, dge_alpha, A, B, d, out["dX"],
                            out["dWp"], out["dA"], out["dB"])
    return out


def gemv2b(X, packed, A16, B16, d, shuffled=False):
    """Allocates Y; `shuffled` says that `packed` holds the decode layout."""
    M = X.shape[0]
    N = packed.shape[0]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    (lcvq_gemv2b_shuffled if shuffled else lcvq_gemv2b)(X, packed, A16, B16, d, Y)
    return Y


def gemv2b_shuffle(packed):
    """Allocates and returns the decode layout of canonical packed codes."""
    codes = torch.empty_like(packed)
    lcvq_gemv2b_shuffle(packed, codes)
    return codes

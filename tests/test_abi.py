"""The C ABI without a GPU: the library loads, exports every declared entry point, and
every argument error is reported before anything is launched."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcvq.h")


@pytest.fixture(scope="module")
def L():
    import bit_weight_only_lc_amd as P
    if not os.path.exists(P.LIB_PATH):
        from bit_weight_only_lc_amd import build
        build.build()
    return P.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lcvq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["lcvq_quantize", "lcvq_linear_fwd", "lcvq_linear_bwd", "lcvq_pack2b",
              "lcvq_gemv2b", "lcvq_unpack2b", "lcvq_status_string", "lcvq_linear_bwd_dge",
              "lcvq_linear_fwd_workspace_size", "lcvq_linear_bwd_workspace_size",
              "lcvq_gemv2b_workspace_size"]:
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(10):
        assert L.lcvq_status_string(s) != b"unknown status"
    assert L.lcvq_status_string(99) == b"unknown status"


# Fake but well-aligned "device" addresses: every check below fails before any launch.
P = 1 << 20          # 16-byte aligned
MIS = P + 4          # misaligned


def test_quantize_errors(L):
    assert L.lcvq_quantize(None, 4, 64, P, P, P, None) == 1           # NULL
    assert L.lcvq_quantize(P, 4, 60, P, P, P, None) == 2              # K % 16
    assert L.lcvq_quantize(P, 0, 64, P, P, P, None) == 2              # N < 1
    assert L.lcvq_quantize(MIS, 4, 64, P, P, P, None) == 5            # alignment
    assert L.lcvq_quantize(P, 4, 64, None, None, None, None) == 0     # nothing to do


def test_pack_errors(L):
    assert L.lcvq_pack2b(None, 4, 64, P, None) == 1
    assert L.lcvq_pack2b(P, 4, 8, P, None) == 2
    assert L.lcvq_unpack2b(P, 4, 64, MIS, None) == 5


def _fwd(L, **kw):
    a = dict(X=P, xdt=1, M=16, N=256, K=256, d=8, Wp=P, A=P, B=P, Y=P, packed=P, mask=P,
             What=None, ws=P, wsb=1 << 30, s=None)
    a.update(kw)
    return L.lcvq_linear_fwd(a["X"], a["xdt"], a["M"], a["N"], a["K"], a["d"], a["Wp"],
                             a["A"], a["B"], a["Y"], a["packed"], a["mask"], a["What"],
                             a["ws"], a["wsb"], a["s"])


def test_linear_fwd_errors(L):
    assert _fwd(L, X=None) == 1
    assert _fwd(L, packed=None) == 1
    assert _fwd(L, xdt=7) == 4
    assert _fwd(L, d=6) == 3
    assert _fwd(L, M=0) == 2
    assert _fwd(L, N=100) == 2
    assert _fwd(L, K=96) == 2
    assert _fwd(L, Y=MIS) == 5
    need = L.lcvq_linear_fwd_workspace_size(16, 256, 256, 8)
    assert need > 0
    assert _fwd(L, xdt=0, wsb=need - 1) == 6   # sized for float32
    assert _fwd(L, ws=None) == 6


def _bwd(L, **kw):
    a = dict(dY=P, X=P, dt=1, M=16, N=256, K=256, d=8, packed=P, mask=P, A=P, B=P, dX=P,
             dWp=P, dA=P, dB=P, ws=P, wsb=1 << 30, s=None)
    a.update(kw)
    return L.lcvq_linear_bwd(a["dY"], a["X"], a["dt"], a["M"], a["N"], a["K"], a["d"],
                             a["packed"], a["mask"], a["A"], a["B"], a["dX"], a["dWp"],
                             a["dA"], a["dB"], a["ws"], a["wsb"], a["s"])


def test_linear_bwd_errors(L):
    assert _bwd(L, dY=None) == 1
    assert _bwd(L, dA=None) == 1
    assert _bwd(L, dt=3) == 4
    assert _bwd(L, d=2) == 3
    assert _bwd(L, K=128 + 32) == 2
    assert _bwd(L, dWp=MIS) == 5
    need = L.lcvq_linear_bwd_workspace_size(16, 256, 256, 8)   # sized for float32
    assert need > 0
    assert _bwd(L, dt=0, wsb=need - 1) == 6
    assert _bwd(L, ws=None) == 6


def _bwd_dge(L, **kw):
    a = dict(dY=P, X=P, dt=1, M=16, N=256, K=256, d=8, packed=P, mask=P, Wp=P, alpha=4.0,
             A=P, B=P, dX=P, dWp=P, dA=P, dB=P, ws=P, wsb=1 << 30, s=None)
    a.update(kw)
    return L.lcvq_linear_bwd_dge(a["dY"], a["X"], a["dt"], a["M"], a["N"], a["K"], a["d"],
                                 a["packed"], a["mask"], a["Wp"], a["alpha"], a["A"], a["B"],
                                 a["dX"], a["dWp"], a["dA"], a["dB"], a["ws"], a["wsb"],
                                 a["s"])


def test_linear_bwd_dge_errors(L):
    assert _bwd_dge(L, Wp=None) == 1
    assert _bwd_dge(L, Wp=MIS) == 5
    assert _bwd_dge(L, alpha=0.0) == 8
    assert _bwd_dge(L, alpha=-1.0) == 8
    assert _bwd_dge(L, alpha=float("nan")) == 8
    assert _bwd_dge(L, alpha=1e4) == 8
    assert _bwd_dge(L, dY=None) == 1          # then the checks of lcvq_linear_bwd
    assert _bwd_dge(L, d=2) == 3
    assert _bwd_dge(L, ws=None) == 6


def test_gemv_errors(L):
    def g(**kw):
        a = dict(X=P, M=1, N=256, K=256, d=8, packed=P, A=P, B=P, Y=P, ws=P, wsb=1 << 30)
        a.update(kw)
        return L.lcvq_gemv2b(a["X"], a["M"], a["N"], a["K"], a["d"], a["packed"], a["A"],
                             a["B"], a["Y"], a["ws"], a["wsb"], None)
    assert g(X=None) == 1
    assert g(M=17) == 2
    assert g(M=0) == 2
    assert g(K=288) == 2                               # K % 64
    assert g(K=32) == 2
    assert g(K=0) == 2
    assert g(N=40) == 2
    assert g(d=5) == 3
    assert g(Y=MIS) == 5
    # a partial last block of 256 columns: sized as the whole block
    assert L.lcvq_gemv2b_workspace_size(1, 256, 320, 8) == \
        L.lcvq_gemv2b_workspace_size(1, 256, 512, 8) > L.lcvq_gemv2b_workspace_size(1, 256, 256, 8)
    assert L.lcvq_gemv2b_workspace_size(1, 256, 64, 8) == L.lcvq_gemv2b_workspace_size(1, 256, 256, 8)
    assert g(wsb=L.lcvq_gemv2b_workspace_size(1, 256, 256, 8) - 1) == 6
    need = L.lcvq_gemv2b_workspace_size(16, 4096, 14336, 8)
    assert need > L.lcvq_gemv2b_workspace_size(1, 4096, 4096, 8) > 0
    assert g(M=16, N=4096, K=14336, wsb=need - 1) == 6
    assert L.lcvq_gemv2b_workspace_size(1, 40, 256, 8) == 0


def test_gemv_shuffle_errors(L):
    def g(packed=P, N=256, K=256, codes=P):
        return L.lcvq_gemv2b_shuffle(packed, N, K, codes, None)
    assert g(packed=None) == 1
    assert g(codes=None) == 1
    assert g(N=40) == 2
    assert g(N=0) == 2
    assert g(K=320) == 2
    assert g(K=128) == 2
    assert g(codes=MIS) == 5

    def s(**kw):
        a = dict(X=P, M=1, N=256, K=256, d=8, codes=P, A=P, B=P, Y=P, ws=P, wsb=1 << 30)
        a.update(kw)
        return L.lcvq_gemv2b_shuffled(a["X"], a["M"], a["N"], a["K"], a["d"], a["codes"],
                                      a["A"], a["B"], a["Y"], a["ws"], a["wsb"], None)
    assert s(codes=None) == 1
    assert s(M=17) == 2
    assert s(K=320) == 2                               # the decode layout needs K % 256
    assert s(d=5) == 3
    assert s(codes=MIS) == 5


def test_gemv_batched_errors(L):
    import bit_weight_only_lc_amd as PK
    mats = (PK.GemvMatrix * 9)(*[PK.GemvMatrix(P, P, P, P, 256) for _ in range(9)])
    ws = L.lcvq_gemv2b_workspace_size(1, 256, 256, 8)

    def g(X=P, M=1, K=256, d=8, m=mats, count=3, wsp=P, wsb=ws):
        return L.lcvq_gemv2b_batched(X, M, K, d, m, count, wsp, wsb, None)
    assert g(X=None) == 1
    assert g(m=None) == 1
    assert g(count=0) == 2
    assert g(count=9) == 2
    assert g(M=17) == 2
    assert g(K=288) == 2
    assert g(d=5) == 3
    assert g(wsb=ws - 1) == 6
    mats[1].layout = 1                                # decode layout: K % 256
    assert g(K=320, wsb=1 << 30) == 2
    mats[1].layout = 0
    mats[1].N = 40
    assert g() == 2
    mats[1].N = 256
    mats[2].Y = MIS
    assert g() == 5
    mats[2].Y = P
    mats[1].layout = 2
    assert g() == 8                                   # LCVQ_ERR_VALUE
    mats[1].layout = 1
    mats[0].packed = None
    assert g() == 1


def test_workspace_sizes_grow_with_shape(L):
    a = L.lcvq_linear_fwd_workspace_size(64, 256, 256, 8)
    b = L.lcvq_linear_fwd_workspace_size(4096, 4096, 4096, 8)
    assert 0 < a < b
    assert L.lcvq_linear_fwd_workspace_size(0, 256, 256, 8) == 0
    assert L.lcvq_linear_bwd_workspace_size(64, 256, 256, 16) > \
        L.lcvq_linear_bwd_workspace_size(64, 256, 256, 4)


def test_profile_hook_ids(L):
    """The timing hook knows kernel ids 1..12; arming with NULL events disarms (no GPU call)."""
    for kid in (0, 13, -1):
        assert L.lcvq_profile_next(kid, None, None) == 2          # LCVQ_ERR_SHAPE
    for kid in range(1, 13):
        assert L.lcvq_profile_next(kid, None, None) == 0


def test_launch_limits_are_shape_errors(L):
    """Shapes whose kernel grids would exceed 2^32 - 1 work-items are rejected on the host
    (LCVQ_ERR_SHAPE, workspace size 0) instead of failing at launch; the largest
    accepted ones still report a workspace size. No GPU call is made."""
    max_m = (1 << 24) - (1 << 17)
    assert L.lcvq_linear_fwd_workspace_size(max_m, 256, 256, 8) > 0
    assert L.lcvq_linear_fwd_workspace_size(max_m + 1, 256, 256, 8) == 0
    assert L.lcvq_linear_bwd_workspace_size(max_m + 1, 256, 256, 8) == 0
    assert _fwd(L, M=max_m + 1) == 2
    assert _bwd(L, M=1 << 24) == 2
    assert L.lcvq_linear_fwd_workspace_size(64, 1 << 21, 256, 8) > 0
    assert L.lcvq_linear_fwd_workspace_size(64, (1 << 21) + 64, 256, 8) == 0
    assert _fwd(L, N=(1 << 21) + 64) == 2
    assert _bwd(L, K=(1 << 21) + 64) == 2
    # M x N product tiles beyond 2^23 - 8 with every dimension inside its own limit
    assert L.lcvq_linear_fwd_workspace_size(max_m, 1 << 20, 64, 8) == 0
    assert _fwd(L, M=max_m, N=1 << 20, K=64) == 2
    # decode: N <= 2^26, N * K <= 2^36, and the batch's rows summed <= 2^26
    assert L.lcvq_gemv2b_workspace_size(1, 1 << 26, 256, 8) > 0
    assert L.lcvq_gemv2b_workspace_size(1, (1 << 26) + 16, 256, 8) == 0
    assert L.lcvq_gemv2b_workspace_size(1, 1 << 20, 1 << 17, 8) == 0
    assert L.lcvq_gemv2b_shuffle(P, (1 << 26) + 16, 256, P, None) == 2
    import bit_weight_only_lc_amd as PK
    mats = (PK.GemvMatrix * 2)(*[PK.GemvMatrix(P, P, P, P, 1 << 25) for _ in range(2)])
    ws = L.lcvq_gemv2b_workspace_size(1, 256, 256, 8)
    mats[1].N = (1 << 25) + 16                      # 2^26 + 16 rows in all
    assert L.lcvq_gemv2b_batched(P, 1, 256, 8, mats, 2, P, ws, None) == 2


def test_gemv_noalloc_errors(L):
    """The no-allocation decode call: argument errors as lcvq_gemv2b's, and K beyond its
    fixed scratch is LCVQ_ERR_SCRATCH, all reported before any GPU call."""
    def g(**kw):
        a = dict(X=P, M=1, N=256, K=256, d=8, packed=P, A=P, B=P, Y=P)
        a.update(kw)
        return L.lcvq_gemv2b_noalloc(a["X"], a["M"], a["N"], a["K"], a["d"], a["packed"],
                                     a["A"], a["B"], a["Y"], None)
    assert g(X=None) == 1
    assert g(Y=None) == 1
    assert g(M=17) == 2
    assert g(N=40) == 2
    assert g(K=288) == 2
    assert g(d=5) == 3
    assert g(K=65536 + 256) == 9                     # LCVQ_ERR_SCRATCH
    assert g(K=65536 + 64) == 9
    assert g(K=1 << 20, N=16) == 9
    assert L.lcvq_status_string(9) != b"unknown status"


def test_ptq_errors(L):
    """lcvq_hessian and lcvq_ptq_init argument checks, all before any GPU call."""
    assert L.lcvq_hessian(None, 16, 64, P, None) == 1
    assert L.lcvq_hessian(P, 0, 64, P, None) == 2
    assert L.lcvq_hessian(P, 16, 96, P, None) == 2                 # K % 64
    assert L.lcvq_hessian(P, 16, 16384 + 64, P, None) == 2
    assert L.lcvq_hessian(P, 16, 64, MIS, None) == 5
    ws = L.lcvq_ptq_workspace_size(64, 256)
    assert ws > 0 and L.lcvq_ptq_workspace_size(40, 256) == 0
    assert L.lcvq_ptq_workspace_size(64, 16384 + 64) == 0

    def g(**kw):
        a = dict(H=P, W0=P, N=64, K=256, damp=0.01, iters=2, pk=P, sb=P, obj=None, U=None,
                 D=None, ws=P, wsb=ws)
        a.update(kw)
        return L.lcvq_ptq_init(a["H"], a["W0"], a["N"], a["K"], a["damp"], a["iters"], a["pk"],
                               a["sb"], a["obj"], a["U"], a["D"], a["ws"], a["wsb"], None)
    assert g(H=None) == 1
    assert g(sb=None) == 1
    assert g(N=40) == 2
    assert g(K=96) == 2
    assert g(damp=0.0) == 8
    assert g(damp=float("nan")) == 8
    assert g(damp=2.0) == 8
    assert g(iters=0) == 8
    assert g(iters=65) == 8
    assert g(U=MIS) == 5
    assert g(wsb=ws - 1) == 6
    assert g(ws=None) == 6


def test_mfma_probe_errors(L):
    assert L.lcvq_mfma_probe(4, None, None) == 1
    assert L.lcvq_mfma_probe(3, P, None) == 2                  # odd
    assert L.lcvq_mfma_probe(0, P, None) == 2
    assert L.lcvq_mfma_probe((1 << 24) + 2, P, None) == 2
    assert L.lcvq_mfma_probe(4, MIS, None) == 5


def test_read_probe_errors(L):
    assert L.lcvq_read_probe(None, 64, P, None) == 1
    assert L.lcvq_read_probe(P, 60, P, None) == 2
    assert L.lcvq_read_probe(P, 0, P, None) == 2
    assert L.lcvq_read_probe(MIS, 64, P, None) == 5

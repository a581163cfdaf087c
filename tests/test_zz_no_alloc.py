"""The no-allocation decode call against the workspace one, on the GPU, through the C ABI.

lcvq_gemv2b_noalloc runs lcvq_gemv2b's kernels with the library's fixed device scratch
in place of a caller workspace. Its output must be the workspace call's bytes (and within
the oracle's tolerance), on calls in a row that reuse the scratch -- the second with a
smaller input -- on both decode paths: the one-launch path for few tokens and the
prologue + product path, which keeps X' in the scratch.
"""

import ctypes

import numpy as np
import pytest
import torch

import synth_inputs as SI
from floatcheck import check
from oracle import coracle as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_lc_amd as P
    P.lib()
    return P


def _case(N, K, M, d, seed):
    wp = SI.make_wp(N, K, seed=seed, device="cuda")
    pk = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    import bit_weight_only_lc_amd as P
    P.lcvq_quantize(wp, None, pk, None)
    A, B = SI.make_ab(d, seed=seed + 1)
    X = SI.make_act(M, K, seed=seed + 2, device="cuda")
    return X, pk, A, B


def _noalloc(P, X, pk, A16, B16, d, Y):
    """Straight through the C ABI (ctypes), no Python-side allocation."""
    M, K = X.shape
    st = P.lib().lcvq_gemv2b_noalloc(ctypes.c_void_p(X.data_ptr()), M, pk.shape[0], K, d,
                                     ctypes.c_void_p(pk.data_ptr()),
                                     ctypes.c_void_p(A16.data_ptr()),
                                     ctypes.c_void_p(B16.data_ptr()),
                                     ctypes.c_void_p(Y.data_ptr()),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st


@pytest.mark.parametrize("d", [8, 4, 16])
@pytest.mark.parametrize("first,second", [
    ((4096, 14336, 16), (1024, 4096, 5)),     # prologue + product path, then a smaller one
    ((14336, 4096, 1), (272, 2048, 2)),       # one-launch path, then a smaller one
    ((4096, 65536, 16), (512, 8192, 3)),      # the largest K the scratch holds
    ((4096, 4160, 16), (1024, 4288, 1)),      # a partial last block of 256 columns
])
def test_noalloc_matches_workspace_call(P, d, first, second):
    outs = []
    for i, (N, K, M) in enumerate((first, second)):
        print(f"noalloc d={d} call {i}: N={N} K={K} M={M}", flush=True)
        X, pk, A, B = _case(N, K, M, d, seed=8800 + N + K + M + d)
        A16, B16 = A.half().cuda(), B.half().cuda()
        y_ws = P.gemv2b(X, pk, A16, B16, d)
        y_na = torch.empty_like(y_ws)
        _noalloc(P, X, pk, A16, B16, d, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), (i, N, K, M)
        ref = C.gemv2b(X.double().cpu().numpy(), pk.cpu().numpy(), A16.double().cpu().numpy(),
                       B16.double().cpu().numpy(), d)
        check(y_na.double().cpu().numpy(), ref, 1e-2, f"noalloc call {i}")
        outs.append(y_na)
    # the first call's output is untouched by the second one
    assert torch.isfinite(outs[0].float()).all()


def test_noalloc_rejects_beyond_scratch(P):
    X, pk, A, B = _case(16, 256, 1, 8, seed=1)
    A16, B16 = A.half().cuda(), B.half().cuda()
    Y = torch.empty((1, 16), dtype=torch.bfloat16, device="cuda")
    st = P.lib().lcvq_gemv2b_noalloc(ctypes.c_void_p(X.data_ptr()), 1, 16, 65536 + 256, 8,
                                     ctypes.c_void_p(pk.data_ptr()),
                                     ctypes.c_void_p(A16.data_ptr()),
                                     ctypes.c_void_p(B16.data_ptr()),
                                     ctypes.c_void_p(Y.data_ptr()), None)
    assert st == 9                                    # LCVQ_ERR_SCRATCH, nothing launched

"""GPU parity of the PTQ initialisation (lcvq_hessian, lcvq_ptq_init) through the C ABI.

Against the plain C++ oracle (oracle/coracle.py):
  * H = X^T X: every 32 x 32 block and element (floatcheck at 1e-5; the products of bf16
    values are exact, only float32 sums differ), and exactly symmetric;
  * the factorisation Hd = U D U^T of the GPU's own H (float32 against float64);
  * the integer step, decision by decision: the GPU's codes after one step from the
    start (s, b) are checked against the oracle's values t_k computed in float64 from the
    GPU's own earlier codes (teacher forcing); every code whose t is farther than 1e-3
    from a half-integer must be exactly clip(round(t), 0, 3) -- nearer ones may round
    either way in float32, since several results are then correct -- and at most 1% of
    the decisions may fall that near (about 0.2% do for evenly spread values);
  * the (s, b) step and the objective: the GPU's (s, b) are the oracle's least-squares
    solve for the GPU's codes, and every objective the GPU reports is the oracle's
    objective of the GPU's codes at the GPU's (s, b);
  * the alternation: the objective never increases, and its end is as good as the
    oracle's own run of the alternation (within 0.2%).
Inputs: calibration activations X ~ N(0, 1) in bf16 with a few input channels scaled by
6 (outlier channels), a weight W0 ~ 0.02 N(0, 1) in float32, damp 0.01.
"""

import numpy as np
import pytest
import torch

import synth_inputs as SI
from floatcheck import check, fmt
from oracle import coracle as C

pytestmark = pytest.mark.gpu

DAMP = 0.01
TIE = 1e-3


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_lc_amd as P
    P.lib()
    return P


def note(msg):
    print(msg, flush=True)


def calib(M, K, seed):
    X = SI.make_act(M, K, seed=seed, dtype="f32")
    X[:, : max(1, K // 256)] *= 6.0
    return X.to(torch.bfloat16).cuda()


def weight(N, K, seed):
    return (SI.make_act(N, K, seed=seed, dtype="f32") * 0.02).cuda()


def unpack(P, packed, K):
    z = torch.empty((packed.shape[0], K), dtype=torch.uint8, device=packed.device)
    P.lcvq_unpack2b(packed, z)
    return z.cpu().numpy()


@pytest.mark.parametrize("M,K", [(1000, 320), (77, 64), (4096, 1024)])
def test_hessian(P, M, K):
    note(f"hessian M={M} K={K}")
    X = calib(M, K, seed=M + K)
    H = torch.empty((K, K), dtype=torch.float32, device="cuda")
    P.lcvq_hessian(X, H)
    torch.cuda.synchronize()
    Hg = H.double().cpu().numpy()
    assert np.array_equal(Hg, Hg.T)
    note("  " + fmt(check(Hg, C.hessian(X.double().cpu().numpy()), 1e-5, "H")))


def test_hessian_full_size(P):
    """8192 calibration tokens, K = 4096: the float64 reference is X^T X through numpy."""
    M, K = 8192, 4096
    X = calib(M, K, seed=5)
    H = torch.empty((K, K), dtype=torch.float32, device="cuda")
    P.lcvq_hessian(X, H)
    torch.cuda.synchronize()
    Xh = X.double().cpu().numpy()
    Hg = H.double().cpu().numpy()
    assert np.array_equal(Hg, Hg.T)
    note("  " + fmt(check(Hg, Xh.T @ Xh, 1e-5, "H full")))


def one_step(P, N, K, M, seed):
    X = calib(M, K, seed)
    W0 = weight(N, K, seed + 1)
    out = P.ptq_init(X, W0, DAMP, 1, want_ud=True)
    torch.cuda.synchronize()
    Hg = out["H"].double().cpu().numpy()
    W0h = W0.double().cpu().numpy()
    return out, Hg, W0h


def check_step(P, out, Hg, W0h, label):
    N, K = W0h.shape
    Hd = C.damp(Hg, DAMP)
    U, D = C.udu(Hd)
    eU = check(out["U"].double().cpu().numpy(), U, 1e-3, f"{label} U")
    eD = check(out["D"].double().cpu().numpy(), D, 1e-3, f"{label} D")
    c = unpack(P, out["packed"], K)
    lo, hi = W0h.min(), W0h.max()
    s0, b0 = (hi - lo) / 3.0, lo
    t = C.ptq_targets(W0h, U, s0, b0, c)
    want = np.clip(np.rint(t), 0, 3)
    near = np.abs(t - np.floor(t) - 0.5) < TIE
    wrong = (want != c) & ~near
    note(f"{label}: U {fmt(eU)} D {fmt(eD)}; {int(near.sum())} of {t.size} decisions within "
         f"{TIE} of a tie, {int((want != c).sum())} differ")
    assert not wrong.any(), np.argwhere(wrong)[:10]
    assert near.mean() <= 1e-2
    sb = out["sb"].cpu().numpy()
    s1, b1, sing = C.ptq_solve_sb(W0h, c, Hd, s0, b0)
    assert not sing
    np.testing.assert_allclose(sb[:2], [s1, b1], rtol=1e-4)
    obj = out["obj"].double().cpu().numpy()
    np.testing.assert_allclose(obj[0], C.ptq_objective(W0h, c, Hd, s0, b0), rtol=1e-4)
    np.testing.assert_allclose(obj[1], C.ptq_objective(W0h, c, Hd, sb[0], sb[1]), rtol=1e-4)
    assert obj[1] <= obj[0]


@pytest.mark.parametrize("N,K,M", [(48, 192, 400), (256, 512, 1024), (64, 1088, 2048)])
def test_ptq_one_step(P, N, K, M):
    note(f"ptq one step N={N} K={K} M={M}")
    out, Hg, W0h = one_step(P, N, K, M, seed=N + K)
    check_step(P, out, Hg, W0h, f"N={N} K={K}")


def test_ptq_one_step_full_size(P):
    """The 4096 x 4096 weight with 8192 calibration tokens: every row's decisions."""
    note("ptq one step 4096 x 4096")
    out, Hg, W0h = one_step(P, 4096, 4096, 8192, seed=11)
    check_step(P, out, Hg, W0h, "4096x4096")


@pytest.mark.parametrize("N,K,M,iters", [(128, 256, 512, 6), (192, 640, 1024, 5)])
def test_ptq_alternation(P, N, K, M, iters):
    note(f"ptq alternation N={N} K={K} iters={iters}")
    X = calib(M, K, seed=N * 3 + K)
    W0 = weight(N, K, seed=N * 3 + K + 1)
    out = P.ptq_init(X, W0, DAMP, iters)
    torch.cuda.synchronize()
    obj = out["obj"].double().cpu().numpy()
    assert np.all(np.diff(obj) <= 1e-6 * obj[0]), obj
    Hg = out["H"].double().cpu().numpy()
    W0h = W0.double().cpu().numpy()
    Hd = C.damp(Hg, DAMP)
    c = unpack(P, out["packed"], K)
    sb = out["sb"].cpu().numpy()
    np.testing.assert_allclose(obj[-1], C.ptq_objective(W0h, c, Hd, sb[0], sb[1]), rtol=1e-4)
    s1, b1, _ = C.ptq_solve_sb(W0h, c, Hd, sb[0], sb[1])
    np.testing.assert_allclose(sb[:2], [s1, b1], rtol=1e-4)
    ref = C.ptq_init(W0h, Hg, DAMP, iters)
    note(f"  objective GPU {obj[-1]:.6e} oracle {ref['obj'][-1]:.6e}; codes equal "
         f"{np.mean(c == ref['codes']):.4f}")
    assert obj[-1] <= ref["obj"][-1] * 1.002


def test_ptq_is_deterministic(P):
    X = calib(512, 256, seed=3)
    W0 = weight(64, 256, seed=4)
    a = P.ptq_init(X, W0, DAMP, 3)
    b = P.ptq_init(X, W0, DAMP, 3)
    torch.cuda.synchronize()
    for k in ("H", "packed", "sb", "obj"):
        assert torch.equal(a[k], b[k]), k

"""GPU parity at the full sizes of the MLP and 8B-stack workloads, on sampled outputs.

Each layer runs through the C ABI at its real shape (8192 tokens). The CPU oracle then
checks, in float64:
  * every code, packed byte and mask byte of the matrix (bit-exact);
  * 64 seeded rows of Y and of dX (a row of either depends only on the same row of X
    and dY, so the oracle runs on those rows alone);
  * 64 seeded rows of dWp (a row depends only on the same column of dY);
  * dB in full through the closed form dB = sum over vectors of (r^T X), r = dY 1 (the
    identity the oracle is pinned to in test_fold_identities);
  * dA and dB in full for a second backward whose dY is zero outside the 64 sampled
    columns (the oracle's backward on those columns is then the whole answer).
Tolerances are those of the full-size tests: 1e-2 max relative Frobenius per tensor.
"""

import numpy as np
import pytest
import torch

import synth_inputs as SI
from oracle import lcvq_oracle as O

pytestmark = pytest.mark.gpu

TOL = 1e-2
NS = 64


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_lc_amd as P
    P.lib()
    return P


def rel(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / (den if den > 0 else 1.0))


def host(t):
    return t.detach().double().cpu().numpy() if t.is_floating_point() \
        else t.detach().cpu().numpy()


def note(msg):
    print(msg, flush=True)


def check_sampled(P, X, Wp, A, B, dY, d, label, seed):
    """X [M,K], Wp [N,K], A, B, dY [M,N] on the GPU. Returns the forward output Y."""
    M, K = X.shape
    N = Wp.shape[0]
    f = P.linear_fwd(X, Wp, A, B, d)
    b = P.linear_bwd(dY, X, f["packed"], f["mask"], A, B, d)
    g = np.random.default_rng(seed)
    rm = torch.from_numpy(np.sort(g.choice(M, NS, replace=False))).cuda()
    rn = torch.from_numpy(np.sort(g.choice(N, NS, replace=False))).cuda()
    dYs = torch.zeros_like(dY)
    dYs[:, rn] = dY[:, rn]
    bs = P.linear_bwd(dYs, X, f["packed"], f["mask"], A, B, d)
    torch.cuda.synchronize()

    wp = Wp.cpu().numpy()
    Ah, Bh = host(A), host(B)
    z, m = O.quantize(wp)
    assert np.array_equal(host(f["packed"]), O.pack2b(z)), label
    assert np.array_equal(host(f["mask"]), O.pack_mask(m)), label

    Xr, dYr = host(X[rm]), host(dY[rm])
    of = O.linear_fwd(Xr, wp, Ah, Bh, d)
    ob = O.linear_bwd(dYr, Xr, z, m, Ah, Bh, d)
    rnh = rn.cpu().numpy()
    Xh = host(X)
    oc = O.linear_bwd(host(dY[:, rn]), Xh, z[rnh], m[rnh], Ah, Bh, d)
    r = host(dY).sum(axis=1)
    dB_closed = (r @ Xh).reshape(K // d, d).sum(axis=0)
    errs = {
        "Y_rows": rel(host(f["Y"][rm]), of["Y"]),
        "dX_rows": rel(host(b["dX"][rm]), ob["dX"]),
        "dWp_rows": rel(host(b["dWp"][rn]), oc["dWp"]),
        "dB": rel(host(b["dB"]), dB_closed),
        "dA_cols": rel(host(bs["dA"]), oc["dA"]),
        "dB_cols": rel(host(bs["dB"]), oc["dB"]),
    }
    note(f"{label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL, (label, k, errs)
    return f["Y"]


def test_mlp_7b_chain(P):
    """Gate and up projections 11008 x 4096 and the down projection 4096 x 11008 at
    8192 tokens, d = 8; the down projection's input is SiLU(gate) * up rounded to bf16
    (elementwise glue outside the library)."""
    c = SI.CONFIGS["c2_mlp_7b"]
    M, d = c["M"], c["d"]
    (Ng, Kg), (Nu, Ku), (Nd, Kd) = c["mats"]
    dev = torch.device("cuda")
    X = SI.make_act(M, Kg, seed=2000, device=dev)
    outs = []
    for i, (N, K) in enumerate(c["mats"][:2]):
        Wp = SI.make_wp(N, K, seed=2001 + i, device=dev)
        A, B = (t.to(dev) for t in SI.make_ab(d, seed=2001 + i))
        dY = SI.make_act(M, N, seed=2101 + i, device=dev)
        note(f"c2 matrix {i}: {N}x{K}")
        outs.append(check_sampled(P, X, Wp, A, B, dY, d, f"c2[{i}] {N}x{K}", 2201 + i))
    h = (torch.nn.functional.silu(outs[0].float()) * outs[1].float()).to(torch.bfloat16)
    Wp = SI.make_wp(Nd, Kd, seed=2003, device=dev)
    A, B = (t.to(dev) for t in SI.make_ab(d, seed=2003))
    dY = SI.make_act(M, Nd, seed=2103, device=dev)
    note(f"c2 matrix 2: {Nd}x{Kd}")
    check_sampled(P, h.contiguous(), Wp, A, B, dY, d, f"c2[2] {Nd}x{Kd}", 2203)


C4_SHAPES = sorted(set(SI.CONFIGS["c4_stack_8b_layer"]["mats"]))


@pytest.mark.parametrize("d", SI.CONFIGS["c4_stack_8b_layer"]["ds"])
@pytest.mark.parametrize("N,K", C4_SHAPES)
def test_stack_8b_shapes(P, N, K, d):
    """Each distinct matrix shape of the 8B-shaped layer at 8192 tokens, for each d."""
    M = SI.CONFIGS["c4_stack_8b_layer"]["M"]
    dev = torch.device("cuda")
    seed = 4000 + N + K + d
    note(f"c4 {N}x{K} d={d}")
    X = SI.make_act(M, K, seed=seed + 1, device=dev)
    dY = SI.make_act(M, N, seed=seed + 2, device=dev)
    Wp = SI.make_wp(N, K, seed=seed, device=dev)
    A, B = (t.to(dev) for t in SI.make_ab(d, seed=seed))
    check_sampled(P, X, Wp, A, B, dY, d, f"c4 {N}x{K} d={d}", seed + 3)

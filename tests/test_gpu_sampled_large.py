"""GPU parity at the full sizes of the MLP and 8B-stack workloads.

Each layer runs through the C ABI at its real shape (8192 tokens).

Sampled (every matrix of the MLP chain and every distinct 8B-layer shape at d = 4, 8,
16), against the plain C++ oracle of record:
  * every code, packed byte and mask byte of the matrix (bit-exact);
  * rows of Y and of dX drawn one from every band of 256 rows plus random ones (a row of
    either depends only on the same row of X and dY, so the oracle runs on those rows);
  * rows of dWp drawn the same way over the weight rows (a row depends only on the same
    column of dY);
  * dB in full through the closed form dB = sum over vectors of (r^T X), r = dY 1 (the
    identity the oracle is pinned to in test_fold_identities);
  * dA and dB in full for a second backward whose dY is zero outside the sampled columns
    (the oracle's backward on those weight rows is then the whole answer).

In full (one matrix of every distinct shape of the two workloads, the 8B shapes at each
d): every output element against the numpy oracle, the second opinion pinned by the same
pins and equal to the C++ oracle to float64 rounding (test_oracle_cross.py); it takes
its matmuls from the BLAS library, which makes a whole 8192-token layer affordable.

Every float comparison is floatcheck.check at 1e-2: tensor, every 32 x 32 block, and
element-wise.
"""

import numpy as np
import pytest
import torch

import synth_inputs as SI
from floatcheck import check, fmt, stratified
from oracle import coracle as C
from oracle import lcvq_oracle as O

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_lc_amd as P
    P.lib()
    return P


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
    rm = stratified(M, seed)
    rn = stratified(N, seed + 1)
    rmd, rnd = torch.from_numpy(rm).cuda(), torch.from_numpy(rn).cuda()
    dYs = torch.zeros_like(dY)
    dYs[:, rnd] = dY[:, rnd]
    bs = P.linear_bwd(dYs, X, f["packed"], f["mask"], A, B, d)
    torch.cuda.synchronize()

    wp = Wp.cpu().numpy()
    Ah, Bh = host(A), host(B)
    z, m = C.quantize(wp)
    assert np.array_equal(host(f["packed"]), C.pack2b(z)), label
    assert np.array_equal(host(f["mask"]), C.pack_mask(m)), label

    Xh, dYh = host(X), host(dY)
    of = C.linear_fwd(Xh, wp, Ah, Bh, d, rows=rm)
    ob = C.linear_bwd(dYh, Xh, z, m, Ah, Bh, d, dx_rows=rm, dw_rows=rn)
    r = dYh.sum(axis=1)
    dB_closed = (r @ Xh).reshape(K // d, d).sum(axis=0)
    errs = {
        "Y_rows": check(host(f["Y"][rmd]), of["Y"], TOL, f"{label} Y rows"),
        "dX_rows": check(host(b["dX"][rmd]), ob["dX"], TOL, f"{label} dX rows"),
        "dWp_rows": check(host(b["dWp"][rnd]), ob["dWp"], TOL, f"{label} dWp rows"),
        "dB": check(host(b["dB"]), dB_closed, TOL, f"{label} dB"),
        "dA_cols": check(host(bs["dA"]), ob["dA"], TOL, f"{label} dA cols"),
        "dB_cols": check(host(bs["dB"]), ob["dB"], TOL, f"{label} dB cols"),
    }
    note(f"{label} ({len(rm)} + {len(rn)} rows): " +
         " ".join(f"{k}={fmt(v)}" for k, v in errs.items()))
    return f["Y"]


def test_mlp_7b_chain(P):
    """Gate and up projections 11008 x 4096 and the down projection 4096 x 11008 at
    8192 tokens, d = 8; the down projection's input is SiLU(gate) * up rounded to bf16
    (elementwise glue outside the library)."""
    c = SI.CONFIGS["c2_mlp_7b"]
    M, d = c["M"], c["d"]
    (Nd, Kd) = c["mats"][2]
    dev = torch.device("cuda")
    X = SI.make_act(M, c["mats"][0][1], seed=2000, device=dev)
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
C2_SHAPES = sorted(set(SI.CONFIGS["c2_mlp_7b"]["mats"]))


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


FULL_CASES = ([("c4", N, K, d) for (N, K) in C4_SHAPES
               for d in SI.CONFIGS["c4_stack_8b_layer"]["ds"]] +
              [("c2", N, K, 8) for (N, K) in C2_SHAPES])


@pytest.mark.parametrize("cfg,N,K,d", FULL_CASES)
def test_full_layer_per_shape(P, cfg, N, K, d):
    """One matrix of every distinct shape, every output element: Y, dX, dWp, dA, dB (and
    the codes), at 8192 tokens; the mask is exercised with Wp ~ U[-2, 5)."""
    M = 8192
    dev = torch.device("cuda")
    seed = 9000 + N + K + d
    note(f"full {cfg} {N}x{K} d={d}: GPU")
    X = SI.make_act(M, K, seed=seed + 1, device=dev)
    dY = SI.make_act(M, N, seed=seed + 2, device=dev)
    Wp = SI.make_wp(N, K, seed=seed, device=dev, lo=-2.0, hi=5.0)
    A, B = (t.to(dev) for t in SI.make_ab(d, seed=seed))
    f = P.linear_fwd(X, Wp, A, B, d)
    b = P.linear_bwd(dY, X, f["packed"], f["mask"], A, B, d)
    torch.cuda.synchronize()
    g = {"Y": host(f["Y"]), "dX": host(b["dX"]), "dWp": host(b["dWp"]), "dA": host(b["dA"]),
         "dB": host(b["dB"])}
    pk, mk = host(f["packed"]), host(f["mask"])
    del f, b
    Xh, dYh, wp = host(X), host(dY), Wp.cpu().numpy()
    del X, dY, Wp
    torch.cuda.empty_cache()
    note(f"full {cfg} {N}x{K} d={d}: oracle")
    Ah, Bh = host(A), host(B)
    of = O.linear_fwd(Xh, wp, Ah, Bh, d)
    assert np.array_equal(pk, of["packed"]) and np.array_equal(mk, of["maskbits"])
    errs = {"Y": check(g.pop("Y"), of["Y"], TOL, "Y")}
    z, m = of["z"], of["m"]
    del of
    ob = O.linear_bwd(dYh, Xh, z, m, Ah, Bh, d)
    for k in ("dX", "dWp", "dA", "dB"):
        errs[k] = check(g.pop(k), ob.pop(k), TOL, k)
    note(f"full {cfg} {N}x{K} d={d}: " + " ".join(f"{k}={fmt(v)}" for k, v in errs.items()))

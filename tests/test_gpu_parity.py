"""GPU parity: the HIP path through the C ABI against the CPU oracle.

The oracle of record is the plain C++ one (oracle/coracle.py). Codes, packed bytes and
mask bytes must match bit for bit. Floating-point outputs must pass floatcheck.check
with tol 1e-5 (float32 decoded weights) or 1e-2 (bf16-input, float32-accumulate
products and gradients): the relative Frobenius error of the whole tensor, of every
32 x 32 block, and an element-wise bound, all within tol.
"""

import numpy as np
import pytest
import torch

import synth_inputs as SI
from floatcheck import check, fmt
from oracle import coracle as O

pytestmark = pytest.mark.gpu

TOL_W = 1e-5
TOL = 1e-2


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_lc_amd as P
    P.lib()
    return P


def rel(gpu, ref):
    """Relative Frobenius distance (used between two GPU results only)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / (den if den > 0 else 1.0))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() \
        else t.detach().cpu().numpy()


def note(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ quantizer / packing
SPECIAL = [-0.6, -0.5, -0.4, 0.0, 0.49, 0.5, 0.50000006, 1.5, 2.5, 2.5000002, 3.49, 3.5,
           3.51, 4.0, -1.0, 1e30, -1e30, float("nan"), float("inf"), float("-inf")]


@pytest.mark.parametrize("N,K", [(64, 256), (3, 48), (1, 16), (129, 1024)])
def test_quantize_bitexact(P, N, K):
    note(f"quantize N={N} K={K}")
    wp = SI.make_wp(N, K, seed=N * 7 + K, lo=-2.0, hi=5.0)
    flat = wp.view(-1)
    sp = torch.tensor(SPECIAL, dtype=torch.float32)
    flat[: min(len(SPECIAL), flat.numel())] = sp[: min(len(SPECIAL), flat.numel())]
    d_wp = wp.cuda()
    z = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    pk = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    mk = torch.empty((N, K // 8), dtype=torch.uint8, device="cuda")
    P.lcvq_quantize(d_wp, z, pk, mk)
    torch.cuda.synchronize()
    zr, mr = O.quantize(wp.numpy())
    assert np.array_equal(host(z), zr)
    assert np.array_equal(host(pk), O.pack2b(zr))
    assert np.array_equal(host(mk), O.pack_mask(mr))


def test_pack_unpack(P):
    note("pack/unpack")
    g = torch.Generator().manual_seed(9)
    z = torch.randint(0, 4, (37, 512), generator=g, dtype=torch.uint8)
    dz = z.cuda()
    pk = torch.empty((37, 128), dtype=torch.uint8, device="cuda")
    P.lcvq_pack2b(dz, pk)
    back = torch.empty_like(dz)
    P.lcvq_unpack2b(pk, back)
    torch.cuda.synchronize()
    assert np.array_equal(host(pk), O.pack2b(z.numpy()))
    assert np.array_equal(host(back), z.numpy())
    allb = torch.arange(256, dtype=torch.uint8).view(1, 256).repeat(2, 1)
    out = torch.empty((2, 1024), dtype=torch.uint8, device="cuda")
    P.lcvq_unpack2b(allb.cuda(), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), O.unpack2b(allb.numpy(), 1024))
    # group counts (N K / 16) that leave 1..3 groups past the last whole set of four, with
    # bits above the code set in the inputs (ignored)
    for (n, k) in ((3, 16), (5, 48), (1, 16), (7, 80), (4097, 4096)):
        zb = torch.randint(0, 256, (n, k), generator=g, dtype=torch.uint8)
        pk2 = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
        P.lcvq_pack2b(zb.cuda(), pk2)
        back2 = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        P.lcvq_unpack2b(pk2, back2)
        torch.cuda.synchronize()
        assert np.array_equal(host(pk2), O.pack2b(zb.numpy() & 3)), (n, k)
        assert np.array_equal(host(back2), zb.numpy() & 3), (n, k)


# ------------------------------------------------------------------ linear layer
def run_layer(P, inp, d, want_what=True):
    X, Wp, A, B, dY = (inp[k].cuda() for k in ("X", "Wp", "A", "B", "dY"))
    f = P.linear_fwd(X, Wp, A, B, d, want_what=want_what)
    b = P.linear_bwd(dY, X, f["packed"], f["mask"], A, B, d)
    torch.cuda.synchronize()
    return f, b


def check_layer(P, inp, d, label):
    f, b = run_layer(P, inp, d)
    X = host(inp["X"])
    dY = host(inp["dY"])
    wp = inp["Wp"].numpy()
    A = inp["A"].double().numpy()
    B = inp["B"].double().numpy()
    of = O.linear_fwd(X, wp, A, B, d)
    ob = O.linear_bwd(dY, X, of["z"], of["m"], A, B, d)
    assert np.array_equal(host(f["packed"]), of["packed"]), label
    assert np.array_equal(host(f["mask"]), of["maskbits"]), label
    errs = {"What": check(host(f["What"]), of["What"], TOL_W, f"{label} What")}
    for k, g, r in (("Y", f["Y"], of["Y"]), ("dX", b["dX"], ob["dX"]),
                    ("dWp", b["dWp"], ob["dWp"]), ("dA", b["dA"], ob["dA"]),
                    ("dB", b["dB"], ob["dB"])):
        errs[k] = check(host(g), r, TOL, f"{label} {k}")
    note(f"{label}: " + " ".join(f"{k}={fmt(v)}" for k, v in errs.items()))
    return errs


def test_config0_single_layer(P):
    """256 x 256 layer, 16 float32 tokens, d = 8, seed 0."""
    c = SI.CONFIGS["c0_single_256"]
    (N, K), M, d = c["mats"][0], c["M"], c["d"]
    inp = SI.make_layer(N, K, M, d, seed=0, x_dtype="f32")
    check_layer(P, inp, d, "c0")


@pytest.mark.parametrize("d", [4, 8, 16])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(16, 256, 256), (1, 64, 64), (300, 320, 192),
                                   (513, 576, 320)])
def test_layer_shapes(P, d, xdt, M, N, K):
    """Several tiles, ragged tails in every dimension, and the clamp mask exercised."""
    inp = SI.make_layer(N, K, M, d, seed=M + N + K + d, x_dtype=xdt, lo=-2.0, hi=5.0)
    check_layer(P, inp, d, f"M={M} N={N} K={K} d={d} {xdt}")


@pytest.mark.parametrize("d,xdt", [(8, "bf16"), (16, "f32")])
def test_backward_without_dx(P, d, xdt):
    """Without dX the dA/dB partials are reduced by a launch of their own instead of by the
    dX product's tiles: dWp is the same bytes, dA and dB the same sums in another order."""
    M, N, K = 513, 576, 320
    inp = SI.make_layer(N, K, M, d, seed=8100 + d, x_dtype=xdt, lo=-2.0, hi=5.0)
    dev = {k: v.cuda() for k, v in inp.items()}
    f = P.linear_fwd(dev["X"], dev["Wp"], dev["A"], dev["B"], d)
    with_dx = P.linear_bwd(dev["dY"], dev["X"], f["packed"], f["mask"], dev["A"], dev["B"], d)
    no_dx = P.linear_bwd(dev["dY"], dev["X"], f["packed"], f["mask"], dev["A"], dev["B"], d,
                         want_dx=False)
    torch.cuda.synchronize()
    assert no_dx["dX"] is None
    assert torch.equal(no_dx["dWp"], with_dx["dWp"])
    for k in ("dA", "dB"):
        assert rel(host(no_dx[k]), host(with_dx[k])) <= 1e-5, k
    wp = inp["Wp"].numpy()
    A, B = inp["A"].double().numpy(), inp["B"].double().numpy()
    z, m = O.quantize(wp)
    ob = O.linear_bwd(host(inp["dY"]), host(inp["X"]), z, m, A, B, d)
    for k in ("dWp", "dA", "dB"):
        check(host(no_dx[k]), ob[k], TOL, k)


def test_degenerate_A(P):
    """A = 0, negative and singular A are valid decodes (decoupleQ section 3.2 allows a
    zero or negative scale)."""
    M, N, K, d = 64, 128, 128, 8
    for name, A in [("zero", torch.zeros(d, d)), ("neg", -0.03 * torch.eye(d)),
                    ("rank1", torch.outer(torch.arange(d, dtype=torch.float32),
                                          torch.ones(d)) * 0.01)]:
        inp = SI.make_layer(N, K, M, d, seed=5, lo=-2.0, hi=5.0)
        inp["A"] = A.contiguous()
        check_layer(P, inp, d, f"A={name}")


def test_backward_is_deterministic(P):
    M, N, K, d = 512, 512, 512, 8
    inp = SI.make_layer(N, K, M, d, seed=77)
    X, Wp, A, B, dY = (inp[k].cuda() for k in ("X", "Wp", "A", "B", "dY"))
    f = P.linear_fwd(X, Wp, A, B, d)
    r1 = P.linear_bwd(dY, X, f["packed"], f["mask"], A, B, d)
    r2 = P.linear_bwd(dY, X, f["packed"], f["mask"], A, B, d)
    f2 = P.linear_fwd(X, Wp, A, B, d)
    torch.cuda.synchronize()
    for k in ("dX", "dWp", "dA", "dB"):
        assert torch.equal(r1[k], r2[k]), k
    assert torch.equal(f["Y"], f2["Y"])


def test_config1_full(P):
    """4096 x 4096 weight, 4096 bf16 tokens, d = 8: every output against the full oracle."""
    c = SI.CONFIGS["c1_square_4096"]
    (N, K), M, d = c["mats"][0], c["M"], c["d"]
    note("c1: generating")
    inp = {k: v.cpu() for k, v in SI.make_layer(N, K, M, d, seed=1000, device="cuda").items()}
    check_layer(P, inp, d, "c1")


# ------------------------------------------------------------------ decode product
@pytest.mark.parametrize("N,K", [(256, 256), (4096, 4096), (14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", [1, 2, 4, 16, 3])
def test_gemv(P, N, K, M):
    d = 8
    note(f"gemv N={N} K={K} M={M}")
    wp = SI.make_wp(N, K, seed=3000 + N + K, device="cuda")
    A, B = SI.make_ab(d, seed=3000 + M)
    X = SI.make_act(M, K, seed=3100 + M, device="cuda")
    pk = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    P.lcvq_quantize(wp, None, pk, None)
    A16, B16 = A.half().cuda(), B.half().cuda()
    Y = P.gemv2b(X, pk, A16, B16, d)
    torch.cuda.synchronize()
    ref = O.gemv2b(host(X), host(pk), A.half().double().numpy(), B.half().double().numpy(), d)
    note(f"  {fmt(check(host(Y), ref, TOL, 'gemv'))}")


@pytest.mark.parametrize("N,K,M,d", [(4096, 4096, 5, 8), (4096, 4096, 8, 8), (4096, 4096, 12, 8),
                                     (4096, 4096, 12, 4), (1024, 4096, 11, 16), (272, 4096, 9, 8),
                                     (4096, 16384, 4, 8), (256, 16384, 3, 16), (2048, 16384, 4, 4),
                                     (4352, 4096, 12, 8), (256, 8192, 12, 8), (4096, 4096, 13, 8),
                                     (4096, 4096, 7, 16), (8192, 4096, 9, 8), (6144, 4096, 5, 8),
                                     (4096, 2048, 16, 8), (4096, 4096, 16, 4), (8192, 4096, 7, 16),
                                     (8208, 4096, 8, 8), (4096, 4096, 15, 8)])
def test_gemv_more_tokens(P, N, K, M, d):
    """Token counts and K at the edges of the one-launch path's range (five to sixteen
    tokens with K up to 16 blocks of 256, three or four tokens with K up to 64 blocks, one
    row group per workgroup up to 4096 rows and two up to 8192, within the bound on the
    activation work), and just past them (more than 8192 rows, K of 32 blocks at 12
    tokens, work past the bound), which take the prologue + product path."""
    note(f"gemv more tokens N={N} K={K} M={M} d={d}")
    wp = SI.make_wp(N, K, seed=3400 + N + K, device="cuda")
    A, B = SI.make_ab(d, seed=3400 + d + M)
    X = SI.make_act(M, K, seed=3500 + M, device="cuda")
    pk = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    P.lcvq_quantize(wp, None, pk, None)
    A16, B16 = A.half().cuda(), B.half().cuda()
    Y = P.gemv2b(X, pk, A16, B16, d)
    Ys = P.gemv2b(X, P.gemv2b_shuffle(pk), A16, B16, d, shuffled=True)
    torch.cuda.synchronize()
    assert torch.equal(Y, Ys)
    ref = O.gemv2b(host(X), host(pk), A.half().double().numpy(), B.half().double().numpy(), d)
    note(f"  {fmt(check(host(Y), ref, TOL, 'gemv more tokens'))}")


@pytest.mark.parametrize("N,K,M,d", [(256, 64, 1, 8), (512, 192, 12, 8), (4096, 4160, 1, 8),
                                     (4096, 4160, 4, 8), (4096, 4160, 16, 8), (14336, 4288, 2, 8),
                                     (1024, 14400, 3, 16), (272, 16320, 1, 4),
                                     (4096, 16448, 1, 8), (2048, 320, 7, 16)])
def test_gemv_partial_block(P, N, K, M, d):
    """K a multiple of 64 but not of 256: the last 256-column block is partial, on the
    one-launch path and on the prologue + product path (K < 256 included)."""
    note(f"gemv partial block N={N} K={K} M={M} d={d}")
    wp = SI.make_wp(N, K, seed=3600 + N + K, device="cuda")
    A, B = SI.make_ab(d, seed=3600 + d + M)
    X = SI.make_act(M, K, seed=3700 + M, device="cuda")
    pk = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    P.lcvq_quantize(wp, None, pk, None)
    ws = torch.empty(P.lcvq_gemv2b_workspace_size(M, N, K, d), dtype=torch.uint8,
                     device="cuda")
    ys = []
    for _ in range(2):                       # repeated calls through one workspace
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        P.lcvq_gemv2b(X, pk, A.half().cuda(), B.half().cuda(), d, Y, ws)
        ys.append(Y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    ref = O.gemv2b(host(X), host(pk), A.half().double().numpy(), B.half().double().numpy(), d)
    note(f"  {fmt(check(host(ys[0]), ref, TOL, 'gemv partial block'))}")


@pytest.mark.parametrize("d", [4, 16])
@pytest.mark.parametrize("N,K", [(4096, 4096), (2048, 14336)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
def test_gemv_d(P, N, K, M, d):
    """The decode product at the other vector lengths, on both the one-launch path (few
    tokens, K within its range) and the prologue + product path."""
    note(f"gemv d={d} N={N} K={K} M={M}")
    wp = SI.make_wp(N, K, seed=3200 + N + K, device="cuda")
    A, B = SI.make_ab(d, seed=3200 + d + M)
    X = SI.make_act(M, K, seed=3300 + M, device="cuda")
    pk = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    P.lcvq_quantize(wp, None, pk, None)
    Y = P.gemv2b(X, pk, A.half().cuda(), B.half().cuda(), d)
    torch.cuda.synchronize()
    ref = O.gemv2b(host(X), host(pk), A.half().double().numpy(), B.half().double().numpy(), d)
    note(f"  {fmt(check(host(Y), ref, TOL, 'gemv d'))}")


@pytest.mark.parametrize("N,K,M", [(4096, 14336, 16), (14336, 4096, 1), (272, 8192, 5),
                                   (256, 16640, 2)])
def test_gemv_repeat_shared_workspace(P, N, K, M):
    """Calls that reuse one workspace give identical bytes, and the partial sums of long
    rows add up to the oracle's product."""
    d = 8
    note(f"gemv repeat N={N} K={K} M={M}")
    wp = SI.make_wp(N, K, seed=5000 + N + K, device="cuda")
    A, B = SI.make_ab(d, seed=5000 + M)
    X = SI.make_act(M, K, seed=5100 + M, device="cuda")
    pk = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    P.lcvq_quantize(wp, None, pk, None)
    A16, B16 = A.half().cuda(), B.half().cuda()
    ws = torch.empty(P.lcvq_gemv2b_workspace_size(M, N, K, d), dtype=torch.uint8, device="cuda")
    ys = []
    for _ in range(3):
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        P.lcvq_gemv2b(X, pk, A16, B16, d, Y, ws)
        ys.append(Y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
    ref = O.gemv2b(host(X), host(pk), A.half().double().numpy(), B.half().double().numpy(), d)
    note(f"  {fmt(check(host(ys[0]), ref, TOL, 'gemv repeat'))}")


def test_graph_replay_matches_eager(P):
    """The forward and backward captured in one HIP graph give the eager step's bytes on
    every replay, with other GPU work and synchronizations between the replays."""
    M, N, K, d = 300, 320, 192, 8
    inp = SI.make_layer(N, K, M, d, seed=91, lo=-2.0, hi=5.0)
    X, Wp, A, B, dY = (inp[k].cuda() for k in ("X", "Wp", "A", "B", "dY"))
    out = {"Y": torch.empty((M, N), dtype=X.dtype, device="cuda"),
           "packed": torch.empty((N, K // 4), dtype=torch.uint8, device="cuda"),
           "mask": torch.empty((N, K // 8), dtype=torch.uint8, device="cuda"),
           "dX": torch.empty((M, K), dtype=X.dtype, device="cuda"),
           "dWp": torch.empty((N, K), dtype=torch.float32, device="cuda"),
           "dA": torch.empty((d, d), dtype=torch.float32, device="cuda"),
           "dB": torch.empty((d,), dtype=torch.float32, device="cuda")}
    wsf = torch.empty(P.lcvq_linear_fwd_workspace_size(M, N, K, d), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(P.lcvq_linear_bwd_workspace_size(M, N, K, d), dtype=torch.uint8,
                      device="cuda")

    def step():
        P.lcvq_linear_fwd(X, Wp, A, B, d, out["Y"], out["packed"], out["mask"], None, wsf)
        P.lcvq_linear_bwd(dY, X, out["packed"], out["mask"], A, B, d, out["dX"], out["dWp"],
                          out["dA"], out["dB"], wsb)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], ref[k]), (i, k)
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)


def test_decode_graph_replay_matches_eager(P):
    """The decode calls (one-launch path, prologue + product path, decode layout and the
    batched call) captured in one HIP graph give the eager calls' bytes on every replay,
    with other GPU work and synchronizations between the replays."""
    d, K = 8, 4096
    note("decode graph replay")
    g = torch.Generator(device="cuda").manual_seed(7700)
    pks = [torch.randint(0, 256, (n, K // 4), generator=g, dtype=torch.uint8, device="cuda")
           for n in (1024, 4096)]
    A, B = SI.make_ab(d, seed=7701)
    A16, B16 = A.half().cuda(), B.half().cuda()
    x1 = SI.make_act(1, K, seed=7702, device="cuda")
    x16 = SI.make_act(16, K, seed=7703, device="cuda")
    codes = P.gemv2b_shuffle(pks[1])
    ys = {"fused": torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda"),
          "two": torch.empty((16, 4096), dtype=torch.bfloat16, device="cuda"),
          "layout": torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda"),
          "b0": torch.empty((16, 1024), dtype=torch.bfloat16, device="cuda"),
          "b1": torch.empty((16, 4096), dtype=torch.bfloat16, device="cuda")}
    ws = torch.empty(P.lcvq_gemv2b_workspace_size(16, 4096, K, d), dtype=torch.uint8,
                     device="cuda")

    def calls():
        P.lcvq_gemv2b(x1, pks[1], A16, B16, d, ys["fused"], ws)
        P.lcvq_gemv2b(x16, pks[1], A16, B16, d, ys["two"], ws)
        P.lcvq_gemv2b_shuffled(x1, codes, A16, B16, d, ys["layout"], ws)
        P.lcvq_gemv2b_batched(x16, [(pks[0], A16, B16, ys["b0"], 0),
                                    (codes, A16, B16, ys["b1"], 1)], d, ws)

    calls()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ys.items()}
    assert torch.equal(ref["fused"], ref["layout"])
    assert torch.equal(ref["two"], ref["b1"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        calls()
    for i in range(4):
        for v in ys.values():
            v.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for k in ys:
            assert torch.equal(ys[k], ref[k]), (i, k)
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
    check(host(ref["two"]), O.gemv2b(host(x16), host(pks[1]), A.half().double().numpy(),
                                     B.half().double().numpy(), d), TOL, "decode graph")


@pytest.mark.parametrize("d,xdt,alpha", [(8, "bf16", 6.0), (4, "f32", 2.0), (16, "bf16", 20.0)])
@pytest.mark.parametrize("M,N,K", [(300, 320, 192), (513, 576, 320)])
def test_dge_backward(P, M, N, K, d, xdt, alpha):
    """The DGE backward: dWp within tolerance of the oracle's DGE backward (including
    proxies that are NaN, infinite or clamped); dX, dA and dB identical to the
    straight-through backward's bytes."""
    note(f"dge M={M} N={N} K={K} d={d} {xdt} alpha={alpha}")
    inp = SI.make_layer(N, K, M, d, seed=M + N + K + 17, x_dtype=xdt, lo=-2.0, hi=5.0)
    flat = inp["Wp"].view(-1)
    flat[: len(SPECIAL)] = torch.tensor(SPECIAL, dtype=torch.float32)
    X, Wp, A, B, dY = (inp[k].cuda() for k in ("X", "Wp", "A", "B", "dY"))
    f = P.linear_fwd(X, Wp, A, B, d)
    b = P.linear_bwd(dY, X, f["packed"], f["mask"], A, B, d, dge_wp=Wp, dge_alpha=alpha)
    b0 = P.linear_bwd(dY, X, f["packed"], f["mask"], A, B, d)
    torch.cuda.synchronize()
    for k in ("dX", "dA", "dB"):
        assert torch.equal(b[k], b0[k]), k
    assert torch.isfinite(b["dWp"]).all()
    wp = inp["Wp"].numpy()
    Xh, dYh = host(inp["X"]), host(inp["dY"])
    Ah, Bh = inp["A"].double().numpy(), inp["B"].double().numpy()
    z, m = O.quantize(wp)
    ob = O.linear_bwd(dYh, Xh, z, m, Ah, Bh, d, wp=wp, dge_alpha=alpha)
    note(f"  dWp {fmt(check(host(b['dWp']), ob['dWp'], TOL, 'dge dWp'))}")


@pytest.mark.parametrize("N,K", [(16, 256), (4096, 4096), (272, 14336)])
def test_gemv_shuffle_layout(P, N, K):
    """The decode layout holds the canonical bytes in the order its definition gives:
    tile (n/16, kb), then 16-byte pieces q = 0..3 of the 64-byte block row, then rows."""
    g = torch.Generator(device="cuda").manual_seed(7000 + N + K)
    pk = torch.randint(0, 256, (N, K // 4), generator=g, dtype=torch.uint8, device="cuda")
    codes = P.gemv2b_shuffle(pk)
    torch.cuda.synchronize()
    a = host(pk).reshape(N // 16, 16, K // 256, 4, 16)      # (r, j, kb, q, byte)
    want = a.transpose(0, 2, 3, 1, 4).reshape(-1)           # (r, kb, q, j, byte)
    assert np.array_equal(host(codes).reshape(-1), want)


@pytest.mark.parametrize("N,K", [(4096, 4096), (14336, 4096), (4096, 14336), (272, 8192)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
def test_gemv_shuffled_matches(P, N, K, M):
    """The product on the decode layout gives the canonical product's bytes, on both the
    one-launch and the prologue + product paths."""
    d = 8
    g = torch.Generator(device="cuda").manual_seed(7100 + N + K)
    pk = torch.randint(0, 256, (N, K // 4), generator=g, dtype=torch.uint8, device="cuda")
    A, B = SI.make_ab(d, seed=7200 + M)
    A16, B16 = A.half().cuda(), B.half().cuda()
    X = SI.make_act(M, K, seed=7300 + M, device="cuda")
    y0 = P.gemv2b(X, pk, A16, B16, d)
    y1 = P.gemv2b(X, P.gemv2b_shuffle(pk), A16, B16, d, shuffled=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("shapes,K", [([4096, 1024, 1024], 4096), ([14336, 14336], 4096),
                                      ([8192, 272], 256), ([4096], 14336), ([1024, 1024], 4096),
                                      ([4096, 1024, 1024], 4160)])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 8])
def test_gemv_batched(P, shapes, K, M):
    """Several matrices sharing X in one call: every output equals the single-matrix
    call's bytes and the oracle's product."""
    d = 8
    note(f"gemv batched N={shapes} K={K} M={M}")
    X = SI.make_act(M, K, seed=6100 + M, device="cuda")
    mats, singles, refs = [], [], []
    for i, n in enumerate(shapes):
        g = torch.Generator(device="cuda").manual_seed(6200 + i)
        pk = torch.randint(0, 256, (n, K // 4), generator=g, dtype=torch.uint8, device="cuda")
        A, B = SI.make_ab(d, seed=6300 + i)
        A16, B16 = A.half().cuda(), B.half().cuda()
        Y = torch.empty((M, n), dtype=torch.bfloat16, device="cuda")
        mats.append((pk, A16, B16, Y))
        singles.append(P.gemv2b(X, pk, A16, B16, d))
        refs.append((pk, A.half().double().numpy(), B.half().double().numpy()))
    P.lcvq_gemv2b_batched(X, mats, d)
    # the same call with every other matrix in the decode layout (whole 256-column blocks)
    mixed = [(P.gemv2b_shuffle(pk), a16, b16, torch.empty_like(y), 1) if i % 2 else
             (pk, a16, b16, torch.empty_like(y), 0)
             for i, (pk, a16, b16, y) in enumerate(mats)] if K % 256 == 0 else None
    if mixed is not None:
        P.lcvq_gemv2b_batched(X, mixed, d)
    torch.cuda.synchronize()
    for i, ((pk, _, _, Y), ys, (pkr, Ah, Bh)) in enumerate(zip(mats, singles, refs)):
        assert torch.equal(Y, ys)
        if mixed is not None:
            assert torch.equal(mixed[i][3], ys)
        check(host(Y), O.gemv2b(host(X), host(pkr), Ah, Bh, d), TOL, "gemv batched")


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 1 << 20, 14 << 20])
def test_read_probe_reads_every_word(P, nbytes):
    """The measurement helper streams every 16-byte word once: the XOR of its per-block
    words equals the XOR of the buffer's 32-bit words (at most 1024 blocks here)."""
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    buf = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    P.lcvq_read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_mfma_probe_runs_and_is_deterministic(P):
    """The MFMA ceiling probe (a measurement helper) writes one finite word per workgroup,
    the same on every call."""
    s1 = torch.zeros(1024, dtype=torch.int32, device="cuda")
    s2 = torch.zeros(1024, dtype=torch.int32, device="cuda")
    P.lcvq_mfma_probe(64, s1)
    P.lcvq_mfma_probe(64, s2)
    torch.cuda.synchronize()
    v = s1[:256].cpu().view(torch.float32)
    assert torch.isfinite(v).all() and (v != 0).all()
    assert torch.equal(s1, s2)


# Shapes whose forward and dW products have few tiles (at most 128 of 256 x 256): their
# contraction is split over up to four workgroups per tile, whose partial tiles a second
# launch adds in split order before the epilogue; except that a forward whose 128 x 256
# tiles occupy more than half of the CUs runs those, without a split.
SPLIT_SHAPES = [(1100, 320, 2112, 8, "bf16"),     # forward 4 ways, dW 2 ways, ragged M, K
                (2500, 192, 1216, 16, "f32"),     # forward 2 ways, dW 4 ways, float32
                (1031, 64, 4096, 4, "bf16"),      # one tile column, forward 4 ways
                (4000, 1280, 1024, 8, "bf16"),    # forward 160 tiles of 128 x 256, dW 4 ways
                (8100, 960, 1088, 16, "f32")]     # forward 256 tiles of 128 x 256, ragged M, N, K


@pytest.mark.parametrize("M,N,K,d,xdt", SPLIT_SHAPES)
def test_split_contraction_shapes(P, M, N, K, d, xdt):
    inp = SI.make_layer(N, K, M, d, seed=M + 3 * N + K, x_dtype=xdt, lo=-2.0, hi=5.0)
    check_layer(P, inp, d, f"split M={M} N={N} K={K} d={d} {xdt}")


# Tail split (dW, and the forward's 256 x 256 tiles): 288 and 272 tiles (one full round of
# the 256 CUs plus 32 or 16 tiles): the full round runs unsplit, the leftover tiles split
# their contraction in two, and a second launch adds the halves before the epilogue.
TAIL_SHAPES = [(1000, 4608, 4096, 8, "bf16"),     # 288 dW tiles, ragged M
               (1100, 4096, 4160, 16, "f32"),     # 272 dW tiles, ragged M and K, float32
               (4352, 4096, 1024, 8, "bf16"),     # 272 forward tiles
               (4400, 4096, 1088, 4, "f32")]      # 288 forward tiles, ragged M and K


@pytest.mark.parametrize("M,N,K,d,xdt", TAIL_SHAPES)
def test_dw_tail_split_shapes(P, M, N, K, d, xdt):
    inp = SI.make_layer(N, K, M, d, seed=M + 5 * N + K, x_dtype=xdt, lo=-2.0, hi=5.0)
    check_layer(P, inp, d, f"tail split M={M} N={N} K={K} d={d} {xdt}")


def test_dw_tail_split_dge_no_dx_determinism(P):
    """The tail split under the DGE estimator and without dX (the dA/dB partial rows then
    reduced by their own launch): repeated calls give identical bytes, and match the
    oracle."""
    M, N, K, d = 1000, 4608, 4096, 8
    inp = SI.make_layer(N, K, M, d, seed=4343, lo=-2.0, hi=5.0)
    X, Wp, A, B, dY = (inp[k].cuda() for k in ("X", "Wp", "A", "B", "dY"))
    f1 = P.linear_fwd(X, Wp, A, B, d)
    g1 = P.linear_bwd(dY, X, f1["packed"], f1["mask"], A, B, d, want_dx=False, dge_wp=Wp,
                      dge_alpha=5.0)
    g2 = P.linear_bwd(dY, X, f1["packed"], f1["mask"], A, B, d, want_dx=False, dge_wp=Wp,
                      dge_alpha=5.0)
    torch.cuda.synchronize()
    for k in ("dWp", "dA", "dB"):
        assert torch.equal(g1[k], g2[k]), k
    wp = inp["Wp"].numpy()
    z, m = O.quantize(wp)
    ob = O.linear_bwd(host(inp["dY"]), host(inp["X"]), z, m, inp["A"].double().numpy(),
                      inp["B"].double().numpy(), d, wp=wp, dge_alpha=5.0)
    note(f"tail split dge: dWp {fmt(check(host(g1['dWp']), ob['dWp'], TOL, 'tail dge dWp'))}")
    note(f"  dA {fmt(check(host(g1['dA']), ob['dA'], TOL, 'tail dge dA'))}")
    note(f"  dB {fmt(check(host(g1['dB']), ob['dB'], TOL, 'tail dge dB'))}")


def test_split_contraction_dge_and_determinism(P):
    M, N, K, d = 1100, 320, 2112, 8
    inp = SI.make_layer(N, K, M, d, seed=4242, lo=-2.0, hi=5.0)
    X, Wp, A, B, dY = (inp[k].cuda() for k in ("X", "Wp", "A", "B", "dY"))
    f1 = P.linear_fwd(X, Wp, A, B, d)
    f2 = P.linear_fwd(X, Wp, A, B, d)
    g1 = P.linear_bwd(dY, X, f1["packed"], f1["mask"], A, B, d, dge_wp=Wp, dge_alpha=5.0)
    g2 = P.linear_bwd(dY, X, f1["packed"], f1["mask"], A, B, d, dge_wp=Wp, dge_alpha=5.0)
    torch.cuda.synchronize()
    assert torch.equal(f1["Y"], f2["Y"])
    for k in ("dX", "dWp", "dA", "dB"):
        assert torch.equal(g1[k], g2[k]), k
    wp = inp["Wp"].numpy()
    z, m = O.quantize(wp)
    ob = O.linear_bwd(host(inp["dY"]), host(inp["X"]), z, m, inp["A"].double().numpy(),
                      inp["B"].double().numpy(), d, wp=wp, dge_alpha=5.0)
    note(f"split dge: dWp {fmt(check(host(g1['dWp']), ob['dWp'], TOL, 'split dge dWp'))}")

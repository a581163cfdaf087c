"""Seeded synthetic inputs for the LC-VQ hot path.

This module holds only random-number recipes and workload shapes; it contains none of
the method's arithmetic, so both the CPU oracle side and the GPU side of every test can
draw the same inputs from it.

Recipe (one LC-VQ linear layer with weight [N, K], d-vectors along K, M tokens):
  Wp = lo + (hi - lo) * U[0, 1)         float32, default [lo, hi) = [-0.5, 3.5)
  A  = 0.02 * I + 0.002 * N(0, 1) off the diagonal        float32 [d, d]
  B  = 0.01 * N(0, 1)                                      float32 [d]
  X  = N(0, 1) -> activation dtype (bfloat16, or float32)  [M, K]
  dY = N(0, 1) -> activation dtype                          [M, N]
The second argument of N(mean, sigma) is the standard deviation.
"""

import torch

# Workloads: Llama-7B/8B-shaped linear layers standing in for the LLaMA-3 / Qwen-3
# layers the method is evaluated on (no weights or data are used or needed).
CONFIGS = {
    "c0_single_256": dict(mats=[(256, 256)], M=16, d=8, x_dtype="f32"),
    "c1_square_4096": dict(mats=[(4096, 4096)], M=4096, d=8, x_dtype="bf16"),
    "c2_mlp_7b": dict(mats=[(11008, 4096), (11008, 4096), (4096, 11008)], M=8192, d=8,
                      x_dtype="bf16"),
    "c3_decode": dict(mats=[(4096, 4096), (14336, 4096), (4096, 14336)], Ms=(1, 4, 16),
                      d=8, x_dtype="bf16"),
    "c4_stack_8b_layer": dict(mats=[(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
                                    (14336, 4096), (14336, 4096), (4096, 14336)],
                              layers=32, M=8192, ds=(4, 8, 16), x_dtype="bf16"),
}

_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_wp(N, K, seed, device="cpu", lo=-0.5, hi=3.5):
    g = generator(seed, device)
    u = torch.rand((N, K), generator=g, device=device, dtype=torch.float32)
    return u.mul_(hi - lo).add_(lo)


def make_ab(d, seed, device="cpu"):
    g = generator(seed + 7919, device)
    off = torch.randn((d, d), generator=g, device=device, dtype=torch.float32) * 0.002
    A = off * (1 - torch.eye(d, device=device)) + 0.02 * torch.eye(d, device=device)
    B = torch.randn((d,), generator=g, device=device, dtype=torch.float32) * 0.01
    return A.contiguous(), B.contiguous()


def make_act(rows, cols, seed, dtype="bf16", device="cpu"):
    g = generator(seed, device)
    x = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    return x.to(_DT[dtype]).contiguous()


def make_layer(N, K, M, d, seed, x_dtype="bf16", device="cpu", lo=-0.5, hi=3.5):
    """All inputs of one forward+backward of one layer, from one seed."""
    return {
        "Wp": make_wp(N, K, seed, device, lo, hi),
        "A": make_ab(d, seed, device)[0],
        "B": make_ab(d, seed, device)[1],
        "X": make_act(M, K, seed + 104729, x_dtype, device),
        "dY": make_act(M, N, seed + 224737, x_dtype, device),
    }

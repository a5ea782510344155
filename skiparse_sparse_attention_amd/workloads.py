"""Seeded synthetic workloads: the configurations and the input generator.

Holds no arithmetic of the method -- only shapes and random numbers -- so both
the HIP path and the oracle can be fed from it.

Shapes follow the pages' latent and patch formulas: a 4x8x8 (or 8x8x8)
video VAE followed by a (1, 2, 2) patchify turns F frames at H x W pixels
into a (1 + (F-1)/4) x H/16 x W/16 token grid (Wan 2.1 report, section
4.2.1; Open-Sora Plan docs, High-Compression WFVAE).  The long joint-attention
shape stands for the ~45k-token joint attention the vidax page reports for
CogVideoX1.5.  Values are i.i.d. Gaussian; no dataset is involved.
"""

from __future__ import annotations

from dataclasses import dataclass

SINGLE = 0
GROUP = 1


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    sparse_k: int
    mode: int
    dtype: str = "bf16"       # "bf16" or "fp32"
    scale: float = 1.0        # inputs are scale * N(0, 1)

    @property
    def N(self):
        return self.T * self.H * self.W

    @property
    def L(self):
        return self.N // self.sparse_k

    @property
    def grid(self):
        return (self.T, self.H, self.W)

    def with_mode(self, mode, sparse_k=None):
        return Workload(self.name, self.B, self.T, self.H, self.W, self.heads, self.head_dim,
                        self.sparse_k if sparse_k is None else sparse_k, mode, self.dtype, self.scale)


# Tiny: 4x8x8 grid, 2 heads of 64, k=2 Single Skip, fp32 inputs.
TINY = Workload("tiny_4x8x8_h2_d64_k2_single_fp32", 1, 4, 8, 8, 2, 64, 2, SINGLE, "fp32")
# 93 frames at 352x640, 4x8x8 VAE, patch 1x2x2 -> 24x22x40 (N=21120); k=4.
OSP_SINGLE = Workload("osp_24x22x40_h24_d128_k4_single", 1, 24, 22, 40, 24, 128, 4, SINGLE)
OSP_GROUP = Workload("osp_24x22x40_h24_d128_k4_group", 1, 24, 22, 40, 24, 128, 4, GROUP)
# 121 frames at 576x1024, 8x8x8 VAE, patch 1x2x2 -> 16x36x64 (N=36864); inputs 0.5*N(0,1).
HC_GROUP = Workload("hc_16x36x64_h24_d128_k4_group", 1, 16, 36, 64, 24, 128, 4, GROUP, scale=0.5)
# Dense k=1 baseline: 81 frames at 832x480, 4x8x8 VAE, patch 1x2x2 -> 21x30x52 (N=32760), 40 heads.
WAN_DENSE = Workload("wan480_21x30x52_h40_d128_k1_dense", 1, 21, 30, 52, 40, 128, 1, SINGLE)
# Long joint attention ~45k tokens: 20x48x48 (N=46080), B=2, k=8.
LONG_GROUP = Workload("long_20x48x48_b2_h24_d128_k8_group", 2, 20, 48, 48, 24, 128, 8, GROUP)
LONG_SINGLE = Workload("long_20x48x48_b2_h24_d128_k8_single", 2, 20, 48, 48, 24, 128, 8, SINGLE)

ALL = [TINY, OSP_SINGLE, OSP_GROUP, HC_GROUP, WAN_DENSE, LONG_GROUP, LONG_SINGLE]


def make_inputs(w: Workload, seed: int = 0, device="cpu"):
    """q, k, v of shape (B, N, heads, head_dim).

    torch CPU generator seeded with ``seed``; randn for q, k, v in that order
    in float32; multiplied by ``w.scale`` (a power of two, so exact); cast to
    bfloat16 (round to nearest even) unless the workload is fp32; then moved
    to ``device``.
    """
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (w.B, w.N, w.heads, w.head_dim)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.scale != 1.0:
            x.mul_(w.scale)
        if w.dtype == "bf16":
            x = x.to(torch.bfloat16)
        out.append(x.to(device))
    return tuple(out)


def make_output_grad(w: Workload, seed: int = 1, device="cpu"):
    """A synthetic gradient of the loss with respect to the attention output, shape
    (B, N, heads, head_dim): torch CPU generator seeded with ``seed``, randn in float32,
    cast like the inputs (bfloat16 unless the workload is fp32), moved to ``device``."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((w.B, w.N, w.heads, w.head_dim), generator=g, dtype=torch.float32)
    if w.dtype == "bf16":
        x = x.to(torch.bfloat16)
    return x.to(device)

"""Workload shapes: model widths and the sample lists of each packed batch.

A sample is (h, w, frames, txt_len) in latent-grid units: one latent token
covers a 16 x 16 pixel patch, so a 64 x 64 grid is a 1024 x 1024 image.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Dims:
    hidden: int
    heads: int
    head_dim: int
    mlp: int
    c_lat: int
    d_txt: int
    t_dim: int = 256
    rope_theta: float = 10000.0
    eps: float = 1e-6
    rope_dims: tuple = None          # (frame, row, col) band widths; None: (d/4, 3d/8, 3d/8)

    @property
    def bands(self):
        d = self.head_dim
        return tuple(self.rope_dims) if self.rope_dims is not None else (d // 4, 3 * d // 8, 3 * d // 8)


@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    dtype: str                        # "f32" or "bf16"
    samples: tuple                    # ((h, w, frames, txt_len), ...)
    img_budget: int
    depth: int = 1
    steps: int = 0                    # sampler steps (0: training forward + loss)
    guidance: float = 0.0
    note: str = ""
    schedule: tuple = field(default=(1.0, 0.75, 0.5, 0.25, 0.0))


TINY = Dims(hidden=256, heads=4, head_dim=64, mlp=1024, c_lat=64, d_txt=256)
B4 = Dims(hidden=3072, heads=24, head_dim=128, mlp=12288, c_lat=128, d_txt=3072)

WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", TINY, "f32", ((16, 16, 1, 32), (8, 8, 1, 32)), img_budget=320,
        note="1 block, hidden 256, 4x64 heads, grids 16x16 + 8x8, 32 text tokens each"),
    "pack256_bf16": Workload(
        "pack256_bf16", B4, "bf16", tuple((16, 16, 1, 128) for _ in range(16)), img_budget=4096,
        note="256^2 stage: 16 x (16x16 grid + 128 text tokens), 1 block + RF loss"),
    "native1024_bf16": Workload(
        "native1024_bf16", B4, "bf16",
        ((64, 64, 1, 256), (48, 84, 1, 256), (84, 48, 1, 256), (32, 128, 1, 256)),
        img_budget=16384,
        note="1024^2 native-resolution stage: grids 64x64, 48x84, 84x48, 32x128 + 256 text each"),
    "sampler1024_cfg_bf16": Workload(
        "sampler1024_cfg_bf16", B4, "bf16", ((64, 64, 1, 256), (64, 64, 1, 256)), img_budget=8192,
        depth=28, steps=4, guidance=4.0,
        note="4-step Euler, packed CFG (cond + uncond, 64x64 grid + 256 text each), 28 blocks"),
    "edit_sampler1024_cfg_bf16": Workload(
        "edit_sampler1024_cfg_bf16", B4, "bf16", ((64, 64, 2, 256), (64, 64, 2, 256)), img_budget=16384,
        depth=28, steps=4, guidance=4.0,
        note="4-step Euler edit, packed CFG (cond + uncond, each 64x64 noised target + 64x64 clean source "
             "+ 256 text), 28 blocks"),
    # the pages' per-GPU training workload: one ~50,000-token native-resolution
    # pack (1024^2-class grids of four aspect ratios and one 768^2 grid, 256
    # text tokens each), forward and backward through 28 blocks
    "train50k_bf16": Workload(
        "train50k_bf16", B4, "bf16",
        tuple((h, w, 1, 256) for h, w in [(64, 64), (48, 84), (84, 48), (32, 128)] * 2
              + [(64, 64), (48, 84), (84, 48), (48, 48)]),
        img_budget=50000, depth=28,
        note="training step: 12 samples (grids 64x64, 48x84, 84x48, 32x128 x3, 48x48) + 256 text each = 50,048 "
             "tokens, 28 blocks forward + backward, every weight gradient"),
    "edit2048_bf16": Workload(
        "edit2048_bf16", B4, "bf16", ((128, 128, 2, 512),), img_budget=32768,
        note="2048^2 edit: target + source 128x128 grids (3D RoPE frames 0/1) + 512 text"),
}


def block_flops(dims, samples):
    """Algorithmic FLOPs of one block: 24 H^2 N (linears) + 4 H sum L_b^2 (attention)."""
    H = dims.hidden
    n = sum(f * h * w + t for h, w, f, t in samples)
    att = sum((f * h * w + t) ** 2 for h, w, f, t in samples)
    lin = 2 * n * (3 * H * H + H * H + 2 * H * dims.mlp)
    return lin + 4 * H * att, lin, 4 * H * att

"""Seeded synthetic inputs shared by the tests, the benchmark and the checks.

This module holds no arithmetic of the method: it only draws random numbers
(NumPy PCG64, one stream per (workload, tensor, index) key) and rounds them to
bfloat16 when the workload computes in bfloat16, so the HIP path and the
oracle consume identical values.  Distributions: weights N(0, 0.02) (or
N(0, 1/sqrt(fan_in)) for the "stress" recipe, which makes every residual
branch O(1)); latents, noise and text features N(0, 1); QK-norm gains 1;
timesteps U(0, 1) per sample.
"""

import zlib

import numpy as np


def _key(*parts):
    return [zlib.crc32(str(p).encode()) for p in parts]


def rng(*parts):
    """Independent generator for one (workload, tensor, index) key, seed 0."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0] + _key(*parts))))


def round_bf16(a):
    """Round a float32 array to the nearest bfloat16 (ties to even), as float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def normal(shape, std, dtype, *key):
    a = rng(*key).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return round_bf16(a) if dtype == "bf16" else a


def uniform(shape, dtype, *key):
    a = rng(*key).random(size=shape, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def _std(recipe, fan_in):
    return 0.02 if recipe == "default" else 1.0 / np.sqrt(fan_in)


def stream_weights(dims, dtype, wl, blk, stream, recipe="default"):
    H, M = dims.hidden, dims.mlp
    k = (wl, recipe, "block", blk, stream)
    return {
        "w_mod": normal((6 * H, H), _std(recipe, H), dtype, *k, "w_mod"),
        "w_qkv": normal((3 * H, H), _std(recipe, H), dtype, *k, "w_qkv"),
        "g_q": np.ones(dims.head_dim, np.float32),
        "g_k": np.ones(dims.head_dim, np.float32),
        "w_o": normal((H, H), _std(recipe, H), dtype, *k, "w_o"),
        "w_up": normal((M, H), _std(recipe, H), dtype, *k, "w_up"),
        "w_down": normal((H, M), _std(recipe, M), dtype, *k, "w_down"),
    }


def block_weights(dims, dtype, wl, blk=0, recipe="default"):
    return {s: stream_weights(dims, dtype, wl, blk, s, recipe) for s in ("img", "txt")}


def wrapper_weights(dims, dtype, wl, recipe="default"):
    H = dims.hidden
    k = (wl, recipe, "wrap")
    return {
        "w_t1": normal((H, dims.t_dim), _std(recipe, dims.t_dim), dtype, *k, "w_t1"),
        "w_t2": normal((H, H), _std(recipe, H), dtype, *k, "w_t2"),
        "w_in": normal((H, dims.c_lat), _std(recipe, dims.c_lat), dtype, *k, "w_in"),
        "w_txt": normal((H, dims.d_txt), _std(recipe, dims.d_txt), dtype, *k, "w_txt"),
        "w_fmod": normal((2 * H, H), _std(recipe, H), dtype, *k, "w_fmod"),
        "w_out": normal((dims.c_lat, H), _std(recipe, H), dtype, *k, "w_out"),
    }


def latents(n_img, c, dtype, wl, name="z"):
    return normal((n_img, c), 1.0, dtype, wl, "latent", name)


def text(n_txt, d, dtype, wl, name="tau"):
    return normal((n_txt, d), 1.0, dtype, wl, "text", name)


def timesteps(B, wl):
    """t_b ~ U(0, 1) per sample, float32 (the RF wrapper takes t in fp32)."""
    return rng(wl, "t").random(size=B, dtype=np.float32)


def residual(n, H, dtype, wl, name):
    """A residual-stream activation N(0, 1), for driving one block in isolation."""
    return normal((n, H), 1.0, dtype, wl, "residual", name)

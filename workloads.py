"""Seeded synthetic inputs for 3D-RoPE full / Skiparse attention.

This module is shared by the test suite, the benchmark and the oracle's
checks.  It holds no arithmetic of the method itself: it only lists the
workload shapes (raw clip sizes, compression factors, heads, head_dim, RoPE
split) and draws seeded Gaussian tensors, rounded to bfloat16.  Turning a clip
size into a latent grid, rotating, regrouping and attending are done separately
by the oracle and by the HIP library.

Workloads (clip sizes from the pages; latent-grid arithmetic is done elsewhere):

* ``tiny``   -- a 5x8x8 latent grid (the grid is given directly), 2 heads, D=64.
* ``osp480`` -- Open-Sora Plan's 93-frame 480p clip (640 wide), 4x8x8 VAE,
  1x2x2 patchify, 24 heads, D=96, inputs scaled by 1/sqrt(96) before rounding.
* ``cogvideox`` -- CogVideoX's 49-frame 480x720 clip, 4x8x8 VAE, 2x2 patchify,
  226 text tokens in front, 48 heads, D=64.
* ``osp480_skiparse`` -- ``osp480``'s tensors with Skiparse k=4 (single and
  group).
* ``osp720`` -- 93-frame 720x1280 clip, 24 heads, D=96, full and k=4; checked
  on 256 seeded query rows.
* ``osp15`` -- Open-Sora Plan v1.5's 121-frame 576x1024 clip through its
  8x8x8 VAE and 1x2x2 patchify, full and k=4; the pages give no head shape
  for that model, so 24 heads of D=128 (split 32/48/48) are taken, which
  also exercises the third head size.  Checked on 256 seeded query rows.
* ``SUV_SCHEDULE`` -- a U-shaped per-layer sparsity schedule (the SUV sparse
  DiT on the OSP blog page, v1.5.0 entry, names U-shaped sparsity but gives
  no schedule): full attention in the outer layers, k rising to 8 toward the
  middle and back, single and group skip alternating at each k.
* ``COGVIDEOX_PACK`` -- a Multi-Resolution Frame Pack (CogVideoX section 3.1):
  clips of 49, 25 and 1 frames at 480x720 and one of 33 frames at 256x384
  (Table 8's smallest resolution), each with its 226 text tokens, in one
  sequence at CogVideoX's 48 heads of D=64.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    # raw clip (frames, height, width) and compression; ``grid`` set instead
    # when the workload is specified directly as a latent grid
    clip: tuple | None
    c_t: int
    c_s: int
    p_t: int
    p_s: int
    grid: tuple | None
    n_text: int
    batch: int
    heads: int
    head_dim: int
    rope_split: tuple
    theta: float
    input_scale: float | None
    seed: int
    modes: tuple
    sparse_k: int
    sample_rows: int | None = None


WORKLOADS = {
    "tiny": Workload("tiny", None, 4, 8, 1, 2, (5, 8, 8), 0, 1, 2, 64,
                     (16, 24, 24), 1e4, None, 0,
                     ("full", "skiparse_single", "skiparse_group"), 4),
    "osp480": Workload("osp480", (93, 480, 640), 4, 8, 1, 2, None, 0, 1, 24, 96,
                       (32, 32, 32), 1e4, 1.0 / math.sqrt(96.0), 1,
                       ("full",), 1),
    "cogvideox": Workload("cogvideox", (49, 480, 720), 4, 8, 1, 2, None, 226, 1,
                          48, 64, (16, 24, 24), 1e4, None, 2, ("full",), 1),
    "osp480_skiparse": Workload("osp480_skiparse", (93, 480, 640), 4, 8, 1, 2,
                                None, 0, 1, 24, 96, (32, 32, 32), 1e4,
                                1.0 / math.sqrt(96.0), 1,
                                ("skiparse_single", "skiparse_group"), 4),
    "osp720": Workload("osp720", (93, 720, 1280), 4, 8, 1, 2, None, 0, 1, 24, 96,
                       (32, 32, 32), 1e4, None, 4,
                       ("full", "skiparse_single", "skiparse_group"), 4,
                       sample_rows=256),
    "osp15": Workload("osp15", (121, 576, 1024), 8, 8, 1, 2, None, 0, 1, 24, 128,
                      (32, 48, 48), 1e4, None, 5,
                      ("full", "skiparse_single", "skiparse_group"), 4,
                      sample_rows=256),
}


def gaussian_bf16(seed, tensor_id: int, shape, scale: float | None = None,
                  mult: float | None = None) -> torch.Tensor:
    """Draw N(0,1) fp32 with ``default_rng([seed, tensor_id])``, optionally
    multiply by ``scale`` and ``mult`` in fp32, round to bfloat16 (RNE).

    ``seed`` may be an int or a tuple of ints (extra entries select variants).
    Returns a CPU bfloat16 tensor.
    """
    key = list(seed) if isinstance(seed, (tuple, list)) else [int(seed)]
    rng = np.random.default_rng(key + [int(tensor_id)])
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    if scale is not None:
        x *= np.float32(scale)
    if mult is not None:
        x *= np.float32(mult)
    return torch.from_numpy(x).to(torch.bfloat16)


def make_qkv(seed, shape, scale: float | None = None, q_mult: float | None = None):
    """Q, K, V as bf16 CPU tensors of ``shape`` = [B, N, H, D] (tensor ids 0/1/2)."""
    q = gaussian_bf16(seed, 0, shape, scale, q_mult)
    k = gaussian_bf16(seed, 1, shape, scale)
    v = gaussian_bf16(seed, 2, shape, scale)
    return q, k, v


def make_dout(seed, shape, scale: float | None = None):
    """Output gradient dO for the backward, bf16 CPU tensor (tensor id 3)."""
    return gaussian_bf16(seed, 3, shape, scale)


def sample_rows(seed: int, n_tokens: int, count: int) -> np.ndarray:
    """Sorted, distinct query rows drawn with ``default_rng([seed, 99])``."""
    rng = np.random.default_rng([int(seed), 99])
    return np.sort(rng.choice(n_tokens, size=min(count, n_tokens), replace=False)).astype(np.int64)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()

# Frame pack: raw clips (frames, height, width) with 226 text tokens each,
# through the cogvideox workload's VAE and patchify factors
COGVIDEOX_PACK = {"clips": ((49, 480, 720), (25, 480, 720), (1, 480, 720), (33, 256, 384)),
                  "n_text": 226, "base": "cogvideox", "seed": 6, "sample_rows": 192}

# U-shaped sparsity over 12 layer positions: (mode, k) per layer
SUV_SCHEDULE = (("full", 1), ("skiparse_single", 2), ("skiparse_group", 2),
                ("skiparse_single", 4), ("skiparse_group", 4), ("skiparse_single", 8),
                ("skiparse_group", 8), ("skiparse_single", 4), ("skiparse_group", 4),
                ("skiparse_single", 2), ("skiparse_group", 2), ("full", 1))

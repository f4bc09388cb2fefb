"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (K rotated by osp_rope3d, then one osp_attn3d_fwd call
that rotates Q in its loader, over the whole tensor; and once with K
rotated in the loader too), checked against the fp64 oracle on seeded
sampled query rows.  O and LSE start filled with NaN, so every element of
both is checked to have been written.  Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import spatiotemporal_attention_amd as osp
import workloads
from parity_util import (LSE_ABS, assert_parity, grid_of, note, oracle_attn, qkv_for, to_np)

pytestmark = pytest.mark.gpu

SAMPLE = 256


def run_sampled(name, mode, sparse_k, variant="as-specified", fuse_rope=True):
    wl = workloads.WORKLOADS[name]
    grid = grid_of(wl)
    n = wl.n_text + int(np.prod(grid))
    shape = (wl.batch, n, wl.heads, wl.head_dim)
    scale = wl.input_scale if variant == "as-specified" else None
    seed = wl.seed if variant == "as-specified" else (wl.seed, 7)
    note(f"full-size {name} grid={grid} shape={shape} mode={mode} k={sparse_k} variant={variant} "
         f"fuse={fuse_rope}")
    cpu, (q, k, v) = qkv_for(seed, shape, scale)
    # outputs start as NaN: every element must be written by the call
    o = torch.full_like(q, float("nan"))
    lse = torch.full((wl.batch, wl.heads, n), float("nan"), dtype=torch.float32, device=q.device)
    osp.osp_attn3d_fwd(q, k, v, grid=grid, n_text=wl.n_text, mode=mode, sparse_k=sparse_k,
                       rope_split=wl.rope_split, theta=wl.theta, fuse_rope=fuse_rope, out=o,
                       lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any(), "O has unwritten elements"
    assert not torch.isnan(lse).any(), "LSE has unwritten elements"
    rows = workloads.sample_rows(wl.seed, n, SAMPLE)
    want_o, want_l = oracle_attn(cpu, grid=grid, n_text=wl.n_text, mode=mode, sparse_k=sparse_k,
                                 rope_split=wl.rope_split, theta=wl.theta, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    got_o = to_np(o.index_select(1, idx))
    got_l = to_np(lse.index_select(2, idx))
    assert_parity(got_o, want_o, f"{name} {mode} k={sparse_k} {variant} ({len(rows)} rows)")
    assert np.abs(got_l - want_l).max() <= LSE_ABS


def test_osp480_full_k_rotated_in_loader():
    run_sampled("osp480", "full", 1, fuse_rope="qk")


@pytest.mark.parametrize("variant", ["as-specified", "unscaled"])
def test_osp480_full(variant):
    run_sampled("osp480", "full", 1, variant)


def test_cogvideox_joint_full():
    run_sampled("cogvideox", "full", 1)


@pytest.mark.parametrize("mode", ["skiparse_single", "skiparse_group"])
@pytest.mark.parametrize("variant", ["as-specified", "unscaled"])
def test_osp480_skiparse_k4(mode, variant):
    run_sampled("osp480_skiparse", mode, 4, variant)


@pytest.mark.parametrize("mode,k", [("full", 1), ("skiparse_single", 4), ("skiparse_group", 4)])
def test_osp720(mode, k):
    run_sampled("osp720", mode, k)


@pytest.mark.parametrize("half", ["spatial", "temporal"])
def test_osp480_separated_spatial_temporal(half):
    # spatial: 24 frames of 1,200 tokens; temporal: 1,200 positions of 24
    grid = grid_of(workloads.WORKLOADS["osp480"])
    mode, k = ("block", grid[0]) if half == "spatial" else ("skiparse_single", grid[1] * grid[2])
    run_sampled("osp480", mode, k, "unscaled")


@pytest.mark.parametrize("mode,k", [("full", 1), ("skiparse_single", 4), ("skiparse_group", 4)])
def test_osp15_8x8x8_d128(mode, k):
    # 121x576x1024 through the 8x8x8 VAE: 16x36x64 = 36,864 tokens, D=128
    run_sampled("osp15", mode, k)


def test_osp480_skiparse2d_single_k4():
    # 2 x 2 lattice over h and w in each of the 24 frames: 4 subsequences of 7,200
    run_sampled("osp480_skiparse", "skiparse2d_single", 4)


@pytest.mark.parametrize("mode", ["skiparse2d_single", "skiparse2d_group"])
def test_osp15_skiparse2d_k4(mode):
    # 16x36x64: H and W divisible by 4, so the 2 x 2 patch rule applies too
    run_sampled("osp15", mode, 4)

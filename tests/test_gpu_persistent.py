"""GPU tests of the persistent forward launch: a call at head_dim 64 or 96
with fixed-row remaps and more query tiles than the GPU holds workgroups
at once takes one workgroup per slot, each walking its XCD's list of tiles.
Every case is run both ways (the default and OSP_ONE_TILE_PER_WORKGROUP)
with O and LSE filled with NaN first, and the two results must be the same
bits and fully written: the per-tile arithmetic is the same, only the
launch differs.  The persistent cases cover full, block, Single and Group
Skip, tiles left over after the XCD split (one more tile for some
workgroups), subsequences shorter than the slot count of key tiles, and Q
already rotated, head_dim 64 with text tokens in front and with Skiparse,
head_dim 96 with text tokens, batch 2 and a strided output, and units of
one query tile with fewer key tiles than prefetch slots; the row-table
and head_dim 128 cases take one tile per workgroup either way and check
that the flag changes nothing there.  One case is also checked against the fp64 oracle on sampled rows.
Needs an MI355X."""
import numpy as np
import pytest
import torch

import spatiotemporal_attention_amd as osp
import workloads
from parity_util import LSE_ABS, assert_parity, note, oracle_attn, qkv_for, to_np

pytestmark = pytest.mark.gpu

# name: (grid, n_text, heads, head_dim, rope split, mode, k, fuse_rope)
CASES = {
    # 24 heads x 113 tiles of 256 rows (fixed rows, Q rotated in the loader)
    "osp480_full": ((24, 30, 40), 0, 24, 96, (32, 32, 32), "full", 1, True),
    "osp480_single_k4": ((24, 30, 40), 0, 24, 96, (32, 32, 32), "skiparse_single", 4, True),
    "osp480_group_k4": ((24, 30, 40), 0, 24, 96, (32, 32, 32), "skiparse_group", 4, True),
    # row table (per-row remap): Skiparse-2D, and Group Skip with 64 % k != 0
    "osp480_s2d_single_k4": ((24, 30, 40), 0, 24, 96, (32, 32, 32), "skiparse2d_single", 4, True),
    "group_k3_rowtable": ((9, 30, 40), 0, 8, 96, (32, 32, 32), "skiparse_group", 3, True),
    # one head, 258 tiles: 32 per XCD plus one for XCDs 0 and 1, ragged last tile
    "one_head_258_tiles": ((25, 44, 60), 0, 1, 96, (32, 32, 32), "full", 1, True),
    # windows of 100 tokens: two key tiles per subsequence, fewer than the slots
    "window_100": ((25, 40, 40), 0, 2, 96, (32, 32, 32), "block", 400, True),
    # Q and K already rotated (the instances without the rotation)
    "osp480_prerotated": ((24, 30, 40), 0, 24, 96, (32, 32, 32), "full", 1, False),
    # head_dim 64 with text tokens in front; head_dim 128
    "cogvideox_joint": ((13, 30, 45), 226, 48, 64, (16, 24, 24), "full", 1, True),
    "osp15_d128": ((16, 36, 64), 0, 24, 128, (32, 48, 48), "full", 1, True),
    # head_dim 96 with text tokens in front (ragged last query and key tiles)
    "d96_text": ((12, 30, 40), 77, 24, 96, (32, 32, 32), "full", 1, True),
    # head_dim 64 Skiparse: Group Skip k=4 and Single Skip k=2 (fixed rows at 32-key tiles)
    "d64_group_k4": ((13, 32, 44), 0, 24, 64, (16, 24, 24), "skiparse_group", 4, True),
    "d64_single_k2": ((13, 30, 45), 0, 16, 64, (16, 24, 24), "skiparse_single", 2, True),
    # one query tile per unit and fewer key tiles than the prefetch slots:
    # 130-token windows (three key tiles, the last with 2 keys), and 65-token
    # windows, the shortest the flash kernel takes, at head_dim 96 and 64
    "window_130": ((10, 26, 50), 0, 24, 96, (32, 32, 32), "block", 100, True),
    "window_65": ((5, 13, 40), 0, 48, 96, (32, 32, 32), "block", 40, True),
    "window_65_d64": ((5, 13, 40), 0, 48, 64, (16, 24, 24), "block", 40, True),
}


def _run(q, k, v, grid, n_text, mode, sk, split, fuse, one_tile, out=None):
    b, n, h, _ = q.shape
    o = torch.full_like(q, float("nan")) if out is None else out.fill_(float("nan"))
    lse = torch.full((b, h, n), float("nan"), dtype=torch.float32, device=q.device)
    osp.osp_attn3d_fwd(q, k, v, grid=grid, n_text=n_text, mode=mode, sparse_k=sk,
                       rope_split=split, fuse_rope=fuse, out=o, lse=lse,
                       one_tile_per_workgroup=one_tile)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any(), "O has unwritten elements"
    assert not torch.isnan(lse).any(), "LSE has unwritten elements"
    return o, lse


@pytest.mark.parametrize("name", list(CASES))
def test_persistent_equals_one_tile_per_workgroup(name):
    grid, n_text, heads, d, split, mode, sk, fuse = CASES[name]
    n = n_text + int(np.prod(grid))
    shape = (1, n, heads, d)
    note(f"persistent {name}: shape={shape} grid={grid} mode={mode} k={sk} fuse={fuse}")
    cpu, (q, k, v) = qkv_for((11, len(name)), shape)
    o1, l1 = _run(q, k, v, grid, n_text, mode, sk, split, fuse, False)
    o2, l2 = _run(q, k, v, grid, n_text, mode, sk, split, fuse, True)
    assert torch.equal(o1, o2), "O differs between the two launches"
    assert torch.equal(l1, l2), "LSE differs between the two launches"
    if name in ("one_head_258_tiles", "window_130", "window_65_d64"):
        rows = workloads.sample_rows(11, n, 256)
        want_o, want_l = oracle_attn(cpu, grid=grid, n_text=n_text, mode=mode, sparse_k=sk,
                                     rope_split=split, rows=rows)
        idx = torch.from_numpy(rows).cuda()
        assert_parity(to_np(o1.index_select(1, idx)), want_o, f"{name} ({len(rows)} rows)")
        assert np.abs(to_np(l1.index_select(2, idx)) - want_l).max() <= LSE_ABS


def test_persistent_back_to_back_calls():
    # two persistent calls in a row on one stream, the second smaller: the
    # second must not see state left by the first
    grid, split = (24, 30, 40), (32, 32, 32)
    shape = (1, 28800, 24, 96)
    note(f"persistent back-to-back: shape={shape}")
    _, (q, k, v) = qkv_for((11, 99), shape)
    a1, la1 = _run(q, k, v, grid, 0, "full", 1, split, True, False)
    small = (12, 30, 40)
    qs, ks, vs = (t[:, :14400].contiguous() for t in (q, k, v))
    b1, lb1 = _run(qs, ks, vs, small, 0, "skiparse_group", 4, split, True, False)
    b2, lb2 = _run(qs, ks, vs, small, 0, "skiparse_group", 4, split, True, True)
    a2, la2 = _run(q, k, v, grid, 0, "full", 1, split, True, True)
    assert torch.equal(a1, a2) and torch.equal(la1, la2)
    assert torch.equal(b1, b2) and torch.equal(lb1, lb2)


def test_persistent_batch_and_strided_output():
    # batch 2 (the tile list spans both batches) with O written into a
    # strided view (every other head of a wider tensor): both launches give
    # the same bits, the untouched heads stay as they were, and sampled rows
    # of the second batch match the oracle
    grid, split = (12, 30, 40), (32, 32, 32)
    shape = (2, 14400, 24, 96)
    note(f"persistent batch 2, strided O: shape={shape}")
    cpu, (q, k, v) = qkv_for((11, 77), shape)
    wide = [torch.zeros((2, 14400, 48, 96), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    res = []
    for one_tile, w in zip((False, True), wide):
        res.append(_run(q, k, v, grid, 0, "full", 1, split, True, one_tile, out=w[:, :, 0::2]))
    (o1, l1), (o2, l2) = res
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for w in wide:
        assert not w[:, :, 1::2].any(), "heads outside the view were written"
    rows = workloads.sample_rows(12, 14400, 96)
    want_o, want_l = oracle_attn(tuple(t[1:2] for t in cpu), grid=grid, n_text=0, mode="full",
                                 sparse_k=1, rope_split=split, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    assert_parity(to_np(o1[1:2].index_select(1, idx)), want_o, f"batch 1 ({len(rows)} rows)")
    assert np.abs(to_np(l1[1:2].index_select(2, idx)) - want_l).max() <= LSE_ABS

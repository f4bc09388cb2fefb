"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element, at sizes that span several tiles and a ragged tail;
plus bit-exact device index maps, fused == unfused RoPE, determinism and
fully-written outputs.  Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle
import spatiotemporal_attention_amd as osp
import workloads
from parity_util import (LSE_ABS, MAX_ABS, REL_L2, assert_parity, note, oracle_attn, qkv_for,
                         to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    osp.lib()
    yield
    torch.cuda.synchronize()


def run_case(seed, *, grid, n_text, heads, head_dim, rope_split, mode="full", sparse_k=1,
             scale=None, q_mult=None, theta=1e4, sm_scale=None, pos_offset=(0, 0, 0),
             batch=1, lse=True, fuse_rope="qk", tag="", tol=1.0):
    n = n_text + int(np.prod(grid))
    shape = (batch, n, heads, head_dim)
    note(f"case {tag} seed={seed} shape={shape} grid={grid} n_text={n_text} mode={mode} "
         f"k={sparse_k} rope={rope_split} fuse={fuse_rope}")
    cpu, (q, k, v) = qkv_for(seed, shape, scale, q_mult)
    if fuse_rope in (False, "k"):
        q = osp.osp_rope3d(q, grid=grid, n_text=n_text, rope_split=rope_split, theta=theta,
                           pos_offset=pos_offset)
    if fuse_rope in (False, "q"):
        k = osp.osp_rope3d(k, grid=grid, n_text=n_text, rope_split=rope_split, theta=theta,
                           pos_offset=pos_offset)
    o, l = osp.osp_attn3d_fwd(q, k, v, grid=grid, n_text=n_text, mode=mode, sparse_k=sparse_k,
                              rope_split=rope_split, theta=theta, sm_scale=sm_scale,
                              pos_offset=pos_offset, fuse_rope=fuse_rope, return_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = oracle_attn(cpu, grid=grid, n_text=n_text, mode=mode, sparse_k=sparse_k,
                                 rope_split=rope_split, theta=theta, sm_scale=sm_scale,
                                 pos_offset=pos_offset)
    assert_parity(to_np(o), want_o, f"O {tag}", MAX_ABS * tol, REL_L2 * tol)
    if lse:
        got_l = to_np(l)
        assert np.isfinite(got_l).all()
        assert np.abs(got_l - want_l).max() <= LSE_ABS * tol, np.abs(got_l - want_l).max()
    return o, l


# ---------------------------------------------------------------- RoPE pass
@pytest.mark.parametrize("grid,n_text,heads,d,split,offset", [
    ((5, 8, 8), 0, 2, 64, (16, 24, 24), (0, 0, 0)),
    ((4, 12, 15), 0, 3, 96, (32, 32, 32), (0, 0, 0)),
    ((3, 10, 12), 37, 2, 64, (16, 24, 24), (2, -1, 5)),
    ((3, 7, 9), 5, 2, 96, (36, 36, 24), (0, 0, 0)),      # chunks straddle 8-channel blocks
    ((2, 6, 7), 0, 2, 128, (32, 48, 48), (0, 0, 0)),
    ((200, 4, 80), 0, 1, 96, (32, 32, 32), (0, 0, 0)),   # cos/sin table too big: direct path
])
def test_rope3d_matches_oracle(grid, n_text, heads, d, split, offset):
    n = n_text + int(np.prod(grid))
    note(f"rope3d grid={grid} n_text={n_text} d={d} split={split}")
    x = workloads.gaussian_bf16(5, 0, (2, n, heads, d))
    y = osp.osp_rope3d(x.cuda(), grid=grid, n_text=n_text, rope_split=split, pos_offset=offset)
    torch.cuda.synchronize()
    xw = workloads.to_f64(x)
    want = oracle.rope3d(xw, grid, n_text, split, 1e4, offset)
    got = to_np(y)
    bound = 2.0 ** -8 * np.abs(want) + 1e-5 * np.abs(xw).max()
    assert (np.abs(got - want) <= bound).all(), np.abs(got - want).max()
    assert np.array_equal(got[:, :n_text], xw[:, :n_text])    # text rows copied


def test_rope3d_in_place_and_strided():
    grid, split = (4, 6, 8), (16, 24, 24)
    n = 192
    x = workloads.gaussian_bf16(6, 0, (1, n, 3, 2, 64))    # packed [B, N, (q,k,v), H, D]
    xd = x.cuda()
    ref = osp.osp_rope3d(xd[:, :, 0].contiguous(), grid=grid, rope_split=split)
    view = xd[:, :, 0]
    osp.osp_rope3d(view, grid=grid, rope_split=split, out=view)
    torch.cuda.synchronize()
    assert torch.equal(xd[:, :, 0], ref)
    assert torch.equal(xd[:, :, 1:].cpu(), x[:, :, 1:])      # neighbours untouched


# ---------------------------------------------------------- attention, small
def test_tiny_full():
    run_case(0, grid=(5, 8, 8), n_text=0, heads=2, head_dim=64, rope_split=(16, 24, 24),
             tag="tiny-full")


@pytest.mark.parametrize("mode", ["skiparse_single", "skiparse_group"])
@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_tiny_skiparse(mode, k):
    run_case(0, grid=(5, 8, 8), n_text=0, heads=2, head_dim=64, rope_split=(16, 24, 24),
             mode=mode, sparse_k=k, tag=f"tiny-{mode}-{k}")


@pytest.mark.parametrize("k", [1, 2, 5, 10, 64, 320])
def test_tiny_block(k):
    run_case(0, grid=(5, 8, 8), n_text=0, heads=2, head_dim=64, rope_split=(16, 24, 24),
             mode="block", sparse_k=k, tag=f"tiny-block-{k}")


@pytest.mark.parametrize("half", ["spatial", "temporal"])
def test_separated_spatial_temporal(half):
    # 2D+1D attention: spatial = block with k = frames (each frame's 150
    # tokens: several key tiles, ragged); temporal = single skip with
    # k = H*W (each (h, w) position's 6 tokens across frames)
    grid = (6, 10, 15)
    mode, k = ("block", grid[0]) if half == "spatial" else ("skiparse_single", grid[1] * grid[2])
    run_case(11, grid=grid, n_text=0, heads=3, head_dim=96, rope_split=(32, 32, 32),
             mode=mode, sparse_k=k, tag=f"2d1d-{half}")


@pytest.mark.parametrize("variant", ["unscaled", "literal", "sharp"])
@pytest.mark.parametrize("mode,k", [("full", 1), ("skiparse_single", 4), ("skiparse_group", 4),
                                    ("skiparse_group", 2), ("skiparse_group", 3), ("block", 3)])
def test_multitile_d96(variant, mode, k):
    # 720 tokens: several 256-row query tiles and 64-key tiles, ragged tails.
    # "sharp" multiplies Q by 4 (logit std ~4 instead of ~1).  The kernel
    # rounds rotated Q and K to bf16 before the MFMA, so its logit error, and
    # with it the output error, grows in proportion to the logit scale: the
    # bound is the unit-scale bound times 4.
    scale = 1 / math.sqrt(96) if variant == "literal" else None
    q_mult = 4.0 if variant == "sharp" else None
    run_case(10, grid=(4, 12, 15), n_text=0, heads=3, head_dim=96, rope_split=(32, 32, 32),
             mode=mode, sparse_k=k, scale=scale, q_mult=q_mult, tag=f"mt96-{variant}-{mode}{k}",
             tol=4.0 if variant == "sharp" else 1.0)


@pytest.mark.parametrize("fuse", ["qk", True])
def test_group_skip_k_not_dividing_the_key_tile(fuse):
    # Group Skip with k = 3 against 32-key tiles (D=64): a tile's rows do not
    # sit at fixed offsets from its first token, so the loader remaps every
    # row (the path Group Skip takes whenever k does not divide the tile).
    # 288 tokens, L = 96: three key tiles per subsequence; batch 2.
    run_case(24, grid=(3, 8, 12), n_text=0, heads=2, head_dim=64, rope_split=(16, 24, 24),
             mode="skiparse_group", sparse_k=3, batch=2, fuse_rope=fuse, tag="group3-d64")
    # k = 5 at D=128 (64-key tiles), 1,200 tokens: L = 240, ragged last tile
    run_case(24, grid=(3, 20, 20), n_text=0, heads=2, head_dim=128, rope_split=(32, 48, 48),
             mode="skiparse_group", sparse_k=5, fuse_rope=fuse, tag="group5-d128")


@pytest.mark.parametrize("mode,k,grid,d,split,batch,fuse", [
    ("skiparse2d_single", 4, (6, 12, 16), 96, (32, 32, 32), 1, "qk"),   # L = 288: 3 tiles, ragged
    ("skiparse2d_single", 4, (6, 12, 16), 96, (32, 32, 32), 1, True),   # K by osp_rope3d, DMA path
    ("skiparse2d_group", 4, (5, 8, 12), 64, (16, 24, 24), 2, "qk"),     # L = 120
    ("skiparse2d_group", 4, (5, 8, 12), 64, (16, 24, 24), 2, False),
    ("skiparse2d_single", 9, (4, 12, 9), 128, (32, 48, 48), 1, "qk"),   # L = 48: short kernel
    ("skiparse2d_group", 9, (3, 18, 18), 96, (32, 32, 32), 1, "qk"),    # L = 108
    ("skiparse2d_single", 16, (24, 8, 8), 64, (16, 24, 24), 1, "qk"),   # L = 96
    ("skiparse2d_single", 1, (2, 6, 10), 64, (16, 24, 24), 1, "qk"),    # k = 1: full attention
])
def test_skiparse2d(mode, k, grid, d, split, batch, fuse):
    run_case(71, grid=grid, n_text=0, heads=2, head_dim=d, rope_split=split, mode=mode,
             sparse_k=k, batch=batch, fuse_rope=fuse, tag=f"{mode} k={k}")


@pytest.mark.parametrize("grid", [(2, 4, 4), (24, 30, 40), (16, 36, 64), (3, 18, 27)])
def test_device_index_maps_2d_bitexact(grid):
    n = int(np.prod(grid))
    for mode in ("skiparse2d_single", "skiparse2d_group"):
        for k in (4, 9):
            step = int(round(k ** 0.5)) * (1 if mode == "skiparse2d_single" else int(round(k ** 0.5)))
            if grid[1] % step or grid[2] % step:
                continue
            note(f"index3d {mode} k={k} grid={grid}")
            perm, inv = osp.osp_skiparse_index3d(mode, k, grid, device="cuda")
            torch.cuda.synchronize()
            want_perm, want_inv = oracle.skiparse_index(mode, k, n, grid)
            assert np.array_equal(perm.cpu().numpy(), want_perm), (mode, k, grid)
            assert np.array_equal(inv.cpu().numpy(), want_inv), (mode, k, grid)


def test_suv_schedule_layers():
    # every layer of the U-shaped schedule on one 768-token grid (a multiple
    # of 8^2, so that group skip at k = 8 divides it), each against the oracle
    for mode, k in workloads.SUV_SCHEDULE:
        run_case(12, grid=(3, 16, 16), n_text=0, heads=2, head_dim=96, rope_split=(32, 32, 32),
                 mode=mode, sparse_k=k, tag=f"suv-{mode}-{k}")


def test_text_tokens_d64():
    run_case(11, grid=(3, 10, 12), n_text=37, heads=2, head_dim=64, rope_split=(16, 24, 24),
             tag="text-d64")


def test_d128_and_batch2():
    run_case(12, grid=(3, 8, 11), n_text=0, heads=2, head_dim=128, rope_split=(32, 48, 48),
             batch=2, tag="d128-b2")
    run_case(12, grid=(3, 8, 12), n_text=0, heads=2, head_dim=128, rope_split=(32, 48, 48),
             mode="skiparse_single", sparse_k=3, tag="d128-single3")


def test_unaligned_rope_split_and_offsets():
    run_case(13, grid=(3, 7, 9), n_text=5, heads=2, head_dim=96, rope_split=(36, 36, 24),
             pos_offset=(3, 1, -2), theta=500.0, tag="split36")


def test_sm_scale_override():
    # logits 0.3 * sqrt(64) = 2.4 times the default's: the rounding error of
    # the bf16 operands grows with them, and so does the bound
    run_case(14, grid=(2, 9, 10), n_text=0, heads=2, head_dim=64, rope_split=(16, 24, 24),
             sm_scale=0.3, tag="scale0.3", tol=0.3 * math.sqrt(64))


def test_single_token_and_singleton_groups():
    # N = 1: the output is V.  single skip with k = N: every group is one token.
    o, _ = run_case(15, grid=(1, 1, 1), n_text=0, heads=2, head_dim=64, rope_split=(16, 24, 24),
                    tag="n1")
    run_case(15, grid=(1, 4, 4), n_text=0, heads=2, head_dim=64, rope_split=(16, 24, 24),
             mode="skiparse_single", sparse_k=16, tag="k=N")


@pytest.mark.parametrize("args", [
    dict(grid=(4, 12, 15), n_text=0, heads=3, head_dim=96, rope_split=(32, 32, 32)),
    dict(grid=(3, 10, 12), n_text=37, heads=2, head_dim=64, rope_split=(16, 24, 24)),
    dict(grid=(3, 7, 9), n_text=5, heads=2, head_dim=96, rope_split=(36, 36, 24)),
], ids=["d96", "d64-text", "d96-split36"])
def test_fused_equals_unfused_bitwise(args):
    # rotating K in the loader gives the same bf16 operands as osp_rope3d;
    # Q is rotated and scaled with one rounding when fused, so the Q path is
    # compared at equal Q handling only
    a, la = run_case(16, **args, tag="fused")
    b, lb = run_case(16, **args, fuse_rope="q", tag="fuse=q")
    assert torch.equal(a, b) and torch.equal(la, lb)
    c, lc = run_case(16, **args, fuse_rope=True, tag="fuse=True")   # K by its own pass
    assert torch.equal(c, b) and torch.equal(lc, lb)
    a, la = run_case(16, **args, fuse_rope="k", tag="fuse=k")
    b, lb = run_case(16, **args, fuse_rope=False, tag="fuse=none")
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_deterministic_and_fully_written():
    grid, split = (4, 12, 15), (32, 32, 32)
    _, (q, k, v) = qkv_for(18, (1, 720, 3, 96))
    outs = []
    for rep in range(2):
        for mode, kk in (("full", 1), ("skiparse_group", 4)):
            o = torch.full_like(q, float("nan"))
            lse = torch.full((1, 3, 720), float("nan"), device=q.device)
            note(f"determinism rep={rep} mode={mode}")
            osp.osp_attn3d_fwd(q, k, v, grid=grid, rope_split=split, mode=mode, sparse_k=kk,
                               out=o, lse=lse)
            torch.cuda.synchronize()
            assert not torch.isnan(o).any() and not torch.isnan(lse).any()
            outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[1][0], outs[3][0])
    assert torch.equal(outs[0][1], outs[2][1])


def test_strided_packed_qkv():
    grid, split = (3, 8, 10), (16, 24, 24)
    n = 240
    cpu = workloads.gaussian_bf16(19, 0, (1, n, 3, 2, 64))
    qkv = cpu.cuda()
    note("strided packed qkv")
    o = torch.empty((1, n, 2, 64), dtype=torch.bfloat16, device="cuda")
    # the default rotates K by its own pass into a temporary with K's strides
    osp.osp_attn3d_fwd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], grid=grid, rope_split=split,
                       out=o)
    o2 = osp.osp_attn3d_fwd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], grid=grid, rope_split=split,
                            fuse_rope="qk")
    torch.cuda.synchronize()
    assert torch.equal(qkv.cpu(), cpu)                  # the inputs are not touched
    assert torch.equal(o, o2)
    f = workloads.to_f64(cpu)
    want, _ = oracle.attn3d(f[:, :, 0], f[:, :, 1], f[:, :, 2], grid=grid, rope_split=split)
    assert_parity(to_np(o), want, "O strided")


def test_output_strides():
    grid, split = (3, 8, 10), (16, 24, 24)
    cpu, (q, k, v) = qkv_for(20, (1, 240, 2, 64))
    big = torch.zeros((1, 240, 4, 64), dtype=torch.bfloat16, device="cuda")
    note("output strides")
    osp.osp_attn3d_fwd(q, k, v, grid=grid, rope_split=split, out=big[:, :, 1:3])
    torch.cuda.synchronize()
    want, _ = oracle_attn(cpu, grid=grid, n_text=0, mode="full", sparse_k=1, rope_split=split)
    assert_parity(to_np(big[:, :, 1:3]), want, "O into a strided view")
    assert not big[:, :, 0].any() and not big[:, :, 3].any()


# --------------------------------------- short subsequences (L <= 64 rows)
# One wave per (batch, head, subsequence): temporal attention, small windows,
# Skiparse at large k, and whole sequences of at most 64 tokens.
@pytest.mark.parametrize("grid,n_text,d,split,mode,k,batch", [
    ((24, 6, 5), 0, 96, (32, 32, 32), "skiparse_single", 30, 1),     # temporal, L = 24
    ((33, 2, 3), 0, 64, (16, 24, 24), "skiparse_single", 6, 2),      # L = 33: two blocks
    ((8, 4, 4), 0, 128, (32, 48, 48), "skiparse_single", 2, 1),      # L = 64
    ((8, 4, 4), 0, 128, (32, 48, 48), "skiparse_group", 4, 1),       # L = 32
    ((5, 4, 8), 0, 96, (36, 36, 24), "block", 5, 2),                 # windows of 32
    ((5, 4, 8), 0, 64, (16, 24, 24), "skiparse_group", 4, 1),        # L = 40
    ((2, 3, 4), 7, 64, (16, 24, 24), "full", 1, 2),                  # text + video, N = 31
    ((3, 4, 5), 2, 96, (32, 32, 32), "full", 1, 1),                  # N = 62
])
def test_short_subsequences(grid, n_text, d, split, mode, k, batch):
    run_case(21, grid=grid, n_text=n_text, heads=3, head_dim=d, rope_split=split, mode=mode,
             sparse_k=k, batch=batch, tag=f"short-{mode}-{k}")
    run_case(22, grid=grid, n_text=n_text, heads=3, head_dim=d, rope_split=split, mode=mode,
             sparse_k=k, batch=batch, q_mult=4.0, tag=f"short-sharp-{mode}-{k}", tol=4.0)


def test_short_fused_equals_unfused_and_fully_written():
    args = dict(grid=(24, 6, 5), n_text=0, heads=5, head_dim=96, rope_split=(32, 32, 32),
                mode="skiparse_single", sparse_k=30)
    a, la = run_case(23, **args, tag="short-fused")
    b, lb = run_case(23, **args, fuse_rope="q", tag="short-fuse=q")
    assert torch.equal(a, b) and torch.equal(la, lb)
    # 5 heads x 30 subsequences = 150 units: a partly filled last workgroup
    _, (q, k, v) = qkv_for(23, (1, 720, 5, 96))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 5, 720), float("nan"), device=q.device)
    osp.osp_attn3d_fwd(q, k, v, grid=(24, 6, 5), rope_split=(32, 32, 32),
                       mode="skiparse_single", sparse_k=30, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    assert torch.equal(o, a)


# ------------------------------------------------------------ index maps
@pytest.mark.parametrize("n,k", [(320, 4), (28800, 4), (86400, 4), (720, 2), (4096, 8),
                                 (1 << 20, 16), (17550, 3), (1, 1)])
def test_device_index_maps_bitexact(n, k):
    for mode in ("full", "skiparse_single", "skiparse_group", "block"):
        div = {"full": 1, "skiparse_single": k, "skiparse_group": k * k, "block": k}[mode]
        if n % div:
            continue
        note(f"device index map mode={mode} n={n} k={k}")
        perm, inv = osp.osp_skiparse_index(mode, k, n, device="cuda")
        torch.cuda.synchronize()
        want_perm, want_inv = oracle.skiparse_index(mode, k, n)
        assert np.array_equal(perm.cpu().numpy(), want_perm)
        assert np.array_equal(inv.cpu().numpy(), want_inv)

"""GPU parity of the attention backward (through the C ABI) against the fp64
oracle: dQ, dK, dV element by element at sizes that span several tiles and
ragged tails, every attention mode, text tokens, strided layouts, and the
RoPE transpose; at a full 28,800-token sequence, Skiparse k=4 gradients
element by element over whole 7,200-row subsequences, and for full
attention sampled dQ rows (each one exact in the oracle) and the column-sum
identities of dK and dV.

Tolerances, from an emulation of the kernel's rounding steps (bf16 output
O and fp32 lse from the forward, P and dS rounded to bf16 for the MFMA
products, outputs rounded to bf16) against fp64 on random inputs: the
worst rel-L2 there is 3.2e-3 and the worst max-abs 5.8e-3 x max|ref|.
The bar is rel-L2 <= 5e-3 and max-abs <= 2e-2 x max|ref|; with the RoPE
chain (rotated q and k rounded to bf16, dq and dk rounded once more after
the transpose) the emulation reaches rel-L2 4.0e-3 and max-abs 9.4e-3 x
max|ref|, and the bar is rel-L2 <= 8e-3.  The emulation is
tests/rounding_model.py; tests/test_rounding_bars.py runs it on these
tests' own inputs on the CPU.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
import spatiotemporal_attention_amd as osp
import workloads
from parity_util import assert_parity, note, qkv_for, to_np

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
REL_L2_ROPE = 8e-3
MAX_REL = 2e-2      # max-abs bound, times max |reference|


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    osp.lib()
    yield
    torch.cuda.synchronize()


def _check(got, want, tag, rel):
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert_parity(to_np(g), w, f"{name} {tag}", MAX_REL * float(np.abs(w).max()),
                      REL_L2_ROPE if (rel and name != "dv") else REL_L2)


def bwd_case(seed, *, grid, n_text=0, heads, head_dim, rope_split=None, mode="full",
             sparse_k=1, sm_scale=None, batch=1, rope_chain=False, tag=""):
    n = n_text + int(np.prod(grid))
    shape = (batch, n, heads, head_dim)
    split = rope_split or (head_dim, 0, 0)
    note(f"bwd {tag} seed={seed} shape={shape} grid={grid} n_text={n_text} mode={mode} "
         f"k={sparse_k} rope_chain={rope_chain}")
    cpu, (q, k, v) = qkv_for(seed, shape)
    do_cpu = workloads.make_dout(seed, shape)
    do = do_cpu.cuda()
    if rope_chain:
        q = osp.osp_rope3d(q, grid=grid, n_text=n_text, rope_split=split)
        k = osp.osp_rope3d(k, grid=grid, n_text=n_text, rope_split=split)
    o, lse = osp.osp_attn3d_fwd(q, k, v, grid=grid, n_text=n_text, mode=mode, sparse_k=sparse_k,
                                rope_split=split, sm_scale=sm_scale, fuse_rope=False,
                                return_lse=True)
    dq, dk, dv = osp.osp_attn3d_bwd(q, k, v, o, lse, do, grid=grid, n_text=n_text, mode=mode,
                                    sparse_k=sparse_k, sm_scale=sm_scale)
    if rope_chain:
        osp.osp_rope3d_inv(dq, grid=grid, n_text=n_text, rope_split=split, out=dq)
        osp.osp_rope3d_inv(dk, grid=grid, n_text=n_text, rope_split=split, out=dk)
    torch.cuda.synchronize()
    want = oracle.attn3d_bwd(*(workloads.to_f64(t) for t in cpu), workloads.to_f64(do_cpu),
                             grid=grid, n_text=n_text, mode=mode, sparse_k=sparse_k,
                             rope_split=split, sm_scale=sm_scale, rope=rope_chain)
    _check((dq, dk, dv), want, tag, rope_chain)


# ------------------------------------------------------------ RoPE transpose
@pytest.mark.parametrize("grid,n_text,d,split", [
    ((5, 8, 8), 0, 64, (16, 24, 24)),
    ((3, 10, 12), 37, 96, (32, 32, 32)),
    ((3, 7, 9), 5, 96, (36, 36, 24)),
    ((2, 6, 7), 0, 128, (32, 48, 48)),
])
def test_rope3d_inv_matches_oracle_transpose(grid, n_text, d, split):
    n = n_text + int(np.prod(grid))
    note(f"rope3d_inv grid={grid} n_text={n_text} d={d} split={split}")
    x = workloads.gaussian_bf16(7, 0, (2, n, 2, d))
    y = osp.osp_rope3d_inv(x.cuda(), grid=grid, n_text=n_text, rope_split=split)
    back = osp.osp_rope3d(y, grid=grid, n_text=n_text, rope_split=split)
    torch.cuda.synchronize()
    xw = workloads.to_f64(x)
    want = oracle.rope3d_transpose(xw, grid, n_text, split, 1e4)
    got = to_np(y)
    bound = 2.0 ** -8 * np.abs(want) + 1e-5 * np.abs(xw).max()
    assert (np.abs(got - want) <= bound).all(), np.abs(got - want).max()
    assert np.array_equal(got[:, :n_text], xw[:, :n_text])
    # rotating back recovers x up to the two bf16 roundings
    assert np.abs(to_np(back) - xw).max() <= 2.0 ** -7 * np.abs(xw).max()


# ----------------------------------------------------------------- backward
@pytest.mark.parametrize("d", [64, 96, 128])
def test_bwd_full_ragged(d):
    # 315 tokens: ragged against the 64-row tiles and the 128-row blocks
    bwd_case(0, grid=(5, 7, 9), heads=2, head_dim=d, tag=f"full-d{d}")


@pytest.mark.parametrize("mode,k", [("skiparse_single", 2), ("skiparse_single", 4),
                                    ("skiparse_group", 2), ("skiparse_group", 4),
                                    ("block", 5), ("block", 64), ("skiparse_single", 1)])
def test_bwd_modes(mode, k):
    bwd_case(1, grid=(5, 8, 8), heads=2, head_dim=64, mode=mode, sparse_k=k,
             tag=f"{mode}-{k}")


@pytest.mark.parametrize("mode,k,grid,d", [
    ("skiparse2d_single", 4, (5, 8, 12), 64),     # L = 120: two tiles, the second ragged
    ("skiparse2d_group", 4, (3, 12, 16), 96),     # L = 144
    ("skiparse2d_single", 9, (4, 12, 9), 128),    # L = 48
    ("skiparse2d_group", 9, (2, 18, 9), 64),      # L = 36
])
def test_bwd_skiparse2d(mode, k, grid, d):
    bwd_case(81, grid=grid, heads=2, head_dim=d, mode=mode, sparse_k=k, batch=2 if d == 64 else 1,
             tag=f"{mode} k={k}")


def test_bwd_text_tokens_batch_and_scale():
    bwd_case(2, grid=(3, 10, 12), n_text=37, heads=3, head_dim=96, batch=2, sm_scale=0.2,
             tag="text-batch-scale")


@pytest.mark.parametrize("d,split", [(64, (16, 24, 24)), (128, (32, 48, 48))])
def test_bwd_rope_chain(d, split):
    # rope3d -> forward -> backward -> rope3d_inv: gradients with respect to
    # q and k before the rotation
    bwd_case(3, grid=(4, 9, 10), n_text=0, heads=2, head_dim=d, rope_split=split,
             rope_chain=True, tag=f"rope-chain-d{d}")


def test_bwd_separated_spatial_temporal():
    grid = (6, 10, 15)
    bwd_case(4, grid=grid, heads=2, head_dim=96, mode="block", sparse_k=grid[0], tag="spatial")
    bwd_case(4, grid=grid, heads=2, head_dim=96, mode="skiparse_single",
             sparse_k=grid[1] * grid[2], tag="temporal")


def test_bwd_strided_layout_and_determinism():
    # q, k, v, dout and o as views of one packed [B, N, 5, H, D] tensor; dq,
    # dk, dv written into a packed [B, N, 3, H, D] tensor
    grid, heads, d = (3, 8, 11), 2, 64
    n = int(np.prod(grid))
    note(f"bwd strided grid={grid}")
    packed = torch.stack([workloads.gaussian_bf16(5, i, (1, n, heads, d)) for i in range(4)]
                         + [torch.zeros(1, n, heads, d, dtype=torch.bfloat16)], 2)
    dev = packed.cuda()
    q, k, v, do, o = (dev[:, :, i] for i in range(5))
    _, lse = osp.osp_attn3d_fwd(q, k, v, grid=grid, rope_split=(d, 0, 0), fuse_rope=False,
                                out=o, return_lse=True)
    out = torch.full((1, n, 3, heads, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    osp.osp_attn3d_bwd(q, k, v, o, lse, do, grid=grid, dq=out[:, :, 0], dk=out[:, :, 1],
                       dv=out[:, :, 2])
    again = osp.osp_attn3d_bwd(*(t.contiguous() for t in (q, k, v, o)), lse, do.contiguous(),
                               grid=grid)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(out[:, :, i], again[i])      # layout-independent, deterministic
    want = oracle.attn3d_bwd(*(workloads.to_f64(packed[:, :, i]) for i in range(4)), grid=grid,
                             rope_split=(d, 0, 0), rope=False)
    _check(again, want, "strided", False)


# ---------------------------------------------------------- full-size checks
@pytest.mark.parametrize("mode,k", [("full", 1), ("skiparse_single", 4), ("skiparse_group", 4),
                                    ("skiparse2d_single", 4)])
def test_bwd_osp480_full_size(mode, k):
    """28,800 tokens (93x480x640 clip: 24x30x40 latent grid), 2 heads of 96,
    in the launch configuration the benchmark times, gradients written into
    NaN-filled tensors (every element must be written).

    Skiparse k=4: each subsequence has 7,200 rows, so the oracle computes
    dQ, dK and dV of every subsequence and head whole (a 7,200 x 7,200 fp64
    problem each), and all three are compared element by element.

    Full attention (one 28,800-row sequence): dQ rows are exact per row in
    the oracle (a row's gradient needs only its own scores), so 48 sampled
    rows are compared; dK and dV are checked through identities that hold
    at any size: over a subsequence's keys, dK sums to 0 (each row of dS
    sums to 0) and dV sums to the sum of dO over its queries (rows of P sum
    to 1)."""
    grid, heads, d = (24, 30, 40), 2, 96
    n = int(np.prod(grid))
    shape = (1, n, heads, d)
    note(f"bwd osp480 full size mode={mode} k={k}")
    cpu, (q, k_, v) = qkv_for(9, shape)
    do_cpu = workloads.make_dout(9, shape)
    o, lse = osp.osp_attn3d_fwd(q, k_, v, grid=grid, mode=mode, sparse_k=k,
                                rope_split=(32, 32, 32), fuse_rope=False, return_lse=True)
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    osp.osp_attn3d_bwd(q, k_, v, o, lse, do_cpu.cuda(), grid=grid, mode=mode, sparse_k=k,
                       dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    for name, g in zip(("dq", "dk", "dv"), grads):
        assert not torch.isnan(g).any(), f"{name} has unwritten elements"
    qw, kw, vw = (workloads.to_f64(t) for t in cpu)
    dow = workloads.to_f64(do_cpu)
    got_q, got_k, got_v = (to_np(t) for t in grads)
    scale = 1.0 / np.sqrt(d)
    rows = workloads.sample_rows(9, n, 48)
    for j, g in enumerate(oracle.skiparse_groups(mode, k, n, grid)):
        for h in range(heads):
            if mode != "full":
                want = oracle.softmax_attention_bwd(qw[0, g, h], kw[0, g, h], vw[0, g, h],
                                                    dow[0, g, h], scale)
                for name, got, w in zip(("dq", "dk", "dv"), (got_q, got_k, got_v), want):
                    assert_parity(got[0, g, h], w, f"{name} subsequence {j} h={h}",
                                  MAX_REL * float(np.abs(w).max()), REL_L2)
                continue
            want_q, _, _ = oracle.softmax_attention_bwd(qw[0, rows, h], kw[0, g, h], vw[0, g, h],
                                                        dow[0, rows, h], scale)
            assert_parity(got_q[0, rows, h], want_q, f"dq rows h={h}",
                          MAX_REL * float(np.abs(want_q).max()), REL_L2)
            # identities over the subsequence g, per channel, relative to the
            # sum of magnitudes (fp64 sums of the bf16 outputs)
            gk, gv = got_k[0, g, h], got_v[0, g, h]
            assert (np.abs(gk.sum(axis=0)) <= 1e-2 * np.abs(gk).sum(axis=0)).all()
            want_dv = dow[0, g, h].sum(axis=0)
            assert (np.abs(gv.sum(axis=0) - want_dv) <= 1e-2 * np.abs(gv).sum(axis=0)).all()

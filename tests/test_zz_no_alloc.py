"""The allocation-free backward (osp_attn3d_bwd_noalloc) against the
workspace backward (osp_attn3d_bwd), through the C ABI: two calls in a row
on one GPU, the second with a smaller input, each bit-identical to the
workspace call on the same inputs (the same kernels run on the same
values; only where the two row arrays live differs) and within the
backward's parity bar of the fp64 oracle.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
import spatiotemporal_attention_amd as osp
import workloads
from parity_util import assert_parity, note, qkv_for, to_np

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3        # the backward's bars (tests/test_gpu_bwd.py)
MAX_REL = 2e-2


def _case(seed, grid, heads, d, mode, k):
    n = int(np.prod(grid))
    shape = (1, n, heads, d)
    note(f"noalloc bwd seed={seed} grid={grid} heads={heads} d={d} mode={mode} k={k}")
    cpu, (q, k_, v) = qkv_for(seed, shape)
    do_cpu = workloads.make_dout(seed, shape)
    do = do_cpu.cuda()
    o, lse = osp.osp_attn3d_fwd(q, k_, v, grid=grid, mode=mode, sparse_k=k, rope_split=(d, 0, 0),
                                fuse_rope=False, return_lse=True)
    want = osp.osp_attn3d_bwd(q, k_, v, o, lse, do, grid=grid, mode=mode, sparse_k=k)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    osp.osp_attn3d_bwd_noalloc(q, k_, v, o, lse, do, grid=grid, mode=mode, sparse_k=k,
                               dq=got[0], dk=got[1], dv=got[2])
    torch.cuda.synchronize()
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert torch.equal(g, w), f"{name}: noalloc differs from the workspace call"
    ref = oracle.attn3d_bwd(*(workloads.to_f64(t) for t in cpu), workloads.to_f64(do_cpu),
                            grid=grid, mode=mode, sparse_k=k, rope_split=(d, 0, 0), rope=False)
    for name, g, w in zip(("dq", "dk", "dv"), got, ref):
        assert_parity(to_np(g), w, f"noalloc {name}", MAX_REL * float(np.abs(w).max()), REL_L2)


def test_noalloc_bwd_two_calls_second_smaller():
    assert torch.cuda.is_available()
    # 2,880 tokens x 3 heads, then 315 tokens x 2 heads: the second call
    # reuses the scratch the first one filled
    _case(31, (4, 24, 30), 3, 96, "skiparse_group", 4)
    _case(32, (5, 7, 9), 2, 64, "full", 1)

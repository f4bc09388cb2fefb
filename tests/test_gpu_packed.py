"""GPU parity of packed sequences (several videos in one sequence,
block-diagonal attention, RoPE from 0 on each video's own grid) against
the fp64 oracle, through the C ABI: small packs element by element (both
the short-subsequence and the flash kernel, Skiparse inside the segments,
fused and unfused K rotation), each segment against a plain forward call on
its slice (bit for bit: a packed launch runs the same arithmetic per
segment), more segments than one launch's table holds, the CogVideoX
frame pack on sampled rows with NaN-filled outputs, and the packed
backward through the RoPE chain (against plain backward calls per segment
and the oracle; at full size element by element on one head).  Needs an
MI355X."""
import numpy as np
import pytest
import torch

import oracle
import spatiotemporal_attention_amd as osp
import workloads
from parity_util import LSE_ABS, MAX_ABS, REL_L2, assert_parity, note, qkv_for, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    osp.lib()
    yield
    torch.cuda.synchronize()


def _packed_case(seed, segments, *, heads, head_dim, split, mode="full", sparse_k=1, batch=1,
                 fuse_rope="qk", tag=""):
    n = sum(nt + int(np.prod(g)) for nt, g in segments)
    shape = (batch, n, heads, head_dim)
    note(f"packed {tag} seed={seed} shape={shape} segments={segments} mode={mode} k={sparse_k}")
    cpu, (q, k, v) = qkv_for(seed, shape)
    o, lse = osp.osp_attn3d_packed_fwd(q, k, v, segments=segments, mode=mode, sparse_k=sparse_k,
                                       rope_split=split, fuse_rope=fuse_rope, return_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = oracle.attn3d_packed(*(workloads.to_f64(t) for t in cpu), segments=segments,
                                          mode=mode, sparse_k=sparse_k, rope_split=split)
    assert_parity(to_np(o), want_o, f"O packed {tag}", MAX_ABS, REL_L2)
    got_l = to_np(lse)
    assert np.abs(got_l - want_l).max() <= LSE_ABS, np.abs(got_l - want_l).max()
    return (q, k, v), o, lse


SMALL = [(3, (2, 3, 4)), (0, (1, 4, 5)), (5, (3, 2, 2)), (0, (2, 8, 10))]


@pytest.mark.parametrize("d,split", [(64, (16, 24, 24)), (96, (32, 32, 32)),
                                     (128, (32, 48, 48))])
def test_packed_small(d, split):
    # three segments of <= 64 tokens (short kernel) and one of 160 (flash kernel)
    _packed_case(30, SMALL, heads=2, head_dim=d, split=split, batch=2, tag=f"d{d}")


@pytest.mark.parametrize("mode,k", [("skiparse_single", 4), ("skiparse_group", 2), ("block", 2)])
def test_packed_skiparse_per_segment(mode, k):
    segs = [(0, (4, 4, 4)), (0, (2, 8, 8)), (0, (1, 6, 8)), (0, (2, 10, 12))]
    _packed_case(31, segs, heads=3, head_dim=64, split=(16, 24, 24), mode=mode, sparse_k=k,
                 tag=f"{mode}-{k}")


def test_packed_many_segments():
    # 21 segments over 64 rows: two launches of the segment table (16 + 5),
    # with short segments between them
    segs = []
    for i in range(21):
        segs.append((i % 3, (1 + i % 2, 5 + i % 4, 16)))
        if i % 7 == 3:
            segs.append((0, (1, 3, 4)))
    _packed_case(33, segs, heads=2, head_dim=64, split=(16, 24, 24), tag="many")


def test_packed_segments_equal_plain_calls_and_fused_k():
    segs = [(7, (3, 6, 8)), (0, (1, 5, 5)), (11, (5, 4, 6))]
    split = (32, 32, 32)
    (q, k, v), o, lse = _packed_case(32, segs, heads=3, head_dim=96, split=split, tag="vs-plain")
    start = 0
    for nt, g in segs:
        end = start + nt + int(np.prod(g))
        os_, ls_ = osp.osp_attn3d_fwd(q[:, start:end], k[:, start:end], v[:, start:end], grid=g,
                                      n_text=nt, rope_split=split, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(os_, o[:, start:end]) and torch.equal(ls_, lse[:, :, start:end])
        start = end
    # K rotated per segment by osp_rope3d, Q in the loader: same bits
    k_rot = torch.empty_like(k)
    start = 0
    for nt, g in segs:
        end = start + nt + int(np.prod(g))
        osp.osp_rope3d(k[:, start:end], grid=g, n_text=nt, rope_split=split,
                       out=k_rot[:, start:end])
        start = end
    o2, l2 = osp.osp_attn3d_packed_fwd(q, k_rot, v, segments=segs, rope_split=split,
                                       fuse_rope="q", return_lse=True)
    k_rot2 = osp.osp_rope3d_packed(k, segments=segs, rope_split=split)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(l2, lse)
    assert torch.equal(k_rot2, k_rot)


def test_cogvideox_frame_pack_sampled_rows():
    pk = workloads.COGVIDEOX_PACK
    wl = workloads.WORKLOADS[pk["base"]]
    segs = [(pk["n_text"], osp.osp_latent_grid(*clip, wl.c_t, wl.c_s, wl.p_t, wl.p_s))
            for clip in pk["clips"]]
    n = sum(nt + int(np.prod(g)) for nt, g in segs)
    shape = (1, n, wl.heads, wl.head_dim)
    note(f"cogvideox frame pack segments={segs} n={n}")
    cpu, (q, k, v) = qkv_for(pk["seed"], shape)
    # outputs start as NaN: every element must be written by the call
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, wl.heads, n), float("nan"), dtype=torch.float32, device=q.device)
    osp.osp_attn3d_packed_fwd(q, k, v, segments=segs, rope_split=wl.rope_split, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    rows = workloads.sample_rows(pk["seed"], n, pk["sample_rows"])
    hs = slice(0, 8)
    want_o, want_l = oracle.attn3d_packed(*(workloads.to_f64(t[:, :, hs]) for t in cpu),
                                          segments=segs, rope_split=wl.rope_split, rows=rows)
    assert_parity(to_np(o[:, rows][:, :, hs]), want_o, "O frame pack rows")
    got_l = to_np(lse[:, hs][:, :, rows])
    assert np.abs(got_l - want_l).max() <= LSE_ABS


# ------------------------------------------------------------------ backward
BWD_REL_L2 = 5e-3        # the backward's bars (tests/test_gpu_bwd.py derives them)
BWD_REL_L2_ROPE = 8e-3
BWD_MAX_REL = 2e-2


@pytest.mark.parametrize("mode,k,segs", [
    ("full", 1, [(7, (3, 6, 8)), (0, (1, 5, 5)), (11, (5, 4, 6))]),
    ("skiparse_single", 2, [(0, (2, 6, 8)), (0, (1, 4, 6)), (0, (3, 8, 10))]),
])
def test_packed_bwd_equals_plain_calls_and_oracle(mode, k, segs):
    """rope3d_packed -> packed forward -> packed backward -> rope3d_packed_inv:
    each segment's gradients equal a plain backward on its slice bit for bit
    (a packed backward runs the same launches per segment), and match the
    oracle's gradients with respect to q and k before the rotation."""
    split, heads, d = (32, 32, 32), 2, 96
    n = sum(nt + int(np.prod(g)) for nt, g in segs)
    shape = (2, n, heads, d)
    note(f"packed bwd mode={mode} k={k} segments={segs}")
    cpu, (q, k_, v) = qkv_for(40, shape)
    do_cpu = workloads.make_dout(40, shape)
    do = do_cpu.cuda()
    qr = osp.osp_rope3d_packed(q, segments=segs, rope_split=split)
    kr = osp.osp_rope3d_packed(k_, segments=segs, rope_split=split)
    o, lse = osp.osp_attn3d_packed_fwd(qr, kr, v, segments=segs, mode=mode, sparse_k=k,
                                       rope_split=split, fuse_rope=False, return_lse=True)
    dq, dk, dv = osp.osp_attn3d_packed_bwd(qr, kr, v, o, lse, do, segments=segs, mode=mode,
                                           sparse_k=k)
    start = 0
    for nt, g in segs:
        end = start + nt + int(np.prod(g))
        sl = slice(start, end)
        pq, pk, pv = osp.osp_attn3d_bwd(qr[:, sl], kr[:, sl], v[:, sl], o[:, sl],
                                        lse[:, :, sl].contiguous(), do[:, sl], grid=g,
                                        n_text=nt, mode=mode, sparse_k=k)
        torch.cuda.synchronize()
        assert torch.equal(pq, dq[:, sl]) and torch.equal(pk, dk[:, sl]) and torch.equal(pv, dv[:, sl])
        start = end
    gq = osp.osp_rope3d_packed_inv(dq, segments=segs, rope_split=split)
    gk = osp.osp_rope3d_packed_inv(dk, segments=segs, rope_split=split)
    torch.cuda.synchronize()
    start = 0
    for i, (nt, g) in enumerate(segs):
        end = start + nt + int(np.prod(g))
        want = oracle.attn3d_bwd(*(workloads.to_f64(t[:, start:end]) for t in (*cpu, do_cpu)),
                                 grid=g, n_text=nt, mode=mode, sparse_k=k, rope_split=split)
        for name, got, w in zip(("dq", "dk", "dv"), (gq, gk, dv), want):
            assert_parity(to_np(got[:, start:end]), w, f"{name} segment {i}",
                          BWD_MAX_REL * float(np.abs(w).max()),
                          BWD_REL_L2 if name == "dv" else BWD_REL_L2_ROPE)
        start = end


def test_packed_bwd_frame_pack_full_size():
    """The CogVideoX frame pack's backward at full size (the launches the
    benchmark times), through the RoPE chain: rope3d_packed of q and k,
    the packed forward, the packed backward into NaN-filled gradients
    (every element must be written), then rope3d_packed_inv of dq and dk.
    For head 0, every segment's dq, dk and dv are compared element by
    element with the oracle's gradients with respect to the unrotated
    inputs (the 17,776-token segment is one 17,776 x 17,776 fp64 problem).
    For head 1, per segment, the column identities of the gradients with
    respect to the rotated k and v: dK sums to 0 over a segment's keys and
    dV to the sum of dO over its queries."""
    pk = workloads.COGVIDEOX_PACK
    wl = workloads.WORKLOADS[pk["base"]]
    segs = [(pk["n_text"], osp.osp_latent_grid(*clip, wl.c_t, wl.c_s, wl.p_t, wl.p_s))
            for clip in pk["clips"]]
    n = sum(nt + int(np.prod(g)) for nt, g in segs)
    shape = (1, n, wl.heads, wl.head_dim)
    note(f"frame pack backward segments={segs} n={n}")
    cpu, (q, k, v) = qkv_for(pk["seed"], shape)
    do_cpu = workloads.make_dout(pk["seed"], shape)
    qr = osp.osp_rope3d_packed(q, segments=segs, rope_split=wl.rope_split)
    kr = osp.osp_rope3d_packed(k, segments=segs, rope_split=wl.rope_split)
    o, lse = osp.osp_attn3d_packed_fwd(qr, kr, v, segments=segs, rope_split=wl.rope_split,
                                       fuse_rope=False, return_lse=True)
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    osp.osp_attn3d_packed_bwd(qr, kr, v, o, lse, do_cpu.cuda(), segments=segs, dq=grads[0],
                              dk=grads[1], dv=grads[2])
    gq = osp.osp_rope3d_packed_inv(grads[0], segments=segs, rope_split=wl.rope_split)
    gk = osp.osp_rope3d_packed_inv(grads[1], segments=segs, rope_split=wl.rope_split)
    torch.cuda.synchronize()
    for name, g in zip(("dq", "dk", "dv"), grads):
        assert not torch.isnan(g).any(), f"{name} has unwritten elements"
    got0 = [to_np(t[:, :, 0:1]) for t in (gq, gk, grads[2])]
    got_k1, got_v1 = to_np(grads[1][:, :, 1]), to_np(grads[2][:, :, 1])
    dow1 = workloads.to_f64(do_cpu[:, :, 1])
    start = 0
    for s_i, (nt, g) in enumerate(segs):
        end = start + nt + int(np.prod(g))
        want = oracle.attn3d_bwd(*(workloads.to_f64(t[:, start:end, 0:1]) for t in (*cpu, do_cpu)),
                                 grid=g, n_text=nt, rope_split=wl.rope_split)
        for name, got, w in zip(("dq", "dk", "dv"), got0, want):
            assert_parity(got[:, start:end], w, f"{name} segment {s_i} h=0",
                          BWD_MAX_REL * float(np.abs(w).max()),
                          BWD_REL_L2 if name == "dv" else BWD_REL_L2_ROPE)
        gk1, gv1 = got_k1[0, start:end], got_v1[0, start:end]
        assert (np.abs(gk1.sum(axis=0)) <= 1e-2 * np.abs(gk1).sum(axis=0)).all()
        want_dv = dow1[0, start:end].sum(axis=0)
        assert (np.abs(gv1.sum(axis=0) - want_dv) <= 1e-2 * np.abs(gv1).sum(axis=0)).all()
        start = end

"""The scaled tolerance bars of the GPU parity tests, reproduced on the CPU.

Three bars in the GPU suite are wider than the unit bar (max-abs 2e-2,
rel-L2 5e-3, |dLSE| 1e-2):

* x4 for the sharpened inputs (Q multiplied by 4: logits 4 times larger),
  in tests/test_gpu_parity.py (multi-tile and short-subsequence cases);
* x2.4 for sm_scale = 0.3 at D = 64 (0.3 * sqrt(64) = 2.4 times the default
  logit scale), tests/test_gpu_parity.py::test_sm_scale_override;
* rel-L2 8e-3 for dq and dk through the RoPE chain (the rotated q and k are
  rounded to bf16 by their own pass, dq and dk once more after the
  transpose), tests/test_gpu_bwd.py and tests/test_gpu_packed.py.

The kernels round their operands to bf16, and that error is relative to
each value, so the logit error grows with the logits.  Here
``rounding_model`` replays those roundings in numpy on the exact inputs of
each GPU case (same seeds and shapes) and measures the error they leave
against the fp64 oracle.  Each test asserts that the case's bar covers the
modelled error.  Where a bar is widened, it also asserts that the unit bar
would NOT cover it, so the widening is needed.  A sweep over more seeds prints
the worst case for the record.
"""
import math

import numpy as np
import pytest

import oracle
import rounding_model as rm
import workloads

MAX_ABS, REL_L2, LSE_ABS = 2e-2, 5e-3, 1e-2          # tests/parity_util.py
BWD_REL, BWD_REL_ROPE, BWD_MAX_REL = 5e-3, 8e-3, 2e-2  # tests/test_gpu_bwd.py


def f64(t):
    return workloads.to_f64(t)


def fwd_errors(seed, shape, *, q_mult=None, scale=None, **kw):
    q, k, v = (f64(t) for t in workloads.make_qkv(seed, shape, scale, q_mult))
    o, lse = rm.attn_fwd(q, k, v, **kw)
    want_o, want_l = oracle.attn3d(q, k, v, **kw)
    return rm.errors(o, want_o) + (float(np.abs(lse - want_l).max()),)


def bwd_errors(seed, shape, *, rope_chain, **kw):
    q, k, v = (f64(t) for t in workloads.make_qkv(seed, shape))
    do = f64(workloads.make_dout(seed, shape))
    got = rm.attn_bwd(q, k, v, do, rope_chain=rope_chain, **kw)
    if not rope_chain:
        kw = dict(kw, rope_split=(shape[-1], 0, 0))
    want = oracle.attn3d_bwd(q, k, v, do, rope=rope_chain, **kw)
    out = {}
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        ma, rl = rm.errors(g, w)
        out[name] = (ma / float(np.abs(w).max()), rl)
    return out


def check_fwd(errs, tol, tag):
    ma, rl, le = errs
    print(f"{tag}: max_abs={ma:.3e} (bar {MAX_ABS * tol:.3e}) rel_l2={rl:.3e} "
          f"(bar {REL_L2 * tol:.3e}) lse={le:.3e} (bar {LSE_ABS * tol:.3e})")
    assert ma <= MAX_ABS * tol and rl <= REL_L2 * tol and le <= LSE_ABS * tol, tag


# ------------------------------------------------------------- the model
@pytest.mark.parametrize("mode,k", [("full", 1), ("skiparse_group", 4), ("block", 5)])
def test_model_without_rounding_is_the_oracle(mode, k):
    """With every rounding off and fp64 arithmetic the model computes the
    plain definition: forward and backward equal the oracle's."""
    shape, grid, split = (1, 320, 2, 64), (5, 8, 8), (16, 24, 24)
    q, k_, v = (f64(t) for t in workloads.make_qkv(0, shape))
    do = f64(workloads.make_dout(0, shape))
    kw = dict(grid=grid, mode=mode, sparse_k=k, rope_split=split)
    o, lse = rm.attn_fwd(q, k_, v, exact=True, **kw)
    want_o, want_l = oracle.attn3d(q, k_, v, **kw)
    assert np.abs(o - want_o).max() <= 1e-10 and np.abs(lse - want_l).max() <= 1e-10
    got = rm.attn_bwd(q, k_, v, do, rope_chain=True, exact=True, **kw)
    want = oracle.attn3d_bwd(q, k_, v, do, **kw)
    for g, w in zip(got, want):
        assert np.abs(g - w).max() <= 1e-10 * max(1.0, np.abs(w).max())


def test_bf16_rounding_is_round_to_nearest_even():
    # bf16 keeps 8 significant bits: the spacing above 1 is 2^-7, above 2 is 2^-6
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5 - 2 ** -7,
                  1.0 + 2 ** -8 + 2 ** -12], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 1.0 + 2 ** -7], dtype=np.float32)
    assert np.array_equal(rm.bf16(x), want)     # ties go to the even neighbour
    y = np.random.default_rng(3).standard_normal(10000).astype(np.float32)
    got = rm.bf16(y)
    assert not (got.view(np.uint32) & np.uint32(0xFFFF)).any()      # bf16 values
    assert np.all(np.abs(got.astype(np.float64) - y) <= 2.0 ** -8 * np.abs(y))   # half a step


# ------------------------------------------------------- forward bars (x4)
MT96 = dict(grid=(4, 12, 15), rope_split=(32, 32, 32))


@pytest.mark.parametrize("mode,k", [("full", 1), ("skiparse_single", 4), ("skiparse_group", 4),
                                    ("skiparse_group", 2), ("skiparse_group", 3), ("block", 3)])
def test_sharp_multitile_bar(mode, k):
    """test_multitile_d96[sharp-*]: seed 10, 720 tokens, 3 heads of 96, Q x 4."""
    errs = fwd_errors(10, (1, 720, 3, 96), q_mult=4.0, mode=mode, sparse_k=k, **MT96)
    check_fwd(errs, 4.0, f"sharp {mode} k={k}")
    assert errs[2] > LSE_ABS        # the unit bar would not hold: the x4 is needed
    # the unit-scale variants of the same case stay within the unit bar
    for variant, scale in (("unscaled", None), ("literal", 1 / math.sqrt(96))):
        check_fwd(fwd_errors(10, (1, 720, 3, 96), scale=scale, mode=mode, sparse_k=k, **MT96),
                  1.0, f"{variant} {mode} k={k}")


@pytest.mark.parametrize("grid,n_text,d,split,mode,k,batch", [
    ((24, 6, 5), 0, 96, (32, 32, 32), "skiparse_single", 30, 1),
    ((33, 2, 3), 0, 64, (16, 24, 24), "skiparse_single", 6, 2),
    ((8, 4, 4), 0, 128, (32, 48, 48), "skiparse_single", 2, 1),
    ((8, 4, 4), 0, 128, (32, 48, 48), "skiparse_group", 4, 1),
    ((5, 4, 8), 0, 96, (36, 36, 24), "block", 5, 2),
    ((5, 4, 8), 0, 64, (16, 24, 24), "skiparse_group", 4, 1),
    ((2, 3, 4), 7, 64, (16, 24, 24), "full", 1, 2),
    ((3, 4, 5), 2, 96, (32, 32, 32), "full", 1, 1),
])
def test_sharp_short_bar(grid, n_text, d, split, mode, k, batch):
    """test_short_subsequences' sharp half: seed 22, Q x 4."""
    n = n_text + int(np.prod(grid))
    errs = fwd_errors(22, (batch, n, 3, d), q_mult=4.0, grid=grid, n_text=n_text, mode=mode,
                      sparse_k=k, rope_split=split)
    check_fwd(errs, 4.0, f"short sharp {mode} k={k}")


# ---------------------------------------------------- forward bar (x2.4)
def test_sm_scale_bar():
    """test_sm_scale_override: seed 14, grid 2x9x10, 2 heads of 64, sm_scale 0.3."""
    tol = 0.3 * math.sqrt(64)
    errs = fwd_errors(14, (1, 180, 2, 64), grid=(2, 9, 10), rope_split=(16, 24, 24),
                      sm_scale=0.3)
    check_fwd(errs, tol, "sm_scale=0.3")
    assert errs[2] > LSE_ABS        # the unit bar would not hold


# ------------------------------------------------------- backward bars
def check_bwd(errs, rope, tag):
    for name, (mr, rl) in errs.items():
        bar = BWD_REL_ROPE if (rope and name != "dv") else BWD_REL
        print(f"{tag} {name}: max_abs/max={mr:.3e} (bar {BWD_MAX_REL:.1e}) rel_l2={rl:.3e} "
              f"(bar {bar:.1e})")
        assert mr <= BWD_MAX_REL and rl <= bar, (tag, name)


@pytest.mark.parametrize("d,split", [(64, (16, 24, 24)), (128, (32, 48, 48))])
def test_bwd_rope_chain_bar(d, split):
    """test_bwd_rope_chain: seed 3, grid 4x9x10, 2 heads."""
    errs = bwd_errors(3, (1, 360, 2, d), rope_chain=True, grid=(4, 9, 10), rope_split=split)
    check_bwd(errs, True, f"rope chain d={d}")


@pytest.mark.parametrize("mode,k,segs", [
    ("full", 1, [(7, (3, 6, 8)), (0, (1, 5, 5)), (11, (5, 4, 6))]),
    ("skiparse_single", 2, [(0, (2, 6, 8)), (0, (1, 4, 6)), (0, (3, 8, 10))]),
])
def test_packed_bwd_rope_chain_bar(mode, k, segs):
    """test_packed_bwd_equals_plain_calls_and_oracle: seed 40, batch 2, 2
    heads of 96; a packed backward is the plain backward of each segment."""
    n = sum(nt + int(np.prod(g)) for nt, g in segs)
    shape = (2, n, 2, 96)
    q, k_, v = (f64(t) for t in workloads.make_qkv(40, shape))
    do = f64(workloads.make_dout(40, shape))
    start = 0
    for i, (nt, g) in enumerate(segs):
        sl = slice(start, start + nt + int(np.prod(g)))
        kw = dict(grid=g, n_text=nt, mode=mode, sparse_k=k, rope_split=(32, 32, 32))
        got = rm.attn_bwd(q[:, sl], k_[:, sl], v[:, sl], do[:, sl], rope_chain=True, **kw)
        want = oracle.attn3d_bwd(q[:, sl], k_[:, sl], v[:, sl], do[:, sl], **kw)
        errs = {}
        for name, a, w in zip(("dq", "dk", "dv"), got, want):
            ma, rl = rm.errors(a, w)
            errs[name] = (ma / float(np.abs(w).max()), rl)
        check_bwd(errs, True, f"packed {mode} segment {i}")
        start = sl.stop


def test_bwd_text_tokens_batch_and_scale_bar():
    """test_bwd_text_tokens_batch_and_scale: seed 2, 37 text tokens and a
    3x10x12 grid, batch 2, 3 heads of 96, sm_scale 0.2 (about twice the
    default logit scale) under the unit bar."""
    errs = bwd_errors(2, (2, 397, 3, 96), rope_chain=False, grid=(3, 10, 12), n_text=37,
                      sm_scale=0.2)
    check_bwd(errs, False, "bwd text+batch+scale")


@pytest.mark.parametrize("d", [64, 96, 128])
def test_bwd_unit_bar(d):
    """test_bwd_full_ragged: seed 0, grid 5x7x9, 2 heads; q and k taken as
    rotated, so the unit bar applies to all three gradients."""
    errs = bwd_errors(0, (1, 315, 2, d), rope_chain=False, grid=(5, 7, 9))
    check_bwd(errs, False, f"bwd d={d}")


def test_seed_sweep_record():
    """More seeds of the three widened cases, printed for the record.  It
    asserts the rel-L2 and max-abs bars over the sweep, which have room.
    The sharp case's LSE bar (0.04) comes within a few percent of the worst
    seed, so the sweep asserts only its mean for that bar."""
    sharp_lse, rows = [], []
    for s in range(1, 11):
        e = fwd_errors((10, s), (1, 720, 3, 96), q_mult=4.0, mode="full", **MT96)
        sharp_lse.append(e[2])
        assert e[0] <= MAX_ABS * 4 and e[1] <= REL_L2 * 4
        e2 = fwd_errors((14, s), (1, 180, 2, 64), grid=(2, 9, 10), rope_split=(16, 24, 24),
                        sm_scale=0.3)
        tol = 0.3 * math.sqrt(64)
        assert e2[0] <= MAX_ABS * tol and e2[1] <= REL_L2 * tol and e2[2] <= LSE_ABS * tol
        b = bwd_errors((3, s), (1, 360, 2, 64), rope_chain=True, grid=(4, 9, 10),
                       rope_split=(16, 24, 24))
        check_bwd(b, True, f"sweep rope chain seed {s}")
        rows.append((s, e, e2))
    for s, e, e2 in rows:
        print(f"seed {s}: sharp {np.round(e, 4).tolist()}  sm_scale=0.3 {np.round(e2, 4).tolist()}")
    print(f"sharp LSE over the sweep: mean {np.mean(sharp_lse):.4f} max {np.max(sharp_lse):.4f}")
    assert np.mean(sharp_lse) <= LSE_ABS * 4

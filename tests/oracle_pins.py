"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself (closed forms, invariants, a library routine, brute force).

Each ``pin_*`` function takes an oracle module (the real one, or a mutated
copy in test_oracle_mutants.py) and raises AssertionError on a mismatch.
"""
from __future__ import annotations

import cmath
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(*key):
    return np.random.default_rng(list(key))


# --------------------------------------------------------------------------
# grid
# --------------------------------------------------------------------------
def pin_latent_grids(o):
    """Golden clip -> grid cases (closed form worked by hand, cited)."""
    with open(os.path.join(GOLDEN, "latent_grids.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        grid = o.latent_grid(*c["clip"], c["c_t"], c["c_s"], c["p_t"], c["p_s"])
        assert tuple(grid) == tuple(c["grid"]), (c, grid)
        assert int(np.prod(grid)) == c["tokens"]
    for c in g["rejected"]:
        try:
            o.latent_grid(*c["clip"], c["c_t"], c["c_s"])
        except ValueError:
            continue
        raise AssertionError(f"accepted {c}")


def pin_video_coords(o):
    """Row-major (t, h, w) unfold, w fastest, by nested loops."""
    grid = (3, 4, 5)
    expect = [(t, h, w) for t in range(3) for h in range(4) for w in range(5)]
    got = [tuple(int(v) for v in row) for row in o.video_coords(grid)]
    assert got == expect


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def pin_rope_closed_form(o):
    """Hand-worked values of RoFormer's rotation.

    Pair 0 of an axis chunk turns at omega_0 = 1 (theta^0); pair 1 of a
    4-channel chunk turns at theta^(-1/2) = 0.01 for theta = 1e4.  Rotation
    (x_a, x_b) -> (x_a cos - x_b sin, x_a sin + x_b cos).
    """
    # t-axis only: split (2,0,0), grid (3,1,1); token t=1 rotates by 1 rad.
    x = np.zeros((1, 3, 1, 2))
    x[0, 1, 0] = [1.0, 0.0]
    x[0, 2, 0] = [0.0, 1.0]
    y = o.rope3d(x, (3, 1, 1), 0, (2, 0, 0), 1e4)
    assert np.allclose(y[0, 1, 0], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    assert np.allclose(y[0, 2, 0], [-math.sin(2.0), math.cos(2.0)], atol=1e-15)
    # w-axis chunk of 4 channels: split (0,0,4), grid (1,1,4); token w=3.
    x = np.zeros((1, 4, 1, 4))
    x[0, 3, 0] = [0.0, 0.0, 2.0, -1.0]
    y = o.rope3d(x, (1, 1, 4), 0, (0, 0, 4), 1e4)
    a = 3 * 0.01
    want = [0.0, 0.0, 2 * math.cos(a) + math.sin(a), 2 * math.sin(a) - math.cos(a)]
    assert np.allclose(y[0, 3, 0], want, atol=1e-15)
    # theta changes the frequency of pair 1 only: theta=100 -> omega_1 = 0.1
    y = o.rope3d(x, (1, 1, 4), 0, (0, 0, 4), 100.0)
    a = 3 * 0.1
    want = [0.0, 0.0, 2 * math.cos(a) + math.sin(a), 2 * math.sin(a) - math.cos(a)]
    assert np.allclose(y[0, 3, 0], want, atol=1e-15)


def pin_rope_complex(o):
    """RoFormer's complex form: pair r of axis a is multiplied by
    exp(i * pos_a * theta^(-2r/d_a)).  Positions by explicit loops."""
    grid, split, n_text, theta = (2, 3, 4), (4, 6, 6), 2, 1e4
    d = sum(split)
    n = n_text + 24
    x = _rng(11).standard_normal((2, n, 3, d))
    y = o.rope3d(x, grid, n_text, split, theta, pos_offset=(1, 0, 2))
    want = x.copy()
    tok = n_text
    for t in range(grid[0]):
        for hh in range(grid[1]):
            for w in range(grid[2]):
                pos = (t + 1, hh, w + 2)
                c0 = 0
                for axis, d_a in enumerate(split):
                    for r in range(d_a // 2):
                        rot = cmath.exp(1j * pos[axis] * theta ** (-2.0 * r / d_a))
                        z = x[:, tok, :, c0 + 2 * r] + 1j * x[:, tok, :, c0 + 2 * r + 1]
                        z = z * rot
                        want[:, tok, :, c0 + 2 * r] = z.real
                        want[:, tok, :, c0 + 2 * r + 1] = z.imag
                    c0 += d_a
                tok += 1
    assert np.allclose(y, want, rtol=0, atol=1e-13)


def pin_rope_invariants(o):
    """Norm per pair kept; (0,0,0) is the identity; text rows unchanged;
    a shift of every position leaves all q.k scores unchanged; with q and
    k constant over tokens the score depends only on the position gap."""
    grid, split, n_text = (3, 4, 5), (16, 24, 24), 3
    n = n_text + 60
    x = _rng(12).standard_normal((1, n, 2, 64))
    y = o.rope3d(x, grid, n_text, split)
    pn = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2
    assert np.allclose(pn(y), pn(x), atol=1e-12)
    assert np.array_equal(y[:, :n_text], x[:, :n_text])
    assert np.allclose(y[:, n_text], x[:, n_text], atol=0)  # token (0,0,0)
    q = o.rope3d(x, grid, n_text, split)
    kx = _rng(13).standard_normal(x.shape)
    k = o.rope3d(kx, grid, n_text, split)
    s0 = np.einsum("bihd,bjhd->bhij", q, k)
    q2 = o.rope3d(x, grid, n_text, split, pos_offset=(5, -3, 7))
    k2 = o.rope3d(kx, grid, n_text, split, pos_offset=(5, -3, 7))
    s1 = np.einsum("bihd,bjhd->bhij", q2, k2)
    vv = (Ellipsis, slice(n_text, None), slice(n_text, None))   # video-video pairs
    assert np.allclose(s0[vv], s1[vv], rtol=0, atol=1e-11 * np.abs(s0).max())
    tt = (Ellipsis, slice(0, n_text), slice(0, n_text))         # text-text pairs
    assert np.array_equal(s0[tt], s1[tt])
    # constant vectors: score(i, j) = f(pos_i - pos_j)
    grid = (4, 4, 4)
    vq = _rng(14).standard_normal(64)
    vk = _rng(15).standard_normal(64)
    qc = o.rope3d(np.broadcast_to(vq, (1, 64, 1, 64)).copy(), grid, 0, split)
    kc = o.rope3d(np.broadcast_to(vk, (1, 64, 1, 64)).copy(), grid, 0, split)
    s = qc[0, :, 0] @ kc[0, :, 0].T
    coords = o.video_coords(grid)
    seen = {}
    for i in range(64):
        for j in range(64):
            key = tuple(coords[i] - coords[j])
            if key in seen:
                assert abs(seen[key] - s[i, j]) < 1e-12
            else:
                seen[key] = s[i, j]


def pin_rope_axis_chunks(o):
    """Moving a token along one axis changes only that axis's channels,
    in the order [t | h | w]."""
    grid, split = (2, 2, 2), (4, 6, 8)
    x = np.broadcast_to(_rng(16).standard_normal(18), (1, 8, 1, 18)).copy()
    y = o.rope3d(x, grid, 0, split)
    base = y[0, 0, 0]            # (0,0,0)
    chunks = {"t": slice(0, 4), "h": slice(4, 10), "w": slice(10, 18)}
    for tok, axis in ((4, "t"), (2, "h"), (1, "w")):   # (1,0,0) (0,1,0) (0,0,1)
        diff = np.abs(y[0, tok, 0] - base) > 1e-14
        for name, sl in chunks.items():
            assert diff[sl].any() == (name == axis), (tok, name)


# --------------------------------------------------------------------------
# Skiparse index maps
# --------------------------------------------------------------------------
def pin_skiparse_reshape(o):
    """The regrouping as a reshape: sequence to 1/k, batch times k
    (Open-Sora Plan 2.2.2).  Single: [N/k, k] transposed; group: blocks of
    k*k tokens, viewed [N/k^2, k(j), k] and moved j to the front."""
    for n, k in ((48, 4), (64, 4), (36, 3), (32, 2), (64, 8), (320, 4), (16, 1)):
        idx = np.arange(n)
        perm, inv = o.skiparse_index("skiparse_single", k, n)
        assert np.array_equal(perm, idx.reshape(n // k, k).T.reshape(-1))
        assert np.array_equal(inv[perm], idx)
        if n % (k * k) == 0:
            perm, inv = o.skiparse_index("skiparse_group", k, n)
            want = idx.reshape(n // (k * k), k, k).transpose(1, 0, 2).reshape(-1)
            assert np.array_equal(perm, want)
            assert np.array_equal(inv[perm], idx)
        perm, inv = o.skiparse_index("full", k, n)
        assert np.array_equal(perm, idx) and np.array_equal(inv, idx)


def pin_skiparse_structure(o):
    """k=1 is the identity; group skip with N = k^2 is contiguous windows;
    single then group connects every pair of tokens in two hops."""
    for mode in ("skiparse_single", "skiparse_group"):
        perm, _ = o.skiparse_index(mode, 1, 20)
        assert np.array_equal(perm, np.arange(20))
    g = o.skiparse_groups("skiparse_group", 4, 16)
    assert [list(x) for x in g] == [list(range(4 * j, 4 * j + 4)) for j in range(4)]
    n, k = 64, 4
    def adj(groups):
        a = np.zeros((n, n), dtype=np.int64)
        for grp in groups:
            a[np.ix_(grp, grp)] = 1
        return a
    two_hop = adj(o.skiparse_groups("skiparse_single", k, n)) @ adj(o.skiparse_groups("skiparse_group", k, n))
    assert (two_hop > 0).all()
    for mode, n in (("skiparse_single", 12), ("skiparse_group", 36)):
        for bad in (n + 1,):
            try:
                o.skiparse_groups(mode, 3 if mode == "skiparse_single" else 3, bad)
            except ValueError:
                continue
            raise AssertionError("accepted a length that does not divide")


def pin_skiparse2d_reshape(o):
    """Skiparse-2D as a reshape of the [T, H, W] token grid: single splits h
    and w into (h', jh) and (w', jw), the factor s last, and moves (jh, jw)
    to the front; group splits them into (a, jh, u) and (b, jw, v) -- s x s
    patches, s - 1 patches apart -- and moves (jh, jw) to the front."""
    for grid, k in (((2, 4, 6), 4), ((3, 6, 6), 9), ((2, 4, 8), 4), ((1, 2, 2), 4),
                    ((2, 3, 5), 1), ((1, 9, 9), 9)):
        t, h, w = grid
        n = t * h * w
        s = math.isqrt(k)
        want = np.arange(n).reshape(t, h // s, s, w // s, s).transpose(2, 4, 0, 1, 3).reshape(-1)
        perm, inv = o.skiparse_index("skiparse2d_single", k, n, grid)
        assert np.array_equal(perm, want), (grid, k)
        assert np.array_equal(inv[perm], np.arange(n))
        if h % (s * s) == 0 and w % (s * s) == 0:
            want = (np.arange(n).reshape(t, h // (s * s), s, s, w // (s * s), s, s)
                    .transpose(2, 5, 0, 1, 3, 4, 6).reshape(-1))
            perm, inv = o.skiparse_index("skiparse2d_group", k, n, grid)
            assert np.array_equal(perm, want), (grid, k)
            assert np.array_equal(inv[perm], np.arange(n))


def pin_skiparse2d_relations(o):
    """Skiparse-2D against the 1D rules: with W divisible by s, the union
    over jh of the 2D single subsequences (jh, jw) is 1D Single Skip
    subsequence jw at k = s; with H and W divisible by s*s, the same holds
    between 2D group and 1D Group Skip; s = H = W makes 2D single the
    temporal half of separated attention (Single Skip, k = H*W); k = 1 is
    full attention; shapes that do not divide, k not a square and a
    missing grid are rejected."""
    for grid, s in (((2, 4, 4), 2), ((3, 6, 9), 3), ((2, 8, 4), 2)):
        n, k = int(np.prod(grid)), s * s
        for m2, m1, step in (("skiparse2d_single", "skiparse_single", s),
                             ("skiparse2d_group", "skiparse_group", s * s)):
            if grid[1] % step or grid[2] % step:
                continue
            g2 = o.skiparse_groups(m2, k, n, grid)
            g1 = o.skiparse_groups(m1, s, n)
            assert len(g2) == k and all(len(g) == n // k for g in g2)
            for jw in range(s):
                union = sorted(np.concatenate([g2[jh * s + jw] for jh in range(s)]).tolist())
                assert union == g1[jw].tolist(), (m2, grid, jw)
    grid = (3, 2, 2)
    a = o.skiparse_groups("skiparse2d_single", 4, 12, grid)
    b = o.skiparse_groups("skiparse_single", 4, 12)
    assert [g.tolist() for g in a] == [g.tolist() for g in b]
    for mode in ("skiparse2d_single", "skiparse2d_group"):
        g = o.skiparse_groups(mode, 1, 24, (2, 3, 4))
        assert len(g) == 1 and g[0].tolist() == list(range(24))
    for mode, k, grid in (("skiparse2d_single", 4, (2, 3, 4)), ("skiparse2d_group", 4, (2, 4, 2)),
                          ("skiparse2d_group", 4, (1, 2, 4)), ("skiparse2d_single", 2, (2, 4, 4)),
                          ("skiparse2d_single", 4, None)):
        n = 32 if grid is None else int(np.prod(grid))
        try:
            o.skiparse_groups(mode, k, n, grid)
        except ValueError:
            continue
        raise AssertionError(f"accepted {mode} k={k} grid={grid}")


def pin_spatial_temporal(o):
    """Separated spatial / temporal attention (CogVideoX 2.2, Table 8) in
    terms of the latent coordinates: block attention with k = T groups the
    tokens of one frame, Single Skip with k = H*W the tokens of one (h, w)
    position across frames; block attention is the reshape [k, N/k]; k = N
    leaves every token alone."""
    for grid in ((3, 4, 5), (5, 8, 8), (2, 3, 3)):
        t, h, w = grid
        n = t * h * w
        c = o.video_coords(grid)
        for j, g in enumerate(o.skiparse_groups("block", t, n)):
            assert set(g.tolist()) == set(np.nonzero(c[:, 0] == j)[0].tolist())
        seen = set()
        for g in o.skiparse_groups("skiparse_single", h * w, n):
            hw = {(int(c[i, 1]), int(c[i, 2])) for i in g}
            assert len(hw) == 1 and len(g) == t
            seen |= hw
        assert len(seen) == h * w
        perm, inv = o.skiparse_index("block", t, n)
        assert np.array_equal(perm, np.arange(n)) and np.array_equal(inv, np.arange(n))
    for n, k in ((48, 4), (48, 48), (48, 1), (320, 5)):
        g = o.skiparse_groups("block", k, n)
        assert np.array_equal(np.stack(g), np.arange(n).reshape(k, n // k))
    try:
        o.skiparse_groups("block", 5, 48)
    except ValueError:
        pass
    else:
        raise AssertionError("accepted a length that does not divide")


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _sdpa64(q, k, v, scale, mask=None):
    """torch CPU float64 scaled_dot_product_attention on [B,N,H,D] arrays."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask),
        scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


def pin_attention_sdpa(o):
    """Full and Skiparse attention equal torch's float64 SDPA on the rotated
    inputs, with Skiparse given as a boolean block mask built from the
    reshape form of the regrouping."""
    grid, split = (4, 4, 4), (16, 24, 24)
    n = 64
    rng = _rng(21)
    q, k, v = (rng.standard_normal((2, n, 3, 64)) for _ in range(3))
    qr = o.rope3d(q, grid, 0, split)
    kr = o.rope3d(k, grid, 0, split)
    for mode, kk in (("full", 1), ("skiparse_single", 4), ("skiparse_group", 4),
                     ("skiparse_single", 2), ("skiparse_group", 2), ("skiparse_single", 8),
                     ("block", 4), ("block", 16), ("block", 1), ("skiparse2d_single", 4),
                     ("skiparse2d_group", 4)):
        idx = np.arange(n)
        if mode == "full":
            lab = np.zeros(n, dtype=np.int64)
        elif mode == "skiparse2d_single":
            # (t, h', jh, w', jw) with s = 2: the label is (jh, jw)
            lab = np.empty(n, dtype=np.int64)
            lab[idx.reshape(4, 2, 2, 2, 2)] = (2 * np.arange(2)[:, None] + np.arange(2)[None, :])[None, None, :, None, :]
        elif mode == "skiparse2d_group":
            # (t, jh, u, jw, v): 2 x 2 patches, label (jh, jw)
            lab = np.empty(n, dtype=np.int64)
            lab[idx.reshape(4, 2, 2, 2, 2)] = (2 * np.arange(2)[:, None] + np.arange(2)[None, :])[None, :, None, :, None]
        elif mode == "block":
            lab = np.repeat(np.arange(kk), n // kk)
        elif mode == "skiparse_single":
            lab = np.empty(n, dtype=np.int64)
            lab[idx.reshape(n // kk, kk).T] = np.arange(kk)[:, None]
        else:
            lab = np.empty(n, dtype=np.int64)
            lab[idx.reshape(n // (kk * kk), kk, kk).transpose(1, 0, 2)] = np.arange(kk)[:, None, None]
        mask = lab[:, None] == lab[None, :]
        want = _sdpa64(qr, kr, v, 0.125, mask)
        got, lse = o.attn3d(q, k, v, grid=grid, mode=mode, sparse_k=kk, rope_split=split)
        assert np.allclose(got, want, rtol=0, atol=1e-12), mode
        # lse by a library log-sum-exp over the same masked logits
        s = 0.125 * np.einsum("bihd,bjhd->bhij", qr, kr)
        s = np.where(mask[None, None], s, -np.inf)
        m = s.max(-1, keepdims=True)
        lse_want = (m + np.log(np.exp(s - m).sum(-1, keepdims=True)))[..., 0]
        assert np.allclose(lse, lse_want, rtol=0, atol=1e-12), mode


def pin_attention_bruteforce(o):
    """Tiny case with pure-Python floats and math.exp, no numpy matmul."""
    rng = _rng(22)
    n, d = 6, 4
    q, k, v = (rng.standard_normal((1, n, 1, d)) for _ in range(3))
    got, lse = o.attn3d(q, k, v, grid=(1, 2, 3), rope=False, rope_split=(0, 2, 2),
                        sm_scale=0.7)
    for i in range(n):
        logits = [0.7 * sum(q[0, i, 0, c] * k[0, j, 0, c] for c in range(d)) for j in range(n)]
        w = [math.exp(x) for x in logits]
        z = sum(w)
        for c in range(d):
            ref = sum(w[j] * v[0, j, 0, c] for j in range(n)) / z
            assert abs(got[0, i, 0, c] - ref) < 1e-13
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-13


def pin_attention_special(o):
    """Closed forms: rows of softmax (V = identity) are non-negative and sum
    to 1; V constant -> O constant; Q = 0 -> O = mean of V over the
    subsequence and LSE = ln|G|; one token per subsequence -> O = V;
    O is linear in V."""
    grid, split = (2, 4, 4), (16, 24, 24)
    n = 32
    rng = _rng(23)
    q, k = (rng.standard_normal((1, n, 2, 64)) for _ in range(2))
    eye = np.broadcast_to(np.eye(n)[None, :, None, :], (1, n, 2, n)).copy()
    # V = I needs D = N: rotate only the first 64 channels' worth -> use rope=False on prerotated
    qr = o.rope3d(q, grid, 0, split)
    kr = o.rope3d(k, grid, 0, split)
    qpad = np.zeros((1, n, 2, n)); qpad[..., :min(n, 64)] = qr[..., :min(n, 64)]
    kpad = np.zeros((1, n, 2, n)); kpad[..., :min(n, 64)] = kr[..., :min(n, 64)]
    pmat, _ = o.attn3d(qpad, kpad, eye, grid=grid, rope=False, rope_split=(0, 0, n),
                       sm_scale=0.3)
    assert (pmat >= 0).all()
    assert np.allclose(pmat.sum(-1), 1.0, atol=1e-13)
    v = rng.standard_normal((1, n, 2, 64))
    const = np.full_like(v, 1.75)
    out, _ = o.attn3d(q, k, const, grid=grid, rope_split=split)
    assert np.allclose(out, 1.75, atol=1e-13)
    for mode, kk in (("full", 1), ("skiparse_single", 4), ("skiparse_group", 2), ("block", 4),
                     ("skiparse2d_single", 4), ("skiparse2d_group", 4)):
        out, lse = o.attn3d(np.zeros_like(q), k, v, grid=grid, mode=mode, sparse_k=kk,
                            rope_split=split)
        for g in o.skiparse_groups(mode, kk, n, grid):
            assert np.allclose(out[:, g], v[:, g].mean(axis=1, keepdims=True), atol=1e-13)
            assert np.allclose(lse[:, :, g], math.log(len(g)), atol=1e-13)
    out, _ = o.attn3d(q, k, v, grid=grid, mode="skiparse_single", sparse_k=n, rope_split=split)
    assert np.allclose(out, v, atol=1e-13)
    a, _ = o.attn3d(q, k, v, grid=grid, rope_split=split)
    b, _ = o.attn3d(q, k, -2.5 * v, grid=grid, rope_split=split)
    assert np.allclose(b, -2.5 * a, atol=1e-12)


def pin_attention_text(o):
    """Joint attention with text in front equals full attention over
    [raw text | rotated video] (rotation applied by hand from the complex
    form), and text rows of Q and K are never rotated."""
    grid, split, n_text = (2, 2, 3), (4, 2, 2), 5
    n = n_text + 12
    rng = _rng(24)
    q, k, v = (rng.standard_normal((1, n, 2, 8)) for _ in range(3))
    got, _ = o.attn3d(q, k, v, grid=grid, n_text=n_text, rope_split=split, theta=50.0)
    def rot(x):
        y = x.copy()
        tok = n_text
        for t in range(2):
            for hh in range(2):
                for w in range(3):
                    pos = (t, hh, w)
                    c0 = 0
                    for axis, d_a in enumerate(split):
                        for r in range(d_a // 2):
                            z = complex(0, 0)
                            for head in range(2):
                                z = (x[0, tok, head, c0 + 2 * r] + 1j * x[0, tok, head, c0 + 2 * r + 1]) \
                                    * cmath.exp(1j * pos[axis] * 50.0 ** (-2.0 * r / d_a))
                                y[0, tok, head, c0 + 2 * r] = z.real
                                y[0, tok, head, c0 + 2 * r + 1] = z.imag
                        c0 += d_a
                    tok += 1
        return y
    want = _sdpa64(rot(q), rot(k), v, 1.0 / math.sqrt(8))
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def pin_rows_subset(o):
    """Computing a subset of query rows gives the same values as the full
    call at those rows (any mode), up to BLAS blocking order."""
    grid, split = (2, 4, 4), (16, 24, 24)
    rng = _rng(25)
    q, k, v = (rng.standard_normal((1, 32, 2, 64)) for _ in range(3))
    rows = np.array([0, 3, 5, 17, 31])
    for mode, kk in (("full", 1), ("skiparse_single", 4), ("skiparse_group", 2), ("block", 2)):
        a, la = o.attn3d(q, k, v, grid=grid, mode=mode, sparse_k=kk, rope_split=split)
        b, lb = o.attn3d(q, k, v, grid=grid, mode=mode, sparse_k=kk, rope_split=split, rows=rows)
        assert np.allclose(a[:, rows], b, rtol=0, atol=1e-14)
        assert np.allclose(la[:, :, rows], lb, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def pin_rope_transpose(o):
    """rope3d_transpose is the adjoint of rope3d: <R x, y> = <x, R^T y>, and
    R^T R = I (text rows, offsets and an uneven split included)."""
    rng = _rng(31)
    for grid, n_text, split, off in (((2, 3, 4), 0, (16, 24, 24), (0, 0, 0)),
                                     ((3, 2, 5), 4, (4, 6, 54), (2, -1, 7))):
        n = n_text + int(np.prod(grid))
        x, y = (rng.standard_normal((2, n, 3, 64)) for _ in range(2))
        lhs = (o.rope3d(x, grid, n_text, split, 1e4, off) * y).sum()
        rhs = (x * o.rope3d_transpose(y, grid, n_text, split, 1e4, off)).sum()
        assert abs(lhs - rhs) <= 1e-10 * abs(lhs)
        back = o.rope3d_transpose(o.rope3d(x, grid, n_text, split, 1e4, off), grid, n_text, split,
                                  1e4, off)
        assert np.allclose(back, x, rtol=0, atol=1e-13)


def pin_bwd_autograd(o):
    """Gradients equal torch float64 autograd through scaled_dot_product_attention
    on the rotated inputs, with the subsequences as a boolean mask."""
    grid, split = (4, 4, 4), (16, 24, 24)
    n = 64
    rng = _rng(32)
    q, k, v, do = (rng.standard_normal((2, n, 3, 64)) for _ in range(4))
    qr = o.rope3d(q, grid, 0, split)
    kr = o.rope3d(k, grid, 0, split)
    for mode, kk in (("full", 1), ("skiparse_single", 4), ("skiparse_group", 2), ("block", 4),
                     ("skiparse2d_single", 4), ("skiparse2d_group", 4)):
        lab = np.zeros(n, dtype=np.int64)
        for j, g in enumerate(o.skiparse_groups(mode, kk, n, grid)):
            lab[g] = j
        mask = torch.from_numpy(lab[:, None] == lab[None, :])
        tq, tk, tv = (torch.from_numpy(a).permute(0, 2, 1, 3).clone().requires_grad_(True)
                      for a in (qr, kr, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                               scale=0.125)
        out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
        want = [t.grad.permute(0, 2, 1, 3).numpy() for t in (tq, tk, tv)]
        got = o.attn3d_bwd(qr, kr, v, do, grid=grid, mode=mode, sparse_k=kk, rope_split=split,
                           rope=False)
        for g_, w_, name in zip(got, want, "qkv"):
            assert np.allclose(g_, w_, rtol=0, atol=1e-12), (mode, name)


def pin_bwd_finite_differences(o):
    """Central differences of the forward oracle, through 3D RoPE, text tokens
    and the subsequence modes, match the backward oracle."""
    rng = _rng(33)
    cases = (((2, 2, 3), 0, "full", 1), ((1, 2, 3), 2, "full", 1),
             ((2, 2, 3), 0, "skiparse_single", 2), ((2, 2, 3), 0, "block", 3),
             ((2, 2, 4), 0, "skiparse_group", 2), ((2, 2, 4), 0, "skiparse2d_single", 4),
             ((1, 4, 4), 0, "skiparse2d_group", 4))
    split, eps = (2, 2, 4), 1e-6
    for grid, n_text, mode, kk in cases:
        n = n_text + int(np.prod(grid))
        q, k, v, w = (rng.standard_normal((1, n, 1, 8)) for _ in range(4))
        kw = dict(grid=grid, n_text=n_text, mode=mode, sparse_k=kk, rope_split=split,
                  pos_offset=(1, 2, 3))
        loss = lambda a, b, c: float((o.attn3d(a, b, c, **kw)[0] * w).sum())
        grads = o.attn3d_bwd(q, k, v, w, **kw)
        for which, g in enumerate(grads):
            num = np.zeros_like(g)
            for idx in np.ndindex(*g.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += eps
                up = loss(*args)
                args[which][idx] -= 2 * eps
                num[idx] = (up - loss(*args)) / (2 * eps)
            assert np.allclose(g, num, rtol=0, atol=1e-7), (mode, "qkv"[which])


def pin_packed_block_diagonal(o):
    """A packed sequence equals torch float64 SDPA over the whole sequence
    with a block-diagonal mask, each segment rotated on its own grid from
    position 0; a single segment equals attn3d; reversing the segments
    reverses the output blocks."""
    split = (16, 24, 24)
    segs = [(3, (2, 3, 4)), (0, (1, 4, 5)), (5, (3, 2, 2)), (0, (2, 2, 2))]
    lay = o.packed_segments(segs)
    n = lay[-1][1]
    rng = _rng(34)
    q, k, v = (rng.standard_normal((2, n, 2, 64)) for _ in range(3))
    qr, kr = np.empty_like(q), np.empty_like(k)
    lab = np.zeros(n, dtype=np.int64)
    for idx, (s0, s1, nt, grid) in enumerate(lay):
        qr[:, s0:s1] = o.rope3d(q[:, s0:s1], grid, nt, split)
        kr[:, s0:s1] = o.rope3d(k[:, s0:s1], grid, nt, split)
        lab[s0:s1] = idx
    mask = lab[:, None] == lab[None, :]
    want = _sdpa64(qr, kr, v, 0.125, mask)
    got, lse = o.attn3d_packed(q, k, v, segments=segs, rope_split=split)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    assert np.isfinite(lse).all()
    one, lone = o.attn3d(q[:, :lay[0][1]], k[:, :lay[0][1]], v[:, :lay[0][1]], grid=(2, 3, 4),
                         n_text=3, rope_split=split)
    g1, l1 = o.attn3d_packed(q[:, :lay[0][1]], k[:, :lay[0][1]], v[:, :lay[0][1]],
                             segments=segs[:1], rope_split=split)
    assert np.array_equal(one, g1) and np.array_equal(lone, l1)
    rev = segs[::-1]
    rlay = o.packed_segments(rev)
    perm = np.concatenate([np.arange(s0, s1) for s0, s1, _, _ in lay[::-1]])
    gr, _ = o.attn3d_packed(q[:, perm], k[:, perm], v[:, perm], segments=rev, rope_split=split)
    assert np.allclose(gr, got[:, perm], rtol=0, atol=1e-12)
    assert rlay[0][1] == lay[-1][1] - lay[-1][0]
    rows = np.array([0, 2, 10, 23, 24, 40, n - 1])
    gs, ls = o.attn3d_packed(q, k, v, segments=segs, rope_split=split, rows=rows)
    assert np.allclose(gs, got[:, rows], rtol=0, atol=1e-12)
    assert np.allclose(ls, lse[:, :, rows], rtol=0, atol=1e-12)


ALL_PINS = [
    pin_latent_grids, pin_video_coords, pin_rope_closed_form, pin_rope_complex,
    pin_rope_invariants, pin_rope_axis_chunks, pin_skiparse_reshape,
    pin_skiparse_structure, pin_skiparse2d_reshape, pin_skiparse2d_relations,
    pin_spatial_temporal, pin_attention_sdpa, pin_attention_bruteforce,
    pin_attention_special, pin_attention_text, pin_rows_subset,
    pin_rope_transpose, pin_bwd_autograd, pin_bwd_finite_differences,
    pin_packed_block_diagonal,
]

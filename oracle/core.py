"""Plain fp64 CPU oracle for 3D-RoPE full and Skiparse attention (forward).

TEST INFRASTRUCTURE ONLY.  This module is the independent definition that the
HIP library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and this
module shares no code, table or helper with the library.

Every step is the plain definition, written out in float64 with numpy:
no tiling, no online softmax, no fused loaders.  Each function names the
passage it follows.  Sources (web pages):

* "Open-Sora Plan: Open-Source Large Video Generation Model" (paper summary
  page), sections 2.2.1 "Model Overview" and 2.2.2 "Skiparse Attention".
* "CogVideoX: Text-to-Video Diffusion Models with an Expert Transformer",
  section 2 (architecture overview), section 2.2 paragraphs "Patchify",
  "3D-RoPE" and "3D Full Attention", section 3.1 and Appendix A (position
  extrapolation), reference [14] (RoFormer).
* "Open Video Models" (book chapter), section "The Mathematics" (latent size
  of a causal video VAE).

Readings taken where the pages are silent (all listed with reasons in the
design notes):

1. the latent grid is unfolded row-major over (t, h, w), w fastest;
2. the head dimension is split into channel chunks [t | h | w];
3. rotation pairs are adjacent channels (2r, 2r+1), as in RoFormer;
4. within an axis chunk of size d_a, pair r turns at omega_r = theta^(-2r/d_a);
5. positions are the integer latent indices (plus optional offsets), used
   unscaled (extrapolation, not interpolation);
6. text tokens sit in front of the video tokens and are not rotated;
7. the softmax scale defaults to 1/sqrt(D);
8. Single Skip subsequence j = tokens whose index is j mod k;
9. Group Skip subsequence j = tokens whose group index floor(i/k) is j mod k
   (groups of k adjacent tokens);
10. subsequences keep increasing token order and are listed by j;
11. every token keeps its own (t, h, w) under Skiparse (RoPE acts per token
    before the regrouping);
12. block attention (the spatial half of separated spatial / temporal
    attention, and window attention) attends within k runs of N/k adjacent
    tokens; with the row-major unfold, k = T gives each frame's H*W tokens,
    and the temporal half (same (h, w) across frames) is Single Skip with
    k = H*W;
13. a packed sequence (several videos in one sequence) attends block
    diagonally, each video within itself, with RoPE positions from 0 on its
    own grid;
14. Skiparse-2D applies the two Skiparse rules along the latent's h and w
    axes, with factor s = sqrt(k) on each, in every frame: subsequence
    j = jh*s + jw holds the tokens with h = jh, w = jw (mod s) (single), or
    those of the s x s patches whose patch row and column are jh, jw
    (mod s) (group).

Parity status: grid arithmetic, rotation and attention are pinned by closed
forms, invariants, a library routine and brute force (tests/test_oracle_*.py).
The readings that no page value can fix -- the RoPE channel order/pairing
(readings 2-3), the Group Skip group size (reading 9) and the Skiparse-2D
rule (reading 14) -- are "parity unpinned" against any outside
implementation: the pages print no example.
"""
from __future__ import annotations

import math

import numpy as np

MODES = ("full", "skiparse_single", "skiparse_group", "block", "skiparse2d_single",
         "skiparse2d_group")


# --------------------------------------------------------------------------
# Latent grid (row a1)
# --------------------------------------------------------------------------
def latent_grid(frames: int, height: int, width: int, c_t: int, c_s: int,
                p_t: int = 1, p_s: int = 2) -> tuple:
    """Latent token grid of a clip.

    "Open Video Models", "The Mathematics": a causal video VAE maps T frames
    of H x W to T' = (T-1)/c_t + 1, H' = H/c_s, W' = W/c_s.  CogVideoX
    section 2.2 "Patchify": patchify by q in time and p in space gives a
    sequence of (T/q)(H/p)(W/p) tokens; Open-Sora Plan section 2.2.1 uses a
    1x2x2 kernel with matching stride.  Non-integral sizes are rejected.
    """
    if (frames - 1) % c_t or height % c_s or width % c_s:
        raise ValueError("clip size not divisible by the VAE compression")
    t_lat = (frames - 1) // c_t + 1
    h_lat = height // c_s
    w_lat = width // c_s
    if t_lat % p_t or h_lat % p_s or w_lat % p_s:
        raise ValueError("latent size not divisible by the patch size")
    return (t_lat // p_t, h_lat // p_s, w_lat // p_s)


def video_coords(grid) -> np.ndarray:
    """(t, h, w) of every video token, in sequence order: shape [T*H*W, 3].

    CogVideoX section 2: the patchified latent is unfolded into one long
    sequence.  Reading 1: row-major unfold, w fastest.
    """
    t, h, w = grid
    return np.indices((t, h, w)).reshape(3, -1).T.astype(np.int64)


# --------------------------------------------------------------------------
# 3D RoPE (row a2)
# --------------------------------------------------------------------------
def rope3d(x: np.ndarray, grid, n_text: int, rope_split, theta: float = 1e4,
           pos_offset=(0, 0, 0)) -> np.ndarray:
    """Rotate channel pairs of x ([B, N, H, D], float64) by 3D RoPE.

    CogVideoX section 2.2 "3D-RoPE": each latent has a 3D coordinate and 1D
    RoPE is applied independently per coordinate on its own share of the
    channels; the three encodings are concatenated along the channel axis.
    RoFormer (reference [14]): a channel pair (x_a, x_b) at position m is
    rotated by the angle m * omega_r, giving (x_a cos - x_b sin,
    x_a sin + x_b cos).  Text tokens (the first ``n_text`` rows, CogVideoX
    section 2) are returned unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if sum(rope_split) != d or any(s % 2 for s in rope_split):
        raise ValueError("rope split must be even chunks summing to head_dim")
    n_video = int(np.prod(grid))
    if x.shape[1] != n_text + n_video:
        raise ValueError("sequence length does not match the grid")
    coords = video_coords(grid) + np.asarray(pos_offset, dtype=np.int64)[None, :]
    out = x.copy()
    c0 = 0
    for axis, d_a in enumerate(rope_split):
        if d_a == 0:
            continue
        r = np.arange(d_a // 2, dtype=np.float64)
        omega = theta ** (-2.0 * r / d_a)                       # [d_a/2]
        phi = coords[:, axis].astype(np.float64)[:, None] * omega[None, :]
        cos = np.cos(phi)[None, :, None, :]                      # [1, Nv, 1, d_a/2]
        sin = np.sin(phi)[None, :, None, :]
        xa = x[:, n_text:, :, c0 + 0:c0 + d_a:2]
        xb = x[:, n_text:, :, c0 + 1:c0 + d_a:2]
        out[:, n_text:, :, c0 + 0:c0 + d_a:2] = xa * cos - xb * sin
        out[:, n_text:, :, c0 + 1:c0 + d_a:2] = xa * sin + xb * cos
        c0 += d_a
    return out


# --------------------------------------------------------------------------
# Skiparse regrouping (row a3)
# --------------------------------------------------------------------------
def skiparse_groups(mode: str, k: int, n: int, grid=None) -> list:
    """Token indices of each subsequence, by membership predicate.

    Open-Sora Plan section 2.2.2: a Skiparse step cuts the attended sequence
    to 1/k of its length and multiplies the batch by k.  Single Skip takes
    every k-th token (reading 8); Group Skip gathers groups of adjacent
    tokens whose groups lie k-1 groups apart (reading 9, group size k).  The
    section assumes the length divides evenly; we require it.

    "block": k runs of N/k adjacent tokens (reading 12).  This is the
    spatial half of the separated spatial / temporal attention that
    CogVideoX section 2.2 "3D Full Attention" and Table 8 compare with 3D
    attention (k = frames: each frame's H*W tokens), and the window
    attention that Open-Sora Plan section 2.2.2 contrasts with Group Skip
    (k = N / window).  The temporal half (tokens with the same (h, w)) is
    Single Skip with k = H*W.

    "skiparse2d_single" / "skiparse2d_group" need ``grid`` (reading 14).
    The Open-Sora Plan blog page lists Skiparse-2D for OSP-Next as a fixed
    sparse rule along H and W that stays FlashAttention-compatible, and
    gives no more.  Here k = s*s: the single rule keeps the tokens whose h
    and w are jh and jw modulo s; the group rule cuts each frame into s x s
    patches and keeps the patches whose patch row and patch column are jh
    and jw modulo s.  Every frame takes part, so each subsequence holds N/k
    tokens.  Single needs H and W divisible by s, group by s*s.
    """
    idx = np.arange(n, dtype=np.int64)
    if mode == "full":
        return [idx]
    if k < 1:
        raise ValueError("sparse ratio must be >= 1")
    if mode == "skiparse_single":
        if n % k:
            raise ValueError("single skip needs N divisible by k")
        key = idx % k
    elif mode == "skiparse_group":
        if n % (k * k):
            raise ValueError("group skip needs N divisible by k*k")
        key = (idx // k) % k
    elif mode == "block":
        if n % k:
            raise ValueError("block attention needs N divisible by k")
        key = idx // (n // k)
    elif mode in ("skiparse2d_single", "skiparse2d_group"):
        if grid is None or int(np.prod(grid)) != n:
            raise ValueError("Skiparse-2D needs the latent grid of the N tokens")
        s = math.isqrt(k)
        if s * s != k:
            raise ValueError("Skiparse-2D needs k = s*s")
        step = s if mode == "skiparse2d_single" else s * s
        if grid[1] % step or grid[2] % step:
            raise ValueError(f"Skiparse-2D needs H and W divisible by {step}")
        c = video_coords(grid)
        hh, ww = c[:, 1], c[:, 2]
        if mode == "skiparse2d_group":
            hh, ww = hh // s, ww // s
        key = (hh % s) * s + (ww % s)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return [np.nonzero(key == j)[0] for j in range(k)]


def skiparse_index(mode: str, k: int, n: int, grid=None):
    """perm[r'] = token at regrouped position r' (subsequences by j, each in
    increasing token order; reading 10); inv is its inverse permutation."""
    perm = np.concatenate(skiparse_groups(mode, k, n, grid)).astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(n, dtype=np.int64)
    return perm.astype(np.int32), inv.astype(np.int32)


def rope3d_transpose(x: np.ndarray, grid, n_text: int, rope_split, theta: float = 1e4,
                     pos_offset=(0, 0, 0)) -> np.ndarray:
    """R^T x for the rotation R of ``rope3d``: every video pair turned by the
    negative angle (x_a cos + x_b sin, -x_a sin + x_b cos).

    The chain rule through y = R x gives dL/dx = R^T dL/dy, and R is a
    product of plane rotations, so R^T turns each pair back.  Text rows are
    unchanged, as in the forward rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    if sum(rope_split) != x.shape[-1] or any(s % 2 for s in rope_split):
        raise ValueError("rope split must be even chunks summing to head_dim")
    n_video = int(np.prod(grid))
    if x.shape[1] != n_text + n_video:
        raise ValueError("sequence length does not match the grid")
    coords = video_coords(grid) + np.asarray(pos_offset, dtype=np.int64)[None, :]
    out = x.copy()
    c0 = 0
    for axis, d_a in enumerate(rope_split):
        if d_a == 0:
            continue
        r = np.arange(d_a // 2, dtype=np.float64)
        omega = theta ** (-2.0 * r / d_a)
        phi = coords[:, axis].astype(np.float64)[:, None] * omega[None, :]
        cos = np.cos(phi)[None, :, None, :]
        sin = np.sin(phi)[None, :, None, :]
        xa = x[:, n_text:, :, c0 + 0:c0 + d_a:2]
        xb = x[:, n_text:, :, c0 + 1:c0 + d_a:2]
        out[:, n_text:, :, c0 + 0:c0 + d_a:2] = xa * cos + xb * sin
        out[:, n_text:, :, c0 + 1:c0 + d_a:2] = -xa * sin + xb * cos
        c0 += d_a
    return out


# --------------------------------------------------------------------------
# Attention (rows a4-a7)
# --------------------------------------------------------------------------
def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      sm_scale: float):
    """softmax(sm_scale * q k^T) v for one sequence, plus log-sum-exp.

    CogVideoX section 2.2 "3D Full Attention": every token attends to every
    other token of the (text + video) sequence; FlashAttention computes this
    exactly.  q: [M, D], k, v: [L, D].  Returns o [M, D], lse [M] (natural
    log of the softmax denominator of the scaled logits).
    """
    s = sm_scale * (q @ k.T)                  # [M, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def attn3d(q, k, v, *, grid, n_text: int = 0, mode: str = "full",
           sparse_k: int = 1, rope_split, theta: float = 1e4,
           sm_scale: float | None = None, pos_offset=(0, 0, 0),
           rope: bool = True, rows=None, block: int = 2048):
    """3D-RoPE attention over [B, N, H, D] float64 inputs.

    Steps, in the pages' order: rotate Q and K by 3D RoPE (Open-Sora Plan
    2.2.1, CogVideoX 2.2 "3D-RoPE"); split the sequence into subsequences
    (one for full attention, k for Skiparse, Open-Sora Plan 2.2.2); attend
    within each subsequence (CogVideoX 2.2 "3D Full Attention"); write each
    output row back at its token's original position.

    ``rows``: optional sorted token indices; then only those query rows are
    computed and o has shape [B, len(rows), H, D], lse [B, H, len(rows)].
    ``rope=False`` takes q and k as already rotated.
    Skiparse and block attention with text tokens are rejected (reading:
    Open-Sora Plan feeds text through cross-attention, so its Skiparse
    self-attention has none; the pages do not say how text joins separated
    spatial or temporal attention).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_sz, n, h_sz, d = q.shape
    if n != n_text + int(np.prod(grid)):
        raise ValueError("sequence length does not match the grid")
    if mode != "full" and n_text:
        raise ValueError("Skiparse and block attention take no text tokens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if rope:
        q = rope3d(q, grid, n_text, rope_split, theta, pos_offset)
        k = rope3d(k, grid, n_text, rope_split, theta, pos_offset)
    groups = skiparse_groups(mode, sparse_k, n, grid)
    if rows is None:
        out_rows = np.arange(n, dtype=np.int64)
    else:
        out_rows = np.asarray(rows, dtype=np.int64)
    where = {int(t): i for i, t in enumerate(out_rows)}
    o = np.full((b_sz, len(out_rows), h_sz, d), np.nan)
    lse = np.full((b_sz, h_sz, len(out_rows)), np.nan)
    for g in groups:
        wanted = g[np.isin(g, out_rows)]
        if wanted.size == 0:
            continue
        dst = np.array([where[int(t)] for t in wanted], dtype=np.int64)
        for b in range(b_sz):
            for h in range(h_sz):
                kk = k[b, g, h, :]
                vv = v[b, g, h, :]
                for s0 in range(0, wanted.size, block):
                    sel = wanted[s0:s0 + block]
                    ob, lb = softmax_attention(q[b, sel, h, :], kk, vv, sm_scale)
                    o[b, dst[s0:s0 + block], h, :] = ob
                    lse[b, h, dst[s0:s0 + block]] = lb
    return o, lse


# --------------------------------------------------------------------------
# Packed sequences (several videos in one sequence)
# --------------------------------------------------------------------------
def packed_segments(segments):
    """(start, end, n_text, grid) of each segment of a packed sequence, in
    order; ``segments`` is a list of (n_text, (T, H, W))."""
    out, start = [], 0
    for n_text, grid in segments:
        end = start + int(n_text) + int(np.prod(grid))
        out.append((start, end, int(n_text), tuple(int(x) for x in grid)))
        start = end
    return out


def attn3d_packed(q, k, v, *, segments, mode: str = "full", sparse_k: int = 1,
                  rope_split, theta: float = 1e4, sm_scale: float | None = None,
                  pos_offset=(0, 0, 0), rope: bool = True, rows=None):
    """Attention over a packed sequence: several videos of different
    durations and resolutions, each with its own text tokens in front, one
    after the other in one sequence (CogVideoX section 3.1 "Multi-Resolution
    Frame Pack", after Patch'n Pack, its reference [21]).

    Reading: every video attends only to its own tokens (the packed
    sequence's attention is block diagonal: packing exists to batch unequal
    shapes, not to let videos see each other), and its 3D RoPE positions
    start from 0 on its own grid (section 3.1 keeps RoPE by extrapolation,
    each video taking the front of the position table).  Each segment is
    then exactly ``attn3d`` on its slice.  Returns o [B, N, H, D] and lse
    [B, H, N] over the packed N; with ``rows`` (sorted packed token
    indices) only those query rows, as o [B, len(rows), H, D] and lse
    [B, H, len(rows)].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_sz, n, h_sz, d = q.shape
    segs = packed_segments(segments)
    if not segs or segs[-1][1] != n:
        raise ValueError("segments do not cover the sequence")
    out_rows = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.full((b_sz, len(out_rows), h_sz, d), np.nan)
    lse = np.full((b_sz, h_sz, len(out_rows)), np.nan)
    for start, end, n_text, grid in segs:
        sel = np.nonzero((out_rows >= start) & (out_rows < end))[0]
        if sel.size == 0:
            continue
        os_, ls_ = attn3d(q[:, start:end], k[:, start:end], v[:, start:end], grid=grid,
                          n_text=n_text, mode=mode, sparse_k=sparse_k, rope_split=rope_split,
                          theta=theta, sm_scale=sm_scale, pos_offset=pos_offset, rope=rope,
                          rows=out_rows[sel] - start)
        o[:, sel] = os_
        lse[:, :, sel] = ls_
    return o, lse


# --------------------------------------------------------------------------
# Backward (the training pass of the same layer)
# --------------------------------------------------------------------------
def softmax_attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                          sm_scale: float):
    """Gradients of o = softmax(sm_scale * q k^T) v for one sequence.

    With p the softmax rows and o = p v: dv = p^T do; dp = do v^T; the
    softmax Jacobian gives ds = p * (dp - sum_j p_ij dp_ij) row by row;
    s = sm_scale * q k^T then gives dq = sm_scale * ds k and
    dk = sm_scale * ds^T q.  q: [M, D], k, v: [L, D], do: [M, D].
    """
    s = sm_scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = sm_scale * (ds @ k)
    dk = sm_scale * (ds.T @ q)
    return dq, dk, dv


def attn3d_bwd(q, k, v, do, *, grid, n_text: int = 0, mode: str = "full",
               sparse_k: int = 1, rope_split, theta: float = 1e4,
               sm_scale: float | None = None, pos_offset=(0, 0, 0), rope: bool = True):
    """Gradients of ``attn3d``'s output o with respect to q, k and v, given
    the output gradient do ([B, N, H, D]).

    The forward steps in reverse: each subsequence's attention is
    differentiated on its own (``softmax_attention_bwd``), the gradients are
    written back at the tokens' positions, and with ``rope`` the q and k
    gradients pass back through the rotation (``rope3d_transpose``).  With
    ``rope=False`` q and k are the rotated inputs and their gradients are
    with respect to those.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    b_sz, n, h_sz, d = q.shape
    if n != n_text + int(np.prod(grid)):
        raise ValueError("sequence length does not match the grid")
    if mode != "full" and n_text:
        raise ValueError("Skiparse and block attention take no text tokens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if rope:
        q = rope3d(q, grid, n_text, rope_split, theta, pos_offset)
        k = rope3d(k, grid, n_text, rope_split, theta, pos_offset)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for g in skiparse_groups(mode, sparse_k, n, grid):
        for b in range(b_sz):
            for h in range(h_sz):
                gq, gk, gv = softmax_attention_bwd(q[b, g, h, :], k[b, g, h, :], v[b, g, h, :],
                                                   do[b, g, h, :], sm_scale)
                dq[b, g, h, :] = gq
                dk[b, g, h, :] = gk
                dv[b, g, h, :] = gv
    if rope:
        dq = rope3d_transpose(dq, grid, n_text, rope_split, theta, pos_offset)
        dk = rope3d_transpose(dk, grid, n_text, rope_split, theta, pos_offset)
    return dq, dk, dv

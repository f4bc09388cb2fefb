"""Python binding of libosp: 3D-RoPE full / Skiparse attention on MI355X.

Argument marshalling only: every step runs in the HIP library
(``libosp.so``, built by ``python -m spatiotemporal_attention_amd.build``).
The functions carry the names of the C entry points in include/osp.h.
Tensors are torch bfloat16 [B, N, H, D] with unit channel stride; device
work goes on torch's current stream of the tensor's device.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libosp.so")

MODES = {"full": 0, "skiparse_single": 1, "skiparse_group": 2, "block": 3, "skiparse2d_single": 4,
         "skiparse2d_group": 5}
OSP_FUSE_ROPE_Q = 1
OSP_FUSE_ROPE_K = 2
OSP_FUSE_ROPE = 3
OSP_ONE_TILE_PER_WORKGROUP = 4
ABI_VERSION = 1


class OspError(RuntimeError):
    """A libosp call returned a non-zero status."""

    def __init__(self, code: int, message: str):
        super().__init__(f"libosp status {code}: {message}")
        self.code = code
        self.message = message


class OspAttn3dDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_text", ctypes.c_int32),
        ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("rope_t", ctypes.c_int32), ("rope_h", ctypes.c_int32), ("rope_w", ctypes.c_int32),
        ("pos_t0", ctypes.c_int32), ("pos_h0", ctypes.c_int32), ("pos_w0", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("stride_b", ctypes.c_int64), ("stride_n", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("ostride_b", ctypes.c_int64), ("ostride_n", ctypes.c_int64), ("ostride_h", ctypes.c_int64),
    ]


class OspSegment(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int32), ("grid_t", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libosp.so once; raise loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m spatiotemporal_attention_amd.build` (there is no fallback)")
        h = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        D = ctypes.POINTER(OspAttn3dDesc)
        sig = {
            "osp_abi_version": (I32, []),
            "osp_status_string": (ctypes.c_char_p, [I32]),
            "osp_last_error": (ctypes.c_char_p, []),
            "osp_latent_grid": (I32, [I32, I32, I32, I32, I32, I32, I32, ctypes.POINTER(I32)]),
            "osp_attn3d_check": (I32, [D, I32, I32, I32]),
            "osp_rope3d": (I32, [D, P, P, P]),
            "osp_rope3d_inv": (I32, [D, P, P, P]),
            "osp_attn3d_fwd": (I32, [D, I32, I32, F32, I32, P, P, P, P, P, P]),
            "osp_attn3d_packed_fwd": (I32, [D, ctypes.POINTER(OspSegment), I32, I32, I32, F32,
                                            I32, P, P, P, P, P, P]),
            "osp_rope3d_packed": (I32, [D, ctypes.POINTER(OspSegment), I32, P, P, P]),
            "osp_rope3d_packed_inv": (I32, [D, ctypes.POINTER(OspSegment), I32, P, P, P]),
            "osp_attn3d_packed_bwd_workspace": (I32, [D, ctypes.POINTER(OspSegment), I32, I32,
                                                      I32, ctypes.POINTER(I64)]),
            "osp_attn3d_packed_bwd": (I32, [D, ctypes.POINTER(OspSegment), I32, I32, I32, F32,
                                            P, P, P, P, P, P, P, P, P, P, I64, P]),
            "osp_attn3d_bwd_workspace": (I32, [D, I32, I32, ctypes.POINTER(I64)]),
            "osp_attn3d_bwd": (I32, [D, I32, I32, F32, P, P, P, P, P, P, P, P, P, P, I64, P]),
            "osp_attn3d_bwd_noalloc": (I32, [D, I32, I32, F32, P, P, P, P, P, P, P, P, P, P]),
            "osp_skiparse_index": (I32, [I32, I32, I64, P, P, I32, P]),
            "osp_skiparse_index3d": (I32, [I32, I32, I32, I32, I32, P, P, I32, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        if h.osp_abi_version() != ABI_VERSION:
            raise RuntimeError("libosp ABI version mismatch; rebuild the library")
        _lib = h
    return _lib


EXPORTED = ("osp_abi_version", "osp_status_string", "osp_last_error", "osp_latent_grid",
            "osp_attn3d_check", "osp_rope3d", "osp_rope3d_inv", "osp_attn3d_fwd",
            "osp_attn3d_packed_fwd", "osp_rope3d_packed", "osp_rope3d_packed_inv",
            "osp_attn3d_bwd_workspace", "osp_attn3d_bwd", "osp_attn3d_bwd_noalloc",
            "osp_attn3d_packed_bwd_workspace",
            "osp_attn3d_packed_bwd", "osp_skiparse_index", "osp_skiparse_index3d")


def _check(status: int):
    if status != 0:
        raise OspError(status, lib().osp_last_error().decode())


def _mode(mode) -> int:
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"unknown mode {mode!r}")
        return MODES[mode]
    return int(mode)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def osp_abi_version() -> int:
    return int(lib().osp_abi_version())


def osp_latent_grid(frames: int, height: int, width: int, c_t: int, c_s: int,
                    p_t: int = 1, p_s: int = 2) -> tuple:
    """Latent token grid (T, H, W) of a clip after the VAE and patchify."""
    out = (ctypes.c_int32 * 3)()
    _check(lib().osp_latent_grid(frames, height, width, c_t, c_s, p_t, p_s, out))
    return (out[0], out[1], out[2])


def make_desc(*, batch: int, n_text: int, grid, heads: int, head_dim: int, rope_split,
              theta: float = 1e4, pos_offset=(0, 0, 0), strides=(0, 0, 0),
              ostrides=(0, 0, 0)) -> OspAttn3dDesc:
    d = OspAttn3dDesc()
    d.batch, d.n_text = batch, n_text
    d.grid_t, d.grid_h, d.grid_w = grid
    d.heads, d.head_dim = heads, head_dim
    d.rope_t, d.rope_h, d.rope_w = rope_split
    d.pos_t0, d.pos_h0, d.pos_w0 = pos_offset
    d.rope_theta = theta
    d.stride_b, d.stride_n, d.stride_h = strides
    d.ostride_b, d.ostride_n, d.ostride_h = ostrides
    return d


def _bnhd(t: torch.Tensor, name: str):
    if t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(-1) != 1:
        raise ValueError(f"{name} must be a bf16 [B, N, H, D] tensor with unit channel stride")
    return tuple(t.stride()[:3])


def osp_attn3d_check(desc: OspAttn3dDesc, mode="full", sparse_k: int = 1,
                     flags: int = OSP_FUSE_ROPE) -> None:
    """Host-only argument check; raises OspError where osp_attn3d_fwd would."""
    _check(lib().osp_attn3d_check(ctypes.byref(desc), _mode(mode), sparse_k, flags))


def osp_rope3d(x: torch.Tensor, *, grid, n_text: int = 0, rope_split, theta: float = 1e4,
               pos_offset=(0, 0, 0), out: torch.Tensor | None = None) -> torch.Tensor:
    """3D RoPE of x ([B, N, H, D] bf16 on the GPU); out may be x (in place)."""
    return _rope_call("osp_rope3d", x, grid=grid, n_text=n_text, rope_split=rope_split,
                      theta=theta, pos_offset=pos_offset, out=out)


def osp_rope3d_inv(x: torch.Tensor, *, grid, n_text: int = 0, rope_split, theta: float = 1e4,
                   pos_offset=(0, 0, 0), out: torch.Tensor | None = None) -> torch.Tensor:
    """Transpose of osp_rope3d (rotation by the negative angle): maps a
    gradient with respect to the rotated tensor back through the rotation."""
    return _rope_call("osp_rope3d_inv", x, grid=grid, n_text=n_text, rope_split=rope_split,
                      theta=theta, pos_offset=pos_offset, out=out)


def _rope_call(name, x, *, grid, n_text, rope_split, theta, pos_offset, out):
    if out is None:
        out = torch.empty_like(x)
    b, n, h, d = x.shape
    desc = make_desc(batch=b, n_text=n_text, grid=grid, heads=h, head_dim=d,
                     rope_split=rope_split, theta=theta, pos_offset=pos_offset,
                     strides=_bnhd(x, "x"), ostrides=_bnhd(out, "out"))
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError("out must have the shape of x")
    _check(getattr(lib(), name)(ctypes.byref(desc), ctypes.c_void_p(x.data_ptr()),
                                ctypes.c_void_p(out.data_ptr()), _stream(x)))
    return out


def osp_attn3d_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, grid,
                   n_text: int = 0, mode="full", sparse_k: int = 1, rope_split,
                   theta: float = 1e4, sm_scale: float | None = None,
                   fuse_rope=True, pos_offset=(0, 0, 0),
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   return_lse: bool = False, one_tile_per_workgroup: bool = False):
    """Attention forward over [B, N, H, D] bf16 q, k, v on the GPU.

    fuse_rope: True (q and k unrotated: k is rotated by osp_rope3d into a
    temporary of k's strides, q in the attention loader), False (both
    already rotated), "q" or "k" (only that one unrotated, rotated in its
    loader), "qk" (both rotated in the loaders, no temporary; slower, since
    every query tile rotates the same K again).  All give the same bits.
    one_tile_per_workgroup: pass OSP_ONE_TILE_PER_WORKGROUP (no persistent
    launch; the same bits).
    Returns o (and lse [B, H, N] fp32 when return_lse or lse is given)."""
    b, n, h, d = q.shape
    st = _bnhd(q, "q")
    if _bnhd(k, "k") != st or _bnhd(v, "v") != st or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must share shape and strides")
    if out is None:
        out = torch.empty((b, n, h, d), dtype=torch.bfloat16, device=q.device)
    if tuple(out.shape) != (b, n, h, d):
        raise ValueError("out must have the shape of q")
    if lse is None and return_lse:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    desc = make_desc(batch=b, n_text=n_text, grid=grid, heads=h, head_dim=d,
                     rope_split=rope_split, theta=theta, pos_offset=pos_offset,
                     strides=st, ostrides=_bnhd(out, "out"))
    if fuse_rope is True:
        k = osp_rope3d(k, grid=grid, n_text=n_text, rope_split=rope_split, theta=theta,
                       pos_offset=pos_offset, out=_like_strided(k))
    _check(lib().osp_attn3d_fwd(
        ctypes.byref(desc), _mode(mode), int(sparse_k),
        float(sm_scale) if sm_scale is not None else 0.0,
        _flags(fuse_rope) | (OSP_ONE_TILE_PER_WORKGROUP if one_tile_per_workgroup else 0),
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr() if lse is not None else 0), _stream(q)))
    return (out, lse) if lse is not None else out


def _flags(fuse_rope) -> int:
    # True: K is rotated by its own pass before the call, Q in the loader
    if fuse_rope is True:
        return OSP_FUSE_ROPE_Q
    if fuse_rope is False or fuse_rope is None:
        return 0
    return {"q": OSP_FUSE_ROPE_Q, "k": OSP_FUSE_ROPE_K, "qk": OSP_FUSE_ROPE}[fuse_rope]


def _like_strided(t: torch.Tensor) -> torch.Tensor:
    """An uninitialised tensor with t's shape and strides (q, k and v of one
    call must share strides)."""
    return torch.empty_strided(t.size(), t.stride(), dtype=t.dtype, device=t.device)


def _segments(segments, n):
    segs = (OspSegment * len(segments))()
    total = 0
    for i, (n_text, grid) in enumerate(segments):
        segs[i].n_text = int(n_text)
        segs[i].grid_t, segs[i].grid_h, segs[i].grid_w = (int(x) for x in grid)
        total += int(n_text) + int(grid[0]) * int(grid[1]) * int(grid[2])
    if n is not None and total != n:
        raise ValueError(f"segments cover {total} tokens, the tensors hold {n}")
    return segs


def osp_rope3d_packed(x: torch.Tensor, *, segments, rope_split, theta: float = 1e4,
                      pos_offset=(0, 0, 0), out: torch.Tensor | None = None) -> torch.Tensor:
    """3D RoPE of a packed [B, N, H, D] sequence, each segment on its own grid."""
    return _rope_packed_call("osp_rope3d_packed", x, segments=segments, rope_split=rope_split,
                             theta=theta, pos_offset=pos_offset, out=out)


def osp_rope3d_packed_inv(x: torch.Tensor, *, segments, rope_split, theta: float = 1e4,
                          pos_offset=(0, 0, 0), out: torch.Tensor | None = None) -> torch.Tensor:
    """Transpose of osp_rope3d_packed (each segment rotated back on its grid)."""
    return _rope_packed_call("osp_rope3d_packed_inv", x, segments=segments,
                             rope_split=rope_split, theta=theta, pos_offset=pos_offset, out=out)


def _rope_packed_call(name, x, *, segments, rope_split, theta, pos_offset, out):
    if out is None:
        out = torch.empty_like(x)
    b, n, h, d = x.shape
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError("out must have the shape of x")
    segs = _segments(segments, n)
    desc = make_desc(batch=b, n_text=0, grid=(1, 1, n), heads=h, head_dim=d,
                     rope_split=rope_split, theta=theta, pos_offset=pos_offset,
                     strides=_bnhd(x, "x"), ostrides=_bnhd(out, "out"))
    _check(getattr(lib(), name)(ctypes.byref(desc), segs, len(segments),
                                ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                _stream(x)))
    return out


def osp_attn3d_packed_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, segments,
                          mode="full", sparse_k: int = 1, rope_split, theta: float = 1e4,
                          sm_scale: float | None = None, fuse_rope=True, pos_offset=(0, 0, 0),
                          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                          return_lse: bool = False):
    """Attention forward over a packed [B, N, H, D] sequence of several
    videos; ``segments`` lists (n_text, (T, H, W)) in order along N.
    fuse_rope as in osp_attn3d_fwd (True rotates k with osp_rope3d_packed
    into a temporary first)."""
    b, n, h, d = q.shape
    st = _bnhd(q, "q")
    if _bnhd(k, "k") != st or _bnhd(v, "v") != st or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must share shape and strides")
    if out is None:
        out = torch.empty((b, n, h, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    segs = _segments(segments, n)
    desc = make_desc(batch=b, n_text=0, grid=(1, 1, n), heads=h, head_dim=d,
                     rope_split=rope_split, theta=theta, pos_offset=pos_offset, strides=st,
                     ostrides=_bnhd(out, "out"))
    if fuse_rope is True:
        k = osp_rope3d_packed(k, segments=segments, rope_split=rope_split, theta=theta,
                              pos_offset=pos_offset, out=_like_strided(k))
    _check(lib().osp_attn3d_packed_fwd(
        ctypes.byref(desc), segs, len(segments), _mode(mode), int(sparse_k),
        float(sm_scale) if sm_scale is not None else 0.0, _flags(fuse_rope),
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr() if lse is not None else 0), _stream(q)))
    return (out, lse) if lse is not None else out


def osp_attn3d_bwd_workspace(desc: OspAttn3dDesc, mode="full", sparse_k: int = 1) -> int:
    """Bytes of workspace osp_attn3d_bwd needs (host-only query)."""
    out = ctypes.c_int64(0)
    _check(lib().osp_attn3d_bwd_workspace(ctypes.byref(desc), _mode(mode), int(sparse_k),
                                          ctypes.byref(out)))
    return int(out.value)


def osp_attn3d_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, dout: torch.Tensor, *, grid, n_text: int = 0,
                   mode="full", sparse_k: int = 1, sm_scale: float | None = None,
                   dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                   dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Attention backward over [B, N, H, D] bf16 tensors on the GPU.

    q and k are the rotated tensors; dq and dk are gradients with respect to
    them (osp_rope3d_inv maps them back through the rotation).  lse is the
    forward's [B, H, N] fp32 log-sum-exp.  Returns (dq, dk, dv)."""
    b, n, h, d = q.shape
    st = _bnhd(q, "q")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if _bnhd(t, name) != st or t.shape != q.shape:
            raise ValueError("q, k, v, o and dout must share shape and strides")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    outs = []
    for t in (dq, dk, dv):
        outs.append(torch.empty((b, n, h, d), dtype=torch.bfloat16, device=q.device)
                    if t is None else t)
    ost = _bnhd(outs[0], "dq")
    if any(_bnhd(t, "dk/dv") != ost or tuple(t.shape) != (b, n, h, d) for t in outs):
        raise ValueError("dq, dk and dv must share the shape of q and one set of strides")
    desc = make_desc(batch=b, n_text=n_text, grid=grid, heads=h, head_dim=d,
                     rope_split=(d, 0, 0), strides=st, ostrides=ost)
    need = osp_attn3d_bwd_workspace(desc, mode, sparse_k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace of {need} bytes needed")
    _check(lib().osp_attn3d_bwd(
        ctypes.byref(desc), _mode(mode), int(sparse_k),
        float(sm_scale) if sm_scale is not None else 0.0,
        *(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse, dout, *outs, workspace)),
        int(workspace.numel() * workspace.element_size()), _stream(q)))
    return tuple(outs)


def osp_attn3d_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                           lse: torch.Tensor, dout: torch.Tensor, *, grid, n_text: int = 0,
                           mode="full", sparse_k: int = 1, sm_scale: float | None = None,
                           dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor):
    """osp_attn3d_bwd without a workspace: the library's own per-GPU scratch
    array holds the row terms, and the call allocates nothing (dq, dk and
    dv are required).  Runs on q's device; calls that overlap on one GPU
    race on the scratch.  Returns (dq, dk, dv)."""
    b, n, h, d = q.shape
    st = _bnhd(q, "q")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if _bnhd(t, name) != st or t.shape != q.shape:
            raise ValueError("q, k, v, o and dout must share shape and strides")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    ost = _bnhd(dq, "dq")
    if any(_bnhd(t, "dk/dv") != ost or tuple(t.shape) != (b, n, h, d) for t in (dq, dk, dv)):
        raise ValueError("dq, dk and dv must share the shape of q and one set of strides")
    desc = make_desc(batch=b, n_text=n_text, grid=grid, heads=h, head_dim=d,
                     rope_split=(d, 0, 0), strides=st, ostrides=ost)
    with torch.cuda.device(q.device):
        _check(lib().osp_attn3d_bwd_noalloc(
            ctypes.byref(desc), _mode(mode), int(sparse_k),
            float(sm_scale) if sm_scale is not None else 0.0,
            *(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse, dout, dq, dk, dv)),
            _stream(q)))
    return dq, dk, dv


def osp_attn3d_packed_bwd_workspace(desc: OspAttn3dDesc, segments, mode="full",
                                    sparse_k: int = 1) -> int:
    """Bytes of workspace osp_attn3d_packed_bwd needs (host-only query)."""
    out = ctypes.c_int64(0)
    segs = _segments(segments, None)
    _check(lib().osp_attn3d_packed_bwd_workspace(ctypes.byref(desc), segs, len(segments),
                                                 _mode(mode), int(sparse_k), ctypes.byref(out)))
    return int(out.value)


def osp_attn3d_packed_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                          lse: torch.Tensor, dout: torch.Tensor, *, segments, mode="full",
                          sparse_k: int = 1, sm_scale: float | None = None,
                          dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                          dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Attention backward over a packed [B, N, H, D] sequence (segments as in
    osp_attn3d_packed_fwd).  q and k are the rotated tensors; dq and dk are
    gradients with respect to them (osp_rope3d_packed_inv maps them back).
    lse is the packed forward's [B, H, N] fp32 log-sum-exp.  Returns
    (dq, dk, dv)."""
    b, n, h, d = q.shape
    st = _bnhd(q, "q")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if _bnhd(t, name) != st or t.shape != q.shape:
            raise ValueError("q, k, v, o and dout must share shape and strides")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    outs = []
    for t in (dq, dk, dv):
        outs.append(torch.empty((b, n, h, d), dtype=torch.bfloat16, device=q.device)
                    if t is None else t)
    ost = _bnhd(outs[0], "dq")
    if any(_bnhd(t, "dk/dv") != ost or tuple(t.shape) != (b, n, h, d) for t in outs):
        raise ValueError("dq, dk and dv must share the shape of q and one set of strides")
    segs = _segments(segments, n)
    desc = make_desc(batch=b, n_text=0, grid=(1, 1, n), heads=h, head_dim=d,
                     rope_split=(d, 0, 0), strides=st, ostrides=ost)
    need = osp_attn3d_packed_bwd_workspace(desc, segments, mode, sparse_k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace of {need} bytes needed")
    _check(lib().osp_attn3d_packed_bwd(
        ctypes.byref(desc), segs, len(segments), _mode(mode), int(sparse_k),
        float(sm_scale) if sm_scale is not None else 0.0,
        *(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse, dout, *outs, workspace)),
        int(workspace.numel() * workspace.element_size()), _stream(q)))
    return tuple(outs)


def osp_skiparse_index(mode, sparse_k: int, n_tokens: int, device=None):
    """(perm, inv) int32 maps.  device=None: numpy arrays filled by the
    library's host path; else torch tensors filled by its device kernel."""
    return _index_call(lambda *ptrs: lib().osp_skiparse_index(
        _mode(mode), int(sparse_k), int(n_tokens), *ptrs), int(n_tokens), device)


def osp_skiparse_index3d(mode, sparse_k: int, grid, device=None):
    """(perm, inv) int32 maps of the N = T*H*W video tokens of ``grid``; the
    only index call that takes the Skiparse-2D modes."""
    t, h, w = (int(x) for x in grid)
    return _index_call(lambda *ptrs: lib().osp_skiparse_index3d(
        _mode(mode), int(sparse_k), t, h, w, *ptrs), t * h * w, device)


def _index_call(call, n_tokens: int, device):
    if device is None:
        perm = np.empty(n_tokens, dtype=np.int32)
        inv = np.empty(n_tokens, dtype=np.int32)
        _check(call(perm.ctypes.data_as(ctypes.c_void_p), inv.ctypes.data_as(ctypes.c_void_p), 0,
                    None))
        return perm, inv
    perm = torch.empty(n_tokens, dtype=torch.int32, device=device)
    inv = torch.empty(n_tokens, dtype=torch.int32, device=device)
    _check(call(ctypes.c_void_p(perm.data_ptr()), ctypes.c_void_p(inv.data_ptr()), 1,
                _stream(perm)))
    return perm, inv

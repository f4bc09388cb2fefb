"""A numpy model of the roundings the HIP attention kernels take.

TEST INFRASTRUCTURE: it sizes the tolerance bars of the GPU parity tests.
It is not the oracle (``oracle/`` is the definition the library is checked
against) and it shares nothing with the library: it restates, in numpy, the
rounding steps that the library's header and kernel comments document, so
that the error those roundings leave against the fp64 oracle can be measured
on the CPU for the exact inputs a GPU test uses.

Forward (the flash kernel and the short-subsequence kernel alike):
  * K rotated in fp32 and rounded to bf16 (RNE);
  * Q rotated in fp32, multiplied by sm_scale * log2(e) in fp32 and rounded
    to bf16 once (a Q passed in already rotated is rounded a second time,
    after the scale);
  * scores z = q k^T accumulated in fp32 (log2 units);
  * p = exp2(z - m) in fp32 with m a row maximum; p rounded to bf16 for the
    PV product, the row sum l of the unrounded fp32 p;
  * O = bf16(sum bf16(p) v / l), LSE = (m + log2 l) ln 2 in fp32.
Backward (q and k the rotated bf16 tensors, o and lse from the forward):
  * -delta = -sum O dO in fp32, -lse / s in fp32;
  * the dK/dV pass forms p = exp2(s log2(e) (q k^T - lse / s)), the dQ pass
    p = exp2(bf16(s log2(e) q) k^T - (lse / s) s log2(e)) (Q scaled in
    registers and rounded to bf16 once), in fp32; p is rounded to bf16 for
    dV = p^T dO;
  * dS = p (dO v^T - delta) in fp32, rounded to bf16 for dQ = s dS k and
    dK = s dS^T q;
  * dq, dk, dv rounded to bf16; the RoPE transpose rotates dq and dk in fp32
    and rounds them once more.

``exact=True`` turns every rounding off and computes in fp64: the model
then is the plain definition, which the tests check against the oracle to
1e-10 before trusting the rounded runs.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

LOG2E = 1.0 / math.log(2.0)


def bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16, ties to even, through fp32 (finite
    inputs); returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


class Precision:
    """The arithmetic of one model run: bf16 roundings and fp32 products, or
    (exact) neither."""

    def __init__(self, exact: bool):
        self.exact = exact
        self.dt = np.float64 if exact else np.float32

    def rnd(self, x):
        return np.asarray(x, dtype=np.float64) if self.exact else bf16(x)

    def f(self, x):
        return np.asarray(x, dtype=self.dt)


def _rotate(x, grid, n_text, rope_split, theta, pos_offset, pr: Precision, inverse=False):
    """3D RoPE (or its transpose) of x [B, N, H, D] in the model's precision:
    the oracle's rotation evaluated in fp64, then brought to fp32 (the
    library rotates in fp32; the difference is far below a bf16 step)."""
    fn = oracle.rope3d_transpose if inverse else oracle.rope3d
    return pr.f(fn(np.asarray(x, np.float64), grid, n_text, rope_split, theta, pos_offset))


def attn_fwd(q, k, v, *, grid, n_text=0, mode="full", sparse_k=1, rope_split, theta=1e4,
             sm_scale=None, pos_offset=(0, 0, 0), q_rotated=False, k_rotated=False,
             exact=False):
    """The forward's arithmetic on [B, N, H, D] bf16-valued inputs.

    q_rotated / k_rotated: the tensor is passed in already rotated (and
    rounded to bf16 by the caller's own pass), so the kernel does not rotate
    it.  Returns (o, lse) as float64 arrays shaped like the oracle's."""
    pr = Precision(exact)
    b_sz, n, h_sz, d = q.shape
    s = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    c2 = pr.f(s * LOG2E)
    qr = pr.f(q) if q_rotated else _rotate(q, grid, n_text, rope_split, theta, pos_offset, pr)
    kr = pr.f(k) if k_rotated else _rotate(k, grid, n_text, rope_split, theta, pos_offset, pr)
    q_op = pr.rnd(qr * c2)
    k_op = pr.rnd(kr)
    v_op = pr.f(v)
    o = np.zeros((b_sz, n, h_sz, d))
    lse = np.zeros((b_sz, h_sz, n))
    for g in oracle.skiparse_groups(mode, sparse_k, n, grid):
        for b in range(b_sz):
            for h in range(h_sz):
                z = q_op[b, g, h].astype(pr.dt) @ k_op[b, g, h].astype(pr.dt).T
                m = z.max(axis=1, keepdims=True)
                p = np.exp2(z - m).astype(pr.dt)
                l = p.sum(axis=1, keepdims=True, dtype=pr.dt)
                ob = (pr.rnd(p).astype(pr.dt) @ v_op[b, g, h]) / l
                o[b, g, h] = pr.rnd(ob)
                lse[b, h, g] = ((m + np.log2(l)) * math.log(2.0))[:, 0]
    return o, lse


def attn_bwd(q, k, v, do, *, grid, n_text=0, mode="full", sparse_k=1, rope_split=None,
             theta=1e4, sm_scale=None, pos_offset=(0, 0, 0), rope_chain=False, exact=False):
    """The backward's arithmetic.  Without ``rope_chain``, q and k are the
    (bf16) rotated inputs and the gradients are with respect to them; with
    it, q and k are rotated by a RoPE pass first (rounded to bf16), the
    forward runs on those, and dq, dk come back through the transpose.
    Returns (dq, dk, dv) as float64 arrays."""
    pr = Precision(exact)
    b_sz, n, h_sz, d = q.shape
    s = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    if rope_chain:
        q = pr.rnd(_rotate(q, grid, n_text, rope_split, theta, pos_offset, pr))
        k = pr.rnd(_rotate(k, grid, n_text, rope_split, theta, pos_offset, pr))
    q, k, v, do = (pr.f(t) for t in (q, k, v, do))
    o, lse = attn_fwd(q, k, v, grid=grid, n_text=n_text, mode=mode, sparse_k=sparse_k,
                      rope_split=rope_split, theta=theta, sm_scale=s, pos_offset=pos_offset,
                      q_rotated=True, k_rotated=True, exact=exact)
    o = pr.f(o)
    neg_delta = -(o * do).sum(axis=-1, dtype=pr.dt)             # [B, N, H]
    neg_lse_s = pr.f(-lse / s)                                  # [B, H, N]
    c2 = pr.f(s * LOG2E)
    dq = np.zeros(q.shape)
    dk = np.zeros(q.shape)
    dv = np.zeros(q.shape)
    for g in oracle.skiparse_groups(mode, sparse_k, n, grid):
        for b in range(b_sz):
            for h in range(h_sz):
                qq, kk, vv, dd = q[b, g, h], k[b, g, h], v[b, g, h], do[b, g, h]
                nls = neg_lse_s[b, h, g][:, None]
                dpd = dd @ vv.T + neg_delta[b, g, h][:, None]
                # the dK/dV pass
                p_kv = np.exp2(c2 * (qq @ kk.T + nls)).astype(pr.dt)
                dv[b, g, h] = pr.rnd(pr.rnd(p_kv).T.astype(pr.dt) @ dd)
                dk[b, g, h] = pr.rnd(s * (pr.rnd(p_kv * dpd).astype(pr.dt).T @ qq))
                # the dQ pass: Q scaled in registers
                p_q = np.exp2(pr.rnd(c2 * qq).astype(pr.dt) @ kk.T + pr.f(nls * c2)).astype(pr.dt)
                dq[b, g, h] = pr.rnd(s * (pr.rnd(p_q * dpd).astype(pr.dt) @ kk))
    if rope_chain:
        dq = pr.rnd(_rotate(dq, grid, n_text, rope_split, theta, pos_offset, pr, inverse=True))
        dk = pr.rnd(_rotate(dk, grid, n_text, rope_split, theta, pos_offset, pr, inverse=True))
    return tuple(np.asarray(t, np.float64) for t in (dq, dk, dv))


def errors(got, want):
    """(max-abs, rel-L2) of got against want."""
    diff = np.asarray(got, np.float64) - np.asarray(want, np.float64)
    return float(np.abs(diff).max()), float(np.linalg.norm(diff) / np.linalg.norm(want))

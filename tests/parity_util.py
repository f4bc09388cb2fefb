"""Helpers for GPU-vs-oracle parity tests."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads

# Parity bar for bf16 inputs with fp32 accumulation against the fp64 oracle.
MAX_ABS = 2e-2
REL_L2 = 5e-3
LSE_ABS = 1e-2


def note(msg: str):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(msg, file=sys.stderr, flush=True)


def errors(got: np.ndarray, want: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), "non-finite values in the GPU result"
    diff = got - want
    return float(np.abs(diff).max()), float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-300))


def assert_parity(got, want, what: str, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = errors(got, want)
    note(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"


def grid_of(wl: workloads.Workload):
    if wl.grid is not None:
        return tuple(wl.grid)
    return oracle.latent_grid(*wl.clip, wl.c_t, wl.c_s, wl.p_t, wl.p_s)


def qkv_for(seed, shape, scale=None, q_mult=None, device="cuda"):
    q, k, v = workloads.make_qkv(seed, shape, scale, q_mult)
    return (q, k, v), tuple(t.to(device) for t in (q, k, v))


def oracle_attn(cpu_qkv, *, grid, n_text, mode, sparse_k, rope_split, theta=1e4,
                sm_scale=None, pos_offset=(0, 0, 0), rows=None):
    q, k, v = (workloads.to_f64(t) for t in cpu_qkv)
    return oracle.attn3d(q, k, v, grid=grid, n_text=n_text, mode=mode, sparse_k=sparse_k,
                         rope_split=rope_split, theta=theta, sm_scale=sm_scale,
                         pos_offset=pos_offset, rows=rows)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()

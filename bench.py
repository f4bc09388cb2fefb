"""Benchmark: 3D-RoPE attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole hot path over one batch of synthetic input
on the Open-Sora-Plan-shaped 93x480p workload (grid 24x30x40 = 28,800
tokens, batch 1, 24 heads, head_dim 96): latent grid of the clip on the
host, 3D RoPE of K in one memory-bound pass (osp_rope3d), then attention
with the rotation of Q fused into its loader, full attention over all
tokens and the output written back in token order (osp_attn3d_fwd).
Inputs are resident in HBM before timing.

Prints ONE JSON line.  value = algorithmic attention TFLOP/s
(4*B*H*N^2*D / k per call).  Also reported: the same kernel on Skiparse k=4
(single and group skip), the roofline of the attention kernel (MFMA bound,
dense bf16 peak 2516.6 TFLOP/s), HBM traffic from rocprofv3 counters (when
taken on the current kernel source) and the fp64 CPU oracle's rate on a
bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
KERNEL_SRC = os.path.join(ROOT, "spatiotemporal_attention_amd", "csrc", "attn3d_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn3d_fwd_osp480_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("attn3d_fwd.hip", "osp_mfma.hpp", "osp_rope.hpp", "osp_common.hpp",
                 "osp_internal.hpp"):
        with open(os.path.join(ROOT, "spatiotemporal_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-skiparse", action="store_true", help="skip the Skiparse k=4 lines")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=6,
                   help="heads of the workload the oracle times (all query rows each)")
    p.add_argument("--profile", action="store_true",
                   help="few steps of one attention mode only (for rocprofv3)")
    p.add_argument("--no-backward", action="store_true", help="skip the backward line")
    p.add_argument("--no-packed", action="store_true", help="skip the frame-pack line")
    p.add_argument("--profile-mode", default="full",
                   choices=("full", "skiparse_single", "skiparse_group", "bwd", "temporal",
                            "packed"),
                   help="what --profile runs: attention over the 28,800-token workload (Skiparse "
                        "with k=4; temporal: Single Skip with k = H*W), its backward (bwd), or the "
                        "CogVideoX frame pack (packed)")
    p.add_argument("--copy", type=int, default=0,
                   help="instead: time a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(each attention unit (batch, head, subsequence) is independent; "
              "see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import spatiotemporal_attention_amd as osp
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy:
        n = args.copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy, "bytes_read": n * 4, "bytes_written": n * 4}))
        return

    wl = workloads.WORKLOADS["osp480"]
    grid = osp.osp_latent_grid(*wl.clip, wl.c_t, wl.c_s, wl.p_t, wl.p_s)      # row a1 on the host
    n_tok = wl.n_text + grid[0] * grid[1] * grid[2]
    B, H, D = wl.batch, wl.heads, wl.head_dim
    shape = (B, n_tok, H, D)
    q, k, v = (t.to(dev) for t in workloads.make_qkv(wl.seed, shape, wl.input_scale))
    o = torch.empty_like(q)
    k_rot = torch.empty_like(k)
    stream = torch.cuda.current_stream(dev)

    def step(mode="full", sk=1, marks=None):
        osp.osp_rope3d(k, grid=grid, n_text=wl.n_text, rope_split=wl.rope_split,
                       theta=wl.theta, out=k_rot)
        if marks:
            marks[0].record(stream)
        osp.osp_attn3d_fwd(q, k_rot, v, grid=grid, n_text=wl.n_text, mode=mode, sparse_k=sk,
                           rope_split=wl.rope_split, theta=wl.theta, fuse_rope="q", out=o)
        if marks:
            marks[1].record(stream)

    def flops(sk=1):
        return 4.0 * B * H * float(n_tok) ** 2 * D / sk

    # backward: gradients with respect to the rotated q and k (then through
    # the RoPE transpose), from the forward's o and lse
    bwd_state = {}

    def bwd_setup():
        if bwd_state:
            return bwd_state
        q_rot = osp.osp_rope3d(q, grid=grid, n_text=wl.n_text, rope_split=wl.rope_split,
                               theta=wl.theta)
        osp.osp_rope3d(k, grid=grid, n_text=wl.n_text, rope_split=wl.rope_split,
                       theta=wl.theta, out=k_rot)
        o_b, lse_b = osp.osp_attn3d_fwd(q_rot, k_rot, v, grid=grid, n_text=wl.n_text,
                                        rope_split=wl.rope_split, theta=wl.theta,
                                        fuse_rope=False, return_lse=True)
        dout = workloads.make_dout(wl.seed, shape, wl.input_scale).to(dev)
        desc = osp.make_desc(batch=B, n_text=wl.n_text, grid=grid, heads=H, head_dim=D,
                             rope_split=wl.rope_split)
        ws = torch.empty(osp.osp_attn3d_bwd_workspace(desc), dtype=torch.uint8, device=dev)
        grads = tuple(torch.empty_like(q) for _ in range(3))
        bwd_state.update(q_rot=q_rot, o=o_b, lse=lse_b, dout=dout, ws=ws, grads=grads)
        return bwd_state

    def bwd_step(marks=None):
        st = bwd_state
        dq, dk, dv = st["grads"]
        if marks:
            marks[0].record(stream)
        osp.osp_attn3d_bwd(st["q_rot"], k_rot, v, st["o"], st["lse"], st["dout"], grid=grid,
                           n_text=wl.n_text, dq=dq, dk=dk, dv=dv, workspace=st["ws"])
        if marks:
            marks[1].record(stream)
        for t in (dq, dk):
            osp.osp_rope3d_inv(t, grid=grid, n_text=wl.n_text, rope_split=wl.rope_split,
                               theta=wl.theta, out=t)

    def packed_setup():
        # CogVideoX Multi-Resolution Frame Pack: four clips with their text
        # in one sequence, block-diagonal attention
        pk = workloads.COGVIDEOX_PACK
        wlc = workloads.WORKLOADS[pk["base"]]
        segs = [(pk["n_text"], osp.osp_latent_grid(*c, wlc.c_t, wlc.c_s, wlc.p_t, wlc.p_s))
                for c in pk["clips"]]
        lens = [nt + g[0] * g[1] * g[2] for nt, g in segs]
        pshape = (1, sum(lens), wlc.heads, wlc.head_dim)
        qp, kp, vp = (t.to(dev) for t in workloads.make_qkv(pk["seed"], pshape))
        op = torch.empty_like(qp)
        kp_rot = torch.empty_like(kp)

        def runp():
            # as in the step above: K rotated by its own pass, Q in the loader
            osp.osp_rope3d_packed(kp, segments=segs, rope_split=wlc.rope_split, out=kp_rot)
            osp.osp_attn3d_packed_fwd(qp, kp_rot, vp, segments=segs, rope_split=wlc.rope_split,
                                      fuse_rope="q", out=op)

        def packed_bwd_setup():
            # the backward of the same pack: q and k rotated, o and lse from
            # one forward, a seeded dO; one call is the packed backward plus
            # the two packed RoPE transposes
            qr = osp.osp_rope3d_packed(qp, segments=segs, rope_split=wlc.rope_split)
            kr = osp.osp_rope3d_packed(kp, segments=segs, rope_split=wlc.rope_split)
            o2, lse2 = osp.osp_attn3d_packed_fwd(qr, kr, vp, segments=segs,
                                                 rope_split=wlc.rope_split, fuse_rope=False,
                                                 return_lse=True)
            dop = workloads.make_dout(pk["seed"], pshape).to(dev)
            grads = tuple(torch.empty_like(qp) for _ in range(3))
            desc = osp.make_desc(batch=1, n_text=0, grid=(1, 1, sum(lens)), heads=wlc.heads,
                                 head_dim=wlc.head_dim, rope_split=wlc.rope_split)
            ws = torch.empty(osp.osp_attn3d_packed_bwd_workspace(desc, segs), dtype=torch.uint8,
                             device=dev)

            def runb():
                osp.osp_attn3d_packed_bwd(qr, kr, vp, o2, lse2, dop, segments=segs, dq=grads[0],
                                          dk=grads[1], dv=grads[2], workspace=ws)
                osp.osp_rope3d_packed_inv(grads[0], segments=segs, rope_split=wlc.rope_split,
                                          out=grads[0])
                osp.osp_rope3d_packed_inv(grads[1], segments=segs, rope_split=wlc.rope_split,
                                          out=grads[1])
            return runb
        runp.bwd_setup = packed_bwd_setup
        return runp, segs, lens, wlc

    if args.profile:
        pm = args.profile_mode
        if pm == "bwd":
            bwd_setup()
            run = bwd_step
        elif pm == "packed":
            run = packed_setup()[0]
        elif pm == "temporal":
            run = lambda: step("skiparse_single", grid[1] * grid[2])   # noqa: E731
        else:
            pk = 1 if pm == "full" else 4
            run = lambda: step(pm, pk)   # noqa: E731
        for _ in range(max(args.warmup, 1)):
            run()
        torch.cuda.synchronize()
        for _ in range(max(args.steps, 1)):
            run()
        torch.cuda.synchronize()
        print(json.dumps({"profile_launches": args.steps, "workload": f"osp480 {pm}"}))
        return

    def timed(mode, sk, steps, warmup):
        for _ in range(warmup):
            step(mode, sk)
        torch.cuda.synchronize()
        # per-launch events on the launch stream (the kernel's own duration)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        t0.record(stream)
        for marks in evs:
            step(mode, sk, marks)     # events bracket the attention launch
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        total_ms = t0.elapsed_time(t1)
        per = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        return total_ms / steps, sum(per) / len(per), per[len(per) // 2], per[0], wall

    ms_step, ms_launch, ms_med, ms_min, wall = timed("full", 1, args.steps, args.warmup)
    f_full = flops(1)
    value = f_full / (ms_step * 1e-3) / 1e12
    achieved = f_full / (ms_launch * 1e-3) / 1e12
    traffic = load_traffic()

    extra = {}
    sep = None
    suv = None
    if not args.no_skiparse:
        # Skiparse-2D group needs H and W divisible by 4 at k = 4, which 30 x 40 is not
        for mode in ("skiparse_single", "skiparse_group", "skiparse2d_single"):
            s_step, s_launch, s_med, s_min, _ = timed(mode, 4, max(args.steps, 5), args.warmup)
            tf = flops(4) / (s_launch * 1e-3) / 1e12
            extra[mode] = {"k": 4, "ms_per_launch": round(s_launch, 4), "ms_min": round(s_min, 4),
                           "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                           "dense_equiv_tflops": round(f_full / (s_launch * 1e-3) / 1e12, 2)}
        # separated spatial / temporal attention on the same tensors: block
        # attention over each frame, then single skip over each (h, w) position
        sep = {}
        for name, mode, kk in (("spatial", "block", grid[0]),
                               ("temporal", "skiparse_single", grid[1] * grid[2])):
            _, s_launch, _, s_min, _ = timed(mode, kk, max(args.steps, 5), args.warmup)
            tf = flops(kk) / (s_launch * 1e-3) / 1e12
            sep[name] = {"mode": mode, "k": kk, "ms_per_launch": round(s_launch, 4),
                         "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        sep["ms_spatial_plus_temporal"] = round(sep["spatial"]["ms_per_launch"] +
                                                sep["temporal"]["ms_per_launch"], 4)
        sep["vs_full_3d"] = round(sep["ms_spatial_plus_temporal"] / ms_launch, 4)
        # a U-shaped per-layer sparsity schedule over the same tensors: the
        # attention time of one pass through its layers against every layer
        # full (each distinct (mode, k) timed once)
        per = {}
        for mode, kk in workloads.SUV_SCHEDULE:
            if (mode, kk) not in per:
                per[(mode, kk)] = timed(mode, kk, max(args.steps // 2, 5), args.warmup)[1]
        ms_pass = sum(per[mk] for mk in workloads.SUV_SCHEDULE)
        f_pass = sum(flops(kk) for _, kk in workloads.SUV_SCHEDULE)
        suv = {"schedule": [[m, kk] for m, kk in workloads.SUV_SCHEDULE],
               "ms_per_pass": round(ms_pass, 4),
               "ms_all_full": round(len(workloads.SUV_SCHEDULE) * ms_launch, 4),
               "vs_all_full": round(ms_pass / (len(workloads.SUV_SCHEDULE) * ms_launch), 4),
               "tflops": round(f_pass / (ms_pass * 1e-3) / 1e12, 2)}

    packed = None
    if not args.no_packed:
        runp, segs, lens, wlc = packed_setup()
        for _ in range(args.warmup):
            runp()
        torch.cuda.synchronize()
        npk = max(args.steps // 2, 5)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(npk):
            runp()
        t1.record(stream)
        torch.cuda.synchronize()
        p_ms = t0.elapsed_time(t1) / npk
        f_pack = sum(4.0 * wlc.heads * float(L) ** 2 * wlc.head_dim for L in lens)
        tf = f_pack / (p_ms * 1e-3) / 1e12
        packed = {"segments": [[nt, list(g)] for nt, g in segs], "tokens": sum(lens),
                  "heads": wlc.heads, "head_dim": wlc.head_dim, "ms_per_call": round(p_ms, 4),
                  "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                  "flop_per_call": f_pack,
                  "launches": f"rope3d of K per segment ({len(segs)}), then one flash "
                              "launch over the segment table, Q rotated in its loader"}
        runb = runp.bwd_setup()
        for _ in range(args.warmup):
            runb()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(npk):
            runb()
        t1.record(stream)
        torch.cuda.synchronize()
        pb_ms = t0.elapsed_time(t1) / npk
        tfb = 2.5 * f_pack / (pb_ms * 1e-3) / 1e12
        packed["backward"] = {"ms_per_call": round(pb_ms, 4), "tflops": round(tfb, 2),
                              "frac_of_peak": round(tfb / PEAK_BF16_TFLOPS, 4),
                              "launches": "one workspace pass, dK/dV and dQ launches over "
                                          "the segment table, then the packed RoPE transpose "
                                          "of dq and dk"}

    bwd = None
    if not args.no_backward:
        bwd_setup()
        nb = max(args.steps // 2, 5)
        for _ in range(args.warmup):
            bwd_step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(nb)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for marks in evs:
            bwd_step(marks)
        t1.record(stream)
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        b_launch = sum(per) / len(per)
        b_step = t0.elapsed_time(t1) / nb
        # FlashAttention convention: the backward counts 2.5x the forward's
        # flops (5 matrix products against 2); the kernels execute 7
        f_bwd = 2.5 * f_full
        tf = f_bwd / (b_launch * 1e-3) / 1e12
        bwd = {"ms_per_call": round(b_launch, 4), "ms_min": round(per[0], 4),
               "ms_per_step_with_rope_transpose": round(b_step, 4),
               "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
               "flop_per_call": f_bwd, "executed_mfma_tflops": round(tf * 7 / 5, 2),
               "kernels": "bwd_prep + bwd_dkdv_kernel (8 waves in pairs, 64 keys per pair) + bwd_dq_kernel (8 waves), D=96",
               "fwd_plus_bwd_ms": round(ms_launch + b_launch, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nh = max(1, min(args.cpu_heads, H))
        hs = slice(0, nh)
        cpu_in = [workloads.to_f64(t[:, :, hs].cpu()) for t in (q, k, v)]
        t_c = time.perf_counter()
        oracle.attn3d(*cpu_in, grid=grid, n_text=wl.n_text, rope_split=wl.rope_split,
                      theta=wl.theta)
        dt = time.perf_counter() - t_c
        cores = torch.get_num_threads()
        try:
            import threadpoolctl
            info = threadpoolctl.threadpool_info()
            cores = max([i.get("num_threads", 0) for i in info if i.get("user_api") == "blas"] or [cores])
        except Exception:  # noqa: BLE001 -- reporting only
            pass
        cpu = {"value": round(4.0 * B * nh * float(n_tok) ** 2 * D / dt / 1e12, 5),
               "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
               "sample": f"fp64 numpy oracle, full attention with 3D RoPE over all {n_tok} query "
                         f"rows of {nh} of {H} heads ({dt:.1f} s)"}

    line = {
        "metric": "attention TFLOP/s and % of bf16 MFMA peak at 28,800 tokens, full vs Skiparse k=4",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "osp480 full attention: 93x480x640 clip, 4x8x8 VAE, 1x2x2 patchify "
                               f"-> grid {grid[0]}x{grid[1]}x{grid[2]} = {n_tok} tokens, batch {B}, "
                               f"{H} heads, head_dim {D}, fused 3D RoPE {wl.rope_split}",
                   "global_batch": B, "seq_len": n_tok, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "attn3d_fwd_kernel<D=96, QB=1, BN=64, NW=8, OCC=2, rope_q, fixed_rows>",
                     "flop_per_launch": f_full, "ms_per_launch": round(ms_launch, 4),
                     "ms_median": round(ms_med, 4), "ms_min": round(ms_min, 4)},
        "skiparse": extra,
        "separated_2d1d": sep,
        "suv_schedule": suv,
        "backward": bwd,
        "packed": packed,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

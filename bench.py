#!/usr/bin/env python3
"""Benchmark of the 3D-RoPE sparse + low-rank attention layer forward on one
MI355X: ms/layer and effective TFLOP/s, with the dominant kernel's roofline,
per-stage times, the in-library dense flash kernel and the CPU oracle.

    python bench.py [--steps K] [--warmup W] [--workload wan13b|wan14b|hunyuan13b]

One step = one slr_attention_fwd over the whole layer (rotate + pool, block
top-k, low-rank summary, block-sparse flash + low-rank readout + gated
combine). Inputs are seeded synthetic layers already resident in HBM.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the sparse flash kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch, scaled x2 and x1 by what the same counters read
# for a plain 1 GiB copy). They hold only for the kernel source they were taken
# on, identified by the sha256 of its files; any other source reports null.
FLASH_TRAFFIC_SOURCES = ["k_flash.hip", "slr_common.h", "slr_launch.h"]
FLASH_TRAFFIC = {
    "sha256": "7d776f0545ef627a151a7e498bce077389493b0a1417e52510607e12c8671b19",
    "bytes_per_launch": {"wan13b": 8202.8e6 + 201.3e6, "wan14b": 220518.4e6 + 1548.4e6},
}


def flash_traffic(workload: str):
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_rank_attention_rope3d_amd", "csrc")
    h = hashlib.sha256()
    try:
        for f in FLASH_TRAFFIC_SOURCES:
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    except OSError:
        return None
    if h.hexdigest() != FLASH_TRAFFIC["sha256"]:
        return None
    return FLASH_TRAFFIC["bytes_per_launch"].get(workload)


def achievable_peaks(torch) -> dict:
    """Rates this GPU sustains, as context for the published peaks: a large
    bf16 GEMM on random operands (the vendor library through torch.matmul;
    random data draws the power that real layers draw, and the clock drops
    with it) and a 1 GiB device-to-device copy (read + write bytes)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    reps = 40
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    nbytes = 2 ** 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"gemm_bf16_TFLOP/s": round(gemm_tf, 1), "copy_GB/s": round(copy_gbs, 1),
            "what": "8192^3 bf16 torch.matmul on random operands; 1 GiB device copy, read + write bytes"}


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def _event(h):
    e = ctypes.c_void_p()
    assert h.hipEventCreate(ctypes.byref(e)) == 0
    return e.value


def _elapsed(h, a, b) -> float:
    ms = ctypes.c_float()
    assert h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
    return ms.value


def make_device_inputs(cfg, torch):
    from sparse_rank_attention_rope3d_amd import synth
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shp = (cfg.B, cfg.H, cfg.L, cfg.D)
    q, k, v = (torch.empty(shp, dtype=tdt, device="cuda") for _ in range(3))
    for b in range(cfg.B):
        for h in range(cfg.H):
            for dst, arr in zip((q, k, v), synth.qkv_slice(cfg, b, h)):
                if cfg.dtype == "bf16":
                    bits = synth.f32_to_bf16_bits(arr)
                    dst[b, h] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
                else:
                    dst[b, h] = torch.from_numpy(arr).cuda()
    params = {kk: torch.from_numpy(vv).cuda() for kk, vv in synth.lowrank_params(cfg).items()}
    return q, k, v, params


def cpu_baseline(cfg, blocks: int):
    """The CPU oracle (one thread, fp64) on one (b, h) slice: the whole
    selection and summary plus `blocks` sampled query blocks of the sparse
    branch and readout, extrapolated linearly to the full layer."""
    import oracle
    from sparse_rank_attention_rope3d_amd import synth
    q, k, v = synth.qkv_slice(cfg, 0, 0)
    p = synth.lowrank_params(cfg)
    E = (p["et"], p["eh"], p["ew"]) if cfg.lr_mode == "abspe" else None
    rng = np.random.default_rng([cfg.seed, synth.TID_SAMPLE, 0, 0])
    qblocks = np.sort(rng.choice(cfg.nblk, size=min(blocks, cfg.nblk), replace=False)).astype(np.int32)
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    t0 = time.perf_counter()
    qr = oracle.rope3d(q, grid, cfg.base, cfg.pairs)
    kr = oracle.rope3d(k, grid, cfg.base, cfg.pairs)
    s = oracle.block_scores(oracle.block_mean(qr, cfg.block), oracle.block_mean(kr, cfg.block))
    idx, _, _ = oracle.topk_blocks(s, cfg.keep)
    if cfg.lr_mode == "rola":
        u = oracle.lowrank_features(k, p["wk"][0], grid, fmap=cfg.fmap)
        w = oracle.lowrank_features(q, p["wq"][0], grid, fmap=cfg.fmap)
        fk = oracle.lowrank_rotate(u, grid, cfg.base, cfg.pairs, cfg.lr_pairs)
        fq = oracle.lowrank_rotate(w, grid, cfg.base, cfg.pairs, cfg.lr_pairs)
    else:
        u = oracle.lowrank_features(k, p["wk"][0], grid, E, fmap=cfg.fmap)
        w = oracle.lowrank_features(q, p["wq"][0], grid, E, fmap=cfg.fmap)
        fk, fq = u, w
    S, z = oracle.lowrank_summary(fk, u, v)
    t1 = time.perf_counter()
    rows = (qblocks[:, None].astype(np.int64) * cfg.block + np.arange(cfg.block)[None, :]).reshape(-1)
    rows = rows[rows < cfg.L]
    oracle.block_sparse_attention(qr, kr, v, cfg.block, idx, qblocks)
    o_lr = oracle.lowrank_readout(fq, w, S, z, cfg.eps, rows, count=float(cfg.L) if cfg.fmap == "silu" else 0.0)
    if cfg.gate == "token":
        o_sp = np.zeros_like(o_lr)   # the gate's cost does not depend on the values
        oracle.token_gate(q[rows], p["wg"][0], float(p["bg"][0]), o_sp, o_lr, cfg.eps)
    t2 = time.perf_counter()
    per_slice = (t1 - t0) + (t2 - t1) * cfg.nblk / len(qblocks)
    layer_s = per_slice * cfg.B * cfg.H
    return layer_s, {"measured_s": round(t2 - t0, 2), "sampled_blocks": int(len(qblocks))}


def cpu_backward_baseline(cfg, blocks: int):
    """The oracle's backward (numpy fp64, BLAS held to one thread) on one
    (b, h) slice: the whole low-rank backward plus the sparse backward of
    `blocks` sampled query blocks (their dq and their keys' dk, dv), the
    selection held as the oracle's, extrapolated linearly to the layer."""
    import oracle
    from oracle import backward as OB
    from sparse_rank_attention_rope3d_amd import synth
    from threadpoolctl import threadpool_limits
    q, k, v = synth.qkv_slice(cfg, 0, 0)
    p = synth.lowrank_params(cfg)
    E = (p["et"], p["eh"], p["ew"]) if cfg.lr_mode == "abspe" else None
    dout = np.asarray(synth.dout_slice(cfg, 0, 0), np.float64)
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    qr = oracle.rope3d(q, grid, cfg.base, cfg.pairs)
    kr = oracle.rope3d(k, grid, cfg.base, cfg.pairs)
    idx, _, _ = oracle.topk_blocks(oracle.block_scores(oracle.block_mean(qr, cfg.block),
                                                       oracle.block_mean(kr, cfg.block)), cfg.keep)
    rng = np.random.default_rng([cfg.seed, synth.TID_SAMPLE, 0, 1])
    qblocks = np.sort(rng.choice(cfg.nblk, size=min(blocks, cfg.nblk), replace=False))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        OB.lowrank_bwd(cfg, q, k, v, p["wq"][0], p["wk"][0], float(p["gate"][0]) * dout, E=E)
        t1 = time.perf_counter()
        OB.sparse_attention_bwd(qr, kr, v, cfg.block, idx, dout, qblocks=qblocks)
        t2 = time.perf_counter()
    per_slice = (t1 - t0) + (t2 - t1) * cfg.nblk / len(qblocks)
    return per_slice * cfg.B * cfg.H, {"measured_s": round(t2 - t0, 2), "sampled_blocks": int(len(qblocks))}


def _time_ms(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_sweep(args, torch, B, synth):
    """Keep fraction x rank sweep at the Wan2.1-1.3B shape: layer time of
    every point and the dense kernel's time on the same inputs."""
    points = synth.sweep()
    base = points[0]
    q, k, v, _ = make_device_inputs(base, torch)
    shape, rope = B.shape_of(base), B.rope_of(base)
    wsd = B.workspace(B.slr_workspace_bytes(B.SLR_OP_DENSE, shape, rope), "cuda")
    out = torch.empty_like(q)
    dense_ms = _time_ms(torch, lambda: B.slr_dense_attention_fwd(q, k, v, shape, rope, out=out, ws=wsd), 3)
    del wsd
    rows = []
    for cfg in points:
        params = {kk: torch.from_numpy(vv).cuda() for kk, vv in synth.lowrank_params(cfg).items()}
        sparse, lowrank = B.sparse_of(cfg), B.lowrank_of(cfg, params)
        ws = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lowrank), "cuda")
        ms = _time_ms(torch, lambda: B.slr_attention_fwd(q, k, v, shape, rope, sparse, lowrank, out=out, ws=ws),
                      args.steps)
        F = cfg.flops()
        row = {"keep": cfg.keep, "keep_pct": round(100.0 * cfg.keep / cfg.nblk, 1), "rank": cfg.rank,
               "layer_ms": round(ms, 4), "dense_ms": round(dense_ms, 3), "speedup_vs_dense": round(dense_ms / ms, 2),
               "effective_tflops": round((F["sparse"] + F["lowrank"] + F["select"]) / (ms * 1e-3) / 1e12, 1)}
        if args.bwd_reps > 0:
            # the layer backward at this point (the training forward saves what it needs)
            saved = B.slr_attention_fwd_train(q, k, v, shape, rope, sparse, lowrank, ws=ws)
            wsb = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lowrank), "cuda")
            dout = torch.ones_like(q)
            grads = B.slr_attention_bwd(q, k, v, saved[1], saved[2], saved[3], dout, shape, rope, sparse, lowrank,
                                        ws=wsb)
            bms = _time_ms(torch, lambda: B.slr_attention_bwd(q, k, v, saved[1], saved[2], saved[3], dout, shape,
                                                              rope, sparse, lowrank, ws=wsb, grads=grads),
                           args.bwd_reps)
            row["backward_ms"] = round(bms, 3)
            row["backward_tflops"] = round((2.5 * F["sparse"] + 22.0 * cfg.B * cfg.H * cfg.L * cfg.D * cfg.rank)
                                           / (bms * 1e-3) / 1e12, 1)
            del saved, wsb, grads, dout
        rows.append(row)
        print(f"[sweep] {row}", file=sys.stderr, flush=True)
        del ws
    with open(args.sweep, "w") as f:
        for row in rows:
            f.write(json.dumps(row) + "\n")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan13b", choices=["wan13b", "wan14b", "hunyuan13b"])
    ap.add_argument("--gate", default="head", choices=["head", "token"],
                    help="combine gate: one scalar per head (the workloads' default) or the token-wise gate")
    ap.add_argument("--fmap", default="elu1", choices=["elu1", "silu"],
                    help="low-rank feature map: elu + 1 (the workloads' default) or SiLU")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--bwd-reps", type=int, default=3,
                    help="timed calls of the layer backward (training forward saves idx, O_sparse, lse); 0 skips")
    ap.add_argument("--cpu-blocks", type=int, default=512, help="query blocks the CPU oracle samples")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", metavar="JSONL", default=None,
                    help="time every keep-fraction x rank point of the Wan2.1-1.3B sweep against the dense "
                         "kernel, write one JSON object per point to JSONL and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; used to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus} GPUs, world size {world}): "
              "the layer shards over (batch, head) with no exchange, so there is no multi-GPU path to time.",
              file=sys.stderr)
        return 2

    import torch
    from sparse_rank_attention_rope3d_amd import binding as B
    from sparse_rank_attention_rope3d_amd import synth

    if args.calibrate_copy:
        n = args.calibrate_copy * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "reps": 3}))
        return 0

    if args.sweep:
        return run_sweep(args, torch, B, synth)

    cfg = synth.by_name(args.workload)
    if args.gate != "head" or args.fmap != "elu1":
        import dataclasses
        cfg = dataclasses.replace(cfg, gate=args.gate, fmap=args.fmap)
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v, params = make_device_inputs(cfg, torch)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, params)
    ws = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lowrank), "cuda")
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    hip = _hip()
    events = [[_event(hip) for _ in range(5)] for _ in range(args.steps)]
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        B.slr_attention_fwd(q, k, v, shape, rope, sparse, lowrank, out=out, ws=ws)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        B.slr_attention_fwd(q, k, v, shape, rope, sparse, lowrank, out=out, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # stage times from the same number of steps of the staged call (its event
    # records add a few microseconds between stages, so it is not the headline)
    print(f"[bench] {args.steps} staged steps for the stage times", file=sys.stderr, flush=True)
    for i in range(args.steps):
        B.slr_attention_fwd_staged(q, k, v, shape, rope, sparse, lowrank, out, ws, events[i])
    torch.cuda.synchronize()
    stage_names = ["rope_pool", "select", "lowrank_summary", "sparse_flash"]
    stages = {n: [] for n in stage_names}
    for ev in events:
        for j, n in enumerate(stage_names):
            stages[n].append(_elapsed(hip, ev[j], ev[j + 1]))
    stage_ms = {n: float(np.mean(vs)) for n, vs in stages.items()}

    F = cfg.flops()
    f_total = F["sparse"] + F["lowrank"] + F["select"]
    tflops = f_total / (ms_step * 1e-3) / 1e12
    flash_ms = stage_ms["sparse_flash"]
    flash_tf = F["sparse"] / (flash_ms * 1e-3) / 1e12
    es = 2 if cfg.dtype == "bf16" else 4
    BHLD = cfg.B * cfg.H * cfg.L * cfg.D
    rows_pad = cfg.B * cfg.H * cfg.nblk * cfg.block * cfg.D
    # rotate + pool: read q, k (and v, for the [K | V^T] tiles of the bf16 D=128 path), write the
    # rotated q, the k and V^T tiles (or rotated k) and the block means
    tiled = cfg.dtype == "bf16" and cfg.D == 128 and cfg.block == 64
    n_io = 3 if tiled else 2
    rope_bytes = n_io * BHLD * es + n_io * rows_pad * es + 2 * cfg.B * cfg.H * cfg.nblk * cfg.D * 4
    summ_bytes = 2 * BHLD * es
    hbm = {
        "rope_pool": {"GB/s": rope_bytes / (stage_ms["rope_pool"] * 1e-3) / 1e9},
        "lowrank_summary": {"GB/s": summ_bytes / (stage_ms["lowrank_summary"] * 1e-3) / 1e9},
    }
    for d in hbm.values():
        d["frac"] = d["GB/s"] / PEAK_HBM_GBS
        d["GB/s"] = round(d["GB/s"], 1)
        d["frac"] = round(d["frac"], 4)
    sel_tf = F["select"] / (stage_ms["select"] * 1e-3) / 1e12

    # in-library dense flash attention (RoPE inside) at the same shape
    dense = None
    if args.dense_reps > 0:
        print("[bench] dense flash baseline", file=sys.stderr, flush=True)
        wsd = B.workspace(B.slr_workspace_bytes(B.SLR_OP_DENSE, shape, rope), "cuda")
        B.slr_dense_attention_fwd(q, k, v, shape, rope, out=out, ws=wsd)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_reps):
            B.slr_dense_attention_fwd(q, k, v, shape, rope, out=out, ws=wsd)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.dense_reps
        dtf = F["dense"] / (dms * 1e-3) / 1e12
        dense = {"ms": round(dms, 3), "TFLOP/s": round(dtf, 1), "frac_bf16_peak": round(dtf / PEAK_BF16_TFLOPS, 4),
                 "speedup_of_slr_layer": round(dms / ms_step, 2)}
        del wsd

    # layer backward (bf16 layers): the training
    # forward saves the selection, O_sparse and the row normalisers once, then
    # the backward is timed on a seeded N(0, 1) output gradient
    backward = None
    if args.bwd_reps > 0 and cfg.dtype == "bf16":
        print("[bench] layer backward", file=sys.stderr, flush=True)
        gen = torch.Generator(device="cuda").manual_seed(1234)
        dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        saved = B.slr_attention_fwd_train(q, k, v, shape, rope, sparse, lowrank, ws=ws)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.bwd_reps):
            B.slr_attention_fwd_train(q, k, v, shape, rope, sparse, lowrank, ws=ws, outs=saved)
        e1.record()
        torch.cuda.synchronize()
        fwd_train_ms = e0.elapsed_time(e1) / args.bwd_reps
        _, idx_s, osp_s, lse_s = saved
        wsb = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lowrank), "cuda")
        grads = B.slr_attention_bwd(q, k, v, idx_s, osp_s, lse_s, dout, shape, rope, sparse, lowrank, ws=wsb)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.bwd_reps):
            B.slr_attention_bwd(q, k, v, idx_s, osp_s, lse_s, dout, shape, rope, sparse, lowrank, ws=wsb,
                                grads=grads)
        e1.record()
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / args.bwd_reps
        # algorithmic: S recomputed once, dP, dV, dK, dQ = 5 products of the
        # forward's 2 over the kept tiles; low-rank: 11 (D x r) products per token
        f_bsp = 2.5 * F["sparse"]
        f_blr = 22.0 * cfg.B * cfg.H * cfg.L * cfg.D * cfg.rank
        btf = (f_bsp + f_blr) / (bms * 1e-3) / 1e12
        backward = {"ms": round(bms, 3), "TFLOP/s (algorithmic)": round(btf, 1),
                    "frac_bf16_peak": round(btf / PEAK_BF16_TFLOPS, 4),
                    "algorithmic_flops": {"sparse": f_bsp, "lowrank": f_blr},
                    "training_forward_ms": round(fwd_train_ms, 3),
                    "training_step_ms": round(fwd_train_ms + bms, 3)}
        if not args.no_cpu_baseline:
            print("[bench] CPU oracle baseline of the backward", file=sys.stderr, flush=True)
            bs_s, binfo = cpu_backward_baseline(cfg, max(1, args.cpu_blocks // 16))
            backward["cpu_baseline"] = {
                "value": (f_bsp + f_blr) / bs_s / 1e12, "unit": "TFLOP/s (algorithmic)", "cores": 1,
                "kind": "oracle", "ms_per_layer": round(bs_s * 1e3, 1),
                "sample": f"one (b,h) slice of {cfg.B * cfg.H}: the whole low-rank backward and the sparse backward "
                          f"of {binfo['sampled_blocks']} of {cfg.nblk} query blocks, numpy fp64 with BLAS on one "
                          f"thread, {binfo['measured_s']} s measured, extrapolated linearly to the layer"}
        del wsb, grads, saved, dout

    print("[bench] achievable GEMM and copy rates", file=sys.stderr, flush=True)
    ach = achievable_peaks(torch)
    for d in hbm.values():
        d["frac_of_copy"] = round(d["GB/s"] / ach["copy_GB/s"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        layer_s, info = cpu_baseline(cfg, args.cpu_blocks)
        cpu = {"value": f_total / layer_s / 1e12, "unit": "TFLOP/s (effective)", "cores": 1, "kind": "oracle",
               "ms_per_layer": round(layer_s * 1e3, 1),
               "sample": f"one (b,h) slice of {cfg.B * cfg.H}: full selection and summary, "
                         f"{info['sampled_blocks']} of {cfg.nblk} query blocks of the sparse branch and readout, "
                         f"fp64 single thread, {info['measured_s']} s measured, extrapolated linearly to the layer"}

    line = {
        "metric": "SLR attn fwd ms/layer + effective TFLOP/s at L=32760/75600/118800, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s (effective)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded clustered Q/K, Gaussian V; random-init projections)",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "D": cfg.D, "L": cfg.L,
                   "grid": [cfg.T, cfg.Hg, cfg.Wg], "block": cfg.block, "keep": cfg.keep, "nblk": cfg.nblk,
                   "rank": cfg.rank, "lowrank": cfg.lr_mode, "gate": cfg.gate, "fmap": cfg.fmap,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "k_flash_tiled (block-sparse flash + low-rank readout + combine)",
                     "bound": "mfma", "achieved": round(flash_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flash_tf / PEAK_BF16_TFLOPS, 4), "traffic": flash_traffic(args.workload),
                     "algorithmic_flops_per_launch": F["sparse"], "avg_launch_ms": round(flash_ms, 4),
                     "frac_of_achievable_gemm": round(flash_tf / ach["gemm_bf16_TFLOP/s"], 4)},
        "achievable": ach,
        "stages_ms": {n: round(vv, 4) for n, vv in stage_ms.items()},
        "hbm_stages": hbm,
        "select": {"TFLOP/s": round(sel_tf, 2), "frac_fp32_peak": round(sel_tf / PEAK_FP32_TFLOPS, 4)},
        "dense_flash": dense,
        "backward": backward,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))
    for ev in events:
        for e in ev:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the 3D-RoPE sparse + low-rank attention layer forward on one
MI355X: ms/layer and effective TFLOP/s, with the dominant kernel's roofline,
per-stage times and their HBM rooflines, the in-library dense flash kernel,
the layer backward and the CPU oracle.

    python bench.py [--steps K] [--warmup W] [--workload wan14b|wan13b|hunyuan13b]
                    [--sub wan13b,hunyuan13b] [--sweep JSONL]

One step = one slr_attention_fwd over the whole layer (rotate + pool, block
top-k, low-rank summary, block-sparse flash + low-rank readout + gated
combine). Inputs are seeded synthetic layers already resident in HBM. The
headline is the Wan2.1-14B layer at 720p, 81 frames (L = 75600); the
Wan2.1-1.3B (L = 32760) and HunyuanVideo-13B (L = 118800) layers are timed
the same way as sub-records. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "SLR attn fwd ms/layer + effective TFLOP/s at L=32760/75600/118800, 1 GPU"

# HBM bytes per launch of the sparse flash kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch, scaled x2 and x1 by what the same counters read
# for a plain 1 GiB copy). They hold only for the kernel source they were taken
# on, identified by the sha256 of its files; any other source reports null.
FLASH_TRAFFIC_SOURCES = ["k_flash.hip", "slr_common.h", "slr_launch.h"]
FLASH_TRAFFIC = {
    "sha256": "c5d34a9a56f37494d5ba0a4dfc70b6437c38dc85473e3a3387bcf7494e636513",
    "bytes_per_launch": {"wan13b": 8203.9e6 + 201.3e6, "wan14b": 218434.0e6 + 1548.4e6,
                         "hunyuan13b": 195059.5e6 + 730.2e6},
}
GEN_THREADS = 8   # input generation: numpy fills each slice's arrays without the GIL


def flash_traffic(workload: str):
    if workload is None:
        return None
    csrc = os.path.join(ROOT, "sparse_rank_attention_rope3d_amd", "csrc")
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


def _pmc_child(counters, workload: str, timeout_s: int):
    """Rows of run_counter_collection.csv of this script's `--pmc-probe`
    child under `rocprofv3 --pmc <counters>`, or an error string."""
    import csv
    import shutil
    import subprocess
    import tempfile
    prof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(prof):
        return "rocprofv3 not found"
    tmp = os.environ.get("TMPDIR") or "/tmp"
    out = tempfile.mkdtemp(prefix="slr_pmc_", dir=tmp)
    cmd = ["timeout", "-s", "KILL", str(timeout_s), prof, "--pmc", *counters, "--output-format", "csv", "-d", out,
           "-o", "run", "--", sys.executable, os.path.abspath(__file__), "--pmc-probe", workload]
    try:
        r = subprocess.run(cmd, cwd=ROOT, env=dict(os.environ, TMPDIR=tmp), capture_output=True, text=True,
                           timeout=timeout_s + 30)
    except (OSError, subprocess.TimeoutExpired) as e:
        shutil.rmtree(out, ignore_errors=True)
        return f"{' '.join(counters)} run failed: {e}"
    path = os.path.join(out, "run_counter_collection.csv")
    rows = None
    if os.path.exists(path):
        with open(path) as f:
            rows = list(csv.DictReader(f))
    shutil.rmtree(out, ignore_errors=True)
    return rows if rows else f"{' '.join(counters)} run wrote no counters (exit {r.returncode})"


def _is_flash(name: str) -> bool:
    # the layer's sparse instance (not the dense one): k_flash_tiled<RP, LR, false, FAV>
    return name.startswith("void slr::k_flash_tiled<") and ", false, false>" in name


def counters_from_rows(fetch_rows, write_rows, sq_rows):
    """Numbers of live_counters from the counter rows of its three child
    runs (each a list of run_counter_collection.csv rows, or an error
    string): (traffic bytes or None, traffic detail, mfma dict or None,
    counted bytes of the HBM-bound stage kernels or None)."""
    copy_kib = 2 ** 30 / 1024
    per = {}
    stage_bytes = {}   # HBM-bound stage kernels: counted bytes per launch, read + written
    tdetail = None
    for counter, rows in (("FETCH_SIZE", fetch_rows), ("WRITE_SIZE", write_rows)):
        if isinstance(rows, str):
            tdetail = rows
            break
        flash = [float(r["Counter_Value"]) for r in rows if _is_flash(r["Kernel_Name"])]
        copies = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        if not flash or len(copies) < 3:
            tdetail = f"{counter}: flash or copy dispatches missing in the counters"
            break
        cal = copy_kib / (sum(sorted(copies)[-3:]) / 3)   # bytes moved per counted KiB, in KiB
        per[counter] = {"KiB_per_launch": round(sum(flash) / len(flash), 1), "scale": round(cal, 4),
                        "bytes": sum(flash) / len(flash) * cal * 1024}
        for stage, prefix in (("rope_pool", "slr::k_rope_pool<"), ("lowrank_summary", "slr::k_lr_summary_bf16")):
            # template instances are listed as "void slr::...", plain kernels as "slr::..."
            v = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].removeprefix("void ").startswith(prefix)]
            if v:
                stage_bytes[stage] = stage_bytes.get(stage, 0.0) + sum(v) / len(v) * cal * 1024
    tb = None
    if len(per) == 2:
        tb = per["FETCH_SIZE"]["bytes"] + per["WRITE_SIZE"]["bytes"]
        tdetail = {"source": "rocprofv3 --pmc child runs of this script (3 launches each; 1 GiB copies calibrate)",
                   "fetch_bytes": round(per["FETCH_SIZE"]["bytes"]), "write_bytes": round(per["WRITE_SIZE"]["bytes"]),
                   "counters": per}
    mfma = None
    if not isinstance(sq_rows, str):
        disp = {}
        for r in sq_rows:
            if _is_flash(r["Kernel_Name"]):
                d = disp.setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
                d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        fr = [(d["SQ_VALU_MFMA_BUSY_CYCLES"] * 8 / (1024 * d["GRBM_COUNT"]), d["GRBM_COUNT"] / 8 / d["ns"] * 1e3)
              for d in disp.values() if d.get("GRBM_COUNT") and "SQ_VALU_MFMA_BUSY_CYCLES" in d and d["ns"] > 0]
        if fr:
            mfma = {"busy_frac": round(sum(f for f, _ in fr) / len(fr), 4),
                    "clock_MHz": round(sum(c for _, c in fr) / len(fr)),
                    "what": "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_COUNT / 8): the fraction of SIMD "
                            "cycles the matrix cores were busy, at the shader clock the kernel ran at "
                            "(rocprofv3 --pmc child run, 3 launches)"}
    return tb, tdetail, mfma, (stage_bytes if len(per) == 2 else None)


def live_counters(workload: str, timeout_s: int = 90):
    """The headline flash kernel, counted in this run by child processes of
    this script (`--pmc-probe`: 1 + 2 layer forwards of the workload, then
    three 1 GiB device copies) under rocprofv3 --pmc:
      traffic: FETCH_SIZE and WRITE_SIZE (one run each), each scaled by what
        it reads for the copies in the same process -> HBM bytes per launch;
      MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x shader cycles),
        shader cycles = GRBM_COUNT / 8 XCDs (duration x clock)."""
    # after any failed run the rest are skipped (a profiler that fails once costs one time limit at most)
    fetch = _pmc_child(["FETCH_SIZE"], workload, timeout_s)
    write = _pmc_child(["WRITE_SIZE"], workload, timeout_s) if not isinstance(fetch, str) else fetch
    sq = (_pmc_child(["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_COUNT"], workload, timeout_s)
          if not isinstance(write, str) else write)
    return counters_from_rows(fetch, write, sq)


def pmc_probe(workload: str, torch, B) -> int:
    """The counted child of live_counters: 1 + 2 layer forwards of the
    workload, then three 1 GiB device copies."""
    from sparse_rank_attention_rope3d_amd import synth
    cfg = synth.by_name(workload)
    q, k, v, params = make_device_inputs(cfg, torch)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, params)
    ws = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lowrank), "cuda")
    out = torch.empty_like(q)
    for _ in range(3):
        B.slr_attention_fwd(q, k, v, shape, rope, sparse, lowrank, out=out, ws=ws)
    torch.cuda.synchronize()
    del q, k, v, ws, out
    src = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": workload}))
    return 0


def host_cpu() -> dict:
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"model": model, "nproc": usable, "logical_cpus": os.cpu_count()}


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
    out = {"gemm_bf16_TFLOP/s": round(gemm_tf, 1), "copy_GB/s": round(copy_gbs, 1),
           "what": "8192^3 bf16 torch.matmul on random operands; 1 GiB device copy, read + write bytes"}
    mf = mfma_loop_rate(torch)
    if mf is not None:
        out["mfma_loop_bf16_TFLOP/s"] = mf
        out["what"] += ("; an MFMA-only loop (libslr_probe.so: eight independent 32x32x16 bf16 chains per wave on "
                        "register operands of varying non-zero values)")
    return out


def mfma_loop_rate(torch):
    """The bf16 MFMA issue rate with operands in registers (no memory, no
    other instructions in the loop), at the clock the part holds under
    that load."""
    path = os.path.join(ROOT, "sparse_rank_attention_rope3d_amd", "libslr_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.slrprobe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.slrprobe_mfma_loop.restype = ctypes.c_int
    nwg, iters = 2048, 2000
    sink = torch.empty(nwg * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda: lib.slrprobe_mfma_loop(nwg, iters, ctypes.c_void_p(sink.data_ptr()), stream)
    for _ in range(3):
        assert call() == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        assert call() == 0
    e1.record()
    torch.cuda.synchronize()
    flops = 32768.0 * 8 * iters * 4 * nwg * reps
    del sink
    return round(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)


def memory_read_probe(torch) -> dict:
    """Read-only streaming rate of a buffer from 8 MB to 4 GiB (the XCDs'
    L2s hold 32 MB, the memory-side cache 256 MB), with ordinary vector
    loads and with the direct global -> LDS copies the flash kernel uses
    (libslr_probe.so)."""
    path = os.path.join(ROOT, "sparse_rank_attention_rope3d_amd", "libslr_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.slrprobe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.slrprobe_stream_read.restype = ctypes.c_int
    nwg = 2048
    sink = torch.empty(nwg * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    big = torch.ones(4 * 2 ** 30, dtype=torch.uint8, device="cuda")
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for mb in (8, 16, 32, 48, 64, 80, 96, 128, 160, 256, 512, 1024, 4096):
        nbytes = mb * 2 ** 20
        passes = max(1, (8 * 2 ** 30) // nbytes)
        for to_lds in (0, 1):
            call = lambda: lib.slrprobe_stream_read(ctypes.c_void_p(big.data_ptr()), nbytes, passes, to_lds, nwg,
                                                    ctypes.c_void_p(sink.data_ptr()), stream)
            assert call() == 0
            torch.cuda.synchronize()
            reps = 3
            e0.record()
            for _ in range(reps):
                assert call() == 0
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes * passes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
            out[f"{mb}MB_{'to_lds' if to_lds else 'vgpr'}_GB/s"] = round(gbs, 1)
    del big, sink
    out["what"] = ("read-only stream, 2048 workgroups x 256 threads, 16-byte loads, each XCD touching one eighth "
                   "of the buffer; up to 32 MB it fits the XCDs' L2s, up to 256 MB the memory-side cache, beyond "
                   "that only HBM")
    return out


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


def _slice_arrays(cfg, b, h):
    from sparse_rank_attention_rope3d_amd import synth
    arrs = synth.qkv_slice(cfg, b, h)
    if cfg.dtype == "bf16":
        return [synth.f32_to_bf16_bits(a).view(np.int16) for a in arrs]
    return list(arrs)


def make_device_inputs(cfg, torch, threads: int = GEN_THREADS):
    """q, k, v [B, H, L, D] on the device from the seeded per-slice
    generators (slices drawn on `threads` host threads), and the low-rank
    parameters."""
    from sparse_rank_attention_rope3d_amd import synth
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shp = (cfg.B, cfg.H, cfg.L, cfg.D)
    q, k, v = (torch.empty(shp, dtype=tdt, device="cuda") for _ in range(3))
    slices = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    with cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for n, ((b, h), arrs) in enumerate(zip(slices, ex.map(lambda bh: _slice_arrays(cfg, *bh), slices))):
            for dst, arr in zip((q, k, v), arrs):
                t = torch.from_numpy(arr)
                dst[b, h] = (t.view(torch.bfloat16) if cfg.dtype == "bf16" else t).cuda()
            if (n + 1) % 20 == 0:
                print(f"[bench]   {n + 1}/{len(slices)} slices on the device", file=sys.stderr, flush=True)
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
    om = p["omega"][0] if cfg.fmap == "favor" else None
    if cfg.lr_mode == "rola":
        u = oracle.lowrank_features(k, p["wk"][0], grid, fmap=cfg.fmap, omega=om)
        w = oracle.lowrank_features(q, p["wq"][0], grid, fmap=cfg.fmap, omega=om)
        fk = oracle.lowrank_rotate(u, grid, cfg.base, cfg.pairs, cfg.lr_pairs)
        fq = oracle.lowrank_rotate(w, grid, cfg.base, cfg.pairs, cfg.lr_pairs)
    else:
        u = oracle.lowrank_features(k, p["wk"][0], grid, E, fmap=cfg.fmap, omega=om)
        w = oracle.lowrank_features(q, p["wq"][0], grid, E, fmap=cfg.fmap, omega=om)
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
        OB.lowrank_bwd(cfg, q, k, v, p["wq"][0], p["wk"][0], float(p["gate"][0]) * dout, E=E,
                       omega=p["omega"][0] if cfg.fmap == "favor" else None)
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
    every point and the dense kernel's time on the same inputs. One JSON
    line per point is appended to the file as soon as the point is done; a
    rerun keeps the points the file already holds and starts at the first
    missing one."""
    points = synth.sweep()
    done = set()
    if os.path.exists(args.sweep):
        with open(args.sweep) as f:
            for ln in f:
                ln = ln.strip()
                if not ln:
                    continue
                try:
                    row = json.loads(ln)
                except json.JSONDecodeError:
                    continue   # a line cut short by an interrupted run: that point runs again
                done.add((row["keep"], row["rank"]))
    todo = [p for p in points if (p.keep, p.rank) not in done]
    print(f"[sweep] {len(done)} of {len(points)} points already in {args.sweep}", file=sys.stderr, flush=True)
    if not todo:
        return 0
    base = points[0]
    q, k, v, _ = make_device_inputs(base, torch)
    shape, rope = B.shape_of(base), B.rope_of(base)
    wsd = B.workspace(B.slr_workspace_bytes(B.SLR_OP_DENSE, shape, rope), "cuda")
    out = torch.empty_like(q)
    dense_ms = _time_ms(torch, lambda: B.slr_dense_attention_fwd(q, k, v, shape, rope, out=out, ws=wsd), 3)
    del wsd
    for cfg in todo:
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
            # the layer backward at this point (the training forward saves what it needs, the summary included)
            summ = (torch.empty((cfg.B, cfg.H, cfg.rank, cfg.D), dtype=torch.float32, device="cuda"),
                    torch.empty((cfg.B, cfg.H, cfg.rank), dtype=torch.float32, device="cuda"))
            saved = B.slr_attention_fwd_train(q, k, v, shape, rope, sparse, lowrank, ws=ws, summary=summ)
            wsb = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lowrank), "cuda")
            dout = torch.ones_like(q)
            grads = B.slr_attention_bwd(q, k, v, saved[1], saved[2], saved[3], dout, shape, rope, sparse, lowrank,
                                        ws=wsb, summary=summ)
            bms = _time_ms(torch, lambda: B.slr_attention_bwd(q, k, v, saved[1], saved[2], saved[3], dout, shape,
                                                              rope, sparse, lowrank, ws=wsb, grads=grads,
                                                              summary=summ),
                           args.bwd_reps)
            row["backward_ms"] = round(bms, 3)
            row["backward_tflops"] = round((2.5 * F["sparse"] + 22.0 * cfg.B * cfg.H * cfg.L * cfg.D * cfg.rank)
                                           / (bms * 1e-3) / 1e12, 1)
            del saved, wsb, grads, dout, summ
        with open(args.sweep, "a") as f:
            f.write(json.dumps(row) + "\n")
        print(f"[sweep] {row}", file=sys.stderr, flush=True)
        del ws
    return 0


def layer_roofline(cfg, F, es, ms) -> dict:
    """Ideal layer time at the published peaks: for each stage the larger of
    its algorithmic FLOPs at the bf16 MFMA peak and its algorithmic bytes at
    the HBM peak, summed over rotate + pool + select (read q, k, write the
    rotated copies and the kept indices), the low-rank summary (read k, v),
    the sparse flash attention (F_sparse) and the low-rank apply + combine
    (read q and O_sparse, write O; fused into the flash kernel here, counted
    as its own stage so the ideal does not depend on the fusion); and the
    measured time's fraction of it."""
    BHLD = cfg.B * cfg.H * cfg.L * cfg.D
    idx_bytes = 4 * cfg.B * cfg.H * cfg.nblk * cfg.keep
    f_lr_half = 4.0 * cfg.B * cfg.H * cfg.L * cfg.rank * cfg.D
    stages = {
        "rotate_pool_select": (F["select"], 4 * BHLD * es + idx_bytes),
        "lowrank_summary": (f_lr_half, 2 * BHLD * es),
        "sparse_flash": (F["sparse"], 0),
        "lowrank_apply_combine": (f_lr_half, 3 * BHLD * es),
    }
    terms = {n: max(f / (PEAK_BF16_TFLOPS * 1e12), b / (PEAK_HBM_GBS * 1e9)) * 1e3 for n, (f, b) in stages.items()}
    ideal = sum(terms.values())
    return {"ideal_ms": round(ideal, 4), "frac": round(ideal / ms, 4),
            "stage_ideal_ms": {n: round(v, 4) for n, v in terms.items()},
            "peaks": {"bf16_TFLOP/s": PEAK_BF16_TFLOPS, "hbm_GB/s": PEAK_HBM_GBS}}


def measure_forward(cfg, args, torch, B, hip, ach=None, dense_reps=0):
    """Time the layer forward of one workload: per-step times (hipEvents on
    the stream the library launches on) over `args.steps` plain forward
    calls, then the same number of staged calls for the stage times; the
    flash kernel's MFMA roofline and the HBM rooflines of the rotate + pool +
    select and summary stages. Returns (record, device inputs)."""
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v, params = make_device_inputs(cfg, torch)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, params)
    ws = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lowrank), "cuda")
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    fwd = lambda: B.slr_attention_fwd(q, k, v, shape, rope, sparse, lowrank, out=out, ws=ws)
    print(f"[bench] {cfg.name}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: timing {args.steps} steps", file=sys.stderr, flush=True)
    # between timed calls a 512 MB buffer is written (outside the timed
    # region), so no call starts with the previous call's data in the 256 MB
    # memory-side cache
    scrub = None if args.no_scrub else torch.empty(512 * 2 ** 20, dtype=torch.uint8, device="cuda")
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev0[i].record()
        fwd()
        ev1[i].record()
        if scrub is not None:
            scrub.fill_(i & 0xFF)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = np.array([ev0[i].elapsed_time(ev1[i]) for i in range(args.steps)])
    wall_ms = (t1 - t0) * 1e3 / args.steps
    # stage times from the same number of staged calls (their event records
    # add a few microseconds between stages, so they are not the headline)
    events = [[_event(hip) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        B.slr_attention_fwd_staged(q, k, v, shape, rope, sparse, lowrank, out, ws, events[i])
        if scrub is not None:
            scrub.fill_(i & 0xFF)
    torch.cuda.synchronize()
    del scrub
    stage_names = ["rope_pool", "select", "lowrank_summary", "sparse_flash"]
    stages = {n: [] for n in stage_names}
    for evs in events:
        for j, n in enumerate(stage_names):
            stages[n].append(_elapsed(hip, evs[j], evs[j + 1]))
    for evs in events:
        for e in evs:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    stage_ms = {n: float(np.mean(vs)) for n, vs in stages.items()}

    F = cfg.flops()
    f_total = F["sparse"] + F["lowrank"] + F["select"]
    ms_mean = float(step_ms.mean())
    flash_ms = stage_ms["sparse_flash"]
    flash_tf = F["sparse"] / (flash_ms * 1e-3) / 1e12
    es = 2 if cfg.dtype == "bf16" else 4
    BHLD = cfg.B * cfg.H * cfg.L * cfg.D
    rows_pad = cfg.B * cfg.H * cfg.nblk * cfg.block * cfg.D
    idx_bytes = 4 * cfg.B * cfg.H * cfg.nblk * cfg.keep
    # algorithmic bytes of the HBM-bound stages: rotate + pool + select
    # read q, k and write the rotated q, k (+ the kept indices); the summary
    # reads k, v; the low-rank apply + combine is fused into the flash kernel
    k1_bytes = 4 * BHLD * es + idx_bytes
    k2_bytes = 2 * BHLD * es
    k1_ms = stage_ms["rope_pool"] + stage_ms["select"]
    # what the rotate + pool kernel itself moves on the tiled path: it also
    # reads v and writes the [K | V^T] tiles and the block means
    tiled = cfg.dtype == "bf16" and cfg.D == 128 and cfg.block == 64
    n_io = 3 if tiled else 2
    own_bytes = n_io * BHLD * es + n_io * rows_pad * es + 2 * cfg.B * cfg.H * cfg.nblk * cfg.D * 4

    def hbm(nbytes, ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        d = {"GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes,
             "ms": round(ms, 4)}
        if ach:
            d["frac_of_copy"] = round(gbs / ach["copy_GB/s"], 4)
        return d

    rec = {
        "workload": cfg.name,
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "D": cfg.D, "L": cfg.L,
                   "grid": [cfg.T, cfg.Hg, cfg.Wg], "block": cfg.block, "keep": cfg.keep, "nblk": cfg.nblk,
                   "rank": cfg.rank, "lowrank": cfg.lr_mode, "gate": cfg.gate, "fmap": cfg.fmap,
                   "parallelism": "single GPU"},
        "ms_per_layer": {"mean": round(ms_mean, 4), "median": round(float(np.median(step_ms)), 4),
                         "min": round(float(step_ms.min()), 4), "max": round(float(step_ms.max()), 4),
                         ("wall_clock_mean" if args.no_scrub else "wall_clock_mean_incl_scrub"): round(wall_ms, 4),
                         "steps": args.steps, "scrub_between_calls_MB": 0 if args.no_scrub else 512,
                         "each_ms": [round(float(x), 3) for x in step_ms]},
        "effective_TFLOP/s": round(f_total / (ms_mean * 1e-3) / 1e12, 2),
        "effective_TFLOP/s_at_median": round(f_total / (float(np.median(step_ms)) * 1e-3) / 1e12, 2),
        "dense_equivalent_TFLOP/s": round(F["dense"] / (ms_mean * 1e-3) / 1e12, 1),
        "flops": {k_: float(v_) for k_, v_ in F.items()},
        "roofline": {"kernel": "k_flash_tiled (block-sparse flash + low-rank readout + combine)",
                     "bound": "mfma", "achieved": round(flash_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flash_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": flash_traffic(args_key(cfg)),
                     "algorithmic_flops_per_launch": F["sparse"], "avg_launch_ms": round(flash_ms, 4)},
        "stages_ms": {n: round(vv, 4) for n, vv in stage_ms.items()},
        "hbm_stages": {
            "rotate_pool_select": hbm(k1_bytes, k1_ms),
            "lowrank_summary": hbm(k2_bytes, stage_ms["lowrank_summary"]),
            "lowrank_apply_combine": "fused into the flash kernel's epilogue (no pass of its own)",
            "rotate_pool_kernel_own_traffic": hbm(own_bytes, stage_ms["rope_pool"]),
        },
        "select": {"TFLOP/s": round(F["select"] / (stage_ms["select"] * 1e-3) / 1e12, 2)},
        "layer_roofline": layer_roofline(cfg, F, es, ms_mean),
    }
    if ach:
        rec["roofline"]["frac_of_achievable_gemm"] = round(flash_tf / ach["gemm_bf16_TFLOP/s"], 4)
        if "mfma_loop_bf16_TFLOP/s" in ach:
            rec["roofline"]["frac_of_achievable_mfma"] = round(flash_tf / ach["mfma_loop_bf16_TFLOP/s"], 4)
    if dense_reps > 0:
        print(f"[bench] {cfg.name}: dense flash baseline", file=sys.stderr, flush=True)
        wsd = B.workspace(B.slr_workspace_bytes(B.SLR_OP_DENSE, shape, rope), "cuda")
        dms = _time_ms(torch, lambda: B.slr_dense_attention_fwd(q, k, v, shape, rope, out=out, ws=wsd), dense_reps)
        dtf = F["dense"] / (dms * 1e-3) / 1e12
        rec["dense_flash"] = {"ms": round(dms, 3), "TFLOP/s": round(dtf, 1),
                              "frac_bf16_peak": round(dtf / PEAK_BF16_TFLOPS, 4),
                              "speedup_of_slr_layer": round(dms / ms_mean, 2)}
        del wsd
    del ws, out
    return rec, (q, k, v, params, shape, rope, sparse, lowrank)


def args_key(cfg) -> str:
    """The short name of a stock workload (None for a modified one)."""
    from sparse_rank_attention_rope3d_amd import synth
    if cfg.gate != "head" or cfg.fmap != "elu1":
        return None
    for key in ("wan13b", "wan14b", "hunyuan13b"):
        if synth.by_name(key).name == cfg.name:
            return key
    return None


def measure_backward(cfg, args, torch, B, dev):
    """The layer backward (bf16): the training forward saves the selection,
    O_sparse, the row normalisers and the low-rank summary S, z once, then
    the backward is timed on a seeded N(0, 1) output gradient (and once
    more recomputing the summary itself)."""
    q, k, v, params, shape, rope, sparse, lowrank = dev
    print(f"[bench] {cfg.name}: layer backward", file=sys.stderr, flush=True)
    gen = torch.Generator(device="cuda").manual_seed(1234)
    dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    ws = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lowrank), "cuda")
    summ = (torch.empty((cfg.B, cfg.H, cfg.rank, cfg.D), dtype=torch.float32, device="cuda"),
            torch.empty((cfg.B, cfg.H, cfg.rank), dtype=torch.float32, device="cuda"))
    saved = B.slr_attention_fwd_train(q, k, v, shape, rope, sparse, lowrank, ws=ws, summary=summ)
    fwd_train_ms = _time_ms(torch, lambda: B.slr_attention_fwd_train(q, k, v, shape, rope, sparse, lowrank, ws=ws,
                                                                     outs=saved, summary=summ), args.bwd_reps)
    del ws
    _, idx_s, osp_s, lse_s = saved
    wsb = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lowrank), "cuda")
    grads = B.slr_attention_bwd(q, k, v, idx_s, osp_s, lse_s, dout, shape, rope, sparse, lowrank, ws=wsb,
                                summary=summ)
    bms = _time_ms(torch, lambda: B.slr_attention_bwd(q, k, v, idx_s, osp_s, lse_s, dout, shape, rope, sparse,
                                                      lowrank, ws=wsb, grads=grads, summary=summ), args.bwd_reps)
    bms_re = _time_ms(torch, lambda: B.slr_attention_bwd(q, k, v, idx_s, osp_s, lse_s, dout, shape, rope, sparse,
                                                         lowrank, ws=wsb, grads=grads), args.bwd_reps)
    F = cfg.flops()
    # algorithmic: S recomputed once, dP, dV, dK, dQ = 5 products of the
    # forward's 2 over the kept tiles; low-rank: 11 (D x r) products per token
    f_bsp = 2.5 * F["sparse"]
    f_blr = 22.0 * cfg.B * cfg.H * cfg.L * cfg.D * cfg.rank
    btf = (f_bsp + f_blr) / (bms * 1e-3) / 1e12
    rec = {"ms": round(bms, 3), "TFLOP/s (algorithmic)": round(btf, 1),
           "frac_bf16_peak": round(btf / PEAK_BF16_TFLOPS, 4),
           "algorithmic_flops": {"sparse": f_bsp, "lowrank": f_blr},
           "ms_recomputing_summary": round(bms_re, 3),
           "training_forward_ms": round(fwd_train_ms, 3),
           "training_step_ms": round(fwd_train_ms + bms, 3)}
    del wsb, grads, saved, dout, summ
    return rec


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan14b", choices=["wan13b", "wan14b", "hunyuan13b"],
                    help="headline workload (default: the Wan2.1-14B layer, L = 75600)")
    ap.add_argument("--sub", default="wan13b,hunyuan13b",
                    help="comma-separated workloads timed as sub-records ('' for none)")
    ap.add_argument("--no-scrub", action="store_true",
                    help="do not write the 512 MB scratch buffer between timed forward calls")
    ap.add_argument("--gate", default="head", choices=["head", "token"],
                    help="combine gate: one scalar per head (the workloads' default) or the token-wise gate")
    ap.add_argument("--fmap", default="elu1", choices=["elu1", "silu", "favor"],
                    help="low-rank feature map: elu + 1 (the workloads' default), SiLU or FAVOR+ random features")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--bwd-reps", type=int, default=3,
                    help="timed calls of the layer backward (training forward saves idx, O_sparse, lse); 0 skips")
    ap.add_argument("--cpu-blocks", type=int, default=0,
                    help="query blocks the CPU oracle samples (default: 64, 512 for the Wan2.1-1.3B layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the GEMM / copy / memory read probes")
    ap.add_argument("--sweep", metavar="JSONL", default=None,
                    help="time every keep-fraction x rank point of the Wan2.1-1.3B sweep against the dense "
                         "kernel, append one JSON object per point to JSONL (resuming after the points it "
                         "holds) and exit")
    ap.add_argument("--no-live-traffic", action="store_true",
                    help="report the flash kernel's stored HBM byte counts and skip its MFMA busy fraction "
                         "instead of counting both in three rocprofv3 --pmc child runs")
    ap.add_argument("--pmc-probe", default=None, help=argparse.SUPPRESS)
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

    if args.pmc_probe:
        return pmc_probe(args.pmc_probe, torch, B)

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

    def workload(name):
        cfg = synth.by_name(name)
        if args.gate != "head" or args.fmap != "elu1":
            import dataclasses
            cfg = dataclasses.replace(cfg, gate=args.gate, fmap=args.fmap)
        return cfg

    hip = _hip()
    cfg = workload(args.workload)
    head, dev = measure_forward(cfg, args, torch, B, hip, dense_reps=args.dense_reps)
    backward = None
    if args.bwd_reps > 0 and cfg.dtype == "bf16":
        backward = measure_backward(cfg, args, torch, B, dev)
    del dev
    torch.cuda.empty_cache()

    subs = []
    for name in [s for s in args.sub.split(",") if s and s != args.workload]:
        rec, dev = measure_forward(workload(name), args, torch, B, hip, dense_reps=args.dense_reps)
        subs.append(rec)
        del dev
        torch.cuda.empty_cache()

    ach = probe = None
    if not args.no_probe:
        print("[bench] achievable GEMM and copy rates, memory read probe", file=sys.stderr, flush=True)
        ach = achievable_peaks(torch)
        probe = memory_read_probe(torch)
        for rec in [head] + subs:
            rec["roofline"]["frac_of_achievable_gemm"] = round(rec["roofline"]["achieved"] / ach["gemm_bf16_TFLOP/s"],
                                                               4)
            if "mfma_loop_bf16_TFLOP/s" in ach:
                rec["roofline"]["frac_of_achievable_mfma"] = round(
                    rec["roofline"]["achieved"] / ach["mfma_loop_bf16_TFLOP/s"], 4)
            for st in rec["hbm_stages"].values():
                if isinstance(st, dict):
                    st["frac_of_copy"] = round(st["GB/s"] / ach["copy_GB/s"], 4)

    cpu = None
    f_total = head["flops"]["sparse"] + head["flops"]["lowrank"] + head["flops"]["select"]
    cpuinfo = host_cpu()
    if not args.no_cpu_baseline:
        blocks = args.cpu_blocks or (512 if cfg.nblk <= 512 else 64)
        print(f"[bench] CPU oracle baseline ({blocks} sampled query blocks of one slice)", file=sys.stderr,
              flush=True)
        layer_s, info = cpu_baseline(cfg, blocks)
        value = f_total / layer_s / 1e12
        n = cpuinfo["nproc"]
        cpu = {"value": value, "unit": "TFLOP/s (effective)", "cores": 1, "kind": "oracle",
               "ms_per_layer": round(layer_s * 1e3, 1),
               "sample": f"one (b,h) slice of {cfg.B * cfg.H} of {cfg.name}: full selection and summary, "
                         f"{info['sampled_blocks']} of {cfg.nblk} query blocks of the sparse branch and readout, "
                         f"fp64 single thread, {info['measured_s']} s measured, extrapolated linearly to the layer",
               "host_cpu": cpuinfo["model"], "nproc": n,
               "ideal_n_core": {"cores": n, "value": value * n, "ms_per_layer": round(layer_s * 1e3 / n, 1),
                                "what": "the single-thread figure times the usable cores (slices are independent)"}}
        if backward is not None:
            print("[bench] CPU oracle baseline of the backward", file=sys.stderr, flush=True)
            bs_s, binfo = cpu_backward_baseline(cfg, 4 if cfg.nblk > 512 else 32)
            fb = backward["algorithmic_flops"]["sparse"] + backward["algorithmic_flops"]["lowrank"]
            backward["cpu_baseline"] = {
                "value": fb / bs_s / 1e12, "unit": "TFLOP/s (algorithmic)", "cores": 1, "kind": "oracle",
                "ms_per_layer": round(bs_s * 1e3, 1), "host_cpu": cpuinfo["model"], "nproc": cpuinfo["nproc"],
                "sample": f"one (b,h) slice of {cfg.B * cfg.H}: the whole low-rank backward and the sparse backward "
                          f"of {binfo['sampled_blocks']} of {cfg.nblk} query blocks, numpy fp64 with BLAS on one "
                          f"thread, {binfo['measured_s']} s measured, extrapolated linearly to the layer"}

    # the headline flash kernel's HBM bytes, counted now (else the stored counts for this source)
    key = args_key(cfg)
    if key is not None and not args.no_live_traffic:
        print("[bench] HBM and MFMA counters of the flash kernel (three rocprofv3 --pmc child runs)",
              file=sys.stderr, flush=True)
        tb, detail, mfma, stage_bytes = live_counters(key)
        if tb is not None:
            head["roofline"]["traffic"] = round(tb)
            head["roofline"]["traffic_detail"] = detail
        else:
            head["roofline"]["traffic_detail"] = {"source": "stored counts for this kernel source "
                                                            f"(live counting unavailable: {detail})"}
        if mfma is not None:
            head["roofline"]["mfma_busy"] = mfma
        # counted bytes of the HBM-bound stage kernels (rotate + pool moves more than the stage's
        # algorithmic bytes by design: the V read and the [K | V^T] tile write)
        for stage, nb in (stage_bytes or {}).items():
            rec_key = "rotate_pool_kernel_own_traffic" if stage == "rope_pool" else "lowrank_summary"
            if isinstance(head["hbm_stages"].get(rec_key), dict):
                head["hbm_stages"][rec_key]["counted_bytes"] = round(nb)
    elif head["roofline"]["traffic"] is not None:
        head["roofline"]["traffic_detail"] = {"source": "stored counts for this kernel source"}

    ms = head["ms_per_layer"]["mean"]
    line = {
        "metric": METRIC,
        "value": head["effective_TFLOP/s"],
        "unit": "TFLOP/s (effective)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded clustered Q/K, Gaussian V; random-init projections)",
        "config": head["config"],
        "ms_per_layer": head["ms_per_layer"],
        "roofline": head["roofline"],
        "stages_ms": head["stages_ms"],
        "hbm_stages": head["hbm_stages"],
        "select": head["select"],
        "layer_roofline": head["layer_roofline"],
        "dense_flash": head.get("dense_flash"),
        "dense_equivalent_TFLOP/s": head["dense_equivalent_TFLOP/s"],
        "backward": backward,
        "cpu_baseline": cpu,
        "achievable": ach,
        "memory_read_probe": probe,
        "workloads": {r["config"]["workload"]: r for r in subs},
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())

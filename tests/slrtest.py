"""Helpers of the GPU parity tests: seeded inputs on the device, the oracle
on the same values, and the comparisons (selection within the near-tie
window, relative Frobenius and max-abs errors)."""
from __future__ import annotations

import dataclasses
import math
import sys
from typing import Dict, Iterable, List, Optional

import numpy as np
import torch

import oracle
from sparse_rank_attention_rope3d_amd import binding as B
from sparse_rank_attention_rope3d_amd import synth

WINDOW = 1e-5            # selection: scores this close to the k-th may go either way
TOL = {"bf16": dict(rel=1e-2, maxabs=3e-2), "f32": dict(rel=1e-5, maxabs=None)}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def custom(base: synth.Layer, **kw) -> synth.Layer:
    return dataclasses.replace(base, **kw)


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class Inputs:
    cfg: synth.Layer
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    params_np: Dict[str, np.ndarray]
    params: Dict[str, torch.Tensor]


def make_inputs(cfg: synth.Layer, device="cuda") -> Inputs:
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shp = (cfg.B, cfg.H, cfg.L, cfg.D)
    q, k, v = (torch.empty(shp, dtype=tdt, device=device) for _ in range(3))
    for b in range(cfg.B):
        for h in range(cfg.H):
            qs, ks, vs = synth.qkv_slice(cfg, b, h)
            q[b, h] = to_device(qs, cfg.dtype, device)
            k[b, h] = to_device(ks, cfg.dtype, device)
            v[b, h] = to_device(vs, cfg.dtype, device)
    pn = synth.lowrank_params(cfg)
    pd = {key: torch.from_numpy(val).to(device) for key, val in pn.items()}
    return Inputs(cfg, q, k, v, pn, pd)


def run_layer(inp: Inputs, debug=True):
    cfg = inp.cfg
    return B.slr_attention_fwd(inp.q, inp.k, inp.v, B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg),
                               B.lowrank_of(cfg, inp.params), debug=debug)


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (den if den > 0 else 1.0))


def max_abs(a: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(a - ref))) if a.size else 0.0


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, branch: bool = False) -> None:
    """Relative Frobenius and max-abs bars. ``branch``: a debug copy of one
    branch (O_sparse, O_lowrank; or the summary S, z) rather than the layer
    output; its values
    can be far larger than the output's (a rotated low-rank numerator over an
    un-rotated normaliser reaches ~10 with FAVOR+ features, where one bf16
    half-ulp is 0.031), so its max-abs bar is max(3e-2, 2^-6 max|ref|), about
    four bf16 half-ulps at its largest value."""
    t = TOL[dtype]
    rf, ma = rel_fro(got, ref), max_abs(got, ref)
    log(f"    {name}: rel_fro={rf:.3e} max_abs={ma:.3e}")
    assert rf <= t["rel"], f"{name}: relative Frobenius error {rf:.3e} > {t['rel']}"
    if t["maxabs"] is not None:
        bar = t["maxabs"]
        if branch and ref.size:
            bar = max(bar, 2.0 ** -6 * float(np.abs(ref).max()))
        assert ma <= bar, f"{name}: max abs error {ma:.3e} > {bar:.3e}"


def check_selection(idx_gpu: np.ndarray, scores: np.ndarray, thr: np.ndarray, keep: int) -> None:
    """The GPU's kept blocks are a valid top-k: exactly `keep` distinct
    ascending indices, every block scoring above thr + WINDOW kept and none
    below thr - WINDOW (inside the window either choice is correct)."""
    nblk = scores.shape[0]
    assert idx_gpu.shape == (nblk, keep)
    assert (np.diff(idx_gpu, axis=1) > 0).all(), "indices not strictly ascending"
    assert idx_gpu.min() >= 0 and idx_gpu.max() < nblk
    kept = np.zeros((nblk, nblk), dtype=bool)
    np.put_along_axis(kept, idx_gpu.astype(np.int64), True, axis=1)
    must = scores > (thr[:, None] + WINDOW)
    never = scores < (thr[:, None] - WINDOW)
    assert not (must & ~kept).any(), "a block clearly above the k-th score was dropped"
    assert not (never & kept).any(), "a block clearly below the k-th score was kept"


def rows_differing(idx_gpu: np.ndarray, idx_ref: np.ndarray) -> int:
    return int((idx_gpu != idx_ref).any(axis=1).sum())


def check_layer(inp: Inputs, out, idx, o_sp, o_lr, slices: Optional[Iterable] = None,
                qblocks_per_slice: Optional[int] = None, S_gpu=None, z_gpu=None) -> Dict[str, float]:
    """Compare the GPU layer with the oracle on the given (b, h) slices (all
    by default) and query blocks (all, or the seeded sample when
    qblocks_per_slice is given)."""
    cfg = inp.cfg
    slices = list(slices) if slices is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    gots, refs = {"out": [], "o_sp": [], "o_lr": []}, {"out": [], "o_sp": [], "o_lr": []}
    differ = 0
    E = None
    if cfg.lr_mode == "abspe":
        E = (inp.params_np["et"], inp.params_np["eh"], inp.params_np["ew"])
    for (b, h) in slices:
        qs, ks, vs = synth.qkv_slice(cfg, b, h)
        ig = idx[b, h].cpu().numpy()
        qblocks = None if qblocks_per_slice is None else synth.sample_query_blocks(cfg, b, h, qblocks_per_slice)
        tg = None
        if cfg.gate == "token":
            tg = (inp.params_np["wg"][h], float(inp.params_np["bg"][h]))
        omega = inp.params_np["omega"][h] if cfg.fmap == "favor" else None
        res = oracle.layer_slice(cfg, qs, ks, vs, inp.params_np["wq"][h], inp.params_np["wk"][h],
                                 inp.params_np["gate"][h], E, qblocks=qblocks, idx=ig, token_gate_wb=tg, omega=omega)
        check_selection(ig, res["scores"], res["thr"], cfg.keep)
        differ += rows_differing(ig, res["idx_ref"])
        qb = res["qblocks"]
        rows = (qb[:, None].astype(np.int64) * cfg.block + np.arange(cfg.block)[None, :]).reshape(-1)
        valid = rows < cfg.L
        for name, t in (("out", out), ("o_sp", o_sp), ("o_lr", o_lr)):
            g = to_host(t[b, h])
            gots[name].append(g[rows[valid]])
            refs[name].append(res[name].reshape(-1, cfg.D)[valid])
        if S_gpu is not None:
            # sums over the L tokens: their max-abs bar scales with their magnitude like a branch's
            assert_close(f"S[{b},{h}]", to_host(S_gpu[b, h]), res["S"], cfg.dtype, branch=True)
            assert_close(f"z[{b},{h}]", to_host(z_gpu[b, h]), res["z"], cfg.dtype, branch=True)
    log(f"    selection rows differing from the oracle inside the window: {differ}")
    for name in ("out", "o_sp", "o_lr"):
        assert_close(name, np.concatenate(gots[name]), np.concatenate(refs[name]), cfg.dtype, branch=name != "out")
    return {"differ": differ}

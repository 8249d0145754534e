"""CPU oracle for the 3D-RoPE sparse + low-rank hybrid attention forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the product path. The arithmetic lives in
``slr_oracle.c`` (plain fp64 loops, one thread); this module builds and loads
it with ctypes and chains its steps in the order the method states
(RoLA, arXiv 2609.06712v3, App. A Algorithm 1 and Fig. 2):

  rotate q, k (3D RoPE) -> block means -> block scores -> top-k blocks
  -> block-sparse softmax attention                        (sparse branch)
  phi(k W_k) -> rotate after phi -> summary S, z
  phi(q W_q) -> rotate after phi -> readout S / (w.z + eps)   (low-rank;
                                    phi = elu + 1, or SiLU with readout S / L)
  O = O_sparse + g_h * O_lowrank                              (combine)
  or, token-wise (RoLA §4.4): O = O_sparse + g(q) * RMS-aligned O_lowrank

Every function takes and returns float64 numpy arrays for one (b, h) slice.
The gradients of this forward (the backward pass) are in ``oracle.backward``.
The absolute-PE variant (RoPeSLR, arXiv 2605.20659, abstract) adds per-axis
tables before phi and skips the rotation after it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "slr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i3 = ctypes.c_int * 3
        lib.orc_rope3d.argtypes = [ctypes.c_int] * 3 + [i3, ctypes.c_int, ctypes.c_double, i3, _dp, _dp]
        lib.orc_block_mean.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _dp, _dp]
        lib.orc_block_scores.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, _dp]
        lib.orc_topk_blocks.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _ip, _dp, _dp]
        lib.orc_block_sparse_attention.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   _dp, _dp, _dp, _ip, ctypes.c_int, _ip, _dp]
        lib.orc_lowrank_features.argtypes = [ctypes.c_int] * 5 + [_dp] * 5 + [ctypes.c_int, _dp, _dp]
        lib.orc_lowrank_rotate.argtypes = [ctypes.c_int] * 3 + [i3, ctypes.c_int, ctypes.c_double, i3, i3, _dp, _dp]
        lib.orc_lowrank_summary.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp]
        lib.orc_lowrank_readout.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _lp, _dp, _dp, _dp, _dp,
                                            ctypes.c_double, ctypes.c_double, _dp]
        lib.orc_token_gate.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, ctypes.c_double, _dp, _dp,
                                       ctypes.c_double, _dp, _dp]
        for f in ("orc_rope3d", "orc_block_mean", "orc_block_scores", "orc_topk_blocks",
                  "orc_block_sparse_attention", "orc_lowrank_features", "orc_lowrank_rotate",
                  "orc_lowrank_summary", "orc_lowrank_readout"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _d(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_dp)


def _i3(v: Sequence[int]):
    return (ctypes.c_int * 3)(*[int(x) for x in v])


# ---------------------------------------------------------------------------
# single steps

def rope3d(x, grid, base, pairs, origin=(0, 0, 0)) -> np.ndarray:
    """3D RoPE of x [L, D] on grid (T, Hg, Wg) (RoLA §3, eq. 1)."""
    x = _d(x)
    T, Hg, Wg = grid
    assert x.shape[0] == T * Hg * Wg and 2 * sum(pairs) == x.shape[1]
    y = np.empty_like(x)
    _load().orc_rope3d(T, Hg, Wg, _i3(origin), x.shape[1], float(base), _i3(pairs), _p(x), _p(y))
    return y


def block_mean(x, bs) -> np.ndarray:
    x = _d(x)
    L, D = x.shape
    out = np.empty(((L + bs - 1) // bs, D))
    _load().orc_block_mean(L, D, bs, _p(x), _p(out))
    return out


def block_scores(qbar, kbar) -> np.ndarray:
    qbar, kbar = _d(qbar), _d(kbar)
    n, D = qbar.shape
    s = np.empty((n, n))
    _load().orc_block_scores(n, D, _p(qbar), _p(kbar), _p(s))
    return s


def topk_blocks(s, k):
    """(idx [n, k] int32 ascending, k-th score [n], (k+1)-th score [n])."""
    s = _d(s)
    n = s.shape[0]
    assert 1 <= k <= n
    idx = np.empty((n, k), dtype=np.int32)
    thr, nxt = np.empty(n), np.empty(n)
    _load().orc_topk_blocks(n, k, _p(s), idx.ctypes.data_as(_ip), _p(thr), _p(nxt))
    return idx, thr, nxt


def block_sparse_attention(qr, kr, v, bs, idx, qblocks=None) -> np.ndarray:
    """Softmax attention of each listed query block over its kept key
    blocks; returns [len(qblocks), bs, D] (rows past L are zero)."""
    qr, kr, v = _d(qr), _d(kr), _d(v)
    L, D = qr.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    nblk, k = idx.shape
    qblocks = np.arange(nblk, dtype=np.int32) if qblocks is None else np.ascontiguousarray(qblocks, dtype=np.int32)
    out = np.empty((len(qblocks), bs, D))
    _load().orc_block_sparse_attention(L, D, bs, k, _p(qr), _p(kr), _p(v), idx.ctypes.data_as(_ip),
                                       len(qblocks), qblocks.ctypes.data_as(_ip), _p(out))
    return out


def dense_attention(qr, kr, v, bs) -> np.ndarray:
    """Every key block kept: plain softmax attention, [L, D]."""
    L = qr.shape[0]
    nblk = (L + bs - 1) // bs
    idx = np.tile(np.arange(nblk, dtype=np.int32), (nblk, 1))
    return block_sparse_attention(qr, kr, v, bs, idx).reshape(-1, qr.shape[1])[:L]


FMAPS = {"elu1": 0, "silu": 1, "favor": 2}


def lowrank_features(x, W, grid, E=None, fmap="elu1", omega=None) -> np.ndarray:
    """phi(x W [+ E]) per token; fmap "elu1" (elu + 1), "silu", or "favor"
    (positive random features exp(omega p - |p|^2/2) / sqrt(r) of p = x W
    [+ E], omega [r, r] the random directions)."""
    x, W = _d(x), _d(W)
    T, Hg, Wg = grid
    D, r = W.shape
    u = np.empty((x.shape[0], r))
    et, eh, ew = (None, None, None) if E is None else tuple(_d(e) for e in E)
    om = None
    if fmap == "favor":
        om = _d(omega)
        assert om.shape == (r, r)
    _load().orc_lowrank_features(T, Hg, Wg, D, r, _p(x), _p(W), _p(et), _p(eh), _p(ew), FMAPS[fmap], _p(om),
                                 _p(u))
    return u


def lowrank_rotate(u, grid, base, pairs, lr_pairs, origin=(0, 0, 0)) -> np.ndarray:
    u = _d(u)
    T, Hg, Wg = grid
    r = u.shape[1]
    assert 2 * sum(lr_pairs) == r
    ur = np.empty_like(u)
    _load().orc_lowrank_rotate(T, Hg, Wg, _i3(origin), r, float(base), _i3(pairs), _i3(lr_pairs), _p(u), _p(ur))
    return ur


LR_ORDERS = ("outside", "inside", "none")


def lowrank_branch(q, k, v, wq, wk, grid, base, pairs, lr_pairs, order="outside", eps=1e-6, fmap="elu1",
                   omega=None, rows=None):
    """The rank-r branch with the rotation placed as ``order`` says (RoLA
    §4.3 and §5.1 / Table 2, the design and its two controls):
      "outside": rho(phi(x W)), the rotation after the activation (RoLA);
      "inside":  phi(rho(x W)), the rotation before the activation;
      "none":    phi(x W), no positional rotation.
    Numerator features fq, fk as above; the normaliser uses phi(x W) for
    "outside" (the un-rotated features, as the layer does) and the numerator
    features themselves otherwise. Returns (O_lr [rows, D], fq, fk, w, u)
    with w, u the normaliser features."""
    if order == "outside":
        w = lowrank_features(q, wq, grid, fmap=fmap, omega=omega)
        u = lowrank_features(k, wk, grid, fmap=fmap, omega=omega)
        fq = lowrank_rotate(w, grid, base, pairs, lr_pairs)
        fk = lowrank_rotate(u, grid, base, pairs, lr_pairs)
    elif order == "inside":
        # the projection x W as features of the identity map, rotated, then phi
        r = _d(wq).shape[1]
        pq = _d(q) @ _d(wq)
        pk = _d(k) @ _d(wk)
        eye = np.eye(r)
        fq = w = lowrank_features(lowrank_rotate(pq, grid, base, pairs, lr_pairs), eye, (pq.shape[0], 1, 1),
                                  fmap=fmap, omega=omega)
        fk = u = lowrank_features(lowrank_rotate(pk, grid, base, pairs, lr_pairs), eye, (pk.shape[0], 1, 1),
                                  fmap=fmap, omega=omega)
    elif order == "none":
        fq = w = lowrank_features(q, wq, grid, fmap=fmap, omega=omega)
        fk = u = lowrank_features(k, wk, grid, fmap=fmap, omega=omega)
    else:
        raise ValueError(order)
    S, z = lowrank_summary(fk, u, v)
    o = lowrank_readout(fq, w, S, z, eps, rows, count=float(_d(q).shape[0]) if fmap == "silu" else 0.0)
    return o, fq, fk, w, u


def lowrank_summary(fk, u, v):
    fk, u, v = _d(fk), _d(u), _d(v)
    L, r = u.shape
    D = v.shape[1]
    S, z = np.empty((r, D)), np.empty(r)
    _load().orc_lowrank_summary(L, D, r, _p(fk), _p(u), _p(v), _p(S), _p(z))
    return S, z


def lowrank_readout(fq, w, S, z, eps, rows=None, count=0.0) -> np.ndarray:
    """count > 0 replaces the denominator w.z + eps by count (mean readout)."""
    fq, w, S, z = _d(fq), _d(w), _d(S), _d(z)
    r, D = S.shape
    rows = np.arange(fq.shape[0], dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows), D))
    _load().orc_lowrank_readout(D, r, len(rows), rows.ctypes.data_as(_lp), _p(fq), _p(w), _p(S), _p(z),
                                float(eps), float(count), _p(out))
    return out


def token_gate(q, wg, bg, o_sp, o_lr, eps):
    """Token-wise gated fusion of [n, D] rows (RoLA §4.4): returns (out, g)."""
    q, wg, o_sp, o_lr = _d(q), _d(wg), _d(o_sp), _d(o_lr)
    n, D = o_sp.shape
    out, g = np.empty((n, D)), np.empty(n)
    _load().orc_token_gate(n, D, _p(q), _p(wg), float(bg), _p(o_sp), _p(o_lr), float(eps), _p(out), _p(g))
    return out, g


# ---------------------------------------------------------------------------
# one (b, h) slice of the whole layer

def layer_slice(cfg, q, k, v, wq, wk, gate_h, E=None, qblocks=None, idx=None,
                origin=(0, 0, 0), token_gate_wb=None, omega=None) -> Dict[str, np.ndarray]:
    """Forward of one (b, h) slice.

    ``cfg`` supplies T, Hg, Wg, base, pairs, block, keep, lr_mode, lr_pairs
    and eps. ``qblocks`` limits the sparse branch and the outputs to those
    query blocks (all when None). ``idx`` replaces the selection for the
    sparse branch (used where a near-tie allows another valid selection).
    Returns the intermediates: q_rot, k_rot, qbar, kbar, scores, idx_ref,
    thr, next, S, z, o_sp, o_lr, out (the last three as [nq, bs, D]).
    ``token_gate_wb = (wg [D], bg)`` replaces the per-head gate by the
    token-wise gate of RoLA §4.4 (then also returns ``g`` per row).
    ``omega`` [r, r] are the head's random directions when cfg.fmap is
    "favor" (positive random features)."""
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    L, bs = cfg.T * cfg.Hg * cfg.Wg, cfg.block
    nblk = (L + bs - 1) // bs
    res: Dict[str, np.ndarray] = {}
    res["q_rot"] = qr = rope3d(q, grid, cfg.base, cfg.pairs, origin)
    res["k_rot"] = kr = rope3d(k, grid, cfg.base, cfg.pairs, origin)
    res["qbar"] = qb = block_mean(qr, bs)
    res["kbar"] = kb = block_mean(kr, bs)
    res["scores"] = s = block_scores(qb, kb)
    res["idx_ref"], res["thr"], res["next"] = topk_blocks(s, cfg.keep)
    use_idx = res["idx_ref"] if idx is None else np.ascontiguousarray(idx, dtype=np.int32)
    qblocks = np.arange(nblk, dtype=np.int32) if qblocks is None else np.asarray(qblocks, dtype=np.int32)
    res["qblocks"] = qblocks
    o_sp = block_sparse_attention(qr, kr, v, bs, use_idx, qblocks)

    fmap = getattr(cfg, "fmap", "elu1")
    if cfg.lr_mode == "rola":
        u = lowrank_features(k, wk, grid, fmap=fmap, omega=omega)
        w = lowrank_features(q, wq, grid, fmap=fmap, omega=omega)
        fk = lowrank_rotate(u, grid, cfg.base, cfg.pairs, cfg.lr_pairs, origin)
        fq = lowrank_rotate(w, grid, cfg.base, cfg.pairs, cfg.lr_pairs, origin)
    else:
        u = lowrank_features(k, wk, grid, E, fmap=fmap, omega=omega)
        w = lowrank_features(q, wq, grid, E, fmap=fmap, omega=omega)
        fk, fq = u, w
    res["S"], res["z"] = S, z = lowrank_summary(fk, u, v)
    rows = (qblocks[:, None].astype(np.int64) * bs + np.arange(bs)[None, :]).reshape(-1)
    valid = rows < L
    o_lr = np.zeros((len(rows), q.shape[1]))
    o_lr[valid] = lowrank_readout(fq, w, S, z, cfg.eps, rows[valid], count=float(L) if fmap == "silu" else 0.0)
    o_lr = o_lr.reshape(len(qblocks), bs, -1)
    res["o_sp"], res["o_lr"] = o_sp, o_lr
    if token_gate_wb is None:
        res["out"] = o_sp + float(gate_h) * o_lr
    else:
        D = q.shape[1]
        qrows = np.zeros((len(rows), D))
        qrows[valid] = _d(q)[rows[valid]]
        out, g = token_gate(qrows, token_gate_wb[0], token_gate_wb[1], o_sp.reshape(-1, D), o_lr.reshape(-1, D),
                            cfg.eps)
        res["out"] = out.reshape(o_sp.shape)
        res["g"] = g.reshape(len(qblocks), bs)
    return res

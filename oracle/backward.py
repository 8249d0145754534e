"""CPU oracle of the hybrid layer's backward pass (gradients of the forward).

TEST INFRASTRUCTURE ONLY: imported by the tests and the bench's CPU-baseline
leg, never by the product path. Plain numpy in float64, one (b, h) slice at
a time, with matrix products as the only library primitive.

The forward is the one ``oracle.layer_slice`` computes (RoLA, arXiv
2609.06712v3, App. A Algorithm 1; §4.1-4.3). The pages fine-tune this layer
(RoLA §4.4 and App. E.2: the projections P_q, P_k and the gate are trained),
so its gradients are those of that forward by the chain rule; no page
states them. Readings:

- the block selection (a top-k) is piecewise constant, so it carries no
  gradient: the kept blocks are those of the forward, held fixed;
- the sparse branch's gradient is that of an exact softmax over the kept
  key tokens of each query row (scale 1/sqrt(D)), taken with respect to the
  rotated q and k, then taken back through the rotation by its transpose
  (each 2x2 pair turned by the opposite angle);
- the low-rank branch's gradient follows phi, the rotation after phi, the
  summary S, z and the normaliser w . z + eps (or the token count for SiLU);
  FAVOR+ features u_c(p) = exp(omega_c . p - |p|^2 / 2) / sqrt(r) (RoPeSLR
  appendix) are not elementwise: du_c / dp = u_c (omega_c - p), so
  dp = omega^T (du * u) - p sum_c du_c u_c;
- the per-head gate's gradient is sum over rows of dout . O_lowrank;
- with RoLA's token-wise gate (§4.4; the forward's reading is that of
  ``oracle.token_gate``) the gradient flows through the gate's logistic of
  q . W_g + b_g and through both RMS terms of its scale.

Each function names the forward step it differentiates.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

import oracle


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _coords(grid, origin=(0, 0, 0)) -> np.ndarray:
    """Integer (t, h, w) of every token, t-major then h then w: [L, 3]."""
    T, Hg, Wg = grid
    l = np.arange(T * Hg * Wg)
    return np.stack([l // (Hg * Wg) + origin[0], (l // Wg) % Hg + origin[1], l % Wg + origin[2]], axis=1)


def _pair_angles(grid, base, pairs, take, origin=(0, 0, 0)) -> np.ndarray:
    """Angle of every used rotary pair at every token, [L, sum(take)]: the
    axes own contiguous chunks t | h | w; pair j of axis a (j < take[a])
    turns by coordinate * base^(-2j / (2 pairs[a])) (RoLA §3, eq. 1; the
    low-rank rotation reuses the backbone's schedule, §4.2)."""
    c = _coords(grid, origin).astype(np.float64)
    cols = []
    for a in range(3):
        for j in range(take[a]):
            theta = float(base) ** (-2.0 * j / (2.0 * pairs[a]))
            cols.append(c[:, a] * theta)
    if not cols:
        return np.zeros((c.shape[0], 0))
    return np.stack(cols, axis=1)


def rotate_transpose(y, angles) -> np.ndarray:
    """x = R^T y for rows rotated pairwise by ``angles`` ([L, P]): each
    adjacent pair (2i, 2i+1) is turned by minus its angle; dims past 2P are
    copied."""
    y = _d(y).copy()
    P = angles.shape[1]
    c, s = np.cos(angles), np.sin(angles)
    y0, y1 = y[:, 0:2 * P:2].copy(), y[:, 1:2 * P:2].copy()
    y[:, 0:2 * P:2] = y0 * c + y1 * s
    y[:, 1:2 * P:2] = -y0 * s + y1 * c
    return y


def rope3d_transpose(y, grid, base, pairs, origin=(0, 0, 0)) -> np.ndarray:
    """Transpose of the 3D RoPE of ``oracle.rope3d`` (the rotation's adjoint)."""
    return rotate_transpose(y, _pair_angles(grid, base, pairs, pairs, origin))


def lowrank_rotate_transpose(y, grid, base, pairs, lr_pairs, origin=(0, 0, 0)) -> np.ndarray:
    """Transpose of ``oracle.lowrank_rotate`` (rank-truncated rotation)."""
    return rotate_transpose(y, _pair_angles(grid, base, pairs, lr_pairs, origin))


# ---------------------------------------------------------------------------
# sparse branch

def _kept_tokens(idx_row, bs, L) -> np.ndarray:
    return np.concatenate([np.arange(j * bs, min((j + 1) * bs, L)) for j in idx_row])


def sparse_attention_bwd(qr, kr, v, bs, idx, dO, qblocks: Optional[Sequence[int]] = None,
                         o: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradient of the block-sparse softmax attention (RoLA §4.1; the
    forward is ``oracle.block_sparse_attention``) with respect to the
    rotated q, the rotated k and v, for the query blocks listed (all when
    None). For each valid query row: P = softmax(q K^T / sqrt(D)) over its
    kept key tokens, dP = dO V^T, dS = P * (dP - dO . o) with o = P V (or the
    row of ``o`` [L, D] when given: the saved forward output), dq = dS K /
    sqrt(D); every kept key receives dk += dS q / sqrt(D) and dv += P dO.
    Returns dq, dk, dv [L, D] (rows the listed blocks do not touch are 0)."""
    qr, kr, v, dO = _d(qr), _d(kr), _d(v), _d(dO)
    L, D = qr.shape
    nblk = idx.shape[0]
    scale = 1.0 / np.sqrt(D)
    dq, dk, dv = np.zeros((L, D)), np.zeros((L, D)), np.zeros((L, D))
    for i in (range(nblk) if qblocks is None else qblocks):
        rows = np.arange(i * bs, min((i + 1) * bs, L))
        if rows.size == 0:
            continue
        keys = _kept_tokens(idx[i], bs, L)
        s = qr[rows] @ kr[keys].T * scale
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        orow = p @ v[keys] if o is None else _d(o)[rows]
        dp = dO[rows] @ v[keys].T
        ds = p * (dp - (dO[rows] * orow).sum(axis=1, keepdims=True))
        dq[rows] += ds @ kr[keys] * scale
        np.add.at(dk, keys, ds.T @ qr[rows] * scale)
        np.add.at(dv, keys, p.T @ dO[rows])
    return {"dq": dq, "dk": dk, "dv": dv}


def row_log2_normaliser(qr, kr, bs, idx, qblocks: Optional[Sequence[int]] = None) -> np.ndarray:
    """log2 of each valid query row's softmax normaliser over its kept key
    tokens, sum_j exp(q . k_j / sqrt(D)) (the statistic a training forward
    saves so the backward need not recompute it). Rows of the listed query
    blocks (all when None), [n_rows]."""
    qr, kr = _d(qr), _d(kr)
    L, D = qr.shape
    out = []
    for i in (range(idx.shape[0]) if qblocks is None else qblocks):
        rows = np.arange(i * bs, min((i + 1) * bs, L))
        s = qr[rows] @ kr[_kept_tokens(idx[i], bs, L)].T / np.sqrt(D)
        m = s.max(axis=1)
        out.append((m + np.log(np.exp(s - m[:, None]).sum(axis=1))) / np.log(2.0))
    return np.concatenate(out) if out else np.zeros(0)


def query_blocks_keeping(idx, kblocks) -> np.ndarray:
    """Query blocks whose kept list holds any of ``kblocks`` (ascending)."""
    want = np.zeros(int(idx.max()) + 1 if idx.size else 1, dtype=bool)
    want[np.asarray(kblocks, dtype=np.int64)] = True
    return np.nonzero(want[idx].any(axis=1))[0]


# ---------------------------------------------------------------------------
# low-rank branch

def _favor(p, omega):
    """FAVOR+ features of the rows of p [n, r]: exp(p omega^T - |p|^2 / 2) / sqrt(r)."""
    om = _d(omega)
    r = om.shape[0]
    return np.exp(p @ om.T - 0.5 * (p * p).sum(axis=1, keepdims=True)) / np.sqrt(r)


def _favor_back(p, u, du, omega):
    """Gradient w.r.t. p of sum(du * u(p)) for FAVOR+ features u of p."""
    g = du * u
    return g @ _d(omega) - p * g.sum(axis=1, keepdims=True)


def _phi_and_grad(x, fmap):
    """phi(x) and phi'(x): elu + 1 (x + 1 | exp x), or SiLU (x sigma(x))."""
    if fmap == "elu1":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0))), np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    sg = 1.0 / (1.0 + np.exp(-x))
    return x * sg, sg * (1.0 + x * (1.0 - sg))


def _axis_scatter(g, grid, r):
    """Per-axis sums of a [L, r] gradient: the adjoint of adding
    E_t[t] + E_h[h] + E_w[w] to every token."""
    c = _coords(grid)
    out = []
    for a, n in enumerate(grid):
        e = np.zeros((n, r))
        np.add.at(e, c[:, a], g)
        out.append(e)
    return tuple(out)


def lowrank_bwd(cfg, q, k, v, wq, wk, dolr, E=None, origin=(0, 0, 0), omega=None) -> Dict[str, np.ndarray]:
    """Gradient of the low-rank branch O_lr (RoLA §4.1-4.3, App. A; the
    forward is ``oracle.lowrank_features`` / ``lowrank_rotate`` /
    ``lowrank_summary`` / ``lowrank_readout``) given dL/dO_lr = ``dolr`` [L, D].

    Forward, per token l:  w_l = phi(q_l W_q [+ E_l]),  fq_l = rho_l(w_l)
    (rotary variant; fq = w with absolute PE), n_l = w_l . z + eps (SiLU:
    n_l = L), O_l = fq_l^T S / n_l; S = sum_m fk_m v_m^T, z = sum_m u_m,
    u_m = phi(k_m W_k [+ E_m]), fk_m = rho_m(u_m).
    Backward:  dfq_l = S dO_l / n_l,  dn_l = -(dO_l . O_l) / n_l,
    dS = sum_l fq_l dO_l^T / n_l,  dz = sum_l dn_l w_l,
    dw_l = rho_l^T dfq_l + dn_l z,  dpq_l = dw_l * phi'(.),
    dW_q = q^T dpq,  dq = dpq W_q^T;  dfk_m = dS v_m,  dv_m = dS^T fk_m,
    du_m = rho_m^T dfk_m + dz,  dpk_m = du_m * phi'(.),  dW_k = k^T dpk,
    dk = dpk W_k^T; the E tables take the per-axis sums of dpq + dpk.
    FAVOR+ (cfg.fmap "favor", ``omega`` [r, r] the head's directions): dpq and
    dpk go through the features' full Jacobian (``_favor_back``)."""
    q, k, v, wq, wk, dolr = _d(q), _d(k), _d(v), _d(wq), _d(wk), _d(dolr)
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    L = q.shape[0]
    r = wq.shape[1]
    fmap = getattr(cfg, "fmap", "elu1")
    pq, pk = q @ wq, k @ wk
    if E is not None:
        c = _coords(grid)
        et, eh, ew = (_d(e) for e in E)
        add = et[c[:, 0]] + eh[c[:, 1]] + ew[c[:, 2]]
        pq, pk = pq + add, pk + add
    favor = fmap == "favor"
    if favor:
        w, u = _favor(pq, omega), _favor(pk, omega)
    else:
        w, dphq = _phi_and_grad(pq, fmap)
        u, dphk = _phi_and_grad(pk, fmap)
    if cfg.lr_mode == "rola":
        ang = _pair_angles(grid, cfg.base, cfg.pairs, cfg.lr_pairs, origin)
        cs, sn = np.cos(ang), np.sin(ang)

        def rho(x):
            y = x.copy()
            y[:, 0::2] = x[:, 0::2] * cs - x[:, 1::2] * sn
            y[:, 1::2] = x[:, 0::2] * sn + x[:, 1::2] * cs
            return y

        def rho_t(y):
            return rotate_transpose(y, ang)
    else:
        def rho(x):
            return x

        def rho_t(y):
            return y
    fq, fk = rho(w), rho(u)
    S = fk.T @ v
    z = u.sum(axis=0)
    silu = fmap == "silu"
    n = np.full(L, float(L)) if silu else w @ z + cfg.eps
    o = fq @ S / n[:, None]

    dfq = dolr @ S.T / n[:, None]
    dS = fq.T @ (dolr / n[:, None])
    if silu:
        dn = np.zeros(L)
        dz = np.zeros(r)
    else:
        dn = -(dolr * o).sum(axis=1) / n
        dz = (dn[:, None] * w).sum(axis=0)
    dw = rho_t(dfq) + dn[:, None] * z[None, :]
    dpq = _favor_back(pq, w, dw, omega) if favor else dw * dphq
    dfk = v @ dS.T
    du = rho_t(dfk) + dz[None, :]
    dpk = _favor_back(pk, u, du, omega) if favor else du * dphk
    res = {"dq": dpq @ wq.T, "dk": dpk @ wk.T, "dv": fk @ dS, "dWq": q.T @ dpq, "dWk": k.T @ dpk,
           "o_lr": o, "dS": dS, "dz": dz}
    if E is not None:
        res["dE"] = _axis_scatter(dpq + dpk, grid, r)
    return res


# ---------------------------------------------------------------------------
# one (b, h) slice of the whole layer

def token_gate_bwd(q, wg, bg, o_sp, o_lr, eps, dout) -> Dict[str, np.ndarray]:
    """Gradient of the token-wise gated fusion (RoLA §4.4; the forward is
    ``oracle.token_gate``), row by row:
        out = o_sp + G o_lr,  G = g c,  g = sigmoid(q . wg + bg),
        c = rs / (rl + eps),  rs = RMS(o_sp), rl = RMS(o_lr) over the D dims.
    Given dout: dG = dout . o_lr, dg = dG c, dc = dG g, drs = dc / (rl + eps),
    drl = -dc rs / (rl + eps)^2, and d RMS(x) / dx = x / (D RMS(x)):
        d o_sp = dout + drs o_sp / (D rs),   d o_lr = G dout + drl o_lr / (D rl),
        dt = dg g (1 - g):  dq = dt wg,  dwg = sum_rows dt q,  dbg = sum_rows dt.
    Rows are [n, D]; returns d_osp, d_olr, dq [n, D], dwg [D], dbg."""
    q, o_sp, o_lr, dout = _d(q), _d(o_sp), _d(o_lr), _d(dout)
    D = o_sp.shape[1]
    g = 1.0 / (1.0 + np.exp(-(q @ _d(wg) + float(bg))))
    rs = np.sqrt((o_sp * o_sp).mean(axis=1))
    rl = np.sqrt((o_lr * o_lr).mean(axis=1))
    c = rs / (rl + eps)
    G = g * c
    dG = (dout * o_lr).sum(axis=1)
    dgl, dc = dG * c, dG * g
    drs = dc / (rl + eps)
    drl = -dc * rs / (rl + eps) ** 2
    with np.errstate(divide="ignore", invalid="ignore"):
        ks = np.where(rs > 0, drs / (D * rs), 0.0)
        kl = np.where(rl > 0, drl / (D * rl), 0.0)
    dt = dgl * g * (1.0 - g)
    return {"d_osp": dout + ks[:, None] * o_sp, "d_olr": G[:, None] * dout + kl[:, None] * o_lr,
            "dq": dt[:, None] * _d(wg)[None, :], "dwg": (dt[:, None] * q).sum(axis=0), "dbg": float(dt.sum()),
            "g": g}


def layer_slice_bwd(cfg, q, k, v, wq, wk, gate_h, dout, E=None, idx=None,
                    o_sp: Optional[np.ndarray] = None, token_gate_wb=None, omega=None) -> Dict[str, np.ndarray]:
    """Gradients of one (b, h) slice of the layer (per-head gate):
    out = O_sparse + g_h O_lowrank, so dO_sparse = dout, dO_lowrank = g_h dout
    and dg_h = sum over rows of dout . O_lowrank. ``idx`` fixes the kept blocks
    (the forward's selection when None); ``o_sp`` [L, D] replaces the sparse
    output used for dO . o (the saved forward output). Returns dq, dk, dv
    [L, D], dWq, dWk [D, r], dg (scalar), dE (absolute PE), idx and the parts.
    ``token_gate_wb = (wg [D], bg)`` uses RoLA's token-wise gate instead of
    g_h (then dWg [D] and dbg replace dg). ``omega`` [r, r]: the head's FAVOR+
    directions when cfg.fmap is "favor"."""
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    dout = _d(dout)
    L = dout.shape[0]
    if idx is None:
        idx = oracle.layer_slice(cfg, q, k, v, wq, wk, gate_h, E=E, omega=omega)["idx_ref"]
    qr = oracle.rope3d(q, grid, cfg.base, cfg.pairs)
    kr = oracle.rope3d(k, grid, cfg.base, cfg.pairs)
    tg = None
    if token_gate_wb is None:
        d_sp, d_lr = dout, float(gate_h) * dout
    else:
        # the gate reads both branch outputs: the forward's O_sparse and O_lowrank
        L, D = dout.shape
        osp = oracle.block_sparse_attention(qr, kr, v, cfg.block, idx).reshape(-1, D)[:L] if o_sp is None else _d(o_sp)
        olr = lowrank_bwd(cfg, q, k, v, wq, wk, np.zeros_like(dout), E=E, omega=omega)["o_lr"]
        tg = token_gate_bwd(q, token_gate_wb[0], token_gate_wb[1], osp, olr, cfg.eps, dout)
        d_sp, d_lr, o_sp = tg["d_osp"], tg["d_olr"], osp
    sp = sparse_attention_bwd(qr, kr, v, cfg.block, idx, d_sp, o=o_sp)
    lr = lowrank_bwd(cfg, q, k, v, wq, wk, d_lr, E=E, omega=omega)
    res = {
        "dq": rope3d_transpose(sp["dq"], grid, cfg.base, cfg.pairs) + lr["dq"],
        "dk": rope3d_transpose(sp["dk"], grid, cfg.base, cfg.pairs) + lr["dk"],
        "dv": sp["dv"] + lr["dv"],
        "dWq": lr["dWq"], "dWk": lr["dWk"],
        "dg": float((dout * lr["o_lr"]).sum()),
        "idx": idx, "sparse": sp, "lowrank": lr,
    }
    if tg is not None:
        res["dq"] = res["dq"] + tg["dq"]
        res["dWg"], res["dbg"], res["gate"] = tg["dwg"], tg["dbg"], tg
        del res["dg"]
    if E is not None:
        res["dE"] = lr["dE"]
    assert res["dq"].shape == (L, q.shape[1])
    return res

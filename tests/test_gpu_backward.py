"""GPU parity of the layer backward (slr_attention_bwd) with the oracle's.

The GPU training forward (slr_attention_fwd_train) supplies the selection
(checked to be a valid top-k), its O_sparse and the rows' log2 softmax
normalisers, as a training step would; the oracle recomputes its own in
float64 on the same selection (the saved normalisers are checked against
it to 3e-2 absolute, in log2 units). Bar: for bf16 layers relative Frobenius
error <= 1e-2 and max-abs error <= 3e-2 x max |reference| for dq, dk, dv,
dW_q, dW_k, the gate gradient and the E tables' gradients (the gradients are
~0.05 RMS, so the forward's absolute 3e-2 is stated relative to the
gradient's own scale); for fp32 layers 1e-5 relative Frobenius and 1e-5 x
max |reference|. The per-head gate's gradient dg_h = sum_l dout_l . O_lr,l
is a sum whose terms cancel (by up to ~130x in these layers), and the
rounding error of a sum scales with the sum of its terms' magnitudes, so its
error is measured against sum_l |dout_l . O_lr,l| instead of |dg_h|.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OB
from sparse_rank_attention_rope3d_amd import binding as B
from sparse_rank_attention_rope3d_amd import synth

import slrtest as T

pytestmark = pytest.mark.gpu

BAR = {"bf16": (1e-2, 3e-2), "f32": (1e-5, 1e-5)}
_dtype = ["bf16"]


def _close(name, got, ref, scale=None):
    """scale: the magnitude errors are measured against (default |ref|)."""
    rel, maxrel = BAR[_dtype[0]]
    if scale is None:
        rf = T.rel_fro(got, ref)
        scale = float(np.abs(ref).max()) if ref.size else 1.0
    else:
        rf = T.max_abs(got, ref) / scale
    ma = T.max_abs(got, ref) / (scale if scale > 0 else 1.0)
    T.log(f"    {name}: rel_fro={rf:.3e} max_abs/max|ref|={ma:.3e}")
    assert rf <= rel, f"{name}: relative Frobenius error {rf:.3e} > {rel}"
    assert ma <= maxrel, f"{name}: max abs error {ma:.3e} x max|ref| > {maxrel}"


def _dout(cfg):
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    g = torch.empty((cfg.B, cfg.H, cfg.L, cfg.D), dtype=tdt, device="cuda")
    for b in range(cfg.B):
        for h in range(cfg.H):
            g[b, h] = T.to_device(synth.dout_slice(cfg, b, h), cfg.dtype)
    return g


def _summary_buffers(cfg):
    S = torch.empty((cfg.B, cfg.H, cfg.rank, cfg.D), dtype=torch.float32, device="cuda")
    return S, torch.empty((cfg.B, cfg.H, cfg.rank), dtype=torch.float32, device="cuda")


def _run_gpu(cfg, saved_summary=True):
    """Training forward then backward; the backward is given the summary the
    forward saved (a training step's path) unless saved_summary is False."""
    inp = T.make_inputs(cfg)
    dout = _dout(cfg)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, inp.params)
    summ = _summary_buffers(cfg) if saved_summary else None
    _, idx, o_sp, lse = B.slr_attention_fwd_train(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank, summary=summ)
    grads = B.slr_attention_bwd(inp.q, inp.k, inp.v, idx, o_sp, lse, dout, shape, rope, sparse, lowrank,
                                summary=summ)
    torch.cuda.synchronize()
    return inp, idx, grads, lse


def _tables(cfg, p):
    return (p["et"], p["eh"], p["ew"]) if cfg.lr_mode == "abspe" else None


def _omega(p, h):
    return p["omega"][h] if "omega" in p else None


def _oracle_lowrank(cfg, inp, b, h):
    qs, ks, vs = synth.qkv_slice(cfg, b, h)
    ds = np.asarray(synth.dout_slice(cfg, b, h), np.float64)
    p = inp.params_np
    return OB.lowrank_bwd(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], float(p["gate"][h]) * ds, E=_tables(cfg, p),
                          omega=_omega(p, h))


def _oracle_slice(cfg, inp, b, h, ig, qblocks=None, kblocks=None):
    """dq rows of qblocks and dk, dv rows of kblocks (all rows when None)."""
    qs, ks, vs = synth.qkv_slice(cfg, b, h)
    ds = np.asarray(synth.dout_slice(cfg, b, h), np.float64)
    p = inp.params_np
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    res = oracle.layer_slice(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], p["gate"][h], E=_tables(cfg, p), qblocks=[0],
                             idx=ig, omega=_omega(p, h))
    T.check_selection(ig, res["scores"], res["thr"], cfg.keep)
    qr, kr = res["q_rot"], res["k_rot"]
    lr = _oracle_lowrank(cfg, inp, b, h)
    spq = OB.sparse_attention_bwd(qr, kr, vs, cfg.block, ig, ds, qblocks=qblocks)
    if kblocks is None:
        spk = spq
    else:
        spk = OB.sparse_attention_bwd(qr, kr, vs, cfg.block, ig, ds, qblocks=OB.query_blocks_keeping(ig, kblocks))
    ref = {
        "dq": OB.rope3d_transpose(spq["dq"], grid, cfg.base, cfg.pairs) + lr["dq"],
        "dk": OB.rope3d_transpose(spk["dk"], grid, cfg.base, cfg.pairs) + lr["dk"],
        "dv": spk["dv"] + lr["dv"],
        "dWq": lr["dWq"], "dWk": lr["dWk"], "dg": float((ds * lr["o_lr"]).sum()),
        "dg_abs": float(np.abs((ds * lr["o_lr"]).sum(axis=1)).sum()),
        "q_rot": qr, "k_rot": kr, "dE": lr.get("dE"),
    }
    return ref


def _rows(cfg, blocks):
    if blocks is None:
        return np.arange(cfg.L)
    r = (np.asarray(blocks, np.int64)[:, None] * cfg.block + np.arange(cfg.block)[None, :]).reshape(-1)
    return r[r < cfg.L]


def _check(cfg, slices=None, qsample=None, ksample=None, heads=None):
    T.log(f"  case {cfg.name}: L={cfg.L} nblk={cfg.nblk} keep={cfg.keep} D={cfg.D} r={cfg.rank} fmap={cfg.fmap} "
          f"{cfg.dtype}")
    _dtype[0] = cfg.dtype
    inp, idx, (dq, dk, dv, dWq, dWk, dg, dE), lse = _run_gpu(cfg)
    slices = slices or [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    heads = sorted({h for _, h in slices}) if heads is None else heads
    got = {"dq": [], "dk": [], "dv": []}
    want = {"dq": [], "dk": [], "dv": []}
    dW = {}
    for (b, h) in [(b, h) for h in heads for b in range(cfg.B)] + slices:
        if (b, h) in dW:
            continue
        ig = idx[b, h].cpu().numpy()
        qb = None if qsample is None else synth.sample_query_blocks(cfg, b, h, qsample)
        kb = None if ksample is None else synth.sample_query_blocks(cfg, b, h + 1000, ksample)
        ref = _oracle_slice(cfg, inp, b, h, ig, qb, kb)
        dW[b, h] = ref
        if (b, h) in slices:
            # the normaliser the training forward saved: log2 units, abs error
            got_l = T.to_host(lse[b, h])[_rows(cfg, qb)]
            want_l = OB.row_log2_normaliser(ref["q_rot"], ref["k_rot"], cfg.block, ig, qb)
            err = float(np.abs(got_l - want_l).max())
            T.log(f"    lse[{b},{h}]: max_abs={err:.3e}")
            assert err <= 3e-2, f"saved log2 normaliser off by {err:.3e}"
            rq, rk = _rows(cfg, qb), _rows(cfg, kb)
            for name, t, rows in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rk)):
                got[name].append(T.to_host(t[b, h])[rows])
                want[name].append(ref[name][rows])
    for name in ("dq", "dk", "dv"):
        _close(name, np.concatenate(got[name]), np.concatenate(want[name]))
    if cfg.lr_mode == "abspe":
        # the tables are shared by every slice: their gradient sums over all of them
        want_e = [np.zeros((n, cfg.rank)) for n in (cfg.T, cfg.Hg, cfg.Wg)]
        for b in range(cfg.B):
            for h in range(cfg.H):
                de = dW[b, h]["dE"] if (b, h) in dW else _oracle_lowrank(cfg, inp, b, h)["dE"]
                for i in range(3):
                    want_e[i] += de[i]
        for i, name in enumerate(("dEt", "dEh", "dEw")):
            _close(name, T.to_host(dE[i]), want_e[i])
    for h in heads:
        _close(f"dWq[{h}]", T.to_host(dWq[h]), sum(dW[b, h]["dWq"] for b in range(cfg.B)))
        _close(f"dWk[{h}]", T.to_host(dWk[h]), sum(dW[b, h]["dWk"] for b in range(cfg.B)))
        _close(f"dgate[{h}]", T.to_host(dg[h:h + 1]), np.array([sum(dW[b, h]["dg"] for b in range(cfg.B))]),
               scale=sum(dW[b, h]["dg_abs"] for b in range(cfg.B)))


SMALL = [
    # (name, changes to the Wan2.1-1.3B layer)
    ("ragged 4x9x13 keep3", dict(B=1, H=2, T=4, Hg=9, Wg=13, keep=3)),
    ("two batches keep1", dict(B=2, H=1, T=3, Hg=8, Wg=16, keep=1)),
    ("every block kept", dict(B=1, H=2, T=4, Hg=9, Wg=13, keep=8)),
    ("silu", dict(B=1, H=2, T=4, Hg=9, Wg=13, keep=3, fmap="silu")),
    ("rank 64", dict(B=1, H=1, T=4, Hg=9, Wg=13, keep=2, rank=64, lr_pairs=(16, 8, 8))),
    ("rank 8", dict(B=1, H=1, T=4, Hg=9, Wg=13, keep=2, rank=8, lr_pairs=(2, 1, 1))),
    ("D64 block32", dict(B=1, H=2, D=64, pairs=(12, 10, 10), T=3, Hg=10, Wg=11, block=32, keep=4, rank=16,
                         lr_pairs=(4, 2, 2))),
    ("D128 block32 one block", dict(B=1, H=1, T=1, Hg=3, Wg=7, block=32, keep=1)),
    ("D128 block64 one ragged block", dict(B=1, H=2, T=1, Hg=3, Wg=7, keep=1)),
    ("absolute PE", dict(B=2, H=2, T=4, Hg=9, Wg=13, keep=3, lr_mode="abspe", lr_pairs=(0, 0, 0))),
    ("absolute PE silu D64 block32", dict(B=1, H=2, D=64, pairs=(12, 10, 10), T=3, Hg=10, Wg=11, block=32, keep=4,
                                          rank=16, lr_mode="abspe", lr_pairs=(0, 0, 0), fmap="silu")),
    ("absolute PE silu rank 64", dict(B=1, H=2, T=3, Hg=10, Wg=11, keep=4, rank=64, lr_mode="abspe",
                                      lr_pairs=(0, 0, 0), fmap="silu")),
    ("rank 16 silu", dict(B=2, H=1, T=4, Hg=9, Wg=13, keep=3, rank=16, lr_pairs=(4, 2, 2), fmap="silu")),
    ("absolute PE rank 8", dict(B=1, H=2, T=3, Hg=10, Wg=11, keep=2, rank=8, lr_mode="abspe", lr_pairs=(0, 0, 0))),
    ("favor", dict(B=2, H=2, T=4, Hg=9, Wg=13, keep=3, fmap="favor")),
    ("favor absolute PE rank 64", dict(B=1, H=2, T=3, Hg=10, Wg=11, keep=4, rank=64, lr_mode="abspe",
                                       lr_pairs=(0, 0, 0), fmap="favor")),
    ("favor rank 16", dict(B=1, H=2, T=4, Hg=9, Wg=13, keep=3, rank=16, lr_pairs=(4, 2, 2), fmap="favor")),
    ("favor D64 block32", dict(B=1, H=2, D=64, pairs=(12, 10, 10), T=3, Hg=10, Wg=11, block=32, keep=4, rank=16,
                               lr_pairs=(4, 2, 2), fmap="favor")),
    ("favor absolute PE D64 rank 32", dict(B=1, H=2, D=64, pairs=(12, 10, 10), T=3, Hg=10, Wg=11, block=32, keep=4,
                                           rank=32, lr_mode="abspe", lr_pairs=(0, 0, 0), fmap="favor")),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_backward_small_layers(name, kw):
    cfg = dataclasses.replace(synth.wan13b(), name=f"bwd {name}", **kw)
    _check(cfg)


F32 = [
    ("tiny fp32 check layer", synth.tiny()),
    ("fp32 ragged D128 block64", dataclasses.replace(synth.wan13b(), name="fp32 ragged", dtype="f32", B=1, H=2, T=4,
                                                     Hg=9, Wg=13, keep=3)),
    ("fp32 absolute PE silu", dataclasses.replace(synth.tiny(), name="fp32 abspe silu", lr_mode="abspe",
                                                  lr_pairs=(0, 0, 0), fmap="silu", T=3, Hg=5, Wg=7)),
    ("fp32 favor", dataclasses.replace(synth.tiny(), name="fp32 favor", fmap="favor")),
    ("fp32 favor ragged D128 absolute PE", dataclasses.replace(synth.wan13b(), name="fp32 favor abspe", dtype="f32",
                                                               B=1, H=2, T=4, Hg=9, Wg=13, keep=3, lr_mode="abspe",
                                                               lr_pairs=(0, 0, 0), fmap="favor")),
]


@pytest.mark.parametrize("name,cfg", F32, ids=[s[0] for s in F32])
def test_backward_fp32_layers(name, cfg):
    _check(cfg)


TOKEN = [
    ("token gate bf16", dataclasses.replace(synth.wan13b(), name="token bf16", B=2, H=2, T=4, Hg=9, Wg=13, keep=3,
                                            gate="token")),
    ("token gate bf16 absolute PE silu", dataclasses.replace(synth.wan13b(), name="token abspe silu", B=1, H=2, T=3,
                                                             Hg=10, Wg=11, keep=4, gate="token", lr_mode="abspe",
                                                             lr_pairs=(0, 0, 0), fmap="silu")),
    ("token gate fp32", dataclasses.replace(synth.tiny(), name="token fp32", gate="token")),
    ("token gate bf16 favor", dataclasses.replace(synth.wan13b(), name="token favor", B=2, H=2, T=4, Hg=9, Wg=13,
                                                  keep=3, gate="token", fmap="favor")),
    ("token gate bf16 absolute PE favor rank 64", dataclasses.replace(synth.wan13b(), name="token abspe favor", B=1,
                                                                      H=2, T=3, Hg=10, Wg=11, keep=4, gate="token",
                                                                      rank=64, lr_mode="abspe", lr_pairs=(0, 0, 0),
                                                                      fmap="favor")),
    ("token gate fp32 favor", dataclasses.replace(synth.tiny(), name="token fp32 favor", gate="token", fmap="favor")),
]


@pytest.mark.parametrize("name,cfg", TOKEN, ids=[s[0] for s in TOKEN])
def test_backward_token_gate(name, cfg):
    """RoLA's token-wise gate: every gradient of every slice against the
    oracle's layer backward (which recomputes O_sparse and O_lowrank in fp64);
    dW_g, db_g summed over the batch."""
    T.log(f"  case {cfg.name}: L={cfg.L} D={cfg.D} r={cfg.rank} fmap={cfg.fmap} {cfg.lr_mode} {cfg.dtype}")
    _dtype[0] = cfg.dtype
    inp, idx, (dq, dk, dv, dWq, dWk, (dWg, dbg), dE), lse = _run_gpu(cfg)
    p = inp.params_np
    E = _tables(cfg, p)
    got = {n: [] for n in ("dq", "dk", "dv")}
    want = {n: [] for n in ("dq", "dk", "dv")}
    sums = {}
    for b in range(cfg.B):
        for h in range(cfg.H):
            qs, ks, vs = synth.qkv_slice(cfg, b, h)
            ig = idx[b, h].cpu().numpy()
            ref_f = oracle.layer_slice(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], 0.0, E=E, qblocks=[0], idx=ig,
                                       omega=_omega(p, h))
            T.check_selection(ig, ref_f["scores"], ref_f["thr"], cfg.keep)
            ds = np.asarray(synth.dout_slice(cfg, b, h), np.float64)
            ref = OB.layer_slice_bwd(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], 0.0, ds, E=E, idx=ig,
                                     token_gate_wb=(p["wg"][h], float(p["bg"][h])), omega=_omega(p, h))
            for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
                got[n].append(T.to_host(t[b, h]))
                want[n].append(ref[n])
            for n in ("dWq", "dWk", "dWg", "dbg"):
                sums[n, h] = sums.get((n, h), 0.0) + np.asarray(ref[n])
            if E is not None:
                for i in range(3):
                    sums["dE", i] = sums.get(("dE", i), 0.0) + ref["dE"][i]
    for n in ("dq", "dk", "dv"):
        _close(n, np.concatenate(got[n]), np.concatenate(want[n]))
    for h in range(cfg.H):
        _close(f"dWq[{h}]", T.to_host(dWq[h]), sums["dWq", h])
        _close(f"dWk[{h}]", T.to_host(dWk[h]), sums["dWk", h])
        _close(f"dWg[{h}]", T.to_host(dWg[h]), sums["dWg", h])
        _close(f"dbg[{h}]", T.to_host(dbg[h:h + 1]), np.array([sums["dbg", h]]))
    if E is not None:
        for i, n in enumerate(("dEt", "dEh", "dEw")):
            _close(n, T.to_host(dE[i]), sums["dE", i])


SAVED = [
    ("bf16 rotary", dataclasses.replace(synth.wan13b(), name="saved bf16", B=2, H=2, T=4, Hg=9, Wg=13, keep=3)),
    ("bf16 FAVOR+ absolute PE rank 64", dataclasses.replace(synth.wan13b(), name="saved favor abspe", B=1, H=2, T=3,
                                                            Hg=10, Wg=11, keep=4, rank=64, lr_mode="abspe",
                                                            lr_pairs=(0, 0, 0), fmap="favor")),
    ("bf16 token gate SiLU", dataclasses.replace(synth.wan13b(), name="saved token silu", B=1, H=2, T=4, Hg=9, Wg=13,
                                                 keep=3, gate="token", fmap="silu")),
    ("fp32 tiny", synth.tiny()),
]


@pytest.mark.parametrize("name,cfg", SAVED, ids=[s[0] for s in SAVED])
def test_backward_saved_summary(name, cfg):
    """slr_attention_fwd_train's S_out, z_out hold the summary the layer
    used (against the oracle's S, z of every slice), and the backward given
    them agrees with the backward that recomputes them (the two summaries
    differ only in the split-L partition of their sums: within 1e-5)."""
    T.log(f"  case {cfg.name}: L={cfg.L} D={cfg.D} r={cfg.rank} fmap={cfg.fmap} {cfg.lr_mode} {cfg.gate} {cfg.dtype}")
    inp = T.make_inputs(cfg)
    dout = _dout(cfg)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, inp.params)
    S, z = _summary_buffers(cfg)
    _, idx, o_sp, lse = B.slr_attention_fwd_train(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank, summary=(S, z))
    g_saved = B.slr_attention_bwd(inp.q, inp.k, inp.v, idx, o_sp, lse, dout, shape, rope, sparse, lowrank,
                                  summary=(S, z))
    g_re = B.slr_attention_bwd(inp.q, inp.k, inp.v, idx, o_sp, lse, dout, shape, rope, sparse, lowrank)
    torch.cuda.synchronize()
    p = inp.params_np
    for b in range(cfg.B):
        for h in range(cfg.H):
            qs, ks, vs = synth.qkv_slice(cfg, b, h)
            tg = (p["wg"][h], float(p["bg"][h])) if cfg.gate == "token" else None
            res = oracle.layer_slice(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], p["gate"][h], _tables(cfg, p),
                                     qblocks=[0], idx=idx[b, h].cpu().numpy(), token_gate_wb=tg, omega=_omega(p, h))
            T.assert_close(f"S[{b},{h}]", T.to_host(S[b, h]), res["S"], cfg.dtype, branch=True)
            T.assert_close(f"z[{b},{h}]", T.to_host(z[b, h]), res["z"], cfg.dtype, branch=True)

    def flat(g):
        out = list(g[:5])
        out += list(g[5]) if isinstance(g[5], tuple) else [g[5]]
        out += list(g[6] or ())
        return out
    for i, (a, c) in enumerate(zip(flat(g_saved), flat(g_re))):
        rf = T.rel_fro(T.to_host(a), T.to_host(c))
        T.log(f"    gradient {i}: saved vs recomputed summary rel_fro={rf:.3e}")
        assert rf <= 1e-5, f"gradient {i}: saved vs recomputed summary differ by {rf:.3e}"


def test_backward_wan13b_sampled():
    """Full Wan2.1-1.3B shape: dq on sampled query blocks, dk, dv on sampled
    key blocks of two slices; dW_q, dW_k and the gate gradient of their heads
    over both batches (the low-rank branch is cheap enough for the oracle in
    full)."""
    cfg = synth.wan13b()
    _check(cfg, slices=[(0, 0), (1, 7)], qsample=4, ksample=4)


def test_backward_favor_wan13b_sampled():
    """FAVOR+ features (RoPeSLR appendix) at the full Wan2.1-1.3B shape,
    sampled as above."""
    cfg = dataclasses.replace(synth.wan13b(), fmap="favor")
    _check(cfg, slices=[(0, 3), (1, 10)], qsample=2, ksample=2)


@pytest.mark.timeout(600)
def test_backward_token_gate_wan13b_sampled():
    """RoLA's token gate at the full Wan2.1-1.3B shape (its query side on the
    VALU kernel, the key side on MFMA). The gate reads each row's RMS of
    O_sparse, so the oracle computes O_sparse for every row of head 0 in both
    batches; dq is compared on sampled query blocks, dk and dv on sampled key
    blocks, dW_q, dW_k, dW_g and db_g of head 0 summed over the batch."""
    cfg = dataclasses.replace(synth.wan13b(), name="token gate wan13b", gate="token")
    T.log(f"  case {cfg.name}: L={cfg.L} nblk={cfg.nblk} keep={cfg.keep} r={cfg.rank}")
    _dtype[0] = cfg.dtype
    inp, idx, (dq, dk, dv, dWq, dWk, (dWg, dbg), _), lse = _run_gpu(cfg)
    p = inp.params_np
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    h = 0
    got = {n: [] for n in ("dq", "dk", "dv")}
    want = {n: [] for n in ("dq", "dk", "dv")}
    sums = {}
    for b in range(cfg.B):
        qs, ks, vs = synth.qkv_slice(cfg, b, h)
        ig = idx[b, h].cpu().numpy()
        res = oracle.layer_slice(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], 0.0, qblocks=[0], idx=ig)
        T.check_selection(ig, res["scores"], res["thr"], cfg.keep)
        qr, kr = res["q_rot"], res["k_rot"]
        ds = np.asarray(synth.dout_slice(cfg, b, h), np.float64)
        osp = oracle.block_sparse_attention(qr, kr, vs, cfg.block, ig).reshape(-1, cfg.D)[:cfg.L]
        olr = OB.lowrank_bwd(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], np.zeros_like(ds))["o_lr"]
        tg = OB.token_gate_bwd(qs, p["wg"][h], float(p["bg"][h]), osp, olr, cfg.eps, ds)
        lr = OB.lowrank_bwd(cfg, qs, ks, vs, p["wq"][h], p["wk"][h], tg["d_olr"])
        qb = synth.sample_query_blocks(cfg, b, h, 3)
        kb = synth.sample_query_blocks(cfg, b, h + 1000, 3)
        spq = OB.sparse_attention_bwd(qr, kr, vs, cfg.block, ig, tg["d_osp"], qblocks=qb, o=osp)
        spk = OB.sparse_attention_bwd(qr, kr, vs, cfg.block, ig, tg["d_osp"], qblocks=OB.query_blocks_keeping(ig, kb),
                                      o=osp)
        ref = {
            "dq": OB.rope3d_transpose(spq["dq"], grid, cfg.base, cfg.pairs) + lr["dq"] + tg["dq"],
            "dk": OB.rope3d_transpose(spk["dk"], grid, cfg.base, cfg.pairs) + lr["dk"],
            "dv": spk["dv"] + lr["dv"],
        }
        rq, rk = _rows(cfg, qb), _rows(cfg, kb)
        got_l = T.to_host(lse[b, h])[rq]
        want_l = OB.row_log2_normaliser(qr, kr, cfg.block, ig, qb)
        err = float(np.abs(got_l - want_l).max())
        T.log(f"    lse[{b},{h}]: max_abs={err:.3e}")
        assert err <= 3e-2, f"saved log2 normaliser off by {err:.3e}"
        for name, t, rows in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rk)):
            got[name].append(T.to_host(t[b, h])[rows])
            want[name].append(ref[name][rows])
        for n, val in (("dWq", lr["dWq"]), ("dWk", lr["dWk"]), ("dWg", tg["dwg"]), ("dbg", tg["dbg"])):
            sums[n] = sums.get(n, 0.0) + np.asarray(val)
    for n in ("dq", "dk", "dv"):
        _close(n, np.concatenate(got[n]), np.concatenate(want[n]))
    _close("dWq[0]", T.to_host(dWq[h]), sums["dWq"])
    _close("dWk[0]", T.to_host(dWk[h]), sums["dWk"])
    _close("dWg[0]", T.to_host(dWg[h]), sums["dWg"])
    _close("dbg[0]", T.to_host(dbg[h:h + 1]), np.atleast_1d(sums["dbg"]))


def test_backward_wan14b_sampled():
    """Full Wan2.1-14B shape (1182 blocks, 119 kept: long kept and inverse
    lists through the two-slot rings of the streaming kernels): sampled rows
    of two slices as above."""
    cfg = synth.wan14b()
    _check(cfg, slices=[(0, 0), (1, 39)], qsample=2, ksample=2)


def test_backward_hunyuan13b_sampled():
    """Full HunyuanVideo-13B shape (absolute-PE low-rank variant): sampled
    rows of two slices as above; the E tables' gradients over all slices."""
    cfg = synth.hunyuan13b()
    _check(cfg, slices=[(0, 0), (0, 11)], qsample=3, ksample=2)


@pytest.mark.parametrize("grid,keep", [((4, 9, 13), 3), ((21, 30, 52), 52)], ids=["small", "wan13b-grid"])
def test_backward_is_deterministic(grid, keep):
    """Bitwise reproducible gradients; the Wan2.1-1.3B grid gives kept and
    inverse lists of dozens of tiles (many turns of the two-slot rings)."""
    cfg = dataclasses.replace(synth.wan13b(), name="bwd determinism", B=1, H=2, T=grid[0], Hg=grid[1], Wg=grid[2],
                              keep=keep)
    _, _, g1, _ = _run_gpu(cfg)
    _, _, g2, _ = _run_gpu(cfg)
    for a, b in zip(g1[:6], g2[:6]):
        assert torch.equal(a, b)


def test_backward_skips_entries_outside_range():
    """Kept-list entries outside [0, nblk) are skipped: with -1, nblk and -7
    written over entries of three rows, and the normalisers and O_sparse of
    the reduced lists (from the oracle) passed in, every gradient equals the
    oracle's layer backward on the reduced lists."""
    cfg = dataclasses.replace(synth.wan13b(), name="bwd skipped entries", B=1, H=1, T=4, Hg=9, Wg=13, keep=3)
    _dtype[0] = cfg.dtype
    inp = T.make_inputs(cfg)
    dout = _dout(cfg)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, inp.params)
    _, idx, _, _ = B.slr_attention_fwd_train(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank)
    ig = idx[0, 0].cpu().numpy().copy()
    nblk = cfg.nblk
    ig[1, 0], ig[4, 2], ig[nblk - 1, 1] = -1, nblk, -7
    red = np.empty(nblk, dtype=object)
    for i in range(nblk):
        red[i] = ig[i][(ig[i] >= 0) & (ig[i] < nblk)]
    qs, ks, vs = synth.qkv_slice(cfg, 0, 0)
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    qr = oracle.rope3d(np.asarray(qs, np.float64), grid, cfg.base, cfg.pairs)
    kr = oracle.rope3d(np.asarray(ks, np.float64), grid, cfg.base, cfg.pairs)
    o = np.concatenate([oracle.block_sparse_attention(qr, kr, vs, cfg.block, np.tile(red[i], (nblk, 1)), qblocks=[i])[0]
                        for i in range(nblk)])[: cfg.L]
    o_dev = T.to_device(o, cfg.dtype).reshape(1, 1, cfg.L, cfg.D)
    lse = torch.tensor(OB.row_log2_normaliser(qr, kr, cfg.block, red), dtype=torch.float32, device="cuda")
    idx_dev = torch.tensor(ig, dtype=torch.int32, device="cuda").reshape(1, 1, nblk, cfg.keep)
    dq, dk, dv, dWq, dWk, dg, _ = B.slr_attention_bwd(inp.q, inp.k, inp.v, idx_dev, o_dev, lse.reshape(1, 1, cfg.L),
                                                      dout, shape, rope, sparse, lowrank)
    torch.cuda.synchronize()
    p = inp.params_np
    ds = np.asarray(synth.dout_slice(cfg, 0, 0), np.float64)
    ref = OB.layer_slice_bwd(cfg, qs, ks, vs, p["wq"][0], p["wk"][0], float(p["gate"][0]), ds, idx=red,
                             o_sp=T.to_host(o_dev[0, 0]))
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _close(n, T.to_host(t[0, 0]), ref[n])
    _close("dWq", T.to_host(dWq[0]), ref["dWq"])
    _close("dgate", T.to_host(dg[0:1]), np.array([ref["dg"]]))

"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Selection: exact outside the 1e-5 near-tie window. Outputs: relative
Frobenius <= 1e-2 and max-abs <= 3e-2 for bf16 layers, relative Frobenius
<= 1e-5 for fp32 layers; the two branches (O_sparse, O_lowrank) and the
summary (S, z) are checked separately because the low-rank term is small
next to the sparse one.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import slrtest as T
from sparse_rank_attention_rope3d_amd import binding as B
from sparse_rank_attention_rope3d_amd import synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_fp32.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()  # fail loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


def _summary(inp):
    cfg = inp.cfg
    return B.slr_lowrank_summary(inp.k, inp.v, B.shape_of(cfg), B.rope_of(cfg), B.lowrank_of(cfg, inp.params))


def _full_check(cfg, with_summary=True):
    T.log(f"  case {cfg.name}: B={cfg.B} H={cfg.H} D={cfg.D} grid={cfg.T}x{cfg.Hg}x{cfg.Wg} "
          f"bs={cfg.block} keep={cfg.keep} r={cfg.rank} {cfg.lr_mode} {cfg.dtype}")
    inp = T.make_inputs(cfg)
    out, idx, o_sp, o_lr = T.run_layer(inp)
    S, z = _summary(inp) if with_summary else (None, None)
    torch.cuda.synchronize()
    return T.check_layer(inp, out, idx, o_sp, o_lr, S_gpu=S, z_gpu=z)


def test_tiny_fp32_layer_matches_oracle_and_fixture():
    cfg = synth.tiny()
    res = _full_check(cfg)
    assert res["differ"] == 0
    inp = T.make_inputs(cfg)
    out, idx, _, _ = T.run_layer(inp)
    doc = json.load(open(GOLDEN))
    for rec in doc["heads"]:
        h = rec["head"]
        assert idx[0, h].cpu().tolist() == rec["idx"]
        probe = T.to_host(out[0, h])[np.ix_(doc["probe_rows"], doc["probe_cols"])]
        np.testing.assert_allclose(probe, rec["out_probe"], rtol=1e-5, atol=1e-6)


SMALL = [
    # D, block, rank, mode, grid, keep, dtype
    (128, 64, 32, "rola", (5, 9, 13), 3, "bf16"),     # 10 blocks, ragged tail of 9
    (128, 64, 32, "abspe", (5, 9, 13), 3, "bf16"),
    (64, 32, 8, "rola", (4, 8, 8), 2, "bf16"),        # the tiny layer in bf16
    (128, 32, 16, "rola", (3, 7, 11), 3, "bf16"),     # 8 blocks, tail of 7
    (128, 64, 64, "rola", (4, 10, 12), 4, "bf16"),    # rank 64: two rank blocks
    (64, 64, 32, "abspe", (2, 6, 9), 1, "bf16"),      # keep 1
    (128, 64, 32, "rola", (3, 5, 17), 4, "bf16"),     # keep = nblk (4 blocks, tail 63)
    (128, 64, 32, "rola", (1, 3, 5), 1, "bf16"),      # L = 15 < one block
    (128, 64, 32, "rola", (2, 4, 16), 2, "bf16"),     # L = 128, no tail
    (128, 64, 32, "rola", (5, 9, 13), 3, "f32"),
    (64, 64, 16, "abspe", (3, 6, 7), 2, "f32"),
    (128, 64, 32, "rola", (20, 7, 2), 2, "bf16"),     # grid rows of 2 tokens (coordinate steps wrap often)
    (128, 64, 32, "abspe", (9, 4, 3), 2, "bf16"),
    # the layer forward's summary stages the low-rank rotation rows in LDS when they fit (at most 1920
    # entries: 8 T + 4 Hg + 4 Wg at rank 32); these two sit just below and just above that limit
    (128, 64, 32, "rola", (236, 2, 4), 3, "bf16"),    # 1912 entries, 30 blocks, tail 32
    (128, 64, 32, "rola", (250, 2, 2), 3, "bf16"),    # 2016 entries: the summary without the LDS copy
]


@pytest.mark.parametrize("D,bs,r,mode,grid,keep,dtype", SMALL)
def test_small_layers_full(D, bs, r, mode, grid, keep, dtype):
    p = r // 2
    lp = (p // 2, p // 4, p - p // 2 - p // 4) if mode == "rola" else (0, 0, 0)
    pairs = (12, 10, 10) if D == 64 else (22, 21, 21)
    cfg = T.custom(synth.wan13b(), name=f"small D{D} bs{bs} r{r} {mode} {grid} k{keep} {dtype}", B=2, H=3, D=D,
                   T=grid[0], Hg=grid[1], Wg=grid[2], block=bs, keep=keep, rank=r, lr_mode=mode, lr_pairs=lp,
                   pairs=pairs, dtype=dtype, seed=7)
    _full_check(cfg)


@pytest.mark.parametrize("grid,keep", [((5, 9, 13), 3), ((5, 30, 30), 7)])
def test_exact_ties_pick_lowest_blocks(grid, keep):
    """q = k = 0: every block score is exactly 0, so every query block keeps
    blocks 0 .. keep-1 (ties go to the lower index); 71 blocks put the keys
    of a row in two register slots per lane."""
    cfg = T.custom(synth.wan13b(), name=f"ties {grid}", B=1, H=2, T=grid[0], Hg=grid[1], Wg=grid[2], keep=keep,
                   gen="zero_qk", seed=11)
    T.log(f"  case {cfg.name}: nblk={cfg.nblk} keep={keep}")
    inp = T.make_inputs(cfg)
    out, idx, o_sp, o_lr = T.run_layer(inp)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    want = np.broadcast_to(np.arange(keep, dtype=got.dtype), got.shape)
    assert np.array_equal(got, want)
    res = T.check_layer(inp, out, idx, o_sp, o_lr)
    assert res["differ"] == 0


def test_gate_zero_gives_sparse_branch():
    cfg = T.custom(synth.wan13b(), name="gate0", B=1, H=2, T=3, Hg=5, Wg=9, keep=2)
    inp = T.make_inputs(cfg)
    inp.params["gate"].zero_()
    out, _, o_sp, _ = T.run_layer(inp)
    torch.cuda.synchronize()
    assert torch.equal(out, o_sp)


TOKEN_GATE = [
    # D, block, rank, mode, grid, keep, dtype: the three flash kernels (tiled bf16, other bf16, fp32)
    (128, 64, 32, "rola", (5, 9, 13), 3, "bf16"),
    (128, 64, 32, "abspe", (3, 5, 17), 4, "bf16"),
    (64, 32, 8, "rola", (4, 8, 8), 2, "bf16"),
    (128, 32, 16, "rola", (3, 7, 11), 3, "bf16"),
    (128, 64, 32, "rola", (5, 9, 13), 3, "f32"),
    (64, 64, 16, "abspe", (3, 6, 7), 2, "f32"),
]


@pytest.mark.parametrize("D,bs,r,mode,grid,keep,dtype", TOKEN_GATE)
def test_token_gate_layers(D, bs, r, mode, grid, keep, dtype):
    """Token-wise gated fusion (RoLA §4.4) against the oracle."""
    p = r // 2
    lp = (p // 2, p // 4, p - p // 2 - p // 4) if mode == "rola" else (0, 0, 0)
    pairs = (12, 10, 10) if D == 64 else (22, 21, 21)
    cfg = T.custom(synth.wan13b(), name=f"token gate D{D} bs{bs} r{r} {mode} {grid} k{keep} {dtype}", B=2, H=3,
                   D=D, T=grid[0], Hg=grid[1], Wg=grid[2], block=bs, keep=keep, rank=r, lr_mode=mode, lr_pairs=lp,
                   pairs=pairs, dtype=dtype, seed=9, gate="token")
    _full_check(cfg)


SILU = [
    # D, block, rank, mode, grid, keep, dtype, gate: the three flash kernels, both gates
    (128, 64, 32, "rola", (5, 9, 13), 3, "bf16", "head"),
    (128, 64, 32, "abspe", (3, 5, 17), 4, "bf16", "token"),
    (64, 32, 8, "rola", (4, 8, 8), 2, "bf16", "head"),
    (128, 32, 16, "rola", (3, 7, 11), 3, "bf16", "token"),
    (128, 64, 32, "rola", (5, 9, 13), 3, "f32", "head"),
    (64, 64, 16, "abspe", (3, 6, 7), 2, "f32", "token"),
]


@pytest.mark.parametrize("D,bs,r,mode,grid,keep,dtype,gate", SILU)
def test_silu_feature_map_layers(D, bs, r, mode, grid, keep, dtype, gate):
    """SiLU low-rank features (RoLA §5.3) with the mean readout, against the oracle (summary included)."""
    p = r // 2
    lp = (p // 2, p // 4, p - p // 2 - p // 4) if mode == "rola" else (0, 0, 0)
    pairs = (12, 10, 10) if D == 64 else (22, 21, 21)
    cfg = T.custom(synth.wan13b(), name=f"silu D{D} bs{bs} r{r} {mode} {grid} k{keep} {dtype} {gate}", B=2, H=3,
                   D=D, T=grid[0], Hg=grid[1], Wg=grid[2], block=bs, keep=keep, rank=r, lr_mode=mode, lr_pairs=lp,
                   pairs=pairs, dtype=dtype, seed=13, gate=gate, fmap="silu")
    _full_check(cfg)


FAVOR = [
    # D, block, rank, mode, grid, keep, dtype, gate: the three flash kernels and both summary paths,
    # both low-rank variants, both gates, rank 64 (two rank blocks)
    (128, 64, 32, "rola", (5, 9, 13), 3, "bf16", "head"),
    (128, 64, 32, "abspe", (3, 5, 17), 4, "bf16", "head"),
    (128, 64, 64, "rola", (4, 10, 12), 4, "bf16", "token"),
    (128, 64, 16, "abspe", (9, 4, 3), 2, "bf16", "token"),
    (64, 32, 8, "rola", (4, 8, 8), 2, "bf16", "head"),
    (128, 32, 16, "abspe", (3, 7, 11), 3, "bf16", "head"),
    (128, 64, 32, "rola", (5, 9, 13), 3, "f32", "head"),
    (64, 64, 16, "abspe", (3, 6, 7), 2, "f32", "token"),
]


@pytest.mark.parametrize("D,bs,r,mode,grid,keep,dtype,gate", FAVOR)
def test_favor_feature_map_layers(D, bs, r, mode, grid, keep, dtype, gate):
    """FAVOR+ positive random features (RoPeSLR appendix) in the summary and
    the readout, against the oracle (S and z included)."""
    p = r // 2
    lp = (p // 2, p // 4, p - p // 2 - p // 4) if mode == "rola" else (0, 0, 0)
    pairs = (12, 10, 10) if D == 64 else (22, 21, 21)
    cfg = T.custom(synth.wan13b(), name=f"favor D{D} bs{bs} r{r} {mode} {grid} k{keep} {dtype} {gate}", B=2, H=3,
                   D=D, T=grid[0], Hg=grid[1], Wg=grid[2], block=bs, keep=keep, rank=r, lr_mode=mode, lr_pairs=lp,
                   pairs=pairs, dtype=dtype, seed=15, gate=gate, fmap="favor")
    _full_check(cfg)


@pytest.mark.timeout(900)
def test_favor_wan13b_full_size():
    """FAVOR+ features at the full Wan2.1-1.3B shape (sampled query blocks
    of two slices; selection of every slice)."""
    import dataclasses
    _big(dataclasses.replace(synth.wan13b(), fmap="favor"), [(0, 2), (1, 9)], nq=3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_token_gate_very_negative_bias_gives_sparse_branch(dtype):
    cfg = T.custom(synth.wan13b(), name=f"token gate off {dtype}", B=1, H=2, T=3, Hg=5, Wg=9, keep=2, dtype=dtype,
                   gate="token")
    inp = T.make_inputs(cfg)
    inp.params["bg"].fill_(-1e4)
    out, _, o_sp, _ = T.run_layer(inp)
    torch.cuda.synchronize()
    assert torch.equal(out, o_sp)


@pytest.mark.parametrize("grid,keep", [((4, 9, 13), 5), ((21, 30, 52), 52)], ids=["small", "wan13b-grid"])
def test_runs_are_bitwise_reproducible(grid, keep):
    cfg = T.custom(synth.wan13b(), name="repro", B=1, H=4 if grid[0] == 4 else 2, T=grid[0], Hg=grid[1], Wg=grid[2],
                   keep=keep)
    inp = T.make_inputs(cfg)
    a = T.run_layer(inp)
    b = T.run_layer(inp)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_rope3d_matches_oracle():
    cfg = T.custom(synth.wan13b(), name="rope", B=1, H=2, T=3, Hg=5, Wg=7)
    inp = T.make_inputs(cfg)
    got = B.slr_rope3d(inp.q, B.shape_of(cfg), B.rope_of(cfg))
    torch.cuda.synchronize()
    for h in range(cfg.H):
        qs, _, _ = synth.qkv_slice(cfg, 0, h)
        ref = oracle.rope3d(qs, (cfg.T, cfg.Hg, cfg.Wg), cfg.base, cfg.pairs)
        T.assert_close(f"rope h{h}", T.to_host(got[0, h]), ref, "bf16")
    cfg32 = T.custom(synth.tiny(), name="rope32")
    inp = T.make_inputs(cfg32)
    got = B.slr_rope3d(inp.k, B.shape_of(cfg32), B.rope_of(cfg32))
    torch.cuda.synchronize()
    _, ks, _ = synth.qkv_slice(cfg32, 0, 1)
    ref = oracle.rope3d(ks, (cfg32.T, cfg32.Hg, cfg32.Wg), cfg32.base, cfg32.pairs)
    T.assert_close("rope fp32", T.to_host(got[0, 1]), ref, "f32")


def test_select_blocks_and_rotated_outputs():
    cfg = T.custom(synth.wan13b(), name="select", B=2, H=2, T=5, Hg=12, Wg=20, keep=9)  # 19 blocks, tail 48
    inp = T.make_inputs(cfg)
    idx, qr, kr = B.slr_select_blocks(inp.q, inp.k, B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg),
                                      want_rot=True)
    torch.cuda.synchronize()
    differ = 0
    for b in range(cfg.B):
        for h in range(cfg.H):
            qs, ks, _ = synth.qkv_slice(cfg, b, h)
            grid = (cfg.T, cfg.Hg, cfg.Wg)
            rq, rk = oracle.rope3d(qs, grid, cfg.base, cfg.pairs), oracle.rope3d(ks, grid, cfg.base, cfg.pairs)
            s = oracle.block_scores(oracle.block_mean(rq, cfg.block), oracle.block_mean(rk, cfg.block))
            ref, thr, _ = oracle.topk_blocks(s, cfg.keep)
            ig = idx[b, h].cpu().numpy()
            T.check_selection(ig, s, thr, cfg.keep)
            differ += T.rows_differing(ig, ref)
            T.assert_close("q_rot", T.to_host(qr[b, h]), rq, "bf16")
            T.assert_close("k_rot", T.to_host(kr[b, h]), rk, "bf16")
    T.log(f"    rows differing inside the window: {differ}")


def test_select_blocks_with_long_rows():
    """2063 blocks of 32 tokens per slice (keep 100): rows of more than 2048
    scores, the widest row top-k instance (up to 64 keys per lane)."""
    cfg = T.custom(synth.wan13b(), name="select 2063 blocks", B=1, H=1, T=6, Hg=100, Wg=110, block=32, keep=100,
                   seed=17)
    assert cfg.nblk > 2048
    inp = T.make_inputs(cfg)
    idx = B.slr_select_blocks(inp.q, inp.k, B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg))
    torch.cuda.synchronize()
    s = _oracle_scores(cfg, 0, 0)
    ref, thr, _ = oracle.topk_blocks(s, cfg.keep)
    ig = idx[0, 0].cpu().numpy()
    T.check_selection(ig, s, thr, cfg.keep)
    T.log(f"    rows differing inside the window: {T.rows_differing(ig, ref)}")


def test_dense_attention_matches_oracle():
    for dtype in ("bf16", "f32"):
        cfg = T.custom(synth.wan13b(), name=f"dense {dtype}", B=1, H=2, T=3, Hg=7, Wg=11, dtype=dtype)  # L=231
        inp = T.make_inputs(cfg)
        out = B.slr_dense_attention_fwd(inp.q, inp.k, inp.v, B.shape_of(cfg), B.rope_of(cfg))
        torch.cuda.synchronize()
        for h in range(cfg.H):
            qs, ks, vs = synth.qkv_slice(cfg, 0, h)
            grid = (cfg.T, cfg.Hg, cfg.Wg)
            ref = oracle.dense_attention(oracle.rope3d(qs, grid, cfg.base, cfg.pairs),
                                         oracle.rope3d(ks, grid, cfg.base, cfg.pairs), vs, 64)
            T.assert_close(f"dense h{h}", T.to_host(out[0, h]), ref, dtype)


def test_keep_all_equals_dense_plus_lowrank():
    """Keep fraction 100%: the layer equals dense softmax attention plus the
    gated low-rank term (checked GPU against GPU and against the oracle)."""
    cfg = T.custom(synth.wan13b(), name="keep all", B=1, H=3, T=4, Hg=7, Wg=9, keep=4)  # 252 tokens, 4 blocks
    inp = T.make_inputs(cfg)
    out, idx, o_sp, o_lr = T.run_layer(inp)
    dense = B.slr_dense_attention_fwd(inp.q, inp.k, inp.v, B.shape_of(cfg), B.rope_of(cfg))
    torch.cuda.synchronize()
    T.assert_close("o_sp vs dense kernel", T.to_host(o_sp), T.to_host(dense), "bf16")
    g = inp.params["gate"].view(1, -1, 1, 1).double().cpu().numpy()
    T.assert_close("out vs dense + g*o_lr", T.to_host(out), T.to_host(dense) + g * T.to_host(o_lr), "bf16")
    T.check_layer(inp, out, idx, o_sp, o_lr)


# ---- full-size layers (sampled query blocks) -----------------------------

# oracle block scores per (seed, shape, b, h): they do not depend on keep or
# rank, so the sweep points reuse them
_SCORES = {}


def _oracle_scores(cfg, b, h):
    key = (cfg.seed, cfg.gen, cfg.B, cfg.H, cfg.D, cfg.T, cfg.Hg, cfg.Wg, cfg.block, cfg.base, cfg.pairs, b, h)
    if key not in _SCORES:
        qs, ks, _ = synth.qkv_slice(cfg, b, h)
        grid = (cfg.T, cfg.Hg, cfg.Wg)
        rq, rk = oracle.rope3d(qs, grid, cfg.base, cfg.pairs), oracle.rope3d(ks, grid, cfg.base, cfg.pairs)
        _SCORES[key] = oracle.block_scores(oracle.block_mean(rq, cfg.block), oracle.block_mean(rk, cfg.block))
    return _SCORES[key]


def _big(cfg, slices, nq=6, inp=None):
    T.log(f"  case {cfg.name} (full size), slices {slices}")
    inp = T.make_inputs(cfg) if inp is None else inp
    out, idx, o_sp, o_lr = T.run_layer(inp)
    S, z = _summary(inp)
    torch.cuda.synchronize()
    T.check_layer(inp, out, idx, o_sp, o_lr, slices=slices, qblocks_per_slice=nq, S_gpu=S, z_gpu=z)
    # selection of every slice is checked in full (cheap on the oracle)
    for b in range(cfg.B):
        for h in range(cfg.H):
            if (b, h) in slices:
                continue
            s = _oracle_scores(cfg, b, h)
            _, thr, _ = oracle.topk_blocks(s, cfg.keep)
            T.check_selection(idx[b, h].cpu().numpy(), s, thr, cfg.keep)
    del inp, out, idx, o_sp, o_lr
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_wan13b_full_size():
    _big(synth.wan13b(), [(0, 0), (1, 11), (0, 5)])


@pytest.mark.timeout(900)
def test_wan14b_full_size():
    _big(synth.wan14b(), [(0, 0), (1, 39)], nq=4)


@pytest.mark.timeout(900)
def test_hunyuan13b_full_size():
    _big(synth.hunyuan13b(), [(0, 0), (0, 23)], nq=4)


_SWEEP_QKV = {}


def _sweep_inputs(cfg):
    """Inputs of a sweep point: q, k, v are the same for every point (same
    seed and shape) and stay on the device; the projections follow the rank."""
    if "qkv" not in _SWEEP_QKV:
        _SWEEP_QKV.clear()
        base = T.make_inputs(cfg)
        _SWEEP_QKV["qkv"] = (base.q, base.k, base.v)
    q, k, v = _SWEEP_QKV["qkv"]
    pn = synth.lowrank_params(cfg)
    pd = {key: torch.from_numpy(val).to("cuda") for key, val in pn.items()}
    return T.Inputs(cfg, q, k, v, pn, pd)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("point", range(15), ids=[f"keep{p.keep}-r{p.rank}" for p in synth.sweep()])
def test_sweep_points(point):
    """Every keep x rank point of the Wan2.1-1.3B sweep (keep 26/52/103/256/512
    of 512, ranks 16/32/64): the selection of all 24 slices, outputs and S, z
    of two slices on sampled query blocks."""
    cfg = synth.sweep()[point]
    _big(cfg, [(0, 3), (1, 8)], nq=2, inp=_sweep_inputs(cfg))
    if point == len(synth.sweep()) - 1:
        _SWEEP_QKV.clear()
        torch.cuda.empty_cache()

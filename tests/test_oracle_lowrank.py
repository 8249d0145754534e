"""Pins of the oracle's low-rank global branch and the combine.

RoLA (arXiv 2609.06712v3): §4.1 one reusable summary per head at
O(L r D); §4.2 the rank-r branch reuses the backbone's rotary schedule;
§4.3 the rotation is applied after phi so the numerator weights depend on
relative offsets only (App. B.1), which §5.1 / Table 2 measures as a
near-zero "shift residual" (inside-phi rotation and absolute positions do
not have it). RoPeSLR (arXiv 2605.20659), abstract: the absolute 3D PE
variant. The FLOP model is RoPeSLR's appendix ("Context Retrieval":
a full-width linear branch costs 4 B H L D^2) and RoLA App. F (equal
leading matmul FLOPs at r = D/2).
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_rank_attention_rope3d_amd import synth


class _Cfg:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def test_phi_is_elu_plus_one():
    x = np.linspace(-6, 6, 97).reshape(1, -1)
    u = oracle.lowrank_features(x, np.eye(97), (1, 1, 1))
    want = torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64)).numpy() + 1.0
    # torch forms expm1(x) + 1, the oracle exp(x): equal up to rounding order
    np.testing.assert_allclose(u, want, rtol=1e-13, atol=0)


def test_full_rank_rotation_equals_backbone_rope():
    """With as many low-rank pairs as backbone pairs, rotating after phi is
    exactly the backbone 3D RoPE applied to the features (same schedule)."""
    rng = np.random.default_rng(30)
    grid, pairs = (2, 3, 4), (3, 2, 3)
    u = rng.random((24, 16))
    np.testing.assert_allclose(oracle.lowrank_rotate(u, grid, 10000.0, pairs, pairs),
                               oracle.rope3d(u, grid, 10000.0, pairs), atol=1e-15)


def test_truncated_rotation_reuses_first_pairs_of_each_axis():
    """lr pairs (2,1,1) of backbone pairs (5,4,4): chunk t of the feature
    turns like backbone t-pairs 0..1, chunk h like backbone h-pair 0 and
    chunk w like backbone w-pair 0."""
    rng = np.random.default_rng(31)
    grid, pairs, lr = (3, 2, 4), (5, 4, 4), (2, 1, 1)
    L = 24
    u = rng.random((L, 8))
    got = oracle.lowrank_rotate(u, grid, 10000.0, pairs, lr)
    emb = np.zeros((L, 26))
    emb[:, 0:4], emb[:, 10:12], emb[:, 18:20] = u[:, 0:4], u[:, 4:6], u[:, 6:8]
    rot = oracle.rope3d(emb, grid, 10000.0, pairs)
    np.testing.assert_allclose(got, np.concatenate([rot[:, 0:4], rot[:, 10:12], rot[:, 18:20]], 1),
                               atol=1e-15)


def _branch(mode, grid, q, k, v, wq, wk, E, pairs, lr_pairs, eps=1e-6):
    u = oracle.lowrank_features(k, wk, grid, E if mode == "abspe" else None)
    w = oracle.lowrank_features(q, wq, grid, E if mode == "abspe" else None)
    if mode == "rola":
        fk = oracle.lowrank_rotate(u, grid, 10000.0, pairs, lr_pairs)
        fq = oracle.lowrank_rotate(w, grid, 10000.0, pairs, lr_pairs)
    else:
        fk, fq = u, w
    S, z = oracle.lowrank_summary(fk, u, v)
    return oracle.lowrank_readout(fq, w, S, z, eps), (fq, fk, w, u, S, z)


@pytest.mark.parametrize("mode", ["rola", "abspe"])
def test_linear_summary_equals_quadratic_form(mode):
    """The reusable summary gives what the explicit L x L form gives:
    num_l = sum_m <fq_l, fk_m> v_m and den_l = sum_m <w_l, u_m> + eps."""
    rng = np.random.default_rng(32)
    grid, pairs, lr = (2, 3, 4), (4, 2, 2), (2, 1, 1)
    L, D, r = 24, 16, 8
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    wq, wk = rng.standard_normal((D, r)) / 4, rng.standard_normal((D, r)) / 4
    E = tuple(rng.standard_normal((n, r)) * 0.14 for n in grid)
    got, (fq, fk, w, u, S, z) = _branch(mode, grid, q, k, v, wq, wk, E, pairs, lr)
    A = np.array([[fq[a] @ fk[b] for b in range(L)] for a in range(L)])
    Z = np.array([[w[a] @ u[b] for b in range(L)] for a in range(L)])
    want = (A @ v) / (Z.sum(1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def _shift_residual(weights, coords):
    groups = {}
    for a, b in itertools.product(range(len(coords)), repeat=2):
        groups.setdefault(tuple(coords[b] - coords[a]), []).append(weights[a, b])
    return max(max(g) - min(g) for g in groups.values()) / np.abs(weights).max()


def test_shift_residual_zero_outside_phi_nonzero_otherwise():
    """Constant content on every token: the numerator weights of the
    rotate-after-phi branch depend only on the offset (residual ~0); the
    absolute-PE variant and a rotate-before-phi control do not."""
    rng = np.random.default_rng(33)
    grid, pairs, lr = (3, 3, 4), (4, 2, 2), (2, 1, 1)
    L, D, r = 36, 16, 8
    q0, k0 = rng.standard_normal(D), rng.standard_normal(D)
    q, k = np.tile(q0, (L, 1)), np.tile(k0, (L, 1))
    wq, wk = rng.standard_normal((D, r)) / 4, rng.standard_normal((D, r)) / 4
    coords = np.array(list(itertools.product(*(range(n) for n in grid))))
    fq = oracle.lowrank_rotate(oracle.lowrank_features(q, wq, grid), grid, 10000.0, pairs, lr)
    fk = oracle.lowrank_rotate(oracle.lowrank_features(k, wk, grid), grid, 10000.0, pairs, lr)
    assert _shift_residual(fq @ fk.T, coords) < 1e-12
    E = tuple(rng.standard_normal((n, r)) * 0.14 for n in grid)
    aq, ak = oracle.lowrank_features(q, wq, grid, E), oracle.lowrank_features(k, wk, grid, E)
    assert _shift_residual(aq @ ak.T, coords) > 1e-3
    # control: rotate the content first, then phi (position enters inside phi)
    iq = oracle.lowrank_features(oracle.rope3d(q, grid, 10000.0, pairs), wq, grid)
    ik = oracle.lowrank_features(oracle.rope3d(k, grid, 10000.0, pairs), wk, grid)
    assert _shift_residual(iq @ ik.T, coords) > 1e-3


def test_abspe_constant_values_closed_form():
    """V = c: S = z c^T, so O_lr = c (w.z) / (w.z + eps)."""
    rng = np.random.default_rng(34)
    grid = (2, 2, 3)
    L, D, r = 12, 8, 4
    q, k = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    v = np.full((L, D), -1.75)
    wq, wk = rng.standard_normal((D, r)) / 3, rng.standard_normal((D, r)) / 3
    E = tuple(rng.standard_normal((n, r)) * 0.14 for n in grid)
    got, (_, _, w, u, _, z) = _branch("abspe", grid, q, k, v, wq, wk, E, None, None)
    wz = w @ z
    np.testing.assert_allclose(got, np.broadcast_to(-1.75 * (wz / (wz + 1e-6))[:, None], got.shape), rtol=1e-14)


def test_denominator_positive_and_uses_unrotated_features():
    rng = np.random.default_rng(35)
    grid, pairs, lr = (2, 3, 4), (4, 2, 2), (2, 1, 1)
    L, D, r = 24, 16, 8
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    wq, wk = rng.standard_normal((D, r)), rng.standard_normal((D, r))
    _, (fq, fk, w, u, S, z) = _branch("rola", grid, q, k, v, wq, wk, None, pairs, lr)
    assert (u > 0).all() and (w > 0).all()
    np.testing.assert_allclose(z, u.sum(0), rtol=1e-14)


def _tiny_slice():
    cfg = synth.tiny()
    q, k, v = synth.qkv_slice(cfg, 0, 1)
    p = synth.lowrank_params(cfg)
    return cfg, q, k, v, p


def test_gate_zero_gives_sparse_branch_and_output_is_affine_in_gate():
    cfg, q, k, v, p = _tiny_slice()
    r0 = oracle.layer_slice(cfg, q, k, v, p["wq"][1], p["wk"][1], 0.0)
    np.testing.assert_array_equal(r0["out"], r0["o_sp"])
    r1 = oracle.layer_slice(cfg, q, k, v, p["wq"][1], p["wk"][1], 1.0)
    rg = oracle.layer_slice(cfg, q, k, v, p["wq"][1], p["wk"][1], 0.3)
    np.testing.assert_allclose(rg["out"], 0.7 * r0["out"] + 0.3 * r1["out"], rtol=1e-13, atol=1e-13)


def test_tiny_layer_all_blocks_is_dense_plus_lowrank():
    """Keep fraction 100%: the layer equals dense softmax attention plus the
    gated low-rank term."""
    base = synth.tiny()
    cfg = _Cfg(**{f: getattr(base, f) for f in ("T", "Hg", "Wg", "base", "pairs", "block", "lr_mode",
                                                 "lr_pairs", "eps")}, keep=base.nblk)
    _, q, k, v, p = _tiny_slice()
    res = oracle.layer_slice(cfg, q, k, v, p["wq"][1], p["wk"][1], 0.4)
    qr, kr = res["q_rot"], res["k_rot"]
    s = qr @ kr.T / 8.0
    e = np.exp(s - s.max(1, keepdims=True))
    dense = (e / e.sum(1, keepdims=True)) @ v
    np.testing.assert_allclose(res["o_sp"].reshape(-1, 64), dense, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res["out"].reshape(-1, 64), dense + 0.4 * res["o_lr"].reshape(-1, 64),
                               rtol=1e-12, atol=1e-12)


def test_flop_model_matches_full_width_linear_branch_at_half_rank():
    """RoPeSLR appendix: a full-width linear branch costs 4 B H L D^2; RoLA
    App. F: the rank-r branch has equal leading matmul FLOPs at r = D/2."""
    for cfg in (synth.wan13b(), synth.wan14b(), synth.hunyuan13b()):
        half = synth.Layer(**{**cfg.__dict__, "rank": cfg.D // 2})
        assert half.flops()["lowrank"] == 4.0 * cfg.B * cfg.H * cfg.L * cfg.D ** 2
    # about 10x fewer FLOPs than dense at ~90% sparsity (RoPeSLR abstract)
    f = synth.wan13b().flops()
    assert 9.5 < f["dense"] / f["sparse"] < 10.0


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_abspe_table_follows_its_axis(axis):
    """With zero content projection and only one non-zero axis table, the
    feature is constant along the other two axes and varies along its own."""
    rng = np.random.default_rng(36)
    grid, r = (3, 4, 5), 4
    E = [np.zeros((n, r)) for n in grid]
    E[axis] = rng.standard_normal((grid[axis], r))
    u = oracle.lowrank_features(np.ones((60, 2)), np.zeros((2, r)), grid, tuple(E))
    u = u.reshape(*grid, r)
    other = tuple(a for a in range(3) if a != axis)
    assert np.ptp(u, axis=other).max() == 0.0
    assert np.ptp(u, axis=axis).min() > 0.0
    want = np.exp(np.minimum(E[axis], 0)) + np.maximum(E[axis], 0)  # elu(x) + 1
    np.testing.assert_allclose(np.moveaxis(u, axis, 0)[:, 0, 0], want, rtol=1e-15)


# ---- SiLU feature map (RoLA §5.3, Table 6: the best of the tested activations) ----

def test_silu_is_x_times_sigmoid():
    x = np.linspace(-30, 30, 241).reshape(1, -1)
    u = oracle.lowrank_features(x, np.eye(241), (1, 1, 1), fmap="silu")
    want = torch.nn.functional.silu(torch.tensor(x, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(u, want, rtol=1e-13, atol=1e-300)
    assert u.min() < -0.27   # sign-indefinite (minimum -0.2785 near x = -1.28)


@pytest.mark.parametrize("mode", ["rola", "abspe"])
def test_silu_mean_readout_equals_quadratic_form(mode):
    """With SiLU features the readout is the mean over the L tokens:
    O_lr,l = (1/L) sum_m <fq_l, fk_m> v_m, from the explicit L x L form."""
    rng = np.random.default_rng(36)
    grid, pairs, lr = (2, 3, 4), (4, 2, 2), (2, 1, 1)
    L, D, r = 24, 16, 8
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    wq, wk = rng.standard_normal((D, r)) / 4, rng.standard_normal((D, r)) / 4
    E = tuple(rng.standard_normal((n, r)) * 0.14 for n in grid)
    Ex = E if mode == "abspe" else None
    u = oracle.lowrank_features(k, wk, grid, Ex, fmap="silu")
    w = oracle.lowrank_features(q, wq, grid, Ex, fmap="silu")
    if mode == "rola":
        fk = oracle.lowrank_rotate(u, grid, 10000.0, pairs, lr)
        fq = oracle.lowrank_rotate(w, grid, 10000.0, pairs, lr)
    else:
        fk, fq = u, w
    S, z = oracle.lowrank_summary(fk, u, v)
    got = oracle.lowrank_readout(fq, w, S, z, 1e-6, count=float(L))
    A = np.array([[fq[a] @ fk[b] for b in range(L)] for a in range(L)])
    np.testing.assert_allclose(got, (A @ v) / L, rtol=1e-12, atol=1e-13)


def test_silu_outside_rotation_keeps_zero_shift_residual():
    """Position-free SiLU features rotated after the activation give offset-
    only numerator weights, as elu + 1 does (RoLA §4.3, App. B.1)."""
    rng = np.random.default_rng(37)
    grid, pairs, lr = (3, 3, 4), (4, 2, 2), (2, 1, 1)
    L, D, r = 36, 16, 8
    q = np.tile(rng.standard_normal(D), (L, 1))
    k = np.tile(rng.standard_normal(D), (L, 1))
    wq, wk = rng.standard_normal((D, r)) / 4, rng.standard_normal((D, r)) / 4
    coords = np.array(list(itertools.product(*(range(n) for n in grid))))
    fq = oracle.lowrank_rotate(oracle.lowrank_features(q, wq, grid, fmap="silu"), grid, 10000.0, pairs, lr)
    fk = oracle.lowrank_rotate(oracle.lowrank_features(k, wk, grid, fmap="silu"), grid, 10000.0, pairs, lr)
    assert _shift_residual(fq @ fk.T, coords) < 1e-12
    iq = oracle.lowrank_features(oracle.rope3d(q, grid, 10000.0, pairs), wq, grid, fmap="silu")
    ik = oracle.lowrank_features(oracle.rope3d(k, grid, 10000.0, pairs), wk, grid, fmap="silu")
    assert _shift_residual(iq @ ik.T, coords) > 1e-3


def test_silu_layer_uses_mean_readout_and_token_gate_ignores_the_scale():
    """The layer with fmap = silu reads out S / L; under the token gate any
    positive per-row scale of O_lr cancels (RMS alignment), so the gated
    output equals the one computed from the unnormalised numerator."""
    base = synth.tiny()
    cfg = synth.Layer(**{**base.__dict__, "fmap": "silu", "eps": 1e-12})
    q, k, v = synth.qkv_slice(cfg, 0, 1)
    p = synth.lowrank_params(cfg)
    wg, bg = np.random.default_rng(38).standard_normal(cfg.D) * 0.1, -0.3
    res = oracle.layer_slice(cfg, q, k, v, p["wq"][1], p["wk"][1], 0.0, token_gate_wb=(wg, bg))
    D = cfg.D
    o_lr = res["o_lr"].reshape(-1, D)
    rows = np.arange(o_lr.shape[0])
    valid = rows < cfg.L
    unnorm = o_lr[valid] * cfg.L
    qrows = np.asarray(q, np.float64)[rows[valid]]
    out2, _ = oracle.token_gate(qrows, wg, bg, res["o_sp"].reshape(-1, D)[valid], unnorm, cfg.eps)
    # (rows whose low-rank RMS is tiny still feel eps = 1e-12 at ~1e-11)
    np.testing.assert_allclose(res["out"].reshape(-1, D)[valid], out2, rtol=1e-9, atol=1e-10)


# ---- rotation order: RoLA §5.1 / Table 2 (outside vs inside vs no RoPE) ----

def _offset_range(weights, coords):
    """Spread over the offsets of the numerator weight (one representative
    per offset), relative to the largest weight: zero for a position-blind
    map."""
    groups = {}
    for a, b in itertools.product(range(len(coords)), repeat=2):
        groups.setdefault(tuple(coords[b] - coords[a]), []).append(weights[a, b])
    reps = np.array([g[0] for g in groups.values()])
    return float(np.ptp(reps) / np.abs(weights).max())


@pytest.mark.parametrize("fmap", ["elu1", "silu", "favor"])
def test_rotation_order_controls_match_table2_contrast(fmap):
    """Content-controlled input (the same q and k row at every token), as in
    RoLA §5.1: only the rotation outside the activation has a zero shift
    residual and a non-zero offset range; inside the activation the residual
    is clearly non-zero; without RoPE the residual is zero but so is the
    offset range (position-blind)."""
    rng = np.random.default_rng(40)
    grid, pairs, lr = (3, 3, 4), (4, 2, 2), (2, 1, 1)
    L, D, r = 36, 16, 8
    q = np.tile(rng.standard_normal(D), (L, 1))
    k = np.tile(rng.standard_normal(D), (L, 1))
    v = rng.standard_normal((L, D))
    wq, wk = rng.standard_normal((D, r)) / 4, rng.standard_normal((D, r)) / 4
    omega = rng.standard_normal((r, r)) if fmap == "favor" else None
    coords = np.array(list(itertools.product(*(range(n) for n in grid))))
    res = {}
    for order in oracle.LR_ORDERS:
        _, fq, fk, _, _ = oracle.lowrank_branch(q, k, v, wq, wk, grid, 10000.0, pairs, lr, order=order, fmap=fmap,
                                                omega=omega)
        A = fq @ fk.T
        res[order] = (_shift_residual(A, coords), _offset_range(A, coords))
    assert res["outside"][0] < 1e-12 and res["outside"][1] > 1e-3
    assert res["inside"][0] > 1e-3
    assert res["none"][0] == 0.0 and res["none"][1] == 0.0


def test_rotation_order_outside_is_the_layer_branch():
    """The "outside" order is exactly the layer's rotary low-rank branch."""
    cfg, q, k, v, p = _tiny_slice()
    res = oracle.layer_slice(cfg, q, k, v, p["wq"][1], p["wk"][1], 0.5)
    got, *_ = oracle.lowrank_branch(q, k, v, p["wq"][1], p["wk"][1], (cfg.T, cfg.Hg, cfg.Wg), cfg.base, cfg.pairs,
                                    cfg.lr_pairs, order="outside", eps=cfg.eps)
    np.testing.assert_array_equal(got, res["o_lr"].reshape(-1, cfg.D)[:cfg.L])


# ---- FAVOR+ positive random features (RoPeSLR appendix: the softmax
# exponential kernel linearised by positive random features, Performers) ----

def _favor_features(x, omega):
    """FAVOR+ features of the rows of x [n, d] with m = omega.shape[0] random
    directions, through the oracle: x is embedded as the first d of m
    components (the projection W = [I_d | 0]), so omega's first d columns are
    the directions that act."""
    n, d = x.shape
    m = omega.shape[0]
    W = np.zeros((d, m))
    W[:, :d] = np.eye(d)
    return oracle.lowrank_features(x, W, (n, 1, 1), fmap="favor", omega=omega)


def test_favor_features_are_positive():
    rng = np.random.default_rng(41)
    r = 16
    x = rng.standard_normal((200, r)) * 2.0
    u = oracle.lowrank_features(x, np.eye(r), (200, 1, 1), fmap="favor", omega=rng.standard_normal((r, r)))
    assert np.isfinite(u).all() and (u > 0).all()


def test_favor_dot_product_is_an_unbiased_estimate_of_exp_kernel():
    """Monte-Carlo check with a fixed seed: u(x) . u(y) over m = 2048 random
    features estimates exp(x . y) within 5 standard errors, the per-feature
    variance being exp(|x|^2 + |y|^2 + 4 x.y) - exp(2 x.y) for Gaussian
    directions. A wrong sign or factor of the |x|^2/2 term, or a 1/r
    instead of 1/sqrt(r) normalisation, misses by far more."""
    rng = np.random.default_rng(42)
    m, d = 2048, 3
    omega = rng.standard_normal((m, m))
    for trial in range(6):
        x, y = rng.standard_normal((2, d)) * 0.4
        ux, uy = _favor_features(np.stack([x, y]), omega)
        est = float(ux @ uy)
        exact = math.exp(float(x @ y))
        var = math.exp(float(x @ x + y @ y + 4 * x @ y)) - math.exp(2 * float(x @ y))
        assert abs(est - exact) <= 5 * math.sqrt(var / m), (trial, est, exact)


def test_favor_branch_approximates_softmax_attention():
    """With many random features and no positional rotation, the linear
    branch's readout sum_m u(x_l).u(y_m) v_m / sum_m u(x_l).u(y_m)
    approaches softmax attention with logits x_l . y_m (the kernel FAVOR+
    linearises): its distance to softmax attention is a small fraction
    (here < 0.35, at m = 2048 features) of the distance between softmax
    attention and the plain mean of v (what a feature map that ignores the
    logits would give)."""
    rng = np.random.default_rng(43)
    m, d, L, D = 2048, 3, 12, 5
    omega = rng.standard_normal((m, m))
    x = rng.standard_normal((L, d)) * 0.4
    y = rng.standard_normal((L, d)) * 0.4
    v = rng.standard_normal((L, D))
    fq, fk = _favor_features(x, omega), _favor_features(y, omega)
    S, z = oracle.lowrank_summary(fk, fk, v)
    got = oracle.lowrank_readout(fq, fq, S, z, 1e-12)
    s = x @ y.T
    p = np.exp(s - s.max(1, keepdims=True))
    want = (p / p.sum(1, keepdims=True)) @ v
    flat = np.broadcast_to(v.mean(0), want.shape)
    assert np.linalg.norm(got - want) < 0.35 * np.linalg.norm(flat - want)


def test_favor_uses_rows_of_omega():
    """Interface convention: feature c uses row c of omega (omega[c, j]
    multiplies component j of x W)."""
    omega = np.array([[1.0, 2.0], [3.0, 4.0]])
    x = np.array([[0.5, -1.0]])
    u = oracle.lowrank_features(x, np.eye(2), (1, 1, 1), fmap="favor", omega=omega)
    sq = 0.25 + 1.0
    np.testing.assert_allclose(u[0], [math.exp(0.5 - 2.0 - sq / 2) / math.sqrt(2),
                                      math.exp(1.5 - 4.0 - sq / 2) / math.sqrt(2)], rtol=1e-15)


@pytest.mark.parametrize("mode", ["rola", "abspe"])
def test_favor_linear_summary_equals_quadratic_form(mode):
    """The reusable summary with FAVOR+ features equals the explicit L x L
    form (normaliser w . z + eps, as for elu + 1: the features are positive)."""
    rng = np.random.default_rng(44)
    grid, pairs, lr = (2, 3, 4), (4, 2, 2), (2, 1, 1)
    L, D, r = 24, 16, 8
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    wq, wk = rng.standard_normal((D, r)) / 4, rng.standard_normal((D, r)) / 4
    omega = rng.standard_normal((r, r))
    E = tuple(rng.standard_normal((n, r)) * 0.14 for n in grid) if mode == "abspe" else None
    u = oracle.lowrank_features(k, wk, grid, E, fmap="favor", omega=omega)
    w = oracle.lowrank_features(q, wq, grid, E, fmap="favor", omega=omega)
    fk, fq = (oracle.lowrank_rotate(u, grid, 10000.0, pairs, lr), oracle.lowrank_rotate(w, grid, 10000.0, pairs, lr)) \
        if mode == "rola" else (u, w)
    S, z = oracle.lowrank_summary(fk, u, v)
    got = oracle.lowrank_readout(fq, w, S, z, 1e-6)
    A = np.array([[fq[a] @ fk[b] for b in range(L)] for a in range(L)])
    Z = np.array([[w[a] @ u[b] for b in range(L)] for a in range(L)])
    np.testing.assert_allclose(got, (A @ v) / (Z.sum(1, keepdims=True) + 1e-6), rtol=1e-12, atol=1e-13)

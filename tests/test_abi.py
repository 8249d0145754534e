"""The C ABI library loads, exports what include/slr.h declares, and rejects
bad arguments on the host before any HIP call (so these run without a GPU).
Pointers below are never dereferenced: every call is rejected first."""
import ctypes
import os
import re

import pytest

from sparse_rank_attention_rope3d_amd import binding as B
from sparse_rank_attention_rope3d_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libslr.so not built")

FAKE = 0x10000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x10008


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slr_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(B.EXPORTS)
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (B.SLR_OK, B.SLR_EINVAL, B.SLR_EUNSUPPORTED, B.SLR_EWORKSPACE, B.SLR_EHIP):
        assert B.status_string(code).startswith("SLR_")
    assert "unknown" in B.status_string(12345)


def _cfgs(layer=None):
    layer = layer or synth.wan13b()
    shape, rope, sparse = B.shape_of(layer), B.rope_of(layer), B.sparse_of(layer)
    lr = B.SlrLowrankCfg(layer.rank, B.SLR_LR_ROPE_OUTSIDE, *layer.lr_pairs, 1e-6, FAKE, FAKE, FAKE, None, None, None)
    return shape, rope, sparse, lr


def _attn(shape, rope, sparse, lr, q=FAKE, k=FAKE, v=FAKE, out=FAKE, ws=None, ws_bytes=0, idx=None):
    r = ctypes.byref
    return B.lib().slr_attention_fwd(r(shape), r(rope), r(sparse), r(lr), q, k, v, out, idx, None, None, ws,
                                     ws_bytes, None)


def test_workspace_bytes_matches_layout_size():
    shape, rope, sparse, lr = _cfgs()
    n = B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lr)
    layer = synth.wan13b()
    # bf16, D = 128, 64-token blocks: rotated q plus per-block [K | V^T] tiles
    rot = 3 * (layer.B * layer.H * layer.nblk * layer.block * layer.D * 2)
    assert rot < n < rot + 128 * 2 ** 20
    assert B.slr_workspace_bytes(B.SLR_OP_ROPE3D, shape, rope) < 2 ** 20
    assert B.slr_workspace_bytes(B.SLR_OP_DENSE, shape, rope) >= rot
    # other shapes keep plain rotated q and k copies
    small = synth.tiny()
    n32 = B.slr_workspace_bytes(B.SLR_OP_ATTENTION, B.shape_of(small), B.rope_of(small), B.sparse_of(small),
                                B.SlrLowrankCfg(small.rank, 0, *small.lr_pairs, 1e-6, FAKE, FAKE, FAKE, None, None,
                                                None))
    assert n32 >= 2 * small.B * small.H * small.nblk * small.block * small.D * 4


@pytest.mark.parametrize("field,value,code", [
    ("D", 96, B.SLR_EUNSUPPORTED), ("D", 7, B.SLR_EINVAL), ("B", 0, B.SLR_EINVAL), ("T", 0, B.SLR_EINVAL),
    ("dtype", 5, B.SLR_EINVAL), ("H", 70000, B.SLR_EUNSUPPORTED)])
def test_bad_shape(field, value, code):
    shape, rope, sparse, lr = _cfgs()
    setattr(shape, field, value)
    assert _attn(shape, rope, sparse, lr) == code


@pytest.mark.parametrize("pairs", [(22, 21, 20), (23, 21, 21), (-1, 33, 32)])
def test_bad_rotary_pairs(pairs):
    shape, rope, sparse, lr = _cfgs()
    rope.pairs_t, rope.pairs_h, rope.pairs_w = pairs
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL


def test_bad_base():
    shape, rope, sparse, lr = _cfgs()
    rope.base = 1.0
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL
    rope.base = float("nan")
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL


@pytest.mark.parametrize("block,keep", [(48, 52), (64, 0), (64, 513), (16, 4)])
def test_bad_sparse(block, keep):
    shape, rope, sparse, lr = _cfgs()
    sparse.block, sparse.keep = block, keep
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL


@pytest.mark.parametrize("change", ["rank", "pairs_sum", "pairs_axis", "mode", "eps", "wq", "abspe_tables",
                                    "gate_mode", "head_gate_null", "token_wg_null", "token_bg_null",
                                    "token_wg_misaligned", "feature_map"])
def test_bad_lowrank(change):
    shape, rope, sparse, lr = _cfgs()
    if change == "rank":
        lr.rank = 24
    elif change == "pairs_sum":
        lr.lr_pairs_t = 9
    elif change == "pairs_axis":
        rope.pairs_t, rope.pairs_h, rope.pairs_w = 2, 31, 31   # lr t pairs 8 > 2
    elif change == "mode":
        lr.mode = 3
    elif change == "eps":
        lr.eps = 0.0
    elif change == "wq":
        lr.Wq = None
    elif change == "abspe_tables":
        lr.mode = B.SLR_LR_ABS_PE
    elif change == "gate_mode":
        lr.gate_mode = 2
    elif change == "feature_map":
        lr.feature_map = 2
    elif change == "head_gate_null":
        lr.gate = None
    elif change.startswith("token"):
        lr.gate_mode, lr.gate, lr.Wg, lr.bg = B.SLR_GATE_TOKEN, None, FAKE, FAKE
        if change == "token_wg_null":
            lr.Wg = None
        elif change == "token_bg_null":
            lr.bg = None
        else:
            lr.Wg = MISALIGNED + 4     # 4-byte aligned, not 16
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL


def test_token_gate_config_is_accepted_by_sizing():
    """With the gate pointers in place the token gate needs no extra
    workspace and passes the host checks (sizing does not read pointers)."""
    shape, rope, sparse, lr = _cfgs()
    n_head = B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lr)
    lr.gate_mode, lr.gate, lr.Wg, lr.bg = B.SLR_GATE_TOKEN, None, FAKE, FAKE
    assert B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lr) == n_head


def test_null_and_misaligned_tensors():
    shape, rope, sparse, lr = _cfgs()
    assert _attn(shape, rope, sparse, lr, q=None) == B.SLR_EINVAL
    assert _attn(shape, rope, sparse, lr, v=MISALIGNED) == B.SLR_EINVAL
    assert _attn(shape, rope, sparse, lr, out=None) == B.SLR_EINVAL
    assert _attn(shape, rope, sparse, lr, idx=FAKE + 2) == B.SLR_EINVAL


def test_workspace_missing_or_short():
    shape, rope, sparse, lr = _cfgs()
    need = B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lr)
    assert _attn(shape, rope, sparse, lr) == B.SLR_EWORKSPACE
    assert _attn(shape, rope, sparse, lr, ws=FAKE, ws_bytes=need - 1) == B.SLR_EWORKSPACE
    assert _attn(shape, rope, sparse, lr, ws=FAKE + 16, ws_bytes=need) == B.SLR_EWORKSPACE  # not 256-aligned


def test_other_entry_points_validate():
    shape, rope, sparse, lr = _cfgs()
    r = ctypes.byref
    L = B.lib()
    assert L.slr_rope3d(r(shape), r(rope), FAKE, FAKE, None, 0, None) == B.SLR_EINVAL      # aliasing
    assert L.slr_rope3d(r(shape), r(rope), FAKE, FAKE + 16, None, 0, None) == B.SLR_EWORKSPACE
    assert L.slr_select_blocks(r(shape), r(rope), r(sparse), FAKE, FAKE, None, None, None, None, 0,
                               None) == B.SLR_EINVAL
    assert L.slr_lowrank_summary(r(shape), r(rope), r(lr), FAKE, FAKE, None, FAKE, None, 0, None) == B.SLR_EINVAL
    assert L.slr_dense_attention_fwd(r(shape), r(rope), FAKE, FAKE, MISALIGNED, FAKE, None, 0,
                                     None) == B.SLR_EINVAL
    n = ctypes.c_size_t()
    assert L.slr_workspace_bytes(9, r(shape), r(rope), None, None, r(n)) == B.SLR_EINVAL
    assert L.slr_workspace_bytes(B.SLR_OP_ATTENTION, r(shape), r(rope), None, r(lr), r(n)) == B.SLR_EINVAL


GIB = 2 ** 30   # the [B,H,L,D] fakes below sit 1 GiB apart: their byte ranges do not overlap


def ctypes_copy(st):
    """A field-by-field copy of a ctypes structure."""
    out = type(st)()
    ctypes.pointer(out)[0] = st
    return out


def _bwd(shape, rope, sparse, lr, q=FAKE, k=FAKE + GIB, v=FAKE + 2 * GIB, idx=FAKE + 8 * GIB + 0x3000,
         osp=FAKE + 3 * GIB, lse=FAKE + 8 * GIB + 0xc000, S=None, z=None, dout=FAKE + 4 * GIB, dq=FAKE + 5 * GIB,
         dk=FAKE + 6 * GIB,
         dv=FAKE + 7 * GIB, dwq=FAKE + 8 * GIB + 0x9000, dwk=FAKE + 8 * GIB + 0xa000, dg=FAKE + 8 * GIB + 0xb000,
         dwg=FAKE + 8 * GIB + 0x10000, dbg=FAKE + 8 * GIB + 0x11000, det=FAKE + 8 * GIB + 0xd000,
         deh=FAKE + 8 * GIB + 0xe000, dew=FAKE + 8 * GIB + 0xf000, ws=None, ws_bytes=0):
    r = ctypes.byref
    return B.lib().slr_attention_bwd(r(shape), r(rope), r(sparse), r(lr), q, k, v, idx, osp, lse, S, z, dout, dq, dk, dv,
                                     dwq, dwk, dg, dwg, dbg, det, deh, dew, ws, ws_bytes, None)


def test_backward_validates_before_launching():
    shape, rope, sparse, lr = _cfgs()
    need = B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lr)
    layer = synth.wan13b()
    bhld = layer.B * layer.H * layer.L * layer.D
    # rotated q, k; no fp32 low-rank gradient parts: the streaming dQ and dK/dV
    # kernels form them from the MFMA low-rank kernels' rank vectors
    assert 2 * 2 * bhld < need < (2 * 2 + 3 * 4) * bhld
    # the token gate's query side runs on the VALU kernel, which stores dq_lr in fp32
    tok = ctypes_copy(lr)
    tok.gate_mode, tok.gate, tok.Wg, tok.bg = B.SLR_GATE_TOKEN, None, FAKE, FAKE
    assert B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, tok) > need + 4 * bhld
    assert _bwd(shape, rope, sparse, lr) == B.SLR_EWORKSPACE
    assert _bwd(shape, rope, sparse, lr, ws=FAKE, ws_bytes=need - 1) == B.SLR_EWORKSPACE
    for bad in ("q", "osp", "lse", "dout", "dq", "dv", "dwq", "dg"):
        assert _bwd(shape, rope, sparse, lr, **{bad: None}) == B.SLR_EINVAL, bad
    assert _bwd(shape, rope, sparse, lr, idx=FAKE + 2) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, dk=MISALIGNED) == B.SLR_EINVAL
    # the forward's saved summary: both or neither, 4-byte aligned
    S, z = FAKE + 8 * GIB + 0x20000, FAKE + 8 * GIB + 0x30000
    assert _bwd(shape, rope, sparse, lr, S=S, z=z) == B.SLR_EWORKSPACE
    assert _bwd(shape, rope, sparse, lr, S=S) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, z=z) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, S=S + 2, z=z) == B.SLR_EINVAL
    # outputs may not share a byte with an input or with each other
    nbytes = 2 * layer.B * layer.H * layer.L * layer.D
    assert _bwd(shape, rope, sparse, lr, dq=FAKE) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, dv=FAKE + 2 * GIB + 0x2000) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, dk=FAKE + 5 * GIB + 0x6000) == B.SLR_EINVAL
    # partial overlaps: the last bytes of an input, the first bytes of another output
    assert _bwd(shape, rope, sparse, lr, dq=FAKE + 4 * GIB + nbytes - 16) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, dk=FAKE + 7 * GIB - nbytes + 16) == B.SLR_EINVAL
    # adjacent ranges are fine (the call then stops at the missing workspace)
    assert _bwd(shape, rope, sparse, lr, dq=FAKE + 4 * GIB + nbytes) == B.SLR_EWORKSPACE
    assert _bwd(shape, rope, sparse, lr, dk=FAKE + 7 * GIB - nbytes) == B.SLR_EWORKSPACE


def test_backward_absolute_pe_needs_the_table_gradients():
    shape, rope, sparse, lr = _cfgs()
    lr.mode, lr.Et, lr.Eh, lr.Ew = B.SLR_LR_ABS_PE, FAKE, FAKE, FAKE
    n_abs = B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lr)
    layer = synth.wan13b()
    # the per-token gradient of x W + E [BH, L, r] fp32 comes on top
    assert n_abs >= 4 * layer.B * layer.H * layer.L * layer.rank
    assert _bwd(shape, rope, sparse, lr) == B.SLR_EWORKSPACE
    for bad in ("det", "deh", "dew"):
        assert _bwd(shape, rope, sparse, lr, **{bad: None}) == B.SLR_EINVAL, bad
    assert _bwd(shape, rope, sparse, lr, dew=FAKE + 2) == B.SLR_EINVAL
    # the rotary variant ignores them
    shape, rope, sparse, lr = _cfgs()
    assert _bwd(shape, rope, sparse, lr, det=None, deh=None, dew=None) == B.SLR_EWORKSPACE


def test_backward_token_gate_outputs():
    """The token gate's backward returns dW_g, db_g (required) instead of
    dgate (ignored), and needs room for the sparse branch's upstream
    gradient (bf16 [B,H,L,D]); the per-head gate's bf16 rank-32 layout
    instead holds the MFMA low-rank path's four bf16 [B,H,L,R] per-token
    rank vectors, which the token gate (VALU path) does without."""
    shape, rope, sparse, lr = _cfgs()
    n_head = B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lr)
    lr.gate_mode, lr.gate, lr.Wg, lr.bg = B.SLR_GATE_TOKEN, None, FAKE, FAKE
    n_tok = B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lr)
    layer = synth.wan13b()
    bhl = layer.B * layer.H * layer.L
    assert n_tok - (n_head - 4 * 2 * bhl * layer.rank) >= 2 * bhl * layer.D
    assert _bwd(shape, rope, sparse, lr, dg=None) == B.SLR_EWORKSPACE
    assert _bwd(shape, rope, sparse, lr, dwg=None) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, dbg=None) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, dbg=FAKE + 2) == B.SLR_EINVAL
    # the per-head gate needs dgate and ignores dW_g, db_g
    shape, rope, sparse, lr = _cfgs()
    assert _bwd(shape, rope, sparse, lr, dg=None) == B.SLR_EINVAL
    assert _bwd(shape, rope, sparse, lr, dwg=None, dbg=None) == B.SLR_EWORKSPACE


def test_training_forward_requires_its_outputs():
    shape, rope, sparse, lr = _cfgs()
    r = ctypes.byref
    L = B.lib()

    def call(idx=FAKE + 0x1000, osp=FAKE + 0x2000, lse=FAKE + 0x3000, S=None, z=None):
        return L.slr_attention_fwd_train(r(shape), r(rope), r(sparse), r(lr), FAKE, FAKE, FAKE, FAKE + 0x4000, idx,
                                         osp, lse, S, z, None, 0, None)
    assert call() == B.SLR_EWORKSPACE
    assert call(idx=None) == B.SLR_EINVAL
    assert call(osp=None) == B.SLR_EINVAL
    assert call(lse=None) == B.SLR_EINVAL
    assert call(lse=FAKE + 2) == B.SLR_EINVAL
    # the saved summary: both or neither, 4-byte aligned
    assert call(S=FAKE + 0x5000, z=FAKE + 0x6000) == B.SLR_EWORKSPACE
    assert call(S=FAKE + 0x5000) == B.SLR_EINVAL
    assert call(z=FAKE + 0x6000) == B.SLR_EINVAL
    assert call(S=FAKE + 0x5002, z=FAKE + 0x6000) == B.SLR_EINVAL


def test_favor_feature_map_needs_omega_and_backward_coverage():
    """FAVOR+ features (SLR_FMAP_FAVOR) need the random directions; the
    backward covers every gate and dtype (the token gate and fp32 layers on
    the VALU low-rank kernels, which need no per-token rank vectors)."""
    shape, rope, sparse, lr = _cfgs()
    lr.feature_map = B.SLR_FMAP_FAVOR
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL          # omega missing
    lr.omega = FAKE + 2
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL          # misaligned
    lr.omega = FAKE
    assert _attn(shape, rope, sparse, lr) == B.SLR_EWORKSPACE
    n_fav = B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lr)
    lr.feature_map = B.SLR_FMAP_ELU1
    n_elu = B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lr)
    nb_elu = B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lr)
    layer = synth.wan13b()
    # four (W omega^T)^T bf16 parts [H, 32, D] on top
    assert n_fav - n_elu >= 4 * 2 * layer.H * 32 * layer.D
    lr.feature_map = B.SLR_FMAP_FAVOR
    # the backward recomputes the summary: two (W_k omega^T)^T parts on top
    nb_fav = B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lr)
    assert nb_fav - nb_elu >= 2 * 2 * layer.H * 32 * layer.D
    assert _bwd(shape, rope, sparse, lr) == B.SLR_EWORKSPACE
    lr.gate_mode, lr.gate, lr.Wg, lr.bg = B.SLR_GATE_TOKEN, None, FAKE, FAKE
    nb_tok = B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lr)
    # no MFMA per-token rank vectors (four bf16 [B,H,L,r]); the sparse branch's upstream gradient instead
    bhl = layer.B * layer.H * layer.L
    assert nb_tok - (nb_fav - 4 * 2 * bhl * layer.rank) >= 2 * bhl * layer.D
    assert _bwd(shape, rope, sparse, lr) == B.SLR_EWORKSPACE
    lr.omega = None
    assert _bwd(shape, rope, sparse, lr) == B.SLR_EINVAL
    lr.omega = FAKE
    small = synth.tiny()   # fp32
    lr32 = B.SlrLowrankCfg(small.rank, 0, *small.lr_pairs, 1e-6, FAKE, FAKE, FAKE, None, None, None)
    lr32.feature_map, lr32.omega = B.SLR_FMAP_FAVOR, FAKE
    assert B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, B.shape_of(small), B.rope_of(small), B.sparse_of(small),
                                 lr32) > 0
    lr.feature_map = 3
    assert _attn(shape, rope, sparse, lr) == B.SLR_EINVAL


def test_noalloc_summary_validates_on_the_host():
    """slr_lowrank_summary_noalloc checks its arguments and the size of its
    fixed scratch before any HIP call."""
    shape, rope, sparse, lr = _cfgs()
    r = ctypes.byref
    L = B.lib()
    assert L.slr_lowrank_summary_noalloc(r(shape), r(rope), r(lr), FAKE, FAKE, None, FAKE, None) == B.SLR_EINVAL
    assert L.slr_lowrank_summary_noalloc(r(shape), r(rope), r(lr), MISALIGNED, FAKE, FAKE, FAKE, None) == B.SLR_EINVAL
    # 1024 slices at rank 64: more partial-sum bytes than the buffer holds, even at one split per slice
    big = synth.Layer(**{**synth.wan13b().__dict__, "B": 16, "H": 64, "rank": 64, "lr_pairs": (16, 8, 8)})
    s2, r2 = B.shape_of(big), B.rope_of(big)
    lr2 = B.SlrLowrankCfg(64, B.SLR_LR_ROPE_OUTSIDE, 16, 8, 8, 1e-6, FAKE, FAKE, FAKE, None, None, None)
    assert L.slr_lowrank_summary_noalloc(r(s2), r(r2), r(lr2), FAKE, FAKE, FAKE, FAKE, None) == B.SLR_ESCRATCH
    assert "scratch" in B.status_string(B.SLR_ESCRATCH)

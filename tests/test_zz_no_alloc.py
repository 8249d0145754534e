"""slr_lowrank_summary_noalloc (the entry point for callers that cannot
allocate: its scratch is the library's fixed per-GPU buffer) against
slr_lowrank_summary with a caller workspace, on two calls in a row, the
second with a smaller input: the bf16 Wan2.1-1.3B layer (24 slices of
32760 tokens), then a small fp32 absolute-PE layer, then the first again
(the same bits as its first call)."""
import dataclasses

import pytest
import torch

import slrtest as T
from sparse_rank_attention_rope3d_amd import binding as B
from sparse_rank_attention_rope3d_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _compare(cfg):
    T.log(f"  case {cfg.name}: B={cfg.B} H={cfg.H} L={cfg.L} r={cfg.rank} {cfg.lr_mode} {cfg.fmap} {cfg.dtype}")
    inp = T.make_inputs(cfg)
    shape, rope, lowrank = B.shape_of(cfg), B.rope_of(cfg), B.lowrank_of(cfg, inp.params)
    # output buffers filled with NaN: every element must be written
    S = torch.full((cfg.B, cfg.H, cfg.rank, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
    z = torch.full((cfg.B, cfg.H, cfg.rank), float("nan"), dtype=torch.float32, device="cuda")
    B.slr_lowrank_summary_noalloc(inp.k, inp.v, shape, rope, lowrank, S=S, z=z)
    S_ref, z_ref = B.slr_lowrank_summary(inp.k, inp.v, shape, rope, lowrank)
    torch.cuda.synchronize()
    T.assert_close("S (no-alloc vs workspace)", T.to_host(S), T.to_host(S_ref), cfg.dtype, branch=True)
    T.assert_close("z (no-alloc vs workspace)", T.to_host(z), T.to_host(z_ref), cfg.dtype, branch=True)
    return S


def test_noalloc_summary_matches_workspace_entry_point_twice():
    big = synth.wan13b()
    first = _compare(big)
    small = dataclasses.replace(synth.wan13b(), name="small abs-PE fp32", B=1, H=3, T=5, Hg=9, Wg=13, rank=16,
                                lr_mode="abspe", lr_pairs=(0, 0, 0), dtype="f32", seed=21)
    _compare(small)
    # a repeat of the first call after the smaller one gives the same bits
    inp = T.make_inputs(big)
    again, _ = B.slr_lowrank_summary_noalloc(inp.k, inp.v, B.shape_of(big), B.rope_of(big),
                                             B.lowrank_of(big, inp.params))
    torch.cuda.synchronize()
    assert torch.equal(again, first)


def test_noalloc_summary_rejects_inputs_beyond_its_buffer():
    """1024 slices at rank 64 need more than the buffer even with one split
    per slice: SLR_ESCRATCH, before anything is launched."""
    cfg = dataclasses.replace(synth.wan13b(), B=16, H=64, rank=64, lr_pairs=(16, 8, 8))
    shape, rope = B.shape_of(cfg), B.rope_of(cfg)
    w = torch.zeros(cfg.H * cfg.D * cfg.rank, dtype=torch.float32, device="cuda")
    lr = B.SlrLowrankCfg(cfg.rank, B.SLR_LR_ROPE_OUTSIDE, *cfg.lr_pairs, 1e-6, w.data_ptr(), w.data_ptr(), None,
                         None, None, None)
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")   # never read: the call stops first
    with pytest.raises(B.SlrError) as e:
        B.slr_lowrank_summary_noalloc(x, x, shape, rope, lr, S=w, z=w)
    assert e.value.code == B.SLR_ESCRATCH

"""The layer forward replays in a HIP graph.

slr_attention_fwd allocates nothing and issues no memset: every launch goes
on the caller's stream, so a caller can capture a whole layer forward once
and replay it. Each replay is checked against the eager result, with eager
work and synchronisations between the replays.
"""
import pytest
import torch

from sparse_rank_attention_rope3d_amd import binding as B
from sparse_rank_attention_rope3d_amd import synth

import slrtest as T

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", ["head", "token"])
def test_layer_forward_replays_in_a_graph(gate):
    cfg = T.custom(synth.wan13b(), name=f"graph {gate}", B=1, H=3, T=4, Hg=9, Wg=13, keep=3, gate=gate)
    T.log(f"  case {cfg.name}: L={cfg.L} nblk={cfg.nblk} keep={cfg.keep}")
    inp = T.make_inputs(cfg)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, inp.params)
    ws = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lowrank), "cuda")
    want = B.slr_attention_fwd(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank, ws=ws)
    torch.cuda.synchronize()

    out = torch.empty_like(inp.q)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # one eager call on the capture stream first
        B.slr_attention_fwd(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        B.slr_attention_fwd(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        ws.fill_(0x5A)          # the replay must not depend on what the workspace held
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep} differs from the eager result"


@pytest.mark.parametrize("keep_summary", [False, True], ids=["recomputed summary", "saved summary"])
def test_training_step_replays_in_a_graph(keep_summary):
    """The training forward and the backward capture together: the backward
    allocates nothing either and clears its scratch with a kernel (no memset
    nodes); every replay equals the eager gradients bit for bit, with the
    backward recomputing the low-rank summary or taking the forward's."""
    cfg = T.custom(synth.wan13b(), name="graph training step", B=1, H=2, T=4, Hg=9, Wg=13, keep=3)
    inp = T.make_inputs(cfg)
    dout = torch.empty_like(inp.q)
    for b in range(cfg.B):
        for h in range(cfg.H):
            dout[b, h] = T.to_device(synth.dout_slice(cfg, b, h), cfg.dtype)
    shape, rope, sparse = B.shape_of(cfg), B.rope_of(cfg), B.sparse_of(cfg)
    lowrank = B.lowrank_of(cfg, inp.params)
    wsf = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION, shape, rope, sparse, lowrank), "cuda")
    wsb = B.workspace(B.slr_workspace_bytes(B.SLR_OP_ATTENTION_BWD, shape, rope, sparse, lowrank), "cuda")
    summ = None
    if keep_summary:
        summ = (torch.empty((cfg.B, cfg.H, cfg.rank, cfg.D), dtype=torch.float32, device="cuda"),
                torch.empty((cfg.B, cfg.H, cfg.rank), dtype=torch.float32, device="cuda"))
    saved = B.slr_attention_fwd_train(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank, ws=wsf, summary=summ)
    want = B.slr_attention_bwd(inp.q, inp.k, inp.v, saved[1], saved[2], saved[3], dout, shape, rope, sparse, lowrank,
                               ws=wsb, summary=summ)
    want = [t.clone() for t in want[:6]]
    torch.cuda.synchronize()

    outs = tuple(torch.empty_like(t) for t in saved)
    grads = tuple(torch.empty_like(t) for t in want) + (None,)

    def step():
        B.slr_attention_fwd_train(inp.q, inp.k, inp.v, shape, rope, sparse, lowrank, ws=wsf, outs=outs,
                                  summary=summ)
        B.slr_attention_bwd(inp.q, inp.k, inp.v, outs[1], outs[2], outs[3], dout, shape, rope, sparse, lowrank,
                            ws=wsb, grads=grads, summary=summ)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in grads[:6]:
            t.zero_()
        wsb.fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv", "dWq", "dWk", "dgate"), grads[:6], want):
            assert torch.equal(g, w), f"replay {rep}: {name} differs from the eager result"

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

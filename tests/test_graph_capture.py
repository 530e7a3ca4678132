"""moe_forward and moe_forward_noalloc inside a captured HIP graph: the library
allocates, clears and synchronises nothing in the forward path, so one captured step
replays the layer.  Every replay, with eager work and synchronisations between the
replays, is compared bit for bit with the eager result."""
from __future__ import annotations

import pytest
import torch

import sparse_mixture_experts_49_amd as moe
from tests import _gpu as G
from tests._inputs import inputs_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,noalloc", [("batch32_bf16", False), ("batch32_bf16", True),
                                          ("toy_fp32", False), ("mid_small_bf16", True)])
def test_captured_step_replays_equal_eager(name, noalloc):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    spec, inp = inputs_for(name)
    desc = G.desc_for(spec)
    x = G.to_dev(inp["x"])
    w = G.weights_for(inp)
    r = moe.Routing.allocate(desc, G.DEV)
    y = torch.empty(spec.tokens, spec.d_model, dtype=torch.float32, device=G.DEV)
    aux = torch.empty((), dtype=torch.float32, device=G.DEV)
    ws = None if noalloc else moe.alloc_workspace(desc, G.DEV)

    def step():
        if noalloc:
            moe.moe_forward_noalloc(desc, x, w, y, aux, r)
        else:
            moe.moe_forward(desc, x, w, y, aux, r, ws)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    y_ref, aux_ref, idx_ref = y.clone(), aux.clone(), r.topk_idx.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        y.fill_(float("nan"))                       # eager work between the replays
        aux.zero_()
        r.topk_idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), (name, i)
        assert torch.equal(aux, aux_ref), (name, i)
        assert torch.equal(r.topk_idx, idx_ref), (name, i)

"""moe_forward_noalloc (the layer on the library's own device scratch, no
workspace) against moe_forward with a caller workspace: two calls in a row, the
second with a smaller layer, each bit for bit equal to moe_forward on the same
inputs."""
from __future__ import annotations

import pytest
import torch

import sparse_mixture_experts_49_amd as moe
from tests import _gpu as G
from tests._inputs import inputs_for

pytestmark = pytest.mark.gpu


def _run(spec, inp, noalloc):
    desc = G.desc_for(spec)
    x = G.to_dev(inp["x"])
    w = G.weights_for(inp)
    r = moe.Routing.allocate(desc, G.DEV)
    y = torch.empty(spec.tokens, spec.d_model, dtype=torch.float32, device=G.DEV)
    aux = torch.empty((), dtype=torch.float32, device=G.DEV)
    if noalloc:
        moe.moe_forward_noalloc(desc, x, w, y, aux, r)
    else:
        moe.moe_forward(desc, x, w, y, aux, r, moe.alloc_workspace(desc, G.DEV))
    torch.cuda.synchronize()
    return y, aux, r


def test_noalloc_matches_forward_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    for name in ("decode_bf16", "decode_small_bf16"):        # 32 tokens, then 5
        spec, inp = inputs_for(name)
        y1, a1, r1 = _run(spec, inp, noalloc=True)
        y2, a2, r2 = _run(spec, inp, noalloc=False)
        assert torch.equal(y1, y2), name
        assert torch.equal(a1, a2), name
        R = int(r2.offsets[-1].item())
        for f in ("topk_idx", "topk_w", "counts", "offsets", "dest", "top1_count", "prob_mean",
                  "z_loss"):
            assert torch.equal(getattr(r1, f), getattr(r2, f)), (name, f)
        assert torch.equal(r1.src[:R], r2.src[:R]), name

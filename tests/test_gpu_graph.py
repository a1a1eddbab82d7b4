"""moe_forward under HIP graph capture: the call enqueues kernels only (no
allocation, memset, copy or synchronisation), so a captured pass replays.
Every replay, with eager passes on other inputs in between, must equal the
eager result bit for bit."""
import pytest
import torch

import synth
from gpu_cases import build_layer, dev, say, weights_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid,quant,M", [(2, None, 64), (2, "mxfp4", 8), (3, None, 16),
                                        (2, None, 1), (4, None, 1)])
def test_captured_forward_replays_exactly(cid, quant, M):
    import dataclasses
    cfg = synth.CONFIGS[cid]
    if quant:
        cfg = dataclasses.replace(cfg, quant=quant)
    say(f"graph {cfg.name} {cfg.quant} M={M}")
    W = weights_for(cfg)
    tok = synth.make_tokens(cfg, M)
    other = synth.make_tokens(cfg, M, seed=4321)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    x, lg = dev(tok["x_bits"]), dev(tok["logits"])
    x2, lg2 = dev(other["x_bits"]), dev(other["logits"])
    out = torch.empty((M, cfg.H), dtype=torch.bfloat16, device="cuda")
    layer.workspace(M)                        # allocated before the capture
    ref = layer.forward(x, lg, out=out).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, lg, out=out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, lg, out=out)
    torch.cuda.synchronize()
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
        o2 = layer.forward(x2, lg2)           # eager work on other inputs in between
        torch.cuda.synchronize()
        assert not torch.equal(o2.view(torch.int16), ref.view(torch.int16))

"""moe_forward_noalloc (the library's fixed per-GPU workspace) against
moe_forward (a caller workspace) through the C ABI: the same kernels on the
same inputs, so the outputs and the routing they return must be bit-identical
-- for two calls in a row on each workload, the second with fewer tokens,
so that it runs over what the first left in the shared array."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
import synth
from gpu_cases import build_layer, dev, say, weights_for

pytestmark = pytest.mark.gpu

CASES = [(1, (64, 9)), (2, (64, 8)), (2, (1, 1)), (3, (16, 5)), (4, (128, 1))]


def _pair(layer, cfg, M, seed):
    tok = synth.make_tokens(cfg, M, seed=seed)
    x, lg = dev(tok["x_bits"]), dev(tok["logits"])
    K = cfg.K_slots
    ref = layer.forward(x, lg)
    ids = torch.full((M, K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((M, K), -7.0, dtype=torch.float32, device="cuda")
    out = torch.full((M, cfg.H), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_forward_noalloc(layer.problem(M), layer.w, x, lg, ids, w, out)
    ids_ref = torch.empty_like(ids)
    w_ref = torch.empty_like(w)
    out_ref2 = torch.empty_like(out)
    moe.moe_forward(layer.problem(M), layer.w, x, lg, ids_ref, w_ref, out_ref2,
                    layer.workspace(M))
    torch.cuda.synchronize()
    return ref, out, ids, w, out_ref2, ids_ref, w_ref


@pytest.mark.parametrize("cid,Ms", CASES, ids=[f"cfg{c}-M{a}-then-M{b}" for c, (a, b) in CASES])
def test_noalloc_matches_forward(cid, Ms):
    cfg = synth.CONFIGS[cid]
    W = weights_for(cfg)
    sc = synth.make_act_scales(cfg, synth.make_tokens(cfg, Ms[0])["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    for i, M in enumerate(Ms):
        say(f"noalloc {cfg.name} call {i} M={M}")
        ref, out, ids, w, ref2, ids_ref, w_ref = _pair(layer, cfg, M, seed=5000 * cid + 17 * i + M)
        assert torch.equal(ref.view(torch.int16), ref2.view(torch.int16))
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"call {i} M={M}"
        assert torch.equal(ids, ids_ref) and torch.equal(w.view(torch.int32),
                                                          w_ref.view(torch.int32))
    del layer
    torch.cuda.empty_cache()


def test_noalloc_refuses_oversized_before_launching():
    cfg = synth.CONFIGS[2]
    W = weights_for(cfg)
    layer = build_layer(cfg, W)
    M = 4096
    p = layer.problem(M)
    assert moe.workspace_bytes(p) > moe.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros((M, cfg.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((M, cfg.E_routed), dtype=torch.float32, device="cuda")
    out = torch.full((M, cfg.H), 2.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_noalloc(p, layer.w, x, lg, None, None, out)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out.float() == 2.0).all())

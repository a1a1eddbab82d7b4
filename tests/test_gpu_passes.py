"""moe_forward on a batch of more than 65536 assignments, which it runs as
consecutive passes of floor(65536 / K') tokens on one pass's workspace
(include/moe.h): the output equals moe_forward called on each pass's tokens
separately, bit for bit, and the oracle's within the usual tolerance; the
fp8 passes here take different kernels (256-row blocks for the full pass,
128-row blocks for the short last one)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
import synth
from gpu_cases import ad_hoc, assert_close, build_layer, dev, oracle_forward, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("quant", ["bf16", "fp8_tensor"])
def test_forward_in_passes(quant):
    cfg = ad_hoc(95, quant, "silu", H=128, I=128, E_routed=16, top_k=8)
    W = synth.make_weights(cfg, seed=781)
    T, chunk = 8500, 65536 // 8          # 68000 assignments: passes of 8192 and 308 tokens
    say(f"passes {quant} T={T}")
    tok = synth.make_tokens(cfg, T, seed=82)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    assert moe.workspace_bytes(layer.problem(T)) == moe.workspace_bytes(layer.problem(chunk))
    if quant == "fp8_tensor":
        assert moe.block_m(layer.problem(chunk)) == 256
        assert moe.block_m(layer.problem(T - chunk)) == 128
    x, lg = dev(tok["x_bits"]), dev(tok["logits"])
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    out = layer.forward(x, lg, topk_ids=ids)
    parts = [layer.forward(x[t0:t0 + chunk].contiguous(), lg[t0:t0 + chunk].contiguous())
             for t0 in range(0, T, chunk)]
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), torch.cat(parts).view(torch.int16))
    ref = oracle_forward(cfg, W, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"])
    assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
    got = out.float().cpu().numpy().astype(np.float64)
    if quant == "bf16":
        assert_close(got, ref, quant, label=f"passes {quant}")
    else:
        # without the intermediate's check (parity()) the rounding flips of
        # the e4m3 intermediate are not accounted for: rel-L2 only
        rel = np.linalg.norm(got - ref["out"]) / np.linalg.norm(ref["out"])
        say(f"  passes {quant}: rel_l2={rel:.3e}")
        assert rel <= 1e-2

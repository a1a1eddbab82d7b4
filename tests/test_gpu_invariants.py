"""The oracle's invariants re-run on the GPU path, against textbook NumPy.

These compare the HIP path with results that have a plain definition of
their own, independent of the oracle (bf16 weights, fp64 NumPy matmuls):

* k = E with equal router logits (renormalised, every gate 1/E) equals the
  dense MLP averaged over the experts (the `topk` / `renormalize` routing
  of the sglang PR 21321 page, section 1);
* a single expert with k = 1 equals a plain gated (or relu^2) MLP;
* a shared expert fused as an extra slot at gate 1.0 equals the routed layer
  plus a separate shared MLP (the Qwen3-Next page, "Shared-Expert Fusion").

Tolerances are those of the parity tests (bf16: max-abs 2e-2, rel-L2 1e-2):
the GPU path rounds the intermediate and the output to bf16.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_cases import assert_close, ad_hoc, build_layer, dev, say
from synth.inputs import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def _act(h, act, I):
    """Textbook activations on fp64 rows of W13 . x (gate rows first)."""
    if act == "relu2":
        return np.maximum(h, 0.0) ** 2
    g, u = h[:, :I], h[:, I:]
    if act == "silu":
        return g / (1.0 + np.exp(-g)) * u
    c = np.sqrt(2.0 / np.pi)
    return 0.5 * g * (1.0 + np.tanh(c * (g + 0.044715 * g ** 3))) * u


def _mlp(x, w13, w2, act, I):
    """out[t] = W2 . act(W13 . x[t]) in fp64 for one expert."""
    return _act(x @ w13.T, act, I) @ w2.T


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _gpu(cfg, W, x_bits, logits):
    layer = build_layer(cfg, W)
    out = layer.forward(dev(x_bits), dev(logits))
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "relu2"])
def test_all_experts_with_equal_gates_is_the_mean_dense_mlp(act):
    E, T, H, I = 8, 37, 256, 256
    cfg = ad_hoc(110, "bf16", act, H=H, I=I, E_routed=E, top_k=E)
    say(f"k=E dense {act}")
    W = synth.make_weights(cfg, seed=9001)
    tok = synth.make_tokens(cfg, T, seed=31)
    logits = np.zeros((T, E), np.float32)           # every gate 1/E after renormalising
    got = _gpu(cfg, W, tok["x_bits"], logits)
    x = _f64(tok["x_bits"])
    w13, w2 = _f64(W["w13"]), _f64(W["w2"])
    ref = sum(_mlp(x, w13[e], w2[e], act, I) for e in range(E)) / E
    assert_close(got, ref, "bf16", f"k=E dense {act}")


@pytest.mark.parametrize("act", ["silu", "relu2"])
def test_single_expert_is_a_plain_mlp(act):
    T, H, I = 19, 384, 256
    cfg = ad_hoc(111, "bf16", act, H=H, I=I, E_routed=1, top_k=1)
    say(f"E=1 {act}")
    W = synth.make_weights(cfg, seed=9002)
    tok = synth.make_tokens(cfg, T, seed=32)
    got = _gpu(cfg, W, tok["x_bits"], tok["logits"])
    ref = _mlp(_f64(tok["x_bits"]), _f64(W["w13"])[0], _f64(W["w2"])[0], act, I)
    assert_close(got, ref, "bf16", f"E=1 {act}")


def test_fused_shared_slot_equals_routed_layer_plus_shared_mlp():
    Er, k, T, H, I = 8, 2, 45, 256, 256
    cfg = ad_hoc(112, "bf16", "silu", H=H, I=I, E_routed=Er, top_k=k, n_shared=1)
    say("shared slot = routed + shared MLP")
    W = synth.make_weights(cfg, seed=9003)
    tok = synth.make_tokens(cfg, T, seed=33)
    fused = _gpu(cfg, W, tok["x_bits"], tok["logits"])
    # the routed experts alone, on the GPU
    cfg_r = ad_hoc(113, "bf16", "silu", H=H, I=I, E_routed=Er, top_k=k)
    W_r = {"w13": W["w13"][:Er], "w2": W["w2"][:Er], "w13_scale": None, "w2_scale": None}
    routed = _gpu(cfg_r, W_r, tok["x_bits"], tok["logits"])
    # the shared expert as a plain MLP, in fp64
    shared = _mlp(_f64(tok["x_bits"]), _f64(W["w13"])[Er], _f64(W["w2"])[Er], "silu", I)
    # routed is bf16-rounded once more than the fused output: compare both
    # against the fp64 sum of its parts
    assert_close(fused, routed.astype(np.float64) + shared, "bf16", "fused vs routed + shared")

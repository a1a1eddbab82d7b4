"""GPU parity of the whole layer (moe_forward through the C ABI) vs the oracle.

All five configurations at every token count they name.  The decode-sized
and tiny passes are compared on every output; the full-size prefill passes
(cfg3 M=4096, cfg4 M=128/8192, cfg5 M=8192, cfg3 M=256) run the whole pass on
the GPU and compare a seeded sample of token rows (first and last included)
with the oracle on those tokens.  Tolerances: max-abs 2e-2 and rel-L2 1e-2
(bf16, fp8), rel-L2 3e-2 (int4 weights); the max-abs bound of an output is
widened by the oracle's flip margin where an fp8 intermediate value sits at a
rounding boundary (either code is a correct rounding).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
import oracle
import synth
from gpu_cases import (ad_hoc, assert_close, build_layer, dev, oracle_forward, say,
                       scalar, weights_for)

pytestmark = pytest.mark.gpu

# (cid, M, sampled token rows or None for all)
FULL = [(1, 64, None), (2, 1, None), (2, 8, None), (2, 32, None), (2, 64, None),
        (3, 16, None), (3, 256, 24), (3, 4096, 12), (4, 1, None), (4, 128, 12),
        (4, 8192, 6), (5, 8192, 8)]


def _sample(M, n, seed):
    if n is None or n >= M:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, M - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], mid]))


@pytest.mark.parametrize("cid,M,n", FULL, ids=[f"cfg{c}-M{m}" for c, m, _ in FULL])
def test_forward_config(cid, M, n):
    cfg = synth.CONFIGS[cid]
    say(f"forward {cfg.name} M={M} sample={n}")
    W = weights_for(cfg)
    tok = synth.make_tokens(cfg, M)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    rows = _sample(M, n, 1000 * cid + M)
    ref = oracle_forward(cfg, W, tok["x_bits"][rows], tok["logits"][rows], sc["a1"], sc["a2"])
    assert_close(got[rows], ref, cfg.quant, f"{cfg.name} M={M}")
    del layer
    torch.cuda.empty_cache()


# The gelu_tanh gate at full size: the decode shape (weight streaming) and
# the fp8 block-scale prefill shape (8-wave LDS pipeline), same weights as
# the SiLU configurations.
GELU_FULL = [(2, 64, None), (3, 4096, 12)]


@pytest.mark.parametrize("cid,M,n", GELU_FULL, ids=[f"cfg{c}-M{m}" for c, m, _ in GELU_FULL])
def test_forward_gelu_tanh_full_size(cid, M, n):
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS[cid], act="gelu_tanh")
    say(f"forward gelu_tanh {cfg.name} M={M} sample={n}")
    W = weights_for(synth.CONFIGS[cid])
    tok = synth.make_tokens(cfg, M)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    rows = _sample(M, n, 7000 * cid + M)
    ref = oracle_forward(cfg, W, tok["x_bits"][rows], tok["logits"][rows], sc["a1"], sc["a2"])
    assert_close(got[rows], ref, cfg.quant, f"gelu_tanh {cfg.name} M={M}")
    del layer
    torch.cuda.empty_cache()


# The MX modes at full size: the decode shape (hidden 2048, 128 experts,
# top-8, intermediate 768) and the fp8 block-scale prefill shape (hidden
# 2048, 512 + 1 experts, top-10, intermediate 512), with MXFP8 and MXFP4
# weights in place of the configuration's own.
MX_FULL = [(2, 64, None, q) for q in ("mxfp8", "mxfp4")] + \
          [(3, 4096, 10, q) for q in ("mxfp8", "mxfp4")] + [(5, 8192, 6, "mxfp4")]


@pytest.mark.parametrize("cid,M,n,quant", MX_FULL,
                         ids=[f"cfg{c}-M{m}-{q}" for c, m, _, q in MX_FULL])
def test_forward_mx_full_size(cid, M, n, quant):
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS[cid], quant=quant)
    say(f"forward {quant} {cfg.name} M={M} sample={n}")
    W = weights_for(cfg)
    tok = synth.make_tokens(cfg, M)
    layer = build_layer(cfg, W)
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    rows = _sample(M, n, 9000 * cid + M)
    ref = oracle_forward(cfg, W, tok["x_bits"][rows], tok["logits"][rows])
    assert_close(got[rows], ref, quant, f"{quant} {cfg.name} M={M}")
    del layer
    torch.cuda.empty_cache()


SMALL = [(q, a) for q in ("bf16", "fp8_tensor", "fp8_block", "w4a8", "mxfp8", "mxfp4")
         for a in ("silu", "relu2", "gelu_tanh")]


@pytest.mark.parametrize("quant,act", SMALL)
@pytest.mark.parametrize("T", [1, 37])
def test_forward_small_ragged(quant, act, T):
    """Several row tiles with a partly filled last workgroup, an odd number
    of k-steps and token counts that leave ragged blocks."""
    I = 160 if quant == "bf16" else 384
    if act == "relu2" and quant == "bf16":
        I = 384
    cfg = ad_hoc(90, quant, act, H=384, I=I, E_routed=10, top_k=3, n_shared=1)
    say(f"small {quant} {act} T={T} I={I}")
    W = synth.make_weights(cfg, seed=4242)
    tok = synth.make_tokens(cfg, T, seed=77 + T)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    ref = oracle_forward(cfg, W, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"])
    assert_close(out.float().cpu().numpy(), ref, quant, f"small {quant} {act} T={T}")


def test_components_equal_forward():
    """The separate entry points produce exactly moe_forward's output."""
    cfg = synth.CONFIGS[2]
    W = weights_for(cfg)
    tok = synth.make_tokens(cfg, 8)
    layer = build_layer(cfg, W)
    x, lg = dev(tok["x_bits"]), dev(tok["logits"])
    out = layer.forward(x, lg)
    b = layer.buffers(8)
    layer.route(8, lg, b)
    layer.align(8, b)
    layer.quant(8, x, b)
    layer.gemm1(8, x, b)
    layer.gemm2(8, b)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), b["out"].view(torch.int16))
    b2 = layer.buffers(8)
    layer.prepare(8, lg, x, b2)
    layer.gemm1(8, x, b2)
    layer.gemm2(8, b2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), b2["out"].view(torch.int16))


@pytest.mark.parametrize("quant,T", [("bf16", 29), ("fp8_block", 29), ("bf16", 13),
                                     ("fp8_block", 13), ("mxfp8", 29), ("mxfp4", 13)])
def test_prerouted_with_masked_slots(quant, T):
    """Routing supplied by the caller; ids outside [0, E) contribute nothing."""
    cfg = ad_hoc(91, quant, "silu", H=256, I=256, E_routed=12, top_k=4)
    W = synth.make_weights(cfg, seed=99)
    tok = synth.make_tokens(cfg, T, seed=5)
    rng = np.random.default_rng(6)
    ids = rng.integers(0, 12, (T, 4)).astype(np.int32)
    ids[rng.random((T, 4)) < 0.25] = -1
    ids[3] = -1                                   # a token with no valid slot
    w = rng.uniform(0.1, 1.0, (T, 4)).astype(np.float32)
    layer = build_layer(cfg, W)
    out = layer.forward(dev(tok["x_bits"]), None, dev(ids), dev(w))
    torch.cuda.synchronize()
    ref = oracle_forward(cfg, W, tok["x_bits"], topk_ids=ids, topk_w=w.astype(np.float64))
    got = out.float().cpu().numpy()
    assert np.all(got[3] == 0.0)
    assert_close(got, ref, quant, "prerouted")


def test_pack_swap_and_padding():
    """[Up, Gate] checkpoints with the swap flag, and an unaligned I padded
    with zeros at pack time, give the unpadded gate-first result."""
    src_I, I = 200, moe.padded_intermediate(200, "silu", "bf16")
    assert I == 224
    cfg = ad_hoc(92, "bf16", "silu", H=256, I=src_I, E_routed=6, top_k=2)
    W = synth.make_weights(cfg, seed=12)
    up_first = np.concatenate([W["w13"][:, src_I:], W["w13"][:, :src_I]], axis=1)
    T = 21
    tok = synth.make_tokens(cfg, T, seed=13)
    from mixture_experts_layer_09_amd.layer import MoELayer
    layer = MoELayer(256, I, 6, 2, "silu", "bf16", dev(up_first), dev(W["w2"]), src_I=src_I,
                     swap_halves=True)
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    ref = oracle_forward(cfg, W, tok["x_bits"], tok["logits"])
    assert_close(out.float().cpu().numpy(), ref, "bf16", "swap+pad")


def test_zero_tokens_is_a_noop():
    cfg = synth.CONFIGS[1]
    W = weights_for(cfg)
    layer = build_layer(cfg, W)
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((0, cfg.E_routed), dtype=torch.float32, device="cuda")
    out = layer.forward(x, lg)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.H)


def test_token_permutation_equivariant_on_gpu():
    cfg = synth.CONFIGS[1]
    W = weights_for(cfg)
    tok = synth.make_tokens(cfg, 64)
    layer = build_layer(cfg, W)
    perm = np.random.default_rng(3).permutation(64)
    a = layer.forward(dev(tok["x_bits"]), dev(tok["logits"])).float().cpu().numpy()
    b = layer.forward(dev(tok["x_bits"][perm]), dev(tok["logits"][perm])).float().cpu().numpy()
    # each token's row is computed by the same kernels in the same order
    assert np.array_equal(a[perm], b)


def test_invalid_call_enqueues_nothing():
    cfg = synth.CONFIGS[1]
    W = weights_for(cfg)
    layer = build_layer(cfg, W)
    p = layer.problem(4)
    out = torch.zeros((4, cfg.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")     # far too small
    x = torch.zeros((4, cfg.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((4, cfg.E_routed), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward(p, layer.w, x, lg, None, None, out, ws)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0


TILED = [(q, a, bm) for q in ("bf16", "fp8_tensor", "fp8_block", "w4a8")
         for a in ("silu", "relu2", "gelu_tanh") for bm in (64, 128)] + \
        [(q, a, 256) for q in ("fp8_tensor", "w4a8") for a in ("silu", "relu2", "gelu_tanh")] + \
        [(q, a, bm) for q in ("mxfp8", "mxfp4") for a in ("silu", "relu2", "gelu_tanh")
         for bm in (128, 256)]


@pytest.mark.parametrize("quant,act,bm", TILED)
def test_forward_tiled_ragged(quant, act, bm):
    """The tiled (prefill) kernels on small shapes: several blocks per expert
    with a ragged last block, three K stages, and a partly filled last weight
    slice for the non-gated case."""
    cfg = ad_hoc(93, quant, act, H=384, I=384, E_routed=4, top_k=2, n_shared=1)
    say(f"tiled {quant} {act} bm={bm}")
    W = synth.make_weights(cfg, seed=777)
    T = 150
    tok = synth.make_tokens(cfg, T, seed=78)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"], block_m=bm)
    assert moe.block_m(layer.problem(T)) == bm
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    ref = oracle_forward(cfg, W, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"])
    assert_close(out.float().cpu().numpy(), ref, quant, f"tiled {quant} {act} bm={bm}")


@pytest.mark.parametrize("quant,act", [(q, a) for q in ("fp8_tensor", "w4a8", "mxfp8", "mxfp4")
                                       for a in ("silu", "relu2", "gelu_tanh")])
def test_forward_wide_blocks_by_default(quant, act):
    """fp8 per-tensor, int4 and MX with 256+ rows per expert take 256-row blocks
    by themselves: several full blocks per expert, ragged last blocks, and
    blocks whose second half of token tiles is empty or partly filled."""
    cfg = ad_hoc(94, quant, act, H=512, I=384, E_routed=4, top_k=2, n_shared=1)
    say(f"wide {quant} {act}")
    W = synth.make_weights(cfg, seed=779)
    T = 700
    tok = synth.make_tokens(cfg, T, seed=80)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    assert moe.block_m(layer.problem(T)) == 256
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    ref = oracle_forward(cfg, W, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"])
    assert_close(out.float().cpu().numpy(), ref, quant, f"wide {quant} {act}")


@pytest.mark.parametrize("quant", ["mxfp8", "mxfp4"])
def test_mx_pack_scale_padding_and_swap(quant):
    """MX checkpoints with an unaligned intermediate (352, padded to 384 at
    pack time together with the [.., I/32] scales) and [Up, Gate] halves give
    the unpadded gate-first result."""
    src_I = 352
    I = moe.padded_intermediate(src_I, "silu", quant)
    assert I == 384
    cfg = ad_hoc(95, quant, "silu", H=256, I=src_I, E_routed=6, top_k=2)
    W = synth.make_weights(cfg, seed=17)
    swap = lambda a: np.concatenate([a[:, src_I:], a[:, :src_I]], axis=1)
    T = 23
    tok = synth.make_tokens(cfg, T, seed=18)
    from mixture_experts_layer_09_amd.layer import MoELayer
    layer = MoELayer(256, I, 6, 2, "silu", quant, dev(swap(W["w13"])), dev(W["w2"]),
                     dev(swap(W["w13_scale"])), dev(W["w2_scale"]), src_I=src_I,
                     swap_halves=True)
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    ref = oracle_forward(cfg, W, tok["x_bits"], tok["logits"])
    assert_close(out.float().cpu().numpy(), ref, quant, f"{quant} swap+pad")


@pytest.mark.parametrize("quant,T", [("bf16", 1), ("bf16", 97), ("fp8_block", 40), ("mxfp4", 128)])
def test_forward_matches_components_with_duplicates_and_empty_tokens(quant, T):
    """moe_forward is bit-identical to the separate entry points, call after
    call, with the same expert twice within a token and tokens without a
    valid slot (whose output rows are zero)."""
    cfg = ad_hoc(96, quant, "silu", H=256, I=384, E_routed=12, top_k=4)
    W = synth.make_weights(cfg, seed=123)
    tok = synth.make_tokens(cfg, T, seed=124)
    rng = np.random.default_rng(125)
    ids = rng.integers(0, 12, (T, 4)).astype(np.int32)
    ids[:, 1] = ids[:, 0]                           # the same expert twice
    ids[rng.random((T, 4)) < 0.2] = -1
    ids[T // 2] = -1                                # no valid slot
    w = rng.uniform(0.1, 1.0, (T, 4)).astype(np.float32)
    layer = build_layer(cfg, W)
    assert moe.block_m(layer.problem(T)) == 16
    x, di, dw = dev(tok["x_bits"]), dev(ids), dev(w)
    outs = []
    for _ in range(3):
        outs.append(layer.forward(x, None, di, dw).clone())
    b = layer.buffers(T)
    b["topk_ids"].copy_(di)
    b["topk_w"].copy_(dw)
    layer.align(T, b)
    layer.quant(T, x, b)
    layer.gemm1(T, x, b)
    layer.gemm2(T, b)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), b["out"].view(torch.int16))
    assert torch.count_nonzero(outs[0][T // 2].float()) == 0
    ref = oracle_forward(cfg, W, tok["x_bits"], topk_ids=ids, topk_w=w.astype(np.float64))
    assert_close(outs[0].float().cpu().numpy(), ref, quant, f"fused combine {quant} T={T}")


@pytest.mark.parametrize("quant,act", [("mxfp4", "gelu_tanh"), ("fp8_tensor", "gelu_tanh"),
                                       ("mxfp8", "relu2")])
def test_forward_without_renormalisation(quant, act):
    """Routing weights taken from the softmax over all routed logits (no
    renormalisation over the k picked), with a shared slot of gate 0.5."""
    cfg = ad_hoc(97, quant, act, H=256, I=256, E_routed=16, top_k=3, n_shared=1,
                 renormalize=False)
    cfg = __import__("dataclasses").replace(cfg, shared_gate=0.5)
    W = synth.make_weights(cfg, seed=321)
    T = 45
    tok = synth.make_tokens(cfg, T, seed=322)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    out = layer.forward(dev(tok["x_bits"]), dev(tok["logits"]))
    torch.cuda.synchronize()
    ref = oracle_forward(cfg, W, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"])
    assert_close(out.float().cpu().numpy(), ref, quant, f"no renorm {quant} {act}")

"""GPU parity of the whole layer (moe_forward through the C ABI) vs the oracle.

All five configurations at every token count they name, every output row
(the full-size prefill passes included: every 256-row block and every round
of the persistent kernels is covered).  Each pass is checked with
gpu_cases.parity: moe_forward equals the separate entry points bit for bit,
the routing and alignment equal the oracle's, and the output is within
max-abs 2e-2 and rel-L2 1e-2 (bf16, fp8) or 3e-2 (int4 weights) of the
oracle's, beyond the change that the intermediate's observed code flips make.
The stored intermediate is compared with the oracle's code for code: up to
1024 tokens every code must lie inside the oracle's rounding window (the
codes a kernel with the matrix cores' arithmetic can store); at the
full-size prefill passes, whose window would take minutes of host time,
every code must lie within one e4m3 step of the exact rounding and the window
is checked on the first row of every row block (so every tile and every
round of the persistent kernels is covered).
"""
import dataclasses
import time

import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
import oracle
import synth
from gpu_cases import (ad_hoc, assert_close, build_layer, dev, oracle_forward, parity, say,
                       scalar, weights_for)

pytestmark = pytest.mark.gpu

FULL = [(1, 64), (2, 1), (2, 8), (2, 32), (2, 64), (3, 16), (3, 256), (3, 4096), (4, 1),
        (4, 128), (4, 8192), (5, 1024), (5, 8192)]
A2_MAX_TOKENS = 1024      # the intermediate's code-level check up to this many tokens


def _full(cfg, M, label):
    W = weights_for(cfg)
    tok = synth.make_tokens(cfg, M)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    t0 = time.perf_counter()
    parity(cfg, W, layer, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"], label=label,
           check_a2=True if M <= A2_MAX_TOKENS else "sampled")
    say(f"  {label}: checked in {time.perf_counter() - t0:.1f} s (GPU passes and oracle)")
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cid,M", FULL, ids=[f"cfg{c}-M{m}" for c, m in FULL])
def test_forward_config(cid, M):
    cfg = synth.CONFIGS[cid]
    say(f"forward {cfg.name} M={M}")
    _full(cfg, M, f"{cfg.name} M={M}")


# The gelu_tanh gate at full size: the decode shape (weight streaming) and
# the fp8 block-scale prefill shape (8-wave LDS pipeline), same weights as
# the SiLU configurations.
GELU_FULL = [(2, 64), (3, 4096)]


@pytest.mark.parametrize("cid,M", GELU_FULL, ids=[f"cfg{c}-M{m}" for c, m in GELU_FULL])
def test_forward_gelu_tanh_full_size(cid, M):
    cfg = dataclasses.replace(synth.CONFIGS[cid], act="gelu_tanh")
    say(f"forward gelu_tanh {cfg.name} M={M}")
    _full(cfg, M, f"gelu_tanh {cfg.name} M={M}")


# bf16 weights at prefill sizes on the decode configuration's shapes (hidden
# 2048, 128 experts, top-8, intermediate 768): 64 rows per expert (128-row
# blocks, the 4-wave LDS pipeline, persistent) and 256 (256-row blocks, the
# 8-wave 256 x 256 tile).
BF16_PREFILL = [(2, 1024), (2, 4096)]


@pytest.mark.parametrize("cid,M", BF16_PREFILL, ids=[f"cfg{c}-M{m}" for c, m in BF16_PREFILL])
def test_forward_bf16_prefill_full_size(cid, M):
    cfg = synth.CONFIGS[cid]
    p = moe.problem(T=M, H=cfg.H, I=cfg.I, E_routed=cfg.E_routed, top_k=cfg.top_k, act=cfg.act,
                    quant=cfg.quant, n_shared=cfg.n_shared)
    assert moe.block_m(p) == (256 if M >= 4096 else 128)
    say(f"forward bf16 prefill {cfg.name} M={M}")
    _full(cfg, M, f"bf16 prefill {cfg.name} M={M}")


# The MX modes at full size: the decode shape (hidden 2048, 128 experts,
# top-8, intermediate 768), the fp8 block-scale prefill shape (hidden 2048,
# 512 + 1 experts, top-10, intermediate 512) and the W4A8 shape, with MXFP8
# and MXFP4 weights in place of the configuration's own.
MX_FULL = [(2, 64, q) for q in ("mxfp8", "mxfp4")] + \
          [(3, 4096, q) for q in ("mxfp8", "mxfp4")] + [(5, 8192, "mxfp4")]


@pytest.mark.parametrize("cid,M,quant", MX_FULL, ids=[f"cfg{c}-M{m}-{q}" for c, m, q in MX_FULL])
def test_forward_mx_full_size(cid, M, quant):
    cfg = dataclasses.replace(synth.CONFIGS[cid], quant=quant)
    say(f"forward {quant} {cfg.name} M={M}")
    _full(cfg, M, f"{quant} {cfg.name} M={M}")


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
    parity(cfg, W, layer, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"],
           label=f"small {quant} {act} T={T}")


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
    got, _ = parity(cfg, W, layer, tok["x_bits"], topk_ids=ids, topk_w=w, label="prerouted")
    assert np.all(got[3] == 0.0)


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
    parity(cfg, W, layer, tok["x_bits"], tok["logits"], label="swap+pad")


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
        [(q, a, 256) for q in ("bf16", "fp8_tensor", "w4a8") for a in ("silu", "relu2", "gelu_tanh")] + \
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
    parity(cfg, W, layer, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"],
           label=f"tiled {quant} {act} bm={bm}")


@pytest.mark.parametrize("quant,act", [(q, a) for q in ("bf16", "fp8_tensor", "w4a8", "mxfp8", "mxfp4")
                                       for a in ("silu", "relu2", "gelu_tanh")])
def test_forward_wide_blocks_by_default(quant, act):
    """bf16, fp8 per-tensor, int4 and MX with 256+ rows per expert take 256-row blocks
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
    parity(cfg, W, layer, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"],
           label=f"wide {quant} {act}")


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
    parity(cfg, W, layer, tok["x_bits"], tok["logits"], label=f"{quant} swap+pad")


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
    got, _ = parity(cfg, W, layer, tok["x_bits"], topk_ids=ids, topk_w=w,
                    label=f"duplicates {quant} T={T}")
    assert np.array_equal(got, outs[0].float().cpu().numpy())


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
    parity(cfg, W, layer, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"],
           label=f"no renorm {quant} {act}")


@pytest.mark.parametrize("quant,act", [("bf16", "silu"), ("fp8_tensor", "relu2"),
                                       ("fp8_block", "silu"), ("w4a8", "gelu_tanh"),
                                       ("mxfp8", "silu"), ("mxfp4", "relu2")])
def test_token_major_gemm2_equals_expert_major_path(quant, act):
    """For one or two tokens (up to 64 assignments) GEMM2 and the combine run
    token by token in one kernel; for more, GEMM2 writes per-assignment rows
    and the combine sums them.  The first two tokens of a three-token batch
    get bit-identical outputs from both paths (same routing: the third token
    only appends)."""
    cfg = ad_hoc(98, quant, act, H=512, I=384, E_routed=12, top_k=3, n_shared=1)
    W = synth.make_weights(cfg, seed=55)
    tok = synth.make_tokens(cfg, 3, seed=56)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    x, lg = dev(tok["x_bits"]), dev(tok["logits"])
    one = layer.forward(x[:1].contiguous(), lg[:1].contiguous())
    two = layer.forward(x[:2].contiguous(), lg[:2].contiguous())
    three = layer.forward(x, lg)
    torch.cuda.synchronize()
    assert torch.equal(two.view(torch.int16), three[:2].view(torch.int16))
    assert torch.equal(one.view(torch.int16), three[:1].view(torch.int16))
    parity(cfg, W, layer, tok["x_bits"][:2], tok["logits"][:2], sc["a1"], sc["a2"],
           label=f"token-major {quant} {act}")


@pytest.mark.parametrize("quant,act,k,ns,T", [("bf16", "silu", 40, 2, 1), ("fp8_tensor", "silu", 63, 1, 1),
                                              ("w4a8", "silu", 30, 2, 2), ("mxfp8", "gelu_tanh", 28, 2, 2)])
def test_token_major_gemm2_many_slots(quant, act, k, ns, T):
    """The token-major GEMM2 with more valid slots than its 16 waves (each
    wave forms the rows of slots w, w + 16, ...): T tokens of up to 64
    assignments against the first T tokens of a batch one token larger
    (expert-major GEMM2 and the combine), bit for bit, and the oracle (one
    shared slot at most, so that |out| stays where the absolute 2e-2 bound
    exceeds the bf16 rounding of the output itself)."""
    cfg = ad_hoc(99, quant, act, H=256, I=256, E_routed=64, top_k=k, n_shared=ns)
    W = synth.make_weights(cfg, seed=57)
    tok = synth.make_tokens(cfg, T + 1, seed=58)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    say(f"token-major many slots {quant} K'={k + ns} T={T}")
    x, lg = dev(tok["x_bits"]), dev(tok["logits"])
    few = layer.forward(x[:T].contiguous(), lg[:T].contiguous())
    more = layer.forward(x, lg)
    torch.cuda.synchronize()
    assert torch.equal(few.view(torch.int16), more[:T].view(torch.int16))
    parity(cfg, W, layer, tok["x_bits"][:T], tok["logits"][:T], sc["a1"], sc["a2"],
           label=f"token-major many slots {quant}")


@pytest.mark.parametrize("quant,routed", [("bf16", True), ("bf16", False), ("fp8_tensor", True),
                                          ("fp8_tensor", False), ("w4a8", False),
                                          ("mxfp4", True)])
def test_one_token_forward_equals_components(quant, routed):
    """One token through moe_forward (a GEMM1 block per assignment, no
    alignment; with caller-given ids an expert repeated and a slot masked)
    against the separate entry points (aligned blocks), bit for bit, and the
    oracle."""
    cfg = ad_hoc(97, quant, "silu", H=256, I=256, E_routed=12, top_k=4, n_shared=1)
    W = synth.make_weights(cfg, seed=131)
    tok = synth.make_tokens(cfg, 1, seed=132)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    say(f"one token {quant} routed={routed}")
    if routed:
        parity(cfg, W, layer, tok["x_bits"], tok["logits"], sc["a1"], sc["a2"],
               label=f"one token {quant}")
    else:
        ids = np.array([[7, 7, -1, 3, 12]], dtype=np.int32)   # repeat, mask, shared slot
        w = np.array([[0.5, 0.25, 0.9, 0.125, 1.0]], dtype=np.float32)
        parity(cfg, W, layer, tok["x_bits"], None, sc["a1"], sc["a2"], topk_ids=ids, topk_w=w,
               label=f"one token prerouted {quant}")


@pytest.mark.parametrize("cid", [2, 4])
def test_one_token_back_to_back(cid):
    """One-token passes (a GEMM1 block per assignment, no alignment) on three
    different tokens, enqueued 8 times over without synchronisation: every
    output equals the separate entry points' for its token, bit for bit (no
    pass reads a workspace value left by an earlier one)."""
    cfg = synth.CONFIGS[cid]
    W = weights_for(cfg)
    toks = [synth.make_tokens(cfg, 1, seed=700 + k) for k in range(3)]
    sc = synth.make_act_scales(cfg, toks[0]["x_bits"])
    layer = build_layer(cfg, W, sc["a1"], sc["a2"])
    say(f"one token back to back {cfg.name}")
    xs = [dev(t["x_bits"]) for t in toks]
    lgs = [dev(t["logits"]) for t in toks]
    refs = []
    for x, lg in zip(xs, lgs):
        b = layer.buffers(1)
        layer.prepare(1, lg, x, b)
        layer.gemm1(1, x, b)
        layer.gemm2(1, b)
        refs.append(b["out"].clone())
    outs = [(k, layer.forward(xs[k], lgs[k])) for _ in range(8) for k in range(3)]
    torch.cuda.synchronize()
    assert len({r.view(torch.int16).cpu().numpy().tobytes() for r in refs}) == 3
    for n, (k, o) in enumerate(outs):
        assert torch.equal(o.view(torch.int16), refs[k].view(torch.int16)), f"pass {n} token {k}"


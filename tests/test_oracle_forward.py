"""Pins for the oracle's layer forward (CPU only).

The layer is pinned to the special cases where it reduces to a plain MLP
written with torch (E = 1, k = E with uniform gates, the shared slot as a
separate MLP), to invariances (token permutation, interleaved vs split
layout, the [Up, Gate] half swap, zero padding of I, linearity in the routing
weights), and to dequantisation written independently with torch's fp8
decoder and explicit block loops.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import codecs

R = np.random.default_rng


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def _mk_bf16(E, N1, H, I, T, seed):
    rng = R(seed)
    w13 = _bf16_bits(rng.standard_normal((E, N1, H)) / np.sqrt(H))
    w2 = _bf16_bits(rng.standard_normal((E, H, I)) / np.sqrt(I))
    x = _bf16_vals(_bf16_bits(rng.standard_normal((T, H))))
    return w13, w2, x


def _torch_mlp(x, w13, w2, act, mid=None):
    x = torch.from_numpy(np.asarray(x, np.float64))
    w13 = torch.from_numpy(np.asarray(w13, np.float64))
    w2 = torch.from_numpy(np.asarray(w2, np.float64))
    I = w2.shape[1]
    if act == "silu":
        a = F.silu(x @ w13[:I].T) * (x @ w13[I:].T)
    elif act == "gelu_tanh":
        a = F.gelu(x @ w13[:I].T, approximate="tanh") * (x @ w13[I:].T)
    else:
        a = F.relu(x @ w13.T) ** 2
    if mid is not None:
        a = mid(a)
    return (a @ w2.T).numpy()


def _fwd(x, w13, w2, **kw):
    base = dict(quant="bf16", act="silu", renormalize=True)
    base.update(kw)
    return oracle.moe_forward(x, w13, w2, **base)["out"]


@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "relu2"])
def test_single_expert_is_plain_mlp(act):
    H, I, T = 64, 48, 9
    N1 = I if act == "relu2" else 2 * I
    w13, w2, x = _mk_bf16(1, N1, H, I, T, 1)
    lg = np.zeros((T, 1), np.float32)
    got = _fwd(x, w13, w2, act=act, E_routed=1, top_k=1, logits=lg, storage="exact")
    ref = _torch_mlp(x, _bf16_vals(w13[0]), _bf16_vals(w2[0]), act)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # with the bf16 storage of the intermediate (torch's own bf16 cast)
    got = _fwd(x, w13, w2, act=act, E_routed=1, top_k=1, logits=lg)
    ref = _torch_mlp(x, _bf16_vals(w13[0]), _bf16_vals(w2[0]), act,
                     mid=lambda a: a.float().bfloat16().double())
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_all_experts_uniform_gates_is_dense_average():
    E, H, I, T = 4, 32, 16, 7
    w13, w2, x = _mk_bf16(E, 2 * I, H, I, T, 2)
    lg = np.full((T, E), 0.3, np.float32)
    got = _fwd(x, w13, w2, E_routed=E, top_k=E, logits=lg, storage="exact")
    ref = sum(_torch_mlp(x, _bf16_vals(w13[e]), _bf16_vals(w2[e]), "silu") for e in range(E)) / E
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_token_permutation_equivariant():
    E, H, I, T = 8, 32, 16, 21
    w13, w2, x = _mk_bf16(E, 2 * I, H, I, T, 3)
    lg = R(4).standard_normal((T, E)).astype(np.float32)
    perm = R(5).permutation(T)
    a = _fwd(x, w13, w2, E_routed=E, top_k=2, logits=lg)
    b = _fwd(x[perm], w13, w2, E_routed=E, top_k=2, logits=lg[perm])
    np.testing.assert_allclose(a[perm], b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("G", [1, 4, 16, 32])
def test_interleaved_equals_split_bf16(G, act):
    E, H, I, T = 3, 32, 32, 10
    w13, w2, x = _mk_bf16(E, 2 * I, H, I, T, 6)
    lg = R(7).standard_normal((T, E)).astype(np.float32)
    a = _fwd(x, w13, w2, act=act, E_routed=E, top_k=2, logits=lg)
    b = _fwd(x, oracle.interleave_rows(w13, G), w2, act=act, E_routed=E, top_k=2, logits=lg,
             layout_g=G)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_gelu_tanh_gate_closed_forms():
    """The gelu_tanh gate, from its definition rather than a library: g(0) = 0,
    g(v) - g(-v) = v (the tanh term is odd), g(v) -> v and g(-v) -> 0 for
    large v, and at v = 1 the value 0.5 (1 + tanh(1.044715 sqrt(2/pi)))."""
    from oracle.moe import GATE_FN
    g = GATE_FN["gelu_tanh"]
    v = np.linspace(-6, 6, 241)
    assert g(np.array(0.0)) == 0.0
    np.testing.assert_allclose(g(v) - g(-v), v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(g(np.array([30.0, -30.0])), [30.0, 0.0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g(np.array(1.0)), 0.8411919906082768, rtol=1e-15)
    # within 1e-3 of the erf form it approximates, and not equal to SiLU
    erf_gelu = 0.5 * v * (1 + np.vectorize(__import__("math").erf)(v / np.sqrt(2)))
    assert np.max(np.abs(g(v) - erf_gelu)) < 1e-3
    assert np.max(np.abs(g(v) - GATE_FN["silu"](v))) > 0.1


def test_interleave_layout_literal():
    # G = 1 gives [gate0, up0, gate1, up1, ...]
    w = np.arange(8)[None, :, None] * np.ones((1, 8, 2))
    got = oracle.interleave_rows(w, 1)[0, :, 0]
    assert list(got) == [0, 4, 1, 5, 2, 6, 3, 7]
    got = oracle.interleave_rows(w, 2)[0, :, 0]
    assert list(got) == [0, 1, 4, 5, 2, 3, 6, 7]


def test_half_swap():
    E, H, I, T = 2, 32, 16, 6
    w13, w2, x = _mk_bf16(E, 2 * I, H, I, T, 8)
    up_first = np.concatenate([w13[:, I:], w13[:, :I]], axis=1)
    lg = R(9).standard_normal((T, E)).astype(np.float32)
    a = _fwd(x, w13, w2, E_routed=E, top_k=1, logits=lg)
    b = _fwd(x, oracle.swap_halves(up_first), w2, E_routed=E, top_k=1, logits=lg)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "relu2"])
def test_zero_padding_leaves_output_unchanged(act):
    E, H, I, T = 3, 32, 40, 8
    gated = act != "relu2"
    N1 = 2 * I if gated else I
    w13, w2, x = _mk_bf16(E, N1, H, I, T, 10)
    p13, p2, Ip = oracle.pad_intermediate(w13, w2, gated)
    assert Ip == (48 if gated else 128)
    lg = R(11).standard_normal((T, E)).astype(np.float32)
    a = _fwd(x, w13, w2, act=act, E_routed=E, top_k=2, logits=lg)
    b = _fwd(x, p13, p2, act=act, E_routed=E, top_k=2, logits=lg)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_shared_slot_equals_separate_shared_mlp():
    Er, H, I, T = 4, 32, 16, 9
    w13, w2, x = _mk_bf16(Er + 1, 2 * I, H, I, T, 12)
    lg = R(13).standard_normal((T, Er)).astype(np.float32)
    fused = _fwd(x, w13, w2, E_routed=Er, top_k=2, n_shared=1, shared_gate=1.0,
                 logits=lg, storage="exact")
    routed = _fwd(x, w13[:Er], w2[:Er], E_routed=Er, top_k=2, logits=lg, storage="exact")
    shared = _torch_mlp(x, _bf16_vals(w13[Er]), _bf16_vals(w2[Er]), "silu")
    np.testing.assert_allclose(fused, routed + shared, rtol=1e-12, atol=1e-13)


def test_linear_in_routing_weights_and_masking():
    E, H, I, T = 5, 32, 16, 6
    w13, w2, x = _mk_bf16(E, 2 * I, H, I, T, 14)
    rng = R(15)
    ids = rng.integers(0, E, (T, 3)).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, 3))
    kw = dict(E_routed=E, top_k=3, topk_ids=ids, storage="exact")
    a = _fwd(x, w13, w2, topk_w=w, **kw)
    b = _fwd(x, w13, w2, topk_w=2.5 * w, **kw)
    np.testing.assert_allclose(b, 2.5 * a, rtol=1e-13, atol=1e-14)
    # an id outside [0, E) contributes nothing (expert-parallel masking)
    ids2 = ids.copy()
    ids2[:, 2] = -1
    c = _fwd(x, w13, w2, topk_w=w, **dict(kw, topk_ids=ids2))
    w3 = w.copy()
    w3[:, 2] = 0
    d = _fwd(x, w13, w2, topk_w=w3, **kw)
    np.testing.assert_allclose(c, d, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- quantised weights
def _torch_e4m3(codes):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()


def test_block_scale_dequant_by_block_loops():
    rng = R(16)
    E, N, K = 2, 384, 256                 # 3 x 2 scale blocks: a transpose would not fit
    codes = rng.integers(0, 256, (E, N, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    s = rng.uniform(0.5, 2, (E, N // 128, K // 128)).astype(np.float32)
    got = oracle.dequant_w13(codes, s, "fp8_block", 1)
    ref = np.empty((N, K))
    dec = _torch_e4m3(codes[1])
    for nb in range(N // 128):
        for kb in range(K // 128):
            blk = (slice(nb * 128, nb * 128 + 128), slice(kb * 128, kb * 128 + 128))
            ref[blk] = dec[blk] * float(s[1, nb, kb])
    assert np.array_equal(got, ref)
    # interleaved storage looks scales up through each row's original index
    G = 16
    inter = oracle.interleave_rows(codes, G)
    got_i = oracle.dequant_w13(inter, s, "fp8_block", 1, layout_g=G)
    assert np.array_equal(got_i, oracle.interleave_rows(ref[None], G)[0])


def test_int4_group_dequant_by_loops():
    rng = R(17)
    E, N, K = 2, 32, 384
    q = rng.integers(-8, 8, (E, N, K))
    packed = ((q[..., 0::2] & 15) | ((q[..., 1::2] & 15) << 4)).astype(np.uint8)
    s = _bf16_bits(rng.uniform(0.01, 0.1, (E, N, K // 128)))
    got = oracle.dequant_w2(packed, s, "w4a8", 0)
    sv = _bf16_vals(s[0])
    ref = np.empty((N, K))
    for n in range(N):
        for k in range(K):
            ref[n, k] = q[0, n, k] * sv[n, k // 128]
    assert np.array_equal(got, ref)
    G = 16
    got_i = oracle.dequant_w13(oracle.interleave_rows(packed, G), s, "w4a8", 0, layout_g=G)
    assert np.array_equal(got_i, oracle.interleave_rows(ref[None], G)[0])


def test_per_tensor_scale_algebra():
    """The TRTLLM-Gen page's scale scalars, in exact arithmetic.

    gated: output1_scales_scalar = w13_scale * a1 / a2 applied to the up
    product after SiLU of the dequantised gate equals dequant -> act -> /a2;
    non-gated: dequantising before relu^2 then dividing by a2 equals
    alpha^2 * relu(acc)^2 / a2.
    """
    rng = R(18)
    acc_g, acc_u = rng.standard_normal(1000) * 50, rng.standard_normal(1000) * 50
    w_s, a1, a2 = 0.013, 0.02, 0.07
    alpha = w_s * a1
    silu = lambda v: v / (1 + np.exp(-v))
    np.testing.assert_allclose(silu(alpha * acc_g) * acc_u * (w_s * a1 * (1.0 / a2)),
                               silu(alpha * acc_g) * (alpha * acc_u) / a2, rtol=1e-13)
    np.testing.assert_allclose(np.maximum(acc_g * alpha, 0) ** 2 / a2,
                               alpha ** 2 * np.maximum(acc_g, 0) ** 2 / a2, rtol=1e-13)


def _fp8_tensor_case(act, seed):
    rng = R(seed)
    H, I, T = 256, 128, 12
    N1 = I if act == "relu2" else 2 * I
    w13f = rng.standard_normal((1, N1, H)) / 16
    w2f = rng.standard_normal((1, H, I)) / np.sqrt(I)
    s13 = np.array([np.abs(w13f).max() / 448], np.float32)
    s2 = np.array([np.abs(w2f).max() / 448], np.float32)
    c13 = torch.from_numpy((w13f / s13[0]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    c2 = torch.from_numpy((w2f / s2[0]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    x = _bf16_vals(_bf16_bits(rng.standard_normal((T, H))))
    a1 = np.float32(np.abs(x).max() / 448)
    return x, c13, s13, c2, s2, a1


@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "relu2"])
def test_fp8_tensor_single_expert_with_torch_casts(act):
    x, c13, s13, c2, s2, a1 = _fp8_tensor_case(act, 19)
    a2 = np.float32(4.0 / 448)
    got = oracle.moe_forward(x, c13, c2, quant="fp8_tensor", act=act, E_routed=1, top_k=1,
                             renormalize=True, logits=np.zeros((len(x), 1), np.float32),
                             w13_scale=s13, w2_scale=s2, a1=a1, a2=a2)["out"]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    xq = t((x / a1).astype(np.float32)).to(torch.float8_e4m3fn).double() * float(a1)
    W13 = t(c13[0]).view(torch.float8_e4m3fn).double() * float(s13[0])
    W2 = t(c2[0]).view(torch.float8_e4m3fn).double() * float(s2[0])

    def mid(a):
        q = torch.clamp((a.float() / torch.tensor(a2)), -448, 448).to(torch.float8_e4m3fn)
        return q.double() * float(a2)
    ref = _torch_mlp(xq.numpy(), W13.numpy(), W2.numpy(), act, mid=mid)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_fp8_block_single_expert_with_torch_casts():
    rng = R(20)
    H, I, T = 256, 256, 5
    w13f = rng.standard_normal((1, 2 * I, H)) / 16
    w2f = rng.standard_normal((1, H, I)) / 16
    s13 = rng.uniform(0.5, 2, (1, 2 * I // 128, H // 128)).astype(np.float32) / 64
    s2 = rng.uniform(0.5, 2, (1, H // 128, I // 128)).astype(np.float32) / 64
    k = lambda s: np.kron(s[0], np.ones((128, 128)))
    c13 = torch.from_numpy((w13f[0] / k(s13)).astype(np.float32)).to(torch.float8_e4m3fn)
    c2 = torch.from_numpy((w2f[0] / k(s2)).astype(np.float32)).to(torch.float8_e4m3fn)
    x = _bf16_vals(_bf16_bits(rng.standard_normal((T, H))))
    got = oracle.moe_forward(x, c13.view(torch.uint8).numpy()[None], c2.view(torch.uint8).numpy()[None],
                             quant="fp8_block", act="silu", E_routed=1, top_k=1, renormalize=True,
                             logits=np.zeros((T, 1), np.float32), w13_scale=s13, w2_scale=s2)["out"]

    def gq(a):   # per-row, per-128 dynamic quantisation with torch's cast
        a = a.float().reshape(a.shape[0], -1, 128)
        s = a.abs().amax(-1, keepdim=True) / 448.0
        s = torch.where(s == 0, torch.ones_like(s), s)
        return ((a / s).to(torch.float8_e4m3fn).double() * s.double()).reshape(a.shape[0], -1)
    xq = gq(torch.from_numpy(x))
    W13 = c13.double() * torch.from_numpy(k(s13))
    W2 = c2.double() * torch.from_numpy(k(s2))
    ref = _torch_mlp(xq.numpy(), W13.numpy(), W2.numpy(), "silu", mid=gq)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)

"""The Python binding checks every tensor before its pointer reaches the C
ABI (which sees raw pointers and cannot check sizes): element type,
contiguity, byte size against the problem, and that it lives on a GPU.  CPU
tensors are used here, so each call must fail in the binding -- a call that
got through would hand the library a host pointer -- and nothing is
launched."""
import pytest
import torch

import mixture_experts_layer_09_amd as moe


def P(**kw):
    base = dict(T=4, H=256, I=512, E_routed=8, top_k=2)
    base.update(kw)
    return moe.problem(**base)


def ids(T=4, K=2):
    return torch.zeros((T, K), dtype=torch.int32)


def w(T=4, K=2):
    return torch.zeros((T, K), dtype=torch.float32)


@pytest.mark.parametrize("logits,match", [
    (torch.zeros((4, 8), dtype=torch.float64), "dtype"),
    (torch.zeros((8, 4), dtype=torch.float32).t(), "contiguous"),
    (torch.zeros((4, 7), dtype=torch.float32), "needs 128"),
    (torch.zeros((4, 8), dtype=torch.float32), "GPU"),
    ([0.0] * 32, "torch.Tensor"),
])
def test_route_checks_logits(logits, match):
    with pytest.raises((ValueError, TypeError), match=match):
        moe.moe_route(P(), logits, ids(), w())


def test_route_checks_outputs():
    lg = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="topk_ids has dtype"):
        moe.moe_route(P(), lg, ids().long(), w())
    with pytest.raises(ValueError, match="topk_w holds 28 bytes"):
        moe.moe_route(P(), lg, ids(), torch.zeros(7, dtype=torch.float32))


def test_forward_checks_x_and_out():
    p = P()
    wt = moe.Weights()
    x32 = torch.zeros((4, 256), dtype=torch.float32)
    out = torch.zeros((4, 256), dtype=torch.bfloat16)
    lg = torch.zeros((4, 8), dtype=torch.float32)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="x has dtype"):
        moe.moe_forward(p, wt, x32, lg, None, None, out, ws)
    x = torch.zeros((4, 255), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x holds"):
        moe.moe_forward(p, wt, x, lg, None, None, out, ws)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out holds"):
        moe.moe_forward(p, wt, x, lg, None, None, out[:3], ws)
    with pytest.raises(ValueError, match="topk_ids is required"):
        moe.moe_forward(p, wt, x, None, None, None, out, ws)
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_forward(p, wt, x, lg, None, None, out, ws)


def test_invalid_problem_raises_before_sizes():
    with pytest.raises(moe.MoEError, match="MOE_ERR_ALIGNMENT"):
        moe.moe_route(P(H=200), None, None, None)


def test_gemm_checks_block_buffers():
    p = P()
    rows, blocks = moe.max_padded_rows(p), moe.max_blocks(p)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    srt = torch.zeros(rows - 1, dtype=torch.int32)
    bexp = torch.zeros(blocks, dtype=torch.int32)
    npad = torch.zeros(1, dtype=torch.int32)
    a2 = torch.zeros((rows, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="sorted_ids holds"):
        moe.moe_gemm1_act(p, x, None, moe.Weights(), srt, bexp, npad, a2, None)
    srt = torch.zeros(rows, dtype=torch.int32)
    with pytest.raises(ValueError, match="a2 holds"):
        moe.moe_gemm1_act(p, x, None, moe.Weights(), srt, bexp, npad, a2[:-1], None)
    with pytest.raises(ValueError, match="a2 has dtype"):
        moe.moe_gemm1_act(p, x, None, moe.Weights(), srt, bexp, npad, a2.float(), None)
    pf = P(quant="fp8_block")
    xq = torch.zeros((4, 256), dtype=torch.uint8)
    a2q = torch.zeros((moe.max_padded_rows(pf), 512), dtype=torch.uint8)
    with pytest.raises(ValueError, match="x_scale is required"):
        moe.moe_gemm1_act(pf, xq, None, moe.Weights(), srt, bexp, npad, a2q, None)


def test_pack_checks_source_and_destination():
    p = P(quant="fp8_block")
    w13 = torch.zeros((8, 1024, 256), dtype=torch.uint8)
    s13 = torch.zeros((8, 8, 2), dtype=torch.float32)
    nb, ns = moe.packed_bytes(p, 13)
    dst, dsc = torch.zeros(nb, dtype=torch.uint8), torch.zeros(ns, dtype=torch.uint8)
    with pytest.raises(ValueError, match="src holds"):
        moe.moe_pack_w13(p, w13[:7], 512, 0, s13, dst, dsc)
    with pytest.raises(ValueError, match="src_scale holds"):
        moe.moe_pack_w13(p, w13, 512, 0, s13[:7], dst, dsc)
    with pytest.raises(ValueError, match="dst holds"):
        moe.moe_pack_w13(p, w13, 512, 0, s13, dst[:-1], dsc)
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_pack_w13(p, w13, 512, 0, s13, dst, dsc)

"""GPU parity of routing, alignment and activation quantisation (bit-exact).

Each entry point is called through the C ABI on cuda:0 and compared with the
oracle on the same seeded inputs: routing ids, alignment offsets / sorted ids /
block experts and the fp8 codes and scales must be identical; routing weights
agree to 1e-5 relative (fp32 exp on the GPU vs fp64 in the oracle).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
import oracle
from gpu_cases import dev, say

pytestmark = pytest.mark.gpu


ROUTE_CASES = [  # T, E_routed, top_k, n_shared, renormalize
    (64, 8, 2, 0, True), (64, 8, 2, 0, False), (1, 128, 8, 0, True), (64, 128, 8, 0, True),
    (16, 512, 10, 1, True), (4096, 512, 10, 1, True), (8192, 20, 8, 0, True),
    (128, 128, 6, 0, False), (33, 1000, 16, 2, True), (5, 64, 64, 0, True),
    # the limits: 1024 experts in all and K' = 64 slots; one logit per lane x 16
    (7, 1020, 60, 4, True), (3, 1024, 1, 0, False)]


@pytest.mark.parametrize("T,Er,k,ns,renorm", ROUTE_CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_route_bitexact(T, Er, k, ns, renorm, ties):
    say(f"route T={T} Er={Er} k={k} ns={ns} renorm={renorm} ties={ties}")
    rng = np.random.default_rng(T * 7 + Er)
    lg = rng.standard_normal((T, Er)).astype(np.float32)
    if ties:  # many equal logits, +0.0 and -0.0 among them
        lg = np.round(lg * 2) / 2
        lg[:, ::7] = -0.0
    p = moe.problem(T=T, H=128, I=128, E_routed=Er, top_k=k, n_shared=ns,
                    renormalize=renorm)
    ids = torch.empty((T, k + ns), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k + ns), dtype=torch.float32, device="cuda")
    moe.moe_route(p, dev(lg), ids, w)
    torch.cuda.synchronize()
    rid, rw = oracle.route(lg, k, renorm, ns, 1.0)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)


def _align_gpu(ids_np, E, K, bm=0):
    T = ids_np.shape[0]
    p = moe.problem(T=T, H=128, I=128, E_routed=E, top_k=min(K, E), block_m=bm)
    p.top_k, p.n_shared = K, 0  # only K' = top_k + n_shared matters to alignment
    p.E_routed, p.E = E, E
    rows, blocks = moe.max_padded_rows(p), moe.max_blocks(p)
    sorted_ids = torch.full((max(rows, 1),), -7, dtype=torch.int32, device="cuda")
    bexp = torch.full((max(blocks, 1),), -7, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    npad = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(moe.align_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    moe.moe_align(p, dev(ids_np), sorted_ids, bexp, offs, npad, ws)
    torch.cuda.synchronize()
    return (moe.block_m(p), int(npad.item()), offs.cpu().numpy(), sorted_ids.cpu().numpy(),
            bexp.cpu().numpy(), rows)


ALIGN_CASES = [  # T, K, E, kind
    (1, 8, 128, "rand"), (64, 2, 8, "rand"), (64, 8, 128, "rand"), (16, 11, 513, "rand"),
    (128, 6, 128, "rand"), (256, 11, 513, "rand"), (4096, 11, 513, "rand"),
    (8192, 8, 20, "rand"), (8192, 6, 128, "rand"), (300, 4, 16, "skew"), (2000, 3, 64, "skew"),
    (100, 4, 32, "masked"), (3000, 5, 40, "masked"), (127, 3, 3, "rand"),
    # no tokens; 1024 experts with exactly one chunk of assignments, and one more
    (0, 8, 128, "rand"), (1024, 1, 1024, "rand"), (1025, 1, 1024, "rand"),
    # chunk histograms of exactly the size scanned in shared memory, and past it
    (32768, 1, 1024, "rand"), (33000, 1, 1024, "skew"), (40000, 1, 1024, "rand")]


@pytest.mark.parametrize("T,K,E,kind", ALIGN_CASES)
def test_align_bitexact(T, K, E, kind):
    say(f"align T={T} K={K} E={E} {kind}")
    rng = np.random.default_rng(T + 31 * E)
    if kind == "skew":   # most assignments on a few experts: long runs, ragged tails
        ids = np.minimum(rng.geometric(0.3, (T, K)) - 1, E - 1)
    else:
        ids = rng.integers(0, E, (T, K))
    if kind == "masked":  # ids outside [0, E) are another rank's experts
        ids = np.where(rng.random((T, K)) < 0.3, rng.choice([-1, E, E + 5], (T, K)), ids)
    ids = ids.astype(np.int32)
    bm, npad, offs, sorted_ids, bexp, rows = _align_gpu(ids, E, K)
    ref = oracle.align(ids, E, bm)
    assert npad == ref["num_padded"] <= rows
    assert np.array_equal(offs, ref["offsets"])
    assert np.array_equal(sorted_ids[:npad], ref["sorted_ids"])
    assert np.array_equal(bexp[:npad // bm], ref["block_expert"])
    assert np.all(sorted_ids[npad:] == -7)  # untouched past num_padded


def test_align_deterministic():
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 513, (4096, 11)).astype(np.int32)
    a = _align_gpu(ids, 513, 11)
    b = _align_gpu(ids, 513, 11)
    for x, y in zip(a[2:5], b[2:5]):
        assert np.array_equal(x, y)


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _bf16_vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("quant", ["fp8_tensor", "fp8_block", "w4a8", "mxfp8"])
@pytest.mark.parametrize("T,H", [(1, 2048), (37, 384), (256, 2048), (8192, 6144)])
def test_quant_act_bitexact(quant, T, H):
    say(f"quant {quant} T={T} H={H}")
    rng = np.random.default_rng(T + H)
    x = rng.standard_normal((T, H)).astype(np.float32) * np.exp(rng.standard_normal((T, 1)))
    if T > 3:
        x[0] = 0.0                                       # all-zero groups
        x[1, :16] = [1.0625, 1.1875, -1.0625, 3.0, 0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10,
                     448.0, 500.0, -1e4, 1e-30, 0.5, 0.25, 7.0, -7.0]
        x[2] *= 1e3
        x[3, 32:64] *= 1e-38                             # subnormal-range blocks
        x[3, 64:96] *= 1e30
    bits = _bf16_bits(x)
    xv = _bf16_vals(bits)
    a1 = np.float32(1.0) if T > 3 else np.float32(np.abs(xv).max() / 448)  # 1.0: ties, saturation
    p = moe.problem(T=T, H=H, I=128, E_routed=8, top_k=2, quant=quant)
    xq = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, H // 128), dtype=torch.float32, device="cuda")
    if quant == "mxfp8":
        xs = torch.empty((T, H // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quant_act(p, dev(bits), torch.tensor(float(a1), device="cuda"), xq, xs)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_x(xv.astype(np.float64), quant, a1)
    assert np.array_equal(xq.cpu().numpy(), rq)
    if quant in ("fp8_block", "mxfp8"):
        assert np.array_equal(xs.cpu().numpy(), rs)


RA_CASES = [  # T, E_routed, top_k, n_shared, renormalize, block_m
    (1, 128, 8, 0, True, 0), (64, 128, 8, 0, True, 0), (16, 512, 10, 1, True, 0),
    (64, 8, 2, 0, False, 0), (128, 128, 6, 0, True, 0), (93, 1000, 11, 0, True, 0),
    (256, 512, 10, 1, True, 0), (4096, 512, 10, 1, True, 0), (8192, 20, 8, 0, True, 0),
    (2, 1020, 60, 4, True, 0),
    # 1024 < A <= 4096 (one workgroup, chunk after chunk) and just past it
    (100, 1000, 30, 2, True, 0), (200, 16, 16, 4, False, 0), (128, 128, 32, 0, True, 0),
    (129, 128, 32, 0, True, 0),
    # small batches: both routing layouts, 64 slots per token, explicit blocks
    (8, 128, 8, 0, True, 0), (3, 1000, 11, 2, False, 0), (1, 1020, 60, 4, True, 0),
    (5, 8, 2, 0, True, 16), (21, 40, 3, 0, False, 64)]


@pytest.mark.parametrize("T,Er,k,ns,renorm,bm", RA_CASES)
def test_prepare_route_align_bitexact(T, Er, k, ns, renorm, bm):
    """moe_prepare (one launch at decode sizes) equals the oracle's routing
    followed by its alignment."""
    say(f"route_align T={T} Er={Er} k={k} ns={ns}")
    rng = np.random.default_rng(3 * T + Er)
    lg = rng.standard_normal((T, Er)).astype(np.float32)
    lg[:, ::5] = np.round(lg[:, ::5])          # some exact ties
    p = moe.problem(T=T, H=128, I=128, E_routed=Er, top_k=k, n_shared=ns,
                    renormalize=renorm, block_m=bm)
    E = Er + ns
    rows, blocks = moe.max_padded_rows(p), moe.max_blocks(p)
    ids = torch.empty((T, k + ns), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k + ns), dtype=torch.float32, device="cuda")
    sorted_ids = torch.full((max(rows, 1),), -7, dtype=torch.int32, device="cuda")
    bexp = torch.full((max(blocks, 1),), -7, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    npad = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(moe.align_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    moe.moe_prepare(p, dev(lg), ids, w, None, None, None, None, sorted_ids, bexp, offs, npad, ws)
    torch.cuda.synchronize()
    rid, rw = oracle.route(lg, k, renorm, ns, 1.0)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)
    bmr = moe.block_m(p)
    ref = oracle.align(rid, E, bmr)
    n = int(npad.item())
    assert n == ref["num_padded"]
    assert np.array_equal(offs.cpu().numpy(), ref["offsets"])
    assert np.array_equal(sorted_ids.cpu().numpy()[:n], ref["sorted_ids"])
    assert np.array_equal(bexp.cpu().numpy()[:n // bmr], ref["block_expert"])


@pytest.mark.parametrize("quant,T,H,Er,k,ns", [("fp8_block", 16, 2048, 512, 10, 1),
                                               ("fp8_tensor", 1, 4096, 128, 6, 0),
                                               ("fp8_tensor", 128, 4096, 128, 6, 0),
                                               ("w4a8", 64, 6144, 20, 8, 0),
                                               ("fp8_block", 300, 2048, 512, 10, 1),
                                               ("fp8_block", 4, 2048, 512, 10, 1),
                                               ("w4a8", 8, 6144, 20, 8, 0),
                                               ("mxfp8", 8, 2048, 128, 8, 0),
                                               ("mxfp4", 64, 2048, 128, 8, 0),
                                               ("mxfp8", 300, 2048, 512, 10, 1),
                                               ("fp8_tensor", 1000, 4096, 128, 6, 0),
                                               ("w4a8", 2049, 6144, 20, 8, 0),
                                               ("mxfp4", 777, 2048, 128, 8, 0)])
def test_prepare_quantise_equals_separate_calls(quant, T, H, Er, k, ns):
    """moe_prepare's fused routing + quantisation + alignment is bit-identical
    to moe_route, moe_quant_act and moe_align called one after another: in one
    workgroup at decode sizes, and above them (T = 300 and up: more than 1024
    assignments) with the routing and the quantisation in one launch -- a
    token per wave (512 routed experts) or per 16-lane row (128 and 20), token
    counts that leave the last routing workgroup partly empty."""
    say(f"prepare {quant} T={T}")
    rng = np.random.default_rng(T + H)
    lg = dev(rng.standard_normal((T, Er)).astype(np.float32))
    x = dev(_bf16_bits(rng.standard_normal((T, H)) * 3))
    a1 = torch.tensor(0.01, device="cuda")
    p = moe.problem(T=T, H=H, I=128, E_routed=Er, top_k=k, n_shared=ns, quant=quant)
    E, K = Er + ns, k + ns
    rows, blocks = moe.max_padded_rows(p), moe.max_blocks(p)

    def bufs():
        return dict(ids=torch.empty((T, K), dtype=torch.int32, device="cuda"),
                    w=torch.empty((T, K), dtype=torch.float32, device="cuda"),
                    xq=torch.empty((T, H), dtype=torch.uint8, device="cuda"),
                    xs=torch.zeros((T, H // 32), dtype=torch.uint8, device="cuda")
                    if quant.startswith("mx") else
                    torch.zeros((T, H // 128), dtype=torch.float32, device="cuda"),
                    si=torch.full((rows,), -7, dtype=torch.int32, device="cuda"),
                    be=torch.full((blocks,), -7, dtype=torch.int32, device="cuda"),
                    off=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                    np=torch.empty(1, dtype=torch.int32, device="cuda"),
                    ws=torch.empty(max(moe.align_workspace_bytes(p), 1), dtype=torch.uint8,
                                   device="cuda"))
    a, b = bufs(), bufs()
    moe.moe_prepare(p, lg, a["ids"], a["w"], x, a1, a["xq"], a["xs"], a["si"], a["be"],
                    a["off"], a["np"], a["ws"])
    moe.moe_route(p, lg, b["ids"], b["w"])
    moe.moe_quant_act(p, x, a1, b["xq"], b["xs"])
    moe.moe_align(p, b["ids"], b["si"], b["be"], b["off"], b["np"], b["ws"])
    torch.cuda.synchronize()
    for key in ("ids", "w", "xq", "xs", "si", "be", "off", "np"):
        assert torch.equal(a[key], b[key]), key

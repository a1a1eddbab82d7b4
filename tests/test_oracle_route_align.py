"""Pins for the oracle's routing, alignment and activation quantisation (CPU).

Routing is pinned to closed forms (softmax via scipy, its ratio identity),
torch.topk, the all-equal and tie special cases and token-permutation
equivariance.  Alignment is pinned to numpy's stable argsort plus the
block invariants.  Quantisation is pinned to torch's fp8 cast and to the
e4m3 error bound.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import codecs


def _logits(T, E, seed):
    return np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)


# ---------------------------------------------------------------- routing
def test_route_full_softmax_closed_form():
    lg = _logits(17, 12, 1)
    ids, w = oracle.route(lg, top_k=12, renormalize=False)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.array_equal(ids, np.argsort(-lg, axis=1, kind="stable"))
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)


@pytest.mark.parametrize("k", [1, 2, 5])
def test_route_topk_matches_torch(k):
    lg = _logits(64, 16, 2)
    ids, w = oracle.route(lg, top_k=k, renormalize=True)
    tv, ti = torch.topk(torch.from_numpy(lg).double(), k, dim=1)
    assert np.array_equal(ids, ti.numpy())
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    # ratio identity of a softmax: w_i / w_j = exp(l_i - l_j)
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), 1)
    np.testing.assert_allclose(w[:, :1] / w, np.exp(sel[:, :1] - sel), rtol=1e-12)
    # without renormalisation the weights are the full-softmax probabilities
    _, w2 = oracle.route(lg, top_k=k, renormalize=False)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(w2, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)


def test_route_all_equal_logits():
    lg = np.full((4, 10), 0.75, np.float32)
    ids, w = oracle.route(lg, top_k=3, renormalize=True)
    assert np.array_equal(ids, np.tile(np.arange(3), (4, 1)))
    np.testing.assert_allclose(w, 1.0 / 3.0, rtol=1e-15)
    _, w2 = oracle.route(lg, top_k=3, renormalize=False)
    np.testing.assert_allclose(w2, 1.0 / 10.0, rtol=1e-15)


def test_route_ties_lower_index_first():
    lg = np.array([[0.5, 2.0, 0.5, 2.0, -1.0, 0.0, -0.0]], np.float32)
    ids, _ = oracle.route(lg, top_k=7, renormalize=True)
    assert list(ids[0]) == [1, 3, 0, 2, 5, 6, 4]


def test_route_token_permutation_equivariant():
    lg = _logits(33, 20, 4)
    perm = np.random.default_rng(5).permutation(33)
    ids, w = oracle.route(lg, 4, True)
    ids_p, w_p = oracle.route(lg[perm], 4, True)
    assert np.array_equal(ids[perm], ids_p)
    assert np.array_equal(w[perm], w_p)


def test_route_shared_slots():
    lg = _logits(5, 8, 6)
    ids, w = oracle.route(lg, 2, True, n_shared=2, shared_gate=0.5)
    assert ids.shape == (5, 4)
    assert np.array_equal(ids[:, 2:], np.tile([8, 9], (5, 1)))
    np.testing.assert_array_equal(w[:, 2:], 0.5)
    np.testing.assert_allclose(w[:, :2].sum(1), 1.0, rtol=1e-14)


# ---------------------------------------------------------------- align
def _check_align(ids, E, bm, res):
    flat = ids.reshape(-1).astype(np.int64)
    A = flat.size
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(res["counts"], counts)
    off = res["offsets"].astype(np.int64)
    assert off[0] == 0 and np.all(off % bm == 0) and np.all(np.diff(off) >= counts)
    assert np.all(np.diff(off) - counts < bm)
    assert res["num_padded"] == off[-1]
    s = res["sorted_ids"].astype(np.int64)
    real = s[s != A]
    # the real entries, in order, are the stable sort of the valid flat ids by expert
    vf = np.nonzero(valid)[0]
    assert np.array_equal(real, vf[np.argsort(flat[vf], kind="stable")])
    assert (s == A).sum() == (np.diff(off) - counts).sum()
    be = res["block_expert"].astype(np.int64)
    assert be.size == off[-1] // bm
    assert np.all(np.diff(be) >= 0)
    for b, e in enumerate(be):
        assert off[e] <= b * bm < off[e + 1]
        blk = s[b * bm:(b + 1) * bm]
        assert np.all(flat[blk[blk != A]] == e)


@pytest.mark.parametrize("T,K,E,bm", [(1, 1, 4, 16), (7, 2, 8, 4), (64, 8, 128, 16),
                                      (200, 6, 20, 128), (50, 11, 513, 16), (9, 3, 5, 1)])
def test_align_invariants(T, K, E, bm):
    rng = np.random.default_rng(T * 100 + E)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    _check_align(ids, E, bm, oracle.align(ids, E, bm))


def test_align_skips_out_of_range_ids():
    ids = np.array([[0, -1], [5, 1], [1, 7]], np.int32)
    res = oracle.align(ids, 5, 2)
    _check_align(ids, 5, 2, res)
    assert res["counts"].sum() == 3


def test_align_offsets_token_permutation_invariant():
    rng = np.random.default_rng(11)
    ids = rng.integers(0, 16, (40, 4)).astype(np.int32)
    perm = rng.permutation(40)
    a, b = oracle.align(ids, 16, 8), oracle.align(ids[perm], 16, 8)
    assert np.array_equal(a["offsets"], b["offsets"])
    assert np.array_equal(a["block_expert"], b["block_expert"])


def test_align_tiny_by_hand():
    ids = np.array([[2, 0], [0, 2], [2, 1]], np.int32)    # f = 0..5
    res = oracle.align(ids, 3, 2)
    assert list(res["counts"]) == [2, 1, 3]
    assert list(res["offsets"]) == [0, 2, 4, 8]
    assert list(res["sorted_ids"]) == [1, 2, 5, 6, 0, 3, 4, 6]
    assert list(res["block_expert"]) == [0, 1, 2, 2]


# ---------------------------------------------------------------- quantisation
def test_quant_group_vs_torch_and_bounds():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((6, 512)) * np.exp(rng.standard_normal((6, 1)) * 3)).astype(np.float32)
    x[2, 128:256] = 0.0
    q, s = oracle.moe.quant_fp8_group(x)
    assert q.shape == x.shape and s.shape == (6, 4) and s.dtype == np.float32
    assert s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)
    # scale = fp32(amax / 448), and the max element of each group encodes to +-448
    g = x.reshape(6, 4, 128)
    amax = np.abs(g).max(-1)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax / np.float32(448)).astype(np.float32)[nz])
    qa = codecs.e4m3_decode(q).reshape(6, 4, 128)
    am = np.abs(g).argmax(-1)
    assert np.all(np.abs(np.take_along_axis(qa, am[..., None], -1))[nz] == 448.0)
    # the codes equal torch's fp8 cast of the same fp32 quotient
    quot = (g / s[..., None]).astype(np.float32).reshape(6, 512)
    assert np.array_equal(q, torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    # error bound of e4m3 round-to-nearest: half a step (2^-4 relative for
    # normals, 2^-10 absolute below 2^-6), in units of the scale
    deq = codecs.e4m3_decode(q).reshape(6, 4, 128) * s[..., None]
    err = np.abs(deq - g)
    bound = np.maximum(np.abs(g) * 2.0 ** -4, 2.0 ** -10 * s[..., None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quant_tensor_vs_torch():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    a1 = np.float32(np.abs(x).max() / 448)
    q = oracle.moe.quant_fp8_tensor(x, a1)
    ref = torch.from_numpy((x / a1).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_padded_intermediate_golden():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "padding_rule.txt")
    for ln in open(path):
        if ln.strip() and not ln.startswith("#"):
            I, gated, want = (int(v) for v in ln.split())
            assert oracle.padded_intermediate(I, bool(gated)) == want

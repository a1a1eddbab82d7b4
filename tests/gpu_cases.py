"""Shared set-up for the GPU parity tests (imported by tests, not collected).

Builds a layer on cuda:0 from the seeded synthetic inputs and checks a pass
against the CPU oracle on the same inputs:
  * moe_forward and the separate entry points (moe_prepare, moe_gemm1_act,
    moe_gemm2_combine) give bit-identical outputs;
  * the routing ids equal the oracle's bit for bit, and the alignment
    (sorted_ids, block_expert, num_padded) equals oracle.align's;
  * the intermediate GEMM1 stores (its codes and scales, read row by row
    through sorted_ids) equals the oracle's code for code, except where the
    oracle's rounding window (oracle.intermediate_window: the fp32
    accumulation error bound) admits the neighbouring code -- every such
    flip is counted and reported;
  * the output is within max-abs 2e-2 of the oracle's, beyond the change the
    observed flips make (routing weight x |code change| x |W2 column|), and
    within rel-L2 1e-2 (3e-2 for int4 weights).
"""
import sys

import numpy as np
import torch

import mixture_experts_layer_09_amd as moe
import oracle
import synth
from synth.configs import MoEConfig
from synth.inputs import bf16_bits_to_f32

TOL = {"bf16": (2e-2, 1e-2), "fp8_tensor": (2e-2, 1e-2), "fp8_block": (2e-2, 1e-2),
       "mxfp8": (2e-2, 1e-2), "mxfp4": (2e-2, 1e-2),
       "w4a8": (None, 3e-2)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    """numpy -> cuda tensor; uint16 bf16 bits become torch.bfloat16."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    t = t.to("cuda")
    return t if dtype is None else t.to(dtype)


def scalar(v):
    return None if v is None else torch.tensor(float(v), dtype=torch.float32, device="cuda")


_weights_cache = {}


def weights_for(cfg: MoEConfig):
    """Host weights of a configuration (one configuration kept at a time)."""
    key = (cfg.name, cfg.quant, cfg.N1)
    if key not in _weights_cache:
        _weights_cache.clear()
        _weights_cache[key] = synth.make_weights(cfg)
    return _weights_cache[key]


def build_layer(cfg: MoEConfig, W, a1=None, a2=None, **kw):
    from mixture_experts_layer_09_amd.layer import MoELayer
    return MoELayer(cfg.H, cfg.I, cfg.E_routed, cfg.top_k, cfg.act, cfg.quant,
                    dev(W["w13"]), dev(W["w2"]), dev(W["w13_scale"]), dev(W["w2_scale"]),
                    scalar(a1), scalar(a2), n_shared=cfg.n_shared, shared_gate=cfg.shared_gate,
                    renormalize=cfg.renormalize, **kw)


def oracle_forward(cfg: MoEConfig, W, x_bits, logits=None, a1=None, a2=None, topk_ids=None,
                   topk_w=None, **kw):
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    return oracle.moe_forward(
        x, W["w13"], W["w2"], quant=cfg.quant, act=cfg.act, E_routed=cfg.E_routed,
        top_k=cfg.top_k, renormalize=cfg.renormalize, n_shared=cfg.n_shared,
        shared_gate=cfg.shared_gate, logits=logits, topk_ids=topk_ids, topk_w=topk_w,
        w13_scale=W["w13_scale"], w2_scale=W["w2_scale"], a1=a1, a2=a2, **kw)


def errors(got, ref, margin=None):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    beyond = err if margin is None else np.maximum(err - margin, 0.0)
    max_beyond = float(beyond.max()) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(err))
    return max_abs, max_beyond, rel


def assert_close(got, ref, quant, label="", margin=None):
    """max-abs 2e-2 (bf16, fp8) beyond each output's margin -- the change the
    intermediate's observed rounding flips make (``parity`` below), none
    otherwise -- and rel-L2 1e-2 (3e-2 for int4 weights) on the full error."""
    if isinstance(ref, dict):
        ref = ref["out"]
    max_abs, beyond, rel = errors(got, ref, margin)
    ma, rl = TOL[quant]
    nmarg = 0 if margin is None else int((margin > 0).sum())
    say(f"  {label}: max_abs={max_abs:.3e} beyond_margin={beyond:.3e} rel_l2={rel:.3e} "
        f"outputs_with_margin={nmarg} of {np.asarray(got).size}")
    assert np.all(np.isfinite(got)), label
    if ma is not None:
        assert beyond <= ma, f"{label}: |err| exceeds {ma} + margin by {beyond - ma}"
    assert rel <= rl, f"{label}: rel_l2 {rel} > {rl}"


def _gpu_intermediate(b, rows, quant, I):
    """The GPU's stored intermediate at padded rows `rows`: values in units
    of their scale [n, I] and the scales (fp32 per 128 columns, E8M0 codes per
    32, or None)."""
    idx = torch.from_numpy(rows).to(b["a2"].device)
    a2 = b["a2"][idx]
    if quant == "bf16":
        v = a2.float().cpu().numpy().astype(np.float64)
    else:
        v = oracle.codecs.e4m3_decode(a2.cpu().numpy())
    sc = None
    if quant == "fp8_block" or quant in ("mxfp8", "mxfp4"):
        sc = b["a2s"][idx].cpu().numpy()
    return v[:, :I], v[:, I:], sc


def _e4m3_rank(v):
    """Signed position of an e4m3 value in the ordered list of values (0 for
    +-0): adjacent values differ by 1."""
    table = oracle.codecs.e4m3_decode(np.arange(127, dtype=np.uint8))
    idx = np.searchsorted(table, np.abs(v))
    return np.where(v < 0, -idx, idx)


def check_intermediate(cfg, W, b, x_bits, ids, ref, a1, a2, label, sample_blocks=None):
    """The intermediate the GPU stored (read through sorted_ids) against the
    oracle.  ``ref``: the oracle forward's result with its stored
    intermediate (return_intermediate).  Every stored value must lie in the
    oracle's rounding window (intermediate_window) -- for all assignments, or,
    with ``sample_blocks`` (the row block size), for the first real row of
    every block, the others being held to one e4m3 step of the exact
    result's rounding.  Returns (margin [T, H] from the stored values that
    differ from the exact result's rounding, counts)."""
    q, act = cfg.quant, cfg.act
    T, K = ids.shape
    A = T * K
    npad = int(b["num_padded"].item())
    srt = b["sorted_ids"][:npad].cpu().numpy().astype(np.int64)
    rows = np.nonzero(srt < A)[0]
    f = srt[rows]
    valid = (ids.reshape(-1) >= 0) & (ids.reshape(-1) < cfg.E)
    assert np.array_equal(np.sort(f), np.nonzero(valid)[0]), f"{label}: row set"
    only = None
    if sample_blocks is not None:
        first = np.unique(rows // sample_blocks, return_index=True)[1]
        only = f[first]
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    win = oracle.intermediate_window(x, W["w13"], quant=q, act=act, topk_ids=ids,
                                     w13_scale=W["w13_scale"], a1=a1, a2=a2, only=only)
    I = win["value"].shape[1]
    v, pad, sc = _gpu_intermediate(b, rows, q, I)
    assert np.all(pad == 0), f"{label}: padded channels not zero"
    ru = ref["units"][f]
    # the scales the values are stored with, GPU and exact
    if q == "bf16":
        sg = sr = 1.0
    elif q in ("fp8_tensor", "w4a8"):
        sg = sr = float(np.float32(a2))
    elif q == "fp8_block":
        gs = sc[:, :I // 128].astype(np.float64)
        rs = ref["scales"][f].astype(np.float64)
        assert np.all(np.abs(gs - rs) <= 1e-3 * rs), f"{label}: block scales"
        sg, sr = np.repeat(gs, 128, axis=1), np.repeat(rs, 128, axis=1)
    else:
        gs = sc[:, :I // 32]
        assert np.all(sc[:, I // 32:] == 0), f"{label}: scales of padded blocks"
        rs = ref["scales"][f]
        assert np.all(np.abs(gs.astype(int) - rs.astype(int)) <= 1), f"{label}: E8M0 scales"
        sg = np.repeat(oracle.codecs.e8m0_decode(gs), 32, axis=1)
        sr = np.repeat(oracle.codecs.e8m0_decode(rs), 32, axis=1)
    vg, vr = v * sg, ru * sr
    differ = vg != vr
    # every stored value near the exact result's rounding: within one e4m3
    # step plus 2^-10 of the format's range (the matrix cores' in-group
    # truncation moves small values of a block by several of the fine steps
    # near zero); bf16 within 2^-6 relative plus 2^-12; the window below is
    # the exact check
    slack_u = 2.0 ** -10 * 448.0
    if q == "bf16":
        far = np.abs(vg - vr) > 2.0 ** -6 * np.abs(vr) + 2.0 ** -12
    elif q in ("mxfp8", "mxfp4"):
        same = sg == sr
        far = np.where(same, (np.abs(_e4m3_rank(v) - _e4m3_rank(ru)) > 1)
                       & (np.abs(v - ru) > slack_u),
                       np.abs(vg - vr) > 0.125 * np.maximum(np.abs(vg), np.abs(vr))
                       + slack_u * np.maximum(sg, sr))
    else:
        far = (np.abs(_e4m3_rank(v) - _e4m3_rank(ru)) > 1) & (np.abs(v - ru) > slack_u)
    nfar = int(far.sum())
    assert nfar == 0, f"{label}: {nfar} stored values far from the exact rounding"
    # the window, on the assignments it was computed for
    done = win["done"][f]
    fw = f[done]
    vw, lo, hi = v[done], win["lo"][fw], win["hi"][fw]
    if q in ("mxfp8", "mxfp4"):
        gsw = gs[done]
        at_lo, at_hi = gsw == win["scale_lo"][fw], gsw == win["scale_hi"][fw]
        nx = int((~(at_lo | at_hi)).sum())
        assert nx == 0, f"{label}: {nx} E8M0 scales outside the kernel's range"
        blk = np.repeat(~at_lo, 32, axis=1)
        lo = np.where(blk, win["lo_x"][fw], lo)
        hi = np.where(blk, win["hi_x"][fw], hi)
    if q == "fp8_block":
        wt = win["tol"][fw]
        assert np.all(np.abs(gs[done] - win["scale"][fw]) <= wt), f"{label}: block scales (window)"
    bad = (vw < lo) | (vw > hi)
    nbad = int(bad.sum())
    if nbad:
        r, c = np.argwhere(bad)[0]
        say(f"  {label}: {nbad} codes outside the window, first at assignment {fw[r]} "
            f"channel {c}: gpu {vw[r, c]} oracle {win['value'][fw][r, c]} "
            f"(window {lo[r, c]} .. {hi[r, c]})")
    assert nbad == 0, f"{label}: {nbad} intermediate codes outside the rounding window"
    # the outputs' margin: routing weight x |change of the stored value| x |W2|
    # over the assignments whose stored values differ from the exact rounding
    # (fp8_block: the code changes at the GPU's scale; the scales' last-bit
    # differences are left to the tolerance)
    dv = np.where(differ, np.abs(v * sg - ru * sg) if q == "fp8_block" else np.abs(vg - vr), 0.0)
    margin = np.zeros((T, cfg.H))
    touched = np.nonzero(dv.max(axis=1) > 0)[0] if dv.size else np.zeros(0, np.int64)
    flat_ids, flat_w = ids.reshape(-1), np.asarray(ref["topk_w"], np.float64).reshape(-1)
    for e in (np.unique(flat_ids[f[touched]]) if touched.size else []):
        sel = touched[flat_ids[f[touched]] == e]
        W2 = np.abs(oracle.dequant_w2(W["w2"], W["w2_scale"], q, int(e)))
        np.add.at(margin, f[sel] // K, np.abs(flat_w[f[sel]])[:, None] * (dv[sel] @ W2.T))
    flips = int(((v != ru) | (sg != sr)).sum()) if q != "fp8_block" else int((v != ru).sum())
    counts = dict(values=int(v.size), flips=flips, windowed=int(vw.size),
                  flagged=int((lo != hi).sum()))
    say(f"  {label}: intermediate {counts['values']} values, {flips} differ from the exact "
        f"result's rounding; window on {counts['windowed']} "
        f"values ({counts['flagged']} with more than one admissible code), 0 outside")
    return margin, counts


def parity(cfg, W, layer, x_bits, logits=None, a1=None, a2=None, topk_ids=None, topk_w=None,
           label="", check_a2=True):
    """moe_forward on the GPU against the oracle (see the module docstring).
    check_a2: True (the intermediate against the window everywhere),
    "sampled" (the window on the first row of every row block, one step of
    the exact rounding elsewhere) or False."""
    T = x_bits.shape[0]
    x = dev(x_bits)
    lg = dev(logits)
    di, dw = dev(topk_ids), dev(topk_w)
    out = layer.forward(x, lg, di, dw)
    b = layer.buffers(T)
    if logits is None:
        b["topk_ids"].copy_(di)
        b["topk_w"].copy_(dw)
    layer.prepare(T, lg, x, b)
    layer.gemm1(T, x, b)
    layer.gemm2(T, b)
    torch.cuda.synchronize()
    same = out.view(torch.int16) == b["out"].view(torch.int16)
    assert bool(same.all()), \
        (f"{label}: moe_forward differs from the separate entry points at "
         f"{int((~same).sum())} of {same.numel()} outputs, first at "
         f"{[tuple(i) for i in (~same).nonzero()[:4].tolist()]}")
    ref = oracle_forward(cfg, W, x_bits, logits, a1, a2, topk_ids=topk_ids,
                         topk_w=None if topk_w is None else np.asarray(topk_w, np.float64),
                         return_intermediate=bool(check_a2))
    ids = ref["topk_ids"]
    if logits is not None:
        assert np.array_equal(b["topk_ids"].cpu().numpy(), ids), f"{label}: routing ids"
    al = oracle.align(ids, cfg.E, moe.block_m(layer.problem(T)))
    npad = int(b["num_padded"].item())
    assert npad == al["num_padded"], f"{label}: num_padded"
    assert np.array_equal(b["sorted_ids"][:npad].cpu().numpy(), al["sorted_ids"])
    margin = None
    if check_a2:
        sample = moe.block_m(layer.problem(T)) if check_a2 == "sampled" else None
        margin, _ = check_intermediate(cfg, W, b, x_bits, ids, ref, a1, a2, label, sample)
    got = out.float().cpu().numpy().astype(np.float64)
    assert_close(got, ref, cfg.quant, label, margin)
    return got, ref


def ad_hoc(cid, quant, act, H, I, E_routed, top_k, n_shared=0, renormalize=True, a2=None):
    """A configuration with arbitrary (small) shapes."""
    return MoEConfig(cid, f"adhoc_{cid}_{quant}_{act}", H=H, I=I, E_routed=E_routed,
                     top_k=top_k, n_shared=n_shared, shared_gate=1.0, act=act, quant=quant,
                     renormalize=renormalize, Ms=(), a2_const=a2 if a2 is not None else
                     (32.0 / 448 if act == "relu2" else 24.0 / 448))

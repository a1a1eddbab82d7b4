"""The fused MoE forward layer, step by step, in fp64 NumPy.

TEST INFRASTRUCTURE (see the package docstring).

Steps, in the order the pages chain them:
  route  -- top-k of the router logits, softmax weights, optional renormalise;
            shared-expert slots appended (Qwen3-Next FP8 page, "Shared-Expert
            Fusion"; TRTLLM-Gen page, op arguments ``topk``/``renormalize``).
  align  -- group the (token, slot) assignments by expert, pad each group to
            the GEMM M tile (Qwen3-Next FP8 page, BLOCK_SIZE_M in the Triton
            config; W4A8 page, ``expert_offsets``/``problem_sizes``).
  quant  -- fp8 activation quantisation for the fp8 / W4A8 modes.
  GEMM1  -- h = W13[e] . x_t, then the activation: SiLU(gate) * up or
            GELU_tanh(gate) * up for gated layers, relu(h)^2 for the non-gated
            one (SwiGLU-fusion page, epilogue; Blackwell gated-MoE page,
            gated activation list; TRTLLM-Gen page, non-gated relu2); the
            intermediate is stored at half width in the compute format.
  GEMM2  -- y = W2[e] . a, weighted by the routing weight and summed back into
            the token's row (Blackwell gated-MoE page: FC2 is non-gated and
            routing/scatter are unchanged).
"""
import numpy as np

from .codecs import (E4M3_MAX, bf16_decode, bf16_round, e2m1_unpack_decode,
                     e4m3_decode, e4m3_encode, e8m0_decode, int4_unpack)

GROUP = 128          # block / group width of the quantised formats
MX_BLOCK = 32        # elements per E8M0 scale in the MX formats
E4M3_EMAX = 8        # exponent of the largest e4m3 power of two (256 <= 448)
MX_MODES = ("mxfp8", "mxfp4")


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def route(logits, top_k, renormalize, n_shared=0, shared_gate=1.0):
    """Top-k routing over fp32 router logits.

    Selection is on the logits: softmax is strictly increasing, so the k
    largest logits are the k largest probabilities.  Order: descending logit,
    lower expert index first on equal logits (+0.0 and -0.0 are equal).
    Weights: with ``renormalize`` the softmax over the k selected logits,
    otherwise the softmax over all routed experts taken at the selected ones.
    ``n_shared`` shared slots follow with ids E_routed..E_routed+n_shared-1 and
    weight ``shared_gate``; they take no part in the renormalisation.

    Returns (ids int32 [T, k+n_shared], weights float64 [T, k+n_shared]).
    """
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, Er = lg.shape
    idx = np.broadcast_to(np.arange(Er), (T, Er))
    key = -lg + 0.0                          # descending; -0.0 folds into +0.0
    order = np.lexsort((idx, key), axis=-1)  # primary key: `key`, then index
    ids = order[:, :top_k]
    sel = np.take_along_axis(lg, ids, axis=1)
    if renormalize:
        m = sel.max(axis=1, keepdims=True)
        ex = np.exp(sel - m)
        w = ex / ex.sum(axis=1, keepdims=True)
    else:
        m = lg.max(axis=1, keepdims=True)
        ex = np.exp(lg - m)
        p = ex / ex.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)
    if n_shared:
        sid = np.broadcast_to(Er + np.arange(n_shared), (T, n_shared))
        ids = np.concatenate([ids, sid], axis=1)
        w = np.concatenate([w, np.full((T, n_shared), float(shared_gate))], axis=1)
    return ids.astype(np.int32), w


# --------------------------------------------------------------------------
# alignment into per-expert blocks
# --------------------------------------------------------------------------
def align(topk_ids, E, block_m):
    """Sort the flat assignments f = t*K' + j by expert into blocks of block_m.

    counts[e]   = number of f with ids[f] == e  (ids outside [0, E) are skipped)
    offsets     = exclusive prefix sum of counts rounded up to block_m (E+1)
    sorted_ids  = for each expert, its f in ascending order, then the sentinel
                  A = T*K' up to the block boundary
    block_expert[b] = the expert whose range holds padded row b*block_m
    num_padded  = offsets[E]
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    A = flat.size
    counts = np.zeros(E, dtype=np.int64)
    members = []
    for e in range(E):
        f = np.nonzero(flat == e)[0]
        counts[e] = f.size
        members.append(f)
    padded = (counts + block_m - 1) // block_m * block_m
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    num_padded = int(offsets[E])
    sorted_ids = np.full(num_padded, A, dtype=np.int64)
    for e in range(E):
        sorted_ids[offsets[e]:offsets[e] + counts[e]] = members[e]
    nblocks = num_padded // block_m
    block_expert = np.empty(nblocks, dtype=np.int64)
    for b in range(nblocks):
        row = b * block_m
        block_expert[b] = int(np.nonzero((offsets[:-1] <= row) & (row < offsets[1:]))[0][0])
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_ids": sorted_ids.astype(np.int32),
        "block_expert": block_expert.astype(np.int32),
        "num_padded": num_padded,
    }


# --------------------------------------------------------------------------
# activation quantisation
# --------------------------------------------------------------------------
def quant_fp8_tensor(v, scale):
    """e4m3(sat(fp32(v) / fp32(scale))) -- one static scale for the tensor."""
    q = np.asarray(v, dtype=np.float32) / np.float32(scale)
    return e4m3_encode(q)


def quant_fp8_group(v, group=GROUP):
    """Per row and per ``group`` consecutive columns: s = fp32(amax / 448)
    (s = 1 when the group is all zero), q = e4m3(fp32(v) / s).

    Returns (codes uint8 [R, C], scales fp32 [R, C/group]).
    """
    f = np.asarray(v, dtype=np.float32)
    R, C = f.shape
    g = f.reshape(R, C // group, group)
    amax = np.abs(g).max(axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = (g / s[..., None]).astype(np.float32)
    return e4m3_encode(q).reshape(R, C), s


def quant_mx8(v):
    """MXFP8 (OCP MX v1.0, conversion of a vector to an MX block): per row
    and per 32 consecutive columns, the shared exponent is
    X = floor(log2(amax)) - 8 (8: the e4m3 emax), kept in [-127, 127], and
    X = -127 for an all-zero block; each element is e4m3(fp32(v) / 2^X),
    nearest even, saturating at 448 (the clamp the specification prescribes
    for magnitudes above the largest normal).

    Returns (codes uint8 [R, C], scale codes uint8 [R, C/32] = X + 127).
    """
    f = np.asarray(v, dtype=np.float32)
    R, C = f.shape
    g = f.reshape(R, C // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.abs(g).max(axis=-1)
    _, ex = np.frexp(amax)                 # amax = m 2^ex, m in [0.5, 1)
    X = np.where(amax > 0, ex - 1 - E4M3_EMAX, -127)
    X = np.clip(X, -127, 127).astype(np.int64)
    q = (g * np.exp2(-X.astype(np.float64))[..., None]).astype(np.float32)
    return e4m3_encode(q).reshape(R, C), (X + 127).astype(np.uint8)


def _mx_scale_full(scale_codes, cols):
    return np.repeat(e8m0_decode(scale_codes), MX_BLOCK, axis=-1)[..., :cols]


def quant_x(x, quant, a1=None):
    """Step a3: the activations as the GEMM1 operand.

    bf16: x itself.  fp8_tensor / w4a8: e4m3 with the static a1.  fp8_block:
    e4m3 per token per 128 columns (dynamic scale).  Returns (codes, scales);
    ``codes`` is None for bf16, ``scales`` is None for the static modes.
    """
    if quant == "bf16":
        return None, None
    if quant in ("fp8_tensor", "w4a8"):
        return quant_fp8_tensor(x, a1), None
    if quant == "fp8_block":
        return quant_fp8_group(x)
    if quant in MX_MODES:
        return quant_mx8(x)
    raise ValueError(quant)


def dequant_x(x, quant, codes, scales, a1=None):
    if quant == "bf16":
        return np.asarray(x, dtype=np.float64)
    if quant in ("fp8_tensor", "w4a8"):
        return e4m3_decode(codes) * float(np.float32(a1))
    if quant == "fp8_block":
        return e4m3_decode(codes) * np.repeat(scales.astype(np.float64), GROUP, axis=1)
    if quant in MX_MODES:
        return e4m3_decode(codes) * _mx_scale_full(scales, codes.shape[1])
    raise ValueError(quant)


# --------------------------------------------------------------------------
# load-time weight preparation (TRTLLM-Gen page, section 2; SwiGLU-fusion
# page, section 3)
# --------------------------------------------------------------------------
def swap_halves(w13):
    """[Up, Gate] -> [Gate, Up] along the row axis of a gated [.., 2I, H] weight."""
    w = np.asarray(w13)
    lead, two_i = w.shape[:-2], w.shape[-2]
    r = w.reshape(lead + (2, two_i // 2) + w.shape[-1:])
    return np.flip(r, axis=len(lead)).reshape(w.shape).copy()


def padded_intermediate(I, gated, align_to=None):
    """Round I up to 16 (gated) or 128 (non-gated), unchanged when aligned."""
    a = align_to if align_to is not None else (16 if gated else 128)
    return (I + a - 1) // a * a


def pad_intermediate(w13, w2, gated, align_to=None):
    """Zero-pad the intermediate dim of W13 [E, (2)I, H] and W2 [E, H, I].

    Gated weights are padded per half, so the gate and up rows of channel c
    stay at rows c and I_p + c (the reading taken for the pages' padding of a
    gated weight; the padded rows are zero either way).
    """
    E, H, I = w2.shape
    Ip = padded_intermediate(I, gated, align_to)
    if Ip == I:
        return w13, w2, I
    halves = 2 if gated else 1
    p13 = np.zeros((E, halves, Ip, w13.shape[-1]), dtype=w13.dtype)
    p13[:, :, :I, :] = w13.reshape(E, halves, I, w13.shape[-1])
    p2 = np.zeros((E, H, Ip), dtype=w2.dtype)
    p2[:, :, :I] = w2
    return p13.reshape(E, halves * Ip, w13.shape[-1]), p2, Ip


def interleave_rows(w13, G):
    """Split [gate(I); up(I)] rows -> [gate 0..G-1, up 0..G-1, gate G..2G-1, ...].

    G = 1 is the layout the SwiGLU-fusion page writes out ([gate0, up0, gate1,
    up1, ...]); larger G keep G gate rows next to their G up rows.
    """
    w = np.asarray(w13)
    lead, two_i, k = w.shape[:-2], w.shape[-2], w.shape[-1]
    I = two_i // 2
    r = w.reshape(lead + (2, I // G, G, k))
    r = np.moveaxis(r, len(lead), len(lead) + 1)      # (.., I/G, 2, G, k)
    return np.ascontiguousarray(r).reshape(w.shape)


def _interleaved_row_origin(two_i, G):
    """Original (split-layout) row of each row of an interleaved W13."""
    I = two_i // 2
    r = np.arange(two_i)
    pair, within = r // (2 * G), r % (2 * G)
    half, c = within // G, pair * G + within % G
    return half * I + c


# --------------------------------------------------------------------------
# weight dequantisation (one expert at a time)
# --------------------------------------------------------------------------
def _dequant(codes, scale, quant, e, row_origin=None):
    if quant == "bf16":
        return bf16_decode(codes[e])
    if quant == "fp8_tensor":
        return e4m3_decode(codes[e]) * float(np.float32(scale[e]))
    if quant == "fp8_block":
        w = e4m3_decode(codes[e])
        n, k = w.shape
        rows = np.arange(n) if row_origin is None else row_origin
        s = scale[e].astype(np.float64)[rows // GROUP]          # [n, K/128]
        return w * np.repeat(s, GROUP, axis=1)[:, :k]
    if quant == "w4a8":
        q = int4_unpack(codes[e]).astype(np.float64)
        n, k = q.shape
        rows = np.arange(n) if row_origin is None else row_origin
        s = bf16_decode(scale[e])[rows]                          # [n, K/128]
        return q * np.repeat(s, GROUP, axis=1)[:, :k]
    if quant in MX_MODES:
        # MX weights: one E8M0 scale per row per 32 K (TRTLLM-Gen page,
        # _align_mxfp8_moe_weights: scales [E, rows, K/32])
        w = e4m3_decode(codes[e]) if quant == "mxfp8" else e2m1_unpack_decode(codes[e])
        n, k = w.shape
        rows = np.arange(n) if row_origin is None else row_origin
        return w * _mx_scale_full(scale[e][rows], k)
    raise ValueError(quant)


def dequant_w13(w13, w13_scale, quant, e, layout_g=None):
    """Expert e's up-projection as fp64 [N1, H], in the row order it is stored.

    For an interleaved layout (``layout_g``), block/group scales are looked up
    through each row's original split-layout index.
    """
    origin = None
    if layout_g is not None:
        origin = _interleaved_row_origin(w13.shape[1], layout_g)
    return _dequant(w13, w13_scale, quant, e, origin)


def dequant_w2(w2, w2_scale, quant, e):
    """Expert e's down-projection as fp64 [H, I]."""
    return _dequant(w2, w2_scale, quant, e)


# --------------------------------------------------------------------------
# intermediate storage (the half-width GEMM1 output in the compute format)
# --------------------------------------------------------------------------
def store_intermediate(a, quant, a2=None):
    """Round the activated intermediate as it is stored, return its value.

    bf16: fp32 then bf16 (nearest even).  fp8_tensor / w4a8: e4m3 of
    fp32(a)/a2, saturating, times a2.  fp8_block: per row and 128 columns,
    s = fp32(amax/448), e4m3 of fp32(a)/s, times s.  mxfp8 / mxfp4: MXFP8 per
    row and 32 columns (quant_mx8).  "exact": unchanged.
    """
    if quant == "exact":
        return a
    if quant == "bf16":
        return bf16_round(a)
    if quant in ("fp8_tensor", "w4a8"):
        return e4m3_decode(quant_fp8_tensor(a, a2)) * float(np.float32(a2))
    if quant == "fp8_block":
        q, s = quant_fp8_group(a)
        return e4m3_decode(q) * np.repeat(s.astype(np.float64), GROUP, axis=1)
    if quant in MX_MODES:
        q, s = quant_mx8(a)
        return e4m3_decode(q) * _mx_scale_full(s, q.shape[1])
    raise ValueError(quant)


# Rounding decisions of the fp8 intermediate that fp32 accumulation in another
# order can take either way: values within this relative distance (plus the
# same absolute amount, for values near zero) of a rounding boundary.
FLIP_REL = 2.0 ** -12


def flip_margin(a, quant, a2=None):
    """Per intermediate value: the change one e4m3 rounding flip can make.

    For the fp8 storage modes, the exact quotient q = a / s (s = a2, or the
    row's per-128-column scale) is compared with the midpoints between
    adjacent e4m3 values (the rounding boundaries; the saturated range above
    448 has none).  Where q lies within FLIP_REL * (|q| + 1) of a boundary,
    either neighbouring code is a correct rounding of a value the kernels may
    have accumulated in fp32; the margin is the gap between the two codes,
    in the intermediate's units.  Elsewhere, and for bf16 / exact storage,
    the margin is 0.
    """
    a = np.asarray(a, dtype=np.float64)
    if quant in ("fp8_tensor", "w4a8"):
        s = np.full(a.shape, float(np.float32(a2)))
    elif quant == "fp8_block":
        _, sg = quant_fp8_group(a)
        s = np.repeat(sg.astype(np.float64), GROUP, axis=1)
    elif quant in MX_MODES:
        return _flip_margin_mx(a)
    else:
        return np.zeros_like(a)
    return _flip_margin_at(a, s)


def _flip_margin_at(a, s):
    q = np.abs(a / s)
    pos = e4m3_decode(np.arange(127, dtype=np.uint8))        # 0 .. 448, increasing
    mids = (pos[1:] + pos[:-1]) / 2.0                        # boundary i: pos[i] | pos[i+1]
    gaps = pos[1:] - pos[:-1]
    i = np.clip(np.searchsorted(mids, q), 1, mids.size - 1)
    near = np.where(np.abs(q - mids[i - 1]) <= np.abs(q - mids[i]), i - 1, i)
    d = np.abs(q - mids[near])
    amb = d <= FLIP_REL * (q + 1.0)
    return np.where(amb, gaps[near] * s, 0.0)


def _silu(g):
    return g / (1.0 + np.exp(-g))


# Gated activations: the gate half goes through one of these, times the up half
# (flashinfer PR 4329 page, sections 1 and 3: silu and gelu_tanh as gated
# activations).  gelu_tanh is GELU in its tanh approximation,
# 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).
def _gelu_tanh(g):
    return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))


GATE_FN = {"silu": _silu, "gelu_tanh": _gelu_tanh}


def _activate(h, act, I, layout_g):
    if act == "relu2":
        r = np.maximum(h, 0.0)
        return r * r
    if layout_g is None:
        gate, up = h[:, :I], h[:, I:]
    else:
        # pair the accumulator columns the way the interleave placed them
        p = h.reshape(h.shape[0], I // layout_g, 2, layout_g)
        gate = p[:, :, 0, :].reshape(h.shape[0], I)
        up = p[:, :, 1, :].reshape(h.shape[0], I)
    return GATE_FN[act](gate) * up


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------
def moe_forward(x, w13, w2, *, quant, act, E_routed, top_k, renormalize,
                n_shared=0, shared_gate=1.0, logits=None, topk_ids=None,
                topk_w=None, w13_scale=None, w2_scale=None, a1=None, a2=None,
                layout_g=None, storage=None, with_margin=False):
    """Route, then per expert: dequantise-then-matmul in fp64.

    x: [T, H] float (bf16 values).  w13/w2: stored codes in the split layout
    (``layout_g`` None) or the interleaved one.  Either ``logits`` or
    (``topk_ids``, ``topk_w``) is given.  ``storage`` overrides how the
    intermediate is rounded ("exact" keeps fp64; default: the quant mode).

    Returns dict(out fp64 [T, H], topk_ids, topk_w, xq, xs) and, with
    ``with_margin``, ``margin`` [T, H]: for each output the largest change
    that rounding flips of ambiguous intermediate values (``flip_margin``)
    can make, sum over them of routing weight * gap * |W2 entry|.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = E_routed + n_shared
    gated = act in GATE_FN
    if logits is not None:
        ids, wts = route(logits, top_k, renormalize, n_shared, shared_gate)
    else:
        ids = np.asarray(topk_ids, dtype=np.int64)
        wts = np.asarray(topk_w, dtype=np.float64)
    K = ids.shape[1]
    xq, xs = quant_x(x, quant, a1)
    xd = dequant_x(x, quant, xq, xs, a1)
    st = storage if storage is not None else quant
    out = np.zeros((T, H), dtype=np.float64)
    margin = np.zeros((T, H), dtype=np.float64) if with_margin else None
    flat_ids = ids.reshape(-1)
    flat_w = wts.reshape(-1)
    for e in range(E):
        f = np.nonzero(flat_ids == e)[0]
        if f.size == 0:
            continue
        t = f // K
        W13 = dequant_w13(w13, w13_scale, quant, e, layout_g)   # [N1, H]
        W2 = dequant_w2(w2, w2_scale, quant, e)                 # [H, I]
        I = W2.shape[1]
        h = xd[t] @ W13.T
        a = _activate(h, act, I, layout_g if gated else None)
        if with_margin:
            mg = flip_margin(a, st, a2) @ np.abs(W2).T
            np.add.at(margin, t, np.abs(flat_w[f])[:, None] * mg)
        a = store_intermediate(a, st, a2)
        y = a @ W2.T
        np.add.at(out, t, flat_w[f][:, None] * y)
    res = {"out": out, "topk_ids": ids.astype(np.int32), "topk_w": wts, "xq": xq, "xs": xs}
    if with_margin:
        res["margin"] = margin
    return res


def _flip_margin_mx(a):
    """flip_margin for the MXFP8 intermediate.  Each element's rounding as
    above, at its block's scale 2^X.  In addition, where the block's amax lies
    within FLIP_REL (relative) of a power of two, fp32 accumulation may put
    it on either side, and the block may take the exponent X or its
    neighbour: there each element's margin also covers the change between its
    values under the two exponents plus one e4m3 step at the coarser one."""
    R, C = a.shape
    nb = C // MX_BLOCK
    q, sc = quant_mx8(a)
    m = _flip_margin_at(a, _mx_scale_full(sc, C))
    f = np.asarray(a, dtype=np.float32).astype(np.float64).reshape(R, nb, MX_BLOCK)
    amax = np.abs(f).max(axis=-1)
    lg = np.log2(np.where(amax > 0, amax, 1.0))
    n = np.round(lg)
    near = (amax > 0) & (np.abs(amax / np.exp2(n) - 1.0) <= FLIP_REL)
    if not near.any():
        return m
    X = sc.astype(np.int64) - 127
    X2 = np.clip(np.where(lg < n, X + 1, X - 1), -127, 127)   # the neighbouring exponent
    v1 = e4m3_decode(q).reshape(R, nb, MX_BLOCK) * np.exp2(X)[..., None]
    q2 = e4m3_encode((f * np.exp2(-X2.astype(np.float64))[..., None]).astype(np.float32))
    v2 = e4m3_decode(q2) * np.exp2(X2)[..., None]
    Xc = np.maximum(X, X2)[..., None].astype(np.float64)
    qc = np.abs(f) * np.exp2(-Xc)
    step = np.exp2(np.floor(np.log2(np.maximum(qc, 2.0 ** -6))) - 3.0) * np.exp2(Xc)
    extra = np.where(near[..., None], np.abs(v1 - v2) + step, 0.0).reshape(R, C)
    return np.maximum(m, extra)

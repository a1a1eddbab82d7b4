"""Fused MoE forward layer for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libmoe.so`` (declared in
``include/moe.h``).  Every step of the layer runs in the library's HIP kernels;
this module only turns torch tensors into device pointers and the current
HIP stream, and raises on a non-zero status.  There is no fallback: importing
the package fails if the library has not been built
(``python mixture_experts_layer_09_amd/build.py``).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")
PLAN_LIB_PATH = os.path.join(HERE, "libmoe_plan.so")

# enum values of include/moe.h
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED = 0, -1, -2
MOE_ERR_ALIGNMENT, MOE_ERR_WORKSPACE, MOE_ERR_HIP = -3, -4, -5
ACT = {"silu": 0, "relu2": 1, "gelu_tanh": 2}
QUANT = {"bf16": 0, "fp8_tensor": 1, "fp8_block": 2, "w4a8": 3, "mxfp8": 4, "mxfp4": 5}

# every entry point declared in include/moe.h
EXPORTS = (
    "moe_status_string", "moe_last_error", "moe_validate", "moe_padded_intermediate",
    "moe_block_m", "moe_max_blocks", "moe_max_padded_rows", "moe_align_workspace_bytes",
    "moe_combine_workspace_bytes", "moe_workspace_bytes", "moe_packed_bytes",
    "moe_pack_w13", "moe_pack_w2", "moe_route", "moe_align", "moe_prepare", "moe_quant_act",
    "moe_gemm1_act", "moe_gemm2_combine", "moe_forward", "moe_forward_noalloc",
)
# bytes of the fixed per-GPU workspace of moe_forward_noalloc
# (MOE_NOALLOC_WORKSPACE_BYTES in include/moe.h)
NOALLOC_WORKSPACE_BYTES = 64 << 20
HOST_ONLY = EXPORTS[:11]
# measurement helpers declared in include/moe_probe.h (not part of the layer)
PROBE_EXPORTS = ("moe_probe_read", "moe_probe_read_blocks", "moe_probe_mfma",
                 "moe_probe_mfma_blocks", "moe_probe_mfma_flops", "moe_probe_mfma_tile")


class MoEError(RuntimeError):
    def __init__(self, status, fn, detail):
        super().__init__(f"{fn}: {status_name(status)} ({status}): {detail}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
        ("E", ctypes.c_int32), ("E_routed", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("n_shared", ctypes.c_int32), ("shared_gate", ctypes.c_float),
        ("renormalize", ctypes.c_int32), ("act", ctypes.c_int32), ("quant", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
    ]


class Weights(ctypes.Structure):
    _fields_ = [
        ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
        ("a1_scale", ctypes.c_void_p), ("a2_scale", ctypes.c_void_p),
    ]


_P = ctypes.POINTER(Problem)
_VP, _SZ, _I32, _I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64


def _declare(lib, host_only=False):
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_validate": (ctypes.c_int, [_P]),
        "moe_padded_intermediate": (_I32, [_I32, _I32, _I32]),
        "moe_block_m": (_I32, [_P]),
        "moe_max_blocks": (_I64, [_P]),
        "moe_max_padded_rows": (_I64, [_P]),
        "moe_align_workspace_bytes": (_SZ, [_P]),
        "moe_combine_workspace_bytes": (_SZ, [_P]),
        "moe_workspace_bytes": (_SZ, [_P]),
        "moe_packed_bytes": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
        "moe_pack_w13": (ctypes.c_int, [_P, _VP, _I32, _I32, _VP, _VP, _VP, _VP]),
        "moe_pack_w2": (ctypes.c_int, [_P, _VP, _I32, _VP, _VP, _VP, _VP]),
        "moe_route": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP]),
        "moe_align": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
        "moe_prepare": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                       _VP, _SZ, _VP]),
        "moe_quant_act": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP]),
        "moe_gemm1_act": (ctypes.c_int, [_P, _VP, _VP, ctypes.POINTER(Weights), _VP, _VP, _VP,
                                         _VP, _VP, _VP]),
        "moe_gemm2_combine": (ctypes.c_int, [_P, _VP, _VP, ctypes.POINTER(Weights), _VP, _VP,
                                             _VP, _VP, _VP, _VP, _SZ, _VP, _VP]),
        "moe_forward": (ctypes.c_int, [_P, ctypes.POINTER(Weights), _VP, _VP, _VP, _VP, _VP,
                                       _VP, _SZ, _VP]),
        "moe_forward_noalloc": (ctypes.c_int, [_P, ctypes.POINTER(Weights), _VP, _VP, _VP, _VP,
                                               _VP, _VP]),
        "moe_probe_read": (ctypes.c_int, [_VP, _SZ, _VP, _VP]),
        "moe_probe_read_blocks": (_I32, []),
        "moe_probe_mfma": (ctypes.c_int, [_I32, _I32, _VP, _VP]),
        "moe_probe_mfma_blocks": (_I32, []),
        "moe_probe_mfma_flops": (_I64, [_I32, _I32]),
        "moe_probe_mfma_tile": (ctypes.c_int, [_I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    }
    for name in (HOST_ONLY if host_only else EXPORTS + PROBE_EXPORTS):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = sig[name]
    return lib


def _hip_runtimes():
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python mixture_experts_layer_09_amd/build.py`")
    # torch ships its own HIP runtime.  Loading it first makes libmoe.so bind to
    # that same runtime (same soname) instead of mapping a second one, so that
    # torch's device memory and streams and the library's kernels live in one
    # runtime.
    import torch  # noqa: F401
    lib = _declare(ctypes.CDLL(LIB_PATH))
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError("two HIP runtimes are mapped into this process: " + ", ".join(rts))
    return lib


lib = _load()


def load_plan_lib():
    """The host-only planner library (g++ build, no HIP) for CPU-side checks."""
    if not os.path.exists(PLAN_LIB_PATH):
        raise ImportError(f"{PLAN_LIB_PATH} is missing")
    return _declare(ctypes.CDLL(PLAN_LIB_PATH), host_only=True)


def status_name(st):
    return lib.moe_status_string(st).decode()


def _check(st, fn):
    if st != MOE_OK:
        raise MoEError(st, fn, lib.moe_last_error().decode())
    return st


# ------------------------------------------------------------------ problem
def problem(T, H, I, E_routed, top_k, act="silu", quant="bf16", n_shared=0,
            shared_gate=1.0, renormalize=True, block_m=0):
    return Problem(T=T, H=H, I=I, E=E_routed + n_shared, E_routed=E_routed, top_k=top_k,
                   n_shared=n_shared, shared_gate=shared_gate, renormalize=int(renormalize),
                   act=ACT[act] if isinstance(act, str) else act,
                   quant=QUANT[quant] if isinstance(quant, str) else quant, block_m=block_m)


def validate(p):
    return lib.moe_validate(ctypes.byref(p))


def padded_intermediate(I, act, quant):
    return lib.moe_padded_intermediate(I, ACT.get(act, act), QUANT.get(quant, quant))


def block_m(p):
    return lib.moe_block_m(ctypes.byref(p))


def max_blocks(p):
    return lib.moe_max_blocks(ctypes.byref(p))


def max_padded_rows(p):
    return lib.moe_max_padded_rows(ctypes.byref(p))


def align_workspace_bytes(p):
    return lib.moe_align_workspace_bytes(ctypes.byref(p))


def combine_workspace_bytes(p):
    return lib.moe_combine_workspace_bytes(ctypes.byref(p))


def workspace_bytes(p):
    return lib.moe_workspace_bytes(ctypes.byref(p))


def packed_bytes(p, which):
    w, s = _SZ(0), _SZ(0)
    _check(lib.moe_packed_bytes(ctypes.byref(p), which, ctypes.byref(w), ctypes.byref(s)),
           "moe_packed_bytes")
    return w.value, s.value


# ------------------------------------------------------------------ marshalling
def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtypes():
    import torch
    bf16 = (torch.bfloat16, torch.int16, torch.uint16)
    u8 = (torch.uint8, torch.int8, torch.float8_e4m3fn)
    return dict(bf16=bf16, u8=u8, f32=(torch.float32,), i32=(torch.int32,))


class _Args:
    """Collects the device pointers of one call after checking what the kernels
    assume of each tensor: a torch tensor of the expected element type,
    contiguous, at least `nbytes` bytes; `on_gpu()` then checks that every one
    lives on a GPU.  Raises ValueError / TypeError before anything reaches the
    library (the C ABI sees raw pointers and cannot check sizes)."""

    def __init__(self):
        self.tensors = []

    def __call__(self, t, name, nbytes, kind=None, required=True):
        import torch
        if t is None:
            if required:
                raise ValueError(f"{name} is required")
            return None
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if kind is not None and t.dtype not in _dtypes()[kind]:
            raise ValueError(f"{name} has dtype {t.dtype}; expected one of "
                             f"{', '.join(str(d) for d in _dtypes()[kind])}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{name} holds {have} bytes; the problem needs {int(nbytes)}")
        self.tensors.append((name, t))
        return t.data_ptr()

    def on_gpu(self):
        for name, t in self.tensors:
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be on a GPU device, not {t.device}")


def _shape(p):
    """Sizes of the problem's buffers (raises MoEError for an invalid problem)."""
    _check(validate(p), "moe_validate")
    K = p.top_k + p.n_shared
    q = p.quant
    return dict(T=p.T, H=p.H, I=p.I, E=p.E, Er=p.E_routed, K=K, A=p.T * K, q=q,
                rows=max_padded_rows(p), blocks=max_blocks(p),
                a2_el=2 if q == QUANT["bf16"] else 1,
                xs=(p.T * (p.H // 128) * 4 if q == QUANT["fp8_block"]
                    else p.T * (p.H // 32) if q in (QUANT["mxfp8"], QUANT["mxfp4"]) else 0),
                a2s_row=((p.I // 128) * 4 if q == QUANT["fp8_block"]
                         else p.I // 32 if q in (QUANT["mxfp8"], QUANT["mxfp4"]) else 0))


def _static_scales(q):
    return q in (QUANT["fp8_tensor"], QUANT["w4a8"])


def _routing_args(a, s, topk_ids, topk_w, required=True):
    return (a(topk_ids, "topk_ids", s["A"] * 4, "i32", required),
            a(topk_w, "topk_w", s["A"] * 4, "f32", required))


def _block_args(a, s, sorted_ids, block_expert, num_padded):
    """The alignment's outputs the GEMMs read."""
    real = s["A"] > 0
    return (a(sorted_ids, "sorted_ids", s["rows"] * 4, "i32", real),
            a(block_expert, "block_expert", s["blocks"] * 4, "i32", real),
            a(num_padded, "num_padded", 4, "i32", real))


def _align_args(a, s, sorted_ids, block_expert, expert_offsets, num_padded):
    """The alignment's outputs, in moe_align's argument order."""
    real = s["A"] > 0
    return (a(sorted_ids, "sorted_ids", s["rows"] * 4, "i32", real),
            a(block_expert, "block_expert", s["blocks"] * 4, "i32", real),
            a(expert_offsets, "expert_offsets", (s["E"] + 1) * 4, "i32"),
            a(num_padded, "num_padded", 4, "i32"))


def _x_args(a, s, x, a1_scale, xq, x_scale):
    """x (bf16), and the quantised copy the fp8 / W4A8 / MX modes make of it."""
    q = s["q"]
    xp = a(x, "x", s["T"] * s["H"] * 2, "bf16", s["T"] > 0)
    if q == QUANT["bf16"] or x is None:
        return xp, None, None, None
    return (xp, a(a1_scale, "a1_scale", 4, "f32", _static_scales(q)),
            a(xq, "xq", s["T"] * s["H"], "u8"),
            a(x_scale, "x_scale", s["xs"], None, s["xs"] > 0))


def _src_bytes(p, which, src_I):
    """Bytes of a checkpoint-layout weight and of its scales (moe_pack_w13/w2)."""
    q, gated = p.quant, p.act != ACT["relu2"]
    n = (2 * src_I if gated else src_I) if which == 13 else p.H
    k = p.H if which == 13 else src_I
    el = {QUANT["bf16"]: 2.0, QUANT["fp8_tensor"]: 1.0, QUANT["fp8_block"]: 1.0,
          QUANT["w4a8"]: 0.5, QUANT["mxfp8"]: 1.0, QUANT["mxfp4"]: 0.5}[q]
    sc = {QUANT["bf16"]: 0, QUANT["fp8_tensor"]: 4,
          QUANT["fp8_block"]: (n // 128) * (k // 128) * 4, QUANT["w4a8"]: n * (k // 128) * 2,
          QUANT["mxfp8"]: n * (k // 32), QUANT["mxfp4"]: n * (k // 32)}[q]
    return int(p.E * n * k * el), int(p.E * sc)


def weights(w13, w2, w13_scale=None, w2_scale=None, a1_scale=None, a2_scale=None):
    """Pointers of packed weights (outputs of moe_pack_w13 / moe_pack_w2)."""
    a = _Args()
    ptrs = [a(t, n, 1, None, False) for t, n in ((w13, "w13"), (w2, "w2"),
                                                   (w13_scale, "w13_scale"),
                                                   (w2_scale, "w2_scale"),
                                                   (a1_scale, "a1_scale"),
                                                   (a2_scale, "a2_scale"))]
    a.on_gpu()
    return Weights(*ptrs)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _pack(which, p, src, src_I, src_scale, dst, dst_scale):
    _check(validate(p), "moe_validate")
    a = _Args()
    sb, ssb = _src_bytes(p, which, src_I)
    db, dsb = packed_bytes(p, which)
    ptrs = (a(src, "src", sb), a(src_scale, "src_scale", ssb, None, ssb > 0),
            a(dst, "dst", db), a(dst_scale, "dst_scale", dsb, None, dsb > 0))
    a.on_gpu()
    return ptrs


def moe_pack_w13(p, src, src_I, swap_halves, src_scale, dst, dst_scale, stream=None):
    s, ss, d, ds = _pack(13, p, src, src_I, src_scale, dst, dst_scale)
    return _check(lib.moe_pack_w13(ctypes.byref(p), s, src_I, int(swap_halves), ss, d, ds,
                                   _stream(stream)), "moe_pack_w13")


def moe_pack_w2(p, src, src_I, src_scale, dst, dst_scale, stream=None):
    s, ss, d, ds = _pack(2, p, src, src_I, src_scale, dst, dst_scale)
    return _check(lib.moe_pack_w2(ctypes.byref(p), s, src_I, ss, d, ds, _stream(stream)),
                  "moe_pack_w2")


def moe_route(p, logits, topk_ids, topk_w, stream=None):
    s, a = _shape(p), _Args()
    lg = a(logits, "logits", s["T"] * s["Er"] * 4, "f32", s["T"] > 0)
    ids, w = _routing_args(a, s, topk_ids, topk_w, s["T"] > 0)
    a.on_gpu()
    return _check(lib.moe_route(ctypes.byref(p), lg, ids, w, _stream(stream)), "moe_route")


def moe_align(p, topk_ids, sorted_ids, block_expert, expert_offsets, num_padded, ws,
              stream=None):
    s, a = _shape(p), _Args()
    ids = a(topk_ids, "topk_ids", s["A"] * 4, "i32", s["A"] > 0)
    al = _align_args(a, s, sorted_ids, block_expert, expert_offsets, num_padded)
    wsp = a(ws, "ws", 0, None, False)
    a.on_gpu()
    return _check(lib.moe_align(ctypes.byref(p), ids, *al, wsp, _nbytes(ws), _stream(stream)),
                  "moe_align")


def moe_prepare(p, logits, topk_ids, topk_w, x, a1_scale, xq, x_scale, sorted_ids,
                block_expert, expert_offsets, num_padded, ws, stream=None):
    s, a = _shape(p), _Args()
    lg = a(logits, "logits", s["T"] * s["Er"] * 4, "f32", False)
    ids, w = _routing_args(a, s, topk_ids, topk_w, False)
    if s["A"] > 0 and (ids is None or (logits is not None and w is None)):
        raise ValueError("topk_ids (and with logits, topk_w) are required")
    xa = _x_args(a, s, x, a1_scale, xq, x_scale) if x is not None else (None,) * 4
    al = _align_args(a, s, sorted_ids, block_expert, expert_offsets, num_padded)
    wsp = a(ws, "ws", 0, None, False)
    a.on_gpu()
    return _check(lib.moe_prepare(ctypes.byref(p), lg, ids, w, *xa, *al, wsp, _nbytes(ws),
                                  _stream(stream)), "moe_prepare")


def moe_quant_act(p, x, a1_scale, xq, x_scale, stream=None):
    s, a = _shape(p), _Args()
    if s["q"] == QUANT["bf16"]:
        return _check(lib.moe_quant_act(ctypes.byref(p), None, None, None, None,
                                        _stream(stream)), "moe_quant_act")
    xa = _x_args(a, s, x, a1_scale, xq, x_scale)
    a.on_gpu()
    return _check(lib.moe_quant_act(ctypes.byref(p), *xa, _stream(stream)), "moe_quant_act")


def moe_gemm1_act(p, x, x_scale, w, sorted_ids, block_expert, num_padded, a2, a2_scale,
                  stream=None):
    s, a = _shape(p), _Args()
    real = s["A"] > 0
    bf = s["q"] == QUANT["bf16"]
    xp = a(x, "x", s["T"] * s["H"] * (2 if bf else 1), "bf16" if bf else "u8", real)
    xs = a(x_scale, "x_scale", s["xs"], None, real and s["xs"] > 0)
    bl = _block_args(a, s, sorted_ids, block_expert, num_padded)
    a2p = a(a2, "a2", s["rows"] * s["I"] * s["a2_el"], "bf16" if bf else "u8", real)
    a2sp = a(a2_scale, "a2_scale", s["rows"] * s["a2s_row"], None, real and s["a2s_row"] > 0)
    a.on_gpu()
    return _check(lib.moe_gemm1_act(ctypes.byref(p), xp, xs, ctypes.byref(w), *bl, a2p, a2sp,
                                    _stream(stream)), "moe_gemm1_act")


def moe_gemm2_combine(p, a2, a2_scale, w, sorted_ids, block_expert, num_padded, topk_ids,
                      topk_w, y_ws, out, stream=None):
    s, a = _shape(p), _Args()
    real = s["T"] > 0
    bf = s["q"] == QUANT["bf16"]
    a2p = a(a2, "a2", s["rows"] * s["I"] * s["a2_el"], "bf16" if bf else "u8", real)
    a2sp = a(a2_scale, "a2_scale", s["rows"] * s["a2s_row"], None, real and s["a2s_row"] > 0)
    bl = _block_args(a, s, sorted_ids, block_expert, num_padded)
    ids, wt = _routing_args(a, s, topk_ids, topk_w, real)
    outp = a(out, "out", s["T"] * s["H"] * 2, "bf16", real)
    yp = a(y_ws, "y_ws", 0, None, False)
    a.on_gpu()
    return _check(lib.moe_gemm2_combine(ctypes.byref(p), a2p, a2sp, ctypes.byref(w), *bl, ids,
                                        wt, yp, _nbytes(y_ws), outp, _stream(stream)),
                  "moe_gemm2_combine")


def moe_forward(p, w, x, logits, topk_ids, topk_w, out, ws, stream=None):
    s, a = _shape(p), _Args()
    real = s["T"] > 0
    xp = a(x, "x", s["T"] * s["H"] * 2, "bf16", real)
    lg = a(logits, "logits", s["T"] * s["Er"] * 4, "f32", False)
    ids, wt = _routing_args(a, s, topk_ids, topk_w, real and logits is None)
    outp = a(out, "out", s["T"] * s["H"] * 2, "bf16", real)
    wsp = a(ws, "ws", 0, None, False)
    a.on_gpu()
    return _check(lib.moe_forward(ctypes.byref(p), ctypes.byref(w), xp, lg, ids, wt, outp, wsp,
                                  _nbytes(ws), _stream(stream)), "moe_forward")


def moe_forward_noalloc(p, w, x, logits, topk_ids, topk_w, out, stream=None):
    """moe_forward with the library's fixed per-GPU workspace (no allocation)."""
    s, a = _shape(p), _Args()
    real = s["T"] > 0
    xp = a(x, "x", s["T"] * s["H"] * 2, "bf16", real)
    lg = a(logits, "logits", s["T"] * s["Er"] * 4, "f32", False)
    ids, wt = _routing_args(a, s, topk_ids, topk_w, real and logits is None)
    outp = a(out, "out", s["T"] * s["H"] * 2, "bf16", real)
    a.on_gpu()
    return _check(lib.moe_forward_noalloc(ctypes.byref(p), ctypes.byref(w), xp, lg, ids, wt,
                                          outp, _stream(stream)), "moe_forward_noalloc")


# ------------------------------------------------------------------ measurement
def probe_read(buf, sink, stream=None):
    """One read-stream launch over the whole tensor `buf` (include/moe_probe.h)."""
    return _check(lib.moe_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                     _stream(stream)), "moe_probe_read")


def probe_mfma(dtype, iters, sink, stream=None):
    """One dense MFMA-loop launch; dtype "bf16" or "fp8".  Returns its FLOPs."""
    d = {"bf16": 0, "fp8": 1}[dtype]
    _check(lib.moe_probe_mfma(d, iters, _ptr(sink), _stream(stream)), "moe_probe_mfma")
    return lib.moe_probe_mfma_flops(d, iters)


def probe_mfma_tile(fmt, a, b, c, d, sa=None, sb=None, stream=None):
    """One matrix-core instruction on one wave (include/moe_probe.h):
    fmt "bf16" (a, b: int16 [64, 8]) or "fp8" (a, b: uint8 [64, 32]); c, d:
    float32 [64, 4]; sa, sb: uint8 [64] E8M0 codes or None."""
    f = {"bf16": 0, "fp8": 1}[fmt]
    per = 16 if f == 0 else 32
    g = _Args()
    ptrs = (g(a, "a", 64 * per), g(b, "b", 64 * per), g(sa, "sa", 64, None, False),
            g(sb, "sb", 64, None, False), g(c, "c", 64 * 16, "f32"), g(d, "d", 64 * 16, "f32"))
    g.on_gpu()
    return _check(lib.moe_probe_mfma_tile(f, *ptrs, _stream(stream)), "moe_probe_mfma_tile")

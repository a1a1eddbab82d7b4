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
    "moe_gemm1_act", "moe_gemm2_combine", "moe_forward",
)
HOST_ONLY = EXPORTS[:11]
# measurement helpers declared in include/moe_probe.h (not part of the layer)
PROBE_EXPORTS = ("moe_probe_read", "moe_probe_read_blocks", "moe_probe_mfma",
                 "moe_probe_mfma_blocks", "moe_probe_mfma_flops")


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
        "moe_probe_read": (ctypes.c_int, [_VP, _SZ, _VP, _VP]),
        "moe_probe_read_blocks": (_I32, []),
        "moe_probe_mfma": (ctypes.c_int, [_I32, _I32, _VP, _VP]),
        "moe_probe_mfma_blocks": (_I32, []),
        "moe_probe_mfma_flops": (_I64, [_I32, _I32]),
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


def weights(w13, w2, w13_scale=None, w2_scale=None, a1_scale=None, a2_scale=None):
    return Weights(_ptr(w13), _ptr(w2), _ptr(w13_scale), _ptr(w2_scale), _ptr(a1_scale),
                   _ptr(a2_scale))


def moe_pack_w13(p, src, src_I, swap_halves, src_scale, dst, dst_scale, stream=None):
    return _check(lib.moe_pack_w13(ctypes.byref(p), _ptr(src), src_I, int(swap_halves),
                                   _ptr(src_scale), _ptr(dst), _ptr(dst_scale), _stream(stream)),
                  "moe_pack_w13")


def moe_pack_w2(p, src, src_I, src_scale, dst, dst_scale, stream=None):
    return _check(lib.moe_pack_w2(ctypes.byref(p), _ptr(src), src_I, _ptr(src_scale), _ptr(dst),
                                  _ptr(dst_scale), _stream(stream)), "moe_pack_w2")


def moe_route(p, logits, topk_ids, topk_w, stream=None):
    return _check(lib.moe_route(ctypes.byref(p), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                _stream(stream)), "moe_route")


def moe_align(p, topk_ids, sorted_ids, block_expert, expert_offsets, num_padded, ws,
              stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return _check(lib.moe_align(ctypes.byref(p), _ptr(topk_ids), _ptr(sorted_ids),
                                _ptr(block_expert), _ptr(expert_offsets), _ptr(num_padded),
                                _ptr(ws), nbytes, _stream(stream)), "moe_align")


def moe_prepare(p, logits, topk_ids, topk_w, x, a1_scale, xq, x_scale, sorted_ids,
                block_expert, expert_offsets, num_padded, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return _check(lib.moe_prepare(ctypes.byref(p), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                  _ptr(x), _ptr(a1_scale), _ptr(xq), _ptr(x_scale),
                                  _ptr(sorted_ids), _ptr(block_expert), _ptr(expert_offsets),
                                  _ptr(num_padded), _ptr(ws), nbytes, _stream(stream)),
                  "moe_prepare")


def moe_quant_act(p, x, a1_scale, xq, x_scale, stream=None):
    return _check(lib.moe_quant_act(ctypes.byref(p), _ptr(x), _ptr(a1_scale), _ptr(xq),
                                    _ptr(x_scale), _stream(stream)), "moe_quant_act")


def moe_gemm1_act(p, x, x_scale, w, sorted_ids, block_expert, num_padded, a2, a2_scale,
                  stream=None):
    return _check(lib.moe_gemm1_act(ctypes.byref(p), _ptr(x), _ptr(x_scale), ctypes.byref(w),
                                    _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
                                    _ptr(a2), _ptr(a2_scale), _stream(stream)), "moe_gemm1_act")


def moe_gemm2_combine(p, a2, a2_scale, w, sorted_ids, block_expert, num_padded, topk_ids,
                      topk_w, y_ws, out, stream=None):
    nbytes = 0 if y_ws is None else y_ws.numel() * y_ws.element_size()
    return _check(lib.moe_gemm2_combine(ctypes.byref(p), _ptr(a2), _ptr(a2_scale),
                                        ctypes.byref(w), _ptr(sorted_ids), _ptr(block_expert),
                                        _ptr(num_padded), _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(y_ws), nbytes, _ptr(out), _stream(stream)),
                  "moe_gemm2_combine")


def moe_forward(p, w, x, logits, topk_ids, topk_w, out, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return _check(lib.moe_forward(ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(logits),
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(ws), nbytes,
                                  _stream(stream)), "moe_forward")


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

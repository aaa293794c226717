"""ctypes binding of libmoe_dispatch.so.

Argument marshalling only: the functions here take torch tensors (device
memory) and the current torch stream, pass raw pointers to the C ABI of
include/moe_dispatch.h, and raise MoEError on a non-OK return.  Workspace is
allocated through torch when the caller does not pass one.  There is no
fallback: if the library is not built, loading raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_F32 = 0
MOE_BF16 = 1
MOE_SILU = 0
MOE_SWIGLU = 1
MOE_FLAG_RECOMPUTE_G = 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe_dispatch.so")

EXPORTED = (
    "moe_dispatch_build",
    "moe_dispatch_build_noalloc",
    "moe_ffn_forward",
    "moe_ffn_backward",
    "moe_last_error",
    "moe_profile_enable",
    "moe_profile_reset",
    "moe_profile_read",
)


class Shape(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("d", ctypes.c_int32), ("h", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("act", ctypes.c_int32), ("flags", ctypes.c_int32)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class MoEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises OSError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run "
                      "python token_dispatch_expert_amd/build_lib.py")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    SZ = ctypes.POINTER(ctypes.c_size_t)
    S = ctypes.POINTER(Shape)
    lib.moe_dispatch_build.argtypes = [S, P, P, P, P, P, P, P, SZ, P]
    lib.moe_dispatch_build_noalloc.argtypes = [S, P, P, P, P, P, P, P]
    lib.moe_ffn_forward.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_ffn_backward.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ,
                                     P]
    for f in ("moe_dispatch_build", "moe_dispatch_build_noalloc", "moe_ffn_forward",
              "moe_ffn_backward",
              "moe_profile_enable", "moe_profile_reset", "moe_profile_read"):
        getattr(lib, f).restype = ctypes.c_int
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_profile_enable.argtypes = [ctypes.c_int]
    lib.moe_profile_reset.argtypes = []
    lib.moe_profile_read.argtypes = [ctypes.POINTER(KernelStat), ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_int)]
    _lib = lib
    return lib


def moe_last_error() -> str:
    return load_library().moe_last_error().decode()


def _check(rc):
    if rc != MOE_OK:
        raise MoEError(rc, moe_last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dt(shape):
    return torch.float32 if shape.dtype == MOE_F32 else torch.bfloat16


def _want(name, t, dtype, numel, optional=False):
    """A tensor argument must be a contiguous device tensor of the expected
    element type and size (raw integer addresses pass unchecked)."""
    if t is None:
        if optional:
            return
        raise MoEError(MOE_ERR_INVALID_ARG, f"{name} is None")
    if isinstance(t, int):
        return
    if not t.is_cuda:
        raise MoEError(MOE_ERR_INVALID_ARG, f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoEError(MOE_ERR_INVALID_ARG, f"{name} must be {dtype} (got {t.dtype})")
    if t.numel() != numel:
        raise MoEError(MOE_ERR_INVALID_ARG, f"{name} must hold {numel} elements (got {t.numel()})")
    if not t.is_contiguous():
        raise MoEError(MOE_ERR_INVALID_ARG, f"{name} must be contiguous")


def _check_routing_args(shape, eti, offsets, tei, tim, gates):
    L, E, K = shape.L, shape.E, shape.K
    _want("expert_token_indices", eti, torch.int32, L * K)
    _want("expert_token_offsets", offsets, torch.int32, E + 1)
    _want("token_expert_indices", tei, torch.int32, L * K)
    _want("token_index_map", tim, torch.int32, L * K)
    _want("gates", gates, torch.float32, L * K)


def _check_ffn_args(shape, x, W1, W3, W2, **outs):
    L, d, h, E, K = shape.L, shape.d, shape.h, shape.E, shape.K
    dt = _dt(shape)
    glu = shape.act == MOE_SWIGLU
    _want("x", x, dt, L * d)
    _want("W1", W1, dt, E * d * h)
    _want("W3", W3, dt, E * d * h, optional=not glu)
    _want("W2", W2, dt, E * h * d)
    sizes = {"y": L * d, "dy": L * d, "dx": L * d, "A": L * K * h, "B": L * K * h,
             "dW1": E * d * h, "dW3": E * d * h, "dW2": E * h * d}
    for name, t in outs.items():
        _want(name, t, dt, sizes[name], optional=(not glu and name in ("B", "dW3")))


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(L, d, h, E, K, dtype=MOE_BF16, act=MOE_SWIGLU, flags=0) -> Shape:
    return Shape(int(L), int(d), int(h), int(E), int(K), int(dtype), int(act), int(flags))


def _run(fn, shape, args, ws, stream, device):
    """Query the workspace size when ws is None, allocate it with torch, call."""
    nbytes = ctypes.c_size_t(0)
    if ws is None:
        _check(fn(ctypes.byref(shape), *args, None, ctypes.byref(nbytes), None))
        ws = torch.empty(max(int(nbytes.value), 256), dtype=torch.uint8, device=device)
    nbytes.value = ws.numel() * ws.element_size()
    _check(fn(ctypes.byref(shape), *args, _ptr(ws), ctypes.byref(nbytes), _stream(stream)))
    return ws


def workspace_bytes(name: str, shape: Shape) -> int:
    """Workspace size of moe_dispatch_build / moe_ffn_forward / moe_ffn_backward
    for `shape` (host-only query, launches nothing).  Pointer arguments are
    passed as 16-byte aligned placeholders that are never dereferenced."""
    lib = load_library()
    fn = getattr(lib, name)
    n = {"moe_dispatch_build": 6, "moe_ffn_forward": 12, "moe_ffn_backward": 16}[name]
    tail = [None] if name == "moe_ffn_backward" else []   # dlogits: optional, not needed
    nbytes = ctypes.c_size_t(0)
    _check(fn(ctypes.byref(shape), *([256] * n), *tail, None, ctypes.byref(nbytes), None))
    return int(nbytes.value)


def moe_dispatch_build(shape, logits, eti, offsets, tei, tim, gates, ws=None, stream=None):
    lib = load_library()
    _want("logits", logits, torch.float32, shape.L * shape.E)
    _check_routing_args(shape, eti, offsets, tei, tim, gates)
    args = [_ptr(logits), _ptr(eti), _ptr(offsets), _ptr(tei), _ptr(tim), _ptr(gates)]
    return _run(lib.moe_dispatch_build, shape, args, ws, stream, logits.device)


def moe_dispatch_build_noalloc(shape, logits, eti, offsets, tei, tim, gates, stream=None):
    """moe_dispatch_build with the library's own scratch array as workspace:
    nothing is allocated (see include/moe_dispatch.h for the size limit and
    the rule that calls overlapping on one GPU race)."""
    lib = load_library()
    _want("logits", logits, torch.float32, shape.L * shape.E)
    _check_routing_args(shape, eti, offsets, tei, tim, gates)
    _check(lib.moe_dispatch_build_noalloc(ctypes.byref(shape), _ptr(logits), _ptr(eti),
                                          _ptr(offsets), _ptr(tei), _ptr(tim), _ptr(gates),
                                          _stream(stream)))


MOE_NOALLOC_WS_BYTES = 24 << 20


def moe_ffn_forward(shape, x, W1, W3, W2, eti, offsets, tei, tim, gates, y, A, B,
                    ws=None, stream=None):
    lib = load_library()
    _check_routing_args(shape, eti, offsets, tei, tim, gates)
    _check_ffn_args(shape, x, W1, W3, W2, y=y, A=A, B=B)
    args = [_ptr(x), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(eti), _ptr(offsets), _ptr(tei),
            _ptr(tim), _ptr(gates), _ptr(y), _ptr(A), _ptr(B)]
    return _run(lib.moe_ffn_forward, shape, args, ws, stream, x.device)


def moe_ffn_backward(shape, dy, x, W1, W3, W2, eti, offsets, tei, tim, gates, A, B,
                     dx, dW1, dW3, dW2, dlogits=None, ws=None, stream=None):
    """dlogits: optional [L, E] float32 output, the router-logit gradient."""
    lib = load_library()
    _check_routing_args(shape, eti, offsets, tei, tim, gates)
    _check_ffn_args(shape, x, W1, W3, W2, dy=dy, A=A, B=B, dx=dx, dW1=dW1, dW3=dW3, dW2=dW2)
    _want("dlogits", dlogits, torch.float32, shape.L * shape.E, optional=True)
    args = [_ptr(dy), _ptr(x), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(eti), _ptr(offsets),
            _ptr(tei), _ptr(tim), _ptr(gates), _ptr(A), _ptr(B), _ptr(dx), _ptr(dW1),
            _ptr(dW3), _ptr(dW2), _ptr(dlogits)]
    return _run(lib.moe_ffn_backward, shape, args, ws, stream, x.device)


def profile_enable(on: bool = True):
    _check(load_library().moe_profile_enable(1 if on else 0))


def profile_reset():
    _check(load_library().moe_profile_reset())


def profile_read() -> dict:
    """{kernel name: (launches, total_ms)} accumulated since the last reset."""
    lib = load_library()
    n = ctypes.c_int(0)
    _check(lib.moe_profile_read(None, 0, ctypes.byref(n)))
    arr = (KernelStat * max(n.value, 1))()
    _check(lib.moe_profile_read(arr, n.value, ctypes.byref(n)))
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms))
            for i in range(n.value)}

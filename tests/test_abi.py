"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/moe_dispatch.h declares, and rejects bad arguments before any
HIP call (so no compute is launched here)."""

import ctypes
import os
import re
import subprocess

import pytest

from token_dispatch_expert_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dispatch.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from token_dispatch_expert_amd import build_lib
        build_lib.build(verbose=False)
    return B.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("moe_dispatch_build", "moe_ffn_forward", "moe_ffn_backward", "moe_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(moe_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    assert set(B.EXPORTED) == set(declared_functions())


FAKE = 4096  # 16-byte aligned placeholder address, never dereferenced: every call
# below either fails validation or stops at the workspace-size check (nbytes=0),
# so nothing is launched


def call_build(lib, shape, ptrs=None, ws=FAKE, nbytes=0):
    p = ptrs or [FAKE] * 6
    n = ctypes.c_size_t(nbytes)
    rc = lib.moe_dispatch_build(ctypes.byref(shape) if shape is not None else None, *p,
                                ws, ctypes.byref(n), None)
    return rc, n.value


def call_fwd(lib, shape, ptrs=None, ws=FAKE, nbytes=0):
    p = ptrs or [FAKE] * 12
    n = ctypes.c_size_t(nbytes)
    rc = lib.moe_ffn_forward(ctypes.byref(shape), *p, ws, ctypes.byref(n), None)
    return rc, n.value


def call_bwd(lib, shape, ptrs=None, ws=FAKE, nbytes=0):
    p = ptrs or [FAKE] * 16
    if len(p) == 16:
        p = p + [None]           # dlogits: optional
    n = ctypes.c_size_t(nbytes)
    rc = lib.moe_ffn_backward(ctypes.byref(shape), *p, ws, ctypes.byref(n), None)
    return rc, n.value


GOOD = dict(L=1024, d=64, h=128, E=8, K=2, dtype=B.MOE_BF16, act=B.MOE_SWIGLU)


def shp(**kw):
    a = dict(GOOD)
    a.update(kw)
    return B.make_shape(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), B.MOE_ERR_INVALID_ARG),
    (dict(L=-5), B.MOE_ERR_INVALID_ARG),
    (dict(E=0), B.MOE_ERR_INVALID_ARG),
    (dict(K=0), B.MOE_ERR_INVALID_ARG),
    (dict(K=9), B.MOE_ERR_INVALID_ARG),
    (dict(E=1025, K=2), B.MOE_ERR_UNSUPPORTED),
    (dict(E=257, K=9), B.MOE_ERR_UNSUPPORTED),      # K > 8 only up to 256 experts
    (dict(E=256, K=256), B.MOE_ERR_UNSUPPORTED),
    (dict(L=1 << 30, K=2), B.MOE_ERR_UNSUPPORTED),
])
def test_routing_shape_errors(lib, kw, code):
    rc, _ = call_build(lib, shp(**kw))
    assert rc == code
    assert lib.moe_last_error().decode()
    rc, _ = call_fwd(lib, shp(**kw))
    assert rc == code
    rc, _ = call_bwd(lib, shp(**kw))
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), B.MOE_ERR_INVALID_ARG),
    (dict(act=3), B.MOE_ERR_INVALID_ARG),
    (dict(d=0), B.MOE_ERR_INVALID_ARG),
    (dict(h=-8), B.MOE_ERR_INVALID_ARG),
    (dict(d=60), B.MOE_ERR_UNSUPPORTED),
    (dict(h=100), B.MOE_ERR_UNSUPPORTED),
    # in-tile byte offsets of the GEMM epilogues are 32-bit: widths are capped
    (dict(d=(1 << 20) + 8), B.MOE_ERR_UNSUPPORTED),
    (dict(h=(1 << 20) + 8), B.MOE_ERR_UNSUPPORTED),
    (dict(h=1 << 24), B.MOE_ERR_UNSUPPORTED),
    (dict(h=(1 << 20) + 8, dtype=B.MOE_F32), B.MOE_ERR_UNSUPPORTED),
])
def test_ffn_shape_errors(lib, kw, code):
    assert call_fwd(lib, shp(**kw))[0] == code
    assert call_bwd(lib, shp(**kw))[0] == code


def test_null_shape(lib):
    n = ctypes.c_size_t(0)
    rc = lib.moe_dispatch_build(None, *([FAKE] * 6), FAKE, ctypes.byref(n), None)
    assert rc == B.MOE_ERR_INVALID_ARG
    assert "shape" in lib.moe_last_error().decode()


@pytest.mark.parametrize("i", range(6))
def test_build_null_or_misaligned_pointer(lib, i):
    p = [FAKE] * 6
    p[i] = None
    assert call_build(lib, shp(), p)[0] == B.MOE_ERR_INVALID_ARG
    p[i] = FAKE + 2
    assert call_build(lib, shp(), p)[0] == B.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("i", range(12))
def test_forward_null_or_misaligned_pointer(lib, i):
    p = [FAKE] * 12
    p[i] = None
    assert call_fwd(lib, shp(), p)[0] == B.MOE_ERR_INVALID_ARG
    # W3 (index 2) and B (index 11) may be NULL for SiLU
    if i in (2, 11):
        assert call_fwd(lib, shp(act=B.MOE_SILU), p, ws=None)[0] == B.MOE_OK
    p[i] = FAKE + 4
    rc = call_fwd(lib, shp(), p)[0]
    if i in (4, 5, 6, 7, 8):     # int32 / float32 arrays need only 4-byte alignment
        assert rc == B.MOE_ERR_WORKSPACE       # reaches the workspace check
    else:
        assert rc == B.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("i", range(16))
def test_backward_null_pointer(lib, i):
    p = [FAKE] * 16
    p[i] = None
    assert call_bwd(lib, shp(), p)[0] == B.MOE_ERR_INVALID_ARG
    if i in (3, 11, 14):          # W3, B, dW3 unused for SiLU
        assert call_bwd(lib, shp(act=B.MOE_SILU), p, ws=None)[0] == B.MOE_OK


def test_backward_optional_router_gradient(lib):
    # dlogits may be NULL or any 4-byte aligned address; 2-byte aligned is rejected
    assert call_bwd(lib, shp(), [FAKE] * 16 + [None])[0] == B.MOE_ERR_WORKSPACE
    assert call_bwd(lib, shp(), [FAKE] * 16 + [FAKE + 4])[0] == B.MOE_ERR_WORKSPACE
    assert call_bwd(lib, shp(), [FAKE] * 16 + [FAKE + 2])[0] == B.MOE_ERR_INVALID_ARG


def test_workspace_query_and_too_small(lib):
    for call, n in ((call_build, 6), (call_fwd, 12), (call_bwd, 16)):
        rc, need = call(lib, shp(), ws=None, nbytes=0)
        assert rc == B.MOE_OK and need > 0
        rc, _ = call(lib, shp(), ws=FAKE, nbytes=need - 1)
        assert rc == B.MOE_ERR_WORKSPACE
        assert "workspace" in lib.moe_last_error().decode()
        rc, _ = call(lib, shp(), ws=FAKE + 16, nbytes=need)
        assert rc == B.MOE_ERR_INVALID_ARG          # ws must be 256-byte aligned
    n = ctypes.c_size_t(0)
    assert lib.moe_dispatch_build(ctypes.byref(shp()), *([FAKE] * 6), None, None, None) \
        == B.MOE_ERR_INVALID_ARG


def test_workspace_grows_with_L(lib):
    a = B.workspace_bytes("moe_ffn_forward", shp(L=1000))
    b = B.workspace_bytes("moe_ffn_forward", shp(L=100000))
    assert b > a
    # forward keeps a [L*K, h] activation buffer and a float32 [L, d] accumulator
    L, K, h, d = 100000, 2, 128, 64
    assert b >= L * K * h * 2 + L * d * 4
    # float32 output needs no separate accumulator
    c = B.workspace_bytes("moe_ffn_forward", shp(L=100000, dtype=B.MOE_F32))
    assert c >= L * K * h * 4


def test_profile_calls_without_gpu(lib):
    assert lib.moe_profile_enable(0) == B.MOE_OK
    assert lib.moe_profile_reset() == B.MOE_OK
    n = ctypes.c_int(-1)
    assert lib.moe_profile_read(None, 0, ctypes.byref(n)) == B.MOE_OK
    assert n.value >= 0


def test_largest_widths_accepted(lib):
    """d = h = MOE_MAX_WIDTH passes validation (the workspace query answers)."""
    for dt in (B.MOE_BF16, B.MOE_F32):
        rc, need = call_fwd(lib, shp(L=256, d=1 << 20, h=1 << 20, dtype=dt), ws=None)
        assert rc == B.MOE_OK and need > 0


def test_binding_rejects_host_or_mistyped_tensors(lib):
    """The Python binding checks device placement, dtype, size and contiguity
    before it reaches the C ABI."""
    import torch
    s = shp(L=16, d=64, h=128, E=4, K=2)
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    with pytest.raises(B.MoEError, match="device tensor"):
        B.moe_dispatch_build(s, torch.zeros(16, 4), i32(32), i32(5), i32(32), i32(32),
                             torch.zeros(32))
    meta = dict(dtype=torch.float32, device="meta")
    with pytest.raises(B.MoEError):
        B.moe_dispatch_build(s, torch.empty(16, 4, **meta), i32(32), i32(5), i32(32), i32(32),
                             torch.zeros(32))


def test_noalloc_rejects_shapes_beyond_the_scratch_array(lib):
    """moe_dispatch_build_noalloc validates like moe_dispatch_build and refuses
    a shape whose workspace exceeds the library's scratch array, before any
    HIP call."""
    big = B.make_shape(1 << 22, 8, 8, 64, 6)        # needs about 84 MiB
    n = ctypes.c_size_t(0)
    assert lib.moe_dispatch_build(ctypes.byref(big), *([FAKE] * 6), None, ctypes.byref(n),
                                  None) == B.MOE_OK
    assert n.value > B.MOE_NOALLOC_WS_BYTES
    assert lib.moe_dispatch_build_noalloc(ctypes.byref(big), *([FAKE] * 6), None) \
        == B.MOE_ERR_UNSUPPORTED
    assert "scratch" in lib.moe_last_error().decode()
    # the 1M-token, 64-expert routing fits
    n = ctypes.c_size_t(0)
    fit = B.make_shape(1 << 20, 8, 8, 64, 6)
    assert lib.moe_dispatch_build(ctypes.byref(fit), *([FAKE] * 6), None, ctypes.byref(n),
                                  None) == B.MOE_OK
    assert n.value <= B.MOE_NOALLOC_WS_BYTES
    for kw, code in ((dict(L=0), B.MOE_ERR_INVALID_ARG), (dict(E=1025, K=2), B.MOE_ERR_UNSUPPORTED)):
        assert lib.moe_dispatch_build_noalloc(ctypes.byref(shp(**kw)), *([FAKE] * 6), None) == code
    p = [FAKE] * 6
    p[3] = FAKE + 2
    assert lib.moe_dispatch_build_noalloc(ctypes.byref(shp()), *p, None) == B.MOE_ERR_INVALID_ARG


def test_library_sources_allocate_nothing():
    """The library's sources call no allocating HIP routine (the caller owns
    every buffer; the allocation-free entry point's array is static)."""
    csrc = os.path.join(ROOT, "token_dispatch_expert_amd", "csrc")
    banned = re.compile(r"\bhip(Malloc\w*|Free\w*|HostMalloc|ExtMallocWithFlags|MallocAsync|"
                        r"MemPool\w*)\s*\(")
    for f in sorted(os.listdir(csrc)):
        src = open(os.path.join(csrc, f)).read()
        src = re.sub(r"//.*", "", src)
        assert not banned.search(src), f"{f} calls an allocating HIP routine"


def test_expert_counts_up_to_1024_accepted(lib):
    for E, K in ((257, 8), (512, 6), (1024, 8), (1024, 1), (256, 255)):
        rc, need = call_build(lib, shp(E=E, K=K), ws=None)
        assert rc == B.MOE_OK and need > 0, (E, K)
        assert call_fwd(lib, shp(E=E, K=K), ws=None)[0] == B.MOE_OK
        assert call_bwd(lib, shp(E=E, K=K), ws=None)[0] == B.MOE_OK


def test_recompute_g_drops_the_g_buffer(lib):
    """MOE_FLAG_RECOMPUTE_G replaces the [L*K, h] G buffer of the forward and
    the backward workspace by one [L, h] piece (a slot pass's rows, or a
    group of experts' routes); unknown flag bits are rejected."""
    for act, dt, es, K in ((B.MOE_SWIGLU, B.MOE_BF16, 2, 2), (B.MOE_SILU, B.MOE_F32, 4, 3)):
        a = dict(L=3000, d=64, h=200, E=8, K=K, dtype=dt, act=act)
        base = B.make_shape(**a)
        low = B.make_shape(**a, flags=B.MOE_FLAG_RECOMPUTE_G)
        for n in ("moe_ffn_forward", "moe_ffn_backward"):
            d = B.workspace_bytes(n, base) - B.workspace_bytes(n, low)
            assert abs(d - 3000 * (K - 1) * 200 * es) < 256, (n, d)
        assert B.workspace_bytes("moe_dispatch_build", base) == \
            B.workspace_bytes("moe_dispatch_build", low)
    bad = B.make_shape(**dict(GOOD), flags=2)
    assert call_fwd(lib, bad)[0] == B.MOE_ERR_INVALID_ARG
    assert call_bwd(lib, bad)[0] == B.MOE_ERR_INVALID_ARG

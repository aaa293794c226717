"""The allocation-free dispatch entry point against moe_dispatch_build, through
the C ABI: indices bit-exact and gates bitwise equal, on two calls in a row,
the second with a smaller input (the scratch array keeps the first call's
contents).  Collected last, so that it also runs after every other test in
the same process."""

import ctypes

import pytest
import torch

from gpu_helpers import require_gpu, say
from token_dispatch_expert_amd import binding as B
from token_dispatch_expert_amd import workloads as W

pytestmark = pytest.mark.gpu


def _outputs(cfg, dev):
    L, E, K = cfg.L, cfg.E, cfg.K
    i32 = dict(dtype=torch.int32, device=dev)
    # filled with a pattern so that an element left unwritten would show
    return dict(eti=torch.full((L * K,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                tei=torch.full((L, K), -7, **i32), tim=torch.full((L, K), -7, **i32),
                gates=torch.full((L, K), -7.0, dtype=torch.float32, device=dev))


def _with_workspace(cfg, logits, dev):
    o = _outputs(cfg, dev)
    shape = B.make_shape(cfg.L, 8, 8, cfg.E, cfg.K)
    B.moe_dispatch_build(shape, logits, o["eti"], o["offsets"], o["tei"], o["tim"], o["gates"])
    return o


def _noalloc(cfg, logits, dev):
    """Straight through the C ABI with ctypes."""
    lib = B.load_library()
    o = _outputs(cfg, dev)
    shape = B.make_shape(cfg.L, 8, 8, cfg.E, cfg.K)
    rc = lib.moe_dispatch_build_noalloc(
        ctypes.byref(shape), logits.data_ptr(), o["eti"].data_ptr(), o["offsets"].data_ptr(),
        o["tei"].data_ptr(), o["tim"].data_ptr(), o["gates"].data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert rc == B.MOE_OK, lib.moe_last_error().decode()
    return o


def _same(a, b):
    for k in ("eti", "offsets", "tei", "tim"):
        assert torch.equal(a[k], b[k]), f"{k} differs"
    assert torch.equal(a["gates"].view(torch.int32), b["gates"].view(torch.int32)), "gates differ"


@pytest.mark.parametrize("first,second", [
    # the 1M-token, 64-expert routing (21 MiB of scratch), then a smaller one
    ((1048576, 64, 6), (1000, 16, 4)),
    # byte-map routing (E > 64), then a bit-mask one with a ragged tail
    ((20000, 128, 8), (777, 8, 2)),
])
def test_noalloc_matches_workspace_build(first, second):
    dev = require_gpu()
    for i, (L, E, K) in enumerate((first, second)):
        cfg = W.MoEConfig(f"noalloc-{L}-{E}-{K}", L, 8, 8, E, K, W.SWIGLU, W.BF16)
        say(f"  call {i + 1}: L={L} E={E} K={K}")
        logits = W.make_logits(cfg, 40 + i, dev)
        ref = _with_workspace(cfg, logits, dev)
        got = _noalloc(cfg, logits, dev)
        torch.cuda.synchronize()
        _same(got, ref)
        # a second call on the same stream gives the same bytes again
        again = _noalloc(cfg, logits, dev)
        torch.cuda.synchronize()
        _same(again, ref)

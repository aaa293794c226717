"""Device memory of one layer step (build + forward + backward): the calls
allocate nothing (the allocator's count and peak do not move during the
step), so the step's peak is the inputs, the declared output and checkpoint
buffers and one workspace of the queried size; the checkpoint kept between
forward and backward is A and B alone, as large as the closed form of the
oracle says."""

import pytest
import torch

import oracle
from gpu_helpers import require_gpu, say
from token_dispatch_expert_amd import binding as B
from token_dispatch_expert_amd import workloads as W
from token_dispatch_expert_amd.layer import MoELayerBuffers

pytestmark = pytest.mark.gpu

# torch's caching allocator hands out blocks of at least the requested size:
# rounded up to 512 bytes, and a large block is not split when less than
# 1 MiB would remain, so one allocation may hold up to about 2 MiB more
SLACK = 2 << 20


@pytest.mark.parametrize("recompute_g", [False, True], ids=["keep_g", "recompute_g"])
@pytest.mark.parametrize("cfg", [
    W.small_config(8192, 512, 1024, 16, 4, W.SWIGLU, W.BF16),
    W.small_config(5000, 256, 768, 8, 2, W.SILU, W.BF16),
    W.CONFIGS[3],
], ids=lambda c: c.name)
def test_step_allocates_only_declared_buffers(cfg, recompute_g):
    dev = require_gpu()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(dev)
    inp = W.make_inputs(cfg, 7, dev)
    torch.cuda.synchronize()
    m_inputs = torch.cuda.memory_allocated(dev) - base
    buf = MoELayerBuffers(cfg, dev, router_grad=True, recompute_g=recompute_g)
    torch.cuda.synchronize()
    m_layer = torch.cuda.memory_allocated(dev) - base - m_inputs

    declared = [t for t in (buf.eti, buf.offsets, buf.tei, buf.tim, buf.gates, buf.y, buf.A, buf.B,
                            buf.dx, buf.dW1, buf.dW3, buf.dW2, buf.dlogits, buf.ws) if t is not None]
    want = sum(t.numel() * t.element_size() for t in declared)
    assert want <= m_layer <= want + SLACK * len(declared)
    ws = max(B.workspace_bytes(n, buf.shape)
             for n in ("moe_dispatch_build", "moe_ffn_forward", "moe_ffn_backward"))
    assert buf.ws.numel() == ws

    torch.cuda.reset_peak_memory_stats(dev)
    before = torch.cuda.memory_allocated(dev)
    n_alloc = torch.cuda.memory_stats(dev)["allocation.all.allocated"]
    buf.step(inp)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats(dev)["allocation.all.allocated"] == n_alloc, \
        "a call allocated device memory"
    assert torch.cuda.max_memory_allocated(dev) == before     # nothing beyond the buffers
    peak = before - base
    assert peak == m_inputs + m_layer
    es = 2 if cfg.dtype == W.BF16 else 4
    ckpt = buf.A.numel() * es + (buf.B.numel() * es if buf.B is not None else 0)
    assert ckpt == oracle.checkpoint_bytes(cfg.L, cfg.K, cfg.h, cfg.act, es)
    say(f"    inputs {m_inputs / 2**20:.1f} MiB, layer buffers {m_layer / 2**20:.1f} MiB "
        f"(checkpoint {ckpt / 2**20:.1f} MiB, workspace {ws / 2**20:.1f} MiB), peak {peak / 2**20:.1f} MiB")

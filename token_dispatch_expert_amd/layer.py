"""Buffers and call sequence for one MoE layer step on a GPU.

Allocates every device buffer once (outputs, checkpoint, one workspace sized
for the largest of the three calls, which run in order on one stream) and
issues moe_dispatch_build -> moe_ffn_forward -> moe_ffn_backward through the
binding.  Plumbing only: all arithmetic happens in the HIP library.
"""

from __future__ import annotations

import torch

from . import binding as B
from .workloads import MoEConfig, SWIGLU, F32


class MoELayerBuffers:
    """router_grad=True also allocates dlogits [L, E] float32 and asks the
    backward for the router-logit gradient.  recompute_g=True sets
    MOE_FLAG_RECOMPUTE_G: no [L*K, h] G buffer in the workspace."""

    def __init__(self, cfg: MoEConfig, device="cuda", router_grad: bool = False,
                 recompute_g: bool = False):
        self.cfg = cfg
        self.device = torch.device(device)
        L, d, h, E, K = cfg.L, cfg.d, cfg.h, cfg.E, cfg.K
        R = L * K
        dt = cfg.torch_dtype
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.shape = B.make_shape(L, d, h, E, K, B.MOE_F32 if cfg.dtype == F32 else B.MOE_BF16,
                                  B.MOE_SWIGLU if cfg.act == SWIGLU else B.MOE_SILU,
                                  B.MOE_FLAG_RECOMPUTE_G if recompute_g else 0)
        self.eti = torch.empty(R, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.tei = torch.empty(L, K, **i32)
        self.tim = torch.empty(L, K, **i32)
        self.gates = torch.empty(L, K, dtype=torch.float32, device=dev)
        self.y = torch.empty(L, d, dtype=dt, device=dev)
        self.A = torch.empty(R, h, dtype=dt, device=dev)
        self.B = torch.empty(R, h, dtype=dt, device=dev) if cfg.act == SWIGLU else None
        self.dx = torch.empty(L, d, dtype=dt, device=dev)
        self.dW1 = torch.empty(E, d, h, dtype=dt, device=dev)
        self.dW3 = torch.empty(E, d, h, dtype=dt, device=dev) if cfg.act == SWIGLU else None
        self.dW2 = torch.empty(E, h, d, dtype=dt, device=dev)
        self.dlogits = torch.empty(L, E, dtype=torch.float32, device=dev) if router_grad else None
        nbytes = max(B.workspace_bytes("moe_dispatch_build", self.shape),
                     B.workspace_bytes("moe_ffn_forward", self.shape),
                     B.workspace_bytes("moe_ffn_backward", self.shape))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def build(self, logits, stream=None):
        B.moe_dispatch_build(self.shape, logits, self.eti, self.offsets, self.tei, self.tim,
                             self.gates, ws=self.ws, stream=stream)

    def forward(self, x, W1, W3, W2, stream=None):
        B.moe_ffn_forward(self.shape, x, W1, W3, W2, self.eti, self.offsets, self.tei, self.tim,
                          self.gates, self.y, self.A, self.B, ws=self.ws, stream=stream)

    def backward(self, dy, x, W1, W3, W2, stream=None):
        B.moe_ffn_backward(self.shape, dy, x, W1, W3, W2, self.eti, self.offsets, self.tei,
                           self.tim, self.gates, self.A, self.B, self.dx, self.dW1, self.dW3,
                           self.dW2, dlogits=self.dlogits, ws=self.ws, stream=stream)

    def step(self, inp: dict, stream=None):
        """Build + forward + backward on the inputs of workloads.make_inputs."""
        self.build(inp["logits"], stream)
        self.forward(inp["x"], inp["W1"], inp["W3"], inp["W2"], stream)
        self.backward(inp["dy"], inp["x"], inp["W1"], inp["W3"], inp["W2"], stream)

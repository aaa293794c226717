"""Synthetic, seeded workloads for the MoE layer.

This module holds only shapes and random-number recipes; it contains none of
the layer's arithmetic.  Tests, the smoke check and the benchmark draw their
inputs from here, for the GPU library and for the CPU oracle alike.

Every tensor comes from its own torch.Generator seeded with
``seed * 16 + tensor_id`` on the device the tensor is created on, so a
(seed, device) pair always gives the same bytes.  The CPU and GPU generators
are different streams; a parity test that runs on the GPU draws once on the
GPU and copies the inputs it needs to the host for the oracle.

Recipe (same for every config unless noted):
  router logits  ~ N(0, 1), float32, shape [L, E]
  x, dy          ~ N(0, 1), shape [L, d]
  W1, W3         ~ N(0, 1) / sqrt(d), shape [E, d, h]
  W2             ~ N(0, 1) / sqrt(d), shape [E, h, d]
Values are drawn in float32 and rounded to nearest-even bfloat16 for bf16
configs; the oracle reads the rounded values, exactly.

The skewed config adds a per-expert bias to the logits:
  b_e = 2 * log(w_{e+1}),  w_r = r^-1.2 / sum_j j^-1.2 (Zipf, s = 1.2),
and replaces the last expert's bias by -1e4 so that it receives no token.
"""

from __future__ import annotations

import dataclasses
import math

import torch

F32 = 0
BF16 = 1
SILU = 0
SWIGLU = 1

TENSOR_IDS = {"logits": 0, "x": 1, "W1": 2, "W3": 3, "W2": 4, "dy": 5}


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    L: int
    d: int
    h: int
    E: int
    K: int
    act: int          # SILU or SWIGLU
    dtype: int        # F32 or BF16
    zipf_skew: bool = False

    @property
    def R(self) -> int:
        return self.L * self.K

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    def flops_fwd_bwd(self) -> int:
        """Dense-GEMM flops of forward + backward (per route: SiLU 12*d*h,
        SwiGLU 18*d*h)."""
        per = 18 if self.act == SWIGLU else 12
        return per * self.R * self.d * self.h


CONFIGS = {
    1: MoEConfig("tiny-silu-f32", 256, 64, 128, 8, 2, SILU, F32),
    2: MoEConfig("L16k-d1024-h4096-E8-K2-silu-bf16", 16384, 1024, 4096, 8, 2, SILU, BF16),
    3: MoEConfig("L64k-d2048-h8192-E16-K4-swiglu-bf16", 65536, 2048, 8192, 16, 4, SWIGLU, BF16),
    4: MoEConfig("L128k-d4096-h14336-E8-K2-swiglu-bf16-zipf", 131072, 4096, 14336, 8, 2,
                 SWIGLU, BF16, zipf_skew=True),
    5: MoEConfig("L1M-d2048-h1408-E64-K6-swiglu-bf16", 1048576, 2048, 1408, 64, 6, SWIGLU, BF16),
}


def zipf_bias(E: int, s: float = 1.2) -> torch.Tensor:
    """Per-expert logit bias of the skewed workload (float32, length E)."""
    w = [r ** (-s) for r in range(1, E + 1)]
    tot = sum(w)
    b = [2.0 * math.log(wi / tot) for wi in w]
    b[E - 1] = -1e4
    return torch.tensor(b, dtype=torch.float64).to(torch.float32)


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 16 + TENSOR_IDS[name])
    return g


def make_logits(cfg: MoEConfig, seed: int, device="cpu") -> torch.Tensor:
    z = torch.randn(cfg.L, cfg.E, generator=_gen(seed, "logits", device),
                    device=device, dtype=torch.float32)
    if cfg.zipf_skew:
        z += zipf_bias(cfg.E).to(device)
    return z


def make_tensor(cfg: MoEConfig, name: str, seed: int, device="cpu") -> torch.Tensor:
    """One of x, W1, W3, W2, dy, in the config's dtype."""
    shapes = {
        "x": (cfg.L, cfg.d),
        "dy": (cfg.L, cfg.d),
        "W1": (cfg.E, cfg.d, cfg.h),
        "W3": (cfg.E, cfg.d, cfg.h),
        "W2": (cfg.E, cfg.h, cfg.d),
    }
    t = torch.randn(*shapes[name], generator=_gen(seed, name, device),
                    device=device, dtype=torch.float32)
    if name in ("W1", "W3", "W2"):
        t *= 1.0 / math.sqrt(cfg.d)
    return t.to(cfg.torch_dtype)


def make_inputs(cfg: MoEConfig, seed: int, device="cpu") -> dict:
    """All layer inputs: logits, x, W1, W3 (None for SiLU), W2, dy."""
    out = {"logits": make_logits(cfg, seed, device)}
    for name in ("x", "W1", "W3", "W2", "dy"):
        if name == "W3" and cfg.act != SWIGLU:
            out[name] = None
            continue
        out[name] = make_tensor(cfg, name, seed, device)
    return out


def small_config(L, d, h, E, K, act=SWIGLU, dtype=BF16, name=None) -> MoEConfig:
    return MoEConfig(name or f"L{L}-d{d}-h{h}-E{E}-K{K}-a{act}-t{dtype}", L, d, h, E, K, act, dtype)

"""Seeded synthetic inputs for the MoE layer forward pass.

This module only draws random tensors of the configured shapes; it holds none
of the layer's arithmetic (no softmax, selection, permutation, MLP or
combine).  Both the HIP path and the CPU oracle are fed from here.

Recipe (every config, seed 0 unless stated):
  * X ~ N(0, 1), stored in the config's dtype (fp32, or fp32 rounded to bf16
    to nearest-even).
  * Router logits, fp32, one of
      - "direct":     logits ~ N(0, 1);
      - "proj":       logits = X @ Wr with Wr ~ N(0, 1/d) (fp32 product of the
                      stored X, computed by torch on the generating device);
      - "proj_bias":  X @ Wr + b, b ~ N(0, bias_var) per expert;
      - "bias":       z + b, z ~ N(0, 1), b ~ N(0, bias_var) per expert.
    N(0, v) names the variance.
  * W1, W3 ~ N(0, 1/d) with shape [E, d, n]; W2 ~ N(0, 1/n) with shape
    [E, n, d]; fp32 rounded to the config's dtype.
  * Each tensor has its own torch.Generator seeded with seed*1000 + id
    (X=1, Wr=2, b=3, W1=4, W3=5, W2=6, logits=7).  Streams differ between the
    CPU and GPU generators, so one test draws its inputs once, on one device,
    and hands the same tensors to both sides.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    E: int
    K: int
    n: int
    dtype: str = "bf16"          # "f32" or "bf16": X, W*, Xp, Act, Y, out
    logits: str = "direct"       # "direct" | "proj" | "proj_bias" | "bias"
    bias_var: float = 0.0
    gate_only: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def A(self) -> int:
        return self.T * self.K

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The workloads named for this layer: a tiny fp32 layer, two gate-only shapes,
# and three bf16 layers shaped like Mixtral, DeepSeek-V3 and a fine-grained MoE.
CONFIGS = {
    "tiny": MoEConfig("tiny", T=256, d=128, E=8, K=2, n=256, dtype="f32", logits="direct"),
    "gate_s": MoEConfig("gate_s", T=2048, d=0, E=8, K=2, n=0, dtype="f32", gate_only=True),
    "gate_l": MoEConfig("gate_l", T=262144, d=0, E=128, K=8, n=0, dtype="f32", gate_only=True),
    "mixtral": MoEConfig("mixtral", T=8192, d=4096, E=8, K=2, n=14336, logits="proj"),
    "dsv3": MoEConfig("dsv3", T=8192, d=7168, E=256, K=8, n=2048, logits="proj_bias", bias_var=1.5),
    "fine": MoEConfig("fine", T=16384, d=1536, E=128, K=4, n=256, logits="bias", bias_var=2.0),
}

_IDS = {"X": 1, "Wr": 2, "b": 3, "W1": 4, "W3": 5, "W2": 6, "logits": 7}


def _gen(device, seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + _IDS[name])
    return g


def _normal(shape, var: float, dtype, device, g) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if var != 1.0:
        x.mul_(math.sqrt(var))
    return x.to(dtype)


def make_router(cfg: MoEConfig, device="cpu", seed: int = 0):
    """Router weights Wr [d, E] ~ N(0, 1/d) fp32 and the per-expert bias [E] ~ N(0, bias_var)
    (None without one) -- the same draws make_logits uses."""
    dev = torch.device(device)
    Wr = _normal((cfg.d, cfg.E), 1.0 / cfg.d, torch.float32, dev, _gen(dev, seed, "Wr"))
    b = _normal((cfg.E,), cfg.bias_var, torch.float32, dev, _gen(dev, seed, "b")) if cfg.bias_var else None
    return Wr, b


def make_logits(cfg: MoEConfig, device="cpu", seed: int = 0, X: torch.Tensor | None = None):
    dev = torch.device(device)
    if cfg.logits == "direct":
        return _normal((cfg.T, cfg.E), 1.0, torch.float32, dev, _gen(dev, seed, "logits"))
    if cfg.logits in ("proj", "proj_bias"):
        assert X is not None
        Wr, b = make_router(cfg, dev, seed)
        lg = X.float() @ Wr
        if cfg.logits == "proj_bias":
            lg += b
        return lg.contiguous()
    if cfg.logits == "bias":
        z = _normal((cfg.T, cfg.E), 1.0, torch.float32, dev, _gen(dev, seed, "logits"))
        return (z + _normal((cfg.E,), cfg.bias_var, torch.float32, dev, _gen(dev, seed, "b"))).contiguous()
    raise ValueError(cfg.logits)


def make_weights(cfg: MoEConfig, device="cpu", seed: int = 0):
    """W1, W3 [E, d, n] ~ N(0, 1/d); W2 [E, n, d] ~ N(0, 1/n); drawn one expert at a time."""
    dev = torch.device(device)
    dt = cfg.torch_dtype
    out = {}
    for name, shape, var in (("W1", (cfg.d, cfg.n), 1.0 / cfg.d), ("W3", (cfg.d, cfg.n), 1.0 / cfg.d),
                             ("W2", (cfg.n, cfg.d), 1.0 / cfg.n)):
        g = _gen(dev, seed, name)
        W = torch.empty((cfg.E,) + shape, dtype=dt, device=dev)
        for e in range(cfg.E):
            W[e] = _normal(shape, var, dt, dev, g)
        out[name] = W
    return out


def make_inputs(cfg: MoEConfig, device="cpu", seed: int = 0) -> dict:
    """All inputs of one config as torch tensors on `device`."""
    dev = torch.device(device)
    out = {}
    if cfg.gate_only:
        out["logits"] = make_logits(cfg, dev, seed)
        return out
    X = _normal((cfg.T, cfg.d), 1.0, cfg.torch_dtype, dev, _gen(dev, seed, "X"))
    out["X"] = X
    out["logits"] = make_logits(cfg, dev, seed, X)
    out.update(make_weights(cfg, dev, seed))
    return out


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 tensors come back as their uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()

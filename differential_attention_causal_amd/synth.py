"""Seeded synthetic inputs for causal differential attention.

This module only draws and casts random tensors; it holds none of the method's
arithmetic.  Both the HIP path and the float64 oracle consume the tensors it
returns (the oracle after a copy to host memory), so neither side generates its
own inputs.

Recipe (the same for every workload):
  * one ``torch.Generator`` on the target device, seeded with ``1000 + workload
    number`` unless a seed is given;
  * tensors are drawn as float32 standard normals in the fixed order
    q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, dout;
  * Q/K/V (and dout) are multiplied in float32 by the workload's scale and then
    cast to the workload's element type (float32 -> bfloat16 rounds to nearest
    even); the oracle reads the exact values of the rounded tensors;
  * the four lambda vectors are float32 with standard deviation 0.1.

The same seed gives the same values on the same device type; a CPU generator
and a GPU generator give different streams, so a parity test draws on one
device and copies to the other.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload shape.

    kind: "fwd" (prefill forward), "decode" (one query per sequence against a
    cache of length ``seqlen``) or "train" (forward then backward).
    """
    number: int
    name: str
    kind: str
    batch: int
    heads: int
    seqlen: int
    head_dim: int
    layer: int
    dtype: str          # "fp32" or "bf16"
    scale: float        # multiplier applied to the standard normals of Q/K/V
    lam_std: float = 0.1

    @property
    def dv(self) -> int:
        return 2 * self.head_dim

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny fp32 forward B1 H2 N64 d16", "fwd", 1, 2, 64, 16, 1, "fp32", 1.0),
    2: Workload(2, "prefill bf16 forward B4 H8 N2048 d64", "fwd", 4, 8, 2048, 64, 4, "bf16",
                1.0 / math.sqrt(2.0)),
    3: Workload(3, "long-context bf16 forward B1 H16 N32768 d64", "fwd", 1, 16, 32768, 64, 12,
                "bf16", 1.0),
    4: Workload(4, "decode bf16 64 seqs x H16 L8192 d64", "decode", 64, 16, 8192, 64, 8, "bf16",
                1.0),
    5: Workload(5, "training bf16 fwd+bwd B8 H12 N4096 d64", "train", 8, 12, 4096, 64, 6, "bf16",
                1.0),
}


def custom(kind: str, batch: int, heads: int, seqlen: int, head_dim: int, layer: int,
           dtype: str, scale: float = 1.0, number: int = 0) -> Workload:
    """A workload outside the five named ones (edge cases, small parity shapes)."""
    return Workload(number, f"custom {kind} B{batch} H{heads} N{seqlen} d{head_dim} {dtype}",
                    kind, batch, heads, seqlen, head_dim, layer, dtype, scale)


def _normal(gen: torch.Generator, shape, device, chunk: int = 1 << 28) -> torch.Tensor:
    """float32 standard normals, drawn in chunks so huge tensors need little scratch."""
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=torch.float32, device=device)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        out[lo:hi] = torch.randn(hi - lo, generator=gen, dtype=torch.float32, device=device)
    return out.view(*shape)


def _cast(x: torch.Tensor, scale: float, dt: torch.dtype) -> torch.Tensor:
    if scale != 1.0:
        x.mul_(scale)          # float32 multiply
    return x if dt == torch.float32 else x.to(dt)  # round to nearest even


def make_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                with_dout: Optional[bool] = None) -> Dict[str, torch.Tensor]:
    """Draw one workload's inputs on ``device``.

    Shapes (row-major, contiguous):
      fwd/train: q1, q2, k1, k2 [B,H,N,d]; v [B,H,N,2d]; dout [B,H,N,2d] (train)
      decode:    q1, q2 [B,H,d]; k1, k2 [B,H,L,d]; v [B,H,L,2d]
      always:    lq1, lk1, lq2, lk2 [d] float32
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    B, H, N, d, dv = w.batch, w.heads, w.seqlen, w.head_dim, w.dv
    dt = w.torch_dtype
    qshape = (B, H, d) if w.kind == "decode" else (B, H, N, d)
    out: Dict[str, torch.Tensor] = {}
    for name in ("q1", "q2"):
        out[name] = _cast(_normal(gen, qshape, device), w.scale, dt)
    for name in ("k1", "k2"):
        out[name] = _cast(_normal(gen, (B, H, N, d), device), w.scale, dt)
    out["v"] = _cast(_normal(gen, (B, H, N, dv), device), w.scale, dt)
    for name in ("lq1", "lk1", "lq2", "lk2"):
        out[name] = _normal(gen, (d,), device).mul_(w.lam_std)
    if with_dout if with_dout is not None else (w.kind == "train"):
        out["dout"] = _cast(_normal(gen, (B, H, N, dv), device), 1.0, dt)
    return out


def make_lambda_layers(n_layers: int, head_dim: int, device="cpu", seed: int = 0,
                       std: float = 0.1) -> Dict[str, torch.Tensor]:
    """The four lambda vectors of n_layers layers, each float32 [n_layers, head_dim]
    (row k belongs to the k-th layer), normal with standard deviation ``std``."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return {name: _normal(gen, (n_layers, head_dim), device).mul_(std)
            for name in ("lq1", "lk1", "lq2", "lk2")}


def make_proj_inputs(batch: int, seqlen: int, heads: int, head_dim: int, d_model: int,
                     device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of the projections, bf16: x [B, N, d_model] standard normal, the fused
    weight w_qkv [3 H 2d, d_model] normal with variance 1 / d_model and w_o
    [d_model, H 2d] with variance 1 / (H 2d) (outputs of order one), and attn
    [B, N, H, 2d] standard normal (an input of the output projection)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    hd2 = 2 * heads * head_dim
    bf = torch.bfloat16
    out = {"x": _normal(gen, (batch, seqlen, d_model), device).to(bf)}
    out["w_qkv"] = _normal(gen, (3 * hd2, d_model), device).mul_(d_model ** -0.5).to(bf)
    out["w_o"] = _normal(gen, (d_model, hd2), device).mul_(hd2 ** -0.5).to(bf)
    out["attn"] = _normal(gen, (batch, seqlen, heads, 2 * head_dim), device).to(bf)
    return out

"""Seeded synthetic inputs for the Hyena-SE / Hyena-MR forward workloads.

This module only draws random numbers and shapes them: it holds none of the
operator's arithmetic.  Both sides of every parity check (the HIP library and
the fp64 oracle) receive the exact tensors made here; neither side imports the
other.

Workloads (all with chunk length 64 and 16 channels per filter group):

=============  ==  =========  ====  ====  =====  =====  ===========================
name           B   L          D     l_h   dtype  seed   filter
=============  ==  =========  ====  ====  =====  =====  ===========================
tiny_se        1   1,024      256   7     f32    1000   N(0, 1/l_h)
se             1   8,192      4096  7     bf16   2000   N(0, 1/l_h)
mr             1   8,192      4096  128   bf16   3000   w*exp(-a*t), w~N(0,1/sqrt(l_h))
mr_b4          4   32,768     4096  128   bf16   4000   as mr
long_se        1   1,048,576  4096  7     bf16   5000   as se   (first layer of a stripe)
long_mr        1   1,048,576  4096  128   bf16   5100   as mr   (second layer of a stripe)
=============  ==  =========  ====  ====  =====  =====  ===========================

Draws: q, k, v ~ N(0, 1) i.i.d. in fp32, then rounded to the I/O dtype.  The
second argument of N(., .) is a variance: the short filter has standard
deviation l_h**-0.5, the medium filter's w has standard deviation l_h**-0.25,
and each group's decay a is U(0.01, 0.1).  Filters are drawn in fp32 on the CPU
and rounded to the I/O dtype; activations are drawn on ``device`` (a CUDA
generator for GPU tensors) in fixed pieces of ``PIECE`` elements so the values
do not depend on the free memory.  Seeds: base + 0 (q), + 1 (k), + 2 (v),
+ 3 (filter weights), + 4 (decays).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import torch

PIECE = 1 << 26  # elements drawn per randn call


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    D: int
    group_size: int
    l_h: int
    dtype: str  # "bf16" or "f32"
    seed: int
    filt: str  # "se" (Gaussian taps) or "mr" (decaying taps)

    @property
    def G(self) -> int:
        return self.D // self.group_size

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def elems(self) -> int:
        return self.B * self.L * self.D

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_se": Workload("tiny_se", 1, 1024, 256, 16, 7, "f32", 1000, "se"),
    "se": Workload("se", 1, 8192, 4096, 16, 7, "bf16", 2000, "se"),
    "mr": Workload("mr", 1, 8192, 4096, 16, 128, "bf16", 3000, "mr"),
    "mr_b4": Workload("mr_b4", 4, 32768, 4096, 16, 128, "bf16", 4000, "mr"),
    "long_se": Workload("long_se", 1, 1 << 20, 4096, 16, 7, "bf16", 5000, "se"),
    "long_mr": Workload("long_mr", 1, 1 << 20, 4096, 16, 128, "bf16", 5100, "mr"),
}


def _generator(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_activation(shape: Tuple[int, ...], dtype: torch.dtype, device, seed: int,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """N(0, 1) draws in fp32, rounded to ``dtype``, filled in pieces of PIECE."""
    device = torch.device(device)
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    g = _generator(device, seed)
    n = flat.numel()
    for s in range(0, n, PIECE):
        e = min(n, s + PIECE)
        flat[s:e].copy_(torch.randn(e - s, generator=g, device=device, dtype=torch.float32))
    return out


def filters(w: Workload) -> torch.Tensor:
    """[G, l_h] filter taps on the CPU, rounded to the workload dtype."""
    g = _generator(torch.device("cpu"), w.seed + 3)
    z = torch.randn(w.G, w.l_h, generator=g, dtype=torch.float32)
    if w.filt == "se":
        h = z * math.sqrt(1.0 / w.l_h)
    elif w.filt == "mr":
        ga = _generator(torch.device("cpu"), w.seed + 4)
        alpha = 0.01 + 0.09 * torch.rand(w.G, 1, generator=ga, dtype=torch.float32)
        t = torch.arange(w.l_h, dtype=torch.float32)[None, :]
        h = z * (1.0 / math.sqrt(w.l_h)) ** 0.5 * torch.exp(-alpha * t)
    else:
        raise ValueError(w.filt)
    return h.to(w.torch_dtype).contiguous()


def make_inputs(w: Workload, device="cpu"):
    """(q, k, v, h) for workload ``w``; q, k, v on ``device``, h on ``device``."""
    shape = (w.B, w.L, w.D)
    q = normal_activation(shape, w.torch_dtype, device, w.seed + 0)
    k = normal_activation(shape, w.torch_dtype, device, w.seed + 1)
    v = normal_activation(shape, w.torch_dtype, device, w.seed + 2)
    h = filters(w).to(device)
    return q, k, v, h


def integer_inputs(B: int, L: int, D: int, group_size: int, l_h: int,
                   dtype: torch.dtype, seed: int, device="cpu"):
    """Small-integer inputs: q, k, v in {-1, 0, 1}, taps in {-2, ..., 2}.

    Every partial sum of the operator is then an integer of magnitude at most
    2*l_h, exactly representable in bf16 and fp32.
    """
    g = _generator(torch.device("cpu"), seed)
    shape = (B, L, D)
    q = torch.randint(-1, 2, shape, generator=g).to(dtype)
    k = torch.randint(-1, 2, shape, generator=g).to(dtype)
    v = torch.randint(-1, 2, shape, generator=g).to(dtype)
    h = torch.randint(-2, 3, (D // group_size, l_h), generator=g).to(dtype)
    return q.to(device), k.to(device), v.to(device), h.to(device)


def gaussian_inputs(B: int, L: int, D: int, group_size: int, l_h: int,
                    dtype: torch.dtype, seed: int, device="cpu"):
    """N(0,1) activations and N(0, 1/l_h) taps at an arbitrary small shape."""
    g = _generator(torch.device("cpu"), seed)
    shape = (B, L, D)
    q = torch.randn(shape, generator=g).to(dtype)
    k = torch.randn(shape, generator=g).to(dtype)
    v = torch.randn(shape, generator=g).to(dtype)
    h = (torch.randn(D // group_size, l_h, generator=g) * math.sqrt(1.0 / l_h)).to(dtype)
    return q.to(device), k.to(device), v.to(device), h.to(device)

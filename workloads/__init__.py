"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

Shared by the tests, the smoke check and the benchmark.  This module holds
only shapes and random-number draws; none of the method's arithmetic lives
here.

Shapes follow the LLaMA layer shapes quoted on the zerotofrontier.app PEFT
page ("Choosing a method": Llama-2-7B, width 4096, MLP width 11008) and the
65B shapes (width 8192, MLP width 22016).  Trained weights are not available,
so Gaussian draws of the same shapes stand in for them:
  W  ~ N(0, 0.02^2) fp32 (optionally 1% of entries scaled by 10 as outliers)
  X, dY ~ N(0, 1) rounded to bf16
  A  ~ N(0, 1/K) (std 1/sqrt(in_dim)) rounded to bf16
  B  ~ N(0, 0.01^2) rounded to bf16
Weights are stored out x in (N x K, row-major).
"""
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np
import torch

# projection order inside a decoder layer: (name, out_dim, in_dim) as a function of (d, ffn)
PROJ_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def layer_projections(d: int, ffn: int) -> List[Tuple[str, int, int]]:
    """(name, N = out features, K = in features) for the 7 linears of one layer."""
    dims = {"q": (d, d), "k": (d, d), "v": (d, d), "o": (d, d),
            "gate": (ffn, d), "up": (ffn, d), "down": (d, ffn)}
    return [(p, dims[p][0], dims[p][1]) for p in PROJ_ORDER]


LLAMA7B = dict(d=4096, ffn=11008, layers=32)
LLAMA65B = dict(d=8192, ffn=22016, layers=80)


@dataclass(frozen=True)
class Workload:
    name: str
    description: str


WORKLOADS = {
    "tiny": Workload("tiny", "W 256x256 fp32 N(0,0.02), X 16x256, r=8, alpha=16, fwd+bwd"),
    "llama7b_layer": Workload("llama7b_layer",
                              "7 LLaMA-7B linears (4096/11008), M=2048 tokens, r=64, alpha=16, fwd+bwd"),
    "gemv65b": Workload("gemv65b", "LLaMA-65B shapes 8192x8192, 22016x8192, 8192x22016, "
                                   "M in {1,4,16}, r=64, forward only"),
    "bulk7b": Workload("bulk7b", "quantize + double-quantize + dequantize over 32 layers x 7 "
                                 "LLaMA-7B weights (6.48e9 params), 1% x10 outliers"),
    "llama65b_layer": Workload("llama65b_layer",
                               "7 LLaMA-65B linears (8192/22016), M=4096 tokens, r=64, alpha=16, "
                               "fwd chain then bwd chain"),
}


def seed_of(*parts: int) -> int:
    """Stable 63-bit seed from a tuple of small integers (numpy SeedSequence)."""
    ss = np.random.SeedSequence([int(p) for p in parts])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) >> 1


class Draw:
    """Sequential seeded draws from one torch generator on `device`."""

    def __init__(self, seed: int, device="cpu"):
        self.device = torch.device(device)
        self.g = torch.Generator(device=self.device)
        self.g.manual_seed(int(seed) & ((1 << 63) - 1))

    def normal(self, shape, std: float, outlier_frac: float = 0.0, outlier_scale: float = 10.0,
               dtype=torch.float32) -> torch.Tensor:
        t = torch.randn(shape, generator=self.g, device=self.device, dtype=torch.float32)
        t.mul_(std)
        if outlier_frac > 0.0:
            mask = torch.rand(shape, generator=self.g, device=self.device) < outlier_frac
            t = torch.where(mask, t * outlier_scale, t)
        return t.to(dtype)

    def bf16(self, shape, std: float) -> torch.Tensor:
        return self.normal(shape, std, dtype=torch.bfloat16)


def linear_inputs(N: int, K: int, M: int, r: int, seed: int, device="cpu",
                  w_outliers: float = 0.0, with_dy: bool = True):
    """W (fp32 N x K), X (bf16 M x K), A (bf16 r x K), B (bf16 N x r), dY (bf16 M x N),
    drawn in that order from one seeded generator."""
    d = Draw(seed, device)
    W = d.normal((N, K), 0.02, outlier_frac=w_outliers)
    X = d.bf16((M, K), 1.0)
    A = d.bf16((r, K), 1.0 / float(np.sqrt(K)))
    B = d.bf16((N, r), 0.01)
    dY = d.bf16((M, N), 1.0) if with_dy else None
    return W, X, A, B, dY


def tiny_inputs(device="cpu"):
    """The tiny layer: W 256x256, X 16x256, r=8, alpha=16, all from seed 0."""
    return linear_inputs(256, 256, 16, 8, seed=0, device=device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 host copy of a float32 or bf16 tensor."""
    return t.detach().cpu().to(torch.float32).contiguous().numpy()

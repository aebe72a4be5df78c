"""Seeded synthetic inputs for the QLoRA linear layer, shared by the tests and the benchmark.

This module only draws random numbers and rounds them to bf16 storage. It holds none of the
layer's arithmetic (no quantisation, no products), so the CPU oracle and the HIP path can both
take their inputs from here without sharing any of the computation they are compared on.

The five workloads are Llama-class projection shapes of a QLoRA fine-tune (a frozen NF4 base
weight, bf16 LoRA adapters A [r,K] and B [N,r], Hu et al.'s Delta W = B A at rank r as restated on
the Unsloth pages' "About the Unsloth Project" section):

  small   M=64    K=256    N=256    r=8   s=2   absmax fp32         fwd+bwd
  q_proj  M=4096  K=4096   N=4096   r=16  s=2   absmax int8/256     fwd
  mlp_up  M=8192  K=4096   N=11008  r=64  s=0.5 absmax int8/256     fwd+bwd
  decode  M=16    K=8192   N=28672  r=16  s=2   absmax int8/256     fwd (weight-stream bound)
  down    M=16384 K=14336  N=4096   r=32  s=1   absmax int8/256     fwd+bwd
  mlp_up_e2m1  the mlp_up shape with an E2M1 base (E4M3 scale per 16)  fwd+bwd
  decode_e2m1  the decode shape with an E2M1 base                      fwd

and one gate/up pair (two projections on the same X joined by SwiGLU, PAIRS below):

  mlp_swiglu  M=8192  K=4096  N=11008 (x2)  r=64 (x2)  s=0.5  absmax int8/256  fwd+bwd

and one grouped mixture-of-experts layer (MOES below):

  moe_mlp_up  E=8 experts of K=4096 N=11008, 8192 tokens x top-2 = 16384 rows, r=16, s=2,
              absmax int8/256, fwd+bwd

Distributions (std is the standard deviation of a normal): X ~ N(0,1); W ~ N(0,0.02) (0.015 for
decode); A ~ N(0, 1/K) read as variance 1/K, i.e. std K**-0.5; B ~ N(0,0.01); dY ~ N(0,1)
(N(0,1e-2) for down). Workloads that name no A/B distribution use the mlp_up one.

Every tensor is drawn as float32 standard normals from numpy's PCG64 generator with
seed = 1000*cfg + t (cfg 1..5 in the order above; t: X=1, W=2, A=3, B=4, dY=5), scaled by its
std in float32 and rounded to bf16 (round-to-nearest-even, by torch's conversion).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np
import torch

TENSOR_IDS = {"X": 1, "W": 2, "A": 3, "B": 4, "dY": 5}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1..5, used in the seeds
    M: int
    K: int
    N: int
    r: int
    s: float
    dq_block: int       # 0: fp32 absmax; 256: int8 absmax + fp32 scale per 256 absmax values
    std_x: float
    std_w: float
    std_b: float
    std_dy: float
    backward: bool
    fmt: str = "nf4"    # "nf4", or "e2m1": 4-bit floats, E4M3 scale per 16, float32 tensor scale

    @property
    def std_a(self) -> float:
        return self.K ** -0.5

    def std(self, tensor: str) -> float:
        return {"X": self.std_x, "W": self.std_w, "A": self.std_a, "B": self.std_b,
                "dY": self.std_dy}[tensor]

    def shape(self, tensor: str) -> Tuple[int, int]:
        return {"X": (self.M, self.K), "W": (self.N, self.K), "A": (self.r, self.K),
                "B": (self.N, self.r), "dY": (self.M, self.N)}[tensor]

    def seed(self, tensor: str) -> int:
        return 1000 * self.index + TENSOR_IDS[tensor]

    def fwd_flops(self) -> int:
        M, K, N, r = self.M, self.K, self.N, self.r
        return 2 * M * N * K + 2 * M * K * r + 2 * M * N * r

    def bwd_flops(self) -> int:
        M, K, N, r = self.M, self.K, self.N, self.r
        # U = dY B, dX = dY deq(W) + s U A, dB = s dY^T T, dA = s U^T X
        return 2 * M * N * r + (2 * M * N * K + 2 * M * r * K) + 2 * N * M * r + 2 * r * M * K

    def weight_stream_bytes(self) -> int:
        nblk = self.N * self.K // 64
        codes = self.N * self.K // 2
        if self.fmt == "e2m1":
            return codes + self.N * self.K // 16 + 4
        if self.dq_block:
            return codes + nblk + 4 * ((nblk + self.dq_block - 1) // self.dq_block)
        return codes + 4 * nblk


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("small", 1, 64, 256, 256, 8, 2.0, 0, 1.0, 0.02, 0.01, 1.0, True),
    Workload("q_proj", 2, 4096, 4096, 4096, 16, 2.0, 256, 1.0, 0.02, 0.01, 1.0, False),
    Workload("mlp_up", 3, 8192, 4096, 11008, 64, 0.5, 256, 1.0, 0.02, 0.01, 1.0, True),
    Workload("decode", 4, 16, 8192, 28672, 16, 2.0, 256, 1.0, 0.015, 0.01, 1.0, False),
    Workload("down", 5, 16384, 14336, 4096, 32, 1.0, 256, 1.0, 0.02, 0.01, 1e-2, True),
    # the mlp_up shape with the E2M1 base weight (the 4-bit float variant of the format)
    Workload("mlp_up_e2m1", 8, 8192, 4096, 11008, 64, 0.5, 0, 1.0, 0.02, 0.01, 1.0, True, "e2m1"),
    # and the decode shape with an E2M1 base
    Workload("decode_e2m1", 9, 16, 8192, 28672, 16, 2.0, 0, 1.0, 0.015, 0.01, 1.0, False, "e2m1"),
]}


@dataclasses.dataclass(frozen=True)
class PairWorkload:
    """A gate/up pair of QLoRA projections on the same X, joined by SwiGLU (H = silu(Yg) * Yu).

    Tensors: X [M,K]; Wgu [2N,K] (gate rows, then up rows: the stacked base weight); Agu [2r,K]
    (gate A, then up A); Bg, Bu [N,r]; dH [M,N]. Seeds 1000*index + t (X=1, Wgu=2, Agu=3, Bg=4,
    dH=5, Bu=6); distributions as the single-layer workloads.
    """
    name: str
    index: int
    M: int
    K: int
    N: int
    r: int
    s: float
    dq_block: int
    std_x: float
    std_w: float
    std_b: float
    std_dh: float

    def shape(self, tensor: str) -> Tuple[int, int]:
        M, K, N, r = self.M, self.K, self.N, self.r
        return {"X": (M, K), "Wgu": (2 * N, K), "Agu": (2 * r, K), "Bg": (N, r), "Bu": (N, r),
                "dH": (M, N)}[tensor]

    def std(self, tensor: str) -> float:
        return {"X": self.std_x, "Wgu": self.std_w, "Agu": self.K ** -0.5, "Bg": self.std_b,
                "Bu": self.std_b, "dH": self.std_dh}[tensor]

    def seed(self, tensor: str) -> int:
        return 1000 * self.index + {"X": 1, "Wgu": 2, "Agu": 3, "Bg": 4, "dH": 5, "Bu": 6}[tensor]

    def projection(self) -> Workload:
        """One of the two projections as a single-layer workload (for its flop counts)."""
        return Workload(self.name, self.index, self.M, self.K, self.N, self.r, self.s, self.dq_block,
                        self.std_x, self.std_w, self.std_b, self.std_dh, True)

    def fwd_flops(self) -> int:
        return 2 * self.projection().fwd_flops()

    def bwd_flops(self) -> int:
        return 2 * self.projection().bwd_flops()

    def weight_stream_bytes(self) -> int:
        return 2 * self.projection().weight_stream_bytes()


# The mlp_up shape as the Llama MLP's gate/up pair (the step straight after the single layer).
PAIRS: Dict[str, PairWorkload] = {p.name: p for p in [
    PairWorkload("mlp_swiglu", 6, 8192, 4096, 11008, 64, 0.5, 256, 1.0, 0.02, 0.01, 1.0),
]}


@dataclasses.dataclass(frozen=True)
class MoeWorkload:
    """A grouped (mixture-of-experts) QLoRA layer: E experts, each with its own NF4 base [N,K] and
    adapters, over `tokens` tokens routed to top_k experts each (M = tokens * top_k rows, grouped by
    expert).

    Routing: counts[e] = the rows of expert e, a multinomial draw of M over expert probabilities
    p_e = exp(z_e) / sum exp(z), z normal with standard deviation `skew`, both from
    PCG64(1000*index + 7) (a seeded, uneven load across experts, as a learned router produces).
    Tensors: X [M,K]; W [E*N,K] (the experts' weights stacked); A [E*r,K]; B [E*N,r]; dY [M,N];
    seeds 1000*index + t (X=1, W=2, A=3, B=4, dY=5); distributions as the single-layer workloads.
    """
    name: str
    index: int
    E: int
    tokens: int
    top_k: int
    K: int
    N: int
    r: int
    s: float
    dq_block: int
    skew: float
    std_x: float
    std_w: float
    std_b: float
    std_dy: float

    @property
    def M(self) -> int:
        return self.tokens * self.top_k

    def counts(self):
        rng = np.random.Generator(np.random.PCG64(1000 * self.index + 7))
        z = rng.standard_normal(self.E) * self.skew
        p = np.exp(z) / np.exp(z).sum()
        return [int(c) for c in rng.multinomial(self.M, p)]

    def shape(self, tensor: str) -> Tuple[int, int]:
        M, E, K, N, r = self.M, self.E, self.K, self.N, self.r
        return {"X": (M, K), "W": (E * N, K), "A": (E * r, K), "B": (E * N, r), "dY": (M, N)}[tensor]

    def std(self, tensor: str) -> float:
        return {"X": self.std_x, "W": self.std_w, "A": self.K ** -0.5, "B": self.std_b,
                "dY": self.std_dy}[tensor]

    def seed(self, tensor: str) -> int:
        return 1000 * self.index + TENSOR_IDS[tensor]

    def rows_workload(self) -> Workload:
        """The layer's flop counts over all M rows (every term is linear in the rows)."""
        return Workload(self.name, self.index, self.M, self.K, self.N, self.r, self.s, self.dq_block,
                        self.std_x, self.std_w, self.std_b, self.std_dy, True)

    def fwd_flops(self) -> int:
        return self.rows_workload().fwd_flops()

    def bwd_flops(self) -> int:
        return self.rows_workload().bwd_flops()

    def weight_stream_bytes(self) -> int:
        return self.E * Workload(self.name, self.index, 1, self.K, self.N, self.r, self.s, self.dq_block,
                                 self.std_x, self.std_w, self.std_b, self.std_dy, True).weight_stream_bytes()


# Eight experts of the mlp_up projection's shape, 8192 tokens routed to two experts each.
MOES: Dict[str, MoeWorkload] = {m.name: m for m in [
    MoeWorkload("moe_mlp_up", 7, 8, 8192, 2, 4096, 11008, 16, 2.0, 256, 0.5, 1.0, 0.02, 0.01, 1.0),
]}


def moe_tensor(w: MoeWorkload, name: str) -> torch.Tensor:
    """The named input of MoE workload w as a bf16 CPU tensor."""
    return normal_bf16(w.seed(name), w.shape(name), w.std(name))


def normal_bf16(seed: int, shape, std: float) -> torch.Tensor:
    """float32 standard normals from PCG64(seed), times std (float32), rounded to bf16 (CPU)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    a *= np.float32(std)
    return torch.from_numpy(a).to(torch.bfloat16)


def uniform_f32(seed: int, shape, lo: float, hi: float) -> torch.Tensor:
    """float32 uniforms on [lo, hi) from PCG64(seed) (CPU)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy(rng.uniform(lo, hi, size=tuple(shape)).astype(np.float32))


def pair_tensor(p: PairWorkload, name: str, rows: int | None = None) -> torch.Tensor:
    """The named input of pair workload p as a bf16 CPU tensor (rows: X and dH only)."""
    t = normal_bf16(p.seed(name), p.shape(name), p.std(name))
    if rows is not None:
        t = t[:rows].contiguous()
    return t


def tensor(w: Workload, name: str, rows: int | None = None) -> torch.Tensor:
    """The named input of workload w as a bf16 CPU tensor.

    rows (X and dY only) keeps just the first `rows` rows of the same draw, which is how the
    bounded CPU samples of the large workloads are taken.
    """
    t = normal_bf16(w.seed(name), w.shape(name), w.std(name))
    if rows is not None:
        t = t[:rows].contiguous()
    return t

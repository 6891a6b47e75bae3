"""Seeded synthetic inputs for the fused NF4-LoRA linear.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds none of the method's arithmetic: only the workload shapes,
seeded random draws and the rounding of those draws to bf16 storage.

Workloads (token count T, projections d_in -> d_out, LoRA rank r, alpha):

  0 "tiny"       T=64,   256->256, r=8,  alpha=16
  1 "llama3-8b-q" T=8192 (batch 4 x seq 2048), q_proj 4096->4096, r=16, alpha=16
  2 "llama3-8b-attn" T=8192, q,o 4096->4096 and k,v 4096->1024, r=64, alpha=16
  3 "qwen14b-attn" T=8192 (batch 1 x seq 8192), q,k,v,o 5120->5120, r=16, alpha=16
  4 "llama3-70b-layer" T=4096 (batch 2 x seq 2048), q,o 8192->8192, k,v 8192->1024,
                       gate,up 8192->28672, down 28672->8192, r=16, alpha=16

The projection shapes are the Llama-3 / Qwen attention and MLP projections that
the pages' LoRA target modules (q/k/v/o/gate/up/down) name. Distributions:
x ~ N(0,1); base weight W ~ N(0, 0.02) (second parameter = standard deviation),
drawn as the nn.Linear-oriented [d_out, d_in] matrix and rounded to bf16 before
NF4 quantization; A ~ U(-1/sqrt(d_in), 1/sqrt(d_in)) (Kaiming-uniform with
a = sqrt(5)); B ~ N(0, 0.01); dY ~ N(0, 1) for the tiny workload and N(0, 0.01)
for all others.

Seeds: numpy PCG64 seeded from SeedSequence([workload, projection, tensor]) with
tensor 0 = x, 1 = W, 2 = A, 3 = B, 4 = dY. Draws are float32, then rounded to
nearest-even bf16.
"""
from __future__ import annotations

import dataclasses
import numpy as np

TENSOR_X, TENSOR_W, TENSOR_A, TENSOR_B, TENSOR_DY = range(5)


@dataclasses.dataclass(frozen=True)
class Projection:
    name: str
    d_in: int
    d_out: int


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    tokens: int
    r: int
    alpha: float
    projections: tuple
    dy_std: float
    batch: int
    seq: int

    @property
    def scale(self) -> float:
        return self.alpha / self.r


def _p(name, k, n):
    return Projection(name, k, n)


WORKLOADS = (
    Workload(0, "tiny", 64, 8, 16.0, (_p("proj", 256, 256),), 1.0, 1, 64),
    Workload(1, "llama3-8b-q_proj", 8192, 16, 16.0, (_p("q_proj", 4096, 4096),), 1e-2, 4, 2048),
    Workload(2, "llama3-8b-attn-r64", 8192, 64, 16.0,
             (_p("q_proj", 4096, 4096), _p("k_proj", 4096, 1024),
              _p("v_proj", 4096, 1024), _p("o_proj", 4096, 4096)), 1e-2, 4, 2048),
    Workload(3, "qwen14b-attn", 8192, 16, 16.0,
             (_p("q_proj", 5120, 5120), _p("k_proj", 5120, 5120),
              _p("v_proj", 5120, 5120), _p("o_proj", 5120, 5120)), 1e-2, 1, 8192),
    Workload(4, "llama3-70b-layer", 4096, 16, 16.0,
             (_p("q_proj", 8192, 8192), _p("k_proj", 8192, 1024), _p("v_proj", 8192, 1024),
              _p("o_proj", 8192, 8192), _p("gate_proj", 8192, 28672),
              _p("up_proj", 8192, 28672), _p("down_proj", 28672, 8192)), 1e-2, 2, 2048),
)


def rng(workload: int, projection: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, projection, tensor])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, std: float) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def uniform_bf16(g: np.random.Generator, shape, bound: float) -> np.ndarray:
    x = g.random(size=shape, dtype=np.float32)
    x = (x * np.float32(2.0) - np.float32(1.0)) * np.float32(bound)
    return f32_to_bf16_bits(x)


def projection_inputs(w: Workload, proj_index: int, tokens: int | None = None,
                      tensors=("x", "W", "A", "B", "dY")) -> dict:
    """bf16 bit patterns (uint16 arrays) for one projection of a workload.

    ``tokens`` overrides T (used by the parity tests to run smaller token
    counts of a real projection shape); the draws for a smaller T are the
    leading rows of the full draw only when T is unchanged, so callers should
    not rely on prefix consistency.
    """
    p = w.projections[proj_index]
    T = w.tokens if tokens is None else tokens
    K, N, r = p.d_in, p.d_out, w.r
    out = {}
    if "x" in tensors:
        out["x"] = normal_bf16(rng(w.index, proj_index, TENSOR_X), (T, K), 1.0)
    if "W" in tensors:
        out["W"] = normal_bf16(rng(w.index, proj_index, TENSOR_W), (N, K), 0.02)
    if "A" in tensors:
        out["A"] = uniform_bf16(rng(w.index, proj_index, TENSOR_A), (K, r), 1.0 / np.sqrt(K))
    if "B" in tensors:
        out["B"] = normal_bf16(rng(w.index, proj_index, TENSOR_B), (r, N), 0.01)
    if "dY" in tensors:
        out["dY"] = normal_bf16(rng(w.index, proj_index, TENSOR_DY), (T, N), w.dy_std)
    return out


def custom_inputs(seed: int, T: int, K: int, N: int, r: int, x_std=1.0, w_std=0.02,
                  b_std=0.01, dy_std=1.0) -> dict:
    """Same recipe as the workloads, for arbitrary (edge-case) shapes."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000, seed, T, K, N, r])))
    return {
        "x": normal_bf16(g, (T, K), x_std),
        "W": normal_bf16(g, (N, K), w_std),
        "A": uniform_bf16(g, (K, r), 1.0 / np.sqrt(K)),
        "B": normal_bf16(g, (r, N), b_std),
        "dY": normal_bf16(g, (T, N), dy_std),
    }


def flops(T: int, K: int, N: int, r: int) -> int:
    """Algorithmic FLOPs of one fused LoRA linear forward + backward (no dW: base frozen)."""
    return 4 * T * K * N + 6 * T * r * (K + N)


def optimizer_inputs(seed: int, n: int, step_scale: float = 1e-3) -> dict:
    """Seeded state of one LoRA factor for an optimizer step: float32 master
    weights ~ U(-1/64, 1/64), bf16 gradient ~ N(0, step_scale) with a spread of
    magnitudes (some near the eps scale), float32 first moment ~ N(0, step_scale / 3)
    and float32 second moment ~ |N(0, step_scale^2)|."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2000, seed, n])))
    p = ((g.random(n, dtype=np.float32) * np.float32(2) - np.float32(1)) * np.float32(1 / 64)).astype(np.float32)
    mag = (np.float32(10.0) ** g.uniform(-6, 0, n).astype(np.float32)).astype(np.float32)
    grad = f32_to_bf16_bits(g.standard_normal(n, dtype=np.float32) * np.float32(step_scale) * mag)
    m32 = (g.standard_normal(n, dtype=np.float32) * np.float32(step_scale / 3)).astype(np.float32)
    v32 = (np.abs(g.standard_normal(n, dtype=np.float32)) * np.float32(step_scale ** 2)).astype(np.float32)
    return {"p": p, "grad": grad, "m": m32, "v": v32}

"""LoRA linear over an NF4 frozen base, forward and backward, in float64 — oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

Definitions followed:

* LoRA factors A in R^{d_in x r} and B in R^{r x d_out} ("Unsloth acceleration
  principles: CUDA kernel fusion and memory optimization", section on the
  compact layout of LoRA tensors); scale s = lora_alpha / r with lora_alpha and
  r the user arguments of get_peft_model (same page, kernel-fusion section;
  "Unlocking AI potential: Unsloth's algorithms and implementation", section on
  optimized LoRA fine-tuning). No dropout and no bias (lora_dropout = 0,
  bias = "none" on both pages).
* The fused chain of the kernel-fusion section (base linear, LoRA_A, LoRA_B,
  add). Its "ReLU" between LoRA_A and LoRA_B is not part of LoRA and is dropped.
* The base weight is frozen: only A and B are trained, so the backward gives the
  input gradient dX and the LoRA gradients dA, dB, and no base-weight gradient.

Layout: the base weight is the nn.Linear-oriented matrix Wt = W^T of shape
[d_out, d_in], stored as NF4; D = deq(Wt) in exact float64. With T tokens:

    U  = x A                      [T, r]
    y  = x D^T + s U B            [T, d_out]
    G  = s dY B^T                 [T, r]
    dX = dY D + G A^T             [T, d_in]
    dA = x^T G                    [d_in, r]
    dB = s U^T dY                 [r, d_out]

After training, the adapters are merged into the base weight and saved at 16 bits
(the "Unsloth in three lines of code" page, section 4; "Reading the Unsloth
changelog", command-line part of section 2, where saving turns the 4-bit model
into a 16-bit one). In the same orientation:

    W' = D + s (A B)^T            [d_out, d_in],   so that x W'^T = y
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def forward(x, D, A, B, alpha: float, r: int):
    """y = x D^T + (alpha/r) (x A) B; returns (y, U) in float64."""
    x, D, A, B = (np.asarray(v, dtype=np.float64) for v in (x, D, A, B))
    s = float(alpha) / float(r)
    U = x @ A
    y = x @ D.T + s * (U @ B)
    return y, U


def backward(x, dY, D, A, B, alpha: float, r: int):
    """Gradients of <dY, y> for the forward above; returns (dX, dA, dB) in float64."""
    x, dY, D, A, B = (np.asarray(v, dtype=np.float64) for v in (x, dY, D, A, B))
    s = float(alpha) / float(r)
    U = x @ A
    G = s * (dY @ B.T)
    dX = dY @ D + G @ A.T
    dA = x.T @ G
    dB = s * (U.T @ dY)
    return dX, dA, dB


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (0 when both are identically zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def lora_factor_grads(x, dY, A, B, alpha: float, r: int):
    """dA = x^T (s dY B^T) and dB = s (x A)^T dY alone (they do not involve the base weight)."""
    x, dY, A, B = (np.asarray(v, dtype=np.float64) for v in (x, dY, A, B))
    s = float(alpha) / float(r)
    G = s * (dY @ B.T)
    return x.T @ G, s * ((x @ A).T @ dY)


def merge(D, A, B, alpha: float, r: int):
    """Merged base weight W' = D + (alpha/r) (A B)^T, [d_out, d_in], in float64."""
    D, A, B = (np.asarray(v, dtype=np.float64) for v in (D, A, B))
    s = float(alpha) / float(r)
    return D + s * (A @ B).T

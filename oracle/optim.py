"""Training-step pieces around the LoRA linear: the optimizer update of the LoRA
factors and the rank-stabilized scale — oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

What the pages fix:

* The optimizer step is one of the timed phases of a training step and runs as
  a GPU kernel with reduced-precision state and no host round trip ("Unsloth
  performance measured: is it really 2x faster?", section 2.2, the
  optimizer.step row of the time table; section 3, the 16-bit storage of the
  gradient states). The changelog's training setup names an 8-bit AdamW
  ("Reading the Unsloth changelog", section 1, memory list).
* The rank-stabilized option --use_rslora ("Reading the Unsloth changelog",
  section 2.1). The page's own formula for the scale is garbled (it says the
  scale is alpha / r "normalized"); the reading taken is the rank-stabilized
  LoRA scale alpha / sqrt(r) (Kalajdzievski, 2023).

Readings for the optimizer (the pages name it but do not define it):

* AdamW with decoupled weight decay (Loshchilov and Hutter, 2019): with the
  gradient g of a LoRA factor, step number t >= 1 and hyper-parameters
  lr, beta1, beta2, eps, wd,
      m' = beta1 m + (1 - beta1) g
      v' = beta2 v + (1 - beta2) g^2
      p' = p (1 - lr wd) - lr (m' / (1 - beta1^t)) / (sqrt(v' / (1 - beta2^t)) + eps)
* The moments m and v are stored as bf16 between steps (16-bit state: the
  bf16 exponent range holds g^2 where float16 would underflow); the parameter
  has a float32 master copy and the bf16 copy the GEMM kernels read.
"""
from __future__ import annotations

import math

import numpy as np


def adamw_step(p, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float):
    """One AdamW update in float64; returns (p', m', v') before any storage rounding.

    p, g, m, v are float64 arrays of one shape (the stored values widened
    exactly); the formulas are those of the module docstring.
    """
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m1 = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v1 = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m1 / (1.0 - beta1 ** step)
    v_hat = v1 / (1.0 - beta2 ** step)
    p1 = p * (1.0 - lr * weight_decay) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p1, m1, v1


def rslora_scale(lora_alpha: float, r: int) -> float:
    """Rank-stabilized LoRA scale alpha / sqrt(r), in float64."""
    if r < 1:
        raise ValueError("r >= 1")
    return lora_alpha / math.sqrt(r)

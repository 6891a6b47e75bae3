"""Training-step pieces around the LoRA linear: the optimizer update of the LoRA
factors and the rank-stabilized scale — oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

What the pages fix:

* The optimizer step is one of the timed phases of a training step and runs as
  a GPU kernel with no host round trip ("Unsloth performance measured: is it
  really 2x faster?", section 2.2, the optimizer.step row of the time table,
  which names a low-bit AdamW kernel). The changelog's training setup names an
  8-bit AdamW that cuts the optimizer-state memory to a quarter ("Reading the
  Unsloth changelog", section 1, memory list).
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
* Default state: m and v stored as float32 (the published algorithm's state;
  a 16-bit v cannot decay at beta2 = 0.999, whose per-step change is below half
  a bf16 step); the parameter has a float32 master copy and the bf16 copy the
  GEMM kernels read.
* Float32 evaluation (adamw_step_f32): the kernels evaluate the update above
  as the sequence of float32 operations written in that function, each rounded
  to nearest-even, with the step constants formed in float64 on the host and
  rounded once to float32. That sequence is the definition the GPU path is
  checked against bit for bit; adamw_step (float64) is the mathematics it
  approximates.
* 8-bit state (adamw8_step; the changelog's 8-bit AdamW, states at a quarter of
  float32): each moment is stored blockwise, 256 consecutive elements per block
  (block-wise quantization of optimizer state, Dettmers et al. 2022, "8-bit
  Optimizers via Block-wise Quantization"), as one E4M3 code per element (the
  OCP FP8 E4M3FN format, nearest code, ties to even, saturating at 448) and one
  float32 scale per block: scale = f32(max |x| over the block / 448), code =
  e4m3(f32(x / scale)) (code 0 when scale = 0), value = f32(e4m3(code) * scale).
  A step decodes both moments, runs the float32 update, and re-encodes them with
  the new block maxima; the parameter copies are as above.
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


def step_constants(step: int, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float):
    """The float32 constants of one step, formed in float64 and rounded once:
    (beta1, 1 - beta1, beta2, 1 - beta2, eps, 1 - lr wd, lr / (1 - beta1^t),
    1 / sqrt(1 - beta2^t)). The hyper-parameters are the float32 values passed."""
    if step < 1:
        raise ValueError("step counts from 1")
    f = np.float32
    b1, b2, lr64, wd64 = float(f(beta1)), float(f(beta2)), float(f(lr)), float(f(weight_decay))
    bc1 = 1.0 - math.pow(b1, step)
    bc2 = 1.0 - math.pow(b2, step)
    return (f(b1), f(1.0 - b1), f(b2), f(1.0 - b2), f(eps), f(1.0 - lr64 * wd64), f(lr64 / bc1),
            f(1.0 / math.sqrt(bc2)))


def adamw_step_f32(p, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
                   weight_decay: float):
    """One AdamW update as the float32 operation sequence the kernels run (module
    docstring), each operation rounded to nearest-even:
        m' = b1 m + (1 - b1) g                       (two products, one sum)
        v' = b2 v + (1 - b2) (g g)
        d  = sqrt(v') * (1 / sqrt(1 - b2^t)) + eps
        p' = p (1 - lr wd) - (lr / (1 - b1^t)) (m' / d)
    p, m, v float32 arrays, g float32 (the widened bf16 gradient, or an exact float32
    sum); returns float32 (p', m', v')."""
    f = np.float32
    b1, omb1, b2, omb2, e, decay, step_size, isb2 = step_constants(step, lr, beta1, beta2, eps, weight_decay)
    p, g, m, v = (np.asarray(a, dtype=f) for a in (p, g, m, v))
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        m1 = (b1 * m).astype(f) + (omb1 * g).astype(f)
        v1 = (b2 * v).astype(f) + (omb2 * (g * g).astype(f)).astype(f)
        d = (np.sqrt(v1).astype(f) * isb2).astype(f) + e
        p1 = (p * decay).astype(f) - (step_size * (m1 / d).astype(f)).astype(f)
    return p1.astype(f), m1.astype(f), v1.astype(f)


STATE_BLOCK = 256
E4M3_MAX = 448.0


def _e4m3_encode(x):
    from oracle.dq import e4m3_encode
    return e4m3_encode(x)


def _e4m3_values():
    from oracle.dq import e4m3_values
    return e4m3_values()


def encode_state(x):
    """float32 [n] moment -> (E4M3 codes uint8 [n], float32 scales [ceil(n / 256)]),
    per the module docstring's 8-bit state."""
    f = np.float32
    x = np.ascontiguousarray(x, dtype=f).ravel()
    n = x.size
    nb = (n + STATE_BLOCK - 1) // STATE_BLOCK
    codes = np.zeros(n, dtype=np.uint8)
    scales = np.zeros(nb, dtype=f)
    for b in range(nb):
        blk = x[b * STATE_BLOCK:(b + 1) * STATE_BLOCK]
        sc = f(f(np.max(np.abs(blk))) / f(E4M3_MAX))
        scales[b] = sc
        if sc > 0:
            codes[b * STATE_BLOCK:b * STATE_BLOCK + blk.size] = _e4m3_encode((blk / sc).astype(f))
    return codes, scales


def decode_state(codes, scales):
    """(codes [n], scales [ceil(n / 256)]) -> float32 [n]: f32(e4m3(code) * scale)."""
    f = np.float32
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    vals = _e4m3_values()[codes].astype(f)
    sc = np.repeat(np.asarray(scales, dtype=f), STATE_BLOCK)[:codes.size]
    return (vals * sc).astype(f)


def adamw8_step(p, g, m_codes, m_scales, v_codes, v_scales, step: int, lr: float, beta1: float,
                beta2: float, eps: float, weight_decay: float):
    """One AdamW update with 8-bit blockwise moments: decode, adamw_step_f32,
    re-encode. Returns (p', (m codes, m scales), (v codes, v scales)) and the
    float32 moments before re-encoding."""
    m = decode_state(m_codes, m_scales)
    v = decode_state(v_codes, v_scales)
    p1, m1, v1 = adamw_step_f32(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay)
    return p1, encode_state(m1), encode_state(v1), (m1, v1)


def rslora_scale(lora_alpha: float, r: int) -> float:
    """Rank-stabilized LoRA scale alpha / sqrt(r), in float64."""
    if r < 1:
        raise ValueError("r >= 1")
    return lora_alpha / math.sqrt(r)

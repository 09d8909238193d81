"""AdamW step on the LoRA parameters: the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * P1 §七 (table of storage and compute precisions): only the LoRA
    parameters are trained, kept in BF16/FP16; optimizer state exists only
    for them, in FP32 (or 8-bit).
  * P4 §三 (English derivation, item 3, paged optimizers): the optimizer is a
    32-bit AdamW whose states belong to the LoRA parameters.
  * P4 §四 ④: the LoRA parameters A and B are kept in 16-bit BF16.

The pages name AdamW but not its update.  Reading (stated in full because the
GPU path must reproduce it bit for bit): AdamW with decoupled weight decay,
first and second moments in fp32, bias-corrected, with the decay applied to
the parameter before the moment update, every operation one IEEE binary32
rounding, no fused multiply-add, in this order:

  host scalars   decay = fl(1 - fl(lr * wd));  omb1 = fl(1 - b1);  omb2 = fl(1 - b2)
                 bc1 = fl32(1 - b1^t), bc2 = fl32(1 - b2^t)   (powers in fp64)
                 sbc2 = fl(sqrt(bc2));  step_size = fl(lr / bc1)
  per element    p = fl(p * decay)
                 m = fl(fl(b1 * m) + fl(omb1 * g))
                 v = fl(fl(b2 * v) + fl(fl(omb2 * g) * g))
                 d = fl(fl(sqrt(v) / sbc2) + eps)
                 p = fl(p - fl(step_size * fl(m / d)))

The parameter is stored as bf16 (widened exactly to fp32 before the step,
rounded to nearest-even after it) or as fp32.

The pins (tests/test_oracle_adamw.py) hold this against the textbook update
evaluated in fp64, against closed forms (the first step, a zero gradient,
beta1 = beta2 = 0) and against a slow scalar loop that follows the steps
above one element at a time.
"""

import math

import numpy as np

from . import nf4

F32 = np.float32


def scalars(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float, step: int) -> dict:
    """The per-step fp32 constants (host side of the reading above)."""
    lr32, b1, b2, wd = F32(lr), F32(beta1), F32(beta2), F32(weight_decay)
    bc1 = F32(1.0 - float(b1) ** step)
    bc2 = F32(1.0 - float(b2) ** step)
    return {
        "b1": b1,
        "b2": b2,
        "eps": F32(eps),
        "decay": F32(F32(1.0) - F32(lr32 * wd)),
        "omb1": F32(F32(1.0) - b1),
        "omb2": F32(F32(1.0) - b2),
        "sbc2": F32(np.sqrt(bc2)),
        "step_size": F32(lr32 / bc1),
    }


def step(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay, step_no,
         param_bf16: bool):
    """One AdamW step.  param: uint16 bf16 bits (param_bf16) or float32;
    grad, exp_avg, exp_avg_sq: float32.  Returns (param, exp_avg, exp_avg_sq)
    as new arrays of the same dtypes."""
    c = scalars(lr, beta1, beta2, eps, weight_decay, step_no)
    g = np.asarray(grad, dtype=F32)
    m = np.asarray(exp_avg, dtype=F32)
    v = np.asarray(exp_avg_sq, dtype=F32)
    p = nf4.bf16_to_f32(np.asarray(param)) if param_bf16 else np.asarray(param, dtype=F32)
    p = (p * c["decay"]).astype(F32)
    m = ((c["b1"] * m).astype(F32) + (c["omb1"] * g).astype(F32)).astype(F32)
    v = ((c["b2"] * v).astype(F32) + ((c["omb2"] * g).astype(F32) * g).astype(F32)).astype(F32)
    d = ((np.sqrt(v).astype(F32) / c["sbc2"]).astype(F32) + c["eps"]).astype(F32)
    p = (p - (c["step_size"] * (m / d).astype(F32)).astype(F32)).astype(F32)
    return (nf4.bf16_bits(p) if param_bf16 else p), m, v


def step_scalar_loop(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay, step_no,
                     param_bf16: bool):
    """The same step, one element at a time with numpy float32 scalars (small
    inputs only): a check on the vectorised form's operation order."""
    c = scalars(lr, beta1, beta2, eps, weight_decay, step_no)
    n = len(grad)
    po = np.empty(n, dtype=np.uint16 if param_bf16 else F32)
    mo = np.empty(n, dtype=F32)
    vo = np.empty(n, dtype=F32)
    for i in range(n):
        if param_bf16:
            p = np.array([param[i]], dtype=np.uint16).astype(np.uint32) << np.uint32(16)
            p = p.view(F32)[0]
        else:
            p = F32(param[i])
        g, m, v = F32(grad[i]), F32(exp_avg[i]), F32(exp_avg_sq[i])
        p = F32(p * c["decay"])
        m = F32(F32(c["b1"] * m) + F32(c["omb1"] * g))
        v = F32(F32(c["b2"] * v) + F32(F32(c["omb2"] * g) * g))
        d = F32(F32(F32(np.sqrt(v)) / c["sbc2"]) + c["eps"])
        p = F32(p - F32(c["step_size"] * F32(m / d)))
        po[i] = nf4.bf16_bits(np.array([p], dtype=F32))[0] if param_bf16 else p
        mo[i], vo[i] = m, v
    return po, mo, vo


def textbook_f64(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step_no):
    """AdamW (decoupled weight decay, bias-corrected moments) in fp64 with the
    textbook arithmetic, no intermediate rounding.  Scalars in, scalars out."""
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step_no)
    v_hat = v / (1.0 - beta2 ** step_no)
    p = p - lr * m_hat / (math.sqrt(v_hat) + eps)
    return p, m, v

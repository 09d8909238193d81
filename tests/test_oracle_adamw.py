"""Pins of the oracle's AdamW step (oracle/adamw.py) on the CPU: the textbook
update in fp64, closed forms, and a scalar loop over the same steps."""

import numpy as np
import pytest

from oracle import adamw, nf4

F32 = np.float32
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def rnd(seed, n, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(F32)


@pytest.mark.parametrize("param_bf16", [False, True])
def test_vectorised_equals_scalar_loop(param_bf16):
    n = 257
    p = rnd(1, n, 0.02)
    p = nf4.bf16_bits(p) if param_bf16 else p
    g, m, v = rnd(2, n, 0.1), rnd(3, n, 0.01), np.abs(rnd(4, n, 1e-3))
    for t in (1, 2, 7):
        a = adamw.step(p, g, m, v, step_no=t, param_bf16=param_bf16, **HP)
        b = adamw.step_scalar_loop(p, g, m, v, step_no=t, param_bf16=param_bf16, **HP)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32 if x.dtype == F32 else np.uint16),
                                  y.view(np.uint32 if y.dtype == F32 else np.uint16))


def test_ten_steps_track_the_fp64_textbook_update():
    # fp32 parameter and state, ten steps with fresh gradients: the result
    # stays within fp32 rounding of AdamW evaluated in fp64
    n = 64
    p32 = rnd(10, n, 0.05)
    m32 = np.zeros(n, F32)
    v32 = np.zeros(n, F32)
    p64, m64, v64 = p32.astype(np.float64), np.zeros(n), np.zeros(n)
    hp64 = {k: float(F32(x)) for k, x in HP.items()}  # the same (fp32) hyperparameters
    for t in range(1, 11):
        g = rnd(100 + t, n, 0.3)
        p32, m32, v32 = adamw.step(p32, g, m32, v32, step_no=t, param_bf16=False, **HP)
        for i in range(n):
            p64[i], m64[i], v64[i] = adamw.textbook_f64(p64[i], float(g[i]), m64[i], v64[i],
                                                        step_no=t, **hp64)
    assert np.max(np.abs(m32 - m64)) < 1e-7
    assert np.max(np.abs(v32 - v64) / v64) < 1e-6
    # each step moves p by about lr; fp32 keeps ~7 digits of p (|p| ~ 0.05)
    assert np.max(np.abs(p32 - p64)) < 1e-7


def test_first_step_is_lr_times_the_gradient_sign():
    # t = 1, no decay: m_hat = g and v_hat = g^2 exactly in real arithmetic,
    # so the update is lr * g / (|g| + eps), i.e. lr * sign(g) for |g| >> eps
    n = 128
    p = rnd(20, n, 0.05)
    g = rnd(21, n, 0.5)
    g[np.abs(g) < 1e-3] = F32(1e-3)
    hp = dict(HP, weight_decay=0.0)
    q, m, v = adamw.step(p, g, np.zeros(n, F32), np.zeros(n, F32), step_no=1, param_bf16=False, **hp)
    exact = p.astype(np.float64) - hp["lr"] * g / (np.abs(g.astype(np.float64)) + hp["eps"])
    assert np.max(np.abs(q - exact)) < 4 * np.spacing(F32(0.2))
    assert np.all(np.sign(p - q) == np.sign(g))
    assert np.array_equal(m, (F32(1 - F32(0.9)) * g).astype(F32))


def test_zero_gradient_and_state_is_weight_decay_only():
    n = 100
    p = rnd(30, n, 1.0)
    z = np.zeros(n, F32)
    q, m, v = adamw.step(p, z, z, z, step_no=3, param_bf16=False, **HP)
    decay = F32(F32(1.0) - F32(F32(HP["lr"]) * F32(HP["weight_decay"])))
    assert np.array_equal(q, (p * decay).astype(F32))
    assert not m.any() and not v.any()


def test_zero_betas_reduce_to_normalised_gradient_descent():
    # beta1 = beta2 = 0: m = g, v = g^2, no bias correction, and the step is
    # p*decay - lr * g / (|g| + eps) (sqrt(fl(g*g)) == |g| for these g)
    n = 200
    p = rnd(40, n, 0.1)
    g = rnd(41, n, 0.2)
    hp = dict(lr=0.01, beta1=0.0, beta2=0.0, eps=1e-6, weight_decay=0.1)
    q, m, v = adamw.step(p, g, rnd(42, n), np.abs(rnd(43, n)), step_no=5, param_bf16=False, **hp)
    assert np.array_equal(m, g)
    assert np.array_equal(v, (g * g).astype(F32))
    assert np.array_equal(np.sqrt(v).astype(F32), np.abs(g))
    decay = F32(F32(1.0) - F32(F32(0.01) * F32(0.1)))
    den = (np.abs(g) + F32(1e-6)).astype(F32)
    expect = ((p * decay).astype(F32) - (F32(0.01) * (g / den).astype(F32)).astype(F32)).astype(F32)
    assert np.array_equal(q, expect)


def test_bf16_parameter_keeps_its_value_under_tiny_updates():
    # an update far below half a bf16 ulp of the parameter rounds away
    n = 32
    p = nf4.bf16_bits(np.full(n, 1.0, F32))
    g = rnd(50, n, 1.0)
    hp = dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    q, _, _ = adamw.step(p, g, np.zeros(n, F32), np.zeros(n, F32), step_no=1, param_bf16=True, **hp)
    assert np.array_equal(q, p)
    # and a large one moves it to the nearest bf16 of the fp32 result
    hp["lr"] = 0.25
    q, _, _ = adamw.step(p, g, np.zeros(n, F32), np.zeros(n, F32), step_no=1, param_bf16=True, **hp)
    assert np.all(np.abs(nf4.bf16_to_f32(q) - (1.0 - 0.25 * np.sign(g))) <= 2 ** -8)


def test_bias_correction_constants():
    c = adamw.scalars(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
    # t = 1: 1 - b^1 is fl32(1 - b) up to the fp64 evaluation
    assert c["step_size"] == F32(F32(1e-3) / F32(1.0 - float(F32(0.9))))
    c = adamw.scalars(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=10 ** 6)
    # large t: the corrections vanish (1 - b^t rounds to 1)
    assert c["step_size"] == F32(1e-3) and c["sbc2"] == F32(1.0)

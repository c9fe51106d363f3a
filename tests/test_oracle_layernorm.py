"""Pins of the oracle's LayerNorm + adaLN modulation prologue (reading R11).

Independent routes: hand-worked fixtures (tests/golden), exact rational
arithmetic (tests/exact.py), closed forms, invariances, torch's float64
LayerNorm, and planted mistakes that these checks must reject.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

import oracle as O
import workloads as W
from tests import exact as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bits_of(values) -> np.ndarray:
    return np.array([E.bf16_bits(Fraction(v)) for v in values], dtype=np.uint16)


def opt_bits(field: str):
    return None if field == "-" else bits_of([Fraction(t) for t in field.split()])


def exact_stats(x_row_bits, eps: float):
    """(fl32(mean), fl32(1/sqrt(var + eps))) from exact rationals."""
    xs = [E.bf16_value(b) for b in x_row_bits]
    k = len(xs)
    mu = sum(xs) / k
    var = sum((x - mu) ** 2 for x in xs) / k
    e = Fraction(float(np.float32(eps)))
    return E.f32(mu), E.inv_sqrt_f32(var + e)


def stats_rows():
    x = W.random_bits((6, 200), seed=61)                     # K not a power of two
    x[1] = W.random_bits((200,), seed=62, std=1.0, mean=50.0)  # mean dominates
    x[2] = W.random_bits((200,), seed=63, std=1e-3)          # eps comparable to var
    x[3] = E.bf16_bits(Fraction(3))                          # constant row: var = 0
    return x


# ---- checks (take the oracle step so planted mistakes can be run through them)

def check_golden(ln_quant_fn) -> bool:
    with open(os.path.join(GOLD, "layernorm_worked_examples.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    for line in lines:
        eps_s, xs, gs, bs, ss, hs, mus, rs, qs = [t.strip() for t in line.split("|")]
        x = bits_of([Fraction(t) for t in xs.split()])[None, :]
        q, s, mu, r = ln_quant_fn(x, float(Fraction(eps_s)), opt_bits(gs), opt_bits(bs),
                                  opt_bits(ss), opt_bits(hs))
        if mus != "-" and Fraction(float(mu[0])) != Fraction(mus.split()[0]):
            return False
        if rs != "-" and Fraction(float(r[0])) != Fraction(rs):
            return False
        if list(q[0]) != [int(t) for t in qs.split()]:
            return False
    return True


def check_stats_exact(stats_fn) -> bool:
    x = stats_rows()
    for eps in (1e-6, 0.25):
        mu, r = stats_fn(x, eps)
        for i in range(x.shape[0]):
            emu, er = exact_stats(x[i], eps)
            if Fraction(float(mu[i])) != emu or Fraction(float(r[i])) != er:
                return False
    return True


def check_apply_exact(apply_fn) -> bool:
    x = W.random_bits((4, 96), seed=64)
    g = W.random_bits((96,), seed=65, std=0.1, mean=1.0)
    b = W.random_bits((96,), seed=66, std=0.2)
    mu, r = O.layernorm_stats(x, 1e-6)
    for gg, bb in ((None, None), (g, b)):
        y = apply_fn(x, mu, r, gg, bb)
        for i in range(4):
            m, ri = Fraction(float(mu[i])), Fraction(float(r[i]))
            for k in range(96):
                u = E.f32(E.f32(E.bf16_value(x[i, k]) - m) * ri)
                if gg is not None:
                    u = E.f32(u * E.bf16_value(gg[k]))
                if bb is not None:
                    u = E.f32(u + E.bf16_value(bb[k]))
                if E.bf16_value(y[i, k]) != E.bf16(u):
                    return False
    return True


def check_modulate_exact(mod_fn) -> bool:
    y = W.random_bits((3, 64), seed=67)
    sc = W.random_bits((64,), seed=68, std=0.3)
    sh = W.random_bits((64,), seed=69, std=0.5)
    z = mod_fn(y, sc, sh)
    for i in range(3):
        for k in range(64):
            m = E.bf16(E.f32(1 + E.bf16_value(sc[k])))
            p = E.bf16(E.f32(E.bf16_value(y[i, k]) * m))
            if E.bf16_value(z[i, k]) != E.bf16(E.f32(p + E.bf16_value(sh[k]))):
                return False
    # identities: scale 0 and shift 0 change nothing; scale -1 leaves the shift
    zero = np.zeros(64, np.uint16)
    if not np.array_equal(O.bf16_to_f32(mod_fn(y, zero, zero)), O.bf16_to_f32(y)):
        return False
    minus1 = np.full(64, E.bf16_bits(Fraction(-1)), np.uint16)
    if not np.array_equal(O.bf16_to_f32(mod_fn(y, minus1, sh)),
                          np.broadcast_to(O.bf16_to_f32(sh), y.shape)):
        return False
    return True


# ---- tests -------------------------------------------------------------------

def test_layernorm_golden_worked_examples():
    assert check_golden(O.layernorm_quant)


def test_layernorm_stats_exact():
    assert check_stats_exact(O.layernorm_stats)


def test_layernorm_apply_exact():
    assert check_apply_exact(O.layernorm_bf16)


def test_modulation_exact_and_identities():
    assert check_modulate_exact(O.modulate_bf16)


def test_layernorm_closed_forms():
    K = 256
    # constant rows: mean c, variance 0, r = fl32(1/sqrt(eps)), y = beta
    for c, eps in ((3.0, 1e-6), (-7.5, 0.25)):
        x = np.full((1, K), E.bf16_bits(Fraction(c)), dtype=np.uint16)
        mu, r = O.layernorm_stats(x, eps)
        assert float(mu[0]) == c
        assert Fraction(float(r[0])) == E.inv_sqrt_f32(Fraction(float(np.float32(eps))))
        q, s, _, _ = O.layernorm_quant(x, eps)
        assert np.all(q == 0) and s[0] == 0
    # two values +-a (mean 0, var a^2): xhat = +-a r, all codes +-127
    a = Fraction(3, 2)
    x = np.tile(bits_of([a, -a]), K // 2)[None, :]
    mu, r = O.layernorm_stats(x, 1e-6)
    assert float(mu[0]) == 0.0
    assert Fraction(float(r[0])) == E.inv_sqrt_f32(a * a + Fraction(float(np.float32(1e-6))))
    q, _, _, _ = O.layernorm_quant(x, 1e-6)
    assert np.array_equal(q[0], np.tile(np.array([127, -127], np.int8), K // 2))


def test_layernorm_invariances():
    # a shift by an exactly representable constant (small integers + 64 stay
    # exact in BF16) changes mu by the constant and leaves r and the codes alone
    rng = np.random.default_rng(70)
    vals = rng.integers(-20, 21, (5, 128))
    x = bits_of([int(v) for v in vals.reshape(-1)]).reshape(5, 128)
    x2 = bits_of([int(v) + 64 for v in vals.reshape(-1)]).reshape(5, 128)
    q1, s1, mu1, r1 = O.layernorm_quant(x, 1e-6)
    q2, s2, mu2, r2 = O.layernorm_quant(x2, 1e-6)
    assert np.array_equal(r1, r2) and np.array_equal(q1, q2) and np.array_equal(s1, s2)
    assert np.array_equal(mu2, mu1 + np.float32(64))
    # a power-of-two scale with eps = 0 leaves the codes alone
    xs = W.random_bits((5, 128), seed=71)
    xs4 = O.f32_to_bf16(O.bf16_to_f32(xs) * np.float32(4))
    qa, sa, _, _ = O.layernorm_quant(xs, 0.0)
    qb, sb, _, _ = O.layernorm_quant(xs4, 0.0)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


def test_layernorm_matches_torch_float64():
    """torch's LayerNorm in float64, rounded to BF16, is within 1 BF16 ulp of the
    oracle's y (which rounds each fp32 step), and its statistics agree."""
    x = W.random_bits((16, 512), seed=72)
    x[3] = W.random_bits((512,), seed=73, std=2.0, mean=-5.0)
    g = W.random_bits((512,), seed=74, std=0.1, mean=1.0)
    b = W.random_bits((512,), seed=75, std=0.1)
    eps = 1e-5
    mu, r = O.layernorm_stats(x, eps)
    y = O.layernorm_bf16(x, mu, r, g, b)
    xt = torch.from_numpy(O.bf16_to_f32(x).astype(np.float64))
    ref = torch.nn.functional.layer_norm(
        xt, (512,), torch.from_numpy(O.bf16_to_f32(g).astype(np.float64)),
        torch.from_numpy(O.bf16_to_f32(b).astype(np.float64)), eps=float(np.float32(eps)))
    ref_bits = O.f32_to_bf16(ref.numpy().astype(np.float32))
    assert O.bf16_ulp_distance(y, ref_bits).max() <= 1
    var, mean = torch.var_mean(xt, dim=1, unbiased=False)
    assert np.allclose(mu, mean.numpy(), rtol=0, atol=1e-6 * np.abs(mean.numpy()).max() + 1e-12)
    assert np.allclose(r, (1 / torch.sqrt(var + float(np.float32(eps)))).numpy(), rtol=2e-7)


# ---- planted mistakes ------------------------------------------------------------

def _stats_unbiased(x_bits, eps):
    x = O.bf16_to_f32(x_bits).astype(np.float64)
    k = x.shape[1]
    mu = x.mean(axis=1)
    var = ((x - mu[:, None]) ** 2).sum(axis=1) / (k - 1)
    return mu.astype(np.float32), (1 / np.sqrt(var + float(np.float32(eps)))).astype(np.float32)


def _stats_eps_outside(x_bits, eps):
    x = O.bf16_to_f32(x_bits).astype(np.float64)
    mu = x.mean(axis=1)
    var = ((x - mu[:, None]) ** 2).mean(axis=1)
    return mu.astype(np.float32), (1 / (np.sqrt(var) + float(np.float32(eps)))).astype(np.float32)


def _apply_no_centering(x_bits, mu, r, g=None, b=None):
    return O.layernorm_bf16(x_bits, np.zeros_like(mu), r, g, b)


def _apply_beta_before_gamma(x_bits, mu, r, g=None, b=None):
    x = O.bf16_to_f32(x_bits)
    u = ((x - mu[:, None]).astype(np.float32) * r[:, None]).astype(np.float32)
    if b is not None:
        u = (u + O.bf16_to_f32(b)[None, :]).astype(np.float32)
    if g is not None:
        u = (u * O.bf16_to_f32(g)[None, :]).astype(np.float32)
    return O.f32_to_bf16(u)


def _mod_scale_not_one_plus(y, sc=None, sh=None):
    z = O.bf16_to_f32(y)
    if sc is not None:
        z = O.bf16_to_f32(O.f32_to_bf16((z * O.bf16_to_f32(sc)[None, :]).astype(np.float32)))
    if sh is not None:
        z = O.bf16_to_f32(O.f32_to_bf16((z + O.bf16_to_f32(sh)[None, :]).astype(np.float32)))
    return O.f32_to_bf16(z)


def _mod_shift_subtracted(y, sc=None, sh=None):
    return O.modulate_bf16(y, sc, None if sh is None else
                           O.f32_to_bf16(-O.bf16_to_f32(sh)))


def _mod_no_bf16_rounding(y, sc=None, sh=None):
    z = O.bf16_to_f32(y)
    if sc is not None:
        z = (z * (np.float32(1) + O.bf16_to_f32(sc))[None, :]).astype(np.float32)
    if sh is not None:
        z = (z + O.bf16_to_f32(sh)[None, :]).astype(np.float32)
    return O.f32_to_bf16(z)


def _ln_quant_with(stats=O.layernorm_stats, apply=O.layernorm_bf16, mod=O.modulate_bf16):
    def f(x, eps, g=None, b=None, sc=None, sh=None):
        mu, r = stats(x, eps)
        z = mod(apply(x, mu, r, g, b), sc, sh)
        q, s = O.quantize_rows(z)
        return q, s, mu, r
    return f


def test_planted_mistakes():
    assert not check_stats_exact(_stats_unbiased)
    assert not check_stats_exact(_stats_eps_outside)
    assert not check_apply_exact(_apply_no_centering)
    assert not check_apply_exact(_apply_beta_before_gamma)
    assert not check_modulate_exact(_mod_scale_not_one_plus)
    assert not check_modulate_exact(_mod_shift_subtracted)
    assert not check_modulate_exact(_mod_no_bf16_rounding)
    # and the end-to-end fixtures catch the same mistakes
    assert not check_golden(_ln_quant_with(stats=_stats_unbiased))
    assert not check_golden(_ln_quant_with(apply=_apply_no_centering))
    assert not check_golden(_ln_quant_with(mod=_mod_scale_not_one_plus))
    assert not check_golden(_ln_quant_with(mod=_mod_shift_subtracted))

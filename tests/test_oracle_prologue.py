"""Pins of the attention-prologue oracle (q/k RMSNorm, RoPE, store) — CPU.

Every pin restates what the definitions fix, independently of the oracle's
own formulas:
* RMSNorm: a unit-weight result has root-mean-square 1 (eps -> 0); it is
  invariant to scaling the input; a constant vector c maps to sign(c) * w;
* RoPE: position 0 is the identity; each (i, i + D/2) pair keeps its length;
  the dot product of a rotated q (position m) and k (position n) depends
  only on m - n (the property RoPE exists for); one pair against the
  complex-number rotation written out by hand;
* the cache: cos^2 + sin^2 = 1, row 0 = (1, 0), theta_0 = 1 (first column is
  cos(p) / sin(p));
* the store: v rows copied bit for bit, k rows equal to the bf16 rounding of
  the prologue's k, every other slot untouched.
"""

import math

import numpy as np
import pytest

import oracle
from workloads import random_bf16


def test_rms_norm_unit_rms_scale_invariance_and_constant():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7, 128))
    y = oracle.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-12)
    assert np.allclose(oracle.rms_norm(3.5 * x, np.ones(128), 0.0), y, atol=1e-12)
    w = rng.standard_normal(128)
    c = np.full((1, 128), -2.0)
    assert np.allclose(oracle.rms_norm(c, w, 0.0), -w[None, :], atol=1e-12)
    assert oracle.rms_norm(x, None, 1e-6) is x


def test_rope_cache_closed_forms():
    cache = oracle.rope_cache(4096, 128, 1_000_000.0)
    assert np.allclose(cache[:, :64] ** 2 + cache[:, 64:] ** 2, 1.0, atol=1e-12)
    assert np.array_equal(cache[0, :64], np.ones(64)) and np.array_equal(cache[0, 64:], np.zeros(64))
    p = np.arange(4096)
    assert np.allclose(cache[:, 0], np.cos(p)) and np.allclose(cache[:, 64], np.sin(p))
    # last frequency: base^(-126/128)
    th = 1_000_000.0 ** (-126.0 / 128.0)
    assert np.allclose(cache[1234, 63], math.cos(1234 * th)) and np.allclose(cache[1234, 127], math.sin(1234 * th))


def test_rope_identity_norm_relative_position_and_complex_form():
    rng = np.random.default_rng(1)
    D, P = 128, 5000
    cache = oracle.rope_cache(P, D, 10_000.0)
    x = rng.standard_normal((3, 2, D))
    assert np.allclose(oracle.rope(x, np.zeros(3, int), cache), x, atol=1e-15)
    y = oracle.rope(x, np.array([5, 77, 4999]), cache)
    n_in = x[..., :64] ** 2 + x[..., 64:] ** 2
    n_out = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(n_in, n_out, atol=1e-12)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    def dot(m, n):
        return float(np.sum(oracle.rope(q, np.array([m]), cache) * oracle.rope(k, np.array([n]), cache)))
    assert abs(dot(100, 40) - dot(1100, 1040)) < 1e-9
    assert abs(dot(100, 40) - dot(61, 1)) < 1e-9
    assert abs(dot(100, 40) - dot(40, 100)) > 1e-3          # not symmetric in general
    # pair i = 3 of one vector, by hand: (a + ib) e^{i p theta_3}
    pos, i = 321, 3
    th = 10_000.0 ** (-2.0 * i / D)
    z = complex(x[0, 0, i], x[0, 0, i + 64]) * complex(math.cos(pos * th), math.sin(pos * th))
    r = oracle.rope(x[:1], np.array([pos]), cache)
    assert abs(r[0, 0, i] - z.real) < 1e-12 and abs(r[0, 0, i + 64] - z.imag) < 1e-12


def test_prologue_store_and_split():
    rng = np.random.default_rng(2)
    Hq, Hkv, D, T, S = 4, 2, 128, 6, 50
    qkv = random_bf16(rng, (T, (Hq + 2 * Hkv) * D))
    kp = random_bf16(rng, (S, Hkv, D))
    vp = random_bf16(rng, (S, Hkv, D))
    qw = random_bf16(rng, (D,))
    kw = random_bf16(rng, (D,))
    pos = rng.integers(0, 1000, T)
    loc = rng.permutation(S)[:T]
    cache = oracle.rope_cache(1000, D, 1_000_000.0)
    q, k, kp2, vp2 = oracle.qk_norm_rope_store(qkv, Hq, Hkv, qw, kw, 1e-6, pos, cache, kp, vp, loc)
    x = oracle.bf16_to_f64(qkv).reshape(T, Hq + 2 * Hkv, D)
    # v heads copied bit for bit to their slots; k slots hold bf16(k)
    assert np.array_equal(vp2[loc], qkv.reshape(T, Hq + 2 * Hkv, D)[:, Hq + Hkv:])
    assert np.array_equal(kp2[loc], oracle.f64_to_bf16_rne(k))
    others = np.setdiff1d(np.arange(S), loc)
    assert np.array_equal(kp2[others], kp[others]) and np.array_equal(vp2[others], vp[others])
    # q: norm with q weight then rotation; at position 0 it is just the norm
    pos0 = np.zeros(T, int)
    q0, _, _, _ = oracle.qk_norm_rope_store(qkv, Hq, Hkv, qw, kw, 1e-6, pos0, cache, kp, vp, loc)
    xq = x[:, :Hq]
    want = xq / np.sqrt(np.mean(xq * xq, axis=-1, keepdims=True) + 1e-6) * oracle.bf16_to_f64(qw)
    assert np.allclose(q0, want, atol=1e-12)
    # without norms the k heads are the raw k slice rotated
    _, k_raw, _, _ = oracle.qk_norm_rope_store(qkv, Hq, Hkv, None, None, 1e-6, pos0, cache, kp, vp, loc)
    assert np.array_equal(k_raw, x[:, Hq:Hq + Hkv])


MUTANTS = [
    ("x1 * cos - x2 * sin, x2 * cos + x1 * sin", "x1 * cos + x2 * sin, x2 * cos - x1 * sin"),
    ("-2.0 * np.arange(half", "-1.0 * np.arange(half"),
    ("[np.cos(ang), np.sin(ang)]", "[np.sin(ang), np.cos(ang)]"),
    ("np.mean(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-1, keepdims=True)"),
    ("c[:, None, :half]", "c[:, None, half:]"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistakes_are_caught(old, new):
    import os
    import types
    import oracle.attention as att
    path = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "prologue.py")
    src = open(path).read()
    assert old in src
    mod = types.ModuleType("prologue_mutant")
    mod.__dict__["__package__"] = "oracle"
    mod.__dict__["__name__"] = "oracle.prologue_mutant"
    exec(compile(src.replace(old, new, 1), "prologue_mutant", "exec"), mod.__dict__)
    failed = 0
    for pin in (test_rms_norm_unit_rms_scale_invariance_and_constant, test_rope_cache_closed_forms,
                test_rope_identity_norm_relative_position_and_complex_form):
        saved = (oracle.rms_norm, oracle.rope, oracle.rope_cache)
        oracle.rms_norm, oracle.rope, oracle.rope_cache = mod.rms_norm, mod.rope, mod.rope_cache
        try:
            pin()
        except AssertionError:
            failed += 1
        finally:
            oracle.rms_norm, oracle.rope, oracle.rope_cache = saved
    assert failed > 0
    assert att is not None

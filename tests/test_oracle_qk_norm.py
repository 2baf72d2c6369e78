"""Pins for the oracle's q/k L2 normalisation (the library's in-kernel normalisation mode):
x / sqrt(sum(x^2) + 1e-6) per token and head, in fp64, before the recurrence."""
import numpy as np

import oracle
from synth import inputs as I


def test_worked_values():
    # (3, 4): length 5, so (0.6, 0.8) up to the epsilon (relative 2e-8).
    x = oracle.qk_normalize(np.array([[3.0, 4.0]]))
    assert np.allclose(x, [[0.6, 0.8]], rtol=1e-7, atol=0)
    # (1e-4, 0): 1e-4 / sqrt(1e-8 + 1e-6) = 1e-4 / 1.0049876e-3 = 0.0995037 (the epsilon sits inside
    # the square root, added to the squared length).
    y = oracle.qk_normalize(np.array([[1e-4, 0.0]]))
    assert abs(y[0, 0] - 0.0995037190) < 1e-9 and y[0, 1] == 0.0
    # a zero vector stays zero
    assert np.all(oracle.qk_normalize(np.zeros((1, 4))) == 0.0)


def test_bf16_upcast_is_exact():
    b = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x4049], dtype=np.uint16)
    assert np.array_equal(oracle.upcast(b), [1.0, -2.0, 1.5, 0.0, 3.140625])


def test_unit_inputs_are_left_alone():
    x = I.draw(T=150, hqk=2, hv=4, dk=16, dtype="fp32", seed=201, s0_std=0.3)
    o0, f0 = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens)
    o1, f1 = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, qk_l2norm=True)
    assert oracle.rel_l2(o1, o0) < 2e-6 and oracle.rel_l2(f1, f0) < 2e-6


def test_only_directions_matter():
    """Rescaling each token's q and k row by its own positive factor (lengths >= 1, so the
    epsilon moves results by < 1e-6) leaves the normalised run unchanged; normalising over
    the wrong axis, or by the squared length, would not."""
    x = I.draw(lengths=[70, 33], hqk=2, hv=4, dk=16, dtype="fp32", seed=202, s0_std=0.3, qk_unit=False)
    rng = np.random.default_rng(7)
    q = x.q.astype(np.float64) / np.linalg.norm(x.q.astype(np.float64), axis=-1, keepdims=True)
    k = x.k.astype(np.float64) / np.linalg.norm(x.k.astype(np.float64), axis=-1, keepdims=True)
    q2 = q * rng.uniform(1.0, 100.0, size=q.shape[:-1] + (1,))
    k2 = k * rng.uniform(1.0, 100.0, size=k.shape[:-1] + (1,))
    v = x.v.astype(np.float64)
    o1, f1 = oracle.recurrent(q2, k2, v, x.g, x.beta, x.s0, x.cu_seqlens, qk_l2norm=True)
    o2, f2 = oracle.recurrent(q, k, v, x.g, x.beta, x.s0, x.cu_seqlens)
    assert oracle.rel_l2(o1, o2) < 2e-6 and oracle.rel_l2(f1, f2) < 2e-6


def test_the_flag_changes_unnormalised_inputs():
    x = I.draw(T=90, hqk=1, hv=2, dk=16, dtype="bf16", seed=203, qk_unit=False)
    o0, _ = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta)
    o1, _ = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, qk_l2norm=True)
    assert oracle.rel_l2(o0, o1) > 0.1

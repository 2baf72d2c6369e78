"""The fp64 oracle against properties of the rule that do not depend on its code."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    assert pin(oracle.recurrent)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_chunked_form_pin(pin):
    # The chunked UT/WY form satisfies the same pins (chunk 4 so that tiny
    # problems span several chunks).
    def run(*a, **kw):
        return oracle.chunked(*a, chunk=4, **kw)
    assert pin(run)


MUTANTS = {1: "no decay", 2: "read-out before write", 3: "state transposed in the correction",
           4: "V head h uses QK head h % Hqk", 5: "correction sign flipped", 6: "decay after the write"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_pins_catch_planted_mistakes(mutant):
    def run(*a, **kw):
        return oracle.recurrent(*a, mutant=mutant, **kw)
    failed = [p.__name__ for p in pins.ALL_PINS if not p(run)]
    assert failed, f"no pin detects mutant {mutant} ({MUTANTS[mutant]})"


@pytest.mark.parametrize("T,d,chunk", [(1, 4, 64), (63, 5, 64), (64, 16, 64), (65, 8, 64),
                                       (130, 8, 64), (200, 8, 64), (131, 5, 16)])
def test_chunked_equals_recurrent(T, d, chunk):
    r = np.random.default_rng(T * 100 + d)
    q = r.standard_normal((T, 1, d)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((T, 1, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, 2, d))
    g = -np.log1p(np.exp(r.standard_normal((T, 2))))
    beta = 1 / (1 + np.exp(-r.standard_normal((T, 2))))
    s0 = r.standard_normal((1, 2, d, d))
    o_r, f_r = oracle.recurrent(q, k, v, g, beta, s0, scale=0.5)
    o_c, f_c = oracle.chunked(q, k, v, g, beta, s0, scale=0.5, chunk=chunk)
    assert oracle.rel_l2(o_c, o_r) <= 1e-12
    assert oracle.rel_l2(f_c, f_r) <= 1e-12


def test_near_parallel_keys_stay_bounded():
    # beta -> 1 with nearly parallel keys makes (I + A) nearly singular in
    # exact arithmetic only when alpha = 1; the recurrence stays finite and the
    # chunked form still agrees.
    T, d = 64, 16
    r = np.random.default_rng(5)
    base = r.standard_normal(d)
    k = base[None, None, :] + 1e-3 * r.standard_normal((T, 1, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = k.copy()
    v = r.standard_normal((T, 1, d))
    g = np.full((T, 1), -1e-3)
    beta = np.full((T, 1), 0.999)
    o_r, f_r = oracle.recurrent(q, k, v, g, beta)
    o_c, f_c = oracle.chunked(q, k, v, g, beta)
    assert np.all(np.isfinite(o_r)) and oracle.rel_l2(o_c, o_r) <= 1e-8


def test_bf16_inputs_are_widened_exactly():
    from synth import inputs as I
    x = I.draw(T=20, hqk=1, hv=2, dk=8, dtype="bf16", seed=3)
    o_bits, f_bits = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta)
    o_f64, f_f64 = oracle.recurrent(I.bf16_bits_to_f32(x.q).astype(np.float64),
                                    I.bf16_bits_to_f32(x.k).astype(np.float64),
                                    I.bf16_bits_to_f32(x.v).astype(np.float64),
                                    x.g.astype(np.float64), x.beta.astype(np.float64))
    assert np.array_equal(o_bits, o_f64) and np.array_equal(f_bits, f_f64)


def test_head_subset_matches_full_run():
    from synth import inputs as I
    x = I.draw(T=50, hqk=2, hv=4, dk=8, dtype="fp32", seed=4, s0_std=0.1)
    o, f = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.s0)
    o2, f2 = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.s0, heads=(1, 3))
    assert np.array_equal(o[:, 1:3], o2) and np.array_equal(f[:, 1:3], f2)

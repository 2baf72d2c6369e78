"""Pins for the fp64 backward oracle: every gradient element against central finite differences of
the C recurrence (a separate implementation of the forward), linearity in the output cotangents,
and zero cotangents giving zero gradients. CPU only."""
import numpy as np

import oracle
from synth import inputs as I


def _case():
    x = I.draw(lengths=[5, 3], hqk=1, hv=2, dk=3, dtype="fp32", seed=11, s0_std=0.3)
    rng = np.random.default_rng(12)
    d_out = rng.standard_normal(x.v.shape)
    d_fin = rng.standard_normal(x.s0.shape)
    return x, d_out, d_fin


def _loss(x, ins, d_out, d_fin):
    q, k, v, g, b, s0 = ins
    o, f = oracle.recurrent(q, k, v, g, b, s0, x.cu_seqlens, scale=x.scale)
    return float(np.sum(o * d_out) + np.sum(f * d_fin))


def test_gradients_match_finite_differences():
    x, d_out, d_fin = _case()
    base = [a.astype(np.float64) for a in (x.q, x.k, x.v, x.g, x.beta, x.s0)]
    gr = oracle.backward(*base[:5], base[5], x.cu_seqlens, d_out, d_fin, scale=x.scale)
    names = ["dq", "dk", "dv", "dg", "dbeta", "ds0"]
    h = 1e-6
    for i, name in enumerate(names):
        num = np.zeros_like(base[i])
        for e in np.ndindex(base[i].shape):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[i][e] += h
            minus[i][e] -= h
            num[e] = (_loss(x, plus, d_out, d_fin) - _loss(x, minus, d_out, d_fin)) / (2 * h)
        err = np.max(np.abs(num - gr[name])) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-7, (name, err)


def test_linear_in_cotangents_and_zero_for_zero():
    x, d_out, d_fin = _case()
    rng = np.random.default_rng(13)
    d2 = rng.standard_normal(d_out.shape)
    args = (x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens)
    a = oracle.backward(*args, d_out, d_fin)
    b = oracle.backward(*args, d2, None)
    c = oracle.backward(*args, d_out + 2.0 * d2, d_fin)
    for name in a:
        assert np.allclose(c[name], a[name] + 2.0 * b[name], rtol=1e-12, atol=1e-12), name
    z = oracle.backward(*args, np.zeros_like(d_out), None)
    assert all(np.all(z[name] == 0.0) for name in z)

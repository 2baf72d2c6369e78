"""Property pins for a gated-delta-rule implementation.

Each pin states something that follows from the rule itself (page
"Qwen3-Next-80B-A3B-Instruct", section "Model Overview", names Gated DeltaNet as
the linear-attention mixer; its update is: decay the state by alpha = exp(g),
correct it along the unit key k with strength beta so that it maps k towards v,
read it out with q). None of them uses the oracle's own code: the expected
values are closed forms, hand-derived sequences, or a different algebraic form
of the rule built from numpy matrix products.

A "runner" is any callable with oracle.recurrent's signature returning
(out, final_state) as fp64 arrays; the same pins run on the oracle, on mutated
oracles (to show each pin has teeth) and on the GPU path.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _random_problem(seed, T=40, hqk=2, hv=4, dk=8, dv=8, s0=True):
    r = _rng(seed)
    return dict(
        q=_unit(r, (T, hqk, dk)), k=_unit(r, (T, hqk, dk)), v=r.standard_normal((T, hv, dv)),
        g=-np.log1p(np.exp(r.standard_normal((T, hv)))),
        beta=1.0 / (1.0 + np.exp(-r.standard_normal((T, hv)))),
        s0=(0.5 * r.standard_normal((1, hv, dv, dk))) if s0 else None,
    )


def _max_rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


# P1: alpha = 1, beta = 0 leaves the state unchanged; the read-out is S0 q.
def pin_identity(run, tol=1e-12, dk=8, dv=6):
    p = _random_problem(11, dk=dk, dv=dv)
    p["g"][:] = 0.0
    p["beta"][:] = 0.0
    out, fin = run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["s0"], scale=1.0)
    hv, hqk = p["v"].shape[1], p["q"].shape[1]
    exp_out = np.stack([np.einsum("ij,tj->ti", p["s0"][0, h], p["q"][:, h // (hv // hqk)])
                        for h in range(hv)], axis=1)
    return _max_rel(fin, p["s0"]) <= tol and _max_rel(out, exp_out) <= tol


# P2: beta = 0 with any g: o_t = exp(sum_{s<=t} g_s) S0 q_t and S_T = exp(sum g) S0.
# S0 is not symmetric and dk != dv, so a transposed state or swapped axes fail.
def pin_pure_decay(run, tol=1e-12):
    p = _random_problem(12, dk=8, dv=5)
    p["beta"][:] = 0.0
    out, fin = run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["s0"], scale=1.0)
    hv, hqk = p["v"].shape[1], p["q"].shape[1]
    decay = np.exp(np.cumsum(p["g"], axis=0))                      # [T, Hv]
    exp_out = np.stack([decay[:, h, None] * np.einsum("ij,tj->ti", p["s0"][0, h], p["q"][:, h // (hv // hqk)])
                        for h in range(hv)], axis=1)
    exp_fin = decay[-1][None, :, None, None] * p["s0"]
    return _max_rel(out, exp_out) <= tol and _max_rel(fin, exp_fin) <= tol


# P3: beta = 1, alpha = 1, S0 = 0 and orthonormal keys: the state is sum_t v_t k_t^T,
# and querying with key k_j returns v_j once token j has been written (0 before).
def pin_orthonormal_retrieval(run, tol=1e-12, d=8):
    r = _rng(13)
    T = d
    keys, _ = np.linalg.qr(r.standard_normal((d, d)))               # columns orthonormal
    k = keys.T[:, None, :].copy()                                   # [T, 1, d]
    sigma = r.permutation(T)
    q = keys.T[sigma][:, None, :].copy()
    v = r.standard_normal((T, 1, d))
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    out, fin = run(q, k, v, g, beta, None, scale=1.0)
    exp_fin = np.einsum("ti,tj->ij", v[:, 0], k[:, 0])
    exp_out = np.where((sigma <= np.arange(T))[:, None], v[sigma, 0], 0.0)
    return (np.max(np.abs(fin[0, 0] - exp_fin)) <= tol * np.max(np.abs(exp_fin))
            and np.max(np.abs(out[:, 0] - exp_out)) <= tol * np.max(np.abs(v)))


# P4: beta_t = 1 and |k_t| = 1 make S_t k_t = v_t whatever the decay and history,
# so a query equal to the key reads v_t back exactly.
def pin_delta_write(run, tol=1e-11):
    p = _random_problem(14, T=30, dk=8, dv=8)
    write = np.zeros(p["beta"].shape, dtype=bool)
    write[5::3] = True
    p["beta"][write] = 1.0
    p["q"] = p["k"].copy()
    out, _ = run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["s0"], scale=1.0)
    return float(np.max(np.abs(out[write] - p["v"][write]))) <= tol


# P5: the scalar case d = 1, k = q = 1: s_t = alpha (1 - beta) s_{t-1} + beta v.
# With alpha = beta = 1/2, v = 1, s0 = 0 the sequence is 1/2, 5/8, 21/32, ...
# = (2/3)(1 - 4^-t), tending to beta v / (1 - alpha (1 - beta)) = 2/3.
def pin_scalar_worked_example(run, tol=1e-15):
    with open(os.path.join(GOLDEN, "scalar_alpha_half_beta_half.json")) as f:
        gold = json.load(f)
    n = len(gold["s"])
    ones = np.ones((n, 1, 1))
    out, fin = run(ones, ones, ones, np.full((n, 1), np.log(0.5)), np.full((n, 1), 0.5), None, scale=1.0)
    s = np.array(gold["s"], dtype=np.float64)
    closed = (2.0 / 3.0) * (1.0 - 4.0 ** -np.arange(1, n + 1))
    return (np.max(np.abs(out[:, 0, 0] - s)) <= tol and abs(fin[0, 0, 0, 0] - s[-1]) <= tol
            and np.max(np.abs(s - closed)) <= 1e-15)


# P6: for fixed q, k, g, beta the map (v, S0) -> (o, S_T) is linear; o is linear in q
# and in the scale argument.
def pin_linearity(run, tol=1e-12):
    p1 = _random_problem(15)
    p2 = _random_problem(16)
    a, b = 0.7, -1.9
    base = dict(q=p1["q"], k=p1["k"], g=p1["g"], beta=p1["beta"])
    o1, f1 = run(base["q"], base["k"], p1["v"], base["g"], base["beta"], p1["s0"], scale=1.0)
    o2, f2 = run(base["q"], base["k"], p2["v"], base["g"], base["beta"], p2["s0"], scale=1.0)
    o3, f3 = run(base["q"], base["k"], a * p1["v"] + b * p2["v"], base["g"], base["beta"],
                 a * p1["s0"] + b * p2["s0"], scale=1.0)
    ok = _max_rel(o3, a * o1 + b * o2) <= tol and _max_rel(f3, a * f1 + b * f2) <= tol
    o4, _ = run(-3.0 * base["q"], base["k"], p1["v"], base["g"], base["beta"], p1["s0"], scale=1.0)
    o5, _ = run(base["q"], base["k"], p1["v"], base["g"], base["beta"], p1["s0"], scale=0.25)
    return ok and _max_rel(o4, -3.0 * o1) <= tol and _max_rel(o5, 0.25 * o1) <= tol


# P7: resuming from a saved state is the same as one run, for a split that is not a
# multiple of the chunk size; one-token runs chained T times equal one run.
def pin_resume(run, tol=1e-12):
    p = _random_problem(17, T=75)
    o, f = run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["s0"], scale=1.0)
    T1 = 37
    oa, fa = run(p["q"][:T1], p["k"][:T1], p["v"][:T1], p["g"][:T1], p["beta"][:T1], p["s0"], scale=1.0)
    ob, fb = run(p["q"][T1:], p["k"][T1:], p["v"][T1:], p["g"][T1:], p["beta"][T1:], fa, scale=1.0)
    ok = _max_rel(np.concatenate([oa, ob]), o) <= tol and _max_rel(fb, f) <= tol
    s = p["s0"]
    steps = []
    for t in range(12):
        ot, s = run(p["q"][t:t + 1], p["k"][t:t + 1], p["v"][t:t + 1], p["g"][t:t + 1],
                    p["beta"][t:t + 1], s, scale=1.0)
        steps.append(ot)
    o12, f12 = run(p["q"][:12], p["k"][:12], p["v"][:12], p["g"][:12], p["beta"][:12], p["s0"], scale=1.0)
    return ok and _max_rel(np.concatenate(steps), o12) <= tol and _max_rel(s, f12) <= tol


# P8: packed variable-length sequences are independent of each other (and a
# zero-length sequence returns its initial state); V heads 2h', 2h'+1 read QK head h'.
def pin_varlen_and_heads(run, tol=1e-12):
    r = _rng(18)
    lengths = [13, 0, 64, 1, 70]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    p = _random_problem(19, T=T)
    s0 = 0.3 * r.standard_normal((len(lengths), 4, 8, 8))
    o, f = run(p["q"], p["k"], p["v"], p["g"], p["beta"], s0, cu, scale=1.0)
    ok = True
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        on, fn = run(p["q"][a:b], p["k"][a:b], p["v"][a:b], p["g"][a:b], p["beta"][a:b], s0[n:n + 1], scale=1.0)
        ok &= _max_rel(o[a:b], on) <= tol if b > a else True
        ok &= _max_rel(f[n:n + 1], fn) <= tol
    ok &= _max_rel(f[1], s0[1]) == 0.0
    # Zeroing QK head 1 silences exactly V heads 2 and 3 (zero initial state).
    q, k = p["q"].copy(), p["k"].copy()
    q[:, 1] = 0.0
    k[:, 1] = 0.0
    oz, _ = run(q, k, p["v"], p["g"], p["beta"], None, scale=1.0)
    ok &= bool(np.all(oz[:, 2:4] == 0.0)) and bool(np.all(np.abs(oz[:, 0:2]).max(axis=(0, 2)) > 0))
    # Swapping the two QK heads together with their V-head pairs swaps the outputs.
    perm_qk = [1, 0]
    perm_v = [2, 3, 0, 1]
    op, fp = run(p["q"][:, perm_qk], p["k"][:, perm_qk], p["v"][:, perm_v], p["g"][:, perm_v],
                 p["beta"][:, perm_v], None, scale=1.0)
    o0, f0 = run(p["q"], p["k"], p["v"], p["g"], p["beta"], None, scale=1.0)
    ok &= _max_rel(op, o0[:, perm_v]) <= tol and _max_rel(fp, f0[:, perm_v]) <= tol
    return bool(ok)


# P9: the product form the rule's description uses: each token applies the
# affine map S -> S (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T.
def pin_product_form(run, tol=1e-12):
    p = _random_problem(20, T=25, hqk=1, hv=2, dk=6, dv=4)
    out, fin = run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["s0"], scale=1.0)
    ok = True
    for h in range(2):
        S = p["s0"][0, h].copy()
        for t in range(p["q"].shape[0]):
            kt = p["k"][t, 0][:, None]
            M = np.exp(p["g"][t, h]) * (np.eye(6) - p["beta"][t, h] * (kt @ kt.T))
            S = S @ M + p["beta"][t, h] * (p["v"][t, h][:, None] @ kt.T)
            ok &= _max_rel(out[t, h], S @ p["q"][t, 0]) <= tol * 10
        ok &= _max_rel(fin[0, h], S) <= tol
    return bool(ok)


ALL_PINS = [pin_identity, pin_pure_decay, pin_orthonormal_retrieval, pin_delta_write,
            pin_scalar_worked_example, pin_linearity, pin_resume, pin_varlen_and_heads,
            pin_product_form]

"""The fp64 short-convolution oracle (oracle/conv.py) against properties of a depthwise causal
convolution that do not depend on its code: a hand-worked example, identity and shift kernels,
linearity, causality, the varlen reset, history continuation and SiLU's closed-form values. A
mutation test plants four plausible mistakes and checks that some pin catches each."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "conv_hand_example.json")


def _problem(seed, lengths=(9, 1, 0, 5), C=6, K=4):
    r = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(x=r.standard_normal((T, C)), w=r.standard_normal((C, K)), cu=cu,
                hist=r.standard_normal((len(lengths), K - 1, C)))


def pin_hand_example(conv):
    g = json.load(open(GOLDEN))
    x = np.array(g["x"], float)[:, None]
    w = np.array(g["w"], float)[None, :]
    y, h = conv(x, w)
    ok = np.array_equal(y[:, 0], g["no_history"]["y"]) and np.array_equal(h[0, :, 0], g["no_history"]["new_history"])
    hist = np.array(g["history_7_8_9"]["history"], float)[None, :, None]
    y, h = conv(x, w, None, hist)
    ok &= np.array_equal(y[:, 0], g["history_7_8_9"]["y"]) and np.array_equal(h[0, :, 0], g["history_7_8_9"]["new_history"])
    s = g["short_sequence_with_history"]
    y, h = conv(np.array(s["x"], float)[:, None], w, None, np.array(s["history"], float)[None, :, None])
    return bool(ok and np.array_equal(y[:, 0], s["y"]) and np.array_equal(h[0, :, 0], s["new_history"]))


def pin_identity_kernel(conv):
    p = _problem(1)
    w = np.zeros_like(p["w"])
    w[:, -1] = 1.0
    y, _ = conv(p["x"], w, p["cu"], p["hist"])
    return bool(np.array_equal(y, p["x"]))


def pin_shift_by_one(conv):
    # w = e_{K-2}: y_t = x_{t-1}; a sequence's first output is the newest history row.
    p = _problem(2)
    w = np.zeros_like(p["w"])
    w[:, -2] = 1.0
    y, _ = conv(p["x"], w, p["cu"], p["hist"])
    cu = p["cu"]
    for n in range(len(cu) - 1):
        b, e = int(cu[n]), int(cu[n + 1])
        if e == b:
            continue
        if not np.array_equal(y[b], p["hist"][n, -1]) or not np.array_equal(y[b + 1:e], p["x"][b:e - 1]):
            return False
    return True


def pin_linearity(conv):
    p, q = _problem(3), _problem(4)
    a, b = 0.75, -1.5
    y1, h1 = conv(p["x"], p["w"], p["cu"], p["hist"])
    y2, h2 = conv(q["x"], p["w"], p["cu"], q["hist"])
    y, h = conv(a * p["x"] + b * q["x"], p["w"], p["cu"], a * p["hist"] + b * q["hist"])
    return bool(np.allclose(y, a * y1 + b * y2, rtol=0, atol=1e-12) and np.allclose(h, a * h1 + b * h2, atol=1e-12))


def pin_causality(conv):
    # Changing x_t leaves every earlier output unchanged and changes y_t.
    p = _problem(5, lengths=(12,))
    y, _ = conv(p["x"], p["w"], p["cu"], p["hist"])
    x2 = p["x"].copy()
    x2[7] += 3.0
    y2, _ = conv(x2, p["w"], p["cu"], p["hist"])
    return bool(np.array_equal(y[:7], y2[:7]) and np.all(y[7] != y2[7]))


def pin_varlen_reset(conv):
    # Packed sequences give what each gives alone with its own history (none leaks into the next).
    p = _problem(6)
    y, h = conv(p["x"], p["w"], p["cu"], p["hist"])
    cu = p["cu"]
    for n in range(len(cu) - 1):
        b, e = int(cu[n]), int(cu[n + 1])
        yn, hn = conv(p["x"][b:e], p["w"], None, p["hist"][n:n + 1])
        if not (np.allclose(y[b:e], yn, atol=1e-13) and np.array_equal(h[n], hn[0])):
            return False
    return True


def pin_continuation(conv):
    # [0, T) in one call equals [0, T1) then [T1, T) from the first call's new history.
    p = _problem(7, lengths=(11,))
    y, h = conv(p["x"], p["w"], None, p["hist"][:1])
    for t1 in (1, 2, 5):
        ya, ha = conv(p["x"][:t1], p["w"], None, p["hist"][:1])
        yb, hb = conv(p["x"][t1:], p["w"], None, ha)
        if not (np.allclose(np.concatenate([ya, yb]), y, atol=1e-13) and np.array_equal(hb, h)):
            return False
    return True


PINS = [pin_hand_example, pin_identity_kernel, pin_shift_by_one, pin_linearity, pin_causality, pin_varlen_reset,
        pin_continuation]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_conv_pin(pin):
    assert pin(oracle.causal_conv1d)


MUTANTS = {1: "taps reversed", 2: "window one token late", 3: "history ignored", 4: "history newest first"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_conv_pins_catch_planted_mistakes(mutant):
    def conv(*a, **kw):
        return oracle.causal_conv1d(*a, mutant=mutant, **kw)
    failed = [p.__name__ for p in PINS if not p(conv)]
    assert failed, f"no pin detects mutant {mutant} ({MUTANTS[mutant]})"


def test_silu_values():
    # silu(y) = y / (1 + e^-y): closed-form values at 0, +-1 and the two limits.
    y = oracle.silu(np.array([0.0, 1.0, -1.0, 40.0, -40.0]))
    e = 1.0 / (1.0 + math.exp(-1.0))
    assert y[0] == 0.0
    assert abs(y[1] - e) < 1e-16 and abs(y[1] - 0.7310585786300049) < 1e-15
    assert abs(y[2] - (e - 1.0)) < 1e-16 and abs(y[2] + 0.2689414213699951) < 1e-15
    assert abs(y[3] - 40.0) < 1e-15 and abs(y[4]) < 1e-15


def test_prologue_splits_and_normalises():
    # The prologue's q, k, v are the convolution's channel ranges; with the flag, the q and k heads
    # come out with unit length (x / sqrt(|x|^2 + 1e-6)) and v is untouched.
    r = np.random.default_rng(8)
    hqk, hv, d, T = 2, 4, 8, 10
    C = 2 * hqk * d + hv * d
    x, w = r.standard_normal((T, C)), r.standard_normal((C, 4))
    y, _ = oracle.causal_conv1d(x, w, silu_act=True)
    q, k, v, _ = oracle.conv_prologue(x, w, hqk, hv, d, d, silu_act=True)
    assert np.array_equal(q.reshape(T, -1), y[:, :hqk * d]) and np.array_equal(v.reshape(T, -1), y[:, 2 * hqk * d:])
    qn, kn, vn, _ = oracle.conv_prologue(x, w, hqk, hv, d, d, silu_act=True, qk_l2norm=True)
    assert np.allclose(np.linalg.norm(qn, axis=-1), np.linalg.norm(q, axis=-1) / np.sqrt(
        np.sum(q * q, axis=-1) + 1e-6), atol=1e-14)
    assert np.array_equal(vn, v) and np.allclose(kn * np.sqrt(np.sum(k * k, -1, keepdims=True) + 1e-6), k, atol=1e-13)

"""fp64 reference of the short causal convolution in front of the Gated DeltaNet mixer.

TEST INFRASTRUCTURE (see oracle/__init__.py): only tests/, the smoke check and
the benchmark's cpu_baseline leg use it.

The model card (page "Qwen3-Next-80B-A3B-Instruct", section "Quickstart")
points to the causal-conv1d kernels beside flash-linear-attention for
efficiency, without saying what they convolve; the reading taken here is a
depthwise causal 1-D convolution over the channels of the mixer's inputs,
q, k and v side by side (channel c < Hqk dk: q; then k; then v), each channel
with its own K taps:

    y_t[c] = sum_{i=0}^{K-1} w[c][i] * x_{t-K+1+i}[c]

(tap K-1 multiplies the current token), where x_s for s before a sequence's
first token comes from that sequence's history (its last K-1 inputs of an
earlier call, oldest first) or is zero when there is none. An optional SiLU
y * sigmoid(y) follows, then optionally the per-head L2 normalisation of the
q and k heads (oracle.qk_normalize). Each sequence's new history is its last
K-1 inputs, reaching back into the old history when it is shorter than K-1.
"""
from __future__ import annotations

import numpy as np


def _upcast(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def silu(y: np.ndarray) -> np.ndarray:
    """y * sigmoid(y) in fp64."""
    return y / (1.0 + np.exp(-y))


def causal_conv1d(x, w, cu_seqlens=None, history=None, silu_act: bool = False, mutant: int = 0):
    """Depthwise causal convolution of packed sequences.

    x: [T, C] (uint16 bf16 bits, float32 or float64); w: [C, K];
    cu_seqlens: [N + 1] offsets (None: one sequence); history: [N, K - 1, C]
    or None (zeros). Returns (y [T, C], new_history [N, K - 1, C]) in fp64.
    mutant (tests only) plants a known mistake: 1 taps reversed, 2 window one
    token late, 3 history ignored, 4 history read newest first.
    """
    x = _upcast(x)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    K = w.shape[1]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    hist = np.zeros((N, K - 1, C)) if history is None else _upcast(history).reshape(N, K - 1, C)
    if mutant == 1:
        w = w[:, ::-1]
    if mutant == 3:
        hist = np.zeros_like(hist)
    if mutant == 4:
        hist = hist[:, ::-1]
    y = np.zeros((T, C))
    new_hist = np.zeros((N, K - 1, C))
    for n in range(N):
        b, e = int(cu[n]), int(cu[n + 1])
        ext = np.concatenate([hist[n], x[b:e]], axis=0)       # rows: K - 1 history rows, then the tokens
        if mutant == 2:
            ext = np.concatenate([np.zeros((1, C)), ext], axis=0)
        for t in range(e - b):
            # token t sits at row t + K - 1 of ext; its window is rows t .. t + K - 1
            y[b + t] = np.sum(w.T * ext[t:t + K], axis=0)
        new_hist[n] = ext[ext.shape[0] - (K - 1):] if K > 1 else np.zeros((0, C))
    if silu_act:
        y = silu(y)
    return y, new_hist


def split_heads(y, hqk: int, hv: int, dk: int, dv: int):
    """[T, C] channels -> q [T, Hqk, dk], k [T, Hqk, dk], v [T, Hv, dv]."""
    T = y.shape[0]
    nq = hqk * dk
    q = y[:, :nq].reshape(T, hqk, dk)
    k = y[:, nq:2 * nq].reshape(T, hqk, dk)
    v = y[:, 2 * nq:2 * nq + hv * dv].reshape(T, hv, dv)
    return q, k, v


def conv_prologue(x, w, hqk: int, hv: int, dk: int, dv: int, cu_seqlens=None, history=None,
                  silu_act: bool = False, qk_l2norm: bool = False):
    """The input prologue in the reading above: convolution, optional SiLU, split into q, k, v and
    optional L2 normalisation of the q and k heads. Returns (q, k, v, new_history), fp64."""
    from . import qk_normalize
    y, h = causal_conv1d(x, w, cu_seqlens, history, silu_act)
    q, k, v = split_heads(y, hqk, hv, dk, dv)
    if qk_l2norm:
        q, k = qk_normalize(q), qk_normalize(k)
    return q, k, v, h

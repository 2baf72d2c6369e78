"""fp64 chunked (UT/WY) form of the gated delta rule, in plain numpy.

TEST INFRASTRUCTURE (see the package docstring). It exists to check, on
small inputs, that the chunk algorithm the GPU kernels use is the same
function as the token-by-token recurrence of gdn_recurrent.c: the chunk size
of 64, the intra-chunk decay masks, the UT transform of the beta-weighted
(I - beta k k^T) factors by a triangular solve and the inter-chunk state
propagation are the steps the layer's description names for the chunked
prefill.

Derivation (for one sequence and one V head; a chunk holds tokens r = 0..n-1
and starts from the state S0, dv x dk):
  gamma_r = sum_{i<=r} g_i, Gamma_r = exp(gamma_r)          in-chunk decay
  u_r     = beta_r (v_r - alpha_r S_{r-1} k_r)               the delta write
  S_r     = Gamma_r S0 + sum_{i<=r} exp(gamma_r - gamma_i) u_i k_i^T
Substituting S_{r-1} gives a unit lower-triangular system for the rows u_r:
  (I + A) U = diag(beta) V - diag(beta Gamma) K S0^T,
  A[r, i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i) for i < r (else 0),
so with Tm = (I + A)^-1, W = Tm diag(beta Gamma) K and Ut = Tm diag(beta) V:
  U   = Ut - W S0^T
  O   = scale * (diag(Gamma) Q S0^T + (D * (Q K^T)) U),  D[r, i] = exp(gamma_r - gamma_i), i <= r
  S_n = Gamma_{n-1} S0 + U^T diag(exp(gamma_{n-1} - gamma)) K
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def _f64(x, dtype_hint=None):
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def chunk_step(S0, Q, K, V, g, beta, scale):
    """One chunk (n <= C tokens). Returns (O [n, dv], S_end [dv, dk])."""
    n = K.shape[0]
    gamma = np.cumsum(g)
    Gamma = np.exp(gamma)
    diff = gamma[:, None] - gamma[None, :]
    lower_strict = np.tril(np.ones((n, n), dtype=bool), -1)
    lower_incl = np.tril(np.ones((n, n), dtype=bool), 0)
    A = np.where(lower_strict, beta[:, None] * np.exp(np.where(lower_strict, diff, 0.0)) * (K @ K.T), 0.0)
    # UT transform: triangular solve of (I + A) Tm = I
    Tm = scipy.linalg.solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
    W = Tm @ ((beta * Gamma)[:, None] * K)
    Ut = Tm @ (beta[:, None] * V)
    U = Ut - W @ S0.T
    D = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
    O = scale * (Gamma[:, None] * (Q @ S0.T) + (D * (Q @ K.T)) @ U)
    decay_to_end = np.exp(gamma[-1] - gamma)
    S_end = Gamma[-1] * S0 + U.T @ (decay_to_end[:, None] * K)
    return O, S_end


def chunked(q, k, v, g, beta, s0=None, cu_seqlens=None, *, scale: float = 1.0, chunk: int = 64):
    """Same arguments and results as oracle.recurrent (all V heads, fp64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    g, beta = _f64(g), _f64(beta)
    T, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    group = Hv // Hqk
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    out = np.zeros((T, Hv, dv))
    fin = np.zeros((N, Hv, dv, dk))
    for n in range(N):
        for h in range(Hv):
            hq = h // group
            S = np.zeros((dv, dk)) if s0 is None else _f64(s0[n, h]).copy()
            for c0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                c1 = min(int(cu[n + 1]), c0 + chunk)
                O, S = chunk_step(S, q[c0:c1, hq], k[c0:c1, hq], v[c0:c1, h], g[c0:c1, h],
                                  beta[c0:c1, h], scale)
                out[c0:c1, h] = O
            fin[n, h] = S
    return out, fin

"""fp64 gradients of the Gated DeltaNet recurrence (TEST INFRASTRUCTURE, like the rest of
oracle/). The forward is the token-by-token rule of recurrent() written with plain PyTorch CPU
ops in float64, and torch.autograd takes its reverse; only small inputs (the loop is over tokens).

For every sequence and V head h (QK head h // (Hv // Hqk)), token by token:
    S = exp(g) S;  S = S + beta (v - S k) k^T;  o = scale S q
Given dO (the gradient of the outputs) and optionally dS_T (of the final states), returns the
gradients of q, k (summed over the V heads that share a QK head), v, g, beta and the initial
states.
"""
from __future__ import annotations

import numpy as np
import torch

from . import upcast


def forward_torch(q, k, v, g, beta, s0, cu, scale):
    """The recurrence on float64 tensors; returns (out [T, Hv, dv], final [N, Hv, dv, dk])."""
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    grp = hv // hqk
    outs = [None] * T
    finals = []
    for n in range(len(cu) - 1):
        S = s0[n].clone()                                  # [Hv, dv, dk]
        for t in range(int(cu[n]), int(cu[n + 1])):
            kt = k[t].repeat_interleave(grp, dim=0)        # [Hv, dk]
            qt = q[t].repeat_interleave(grp, dim=0)
            S = torch.exp(g[t])[:, None, None] * S
            err = v[t] - torch.einsum("hij,hj->hi", S, kt)
            S = S + beta[t][:, None, None] * err[:, :, None] * kt[:, None, :]
            outs[t] = scale * torch.einsum("hij,hj->hi", S, qt)
        finals.append(S)
    out = torch.stack(outs) if T else torch.zeros((0, hv, dv), dtype=torch.float64)
    return out, torch.stack(finals)


def backward(q, k, v, g, beta, s0, cu_seqlens, d_out, d_final=None, *, scale: float = 1.0):
    """fp64 gradients. Inputs as recurrent() takes them (bf16 bits, fp32 or fp64); s0 may be None.
    Returns a dict of numpy float64 arrays: dq, dk [T, Hqk, dk], dv [T, Hv, dv], dg, dbeta [T, Hv],
    ds0 [N, Hv, dv, dk]."""
    T, hqk, dk = np.shape(q)
    hv, dv = np.shape(v)[1], np.shape(v)[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    t64 = lambda a: torch.tensor(upcast(a), dtype=torch.float64, requires_grad=True)
    Q, K, V, G, B = t64(q), t64(k), t64(v), t64(g), t64(beta)
    S0 = t64(np.zeros((N, hv, dv, dk)) if s0 is None else s0)
    out, fin = forward_torch(Q, K, V, G, B, S0, cu, scale)
    loss = (out * torch.tensor(upcast(d_out))).sum()
    if d_final is not None:
        loss = loss + (fin * torch.tensor(upcast(d_final))).sum()
    loss.backward()
    return {"dq": Q.grad.numpy(), "dk": K.grad.numpy(), "dv": V.grad.numpy(), "dg": G.grad.numpy(),
            "dbeta": B.grad.numpy(), "ds0": S0.grad.numpy()}

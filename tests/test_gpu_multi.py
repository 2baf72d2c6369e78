"""Multi-token decode (gdn_decode_multi) against the fp64 oracle: num_tokens
tokens per sequence from one state, the final state, and the state after every
token (the rollback points of draft verification)."""
import numpy as np
import pytest
import torch

import linear_attention_sequence_02_amd as gdn
import oracle
from synth import inputs as I
from tests.gpu_util import log, rel_l2, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}


def _oracle_token_states(x, N, tk):
    """State after token t of every sequence: the oracle run on each sequence's first t + 1 tokens."""
    res = np.zeros((N, tk) + x.s0.shape[1:])
    for t in range(tk):
        rows = (np.arange(N)[:, None] * tk + np.arange(t + 1)[None, :]).ravel()
        cu = (np.arange(N + 1) * (t + 1)).astype(np.int32)
        _, fin = oracle.recurrent(x.q[rows], x.k[rows], x.v[rows], x.g[rows], x.beta[rows], x.s0, cu,
                                  scale=x.scale)
        res[:, t] = fin
    return res


@pytest.mark.parametrize("dtype,d,tk,n", [("bf16", 128, 4, 6), ("fp32", 32, 3, 5), ("bf16", 128, 2, 3)])
def test_decode_multi(dtype, d, tk, n):
    x = I.draw(lengths=[tk] * n, hqk=2, hv=4, dk=d, dtype=dtype, seed=120 + tk, s0_std=0.3,
               name=f"decode_multi_{dtype}_d{d}_k{tk}")
    dev = to_device(x)
    state = dev["s0"].clone()
    log(f"[gpu] gdn_decode_multi {x.name} N={n}")
    out, ts = gdn.gdn_decode_multi(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, tk,
                                   scale=x.scale, token_states=True)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, scale=x.scale)
    o = out.float().cpu().numpy()
    f = state.cpu().numpy()
    ts = ts.cpu().numpy().reshape((n, tk) + f.shape[1:])
    ref_ts = _oracle_token_states(x, n, tk)
    eo, ef, et = rel_l2(o, ref_o), rel_l2(f, ref_f), rel_l2(ts, ref_ts)
    log(f"[parity] {x.name}: out rel={eo:.3e} state rel={ef:.3e} token states rel={et:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype] and et <= TOL[dtype]
    assert np.array_equal(ts[:, -1], f), "the last token state is the final state"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_multi_one_token_is_the_decode_step(dtype):
    """One token per sequence runs the same per-token arithmetic as gdn_decode_step: bit-identical."""
    x = I.draw(lengths=[1] * 7, hqk=2, hv=4, dk=128, dtype=dtype, seed=131, s0_std=0.3, name=f"multi1_{dtype}")
    dev = to_device(x)
    s1, s2 = dev["s0"].clone(), dev["s0"].clone()
    log(f"[gpu] gdn_decode_multi / gdn_decode_step {x.name}")
    o1, _ = gdn.gdn_decode_multi(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], s1, 1, scale=x.scale)
    o2 = gdn.gdn_decode_step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], s2, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_decode_multi_state_pool():
    tk, idx = 3, np.array([4, -1, 1, 7], dtype=np.int32)      # -1 and 7 (>= 6 slots) are padding
    x = I.draw(lengths=[tk] * len(idx), hqk=2, hv=4, dk=128, dtype="bf16", seed=140, name="decode_multi_pool")
    pool0 = I.state_pool(6, 4, 128, seed=141)
    dev = to_device(x)
    pool = torch.from_numpy(pool0).cuda()
    log(f"[gpu] gdn_decode_multi {x.name} on a pool")
    out, _ = gdn.gdn_decode_multi(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool, tk,
                                  state_indices=torch.from_numpy(idx).cuda(), scale=x.scale)
    torch.cuda.synchronize()
    s0 = np.zeros((len(idx),) + pool0.shape[1:])
    for i, s in enumerate(idx):
        if 0 <= s < 6:
            s0[i] = pool0[s]
    ref_o, ref_f = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, s0, x.cu_seqlens, scale=x.scale)
    o = out.float().cpu().numpy()
    p = pool.cpu().numpy()
    for i, s in enumerate(idx):
        rows = slice(i * tk, (i + 1) * tk)
        if 0 <= s < 6:
            e, ef = rel_l2(o[rows], ref_o[rows]), rel_l2(p[s], ref_f[i])
            log(f"[parity] {x.name}: seq {i} -> row {s} out rel={e:.3e} state rel={ef:.3e}")
            assert e <= TOL["bf16"] and ef <= TOL["bf16"]
        else:
            assert np.all(o[rows] == 0.0)
    for r in (0, 2, 3, 5):
        assert np.array_equal(p[r], pool0[r]), f"untouched row {r} changed"

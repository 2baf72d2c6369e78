"""State-pool entry points (gdn_decode_step_slots, gdn_prefill_slots) against the
fp64 oracle, and their replay from a captured HIP graph.

Each sequence reads and writes the pool row its index names; an index outside
the pool is a padding entry. The oracle runs each sequence from the state the
contract gives it (its pool row, or zeros), and every pool row no sequence
names must come back bit for bit unchanged.
"""
import numpy as np
import pytest
import torch

import linear_attention_sequence_02_amd as gdn
import oracle
from synth import inputs as I
from tests.gpu_util import log, rel_l2, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}


def _expected(x, pool, idx, has):
    """Oracle outputs and final states when sequence n starts from pool[idx[n]] (or zeros)."""
    N = len(idx)
    s0 = np.zeros((N,) + pool.shape[1:], dtype=np.float64)
    for n in range(N):
        if 0 <= idx[n] < pool.shape[0] and (has is None or has[n]):
            s0[n] = pool[idx[n]]
    return oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, s0, x.cu_seqlens, scale=x.scale)


def _check_pool(pool0, pool_gpu, idx, ref_fin, tol, name):
    written = {int(s) for s in idx if 0 <= s < pool0.shape[0]}
    for r in range(pool0.shape[0]):
        if r not in written:
            assert np.array_equal(pool_gpu[r], pool0[r]), f"{name}: untouched row {r} changed"
    for n, s in enumerate(idx):
        if 0 <= s < pool0.shape[0]:
            e = rel_l2(pool_gpu[s], ref_fin[n])
            log(f"[parity] {name}: seq {n} -> row {s} state rel={e:.3e}")
            assert e <= tol


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_decode_slots(dtype, d):
    idx = np.array([7, 2, -1, 9, 0, 12], dtype=np.int32)        # -1 and 12 (>= 10 slots) are padding
    x = I.draw(lengths=[1] * len(idx), hqk=2, hv=4, dk=d, dtype=dtype, seed=80 + d, name=f"decode_slots_{dtype}")
    pool0 = I.state_pool(10, 4, d, seed=90 + d)
    dev = to_device(x)
    pool = torch.from_numpy(pool0).cuda()
    ti = torch.from_numpy(idx).cuda()
    log(f"[gpu] gdn_decode_step_slots {x.name}")
    out = gdn.gdn_decode_step_slots(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool, ti, scale=x.scale)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy().astype(np.float64)
    ref_o, ref_f = _expected(x, pool0, idx, None)
    for n, s in enumerate(idx):
        if 0 <= s < 10:
            e = rel_l2(out[n], ref_o[n])
            log(f"[parity] {x.name}: seq {n} out rel={e:.3e}")
            assert e <= TOL[dtype]
        else:
            assert np.all(out[n] == 0.0), "padding entry outputs must be zero"
    _check_pool(pool0, pool.cpu().numpy(), idx, ref_f, TOL[dtype], x.name)


@pytest.mark.parametrize("dtype,d,n", [
    ("bf16", 128, 512),   # 512-thread workgroups: the batch is taken in pool-row order
    ("bf16", 128, 600),   # more sequences than threads: batch order
    ("fp32", 64, 256),    # 256-thread workgroups, at the limit
    ("fp32", 64, 257),
])
def test_decode_slots_row_order(dtype, d, n):
    """A batch in random pool-row order: each workgroup finds its sequence by rank of pool row
    (up to one sequence per thread of a workgroup) or takes them in batch order (beyond). Either
    way every sequence must come out bit for bit as the contiguous step computes it from the
    same state, padding entries give zeros and rows no sequence names stay unchanged."""
    slots = n + 40
    rng = np.random.default_rng(n + d)
    idx = rng.permutation(slots)[:n].astype(np.int32)
    idx[rng.choice(n, size=5, replace=False)] = [-1, slots, -7, slots + 3, -1]   # padding entries
    x = I.draw(lengths=[1] * n, hqk=1, hv=2, dk=d, dtype=dtype, seed=70 + d, name=f"decode_row_order_{dtype}_{n}")
    pool0 = I.state_pool(slots, 2, d, seed=71 + n)
    dev = to_device(x)
    pool = torch.from_numpy(pool0).cuda()
    ti = torch.from_numpy(idx).cuda()
    valid = (idx >= 0) & (idx < slots)
    gathered = np.zeros((n,) + pool0.shape[1:], dtype=np.float32)
    gathered[valid] = pool0[idx[valid]]
    state = torch.from_numpy(gathered).cuda()
    log(f"[gpu] gdn_decode_step_slots {x.name} N={n} slots={slots}")
    out_s = gdn.gdn_decode_step_slots(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool, ti, scale=x.scale)
    out_c = gdn.gdn_decode_step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, scale=x.scale)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    o_s, o_c = out_s.view(bits).cpu().numpy(), out_c.view(bits).cpu().numpy()
    assert np.array_equal(o_s[valid], o_c[valid]), "outputs differ from the contiguous step"
    assert not o_s[~valid].any(), "padding entry outputs must be zero"
    p, st = pool.cpu().numpy(), state.cpu().numpy()
    assert np.array_equal(p[idx[valid]].view(np.int32), st[valid].view(np.int32)), "states differ"
    untouched = np.setdiff1d(np.arange(slots), idx[valid])
    assert np.array_equal(p[untouched].view(np.int32), pool0[untouched].view(np.int32)), "untouched rows changed"


@pytest.mark.parametrize("dtype,lengths", [
    ("bf16", [1100, 33, 700, 5]),     # the first and third sequences span several segments
    ("fp32", [70, 33, 130, 5]),
])
def test_prefill_slots(dtype, lengths):
    idx = np.array([3, -1, 0, 5], dtype=np.int32)
    has = np.array([1, 1, 0, 1], dtype=np.int32)               # sequence 2 starts from zeros
    d = 128 if dtype == "bf16" else 32
    x = I.draw(lengths=lengths, hqk=2, hv=4, dk=d, dtype=dtype, seed=85, name=f"prefill_slots_{dtype}")
    pool0 = I.state_pool(6, 4, d, seed=95)
    dev = to_device(x)
    pool = torch.from_numpy(pool0).cuda()
    log(f"[gpu] gdn_prefill_slots {x.name} T={x.T}")
    out = gdn.gdn_prefill_slots(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool,
                                torch.from_numpy(idx).cuda(), torch.from_numpy(has).cuda(), dev["cu"],
                                scale=x.scale)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy().astype(np.float64)
    ref_o, ref_f = _expected(x, pool0, idx, has)
    e = rel_l2(out, ref_o)
    log(f"[parity] {x.name}: out rel={e:.3e}")
    assert e <= TOL[dtype]
    _check_pool(pool0, pool.cpu().numpy(), idx, ref_f, TOL[dtype], x.name)


def _replays(step, reset, vary, n=3):
    """Capture `step` in a HIP graph, then replay it n times; before each replay the inputs are
    changed (`vary(r)`) and the state reset eagerly, and the replay's results are compared with the
    same step run eagerly on the same inputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(n):
        vary(r)
        reset()
        eager = step(clone=True)
        torch.cuda.synchronize()
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = step(read=True)
        for a, b in zip(eager, got):
            assert torch.equal(a, b), f"replay {r} differs from the eager call"
        log(f"[gpu] graph replay {r}: identical to eager")


def test_decode_slots_graph_replay():
    idx = np.array([5, 1, -1, 3], dtype=np.int32)
    x = I.draw(lengths=[1] * 4, hqk=2, hv=4, dk=128, dtype="bf16", seed=88, name="decode_slots_graph")
    dev = to_device(x)
    pool0 = torch.from_numpy(I.state_pool(8, 4, 128, seed=98)).cuda()
    pool = pool0.clone()
    ti = torch.from_numpy(idx).cuda()
    out = torch.empty_like(dev["v"])
    v0 = dev["v"].clone()

    def step(clone=False, read=False):
        if read:
            return out.clone(), pool.clone()
        gdn.gdn_decode_step_slots(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool, ti, out=out)
        return (out.clone(), pool.clone()) if clone else None

    def reset():
        pool.copy_(pool0)

    def vary(r):
        dev["v"].copy_(torch.roll(v0, shifts=r + 1, dims=0))

    log("[gpu] capture gdn_decode_step_slots")
    _replays(step, reset, vary)


def test_prefill_slots_graph_replay():
    lengths = [700, 40, 300]
    idx = np.array([2, 0, -1], dtype=np.int32)
    x = I.draw(lengths=lengths, hqk=2, hv=4, dk=128, dtype="bf16", seed=89, name="prefill_slots_graph")
    dev = to_device(x)
    pool0 = torch.from_numpy(I.state_pool(4, 4, 128, seed=99)).cuda()
    pool = pool0.clone()
    ti = torch.from_numpy(idx).cuda()
    out = torch.empty_like(dev["v"])
    ws = torch.empty(max(1, gdn.gdn_prefill_workspace_size(x.T, 3, 2, 4, 128, 128, gdn.GDN_BF16)),
                     dtype=torch.uint8, device="cuda")
    v0 = dev["v"].clone()

    def step(clone=False, read=False):
        if read:
            return out.clone(), pool.clone()
        gdn.gdn_prefill_slots(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool, ti, None, dev["cu"],
                              out=out, workspace=ws)
        return (out.clone(), pool.clone()) if clone else None

    def reset():
        pool.copy_(pool0)

    def vary(r):
        dev["v"].copy_(v0 * (1.0 + 0.25 * r))

    log("[gpu] capture gdn_prefill_slots")
    _replays(step, reset, vary)

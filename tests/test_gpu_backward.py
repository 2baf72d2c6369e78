"""Backward of the prefill (gdn_backward) against the fp64 oracle's gradients (PyTorch CPU
autograd of the recurrence, itself pinned by finite differences). The GPU computes the gradients
in fp32 from inputs that are exact in fp32 (bf16 inputs widen exactly), so every gradient is held
to the fp32 bar, relative L2 <= 1e-4 per tensor."""
import numpy as np
import pytest
import torch

import linear_attention_sequence_02_amd as gdn
import oracle
from synth import inputs as I
from tests.gpu_util import log, rel_l2, to_device

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.mark.parametrize("dtype,d,lengths,with_dfinal", [
    ("fp32", 16, [37, 0, 70, 16], True),
    ("fp32", 32, [50, 19], False),
    ("fp32", 64, [33, 48], True),
    ("bf16", 128, [45, 20], True),
    ("bf16", 128, [81], False),
])
def test_backward(dtype, d, lengths, with_dfinal):
    x = I.draw(lengths=lengths, hqk=1 if d == 128 else 2, hv=2 if d == 128 else 4, dk=d, dtype=dtype,
               seed=400 + d + len(lengths), s0_std=0.3, scale=0.5, name=f"backward_{dtype}_d{d}")
    rng = np.random.default_rng(401 + d)
    d_out = rng.standard_normal(x.v.shape).astype(np.float32)
    d_fin = rng.standard_normal(x.s0.shape).astype(np.float32) if with_dfinal else None
    if dtype == "bf16":   # d_out in the inputs' dtype: round to bf16 bits
        d_out_in = I.f32_to_bf16_bits(d_out)
        d_out = oracle.upcast(d_out_in)
        dev_dout = torch.from_numpy(d_out_in).view(torch.bfloat16).cuda()
    else:
        dev_dout = torch.from_numpy(d_out).cuda()
    dev = to_device(x)
    log(f"[gpu] gdn_backward {x.name} T={x.T} lengths={lengths}")
    res = gdn.gdn_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev_dout, dev["s0"], dev["cu"],
                           None if d_fin is None else torch.from_numpy(d_fin).cuda(), scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.backward(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, d_out, d_fin, scale=x.scale)
    pairs = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"), ("d_initial_state", "ds0")]
    for mine, theirs in pairs:
        e = rel_l2(res[mine].cpu().numpy(), ref[theirs])
        log(f"[parity] {x.name} {mine}: rel={e:.3e}")
        assert e <= TOL, (mine, e)


def test_backward_layer_heads():
    """The layer's own head layout (16 QK heads shared by 32 V heads, d = 128, scale 1/sqrt(d)),
    two ragged sequences with initial states and a final-state gradient: 32 chunks of 16 tokens
    over the scans, the per-chunk gradients and the sums over the V heads of each QK head."""
    lengths = [300, 212]
    x = I.draw(lengths=lengths, hqk=16, hv=32, dk=128, dtype="bf16", seed=431, s0_std=0.1,
               scale=128 ** -0.5, name="backward_layer_heads")
    rng = np.random.default_rng(432)
    d_out_in = I.f32_to_bf16_bits(rng.standard_normal(x.v.shape).astype(np.float32))
    d_out = oracle.upcast(d_out_in)
    d_fin = rng.standard_normal(x.s0.shape).astype(np.float32)
    dev = to_device(x)
    log(f"[gpu] gdn_backward {x.name} T={x.T} lengths={lengths} heads 16/32")
    res = gdn.gdn_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                           torch.from_numpy(d_out_in).view(torch.bfloat16).cuda(), dev["s0"], dev["cu"],
                           torch.from_numpy(d_fin).cuda(), scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.backward(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, d_out, d_fin, scale=x.scale)
    for mine, theirs in [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
                         ("d_initial_state", "ds0")]:
        e = rel_l2(res[mine].cpu().numpy(), ref[theirs])
        log(f"[parity] {x.name} {mine}: rel={e:.3e}")
        assert e <= TOL, (mine, e)


def test_backward_layer_T4096_sampled_head():
    """The timed backward workload itself (T = 4096, 16 QK / 32 V heads, bf16, zero initial state,
    d_out the values drawn with seed 1007) in its own launch configuration; the oracle recomputes
    QK head 5 and its two V heads (heads are independent: a QK head's gradient depends only on the
    V heads that share it)."""
    x = I.qwen3_next_prefill(T=4096)
    d_out_in = I.draw(T=4096, hqk=x.hqk, hv=x.hv, dk=x.dk, seed=1007).v
    dev = to_device(x)
    log(f"[gpu] gdn_backward {x.name} T={x.T} heads 16/32")
    res = gdn.gdn_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                           torch.from_numpy(d_out_in).view(torch.bfloat16).cuda(), None, None, scale=x.scale)
    torch.cuda.synchronize()
    hq, hv = 5, slice(10, 12)
    ref = oracle.backward(x.q[:, hq:hq + 1], x.k[:, hq:hq + 1], x.v[:, hv], x.g[:, hv], x.beta[:, hv], None, None,
                          oracle.upcast(d_out_in)[:, hv], None, scale=x.scale)
    mine = {"dq": res["dq"][:, hq:hq + 1], "dk": res["dk"][:, hq:hq + 1], "dv": res["dv"][:, hv],
            "dg": res["dg"][:, hv], "dbeta": res["dbeta"][:, hv], "ds0": res["d_initial_state"][:, hv]}
    for name, t in mine.items():
        e = rel_l2(t.cpu().numpy(), ref[name])
        log(f"[parity] {x.name} {name}: rel={e:.3e}")
        assert e <= TOL, (name, e)


def test_backward_no_tokens():
    """No tokens in any sequence: the gradient of each initial state is the gradient of its final
    state (the recurrence is the identity), and the token gradients are empty."""
    n, hqk, hv, d = 3, 1, 2, 32
    rng = np.random.default_rng(441)
    d_fin = torch.from_numpy(rng.standard_normal((n, hv, d, d)).astype(np.float32)).cuda()
    s0 = torch.from_numpy(rng.standard_normal((n, hv, d, d)).astype(np.float32)).cuda()
    z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device="cuda")
    cu = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    log("[gpu] gdn_backward no tokens, 3 sequences")
    res = gdn.gdn_backward(z(0, hqk, d), z(0, hqk, d), z(0, hv, d), z(0, hv), z(0, hv), z(0, hv, d), s0, cu, d_fin)
    torch.cuda.synchronize()
    assert torch.equal(res["d_initial_state"], d_fin)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert res[name].shape[0] == 0


@pytest.mark.parametrize("hqk,hv", [(16, 32), (4, 12)])
def test_backward_unaligned_dq_dk(hqk, hv):
    """dq and dk at addresses that are not 16-byte aligned give the same bits as aligned outputs
    (d = 128, a ragged length). With two V heads per QK head (the layer's 16 / 32) both add their
    shares into the output; with three (4 / 12) the shares are summed by the one-element-per-thread
    launch, in the same order as the 16-byte one."""
    x = I.draw(lengths=[150], hqk=hqk, hv=hv, dk=128, dtype="bf16", seed=451, s0_std=0.1,
               scale=128 ** -0.5, name=f"backward_unaligned_{hqk}_{hv}")
    rng = np.random.default_rng(452)
    dev = to_device(x)
    d_out = torch.from_numpy(I.f32_to_bf16_bits(rng.standard_normal(x.v.shape).astype(np.float32))).view(
        torch.bfloat16).cuda()
    log(f"[gpu] gdn_backward {x.name} T={x.T}, aligned reference")
    ref = gdn.gdn_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], d_out, dev["s0"], dev["cu"],
                           scale=x.scale)
    T, hqk, hv, d = x.T, x.hqk, x.hv, x.dk
    f32 = dict(dtype=torch.float32, device="cuda")
    dq_buf = torch.full((T * hqk * d + 1,), float("nan"), **f32)
    dk_buf = torch.full((T * hqk * d + 1,), float("nan"), **f32)
    dv, dg, dbeta = torch.empty((T, hv, d), **f32), torch.empty((T, hv), **f32), torch.empty((T, hv), **f32)
    ds0 = torch.empty((1, hv, d, d), **f32)
    need = gdn.gdn_backward_workspace_size(T, 1, hqk, hv, d, d, gdn.GDN_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    p = lambda t: t.data_ptr()
    log(f"[gpu] gdn_backward {x.name}: dq, dk 4 bytes past 16-byte alignment")
    st = gdn._load().gdn_backward(p(dev["q"]), p(dev["k"]), p(dev["v"]), p(dev["g"]), p(dev["beta"]), p(dev["s0"]),
                                  p(dev["cu"]), 1, T, hqk, hv, d, d, float(x.scale), gdn.GDN_BF16, p(d_out), None,
                                  p(dq_buf) + 4, p(dk_buf) + 4, p(dv), p(dg), p(dbeta), p(ds0), p(ws), need,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == gdn.GDN_OK
    assert p(dq_buf) % 16 == 0   # so that + 4 bytes is not 16-byte aligned
    assert torch.equal(dq_buf[1:].view(T, hqk, d), ref["dq"])
    assert torch.equal(dk_buf[1:].view(T, hqk, d), ref["dk"])
    assert torch.equal(dv, ref["dv"]) and torch.equal(dg, ref["dg"]) and torch.equal(dbeta, ref["dbeta"])


@pytest.mark.parametrize("dtype,d,hqk,hv", [
    ("fp32", 32, 2, 2),     # one V head per QK head: dq, dk stored directly
    ("fp32", 32, 1, 3),     # three: shares summed in a fixed order by a last launch
    ("bf16", 128, 2, 4),    # two: both shares added into the zeroed output
])
def test_backward_head_groups(dtype, d, hqk, hv):
    """Each way of forming dq and dk from the V heads that share a QK head, against the oracle."""
    lengths = [70, 0, 33]
    x = I.draw(lengths=lengths, hqk=hqk, hv=hv, dk=d, dtype=dtype, seed=460 + hv, s0_std=0.3, scale=0.5,
               name=f"backward_groups_{hqk}_{hv}")
    rng = np.random.default_rng(461 + hv)
    d_out = rng.standard_normal(x.v.shape).astype(np.float32)
    d_fin = rng.standard_normal(x.s0.shape).astype(np.float32)
    if dtype == "bf16":
        d_out_in = I.f32_to_bf16_bits(d_out)
        d_out = oracle.upcast(d_out_in)
        dev_dout = torch.from_numpy(d_out_in).view(torch.bfloat16).cuda()
    else:
        dev_dout = torch.from_numpy(d_out).cuda()
    dev = to_device(x)
    log(f"[gpu] gdn_backward {x.name} T={x.T} heads {hqk}/{hv}")
    res = gdn.gdn_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev_dout, dev["s0"], dev["cu"],
                           torch.from_numpy(d_fin).cuda(), scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.backward(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, d_out, d_fin, scale=x.scale)
    for mine, theirs in [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
                         ("d_initial_state", "ds0")]:
        e = rel_l2(res[mine].cpu().numpy(), ref[theirs])
        log(f"[parity] {x.name} {mine}: rel={e:.3e}")
        assert e <= TOL, (mine, e)


def test_backward_deterministic():
    """Three calls on the layer's head layout (two V heads add into each QK head's dq, dk) give the
    same bits."""
    x = I.draw(lengths=[700, 333], hqk=16, hv=32, dk=128, dtype="bf16", seed=471, s0_std=0.1,
               scale=128 ** -0.5, name="backward_deterministic")
    rng = np.random.default_rng(472)
    d_out = torch.from_numpy(I.f32_to_bf16_bits(rng.standard_normal(x.v.shape).astype(np.float32))).view(
        torch.bfloat16).cuda()
    dev = to_device(x)
    log(f"[gpu] gdn_backward {x.name} T={x.T}, three calls")
    runs = [gdn.gdn_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], d_out, dev["s0"], dev["cu"],
                             scale=x.scale) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for name in ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state"):
            assert torch.equal(r[name], runs[0][name]), name

"""GPU path against the fp64 oracle on identical seeded inputs.

Tolerances are the layer's parity bar: relative L2 <= 1e-2 for bf16 inputs
and <= 1e-4 in the fp32-input mode, for outputs and final states, over the
whole tensor; the worst (sequence, V head) slice is checked too so that an
error confined to one short sequence cannot hide in the global norm.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import inputs as I
from tests.gpu_util import log, per_seq_head_rel, per_state_rel, rel_l2, run_prefill, to_device

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_FP32 = 1e-4
# The worst single (sequence, V head) slice is held to the same bar as the whole tensor, so that an
# error confined to one short sequence or one head cannot hide in the global norm.
TOL_BF16_SLICE = TOL_BF16


def _oracle(x, heads=None):
    return oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, scale=x.scale, heads=heads)


def _check(x, out, fin, tol, slice_tol=None, heads=None):
    ref_o, ref_f = _oracle(x, heads)
    if heads is not None:
        out = out[:, heads[0]:heads[1]]
        fin = fin[:, heads[0]:heads[1]]
    eo, ef = rel_l2(out, ref_o), rel_l2(fin, ref_f)
    so = per_seq_head_rel(out, ref_o, x.cu_seqlens)
    sf = per_state_rel(fin, ref_f)
    log(f"[parity] {x.name}: out rel={eo:.3e} (worst slice {so:.3e})  state rel={ef:.3e} (worst {sf:.3e})")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))
    assert eo <= tol and ef <= tol
    st = tol if slice_tol is None else slice_tol
    assert so <= st and sf <= st


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("dtype,d,n", [("bf16", 128, 256), ("fp32", 128, 7), ("fp32", 64, 5),
                                       ("fp32", 32, 3), ("fp32", 16, 9), ("bf16", 16, 4)])
def test_decode_step(dtype, d, n):
    x = I.draw(lengths=[1] * n, hqk=16 if d == 128 else 2, hv=32 if d == 128 else 4, dk=d, dtype=dtype,
               seed=1003 if n == 256 else 50 + d, s0_std=0.01 if n == 256 else 0.3,
               name=f"decode_{dtype}_d{d}_N{n}")
    dev = to_device(x)
    state = dev["s0"].clone()
    log(f"[gpu] gdn_decode_step {x.name}")
    import linear_attention_sequence_02_amd as gdn
    out = gdn.gdn_decode_step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, scale=x.scale)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_FP32
    _check(x, out.float().cpu().numpy().astype(np.float64), state.cpu().numpy().astype(np.float64), tol)


def test_decode_step_state_past_4gib():
    """2,048 sequences x 32 V heads x 128 x 128 fp32 = 4 GiB of state, so the last sequences'
    states start past byte offset 2^32; sampled sequences from both ends are checked against the
    oracle."""
    import linear_attention_sequence_02_amd as gdn
    n = 2048
    x = I.draw(lengths=[1] * n, hqk=16, hv=32, dk=128, dtype="bf16", seed=1010, name="decode_bf16_N2048")
    s0 = I.large_state(n, 32, 128, seed=1011)
    dev = to_device(x)
    state = torch.from_numpy(s0).cuda()
    log(f"[gpu] gdn_decode_step {x.name} state {state.numel() * 4 / 2**30:.1f} GiB")
    out = gdn.gdn_decode_step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, scale=x.scale)
    torch.cuda.synchronize()
    pick = [0, 1, 1023, 1024, 2046, 2047]
    ref_o, ref_f = oracle.recurrent(x.q[pick], x.k[pick], x.v[pick], x.g[pick], x.beta[pick], s0[pick],
                                    np.arange(len(pick) + 1, dtype=np.int32), scale=x.scale)
    idx = torch.tensor(pick, device="cuda")
    got_o = out.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    got_f = state.index_select(0, idx).cpu().numpy().astype(np.float64)
    eo, ef = rel_l2(got_o, ref_o), rel_l2(got_f, ref_f)
    log(f"[parity] {x.name} sequences {pick}: out rel={eo:.3e} state rel={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_group3(dtype):
    """d = 128 decode with three V heads sharing one QK head, 5 sequences (an odd head count
    and a grouping the Qwen3-Next shape does not use)."""
    x = I.draw(lengths=[1] * 5, hqk=1, hv=3, dk=128, dtype=dtype, seed=71, s0_std=0.3,
               name=f"decode_{dtype}_d128_items15")
    dev = to_device(x)
    state = dev["s0"].clone()
    log(f"[gpu] gdn_decode_step {x.name}")
    import linear_attention_sequence_02_amd as gdn
    out = gdn.gdn_decode_step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, scale=x.scale)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_FP32
    _check(x, out.float().cpu().numpy().astype(np.float64), state.cpu().numpy().astype(np.float64), tol)


# ---------------------------------------------------------------- fp32-input prefill

def test_prefill_fp32_tiny():
    x = I.tiny()
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_FP32)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_prefill_fp32_varlen_shapes(d):
    x = I.draw(lengths=[1, 63, 64, 65, 0, 130, 200], hqk=2, hv=4, dk=d, dtype="fp32", seed=60 + d,
               s0_std=0.3, name=f"fp32_varlen_d{d}")
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_FP32)


def test_prefill_fp32_qwen_shape():
    x = I.qwen3_next_prefill(T=1000, dtype="fp32", seed=71)
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_FP32)


def test_prefill_fp32_long_layer():
    # 16,384 tokens on the layer's head shape in the fp32 mode: 256 chunks of accumulated state,
    # still held to the 1e-4 bar.
    x = I.qwen3_next_prefill(T=16384, dtype="fp32", seed=72)
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_FP32)


# ---------------------------------------------------------------- bf16 MFMA prefill

def test_prefill_bf16_small_varlen():
    x = I.draw(lengths=[1, 63, 64, 65, 0, 200, 17, 128], hqk=2, hv=4, dk=128, dtype="bf16", seed=80,
               s0_std=0.3, name="bf16_small_varlen")
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


def test_prefill_bf16_many_short_sequences():
    # 24 sequences x 32 heads = 768 (sequence, head) pairs: the whole-head chain kernel.
    lengths = [1, 5, 63, 64, 65, 0, 128, 300, 17, 200, 129, 2, 90, 64, 191, 40, 3, 77, 256, 1, 33, 100, 12, 70]
    x = I.draw(lengths=lengths, hqk=16, hv=32, dk=128, dtype="bf16", seed=88, s0_std=0.1, name="bf16_many_short")
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


def test_prefill_bf16_thousand_tiny_sequences():
    # 1,000 sequences of 0-130 tokens (empty, single-token and chunk-boundary lengths among them),
    # with initial states: the segment slot indexing and the many-chain launch at scale.
    lengths = [int(x) for x in np.random.default_rng(89).integers(0, 131, size=1000)]
    lengths[:6] = [0, 1, 63, 64, 65, 128]
    x = I.draw(lengths=lengths, hqk=2, hv=4, dk=128, dtype="bf16", seed=89, s0_std=0.1, name="bf16_1000_tiny")
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


def test_prefill_states_past_4gib():
    """2,048 sequences (mostly one token; the last two 130 and 64 tokens) with 4 GiB of initial and
    4 GiB of final states: the far sequences' states sit past byte offset 2^32. Sampled sequences
    from both ends against the oracle."""
    import linear_attention_sequence_02_amd as gdn
    n = 2048
    lengths = [1] * n
    lengths[0], lengths[-2], lengths[-1] = 70, 130, 64
    x = I.draw(lengths=lengths, hqk=16, hv=32, dk=128, dtype="bf16", seed=1012, name="prefill_bf16_N2048")
    s0 = I.large_state(n, 32, 128, seed=1013)
    dev = to_device(x)
    log(f"[gpu] gdn_prefill {x.name} T={x.T} initial and final states 4.0 GiB each")
    out, fin = gdn.gdn_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], torch.from_numpy(s0).cuda(),
                               dev["cu"], scale=x.scale)
    torch.cuda.synchronize()
    cu = x.cu_seqlens
    pick = [0, 1, 1024, 2046, 2047]
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in pick])
    sub_cu = np.concatenate([[0], np.cumsum([cu[i + 1] - cu[i] for i in pick])]).astype(np.int32)
    ref_o, ref_f = oracle.recurrent(x.q[rows], x.k[rows], x.v[rows], x.g[rows], x.beta[rows], s0[pick], sub_cu,
                                    scale=x.scale)
    got_o = out.index_select(0, torch.from_numpy(rows).cuda()).float().cpu().numpy().astype(np.float64)
    got_f = fin.index_select(0, torch.tensor(pick, device="cuda")).cpu().numpy().astype(np.float64)
    eo, ef = rel_l2(got_o, ref_o), rel_l2(got_f, ref_f)
    log(f"[parity] {x.name} sequences {pick}: out rel={eo:.3e} state rel={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16


def test_prefill_bf16_qwen_layer_T4096():
    x = I.qwen3_next_prefill(T=4096)
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


def test_prefill_bf16_qwen_layer_T65536():
    # The timed prefill workload itself (same seed, same launches: 114-chunk segments, 9 per head);
    # the C oracle covers all 65,536 tokens of every head in a few seconds.
    x = I.qwen3_next_prefill(T=65536)
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


def test_prefill_bf16_tp4_share():
    # One GPU's share at tensor parallelism 4 (4 QK / 8 V heads, the full 65,536 tokens): with
    # fewer heads the segment rule picks 32-chunk segments, 33 per head.
    x = I.tp_share_prefill()
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


def test_prefill_bf16_varlen8():
    x = I.varlen_prefill()
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


def _check_by_head_groups(x, out, fin, tol, group=16):
    """Whole-tensor and per-(sequence, V head) rel-L2 of device results against the oracle, run on
    `group` V heads at a time: the sums of squared differences and of squared reference values are
    accumulated over the groups, so the whole-tensor figure is exact without holding the fp64
    reference of every head at once."""
    num_o = den_o = num_f = den_f = 0.0
    worst_o = worst_f = 0.0
    cu = x.cu_seqlens
    for h0 in range(0, x.hv, group):
        h1 = min(x.hv, h0 + group)
        log(f"[oracle] {x.name}: V heads {h0}..{h1 - 1}")
        ref_o, ref_f = _oracle(x, heads=(h0, h1))
        got_o = out[:, h0:h1].float().cpu().numpy().astype(np.float64)
        got_f = fin[:, h0:h1].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_f))
        do = got_o - ref_o
        df = got_f - ref_f
        num_o += float(np.sum(do * do))
        den_o += float(np.sum(ref_o * ref_o))
        num_f += float(np.sum(df * df))
        den_f += float(np.sum(ref_f * ref_f))
        worst_o = max(worst_o, per_seq_head_rel(got_o, ref_o, cu))
        worst_f = max(worst_f, per_state_rel(got_f, ref_f))
        del ref_o, ref_f, got_o, got_f, do, df
    eo, ef = math.sqrt(num_o / den_o), math.sqrt(num_f / den_f)
    log(f"[parity] {x.name}: out rel={eo:.3e} (worst slice {worst_o:.3e})  state rel={ef:.3e} "
        f"(worst {worst_f:.3e})")
    assert eo <= tol and ef <= tol
    assert worst_o <= TOL_BF16_SLICE and worst_f <= TOL_BF16_SLICE


def _run_prefill_device(x):
    import linear_attention_sequence_02_amd as gdn
    d = to_device(x)
    log(f"[gpu] gdn_prefill {x.name} T={x.T} N={x.num_seqs} Hqk={x.hqk} Hv={x.hv} d={x.dk} {x.dtype}")
    out, fin = gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["cu"], scale=x.scale)
    torch.cuda.synchronize()
    del d
    return out, fin


def test_prefill_bf16_long_context():
    # T = 262144 in the launch configuration of the full layer, compared with the oracle on every
    # V head (in two groups of 16 heads).
    x = I.long_context()
    log(f"[case] long context mean alpha={x.meta['mean_alpha']:.4f}")
    out, fin = _run_prefill_device(x)
    _check_by_head_groups(x, out, fin, TOL_BF16)


# Bound for the bf16 path on the near-parallel-key case below, which the 1e-2 parity bar of the
# five workloads does not cover: with every key of a head within about 0.05 of one direction,
# beta = 0.999 and alpha = exp(-1e-3), the chunk quantities built from the key Gram (the masked
# Gram A with entries near 1, the block inverses, the delta writes U and their decayed copies) are
# sums of near-unit terms that telescope, and rounding each such MFMA operand to bf16 (2^-9 of an
# entry near 1) leaves errors of about 1% in out and 2% in the final state. A host emulation of the
# kernel's roundings reproduces the figures and attributes them to those operands, not to a defect
# of the algebra (the same emulation without the roundings agrees with the oracle to 1e-14). The
# fp32 mode meets the 1e-4 bar on the same inputs.
TOL_BF16_NEAR_PARALLEL = 3e-2


def test_prefill_bf16_near_parallel_keys():
    # The chunk solve near its worst conditioning: every key of a QK head within about 0.05 of one
    # direction (the masked key Gram close to all ones), beta = 0.999 and alpha = exp(-1e-3), so
    # (I + A) is close to the lower triangle of ones and each write nearly cancels the previous one.
    # The layer's head shape at T = 4096 runs 8 segments of 8 chunks, so the segment maps and the
    # combine see the same inputs.
    x = I.draw(T=4096, hqk=16, hv=32, dk=128, dtype="bf16", seed=1020, k_spread=0.05, fixed_beta=0.999,
               fixed_g=-1e-3, s0_std=0.1, name="bf16_near_parallel_keys_T4096")
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16_NEAR_PARALLEL, TOL_BF16_NEAR_PARALLEL)


def test_prefill_fp32_near_parallel_keys():
    # The same inputs (bf16 values widened exactly to fp32) through the fp32 mode, at its 1e-4 bar.
    x = I.draw(T=4096, hqk=16, hv=32, dk=128, dtype="bf16", seed=1020, k_spread=0.05, fixed_beta=0.999,
               fixed_g=-1e-3, s0_std=0.1, name="fp32_near_parallel_keys_T4096")
    x = I.GdnInputs(q=I.bf16_bits_to_f32(x.q), k=I.bf16_bits_to_f32(x.k), v=I.bf16_bits_to_f32(x.v), g=x.g,
                    beta=x.beta, s0=x.s0, cu_seqlens=x.cu_seqlens, dtype="fp32", scale=x.scale, name=x.name,
                    seed=x.seed, meta=x.meta)
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_FP32)


@pytest.mark.parametrize("g,beta", [(-1e-3, None), (-1e-4, 0.02)], ids=["g1e-3", "g1e-4_beta0.02"])
def test_prefill_bf16_full_scale_carry(g, beta):
    # The timed workload's launch configuration (T = 65536, 16/32 heads, 9 segments of 114 chunks)
    # with slow decay and initial states, so the state carried across segment boundaries (the
    # bf16-built segment maps composed by the combine) decides the result. With g = -1e-4 and
    # beta = 0.02 the map of one segment keeps a norm of order 0.1.
    x = I.draw(T=65536, hqk=16, hv=32, dk=128, dtype="bf16", seed=1021, fixed_g=g, fixed_beta=beta,
               s0_std=0.5, name=f"bf16_carry_T65536_g{g:g}")
    out, fin = _run_prefill_device(x)
    _check_by_head_groups(x, out, fin, TOL_BF16, group=32)


def test_prefill_bf16_scale_argument():
    x = I.draw(lengths=[300], hqk=2, hv=4, dk=128, dtype="bf16", seed=81, s0_std=0.1,
               scale=1.0 / math.sqrt(128.0), name="bf16_scale")
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16, TOL_BF16_SLICE)


# Carry-sensitive cases: with the default decay (mean alpha 0.5) the state
# forgets a chunk within a few tokens, so a broken carry between chunks or a
# wrong initial state could still pass; these keep the carry alive.

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_long_carry_no_decay(dtype):
    x = I.draw(lengths=[1000, 517], hqk=2, hv=4, dk=128, dtype=dtype, seed=82, s0_std=0.5,
               fixed_g=0.0, fixed_beta=0.05, name=f"{dtype}_no_decay_small_beta")
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16 if dtype == "bf16" else TOL_FP32, TOL_BF16_SLICE if dtype == "bf16" else None)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_degenerate_gates_and_boundaries(dtype):
    """The gates at their limits and lengths at the chunk and segment boundaries, against the oracle:
    stretches of tokens with g = -30 (alpha = 9e-14: the state is all but reset at every token),
    g = 0 (no decay), beta = 0 (no write), beta = 1 (full replacement along the key), zero keys and
    zero queries; sequence lengths 64, 1, 63, 65, 512 (one whole segment of 8 chunks here), 513,
    1024 and 0, with initial states."""
    lengths = [64, 1, 63, 65, 512, 513, 1024, 0]
    x = I.draw(lengths=lengths, hqk=2, hv=4, dk=128, dtype=dtype, seed=91, s0_std=0.3,
               name=f"{dtype}_degenerate_gates")
    T = x.T
    t = np.arange(T)
    x.g[(t % 97) < 9] = -30.0
    x.g[(t % 89) > 79] = 0.0
    x.beta[(t % 83) < 7] = 0.0
    x.beta[(t % 79) > 70] = 1.0
    x.k[(t % 101) < 3] = 0
    x.q[(t % 103) < 3] = 0
    assert T == sum(lengths)
    out, fin = run_prefill(x)
    _check(x, out, fin, TOL_BF16 if dtype == "bf16" else TOL_FP32, TOL_BF16_SLICE if dtype == "bf16" else None)


def test_prefill_bf16_pure_decay_closed_form():
    # beta = 0: o_t = exp(sum_{s<=t} g_s) S0 q_t, S_T = exp(sum g) S0 (no oracle involved).
    x = I.draw(lengths=[333], hqk=1, hv=2, dk=128, dtype="bf16", seed=83, s0_std=1.0, g_mean=-6.0,
               fixed_beta=0.0, name="bf16_pure_decay")
    out, fin = run_prefill(x)
    qf = I.bf16_bits_to_f32(x.q).astype(np.float64)
    decay = np.exp(np.cumsum(x.g.astype(np.float64), axis=0))
    s0 = x.s0.astype(np.float64)
    exp_out = np.stack([decay[:, h, None] * (qf[:, 0] @ s0[0, h].T) for h in range(2)], axis=1)
    exp_fin = decay[-1][None, :, None, None] * s0
    log(f"[parity] pure decay: out {rel_l2(out, exp_out):.3e} state {rel_l2(fin, exp_fin):.3e}")
    assert rel_l2(out, exp_out) <= TOL_BF16 and rel_l2(fin, exp_fin) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_resume_split(dtype):
    # [0, T) in one call equals [0, T1) then [T1, T) from the saved state, T1 not a multiple of 64.
    x = I.draw(lengths=[900], hqk=2, hv=4, dk=128, dtype=dtype, seed=84, s0_std=0.2, g_mean=-3.0,
               name=f"{dtype}_resume")
    out, fin = run_prefill(x)
    T1 = 397
    xa = I.GdnInputs(q=x.q[:T1], k=x.k[:T1], v=x.v[:T1], g=x.g[:T1], beta=x.beta[:T1], s0=x.s0,
                     cu_seqlens=np.array([0, T1], np.int32), dtype=dtype, scale=1.0, name="resume_a",
                     seed=0, meta={})
    oa, fa = run_prefill(xa)
    xb = I.GdnInputs(q=x.q[T1:], k=x.k[T1:], v=x.v[T1:], g=x.g[T1:], beta=x.beta[T1:],
                     s0=fa.astype(np.float32), cu_seqlens=np.array([0, 900 - T1], np.int32), dtype=dtype,
                     scale=1.0, name="resume_b", seed=0, meta={})
    ob, fb = run_prefill(xb)
    tol = TOL_BF16 if dtype == "bf16" else TOL_FP32
    ref_o, ref_f = _oracle(x)
    split_o = np.concatenate([oa, ob])
    log(f"[parity] resume {dtype}: split vs oracle out {rel_l2(split_o, ref_o):.3e} state {rel_l2(fb, ref_f):.3e}")
    assert rel_l2(split_o, ref_o) <= tol and rel_l2(fb, ref_f) <= tol
    assert rel_l2(split_o, out) <= tol and rel_l2(fb, fin) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_steps_equal_prefill(dtype):
    import linear_attention_sequence_02_amd as gdn
    T = 12
    x = I.draw(lengths=[T], hqk=2, hv=4, dk=128, dtype=dtype, seed=85, s0_std=0.3, g_mean=-2.0,
               name=f"{dtype}_decode_chain")
    d = to_device(x)
    state = d["s0"].clone()
    outs = []
    log(f"[gpu] {T} chained decode steps {dtype}")
    for t in range(T):
        o = gdn.gdn_decode_step(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1], d["g"][t:t + 1],
                                d["beta"][t:t + 1], state)
        outs.append(o.float().cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    ref_o, ref_f = _oracle(x)
    tol = TOL_BF16 if dtype == "bf16" else TOL_FP32
    assert rel_l2(np.concatenate(outs), ref_o) <= tol
    assert rel_l2(state.cpu().numpy(), ref_f) <= tol


def test_prefill_final_state_aliases_initial_state():
    import linear_attention_sequence_02_amd as gdn
    x = I.draw(lengths=[100, 0, 70], hqk=2, hv=4, dk=128, dtype="bf16", seed=86, s0_std=0.2,
               name="bf16_alias")
    d = to_device(x)
    st = d["s0"].clone()
    log("[gpu] prefill with final_state == initial_state")
    out, fin = gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu"], final_state=st)
    torch.cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    ref_o, ref_f = _oracle(x)
    assert rel_l2(out.float().cpu().numpy(), ref_o) <= TOL_BF16
    assert rel_l2(st.cpu().numpy(), ref_f) <= TOL_BF16
    assert np.array_equal(st[1].cpu().numpy(), x.s0[1])   # the empty sequence keeps its state exactly


def test_prefill_no_tokens_copies_states():
    import linear_attention_sequence_02_amd as gdn
    dev = "cuda"
    s0 = torch.randn(3, 4, 128, 128, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    e = torch.empty(0, 2, 128, dtype=torch.bfloat16, device=dev)
    ev = torch.empty(0, 4, 128, dtype=torch.bfloat16, device=dev)
    eg = torch.empty(0, 4, dtype=torch.float32, device=dev)
    log("[gpu] prefill with zero tokens")
    out, fin = gdn.gdn_prefill(e, e, ev, eg, eg, s0, cu)
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 128) and torch.equal(fin, s0)


def test_prefill_deterministic():
    x = I.draw(lengths=[500, 300], hqk=2, hv=4, dk=128, dtype="bf16", seed=87, s0_std=0.1, name="bf16_det")
    o1, f1 = run_prefill(x)
    o2, f2 = run_prefill(x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)

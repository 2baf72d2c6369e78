"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module only draws random tensors with the shapes and distributions of the
Qwen3-Next Gated DeltaNet layer (page "Qwen3-Next-80B-A3B-Instruct" model card,
section "Model Overview": 16 QK heads, 32 V heads, head dimension 128) and
packs them the way the library and the fp64 oracle both take them. It holds
none of the recurrence's arithmetic; both the GPU path and the oracle read the
arrays it returns.

Conventions shared with the library's C header:
  q, k  [T, Hqk, d]  bf16 (stored as uint16 bit patterns) or fp32
  v     [T, Hv, d]   same dtype as q, k
  g     [T, Hv]      fp32, log of the decay alpha (g <= 0)
  beta  [T, Hv]      fp32 in (0, 1)
  s0    [N, Hv, d, d] fp32, element [i][j] = value index i, key index j
  cu    [N + 1]      int32 token offsets of the packed sequences

q and k are L2-normalised per token per head in fp64 before the cast to the
storage dtype: the normalisation is a precondition of the layer, done by its
caller, so neither side renormalises. For the library's in-kernel
normalisation mode, draw(qk_unit=False) returns q and k rows of varied length
instead (N(0, 1) times 10^U(-1, 1) per row).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

QWEN3_NEXT_HQK = 16
QWEN3_NEXT_HV = 32
QWEN3_NEXT_D = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


_BLOCK = 8192


def _block_rng(seed: int, stream: int, block: int) -> np.random.Generator:
    # One child generator per (tensor, token block): the values do not depend on
    # how many threads fill the blocks.
    return np.random.default_rng([int(seed), int(stream), int(block)])


def _fill_blocks(shape, fn, workers: int | None = None) -> np.ndarray:
    T = shape[0]
    out = np.empty(shape, dtype=np.float32)
    blocks = list(range(0, T, _BLOCK))
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))

    def work(t0):
        t1 = min(T, t0 + _BLOCK)
        out[t0:t1] = fn(t0 // _BLOCK, (t1 - t0,) + tuple(shape[1:]))

    if len(blocks) <= 1 or workers == 1:
        for t0 in blocks:
            work(t0)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, blocks))
    return out


def _unit_rows(seed: int, stream: int, shape) -> np.ndarray:
    """N(0,1) vectors along the last axis, L2-normalised in fp64; returned as fp32."""
    def fn(b, shp):
        x = _block_rng(seed, stream, b).standard_normal(shp, dtype=np.float32).astype(np.float64)
        x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return x
    return _fill_blocks(shape, fn)


def _scaled_rows(seed: int, stream: int, shape) -> np.ndarray:
    """N(0,1) vectors along the last axis times 10^U(-1, 1) per vector (lengths spread over two
    decades); the factors come from their own child generators (stream + 10)."""
    def fn(b, shp):
        x = _block_rng(seed, stream, b).standard_normal(shp, dtype=np.float32).astype(np.float64)
        f = 10.0 ** _block_rng(seed, stream + 10, b).uniform(-1.0, 1.0, size=shp[:-1] + (1,))
        return x * f
    return _fill_blocks(shape, fn)


def _normal_rows(seed: int, stream: int, shape) -> np.ndarray:
    return _fill_blocks(shape, lambda b, shp: _block_rng(seed, stream, b).standard_normal(shp, dtype=np.float32))


@dataclasses.dataclass
class GdnInputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    s0: np.ndarray | None
    cu_seqlens: np.ndarray
    dtype: str                 # "bf16" or "fp32": storage of q, k, v (and the output)
    scale: float
    name: str
    seed: int
    meta: dict

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def hqk(self) -> int:
        return int(self.q.shape[1])

    @property
    def hv(self) -> int:
        return int(self.v.shape[1])

    @property
    def dk(self) -> int:
        return int(self.q.shape[2])

    @property
    def dv(self) -> int:
        return int(self.v.shape[2])


def draw(
    *,
    T: int | None = None,
    lengths=None,
    hqk: int,
    hv: int,
    dk: int,
    dv: int | None = None,
    dtype: str = "bf16",
    seed: int = 0,
    g_mean: float = 0.0,
    s0_std: float | None = None,
    scale: float = 1.0,
    name: str = "custom",
    varlen_draw=None,
    fixed_g: float | None = None,
    fixed_beta: float | None = None,
    qk_unit: bool = True,
    k_spread: float | None = None,
) -> GdnInputs:
    """Draw one seeded input set.

    Streams (fixed so that every consumer gets identical tensors): the main
    generator default_rng(seed) draws, in order, the varlen lengths, the g
    noise, the beta noise and the initial states; q, k and v come from child
    generators default_rng([seed, 1|2|3, block]) per 8192-token block.
    g = -softplus(N(g_mean, 1)), beta = sigmoid(N(0, 1)), v ~ N(0, 1),
    initial states s0_std * N(0, 1) when s0_std is given (else none).
    fixed_g / fixed_beta replace the drawn values by a constant (used by
    the special cases whose closed forms the tests check). qk_unit=False
    leaves q and k unnormalised (for the in-kernel normalisation mode).
    k_spread, when given, makes the keys of each QK head nearly parallel:
    k = unit(b_h + k_spread * n_t) with one N(0, 1) direction b_h per QK head
    (child generator [seed, 4, 0]) and n_t the usual key noise, so that the
    decay-masked key Gram of a chunk is close to all ones.
    """
    if dtype not in ("bf16", "fp32"):
        raise ValueError(dtype)
    dv = dk if dv is None else dv
    rng = np.random.default_rng(seed)
    if varlen_draw is not None:
        lengths = varlen_draw(rng)
    if lengths is None:
        if T is None:
            raise ValueError("T or lengths required")
        lengths = [T]
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)

    rows = _unit_rows if qk_unit else _scaled_rows
    q = rows(seed, 1, (T, hqk, dk))
    if k_spread is None:
        k = rows(seed, 2, (T, hqk, dk))
    else:
        base = _block_rng(seed, 4, 0).standard_normal((hqk, dk))

        def near(b, shp):
            x = base[None] + k_spread * _block_rng(seed, 2, b).standard_normal(shp, dtype=np.float32).astype(np.float64)
            return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        k = _fill_blocks((T, hqk, dk), near)
    v = _normal_rows(seed, 3, (T, hv, dv))
    g = (-_softplus(rng.standard_normal((T, hv)) + g_mean)).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((T, hv))).astype(np.float32)
    if fixed_g is not None:
        g[...] = np.float32(fixed_g)
    if fixed_beta is not None:
        beta[...] = np.float32(fixed_beta)
    s0 = None
    if s0_std is not None:
        s0 = (s0_std * rng.standard_normal((len(lengths), hv, dv, dk), dtype=np.float32)).astype(np.float32)

    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    meta = {
        "lengths": lengths,
        "g_mean_param": g_mean,
        "s0_std": s0_std,
        "mean_alpha": float(np.mean(np.exp(g.astype(np.float64)))) if T else None,
        "k_spread": k_spread,
    }
    return GdnInputs(q=q, k=k, v=v, g=g, beta=beta, s0=s0, cu_seqlens=cu, dtype=dtype,
                     scale=float(scale), name=name, seed=seed, meta=meta)


def _varlen_lengths(rng: np.random.Generator, n: int = 8, lo: int = 1024, hi: int = 16384,
                    padded_cap: int = 65536, chunk: int = 64):
    """n lengths uniform in [lo, hi]; the whole tuple is redrawn until the total,
    with each length rounded up to a whole chunk, fits padded_cap."""
    while True:
        L = rng.integers(lo, hi + 1, size=n)
        if int(np.sum(-(-L // chunk) * chunk)) <= padded_cap:
            return [int(x) for x in L]


# Named workloads.  Seeds are 1000 + index; the T=65536 prefill uses 1005.
def tiny(dtype: str = "fp32", seed: int = 1000) -> GdnInputs:
    """B=1, T=64, one QK and one V head, d=16, fp32, zero initial state."""
    return draw(T=64, hqk=1, hv=1, dk=16, dtype=dtype, seed=seed, name="tiny_T64_d16")


def qwen3_next_prefill(T: int = 4096, dtype: str = "bf16", seed: int | None = None,
                       scale: float = 1.0) -> GdnInputs:
    """One Qwen3-Next GDN layer prefill: B=1, 16 QK / 32 V heads, d=128, zero initial state."""
    if seed is None:
        seed = 1005 if T == 65536 else 1001
    return draw(T=T, hqk=QWEN3_NEXT_HQK, hv=QWEN3_NEXT_HV, dk=QWEN3_NEXT_D, dtype=dtype,
                seed=seed, scale=scale, name=f"qwen3next_gdn_prefill_T{T}")


def tp_share_prefill(T: int = 65536, tp: int = 4, dtype: str = "bf16", seed: int = 1008) -> GdnInputs:
    """One GPU's share of the layer under tensor parallelism of degree tp: the QK heads and their V
    heads split evenly (16/tp QK, 32/tp V heads), the full sequence, the layer's distributions."""
    return draw(T=T, hqk=QWEN3_NEXT_HQK // tp, hv=QWEN3_NEXT_HV // tp, dk=QWEN3_NEXT_D, dtype=dtype,
                seed=seed, name=f"qwen3next_gdn_prefill_T{T}_tp{tp}_share")


def varlen_prefill(dtype: str = "bf16", seed: int = 1002) -> GdnInputs:
    """8 packed sequences, lengths uniform in [1024, 16384], chunk-padded total <= 65536,
    initial states 0.01 * N(0, 1)."""
    return draw(varlen_draw=_varlen_lengths, hqk=QWEN3_NEXT_HQK, hv=QWEN3_NEXT_HV,
                dk=QWEN3_NEXT_D, dtype=dtype, seed=seed, s0_std=0.01,
                name="qwen3next_gdn_varlen8")


def decode_batch(n: int = 256, dtype: str = "bf16", seed: int = 1003) -> GdnInputs:
    """n independent sequences of one token each; state [n, 32, 128, 128] = 0.01 * N(0, 1)."""
    return draw(lengths=[1] * n, hqk=QWEN3_NEXT_HQK, hv=QWEN3_NEXT_HV, dk=QWEN3_NEXT_D,
                dtype=dtype, seed=seed, s0_std=0.01, name=f"qwen3next_gdn_decode_N{n}")


def long_context(T: int = 262144, dtype: str = "bf16", seed: int = 1004) -> GdnInputs:
    """B=1 long prefill with g = -softplus(N(-4, 1)) (decay close to 1)."""
    return draw(T=T, hqk=QWEN3_NEXT_HQK, hv=QWEN3_NEXT_HV, dk=QWEN3_NEXT_D, dtype=dtype,
                seed=seed, g_mean=-4.0, name=f"qwen3next_gdn_long_T{T}")


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 view of a q/k/v array in either storage dtype."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def chunk_count(lengths, chunk: int = 64) -> int:
    return int(sum(math.ceil(L / chunk) for L in lengths))


def large_state(num: int, hv: int, d: int, seed: int, std: float = 0.01) -> np.ndarray:
    """States [num, hv, d, d] fp32 = std * N(0, 1), drawn in fp32 from default_rng(seed) (no fp64
    temporary: for state arrays of several GiB)."""
    rng = np.random.default_rng(seed)
    out = rng.standard_normal((num, hv, d, d), dtype=np.float32)
    out *= np.float32(std)
    return out


def state_pool(num_slots: int, hv: int, d: int, seed: int, std: float = 0.3) -> np.ndarray:
    """A state pool [num_slots, hv, d, d] fp32 = std * N(0, 1) from default_rng(seed) (the per-request
    states a serving cache holds, addressed by slot)."""
    rng = np.random.default_rng(seed)
    return (std * rng.standard_normal((num_slots, hv, d, d))).astype(np.float32)


@dataclasses.dataclass
class ConvInputs:
    x: np.ndarray              # [T, C] the mixer's input channels (q, k, v side by side), bf16 bits or fp32
    w: np.ndarray              # [C, K] fp32 taps
    history: np.ndarray | None  # [N, K - 1, C] (dtype of x) or None
    cu_seqlens: np.ndarray
    hqk: int
    hv: int
    d: int
    dtype: str
    name: str


def conv_inputs(*, lengths, hqk: int, hv: int, d: int, K: int = 4, dtype: str = "bf16", seed: int = 0,
                history: bool = True, name: str = "conv") -> ConvInputs:
    """Inputs of the short causal convolution in front of the mixer: x ~ N(0, 1) over C = 2 Hqk d + Hv d
    channels, taps w ~ N(0, 1) / sqrt(K), histories N(0, 1) (main generator default_rng(seed), in that
    order)."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    C = (2 * hqk + hv) * d
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x = rng.standard_normal((T, C), dtype=np.float32)
    w = (rng.standard_normal((C, K)) / math.sqrt(K)).astype(np.float32)
    h = rng.standard_normal((len(lengths), K - 1, C), dtype=np.float32) if history else None
    if dtype == "bf16":
        x = f32_to_bf16_bits(x)
        h = None if h is None else f32_to_bf16_bits(h)
    return ConvInputs(x=x, w=w, history=h, cu_seqlens=cu, hqk=hqk, hv=hv, d=d, dtype=dtype, name=name)

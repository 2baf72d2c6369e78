"""Python binding of libgdn, the Gated DeltaNet token mixer for MI355X (gfx950).

The functions carry the C ABI's names (include/gdn.h) and only marshal
arguments: torch tensors supply device pointers and the current HIP stream,
every step of the layer runs in the library's kernels. There is no CPU or
PyTorch fallback: if libgdn.so is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["gdn_prefill", "gdn_prefill_noalloc", "GDN_ERR_SCRATCH_LIMIT", "GDN_PREFILL_NOALLOC_SCRATCH_BYTES", "gdn_decode_step", "gdn_prefill_slots", "gdn_decode_step_slots", "gdn_decode_multi",
           "gdn_prefill_ex", "gdn_decode_ex", "GDN_FLAG_QK_L2NORM", "gdn_backward", "gdn_backward_workspace_size",
           "gdn_prefill_workspace_size", "gdn_prefill_segment_chunks", "gdn_conv_prologue", "gdn_decode_conv", "GDN_FLAG_CONV_SILU",
           "gdn_status_string",
           "gdn_build_info", "gdn_profile_start", "gdn_profile_stop", "GDN_BF16", "GDN_FP32", "GdnError", "library_path"]

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP, GDN_ERR_SCRATCH_LIMIT = range(6)
GDN_PREFILL_NOALLOC_SCRATCH_BYTES = 192 << 20
GDN_BF16, GDN_FP32 = 0, 1
GDN_FLAG_QK_L2NORM = 1
GDN_FLAG_CONV_SILU = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libgdn.so")
_lock = threading.Lock()
_lib = None

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gdn_status_string(status)} (status {status})")


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(library_path):
                raise RuntimeError(f"libgdn.so not built at {library_path}; run "
                                   "`python -m linear_attention_sequence_02_amd.build`")
            lib = ctypes.CDLL(library_path)
            lib.gdn_prefill_workspace_size.restype = _sz
            lib.gdn_prefill_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_int]
            lib.gdn_prefill_segment_chunks.restype = _i32
            lib.gdn_prefill_segment_chunks.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_int]
            lib.gdn_prefill.restype = ctypes.c_int
            lib.gdn_prefill.argtypes = ([_vp] * 7 + [_i32, _i64, _i32, _i32, _i32, _i32, _f32, ctypes.c_int]
                                        + [_vp, _vp, _vp, _sz, _vp])
            lib.gdn_decode_step.restype = ctypes.c_int
            lib.gdn_decode_step.argtypes = [_vp] * 6 + [_i32] * 5 + [_f32, ctypes.c_int, _vp, _vp]
            lib.gdn_decode_step_slots.restype = ctypes.c_int
            lib.gdn_decode_step_slots.argtypes = [_vp] * 7 + [_i32] * 6 + [_f32, ctypes.c_int, _vp, _vp]
            lib.gdn_decode_multi.restype = ctypes.c_int
            lib.gdn_decode_multi.argtypes = [_vp] * 7 + [_i32] * 7 + [_f32, ctypes.c_int, _vp, _vp, _vp]
            lib.gdn_backward_workspace_size.restype = _sz
            lib.gdn_backward_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_int]
            lib.gdn_backward.restype = ctypes.c_int
            lib.gdn_backward.argtypes = ([_vp] * 7 + [_i32, _i64, _i32, _i32, _i32, _i32, _f32, ctypes.c_int]
                                         + [_vp] * 9 + [_sz, _vp])
            lib.gdn_prefill_ex.restype = ctypes.c_int
            lib.gdn_prefill_ex.argtypes = ([_vp] * 9 + [_i32, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                                                       ctypes.c_int, ctypes.c_uint32, _vp, _vp, _sz, _vp])
            lib.gdn_decode_ex.restype = ctypes.c_int
            lib.gdn_decode_ex.argtypes = ([_vp] * 7 + [_i32] * 7 + [_f32, ctypes.c_int, ctypes.c_uint32]
                                          + [_vp, _vp, _vp])
            lib.gdn_prefill_slots.restype = ctypes.c_int
            lib.gdn_prefill_slots.argtypes = ([_vp] * 8 + [_i32, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                                                          ctypes.c_int, _vp, _vp, _sz, _vp])
            lib.gdn_prefill_noalloc.restype = ctypes.c_int
            lib.gdn_prefill_noalloc.argtypes = ([_vp] * 7 + [_i32, _i64, _i32, _i32, _i32, _i32, _f32, ctypes.c_int]
                                                + [_vp, _vp, _vp])
            lib.gdn_conv_prologue.restype = ctypes.c_int
            lib.gdn_conv_prologue.argtypes = ([_vp] * 4 + [_i32, _i64] + [_i32] * 5 + [ctypes.c_int, ctypes.c_uint32]
                                              + [_vp] * 5)
            lib.gdn_decode_conv.restype = ctypes.c_int
            lib.gdn_decode_conv.argtypes = ([_vp] * 7 + [_i32] * 6 + [_f32, ctypes.c_int, ctypes.c_uint32]
                                            + [_vp, _vp])
            lib.gdn_status_string.restype = ctypes.c_char_p
            lib.gdn_status_string.argtypes = [ctypes.c_int]
            lib.gdn_build_info.restype = ctypes.c_char_p
            lib.gdn_build_info.argtypes = []
            lib.gdn_profile_start.restype = ctypes.c_int
            lib.gdn_profile_start.argtypes = []
            lib.gdn_profile_stop.restype = ctypes.c_int32
            lib.gdn_profile_stop.argtypes = [_i32, ctypes.c_char_p, ctypes.POINTER(_i32),
                                             ctypes.POINTER(ctypes.c_double)]
            _lib = lib
    return _lib


def gdn_status_string(status: int) -> str:
    return _load().gdn_status_string(int(status)).decode()


def gdn_build_info() -> str:
    return _load().gdn_build_info().decode()


def gdn_profile_start() -> None:
    """Start per-kernel event timing of every library launch (see include/gdn.h)."""
    _load().gdn_profile_start()


def gdn_profile_stop(max_kernels: int = 16) -> dict:
    """Stop timing; returns {kernel name: (launch count, total milliseconds)}."""
    names = ctypes.create_string_buffer(64 * max_kernels)
    counts = (_i32 * max_kernels)()
    totals = (ctypes.c_double * max_kernels)()
    n = _load().gdn_profile_stop(max_kernels, names, counts, totals)
    if n < 0:
        raise RuntimeError("gdn_profile_stop: a HIP event call failed")
    raw = names.raw
    res = {}
    for j in range(n):
        name = raw[64 * j:64 * j + 64].split(b"\0", 1)[0].decode()
        res[name] = (int(counts[j]), float(totals[j]))
    return res


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_FP32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, dtype=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _expect(t, name, shape):
    """Raise ValueError unless t is None or has `shape` (None entries match any size)."""
    if t is None:
        return
    if t.dim() != len(shape) or any(e is not None and int(a) != int(e) for a, e in zip(t.shape, shape)):
        want = "[" + ", ".join("*" if e is None else str(int(e)) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")


def _token_shapes(q, k, v, g, beta, out=None, out_name="out"):
    """Shapes shared by every entry point: q, k [T, Hqk, dk], v and out [T, Hv, dv], g, beta [T, Hv]."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError(f"q and v must be 3-D [tokens, heads, dim], got {list(q.shape)} and {list(v.shape)}")
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    _expect(k, "k", (T, hqk, dk))
    _expect(v, "v", (T, hv, dv))
    _expect(g, "g", (T, hv))
    _expect(beta, "beta", (T, hv))
    _expect(out, out_name, (T, hv, dv))
    return T, hqk, dk, hv, dv


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _seq_count(cu_seqlens) -> int:
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError(f"cu_seqlens must be 1-D [N + 1], got shape {list(cu_seqlens.shape)}")
    return cu_seqlens.shape[0] - 1


def gdn_prefill_workspace_size(total_tokens: int, num_seqs: int, num_qk_heads: int, num_v_heads: int,
                               d_k: int, d_v: int, dtype: int) -> int:
    return int(_load().gdn_prefill_workspace_size(total_tokens, num_seqs, num_qk_heads, num_v_heads,
                                                  d_k, d_v, dtype))


def gdn_prefill_segment_chunks(total_tokens: int, num_seqs: int, num_qk_heads: int, num_v_heads: int,
                               d_k: int, d_v: int, dtype: int) -> int:
    return int(_load().gdn_prefill_segment_chunks(total_tokens, num_seqs, num_qk_heads, num_v_heads,
                                                  d_k, d_v, dtype))


def gdn_prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *, scale: float = 1.0,
                out=None, final_state=None, output_final_state: bool = True, workspace=None, stream=None):
    """Chunked prefill. Shapes as in include/gdn.h; returns (out, final_state).

    q, k [T, Hqk, d] and v [T, Hv, d] (bf16 or fp32, one dtype), g and beta
    [T, Hv] fp32, initial_state [N, Hv, d, d] fp32 or None, cu_seqlens [N + 1]
    int32 on the device or None (one sequence). Missing outputs and the
    workspace are allocated with torch; pass them to avoid allocation.
    """
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state)):
        _check(t, name, torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    T, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    n = 1 if cu_seqlens is None else _seq_count(cu_seqlens)
    _expect(initial_state, "initial_state", (n, hv, dv, dk))
    _expect(final_state, "final_state", (n, hv, dv, dk))
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=dev)
    _check(out, "out", q.dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, hv, dv, dk), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", torch.float32, dev)
    need = gdn_prefill_workspace_size(T, n, hqk, hv, dk, dv, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                             _ptr(cu_seqlens), n, T, hqk, hv, dk, dv, float(scale), dt, _ptr(out),
                             _ptr(final_state), _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill")
    return out, final_state


def gdn_decode_step(q, k, v, g, beta, state, *, scale: float = 1.0, out=None, stream=None):
    """One decode step, state [N, Hv, d, d] fp32 updated in place; returns out [N, Hv, d]."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("state", state)):
        _check(t, name, torch.float32, dev)
    N, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    _expect(state, "state", (N, hv, dv, dk))
    if out is None:
        out = torch.empty((N, hv, dv), dtype=q.dtype, device=dev)
    _check(out, "out", q.dtype, dev)
    st = _load().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), N, hqk, hv,
                                 dk, dv, float(scale), dt, _ptr(out), _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_step")
    return out


def gdn_decode_step_slots(q, k, v, g, beta, state_pool, state_indices, *, scale: float = 1.0, out=None,
                          stream=None):
    """One decode step on a state pool [S, Hv, d, d] fp32: sequence n updates row state_indices[n]
    (int32 [N] on the device; an index outside [0, S) is a padding entry with zero outputs).
    Returns out [N, Hv, d]."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("state_pool", state_pool)):
        _check(t, name, torch.float32, dev)
    _check(state_indices, "state_indices", torch.int32, dev)
    N, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    _expect(state_pool, "state_pool", (None, hv, dv, dk))
    _expect(state_indices, "state_indices", (N,))
    if out is None:
        out = torch.empty((N, hv, dv), dtype=q.dtype, device=dev)
    _check(out, "out", q.dtype, dev)
    st = _load().gdn_decode_step_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                       _ptr(state_indices), state_pool.shape[0], N, hqk, hv, dk, dv,
                                       float(scale), dt, _ptr(out), _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_step_slots")
    return out


def gdn_prefill_slots(q, k, v, g, beta, state_pool, state_indices, has_initial_state=None, cu_seqlens=None, *,
                      scale: float = 1.0, out=None, workspace=None, stream=None):
    """Chunked prefill on a state pool [S, Hv, d, d] fp32: sequence n starts from row state_indices[n]
    (from zeros where has_initial_state[n] == 0) and writes its final state back to that row.
    state_indices and has_initial_state are int32 [N] on the device. Returns out."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("state_pool", state_pool)):
        _check(t, name, torch.float32, dev)
    for name, t in (("state_indices", state_indices), ("has_initial_state", has_initial_state),
                    ("cu_seqlens", cu_seqlens)):
        _check(t, name, torch.int32, dev)
    T, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    n = 1 if cu_seqlens is None else _seq_count(cu_seqlens)
    _expect(state_pool, "state_pool", (None, hv, dv, dk))
    _expect(state_indices, "state_indices", (n,))
    _expect(has_initial_state, "has_initial_state", (n,))
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=dev)
    _check(out, "out", q.dtype, dev)
    need = gdn_prefill_workspace_size(T, n, hqk, hv, dk, dv, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().gdn_prefill_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                   _ptr(state_indices), _ptr(has_initial_state), state_pool.shape[0],
                                   _ptr(cu_seqlens), n, T, hqk, hv, dk, dv, float(scale), dt, _ptr(out),
                                   _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_slots")
    return out


def gdn_decode_multi(q, k, v, g, beta, state, num_tokens: int, *, state_indices=None, scale: float = 1.0,
                     out=None, token_states=None, stream=None):
    """num_tokens consecutive tokens per sequence from its state. q, k [N * num_tokens, Hqk, d], v
    [N * num_tokens, Hv, d] (token t of sequence n at row n * num_tokens + t), g, beta [N * num_tokens, Hv];
    state [N, Hv, d, d] fp32 (or a pool [S, Hv, d, d] with state_indices int32 [N]) advanced in place.
    token_states: None, True (allocate) or a [N * num_tokens, Hv, d, d] fp32 tensor for the state after
    every token. Returns (out, token_states)."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("state", state)):
        _check(t, name, torch.float32, dev)
    _check(state_indices, "state_indices", torch.int32, dev)
    rows, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    if num_tokens < 1 or rows % num_tokens:
        raise ValueError(f"{rows} token rows are not a whole number of sequences of {num_tokens} tokens")
    N = rows // num_tokens
    _expect(state, "state", (None if state_indices is not None else N, hv, dv, dk))
    _expect(state_indices, "state_indices", (N,))
    _expect(token_states if isinstance(token_states, torch.Tensor) else None, "token_states", (rows, hv, dv, dk))
    if out is None:
        out = torch.empty((rows, hv, dv), dtype=q.dtype, device=dev)
    _check(out, "out", q.dtype, dev)
    if token_states is True:
        token_states = torch.empty((rows, hv, dv, dk), dtype=torch.float32, device=dev)
    elif token_states is False:
        token_states = None
    _check(token_states, "token_states", torch.float32, dev)
    num_slots = state.shape[0] if state_indices is not None else 0
    st = _load().gdn_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                  _ptr(state_indices), num_slots, N, num_tokens, hqk, hv, dk, dv, float(scale), dt,
                                  _ptr(out), _ptr(token_states), _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_multi")
    return out, token_states


def gdn_prefill_ex(q, k, v, g, beta, initial_state=None, final_state=None, state_indices=None,
                   has_initial_state=None, cu_seqlens=None, *, flags: int = 0, scale: float = 1.0, out=None,
                   workspace=None, stream=None):
    """General prefill with option flags (GDN_FLAG_QK_L2NORM: q and k normalised in the kernels).
    Without state_indices, initial_state / final_state are [N, Hv, d, d] arrays (or None); with it they
    are pools [S, Hv, d, d] addressed by slot. Returns out."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state), ("final_state", final_state)):
        _check(t, name, torch.float32, dev)
    for name, t in (("state_indices", state_indices), ("has_initial_state", has_initial_state),
                    ("cu_seqlens", cu_seqlens)):
        _check(t, name, torch.int32, dev)
    T, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    n = 1 if cu_seqlens is None else _seq_count(cu_seqlens)
    num_slots = 0
    rows = None if state_indices is not None else n
    _expect(initial_state, "initial_state", (rows, hv, dv, dk))
    _expect(final_state, "final_state", (rows, hv, dv, dk))
    _expect(state_indices, "state_indices", (n,))
    _expect(has_initial_state, "has_initial_state", (n,))
    if state_indices is not None:
        if (initial_state is not None and final_state is not None
                and initial_state.shape[0] != final_state.shape[0]):
            raise ValueError(f"initial_state and final_state pools differ in size ({initial_state.shape[0]} "
                             f"and {final_state.shape[0]} slots); slot indices address both")
        pool = initial_state if initial_state is not None else final_state
        num_slots = 0 if pool is None else pool.shape[0]
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=dev)
    _check(out, "out", q.dtype, dev)
    need = gdn_prefill_workspace_size(T, n, hqk, hv, dk, dv, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().gdn_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                _ptr(final_state), _ptr(state_indices), _ptr(has_initial_state), num_slots,
                                _ptr(cu_seqlens), n, T, hqk, hv, dk, dv, float(scale), dt, int(flags), _ptr(out),
                                _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_ex")
    return out


def gdn_decode_ex(q, k, v, g, beta, state, *, num_tokens: int = 1, state_indices=None, flags: int = 0,
                  scale: float = 1.0, out=None, token_states=None, stream=None):
    """General decode with option flags: num_tokens tokens per sequence (layout as gdn_decode_multi),
    optional state pool (state_indices) and per-token states. Returns (out, token_states)."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("state", state)):
        _check(t, name, torch.float32, dev)
    _check(state_indices, "state_indices", torch.int32, dev)
    rows, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    if num_tokens < 1 or rows % num_tokens:
        raise ValueError(f"{rows} token rows are not a whole number of sequences of {num_tokens} tokens")
    N = rows // num_tokens
    _expect(state, "state", (None if state_indices is not None else N, hv, dv, dk))
    _expect(state_indices, "state_indices", (N,))
    _expect(token_states if isinstance(token_states, torch.Tensor) else None, "token_states", (rows, hv, dv, dk))
    if out is None:
        out = torch.empty((rows, hv, dv), dtype=q.dtype, device=dev)
    _check(out, "out", q.dtype, dev)
    if token_states is True:
        token_states = torch.empty((rows, hv, dv, dk), dtype=torch.float32, device=dev)
    elif token_states is False:
        token_states = None
    _check(token_states, "token_states", torch.float32, dev)
    num_slots = state.shape[0] if state_indices is not None else 0
    st = _load().gdn_decode_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(state_indices),
                               num_slots, rows // num_tokens, num_tokens, hqk, hv, dk, dv, float(scale), dt,
                               int(flags), _ptr(out), _ptr(token_states), _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_ex")
    return out, token_states


def gdn_backward_workspace_size(total_tokens: int, num_seqs: int, num_qk_heads: int, num_v_heads: int,
                                d_k: int, d_v: int, dtype: int) -> int:
    return int(_load().gdn_backward_workspace_size(total_tokens, num_seqs, num_qk_heads, num_v_heads, d_k, d_v,
                                                   dtype))


def gdn_backward(q, k, v, g, beta, d_out, initial_state=None, cu_seqlens=None, d_final_state=None, *,
                 scale: float = 1.0, output_d_initial_state: bool = True, workspace=None, stream=None):
    """Gradients of the prefill given d_out [T, Hv, d] (dtype of q) and optionally d_final_state
    [N, Hv, d, d]. Returns a dict of fp32 tensors: dq, dk [T, Hqk, d], dv [T, Hv, d], dg, dbeta [T, Hv],
    d_initial_state [N, Hv, d, d] (or None)."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("d_out", d_out)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state), ("d_final_state", d_final_state)):
        _check(t, name, torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    T, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, d_out, "d_out")
    n = 1 if cu_seqlens is None else _seq_count(cu_seqlens)
    _expect(initial_state, "initial_state", (n, hv, dv, dk))
    _expect(d_final_state, "d_final_state", (n, hv, dv, dk))
    f32 = dict(dtype=torch.float32, device=dev)
    res = {"dq": torch.empty((T, hqk, dk), **f32), "dk": torch.empty((T, hqk, dk), **f32),
           "dv": torch.empty((T, hv, dv), **f32), "dg": torch.empty((T, hv), **f32),
           "dbeta": torch.empty((T, hv), **f32),
           "d_initial_state": torch.empty((n, hv, dv, dk), **f32) if output_d_initial_state else None}
    need = gdn_backward_workspace_size(T, n, hqk, hv, dk, dv, dt)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _load().gdn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
                              n, T, hqk, hv, dk, dv, float(scale), dt, _ptr(d_out), _ptr(d_final_state),
                              _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dg"]), _ptr(res["dbeta"]),
                              _ptr(res["d_initial_state"]), _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_backward")
    return res


def gdn_conv_prologue(x, weight, conv_state=None, cu_seqlens=None, *, num_qk_heads: int, num_v_heads: int,
                      num_seqs: int | None = None, silu: bool = False, qk_l2norm: bool = False, q=None, k=None,
                      v=None, conv_state_out=None, stream=None):
    """Short causal convolution + optional SiLU + split into q, k, v (+ optional q/k L2 norm).

    x [T, C] bf16 or fp32 with C = 2 Hqk d + Hv d (q, k, v channels side by side), weight [C, K] fp32,
    conv_state [N, K - 1, C] (dtype of x) or None (zero history), cu_seqlens int32 [N + 1] or None
    (num_seqs equal-length sequences; default one). conv_state_out: None (not written), True (allocate)
    or a tensor (may be conv_state itself). Returns (q, k, v, conv_state_out)."""
    dev = x.device
    _check(x, "x", device=dev)
    dt = _dtype_code(x)
    _check(weight, "weight", torch.float32, dev)
    _check(conv_state, "conv_state", x.dtype, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError(f"x must be [T, C] and weight [C, K], got {list(x.shape)} and {list(weight.shape)}")
    T, C = x.shape
    K = weight.shape[1]
    hqk, hv = int(num_qk_heads), int(num_v_heads)
    if C % (2 * hqk + hv):
        raise ValueError(f"{C} channels are not 2 * {hqk} + {hv} heads of one size")
    d = C // (2 * hqk + hv)
    _expect(weight, "weight", (C, K))
    n = _seq_count(cu_seqlens) if cu_seqlens is not None else (1 if num_seqs is None else int(num_seqs))
    _expect(conv_state, "conv_state", (n, K - 1, C))
    if conv_state_out is True:
        conv_state_out = torch.empty((n, K - 1, C), dtype=x.dtype, device=dev)
    elif conv_state_out is False:
        conv_state_out = None
    _check(conv_state_out, "conv_state_out", x.dtype, dev)
    _expect(conv_state_out, "conv_state_out", (n, K - 1, C))
    q = torch.empty((T, hqk, d), dtype=x.dtype, device=dev) if q is None else q
    k = torch.empty((T, hqk, d), dtype=x.dtype, device=dev) if k is None else k
    v = torch.empty((T, hv, d), dtype=x.dtype, device=dev) if v is None else v
    for name, t, shp in (("q", q, (T, hqk, d)), ("k", k, (T, hqk, d)), ("v", v, (T, hv, d))):
        _check(t, name, x.dtype, dev)
        _expect(t, name, shp)
    flags = (GDN_FLAG_CONV_SILU if silu else 0) | (GDN_FLAG_QK_L2NORM if qk_l2norm else 0)
    st = _load().gdn_conv_prologue(_ptr(x), _ptr(weight), _ptr(conv_state), _ptr(cu_seqlens), n, T, hqk, hv, d, d,
                                   K, dt, flags, _ptr(q), _ptr(k), _ptr(v), _ptr(conv_state_out),
                                   _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_conv_prologue")
    return q, k, v, conv_state_out


def gdn_decode_conv(x, weight, g, beta, state, conv_state=None, *, num_qk_heads: int, num_v_heads: int,
                    conv_state_out=None, silu: bool = False, qk_l2norm: bool = False, scale: float = 1.0,
                    out=None, stream=None):
    """One decode step with the input prologue fused in (one launch): the causal convolution of the
    token's q, k, v channels over each sequence's history, optional SiLU and q/k L2 normalisation,
    then the decode step on `state` (updated in place).

    x [N, C] bf16 or fp32 (C = 2 Hqk d + Hv d), weight [C, K] fp32, g and beta [N, Hv] fp32, state
    [N, Hv, d, d] fp32, conv_state [N, K - 1, C] (dtype of x) or None (zero history). conv_state_out:
    None (not written), True (allocate) or a tensor that must not overlap conv_state (alternate two).
    Returns (out [N, Hv, d], conv_state_out)."""
    dev = x.device
    _check(x, "x", device=dev)
    dt = _dtype_code(x)
    _check(weight, "weight", torch.float32, dev)
    for name, t in (("g", g), ("beta", beta), ("state", state)):
        _check(t, name, torch.float32, dev)
    _check(conv_state, "conv_state", x.dtype, dev)
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError(f"x must be [N, C] and weight [C, K], got {list(x.shape)} and {list(weight.shape)}")
    n, C = x.shape
    K = weight.shape[1]
    hqk, hv = int(num_qk_heads), int(num_v_heads)
    if C % (2 * hqk + hv):
        raise ValueError(f"{C} channels are not 2 * {hqk} + {hv} heads of one size")
    d = C // (2 * hqk + hv)
    _expect(weight, "weight", (C, K))
    _expect(g, "g", (n, hv))
    _expect(beta, "beta", (n, hv))
    _expect(state, "state", (n, hv, d, d))
    _expect(conv_state, "conv_state", (n, K - 1, C))
    if conv_state_out is True:
        conv_state_out = torch.empty((n, K - 1, C), dtype=x.dtype, device=dev)
    elif conv_state_out is False:
        conv_state_out = None
    _check(conv_state_out, "conv_state_out", x.dtype, dev)
    _expect(conv_state_out, "conv_state_out", (n, K - 1, C))
    out = torch.empty((n, hv, d), dtype=x.dtype, device=dev) if out is None else out
    _check(out, "out", x.dtype, dev)
    _expect(out, "out", (n, hv, d))
    flags = (GDN_FLAG_CONV_SILU if silu else 0) | (GDN_FLAG_QK_L2NORM if qk_l2norm else 0)
    st = _load().gdn_decode_conv(_ptr(x), _ptr(weight), _ptr(conv_state), _ptr(conv_state_out), _ptr(g),
                                 _ptr(beta), _ptr(state), n, hqk, hv, d, d, K, float(scale), dt, flags, _ptr(out),
                                 _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_conv")
    return out, conv_state_out


def gdn_prefill_noalloc(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *, out, final_state=None,
                        scale: float = 1.0, stream=None):
    """gdn_prefill without a workspace argument (the library's static device array serves as the
    workspace, so the call allocates nothing). `out` must be given; final_state may be None (not
    written). Calls that may overlap on one GPU must be serialised by the caller. Returns
    (out, final_state)."""
    dev = q.device
    _check(q, "q", device=dev)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("out", out)):
        _check(t, name, q.dtype, dev)
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state), ("final_state", final_state)):
        _check(t, name, torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if out is None:
        raise ValueError("gdn_prefill_noalloc needs `out` (it allocates nothing)")
    T, hqk, dk, hv, dv = _token_shapes(q, k, v, g, beta, out)
    n = 1 if cu_seqlens is None else _seq_count(cu_seqlens)
    _expect(initial_state, "initial_state", (n, hv, dv, dk))
    _expect(final_state, "final_state", (n, hv, dv, dk))
    st = _load().gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                     _ptr(cu_seqlens), n, T, hqk, hv, dk, dv, float(scale), dt, _ptr(out),
                                     _ptr(final_state), _stream(stream, dev))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_noalloc")
    return out, final_state

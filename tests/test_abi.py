"""The C ABI library loads, exports what include/gdn.h declares, and rejects bad
arguments on the host. Every call here fails validation (or has nothing to do)
before any kernel is enqueued, so these run without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_sequence_02_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.library_path):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    return gdn._load()


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == {"gdn_prefill_workspace_size", "gdn_prefill_segment_chunks", "gdn_prefill",
                                         "gdn_decode_step", "gdn_prefill_slots", "gdn_decode_step_slots",
                                         "gdn_decode_multi", "gdn_prefill_ex", "gdn_decode_ex",
                                         "gdn_backward", "gdn_backward_workspace_size",
                                         "gdn_status_string", "gdn_build_info", "gdn_profile_start",
                                         "gdn_profile_stop", "gdn_conv_prologue", "gdn_prefill_noalloc",
                                         "gdn_decode_conv"}


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.library_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(\S+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for s in range(5):
        assert gdn.gdn_status_string(s).startswith("GDN_")
    assert "unknown" in gdn.gdn_status_string(99)
    assert "gfx950" in gdn.gdn_build_info()


def test_workspace_size(lib):
    ws = gdn.gdn_prefill_workspace_size
    assert ws(65536, 1, 16, 32, 128, 128, gdn.GDN_BF16) > 0
    assert ws(65536, 1, 16, 32, 128, 128, gdn.GDN_FP32) == 0
    assert ws(65536, 1, 3, 32, 128, 128, gdn.GDN_BF16) == 0          # rejected shape
    assert ws(-1, 1, 16, 32, 128, 128, gdn.GDN_BF16) == 0
    # grows with tokens and sequences (one chunk slot per 64 tokens plus one per sequence)
    assert ws(64 * 10, 1, 16, 32, 128, 128, 0) < ws(64 * 10, 5, 16, 32, 128, 128, 0) < ws(64 * 20, 5, 16, 32, 128, 128, 0)


def test_segment_chunks_query(lib):
    sc = gdn.gdn_prefill_segment_chunks
    assert sc(65536, 1, 16, 32, 128, 128, gdn.GDN_FP32) == 0
    assert sc(65536, 1, 3, 32, 128, 128, gdn.GDN_BF16) == 0          # rejected shape
    L = sc(65536, 1, 16, 32, 128, 128, gdn.GDN_BF16)
    assert L >= 8
    # enough segments per sequence for the CU count, never shorter than 8 chunks
    assert sc(64 * 8, 1, 16, 32, 128, 128, gdn.GDN_BF16) == 8
    assert sc(64 * 100000, 1, 16, 32, 128, 128, gdn.GDN_BF16) >= sc(65536, 1, 16, 32, 128, 128, gdn.GDN_BF16)


def _prefill(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, cu=FAKE, n=2, T=100, hqk=16, hv=32, dk=128,
             dv=128, scale=1.0, dt=gdn.GDN_BF16, out=FAKE, fin=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return lib.gdn_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["n"], a["T"],
                           a["hqk"], a["hv"], a["dk"], a["dv"], a["scale"], a["dt"], a["out"], a["fin"],
                           a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(hqk=3), gdn.GDN_ERR_INVALID_ARG),                 # Hv not a multiple of Hqk
    (dict(hqk=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(T=-5), gdn.GDN_ERR_INVALID_ARG),
    (dict(n=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(dt=7), gdn.GDN_ERR_INVALID_ARG),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(out=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(cu=None, n=2), gdn.GDN_ERR_INVALID_ARG),          # no offsets needs exactly one sequence
    (dict(dk=64, dv=64), gdn.GDN_ERR_UNSUPPORTED),          # bf16 path is d = 128
    (dict(dk=128, dv=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dt=gdn.GDN_FP32, dk=48, dv=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(ws=None), gdn.GDN_ERR_WORKSPACE),
    (dict(wsb=1024), gdn.GDN_ERR_WORKSPACE),
    (dict(T=1 << 33), gdn.GDN_ERR_UNSUPPORTED),             # int32 offsets
])
def test_prefill_rejects(lib, over, status):
    assert _prefill(lib, **over) == status


def test_prefill_with_no_sequences_is_a_no_op(lib):
    assert _prefill(lib, n=0) == gdn.GDN_OK


def _decode(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, n=4, hqk=16, hv=32, dk=128, dv=128,
             scale=1.0, dt=gdn.GDN_BF16, out=FAKE, stream=None)
    a.update(over)
    return lib.gdn_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["n"], a["hqk"],
                               a["hv"], a["dk"], a["dv"], a["scale"], a["dt"], a["out"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(hqk=5), gdn.GDN_ERR_INVALID_ARG),
    (dict(n=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(state=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(out=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(dt=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=100, dv=100), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dk=128, dv=64), gdn.GDN_ERR_UNSUPPORTED),
])
def test_decode_rejects(lib, over, status):
    assert _decode(lib, **over) == status


def test_decode_with_no_sequences_is_a_no_op(lib):
    assert _decode(lib, n=0) == gdn.GDN_OK


def _decode_slots(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, idx=FAKE, slots=8, n=4, hqk=16, hv=32, dk=128,
             dv=128, scale=1.0, dt=gdn.GDN_BF16, out=FAKE, stream=None)
    a.update(over)
    return lib.gdn_decode_step_slots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["idx"], a["slots"],
                                     a["n"], a["hqk"], a["hv"], a["dk"], a["dv"], a["scale"], a["dt"], a["out"],
                                     a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(slots=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(idx=None), gdn.GDN_ERR_INVALID_ARG),              # indices are required with sequences
    (dict(pool=None), gdn.GDN_ERR_INVALID_ARG),             # a non-empty pool needs its pointer
    (dict(hqk=5), gdn.GDN_ERR_INVALID_ARG),
    (dict(out=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=100, dv=100), gdn.GDN_ERR_UNSUPPORTED),
])
def test_decode_slots_rejects(lib, over, status):
    assert _decode_slots(lib, **over) == status


def test_decode_slots_with_no_sequences_is_a_no_op(lib):
    assert _decode_slots(lib, n=0, idx=None) == gdn.GDN_OK


def _decode_multi(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, idx=None, slots=0, n=4, tk=3, hqk=16, hv=32,
             dk=128, dv=128, scale=1.0, dt=gdn.GDN_BF16, out=FAKE, ts=None, stream=None)
    a.update(over)
    return lib.gdn_decode_multi(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["idx"], a["slots"],
                                a["n"], a["tk"], a["hqk"], a["hv"], a["dk"], a["dv"], a["scale"], a["dt"], a["out"],
                                a["ts"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(tk=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(tk=65), gdn.GDN_ERR_UNSUPPORTED),                 # long runs belong to the chunked prefill
    (dict(state=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(idx=FAKE, slots=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(idx=FAKE, slots=4, state=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(hqk=5), gdn.GDN_ERR_INVALID_ARG),
    (dict(out=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=100, dv=100), gdn.GDN_ERR_UNSUPPORTED),
])
def test_decode_multi_rejects(lib, over, status):
    assert _decode_multi(lib, **over) == status


def test_decode_multi_with_no_sequences_is_a_no_op(lib):
    assert _decode_multi(lib, n=0) == gdn.GDN_OK


def test_unknown_flags_are_rejected(lib):
    st = lib.gdn_prefill_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, FAKE, 2, 100, 16, 32, 128, 128,
                            1.0, gdn.GDN_BF16, 0x2, FAKE, FAKE, 1 << 40, None)
    assert st == gdn.GDN_ERR_INVALID_ARG
    st = lib.gdn_decode_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 1, 16, 32, 128, 128, 1.0, gdn.GDN_BF16,
                           0x80000000, FAKE, None, None)
    assert st == gdn.GDN_ERR_INVALID_ARG
    # the general decode keeps the token-count checks of gdn_decode_multi
    st = lib.gdn_decode_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 0, 16, 32, 128, 128, 1.0, gdn.GDN_BF16,
                           gdn.GDN_FLAG_QK_L2NORM, FAKE, None, None)
    assert st == gdn.GDN_ERR_INVALID_ARG


def _backward(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, cu=FAKE, n=2, T=100, hqk=16, hv=32, dk=128, dv=128,
             scale=1.0, dt=gdn.GDN_BF16, dout=FAKE, dfin=None, dq=FAKE, dkk=FAKE, dvv=FAKE, dg=FAKE, db=FAKE,
             dinit=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return lib.gdn_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["n"], a["T"], a["hqk"],
                            a["hv"], a["dk"], a["dv"], a["scale"], a["dt"], a["dout"], a["dfin"], a["dq"], a["dkk"],
                            a["dvv"], a["dg"], a["db"], a["dinit"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(hqk=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(dout=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(dq=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(cu=None, n=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=100, dv=100), gdn.GDN_ERR_UNSUPPORTED),
    (dict(ws=None), gdn.GDN_ERR_WORKSPACE),
    (dict(wsb=1024), gdn.GDN_ERR_WORKSPACE),
])
def test_backward_rejects(lib, over, status):
    assert _backward(lib, **over) == status


def test_backward_workspace_size(lib):
    ws = gdn.gdn_backward_workspace_size
    # state and state-gradient checkpoints per 16-token chunk (plus one per sequence), dq and dk
    # per V head (summed over the V heads of each QK head at the end), and per chunk and V head
    # its factors (four 16-vectors and three 16 x 16 matrices in fp32: 3328 bytes)
    slots = 4096 // 16 + 1
    assert ws(4096, 1, 16, 32, 128, 128, gdn.GDN_BF16) == (2 * slots * 32 * 128 * 128 * 4
                                                          + 2 * 4096 * 32 * 128 * 4 + slots * 32 * 3328)
    assert ws(100, 1, 3, 32, 128, 128, gdn.GDN_BF16) == 0


def _prefill_slots(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, idx=FAKE, has=None, slots=8, cu=FAKE, n=2,
             T=100, hqk=16, hv=32, dk=128, dv=128, scale=1.0, dt=gdn.GDN_BF16, out=FAKE, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(over)
    return lib.gdn_prefill_slots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["idx"], a["has"],
                                 a["slots"], a["cu"], a["n"], a["T"], a["hqk"], a["hv"], a["dk"], a["dv"],
                                 a["scale"], a["dt"], a["out"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(slots=-2), gdn.GDN_ERR_INVALID_ARG),
    (dict(idx=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(pool=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(hqk=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(cu=None, n=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=64, dv=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(ws=None), gdn.GDN_ERR_WORKSPACE),
])
def test_prefill_slots_rejects(lib, over, status):
    assert _prefill_slots(lib, **over) == status


def test_python_binding_raises_on_bad_dtype():
    import torch
    q = torch.zeros(4, 2, 128, dtype=torch.float16)
    with pytest.raises(TypeError):
        gdn.gdn_prefill(q, q, q, q, q)


def _conv(lib, **over):
    a = dict(x=FAKE, w=FAKE, hin=None, cu=FAKE, n=2, T=100, hqk=16, hv=32, dk=128, dv=128, K=4, dt=gdn.GDN_BF16,
             flags=0, q=FAKE, k=FAKE, v=FAKE, hout=None, stream=None)
    a.update(over)
    return lib.gdn_conv_prologue(a["x"], a["w"], a["hin"], a["cu"], a["n"], a["T"], a["hqk"], a["hv"], a["dk"],
                                 a["dv"], a["K"], a["dt"], a["flags"], a["q"], a["k"], a["v"], a["hout"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(x=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(w=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(K=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(K=5), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dk=100, dv=100), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dk=128, dv=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(flags=0x4), gdn.GDN_ERR_INVALID_ARG),
    (dict(cu=None, n=3, T=100), gdn.GDN_ERR_INVALID_ARG),   # 100 tokens are not 3 equal sequences
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(n=0, T=5), gdn.GDN_ERR_INVALID_ARG),
])
def test_conv_prologue_rejects(lib, over, status):
    assert _conv(lib, **over) == status


def test_conv_prologue_with_no_sequences_is_a_no_op(lib):
    assert _conv(lib, n=0, T=0) == gdn.GDN_OK


def _dconv(lib, **over):
    a = dict(x=FAKE, w=FAKE, hin=None, hout=None, g=FAKE, b=FAKE, s=FAKE, n=2, hqk=16, hv=32, dk=128, dv=128, K=4,
             scale=1.0, dt=gdn.GDN_BF16, flags=0, out=FAKE, stream=None)
    a.update(over)
    return lib.gdn_decode_conv(a["x"], a["w"], a["hin"], a["hout"], a["g"], a["b"], a["s"], a["n"], a["hqk"],
                               a["hv"], a["dk"], a["dv"], a["K"], a["scale"], a["dt"], a["flags"], a["out"],
                               a["stream"])


# History of 2 sequences x 3 rows x 8192 channels x 2 bytes = 98,304 bytes.
@pytest.mark.parametrize("over,status", [
    (dict(x=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(w=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(s=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(out=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(K=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(K=5), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dk=100, dv=100), gdn.GDN_ERR_UNSUPPORTED),
    (dict(hqk=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(flags=0x4), gdn.GDN_ERR_INVALID_ARG),
    (dict(hin=ctypes.c_void_p(0x100000), hout=ctypes.c_void_p(0x100000)), gdn.GDN_ERR_INVALID_ARG),
    (dict(hin=ctypes.c_void_p(0x100000), hout=ctypes.c_void_p(0x100000 + 98303)), gdn.GDN_ERR_INVALID_ARG),
    (dict(hin=ctypes.c_void_p(0x100000 + 98303), hout=ctypes.c_void_p(0x100000)), gdn.GDN_ERR_INVALID_ARG),
])
def test_decode_conv_rejects(lib, over, status):
    assert _dconv(lib, **over) == status


def test_decode_conv_with_no_sequences_is_a_no_op(lib):
    assert _dconv(lib, n=0) == gdn.GDN_OK
    # histories that merely touch (one ends where the other starts) do not overlap; with no
    # sequences nothing is enqueued either way
    assert _dconv(lib, n=0, hin=ctypes.c_void_p(0x100000), hout=ctypes.c_void_p(0x100000 + 98304)) == gdn.GDN_OK


def test_noalloc_rejects_sizes_beyond_its_array(lib):
    # 2,000 sequences of the layer's head shape need far more segment workspace than the static array.
    need = gdn.gdn_prefill_workspace_size(2_000_000, 2000, 16, 32, 128, 128, gdn.GDN_BF16)
    assert need > gdn.GDN_PREFILL_NOALLOC_SCRATCH_BYTES
    st = lib.gdn_prefill_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 2000, 2_000_000, 16, 32, 128, 128, 1.0,
                                 gdn.GDN_BF16, FAKE, None, None)
    assert st == gdn.GDN_ERR_SCRATCH_LIMIT
    assert "static array" in gdn.gdn_status_string(st)
    # invalid arguments are still gdn_prefill's errors
    st = lib.gdn_prefill_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 100, 3, 32, 128, 128, 1.0,
                                 gdn.GDN_BF16, FAKE, None, None)
    assert st == gdn.GDN_ERR_INVALID_ARG

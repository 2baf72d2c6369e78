"""In-kernel q/k L2 normalisation (GDN_FLAG_QK_L2NORM) against the fp64 oracle
run with the same normalisation, on inputs whose q and k rows have lengths
spread over two decades; and the general entry points with no flags against
the plain ones, bit for bit."""
import numpy as np
import pytest
import torch

import linear_attention_sequence_02_amd as gdn
import oracle
from synth import inputs as I
from tests.gpu_util import log, rel_l2, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}
F = gdn.GDN_FLAG_QK_L2NORM


def _ref(x):
    return oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, scale=x.scale, qk_l2norm=True)


@pytest.mark.parametrize("dtype,d,lengths", [
    ("bf16", 128, [1100, 0, 260, 700]),    # several segments per sequence, an empty one
    ("fp32", 64, [70, 1, 130, 64]),
])
def test_prefill_qk_norm(dtype, d, lengths):
    x = I.draw(lengths=lengths, hqk=2, hv=4, dk=d, dtype=dtype, seed=300 + d, s0_std=0.3, qk_unit=False,
               name=f"prefill_qknorm_{dtype}_d{d}")
    dev = to_device(x)
    fin = torch.empty_like(dev["s0"])
    log(f"[gpu] gdn_prefill_ex qk_l2norm {x.name} T={x.T}")
    out = gdn.gdn_prefill_ex(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["s0"], fin, None, None,
                             dev["cu"], flags=F, scale=x.scale)
    torch.cuda.synchronize()
    ref_o, ref_f = _ref(x)
    eo = rel_l2(out.float().cpu().numpy(), ref_o)
    ef = rel_l2(fin.cpu().numpy(), ref_f)
    log(f"[parity] {x.name}: out rel={eo:.3e} state rel={ef:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


@pytest.mark.parametrize("dtype,tk", [("bf16", 1), ("fp32", 1), ("bf16", 3), ("fp32", 4)])
def test_decode_qk_norm(dtype, tk):
    x = I.draw(lengths=[tk] * 6, hqk=2, hv=4, dk=128, dtype=dtype, seed=310 + tk, s0_std=0.3, qk_unit=False,
               name=f"decode_qknorm_{dtype}_k{tk}")
    dev = to_device(x)
    state = dev["s0"].clone()
    log(f"[gpu] gdn_decode_ex qk_l2norm {x.name}")
    out, _ = gdn.gdn_decode_ex(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, num_tokens=tk, flags=F,
                               scale=x.scale)
    torch.cuda.synchronize()
    ref_o, ref_f = _ref(x)
    eo = rel_l2(out.float().cpu().numpy(), ref_o)
    ef = rel_l2(state.cpu().numpy(), ref_f)
    log(f"[parity] {x.name}: out rel={eo:.3e} state rel={ef:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


def test_general_forms_without_flags_are_the_plain_calls():
    x = I.draw(lengths=[700, 90], hqk=2, hv=4, dk=128, dtype="bf16", seed=320, s0_std=0.3, name="ex_vs_plain")
    dev = to_device(x)
    log(f"[gpu] gdn_prefill_ex / gdn_prefill {x.name}")
    o1, f1 = gdn.gdn_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["s0"], dev["cu"])
    f2 = torch.empty_like(f1)
    o2 = gdn.gdn_prefill_ex(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["s0"], f2, None, None,
                            dev["cu"])
    y = I.draw(lengths=[1] * 5, hqk=2, hv=4, dk=128, dtype="bf16", seed=321, s0_std=0.3, name="ex_vs_plain_dec")
    dy = to_device(y)
    s1, s2 = dy["s0"].clone(), dy["s0"].clone()
    d1 = gdn.gdn_decode_step(dy["q"], dy["k"], dy["v"], dy["g"], dy["beta"], s1)
    d2, _ = gdn.gdn_decode_ex(dy["q"], dy["k"], dy["v"], dy["g"], dy["beta"], s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    assert torch.equal(d1, d2) and torch.equal(s1, s2)

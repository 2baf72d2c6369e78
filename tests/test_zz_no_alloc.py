"""gdn_prefill_noalloc (the entry point that allocates nothing: its workspace is the library's static
device array) against gdn_prefill with a caller workspace, on two calls in a row, the second with a
smaller input, so the second call runs over the first call's leftovers in the shared array."""
import numpy as np
import pytest
import torch

import linear_attention_sequence_02_amd as gdn
from synth import inputs as I
from tests.gpu_util import log, rel_l2, to_device

pytestmark = pytest.mark.gpu


def _both(x):
    d = to_device(x)
    log(f"[gpu] gdn_prefill (workspace) {x.name} T={x.T} N={x.num_seqs}")
    out_a, fin_a = gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["cu"], scale=x.scale)
    out_b = torch.empty_like(out_a)
    fin_b = torch.empty_like(fin_a)
    log(f"[gpu] gdn_prefill_noalloc {x.name}")
    gdn.gdn_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["cu"], out=out_b,
                            final_state=fin_b, scale=x.scale)
    torch.cuda.synchronize()
    return out_a, fin_a, out_b, fin_b


def test_prefill_noalloc_matches_workspace_entry_point():
    big = I.draw(lengths=[5000, 3192], hqk=16, hv=32, dk=128, dtype="bf16", seed=1030, s0_std=0.1,
                 name="noalloc_layer_T8192")
    small = I.draw(lengths=[400, 0, 300], hqk=2, hv=4, dk=128, dtype="bf16", seed=1031, s0_std=0.1,
                   name="noalloc_small")
    for x in (big, small):
        need = gdn.gdn_prefill_workspace_size(x.T, x.num_seqs, x.hqk, x.hv, x.dk, x.dv, gdn.GDN_BF16)
        assert 0 < need <= gdn.GDN_PREFILL_NOALLOC_SCRATCH_BYTES
        out_a, fin_a, out_b, fin_b = _both(x)
        oa, ob = out_a.float().cpu().numpy(), out_b.float().cpu().numpy()
        fa, fb = fin_a.cpu().numpy(), fin_b.cpu().numpy()
        eo, ef = rel_l2(ob, oa), rel_l2(fb, fa)
        log(f"[parity] {x.name}: no-alloc vs workspace out {eo:.3e} state {ef:.3e}")
        assert eo <= 1e-2 and ef <= 1e-2
        # same kernels, same segment schedule: the results are identical
        assert np.array_equal(oa, ob) and np.array_equal(fa, fb)

"""The binding rejects mismatched shapes on the host, before any library call (CPU tensors suffice:
every check runs before a device pointer is used)."""
import pytest
import torch

import linear_attention_sequence_02_amd as gdn


def _inputs(T=10, hqk=2, hv=4, d=16, n=1):
    bf = dict(dtype=torch.bfloat16)
    f = dict(dtype=torch.float32)
    return dict(q=torch.zeros(T, hqk, d, **bf), k=torch.zeros(T, hqk, d, **bf), v=torch.zeros(T, hv, d, **bf),
                g=torch.zeros(T, hv, **f), beta=torch.zeros(T, hv, **f), s=torch.zeros(n, hv, d, d, **f))


@pytest.mark.parametrize("bad", ["k", "v", "g", "beta"])
def test_prefill_token_rows(bad):
    x = _inputs()
    x[bad] = x[bad][:-1].contiguous()
    with pytest.raises(ValueError, match=bad):
        gdn.gdn_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"])


def test_prefill_state_shapes():
    x = _inputs(n=2)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="initial_state"):
        gdn.gdn_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s"][:1].contiguous(), cu)
    with pytest.raises(ValueError, match="final_state"):
        gdn.gdn_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s"], cu,
                        final_state=torch.zeros(1, 4, 16, 16))
    with pytest.raises(ValueError, match="out"):
        gdn.gdn_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s"], cu,
                        out=torch.zeros(10, 3, 16, dtype=torch.bfloat16))


def test_decode_state_and_indices():
    x = _inputs(T=3, n=3)
    with pytest.raises(ValueError, match="state"):
        gdn.gdn_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s"][:2].contiguous())
    pool = torch.zeros(8, 4, 16, 16)
    with pytest.raises(ValueError, match="state_indices"):
        gdn.gdn_decode_step_slots(x["q"], x["k"], x["v"], x["g"], x["beta"], pool,
                                  torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="state_pool"):
        gdn.gdn_decode_step_slots(x["q"], x["k"], x["v"], x["g"], x["beta"], torch.zeros(8, 4, 16, 8),
                                  torch.zeros(3, dtype=torch.int32))


def test_prefill_pools_must_match():
    x = _inputs()
    idx = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="pools differ"):
        gdn.gdn_prefill_ex(x["q"], x["k"], x["v"], x["g"], x["beta"], torch.zeros(8, 4, 16, 16),
                           torch.zeros(4, 4, 16, 16), idx)
    with pytest.raises(ValueError, match="has_initial_state"):
        gdn.gdn_prefill_slots(x["q"], x["k"], x["v"], x["g"], x["beta"], torch.zeros(8, 4, 16, 16), idx,
                              torch.zeros(2, dtype=torch.int32))


def test_multi_token_states():
    x = _inputs(T=6, n=3)
    with pytest.raises(ValueError, match="token_states"):
        gdn.gdn_decode_multi(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s"], 2,
                             token_states=torch.zeros(5, 4, 16, 16))
    with pytest.raises(ValueError, match="state"):
        gdn.gdn_decode_multi(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s"], 3)


def test_backward_d_out():
    x = _inputs()
    with pytest.raises(ValueError, match="d_out"):
        gdn.gdn_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], torch.zeros(9, 4, 16, dtype=torch.bfloat16))

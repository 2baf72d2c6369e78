"""The benchmark's accounting, checked without a GPU: the algorithmic work per token and per step that
every roofline fraction divides by, re-derived here from the layer's shapes, the split of tokens
between the segment launches, and the one-GPU contract of the command line."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HQK, HV, D, C = 16, 32, 128, 64


def test_prefill_flop_per_token():
    # per QK head: the two lower-triangular Gram products (K K^T, Q K^T) at C d each;
    # per V head: T K, T V and (P) U at C d each, and W S^T, Q S^T, U^T K at 2 d^2 each
    per_qk = 2 * C * D
    per_v = 3 * C * D + 3 * 2 * D * D
    assert bench.PREFILL_FLOP_PER_TOKEN == HQK * per_qk + HV * per_v == 4_194_304


def test_prefill_work_follows_the_head_counts():
    assert bench.prefill_work_per_token(16, 32, 128) == (bench.PREFILL_FLOP_PER_TOKEN, bench.PREFILL_BYTES_PER_TOKEN)
    # one GPU's share under tensor parallelism 4 does a quarter of the layer's work per token
    f4, b4 = bench.prefill_work_per_token(4, 8, 128)
    assert 4 * f4 == bench.PREFILL_FLOP_PER_TOKEN and 4 * b4 == bench.PREFILL_BYTES_PER_TOKEN


def test_prefill_bytes_per_token():
    # q, k (bf16, per QK head), v and out (bf16, per V head), g and beta (fp32, per V head)
    assert bench.PREFILL_BYTES_PER_TOKEN == 2 * HQK * D * 2 + 2 * HV * D * 2 + 2 * HV * 4 == 24_832


def test_decode_bytes():
    n = 256
    state = 2 * n * HV * D * D * 4                     # read and written once, fp32
    others = n * (2 * HQK * D * 2 + 2 * HV * D * 2 + 2 * HV * 4)
    assert bench.decode_bytes(n) == state + others == 1_080_098_816
    # k tokens per sequence: the state once, every token's inputs and outputs
    assert bench.decode_bytes(n, tokens=4) == state + 4 * others == 1_099_169_792


def test_backward_flop_per_token():
    assert bench.BACKWARD_FLOP_PER_TOKEN == 17 * D * D * HV


class _X:
    def __init__(self, lengths):
        self.cu_seqlens = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        self.T = int(sum(lengths))
        self.num_seqs = len(lengths)


def test_launch_tokens_split():
    L = 114
    # one sequence of 65,536 tokens: the first segment's 7,296 tokens are produced by the map launch
    assert bench.launch_tokens(_X([65536]), L) == {"gdn_segment_maps": 64 * L,
                                                   "gdn_segment_out": 65536 - 64 * L}
    # a sequence that fits one segment runs the output launch only
    assert bench.launch_tokens(_X([4000]), L) == {"gdn_segment_out": 4000}
    # several sequences: each one's first segment in the map launch
    got = bench.launch_tokens(_X([100, 8000, 0]), 8)
    assert got == {"gdn_segment_maps": 100 + 512, "gdn_segment_out": 8000 - 512}


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""

"""Benchmark of the Gated DeltaNet token mixer on one MI355X.

One step = one gdn_prefill call over the Qwen3-Next GDN layer at T = 65536
(B = 1, 16 QK / 32 V heads, d = 128, bf16 q/k/v, fp32 g/beta/state, chunk 64)
with every input resident in HBM. The decode step (256 sequences x 32 heads,
512 MiB fp32 state updated in place) is timed separately and reported under
"decode". Per-kernel durations come from the library's HIP-event
instrumentation (events around each launch, on the stream the kernels run on)
over a second run of the same steps.

Roofline figures use algorithmic work only:
  prefill: 4,194,304 flop and 24,832 bytes per token. The bf16 prefill runs
      segment-parallel in three launches: the first produces the outputs of
      each sequence's first segment and the maps of the other segments, a
      combine, and the output pass for segments 1 onward. The roofline object
      is the output pass ("gdn_segment_out"), priced at 4,194,304 flop per
      token it produces (all tokens but the first segment's, whose length
      comes from gdn_prefill_segment_chunks); the map pass and the combine are
      extra work of the schedule and count only in "prefill_path".
  decode: 1,080,098,816 bytes per step for 256 sequences (state read + write
      plus q, k, v, g, beta, out); also on a state pool addressed by slot
      ("decode.slots"), and as eager calls against graph replays, wall clock
      per step ("decode.graph_replay", 256 and 8 sequences; a graph holds 16 steps)
  multi-token decode ("decode_multi"): 4 tokens per sequence from one state,
      256 sequences: the state read and written once plus 4 tokens' inputs and
      outputs, 1,099,169,792 bytes per step
  short prefill ("prefill_graph_replay"): the T = 4096 layer, eager calls against
      replays of a graph holding 16 calls, wall clock per step
  backward ("backward"): gradients of the prefill on the T = 4096 layer shape,
      against the fp32 peak (157.3 TFLOP/s) at 17 d^2 flop per token and V head
      (the recomputation of forward states not counted), over its four kernels
  with q and k L2-normalised in the kernels ("prefill_qk_l2norm",
      "decode.qk_l2norm"): the same inputs and algorithmic work
Peaks: bf16 dense MFMA 2516.6 TFLOP/s, HBM 8.0 TB/s.
"step_ms" gives the mean, median and min of the prefill step over a further pass
with events around each call (so its mean can differ from "ms_per_step", the
timed run's). The timed run behind `value` has no
per-kernel instrumentation; the per-kernel launch times come from a separate
run of the same number of steps. "parity" is the rel-L2 (fp64) of the timed
run's output, and of its final state when the oracle sample covers the
whole input, against the fp64 oracle run for "cpu_baseline" on the same
inputs ("cpu_baseline" also gives the oracle on one core and the host CPU model).
HBM traffic per launch ("traffic") comes from rocprofv3 FETCH_SIZE and
WRITE_SIZE passes recorded in profiles/traffic.json, scaled by the same
counters read for a plain device copy of known size (--calibration-copy); it
is reported only while the kernel source matches the recorded hash.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s at T=64K (16 QK/32 V heads, d=128); decode GB/s vs peak"
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PREFILL_FLOP_PER_TOKEN = 4_194_304
PREFILL_BYTES_PER_TOKEN = 24_832
PEAK_FP32_VECTOR_TFLOPS = 157.3
# Backward, per token over all 32 V heads (d = 128): the reverse step's products with the state
# (S k, dS update by do q^T, dS k, S^T do, dS^T u and S^T du, <dS, S>, the dS recurrence) at
# 17 d^2 flop per V head; the recomputation of the forward states is the implementation's own.
BACKWARD_FLOP_PER_TOKEN = 17 * 128 * 128 * 32
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"gdn_segment_out": "gdn_segment.hip", "gdn_segment_maps": "gdn_segment.hip",
                  "gdn_decode_step": "gdn_decode.hip", "gdn_decode_multi": "gdn_decode.hip"}


def decode_bytes(n, hqk=16, hv=32, d=128, tokens=1):
    """Algorithmic bytes of one decode call: each state read and written once, and per token q, k
    (bf16), v, out (bf16) and g, beta (fp32)."""
    state = n * hv * d * d * 4 * 2
    other = n * tokens * (2 * hqk * d * 2 + hv * d * 2 + hv * d * 2 + hv * 4 * 2)
    return state + other


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_calls(fn, steps, warmup, torch, profile=True, per_step=None):
    """Mean ms per call over `steps` back-to-back calls, HIP events on the current stream around the
    whole run and nothing else inside it (this is the number `value` comes from). If `profile`, a
    second run of `steps` calls with the library's per-launch HIP events on gives each kernel's mean
    launch time (the roofline's figure). If `per_step` is a list, a third run brackets each call with
    its own events and appends the per-call times (median and min)."""
    import linear_attention_sequence_02_amd as gdn
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    kernels = {}
    if profile:
        gdn.gdn_profile_start()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        kernels = gdn.gdn_profile_stop()
    if per_step is not None:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        per_step.extend(a.elapsed_time(b) for a, b in ev)
    return ms, {k: (c, t / c) for k, (c, t) in kernels.items()}


def graph_vs_eager(fn, steps, torch, per_graph=16):
    """Microseconds per step: eager calls back to back, against replays of one HIP graph holding
    `per_graph` consecutive calls (captured on a side stream after one warm-up call), about `steps`
    calls of each."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    res = {"calls_per_graph": per_graph}
    for name, call, n_calls in (("eager_us_per_step", fn, reps * per_graph), ("graph_us_per_step", graph.replay, reps)):
        call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_calls):
            call()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / (reps * per_graph) * 1e6
    return res


def source_hash(kernel):
    import hashlib
    src = KERNEL_SOURCES.get(kernel)
    if src is None:
        return None
    h = hashlib.sha256()
    for f in (src, "gdn_mfma.h", "gdn_common.h"):
        path = os.path.join(ROOT, "linear_attention_sequence_02_amd", "csrc", f)
        if os.path.exists(path):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 for this kernel source, or None."""
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def to_device(x, dev):
    import torch
    if x.dtype == "bf16":
        def qkv(a):
            return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)
    else:
        def qkv(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return dict(q=qkv(x.q), k=qkv(x.k), v=qkv(x.v), g=torch.from_numpy(x.g).to(dev),
                beta=torch.from_numpy(x.beta).to(dev),
                s0=None if x.s0 is None else torch.from_numpy(x.s0).to(dev),
                cu=torch.from_numpy(x.cu_seqlens).to(dev))


def cpu_baseline(x, budget_s=20.0):
    """The fp64 oracle, as it is, on the host cores: a prefix of the same
    workload (all 32 heads), grown until it takes a few seconds, scaled to tokens/s."""
    import oracle
    T = 512
    while True:
        t0 = time.perf_counter()
        o_ref, s_ref, threads = oracle.recurrent(x.q[:T], x.k[:T], x.v[:T], x.g[:T], x.beta[:T], None, None,
                                                 scale=x.scale, return_threads=True)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or T >= x.T:
            break
        T = min(x.T, int(T * max(2.0, budget_s / 4 / max(dt, 1e-3))))
    base = {"value": T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {T} of {x.T} tokens of the same input, all {x.hv} V heads, fp64 recurrence, "
                      f"{dt:.1f} s"}
    # The same oracle on one core, over a shorter prefix (about a second of work).
    T1 = max(16, min(x.T, int(T / dt / max(int(threads), 1))))
    t0 = time.perf_counter()
    oracle.recurrent(x.q[:T1], x.k[:T1], x.v[:T1], x.g[:T1], x.beta[:T1], None, None, scale=x.scale, threads=1)
    base["one_core"] = {"value": T1 / (time.perf_counter() - t0), "unit": "tokens/s", "sample": f"first {T1} tokens"}
    base["cpu_model"] = cpu_model()
    return base, T, o_ref, (s_ref if T == x.T else None)


def cpu_model():
    """The host CPU's model name as the kernel reports it (None where /proc/cpuinfo has none)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def rel_l2(a, ref):
    """||a - ref||_2 / ||ref||_2 in fp64."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((a - ref).ravel()) / np.linalg.norm(ref.ravel()))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--T", type=int, default=65536)
    ap.add_argument("--decode-seqs", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one 256 MiB device-to-device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the Gated DeltaNet layer "
              "shards by heads or sequences with no exchange inside the mixer, so this build times the "
              "one-GPU share.", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_sequence_02_amd as gdn
    from synth import inputs as I

    dev = torch.device("cuda:0")
    log(f"[bench] generating T={args.T} inputs")
    x = I.qwen3_next_prefill(T=args.T)
    d = to_device(x, dev)
    out = torch.empty_like(d["v"])
    fin = torch.empty((1, x.hv, x.dv, x.dk), dtype=torch.float32, device=dev)
    ws_bytes = gdn.gdn_prefill_workspace_size(x.T, 1, x.hqk, x.hv, x.dk, x.dv, gdn.GDN_BF16)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)

    def prefill():
        gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, None, out=out, final_state=fin,
                        workspace=ws)

    log(f"[bench] prefill: {args.warmup} warmup + {args.steps} timed steps")
    each = []
    ms, kern = time_calls(prefill, args.steps, args.warmup, torch, per_step=each)
    tokens_per_s = x.T / (ms / 1e3)
    by_time = max(kern, key=lambda k_: kern[k_][0] * kern[k_][1]) if kern else None
    seg_chunks = gdn.gdn_prefill_segment_chunks(x.T, 1, x.hqk, x.hv, x.dk, x.dv, gdn.GDN_BF16)
    out_tokens = x.T - min(x.T, 64 * seg_chunks) if "gdn_segment_maps" in kern else x.T
    dom = "gdn_segment_out"
    dom_ms = kern[dom][1] if dom in kern else float("nan")
    dom_tflops = PREFILL_FLOP_PER_TOKEN * out_tokens / (dom_ms / 1e3) / 1e12
    path_tflops = PREFILL_FLOP_PER_TOKEN * x.T / (ms / 1e3) / 1e12
    path_gbs = PREFILL_BYTES_PER_TOKEN * x.T / (ms / 1e3) / 1e9
    workload = f"qwen3next_gdn_prefill_T{x.T}"
    log(f"[bench] prefill {ms:.3f} ms/step, {tokens_per_s:.3e} tokens/s; kernels {kern}")

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "batch": 1, "seq_len": x.T,
                   "num_qk_heads": x.hqk, "num_v_heads": x.hv, "head_dim": x.dk, "chunk": 64,
                   "seed": x.seed, "initial_state": "zeros"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": dom_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": dom_tflops / PEAK_BF16_TFLOPS,
                     "traffic": recorded_traffic(dom, workload), "ms_per_launch": dom_ms,
                     "tokens_per_launch": out_tokens, "flop_per_launch": PREFILL_FLOP_PER_TOKEN * out_tokens,
                     "longest_launch": by_time, "segment_chunks": seg_chunks},
        "step_ms": {"mean": float(np.mean(each)), "median": float(np.median(each)), "min": float(np.min(each)),
                    "n": len(each)},
        "prefill_path": {"tflops_algorithmic": path_tflops, "frac_mfma_peak": path_tflops / PEAK_BF16_TFLOPS,
                         "gbs_algorithmic": path_gbs, "frac_hbm_peak": path_gbs / PEAK_HBM_GBS,
                         "kernels_ms_per_launch": {k_: v_[1] for k_, v_ in kern.items()}},
    }
    out_host = out.view(torch.int16).cpu().numpy()
    fin_host = fin.cpu().numpy()

    # The same step with q and k L2-normalised in the kernels (GDN_FLAG_QK_L2NORM), on the same inputs.
    out_n, fin_n = torch.empty_like(out), torch.empty_like(fin)

    def prefill_norm():
        gdn.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, fin_n, None, None, None,
                           flags=gdn.GDN_FLAG_QK_L2NORM, out=out_n, workspace=ws)

    nms, nkern = time_calls(prefill_norm, args.steps, args.warmup, torch)
    result["prefill_qk_l2norm"] = {"ms_per_step": nms, "tokens_per_s": x.T / (nms / 1e3),
                                   "relative_to_plain": nms / ms,
                                   "kernels_ms_per_launch": {k_: v_[1] for k_, v_ in nkern.items()}}
    log(f"[bench] prefill with in-kernel q/k normalisation {nms:.3f} ms/step")
    del out_n, fin_n
    del d, out, fin, ws
    torch.cuda.empty_cache()

    if not args.no_decode:
        n = args.decode_seqs
        log(f"[bench] decode: {n} sequences")
        y = I.decode_batch(n)
        dd = to_device(y, dev)
        state = dd["s0"].clone()
        dout = torch.empty_like(dd["v"])

        def decode():
            gdn.gdn_decode_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state, out=dout)

        dms, dkern = time_calls(decode, args.steps, args.warmup, torch)
        kms = dkern.get("gdn_decode_step", (0, dms))[1]
        nbytes = decode_bytes(n)
        gbs = nbytes / (kms / 1e3) / 1e9
        result["decode"] = {"workload": f"qwen3next_gdn_decode_N{n}", "ms_per_step": dms,
                            "kernel_ms_per_launch": kms, "bytes_per_step": nbytes, "GB_per_s": gbs,
                            "frac_hbm_peak": gbs / PEAK_HBM_GBS, "tokens_per_s": n / (dms / 1e3),
                            "roofline": {"kernel": "gdn_decode_step", "bound": "hbm", "achieved": gbs,
                                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                         "traffic": recorded_traffic("gdn_decode_step", f"qwen3next_gdn_decode_N{n}")}}
        log(f"[bench] decode {dms:.3f} ms/step, {gbs:.1f} GB/s")

        # The same step on a state pool: the 256 sequences' states are 256 scattered rows of a
        # 384-row pool (seeded choice), addressed by slot index.
        slots = 384
        pool = torch.zeros((slots,) + tuple(dd["s0"].shape[1:]), dtype=torch.float32, device=dev)
        idx = torch.from_numpy(np.random.default_rng(7).choice(slots, size=n, replace=False).astype(np.int32)).to(dev)
        pool[idx.long()] = dd["s0"]

        def decode_slots():
            gdn.gdn_decode_step_slots(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], pool, idx, out=dout)

        sms, skern = time_calls(decode_slots, args.steps, args.warmup, torch)
        skms = skern.get("gdn_decode_step", (0, sms))[1]
        st_n = dd["s0"].clone()

        def decode_norm():
            gdn.gdn_decode_ex(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st_n, flags=gdn.GDN_FLAG_QK_L2NORM,
                              out=dout)

        qms, qkern = time_calls(decode_norm, args.steps, args.warmup, torch)
        qkms = qkern.get("gdn_decode_step", (0, qms))[1]
        result["decode"]["qk_l2norm"] = {"ms_per_step": qms, "kernel_ms_per_launch": qkms,
                                         "GB_per_s": nbytes / (qkms / 1e3) / 1e9,
                                         "frac_hbm_peak": nbytes / (qkms / 1e3) / 1e9 / PEAK_HBM_GBS}
        del st_n
        result["decode"]["slots"] = {"pool_slots": slots, "ms_per_step": sms, "kernel_ms_per_launch": skms,
                                     "GB_per_s": nbytes / (skms / 1e3) / 1e9,
                                     "frac_hbm_peak": nbytes / (skms / 1e3) / 1e9 / PEAK_HBM_GBS}
        log(f"[bench] decode on a state pool {sms:.3f} ms/step")
        result["decode"]["graph_replay"] = {f"N{n}": graph_vs_eager(decode_slots, args.steps, torch)}
        del dd, state, dout, pool, idx
        torch.cuda.empty_cache()

        # Launch overhead: a small batch (8 sequences), eager calls against replays of a captured graph.
        y8 = I.decode_batch(8)
        d8 = to_device(y8, dev)
        st8 = d8["s0"].clone()
        o8 = torch.empty_like(d8["v"])

        def decode8():
            gdn.gdn_decode_step(d8["q"], d8["k"], d8["v"], d8["g"], d8["beta"], st8, out=o8)

        result["decode"]["graph_replay"]["N8"] = graph_vs_eager(decode8, args.steps, torch)
        log(f"[bench] decode graph replay {result['decode']['graph_replay']}")
        del d8, st8, o8

        # Multi-token step: 4 tokens per sequence from one state (draft verification), 256 sequences.
        tk = 4
        ym = I.draw(lengths=[tk] * n, hqk=y.hqk, hv=y.hv, dk=y.dk, dtype="bf16", seed=1003, s0_std=0.01,
                    name=f"qwen3next_gdn_decode_multi_N{n}_k{tk}")
        dm = to_device(ym, dev)
        stm = dm["s0"].clone()
        om = torch.empty_like(dm["v"])

        def decode_multi():
            gdn.gdn_decode_multi(dm["q"], dm["k"], dm["v"], dm["g"], dm["beta"], stm, tk, out=om)

        mms, mkern = time_calls(decode_multi, args.steps, args.warmup, torch)
        mkms = mkern.get("gdn_decode_multi", (0, mms))[1]
        mbytes = decode_bytes(n, tokens=tk)
        mgbs = mbytes / (mkms / 1e3) / 1e9
        result["decode_multi"] = {"workload": ym.name, "tokens_per_seq": tk, "ms_per_step": mms,
                                  "kernel_ms_per_launch": mkms, "bytes_per_step": mbytes,
                                  "tokens_per_s": n * tk / (mms / 1e3),
                                  "roofline": {"kernel": "gdn_decode_multi", "bound": "hbm", "achieved": mgbs,
                                               "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": mgbs / PEAK_HBM_GBS,
                                               "traffic": recorded_traffic("gdn_decode_multi", ym.name)}}
        log(f"[bench] multi-token decode {mms:.3f} ms/step, {mgbs:.1f} GB/s")
        del dm, stm, om

    # Launch overhead of a short prefill (the 4,096-token layer: three launches of ~0.04 ms and the
    # combine), eager calls against replays of a captured graph.
    x4 = I.qwen3_next_prefill(T=4096)
    d4 = to_device(x4, dev)
    o4 = torch.empty_like(d4["v"])
    f4 = torch.empty((1, x4.hv, x4.dv, x4.dk), dtype=torch.float32, device=dev)
    ws4 = torch.empty(max(1, gdn.gdn_prefill_workspace_size(x4.T, 1, x4.hqk, x4.hv, x4.dk, x4.dv, gdn.GDN_BF16)),
                      dtype=torch.uint8, device=dev)

    def prefill4():
        gdn.gdn_prefill(d4["q"], d4["k"], d4["v"], d4["g"], d4["beta"], out=o4, final_state=f4, workspace=ws4)

    result["prefill_graph_replay"] = {"workload": "qwen3next_gdn_prefill_T4096",
                                      **graph_vs_eager(prefill4, args.steps, torch)}
    log(f"[bench] prefill T=4096 graph replay {result['prefill_graph_replay']}")
    del d4, o4, f4, ws4

    if not args.no_backward:
        # Backward of the prefill on the 4,096-token Qwen3-Next layer shape (bf16 inputs, fp32 gradients).
        xb = I.qwen3_next_prefill(T=4096)
        db = to_device(xb, dev)
        gout = torch.from_numpy(I.draw(T=4096, hqk=xb.hqk, hv=xb.hv, dk=xb.dk, seed=1007).v).view(torch.bfloat16).to(dev)
        wsb = torch.empty(gdn.gdn_backward_workspace_size(xb.T, 1, xb.hqk, xb.hv, xb.dk, xb.dv, gdn.GDN_BF16),
                          dtype=torch.uint8, device=dev)

        def backward():
            gdn.gdn_backward(db["q"], db["k"], db["v"], db["g"], db["beta"], gout, None, None, workspace=wsb)

        bsteps = max(2, args.steps // 4)
        bms, bkern = time_calls(backward, bsteps, 2, torch)
        # four stages per call: chunk factors, the two scans, the per-chunk gradients, the fixed-order sums
        bparts = {k: bkern[k][1] for k in ("gdn_backward_prep", "gdn_backward_scan", "gdn_backward_grad",
                                            "gdn_backward_sums") if k in bkern}
        bkms = sum(bparts.values()) or bms
        btf = BACKWARD_FLOP_PER_TOKEN * xb.T / (bkms / 1e3) / 1e12
        result["backward"] = {"workload": "qwen3next_gdn_backward_T4096", "steps": bsteps, "ms_per_step": bms,
                              "kernel_ms_per_launch": bparts, "tokens_per_s": xb.T / (bms / 1e3),
                              "roofline": {"kernel": "gdn_backward_prep+scan+grad+sums", "bound": "alu",
                                           "achieved": btf,
                                           "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                                           "frac": btf / PEAK_FP32_VECTOR_TFLOPS}}
        log(f"[bench] backward {bms:.3f} ms/step")
        del db, gout, wsb

    if args.calibration_copy:
        a_ = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b_ = torch.empty_like(a_)
        torch.cuda.synchronize()
        b_.copy_(a_)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written")
        del a_, b_

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle on host cores)")
        base, Tref, o_ref, s_ref = cpu_baseline(x)
        result["cpu_baseline"] = base
        # The timed run's own output against the oracle's (the same inputs): rel-L2 in fp64.
        o_gpu = (out_host[:Tref].astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
        result["parity"] = {"tokens_compared": Tref, "out_rel_l2": rel_l2(o_gpu, o_ref),
                            "state_rel_l2": None if s_ref is None else rel_l2(fin_host, s_ref),
                            "tolerance": 1e-2}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

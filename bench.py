#!/usr/bin/env python3
"""Benchmark of the fused 4-bit-weight GEMV/GEMM library on one MI355X.

The timed step is one replay of the decode step's HIP graph: 48 layers x 7
INT4 linears (q 3840->4096, k and v 3840->2048, o 4096->3840, gate and up
3840->15360, down 15360->3840), group 128, FP16 scale and zero, BF16
activations, M = 1, each linear reading the output it reads in a decoder:
layer 0's q, k and v read one seeded N(0,1) input; o reads q's output, gate
and up read o's, down reads gate's, and the next layer's q, k and v read
down's (attention and the gate/up product are outside this path).  Values
grow about 1000x per layer and overflow BF16 after about a dozen layers;
no kernel's timing depends on the values.  The graph holds one launch of
the persistent decode-chain kernel, in which each GEMV waits for exactly
the output it reads; each layer runs in six stages, q | k, v | o | gate |
up | down (k, v and up, read by no later linear here, stream while o's and
down's inputs are awaited).  Inputs are seeded synthetic data already resident in
device memory.  ``value`` is the algorithmic bytes of one step (packed
weights + scales + zeros + x + y, each once) divided by the measured time
per step.

Also reported, outside the timed step:
  * ``roofline``: the chain kernel's own achieved bandwidth, from HIP events
    around each of its launches on the stream it runs on;
  * ``extra.decode_step_independent_inputs``: the same linears, each reading
    its own N(0,1) input (no GEMV waits for another), in one chain launch;
  * ``extra.decode_step_336_launch_graph``: the same step as a graph of 336
    separate w4_gemv launches, with per-shape kernel timings;
  * ``extra``: the single 3840 x 3840 GEMV (also one cold launch, and all its
    rotated copies as one stage of one chain launch), the
    262144-row logits GEMV, the two M = 128 prefill GEMMs (TFLOP/s) and the
    six-expert FP4 MoE pair, each replayed over rotated weight copies so the
    data comes from HBM (medians of 5 trials);
  * ``extra.hbm_read_probe``: the read rate of a plain streaming read kernel
    over 2 GiB, the measured ceiling for the weight-streaming kernels, and
    ``extra.empty_336_launch_graph_us``, a graph of 336 empty launches (the
    launch floor of the 336-launch step);
  * ``cpu_baseline``: the FP64 oracle timed on host cores on a sample of the
    same step.

    python bench.py [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]
    python bench.py --counters   # only the kernels that HBM counters are read for
    python bench.py --gemm-calls # only w4_gemm at M = 128 and M = 16 on the two decode shapes, 5 calls each,
                                 # then the grouped FP4 GEMM pair (6 x 16 rows), 5 calls

``--counters`` runs five chain-kernel launches of the (timed, linked) decode step, then five
copies of 512 MiB by torch (a plain copy of known size, read once and
written once), for ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``
runs.  The counters' per-launch figures for the chain kernel, scaled by
what the same counters read for the copy, give ``roofline.traffic``; the
result is kept in profiles/chain_kernel_traffic.json together with a hash
of the chain kernel's sources, and ``traffic`` is reported only while that
hash still matches.
"""
from __future__ import annotations

import argparse
import json
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "M=1 W4A16 GEMV achieved HBM GB/s (% of peak) + µs/decode-step; M=128 TFLOP/s"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the FP64 oracle")
    p.add_argument("--cpu-layers", type=int, default=12, help="decode layers the oracle sample covers")
    p.add_argument("--counters", action="store_true",
                   help="run only five chain launches and five 512 MiB copies (for HBM counter runs)")
    p.add_argument("--gemm-calls", action="store_true",
                   help="run only w4_gemm at M = 128 and M = 16 on the two decode shapes, five calls each "
                        "(for kernel traces and SQ counter runs of the GEMM kernels)")
    return p.parse_args()


# Sources that define the chain kernel; a traffic figure measured on other
# sources is not reported.
CHAIN_SOURCES = ["gemm_w4_gemv_amd/csrc/chain.hip", "gemm_w4_gemv_amd/csrc/chain.hpp",
                 "gemm_w4_gemv_amd/csrc/gemv_common.hpp", "gemm_w4_gemv_amd/csrc/w4_device.hpp"]
TRAFFIC_FILE = ROOT / "profiles" / "chain_kernel_traffic.json"


def chain_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in CHAIN_SOURCES:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per chain launch from the committed counter runs, if they match the current sources."""
    try:
        rec = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    if rec.get("chain_source_sha256") != chain_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


# ------------------------------------------------------------------ helpers
def time_graph(torch, replay, stream, reps: int, warmup: int = 2, trials: int = 5):
    """Milliseconds per replay: the median over ``trials`` of HIP events on ``stream`` around ``reps`` replays."""
    for _ in range(warmup):
        replay()
    stream.synchronize()
    per = []
    for _ in range(trials):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            replay()
        b.record(stream)
        b.synchronize()
        per.append(a.elapsed_time(b) / reps)
    return sorted(per)[len(per) // 2]


# The source pages' own figures, on other GPUs and workloads: context for the
# numbers above, not a target and not a same-node comparison.
PAGES_FIGURES = {
    "note": "the pages' figures on other hardware; context only",
    "gemma4_decode_step_328_int4_gemvs_ms": {"value": 73, "hardware": "14-SM 10 GB MIG slice",
                                             "source": "Lab 5: Gemma4 端到端推理优化, 性能分析"},
    "gemma4_logits_gemv_ms": {"value": 8.67, "hardware": "14-SM 10 GB MIG slice",
                              "source": "Lab 5: Gemma4 端到端推理优化, 性能分析"},
    "int4_gemv_eager_us": {"value": 348, "hardware": "14-SM 10 GB MIG slice",
                           "source": "Lab 5: Gemma4 端到端推理优化, INT4 融合 GEMV"},
    "fp4_moe_gemm_ms_fallback_cublas_fused": {"value": [52, 14, 6.4], "tok_per_s": [0.79, 1.87],
                                              "hardware": "SM121 (DGX Spark)",
                                              "source": "DeepSeek V4 Triton FP4 优化实战, 关键数据"},
}


def floors(w4, torch, stream):
    """Measured ceilings for context: the HBM read rate of a plain streaming read kernel over
    2 GiB (well past the 256 MB MALL), and a graph of 336 empty launches (the launch floor of
    the 336-launch decode step)."""
    src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(0x5A)
    sink = torch.zeros(w4.READ_PROBE_SINK, dtype=torch.int32, device="cuda")
    ms = time_graph(torch, lambda: w4.w4_read_probe(src, sink, stream=stream), stream, reps=5)
    read_gbps = src.numel() / (ms * 1e-3) / 1e9
    g = capture(w4, torch, stream, lambda: [w4.w4_read_probe(src, sink, 0, stream=stream) for _ in range(336)])
    empty_ms = time_graph(torch, lambda: g.replay(stream), stream, reps=20)
    g.destroy()
    log(f"read probe: {read_gbps:.0f} GB/s over 2 GiB; 336 empty launches: {empty_ms * 1e3:.1f} us per replay")
    return src, sink, {"hbm_read_probe": {"GBps": round(read_gbps, 1), "frac_hbm": round(read_gbps / 8000.0, 4),
                                          "bytes": src.numel(),
                                          "note": "plain streaming read kernel of this library (w4_read_probe: "
                                                  "512 workgroups, each streaming one contiguous 4 MiB region); "
                                                  "median of 5 trials of 5 launches"},
                       "empty_336_launch_graph_us": round(empty_ms * 1e3, 1)}


def capture(w4, torch, stream, body):
    torch.cuda.synchronize()
    w4.w4_graph_begin(stream)
    try:
        body()
    finally:
        g = w4.w4_graph_end(stream)
    return g


def per_launch_durations(w4, torch, step):
    """Eager pass of the step with an event pair around every launch (same stream)."""
    stream = step.stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in step.linears]
    torch.cuda.synchronize()
    for (a, b), lin in zip(evs, step.linears):
        a.record(stream)
        w4.w4_gemv(lin["x"], lin["qw"], lin["s"], lin["z"], lin["y"], stream=stream)
        b.record(stream)
    stream.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]  # microseconds


def extra_workloads(w4, host, si, torch, rf):
    """Other workloads, each as a graph over rotated weight copies (>= 512 MB walked)."""
    stream = torch.cuda.Stream()
    flush_src, flush_sink, out = floors(w4, torch, stream)
    MB = 1 << 20

    # single 3840 x 3840 GEMV
    K, N = 3840, 3840
    copies = []
    per = rf.int4_weight_bytes(K, N)
    n_copies = -(-(512 * MB) // per) + 1
    for c in range(n_copies):
        lin = si.int4_linear(100, (c,), K, N)
        t = host.int4_tensors(lin)
        copies.append(t)
    x = host.bf16_tensor(si.bf16_normal(100, (9,), (K,)))
    y = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    g = capture(w4, torch, stream, lambda: [w4.w4_gemv(x, t["qw"], t["s"], t["z"], y, stream=stream) for t in copies])
    ms = time_graph(torch, lambda: g.replay(stream), stream, reps=20)
    us = ms * 1e3 / n_copies
    gbps = rf.int4_linear_bytes(K, N) / (us * 1e-6) / 1e9
    # one cold launch: the GEMV's weights evicted from every cache by a 2 GiB read first
    w4.w4_read_probe(flush_src, flush_sink, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    w4.w4_gemv(x, copies[0]["qw"], copies[0]["s"], copies[0]["z"], y, stream=stream)
    b.record(stream)
    b.synchronize()
    cold_us = a.elapsed_time(b) * 1e3
    g.destroy()
    # the same copies as one stage of the persistent chain kernel (one launch, one shared x,
    # one output each): the shape's streaming rate with the per-launch cost amortised
    from gemm_w4_gemv_amd.decode import DecodeStep
    batch = [dict(t, x=x, y=torch.empty(N, dtype=torch.bfloat16, device="cuda"), stage=0) for t in copies]
    step = DecodeStep(batch, stream=stream, mode="chain")
    step.capture()
    ms_b = time_graph(torch, step.replay, stream, reps=20)
    us_b = ms_b * 1e3 / n_copies
    gbps_b = rf.int4_linear_bytes(K, N) / (us_b * 1e-6) / 1e9
    err_b = step.chain.error()
    step.destroy()
    out["single_gemv_3840x3840"] = {"us_per_call": round(us, 3), "GBps": round(gbps, 1),
                                    "frac_hbm": round(gbps / rf.HBM_PEAK_GBPS, 4), "copies": n_copies,
                                    "cold_launch_us": round(cold_us, 2),
                                    "batched_in_one_chain_launch": {
                                        "us_per_gemv": round(us_b, 3), "GBps": round(gbps_b, 1),
                                        "frac_hbm": round(gbps_b / rf.HBM_PEAK_GBPS, 4), "error_word": err_b}}
    del copies, batch
    log(f"single GEMV 3840x3840: {us:.2f} us, {gbps:.0f} GB/s; one cold launch {cold_us:.1f} us; "
        f"{n_copies} in one chain launch: {us_b:.2f} us each, {gbps_b:.0f} GB/s")

    # logits GEMV 3840 -> 262144
    K, N = si.LOGITS_SHAPE
    copies = [host.int4_tensors(si.int4_linear(101, (c,), K, N)) for c in range(2)]
    x = host.bf16_tensor(si.bf16_normal(101, (9,), (K,)))
    y = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    g = capture(w4, torch, stream, lambda: [w4.w4_gemv(x, t["qw"], t["s"], t["z"], y, stream=stream) for t in copies])
    ms = time_graph(torch, lambda: g.replay(stream), stream, reps=20)
    us = ms * 1e3 / 2
    gbps = rf.int4_linear_bytes(K, N) / (us * 1e-6) / 1e9
    out["logits_gemv_3840x262144"] = {"us_per_call": round(us, 2), "GBps": round(gbps, 1),
                                      "frac_hbm": round(gbps / rf.HBM_PEAK_GBPS, 4)}
    g.destroy()
    del copies
    log(f"logits GEMV: {us:.1f} us, {gbps:.0f} GB/s")

    # prefill M = 128
    M = si.PREFILL_M
    for si_idx, (K, N) in enumerate(si.PREFILL_SHAPES):
        per = rf.int4_weight_bytes(K, N)
        n_copies = -(-(512 * MB) // per) + 1
        copies = [host.int4_tensors(si.int4_linear(102 + si_idx, (c,), K, N)) for c in range(n_copies)]
        x = host.bf16_tensor(si.bf16_normal(102 + si_idx, (9,), (M, K)))
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        nbytes = w4.w4_gemm_workspace_bytes(M, K, N)
        ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda") if nbytes else None
        g = capture(w4, torch, stream,
                    lambda: [w4.w4_gemm(x, t["qw"], t["s"], t["z"], y, workspace=ws, stream=stream) for t in copies])
        ms = time_graph(torch, lambda: g.replay(stream), stream, reps=10)
        us = ms * 1e3 / n_copies
        tf = rf.flops(M, K, N) / (us * 1e-6) / 1e12
        out[f"prefill_m128_k{K}_n{N}"] = {"us_per_call": round(us, 2), "TFLOPs": round(tf, 1),
                                          "frac_mfma_bf16": round(tf / rf.MFMA_BF16_PEAK_TFLOPS, 4),
                                          "split_k_workspace_bytes": nbytes}
        g.destroy()
        del copies
        log(f"prefill M=128 K={K} N={N}: {us:.1f} us, {tf:.0f} TFLOP/s")

    # small-M decode (a few tokens at once) through w4_gemm (M = 1: the GEMV kernel,
    # M = 2: the two-row GEMV, M = 4 and 16: the matrix-core block), on the gate/up
    # and down shapes: weights are read once per call, so the rate is in GB/s
    small = {}
    for si_idx, (K, N) in enumerate(si.PREFILL_SHAPES):
        per = rf.int4_weight_bytes(K, N)
        n_copies = -(-(512 * MB) // per) + 1
        copies = [host.int4_tensors(si.int4_linear(102 + si_idx, (c,), K, N)) for c in range(n_copies)]
        for M in (1, 2, 4, 16):
            x = host.bf16_tensor(si.bf16_normal(102 + si_idx, (10, M), (M, K)))
            y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            g = capture(w4, torch, stream,
                        lambda: [w4.w4_gemm(x, t["qw"], t["s"], t["z"], y, stream=stream) for t in copies])
            ms = time_graph(torch, lambda: g.replay(stream), stream, reps=10)
            us = ms * 1e3 / n_copies
            gbps = rf.int4_linear_bytes(K, N, M) / (us * 1e-6) / 1e9
            small[f"m{M}_k{K}_n{N}"] = {"us_per_call": round(us, 2), "GBps": round(gbps, 1),
                                        "frac_hbm": round(gbps / rf.HBM_PEAK_GBPS, 4)}
            g.destroy()
            log(f"small-M GEMM M={M} K={K} N={N}: {us:.1f} us, {gbps:.0f} GB/s")
        del copies
    out["small_m_gemm"] = small

    # FP4 MoE: FC1 (shared x) then FC2 (one x per slot), a fresh id set per token
    pools = [host.fp4_tensors(p) for p in si.moe_pools()]
    tokens = 64
    ids = torch.from_numpy(__import__("numpy").stack([si.moe_inputs(t)[0] for t in range(tokens)])).to("cuda")
    _, x1b, x2b = si.moe_inputs(0)
    x1, x2 = host.bf16_tensor(x1b), host.bf16_tensor(x2b)
    (K1, N1), (K2, N2) = si.MOE_FC
    y1 = torch.empty(si.MOE_SLOTS, N1, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty(si.MOE_SLOTS, N2, dtype=torch.bfloat16, device="cuda")

    def moe_tokens():  # one launch per token: FC1 and FC2 together (w4_moe_gemv2)
        for t in range(tokens):
            w4.w4_moe_gemv2((x1, pools[0]["qw"], pools[0]["s"], y1), (x2, pools[1]["qw"], pools[1]["s"], y2),
                            ids[t], stream=stream)

    def moe_tokens_two():  # two launches per token
        for t in range(tokens):
            w4.w4_moe_gemv(x1, pools[0]["qw"], pools[0]["s"], ids[t], y1, stream=stream)
            w4.w4_moe_gemv(x2, pools[1]["qw"], pools[1]["s"], ids[t], y2, stream=stream)

    nb = rf.moe_bytes(si.MOE_SLOTS, K1, N1, True) + rf.moe_bytes(si.MOE_SLOTS, K2, N2, False)
    g = capture(w4, torch, stream, moe_tokens)
    ms = time_graph(torch, lambda: g.replay(stream), stream, reps=10)
    g.destroy()
    g = capture(w4, torch, stream, moe_tokens_two)
    ms2 = time_graph(torch, lambda: g.replay(stream), stream, reps=10)
    g.destroy()
    us, us2 = ms * 1e3 / tokens, ms2 * 1e3 / tokens
    gbps = nb / (us * 1e-6) / 1e9
    out["moe_fp4_6x2fc"] = {"us_per_token": round(us, 2), "GBps": round(gbps, 1),
                            "frac_hbm": round(gbps / rf.HBM_PEAK_GBPS, 4), "bytes_per_token": nb,
                            "launches_per_token": 1,
                            "two_launches_per_token": {"us_per_token": round(us2, 2),
                                                       "GBps": round(nb / (us2 * 1e-6) / 1e9, 1)}}
    log(f"FP4 MoE 6 experts x 2 FC: {us:.1f} us/token in one launch ({us2:.1f} in two), {gbps:.0f} GB/s")

    # grouped FP4 expert GEMM: 6 experts x 16 tokens each, FC1 and FC2 (FC2 reads its own
    # activations) in one w4_moe_gemm2 launch, and as two w4_moe_gemm launches; a fresh
    # id set per call (the same 64 id sets)
    rows = 16
    R = si.MOE_SLOTS * rows
    row_start = torch.arange(0, R + 1, rows, dtype=torch.int32, device="cuda")
    xg1 = host.bf16_tensor(si.bf16_normal(si.SEED, (60, 1), (R, K1)))
    xg2 = host.bf16_tensor(si.bf16_normal(si.SEED, (60, 2), (R, K2)))
    yg1 = torch.empty(R, N1, dtype=torch.bfloat16, device="cuda")
    yg2 = torch.empty(R, N2, dtype=torch.bfloat16, device="cuda")

    def moe_groups():  # one launch per id set: both FCs (w4_moe_gemm2)
        for t in range(tokens):
            w4.w4_moe_gemm2((xg1, pools[0]["qw"], pools[0]["s"], yg1), (xg2, pools[1]["qw"], pools[1]["s"], yg2),
                            row_start, ids[t], rows, stream=stream)

    def moe_groups_two():  # two launches per id set
        for t in range(tokens):
            w4.w4_moe_gemm(xg1, row_start, ids[t], pools[0]["qw"], pools[0]["s"], yg1, rows, stream=stream)
            w4.w4_moe_gemm(xg2, row_start, ids[t], pools[1]["qw"], pools[1]["s"], yg2, rows, stream=stream)

    g = capture(w4, torch, stream, moe_groups)
    us = time_graph(torch, lambda: g.replay(stream), stream, reps=10) * 1e3 / tokens
    g.destroy()
    g = capture(w4, torch, stream, moe_groups_two)
    us2 = time_graph(torch, lambda: g.replay(stream), stream, reps=10) * 1e3 / tokens
    g.destroy()
    nb = (si.MOE_SLOTS * (rf.fp4_expert_bytes(K1, N1) + rf.fp4_expert_bytes(K2, N2))
          + 2 * R * (K1 + N1 + K2 + N2))
    fl = 2.0 * R * (K1 * N1 + K2 * N2)
    out["moe_fp4_grouped_gemm_6x16rows_2fc"] = {
        "us_per_call_pair": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
        "frac_hbm": round(nb / (us * 1e-6) / 1e9 / rf.HBM_PEAK_GBPS, 4),
        "TFLOPs": round(fl / (us * 1e-6) / 1e12, 2), "bytes": nb,
        "two_launches": {"us_per_call_pair": round(us2, 2), "GBps": round(nb / (us2 * 1e-6) / 1e9, 1)}}
    log(f"FP4 grouped GEMM 6 experts x 16 rows x 2 FC: {us:.1f} us in one launch ({us2:.1f} in two), "
        f"{nb / (us * 1e-6) / 1e9:.0f} GB/s")
    return out


def cpu_baseline(si, rf, layers: int):
    """The FP64 oracle (as it stands) on the first ``layers`` decode layers: GB/s of algorithmic bytes."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the process affinity
        blas_threads = len(os.sched_getaffinity(0))
    inputs = [si.decode_linear(layer, idx) for layer in range(layers) for idx in range(len(si.DECODE_LAYER))]
    nbytes = sum(rf.int4_linear_bytes(lin["qw"].shape[1] * 8, lin["qw"].shape[0]) for lin, _ in inputs)
    t0 = time.perf_counter()
    for lin, x in inputs:
        y = oracle.gemv_int4(x, lin["qw"], lin["s"], lin["z"])
        assert np.all(np.isfinite(y))
    dt = time.perf_counter() - t0
    out = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
           "sample": f"decode layers 0..{layers - 1}: {len(inputs)} linears, {nbytes} algorithmic bytes, "
                     f"{dt:.1f} s (FP64 numpy unpack + dequant + matmul)",
           "seconds": round(dt, 2),
           "host_cores": len(os.sched_getaffinity(0)),
           "threads_note": "cores = the BLAS threads available to the oracle's matrix-vector products; "
                           "its unpack and dequantisation are single-threaded numpy, so the run is mostly "
                           "one core (compare single_thread)"}
    # the same oracle on one thread, on layer 0 only
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return out
    first = inputs[:len(si.DECODE_LAYER)]
    nb1 = sum(rf.int4_linear_bytes(lin["qw"].shape[1] * 8, lin["qw"].shape[0]) for lin, _ in first)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for lin, x in first:
            oracle.gemv_int4(x, lin["qw"], lin["s"], lin["z"])
        dt1 = time.perf_counter() - t0
    out["single_thread"] = {"value": round(nb1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "sample": f"decode layer 0: {len(first)} linears, {nb1} algorithmic bytes",
                            "seconds": round(dt1, 2)}
    return out


# --------------------------------------------------------------------- main
def counter_run(torch, host, si) -> int:
    """Five chain launches of the decode step, then five 512 MiB torch copies."""
    from gemm_w4_gemv_amd.decode import DecodeStep, decode_linears, linked_copy
    lins = linked_copy(decode_linears())
    step = DecodeStep(lins, mode="chain")
    torch.cuda.synchronize()
    for _ in range(5):
        step.run_eager()
    step.stream.synchronize()
    err = step.chain.error()
    step.destroy()
    del lins
    src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"counters run: 5 chain launches (error word {err:#x}), 5 copies of {src.numel()} bytes")
    return 1 if err else 0


def gemm_calls(w4, torch, host, si) -> int:
    """w4_gemm at M = 128 (the tiled kernel; K15360 -> N3840 splits K) and M = 16
    (the small-M kernel) on the two decode shapes, five calls each."""
    for M in (si.PREFILL_M, 16):
        for idx, (K, N) in enumerate(si.PREFILL_SHAPES):
            t = host.int4_tensors(si.int4_linear(102 + idx, (0,), K, N))
            x = host.bf16_tensor(si.bf16_normal(102 + idx, (9, M), (M, K)))
            y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            nbytes = w4.w4_gemm_workspace_bytes(M, K, N)
            ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda") if nbytes else None
            for _ in range(5):
                w4.w4_gemm(x, t["qw"], t["s"], t["z"], y, workspace=ws)
            torch.cuda.synchronize()
            log(f"gemm calls: M={M} K={K} N={N} x5")
    # the grouped FP4 expert GEMM: 6 experts x 16 rows, FC1 and FC2 in one launch
    pools = [host.fp4_tensors(p) for p in si.moe_pools()]
    (K1, N1), (K2, N2) = si.MOE_FC
    rows = 16
    R = si.MOE_SLOTS * rows
    row_start = torch.arange(0, R + 1, rows, dtype=torch.int32, device="cuda")
    ids = torch.from_numpy(si.moe_inputs(0)[0]).to("cuda")
    xg1 = host.bf16_tensor(si.bf16_normal(si.SEED, (60, 1), (R, K1)))
    xg2 = host.bf16_tensor(si.bf16_normal(si.SEED, (60, 2), (R, K2)))
    yg1 = torch.empty(R, N1, dtype=torch.bfloat16, device="cuda")
    yg2 = torch.empty(R, N2, dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        w4.w4_moe_gemm2((xg1, pools[0]["qw"], pools[0]["s"], yg1), (xg2, pools[1]["qw"], pools[1]["s"], yg2),
                        row_start, ids, rows)
    torch.cuda.synchronize()
    log(f"moe_gemm2 calls: {si.MOE_SLOTS} groups x {rows} rows, K{K1}->N{N1} and K{K2}->N{N2} x5")
    return 0


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode GEMV path is single-GPU here "
              "(row sharding across GPUs is a design note, not built); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if not (ROOT / "gemm_w4_gemv_amd" / "libw4.so").exists():
        import __graft_entry__
        __graft_entry__.build()
    import gemm_w4_gemv_amd as w4
    import seeded_inputs as si
    from gemm_w4_gemv_amd import host
    from gemm_w4_gemv_amd import roofline as rf

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    from gemm_w4_gemv_amd.decode import DecodeStep, decode_linears, linked_copy

    if args.counters:
        return counter_run(torch, host, si)
    if args.gemm_calls:
        return gemm_calls(w4, torch, host, si)

    log("generating and uploading the decode step (336 INT4 linears)")
    own = decode_linears()
    lins = linked_copy(own)
    n_stages = len({l["stage"] for l in lins})
    step_bytes = sum(rf.int4_linear_bytes(l["K"], l["N"]) for l in lins)
    step_flops = sum(rf.flops(1, l["K"], l["N"]) for l in lins)
    step = DecodeStep(lins, mode="chain")
    step.capture()
    log(f"chain planned ({step.chain.handle:#x}); graph captured; warm-up")

    for _ in range(args.warmup):
        step.replay()
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(step.stream)
    for _ in range(args.steps):
        step.replay()
    ev1.record(step.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"decode step (chain graph): {ms_per_step * 1e3:.1f} us/step (events {gpu_ms_per_step * 1e3:.1f} us), "
        f"{value:.0f} GB/s")
    chain_err = step.chain.error()
    if chain_err:
        log(f"chain error word {chain_err:#x}")
        return 1

    # roofline of the dominant kernel (the chain kernel): an event pair around each launch
    reps = 20
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(step.stream)
        step.run_eager()
        b.record(step.stream)
    step.stream.synchronize()
    avg_us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / reps
    achieved = step_bytes / (avg_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": rf.HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / rf.HBM_PEAK_GBPS, 4), "traffic": measured_traffic(),
                "kernel": f"chain_kernel (336 INT4 GEMVs in {n_stages} stages, each waiting for the output it reads; "
                          "one launch per decode step)",
                "bytes_per_launch": step_bytes, "avg_launch_us": round(avg_us, 2), "launches_timed": reps}
    log(f"chain kernel: {avg_us:.1f} us/launch, {achieved:.0f} GB/s")
    step.destroy()

    # the same linears each reading its own input: no GEMV waits for another, so the grouped
    # schedule (q, k, v in one stage, gate and up in one) suits it best
    extra = {}
    from gemm_w4_gemv_amd.decode import decoder_stages
    grouped = [dict(t, stage=decoder_stages([t["name"]], [t["layer"]], grouped=True)[0]) for t in own]
    step3 = DecodeStep(grouped, mode="chain")
    step3.capture()
    ms3 = time_graph(torch, step3.replay, step3.stream, reps=args.steps, warmup=args.warmup)
    err3 = step3.chain.error()
    extra["decode_step_independent_inputs"] = {
        "us_per_step": round(ms3 * 1e3, 1), "GBps": round(step_bytes / (ms3 * 1e-3) / 1e9, 1),
        "note": "same 336 linears, each reading its own N(0,1) input, so no GEMV waits for another "
                "(weight streaming with no dependencies, not a decode step); 4 stages per layer "
                "(q,k,v | o | gate,up | down)", "error_word": err3}
    log(f"336 GEMVs with independent inputs (chain): {ms3 * 1e3:.1f} us")
    step3.destroy()

    # the same step as 336 separate launches
    step2 = DecodeStep(lins, mode="launches")
    step2.capture()
    ms2 = time_graph(torch, step2.replay, step2.stream, reps=args.steps, warmup=args.warmup)
    durs = per_launch_durations(w4, torch, step2)
    by_shape = {}
    for lin, d in zip(lins, durs):
        key = (lin["K"], lin["N"])
        e = by_shape.setdefault(key, {"names": set(), "us": [], "bytes": rf.int4_linear_bytes(*key)})
        e["names"].add(lin["name"])
        e["us"].append(d)
    extra["decode_step_336_launch_graph"] = {
        "us_per_step": round(ms2 * 1e3, 1), "GBps": round(step_bytes / (ms2 * 1e-3) / 1e9, 1),
        "per_shape_eager_event_us": {f"{'/'.join(sorted(v['names']))} K{k[0]}->N{k[1]}":
                                     {"launches": len(v["us"]), "avg_us": round(sum(v["us"]) / len(v["us"]), 3),
                                      "GBps": round(v["bytes"] / (sum(v["us"]) / len(v["us"]) * 1e-6) / 1e9, 1)}
                                     for k, v in by_shape.items()}}
    log(f"decode step (336-launch graph): {ms2 * 1e3:.1f} us/step")
    step2.destroy()

    if not args.no_extra:
        extra.update(extra_workloads(w4, host, si, torch, rf))
    n_lins = len(lins)
    del lins
    extra["pages_figures_context"] = PAGES_FIGURES

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the FP64 oracle on {args.cpu_layers} decode layer(s)")
        cpu = cpu_baseline(si, rf, args.cpu_layers)
        log(f"oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['seconds']} s)")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode step: one hipGraph replay of 48 layers x 7 INT4 GEMVs "
                               "(q,k,v,o,gate,up,down; hidden 3840; group 128; M=1), each reading the output "
                               "it reads in a decoder (o<-q, gate/up<-o, down<-gate, next q/k/v<-down), "
                               "run by the persistent chain kernel",
                   "linears": n_lins, "stages": n_stages, "bytes_per_step": step_bytes, "flops_per_step": step_flops,
                   "us_per_step": round(ms_per_step * 1e3, 1), "gpu_us_per_step": round(gpu_ms_per_step * 1e3, 1),
                   "frac_hbm": round(value / rf.HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

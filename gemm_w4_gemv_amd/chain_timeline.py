"""Per-stage timeline of the decode step run by the persistent chain kernel.

A separate build of the library with ``-DW4_CHAIN_TIMELINE`` stamps, per
workgroup and stage of the last launch, when the stage's staging starts,
when its x is staged, when its first tile's math starts and when its last
tile is done (s_memrealtime, 100 MHz).  This script builds that library and,
on a GPU, runs the decode step that ``bench.py`` times (48 layers, 336 INT4 GEMVs
linked as a decoder reads them, six stages per layer) with it and prints a
per-stage summary as Markdown.

    python gemm_w4_gemv_amd/chain_timeline.py build   # CPU: writes gemm_w4_gemv_amd/libw4_timeline.so
    python gemm_w4_gemv_amd/chain_timeline.py run     # one MI355X

The stamps cost the kernel a few per cent; the product library is built
without them.
"""
from __future__ import annotations

import ctypes
import importlib.util
import os
import pathlib
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
TIMELINE_LIB = PKG / "libw4_timeline.so"
STAGES, WORKERS, EVENTS = 512, 256, 4  # the kernel's kTimelineStages, kTimelineWorkers, stamps per stage
TICKS_PER_US = 100.0
ROLES = ["q", "k, v", "o", "gate", "up", "down"]   # the six stages of a layer, in order
PRODUCER = {0: -1, 1: -1, 2: 0, 3: 2, 4: 2, 5: 3}   # stage of the layer whose output each one reads (-1: previous layer's down)


def build() -> pathlib.Path:
    spec = importlib.util.spec_from_file_location("_w4_build", PKG / "build.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build(defines=["W4_CHAIN_TIMELINE"], lib=TIMELINE_LIB, build_dir=ROOT / "_build" / "timeline")


def summarize(ts, num_layers: int, per_layer: int) -> str:
    import numpy as np
    t0 = ts[:, 0, 0].min()
    T = (ts - t0) / TICKS_PER_US
    started = ts[..., 2] != 0xFFFFFFFF
    done = ts[..., 3] != 0
    end_all = np.where(done, T[..., 3], -np.inf).max(axis=0)  # last workgroup done with each stage
    layers = range(2, num_layers - 2)
    rows = []
    for k, role in enumerate(ROLES):
        detect, first, span, staged_spread = [], [], [], []
        for layer in layers:
            t = per_layer * layer + k
            p = per_layer * layer + PRODUCER[k] if PRODUCER[k] >= 0 else per_layer * layer - 1
            staged = T[:, t, 1]
            detect.append(np.median(staged) - end_all[p])
            staged_spread.append(np.percentile(staged, 90) - np.percentile(staged, 10))
            m = started[:, t] & done[:, t]
            first.append(np.median(T[m, t, 2] - staged[m]))
            span.append(np.median(T[m, t, 3] - T[m, t, 2]))
        rows.append(f"| {role} | {'previous down' if PRODUCER[k] < 0 else ROLES[PRODUCER[k]]} | "
                    f"{np.mean(detect):.2f} | {np.mean(staged_spread):.2f} | {np.mean(first):.2f} | "
                    f"{np.mean(span):.2f} |")
    layer_us = [end_all[per_layer * (l + 1) - 1] - end_all[per_layer * l - 1] for l in layers]
    head = ("| stage | reads the output of | its x staged after the producer's last workgroup is done (median, us) "
            "| spread of staging over workgroups (p10-p90, us) | first tile's math starts after staging (median, us) "
            "| workgroup's math span for the stage (median, us) |\n|---|---|---:|---:|---:|---:|")
    return (head + "\n" + "\n".join(rows) + "\n\n"
            f"Layers {layers.start}-{layers.stop - 1} (of {num_layers}) averaged; a layer takes {np.mean(layer_us):.2f} us "
            f"(last stage done to last stage done); the launch spans {np.nanmax(np.where(done, T[..., 3], np.nan)):.1f} us.")


def run() -> int:
    os.environ["W4_LIBRARY"] = str(TIMELINE_LIB)
    sys.path.insert(0, str(ROOT))
    import numpy as np
    import torch
    import gemm_w4_gemv_amd as w4
    from gemm_w4_gemv_amd.decode import DecodeStep, LAYER_STAGES, decode_linears, linked_copy

    assert w4.LIB_PATH == TIMELINE_LIB, w4.LIB_PATH
    read = w4.lib.w4_chain_timeline_read
    read.restype = ctypes.c_int
    read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lins = linked_copy(decode_linears("cuda"))
    step = DecodeStep(lins, mode="chain")
    step.capture()
    for _ in range(5):
        step.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(step.stream)
    for _ in range(20):
        step.replay()
    b.record(step.stream)
    b.synchronize()
    us = a.elapsed_time(b) * 1e3 / 20
    err = step.chain.error()
    buf = np.zeros(WORKERS * STAGES * EVENTS, dtype=np.uint32)
    rc = read(buf.ctypes.data, buf.nbytes)
    if rc != 0 or err != 0:
        print(f"timeline read status {rc}, chain error word {err:#x}", file=sys.stderr)
        return 1
    num_stages = len({t["stage"] for t in lins})
    ts = buf.astype(np.int64).reshape(WORKERS, STAGES, EVENTS)[:, :num_stages]
    print(f"decode step with the timeline build: {us:.1f} us/step (20 graph replays); last launch below\n")
    print(summarize(ts, num_stages // LAYER_STAGES, LAYER_STAGES))
    step.destroy()
    return 0


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "build":
        print(build())
    elif cmd == "run":
        sys.exit(run())
    else:
        print(__doc__)
        sys.exit(2)

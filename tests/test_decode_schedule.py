"""Host-side checks of the decode step's stage schedules and input wiring (no GPU)."""
from __future__ import annotations

import pytest

import seeded_inputs as si

w4 = pytest.importorskip("gemm_w4_gemv_amd")
from gemm_w4_gemv_amd.decode import DECODER_INPUT, decoder_stages, link_decoder_inputs  # noqa: E402


def _linears():
    out = []
    for layer, idx, name, K, N in si.decode_step_specs():
        out.append({"name": name, "layer": layer, "K": K, "N": N, "x": ("x", layer, name), "y": ("y", layer, name)})
    return out


@pytest.mark.parametrize("grouped", [False, True])
def test_schedule_orders_every_reader_after_its_producer(grouped):
    lins = _linears()
    stages = decoder_stages([l["name"] for l in lins], [l["layer"] for l in lins], grouped)
    assert stages == sorted(stages), "descriptors must be in non-decreasing stage order"
    per = 4 if grouped else 6
    assert len(set(stages)) == per * max(l["layer"] for l in lins) + per
    link_decoder_inputs(lins)
    producer = {l["y"]: s for l, s in zip(lins, stages)}
    for l, s in zip(lins, stages):
        if l["x"] in producer:  # reads an earlier linear's output
            assert producer[l["x"]] < s, f"layer {l['layer']} {l['name']} reads an output of its own or a later stage"
            src = [m for m in lins if m["y"] == l["x"]][0]
            assert src["N"] == l["K"]
        else:
            assert l["layer"] == 0 and DECODER_INPUT[l["name"]] == "h"


def test_six_stage_schedule_separates_unread_linears():
    """k, v and up, read by no linear of the path, get stages of their own next to the linear
    that shares their input; q, o, gate and down are each alone in a stage."""
    lins = _linears()[:7]
    stages = dict(zip([l["name"] for l in lins], decoder_stages([l["name"] for l in lins], [0] * 7)))
    assert stages["k"] == stages["v"] == stages["q"] + 1
    assert stages["o"] == stages["k"] + 1
    assert stages["up"] == stages["gate"] + 1 and stages["down"] == stages["up"] + 1
    assert len({stages[n] for n in ("q", "o", "gate", "down", "up", "k")}) == 6

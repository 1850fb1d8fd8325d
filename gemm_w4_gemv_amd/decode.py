"""The decode step's GEMV chain captured once into a HIP graph.

Two ways to run the step are offered:

* ``launches``: one ``w4_gemv`` launch per linear (336 graph nodes);
* ``chain``: one ``w4_chain_run`` launch (a single graph node) of the
  persistent chain kernel, with the decoder's linears as stages: per layer
  {q, k, v} -> {o} -> {gate, up} -> {down}.  A linear whose input is another
  linear's output (see ``link_decoder_inputs``) waits for exactly that
  output.

"Lab 5: Gemma4 端到端推理优化", section "CUDA Graph": after the fused GEMV the
remaining cost was launch and Python overhead, so the whole decode step is
captured once into a static graph and replayed once per token; the graph
needs static buffers.  Here the step is the chain of INT4 linears of every
layer in launch order (q, k, v, o, gate, up, down), each an ``w4_gemv``
recorded on one stream; every linear keeps its own static input and output
buffers, so one replay recomputes every output.
"""
from __future__ import annotations

import torch

from . import w4_gemv, w4_graph_begin, w4_graph_end, W4Graph, w4_chain_create, w4_chain_run, \
    w4_chain_workspace_bytes

# Stage of each decoder linear within its layer.  Along the decoder's data
# flow q -> o -> gate -> down -> (next layer's) q each of these waits for the
# one before; k, v and up are read by no linear of this path, so each pair
# gets a stage of its own right after the linear that shares its input
# (k, v after q; up after gate): their weights stream while the chain
# kernel awaits the next reader's input (o's, down's), instead of delaying it.
LAYER_STAGES = 6
LAYER_STAGE = {"q": 0, "k": 1, "v": 1, "o": 2, "gate": 3, "up": 4, "down": 5}
# The grouped schedule: linears that share an input in one stage.
LAYER_STAGES_GROUPED = 4
LAYER_STAGE_GROUPED = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}


# the output each decoder linear reads: "h" is the layer's input (the first
# layer's own input; for later layers the previous layer's down output)
DECODER_INPUT = {"q": "h", "k": "h", "v": "h", "o": "q", "gate": "o", "up": "o", "down": "gate"}


def decoder_stages(names, layers_of, grouped: bool = False):
    """Stage number of every linear, from its name and layer index."""
    per, table = (LAYER_STAGES_GROUPED, LAYER_STAGE_GROUPED) if grouped else (LAYER_STAGES, LAYER_STAGE)
    return [per * layer + table[name] for name, layer in zip(names, layers_of)]


def link_decoder_inputs(linears) -> None:
    """Make every linear read the output it reads in a decoder layer.

    ``linears`` are dicts with ``name``, ``layer``, ``x`` and ``y``, in layer
    order.  The first layer's q, k and v keep their own ``x`` (they must share
    one buffer); every other input becomes the producing linear's ``y``: o
    reads q's output, gate and up read o's, down reads gate's (the gate/up
    product and the attention between q and o are outside this path), and a
    layer's q, k and v read the previous layer's down output.
    """
    out = {}
    for lin in linears:
        layer, name = lin["layer"], lin["name"]
        src = DECODER_INPUT[name]
        if src == "h":
            if layer > 0:
                lin["x"] = out[(layer - 1, "down")]
        else:
            lin["x"] = out[(layer, src)]
        out[(layer, name)] = lin["y"]


def decode_linears(device: str = "cuda"):
    """The decode step's 336 INT4 linears as device tensors, from the seeded
    synthetic workload (48 layers x q, k, v, o, gate, up, down; hidden 3840;
    group 128), each reading its own seeded N(0,1) input and writing its own
    zeroed output.  Each dict holds ``qw``, ``s``, ``z``, ``x``, ``y``,
    ``name``, ``layer``, ``index`` (position in its layer), ``K``, ``N`` and
    ``stage`` (six stages per layer).  The seeded inputs are synthetic data,
    not part of the method: the generator module is imported here only."""
    import seeded_inputs as si
    from . import host

    lins = []
    for layer, idx, name, K, N in si.decode_step_specs():
        lin_np, x_bits = si.decode_linear(layer, idx)
        t = host.int4_tensors(lin_np, device)
        t["x"] = host.bf16_tensor(x_bits, device)
        t["y"] = torch.zeros(N, dtype=torch.bfloat16, device=device)
        t["name"], t["layer"], t["index"], t["K"], t["N"] = name, layer, idx, K, N
        t["stage"] = decoder_stages([name], [layer])[0]
        lins.append(t)
    torch.cuda.synchronize()
    return lins


def linked_copy(lins):
    """The same linears (same weights and output buffers), each reading the
    output it reads in a decoder (``link_decoder_inputs``); layer 0's q, k
    and v share q's input.  This is the decode step as it is timed."""
    out = [dict(t) for t in lins]
    for t in out[1:3]:
        t["x"] = out[0]["x"]
    link_decoder_inputs(out)
    return out


class DecodeStep:
    """A captured chain of ``w4_gemv`` calls.

    ``linears`` is a sequence of dicts with device tensors ``qw`` (int32
    [N, K/8]), ``s``, ``z`` (float16 [N, K/128]), ``x`` (bfloat16 [K]) and
    ``y`` (bfloat16 [N]).  The tensors must stay alive while the graph does.
    """

    def __init__(self, linears, stream: torch.cuda.Stream | None = None, mode: str = "launches"):
        if mode not in ("launches", "chain"):
            raise ValueError("mode must be 'launches' or 'chain'")
        self.linears = list(linears)
        self.stream = stream if stream is not None else torch.cuda.Stream()
        self.mode = mode
        self.graph: W4Graph | None = None
        self.chain = None
        if mode == "chain":
            nbytes = w4_chain_workspace_bytes(self.linears)
            self.workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device="cuda")
            off = (-self.workspace.data_ptr()) % 256
            self.chain = w4_chain_create(self.linears, self.workspace[off:off + nbytes])

    def run_eager(self) -> None:
        """Run the step directly on the step's stream (no graph)."""
        if self.mode == "chain":
            w4_chain_run(self.chain, stream=self.stream)
            return
        for lin in self.linears:
            w4_gemv(lin["x"], lin["qw"], lin["s"], lin["z"], lin["y"], stream=self.stream)

    def capture(self) -> W4Graph:
        """Record the chain into a graph (nothing runs during capture)."""
        if self.graph is not None:
            self.graph.destroy()
        torch.cuda.synchronize()
        w4_graph_begin(self.stream)
        try:
            self.run_eager()
        finally:
            # ending the capture also ends it after a failed launch
            graph = w4_graph_end(self.stream)
        self.graph = graph
        return graph

    def replay(self) -> None:
        if self.graph is None:
            self.capture()
        self.graph.replay(self.stream)

    def destroy(self) -> None:
        if self.graph is not None:
            self.graph.destroy()
            self.graph = None
        if self.chain is not None:
            self.chain.destroy()
            self.chain = None

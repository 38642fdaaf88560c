"""The layer captured in a HIP graph and replayed.

A serving loop captures the decode step once and replays it.  The library
launches only kernels on the caller's stream (no allocation, no memset, no
synchronisation), so the captured graph is the layer.  Each case captures
`moe_layer_forward` on a static input buffer, then replays it several times
with eager work between the replays (new rows copied into the input, an eager
forward of the same rows into other buffers, synchronisations), and checks
that every replay gives exactly the eager result: y, expert indices and
weights, bit for bit.
"""

import pytest
import torch

import mixture_experts_ffn_07_amd as moe
from moe_synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _variants(x: torch.Tensor) -> list:
    """Input rows for the replays: as generated, negated (sign bit flipped), columns rotated."""
    neg = torch.bitwise_xor(x, torch.tensor(-0x8000, dtype=torch.int16, device=x.device))
    return [x.clone(), neg, torch.roll(x, shifts=7, dims=1).contiguous(), x.clone()]


def _outputs(t: int, cfg):
    y = torch.empty((t, cfg.hidden), dtype=torch.int16, device=DEV)
    idx = torch.empty((t, cfg.top_k), dtype=torch.int32, device=DEV)
    wt = torch.empty((t, cfg.top_k), dtype=torch.float32, device=DEV)
    return y, idx, wt


# beside the workloads: the MXFP8 few-token GEMVs (5 tokens) and the MXFP6 kernels with E4M3 weights and h
# records on a small layer (1100 tokens); the 4096-token layer takes the MXFP6 down projection on h records
EXTRA = {"fp8_t5": CONFIGS["decode_t1_h5120_e384_fp8"].with_(tokens=5),
         "fp8_t1100_small": CONFIGS["tiny_t8_h512_e32"].with_(tokens=1100, expert_format="mxfp8")}


@pytest.mark.parametrize("name", ["tiny_t8_h512_e32", "decode_t1_h5120_e384", "decode_t1_h5120_e384_norm",
                                  "decode_t64_h5120_e384", "prefill_t4096_h5120_e384", "decode_t1_h5120_e384_fp8",
                                  "fp8_t5", "fp8_t1100_small"])
def test_graph_replay_matches_eager(name):
    inp = make_inputs(EXTRA[name] if name in EXTRA else CONFIGS[name], seed=3, device=DEV)
    cfg = moe.config_from(inp.cfg)
    w = moe.weights_from(inp)
    t = inp.cfg.tokens
    x_static = inp.x.clone()
    y_s, idx_s, wt_s = _outputs(t, inp.cfg)
    ws_graph = moe.workspace(cfg, t, device=DEV)
    ws_eager = moe.workspace(cfg, t, device=DEV)
    y_e, idx_e, wt_e = _outputs(t, inp.cfg)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        # one eager call on the capture stream first, as torch recommends before capture
        moe.moe_layer_forward(cfg, w, x_static, t, y_s, idx_s, wt_s, ws_graph, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_layer_forward(cfg, w, x_static, t, y_s, idx_s, wt_s, ws_graph)
    torch.cuda.synchronize()

    for i, x in enumerate(_variants(inp.x)):
        x_static.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        # eager forward of the same rows into other buffers (own workspace), between replays
        moe.moe_layer_forward(cfg, w, x, t, y_e, idx_e, wt_e, ws_eager)
        torch.cuda.synchronize()
        for what, g, e in (("y", y_s, y_e), ("idx", idx_s, idx_e), ("w", wt_s, wt_e)):
            assert torch.equal(g, e), f"{name}: replay {i}: {what} differs from the eager forward"
    # the replays changed the routing (the variants are different rows)
    assert t > 0

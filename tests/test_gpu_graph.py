"""A training step captured in one HIP graph: every replay equals the eager step.

The layer's forward and backward enqueue their kernels on the current stream
and allocate nothing, so a caller can capture the step.  Each replay is
checked against an eager step, with eager work between the replays.
"""
import pytest
import torch

from irregular_gather_cnn_amd.synth import WORKLOADS, make_inputs
from test_gpu_parity import dev, make_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_training_step_graph_replays_match_eager(dtype):
    wl = WORKLOADS["tiny_fp32_n1_c16_16x16"].scaled(dtype=dtype, train=True, n=2, c_in=32, c_out=24, h=12, w=13)
    inp = make_inputs(wl, with_dy=True)
    t = {k: dev(v, wl.dtype) for k, v in inp.items()}
    layer = make_layer(wl, training=True)

    def step():
        y, off = layer.forward(t["x"], t["w_off"], t["b_off"], t["w"], t["b"])
        g = layer.backward(t["x"], t["w_off"], t["w"], off, t["dy"])
        return [y, off] + [g[k] for k in ("dx", "dw_off", "db_off", "dw", "db")]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            ref = step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [r.clone() for r in ref]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "offsets", "dx", "dw_off", "db_off", "dw", "db"), out, ref):
            assert torch.equal(a, b), name
        step()  # eager work between the replays
        torch.cuda.synchronize()

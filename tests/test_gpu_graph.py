"""The attention calls inside a captured HIP graph.  Once a cache exists, its
calls only launch kernels: nothing allocates, copies or clears memory, so a
call can be recorded into a graph (torch.cuda.CUDAGraph, a hipGraph on ROCm).
The state of each stream travels in the captured kernel arguments, so a graph
replays the attention of the window as it was at capture time; the test keeps
the window fixed while it replays.  Each replay, with eager calls and
synchronizations between them, must give exactly the eager result."""

import numpy as np
import pytest

import synth
from gpu_util import Twin, say, to_device, empty_out, to_host_f64

pytestmark = pytest.mark.gpu


def draw(rng, shape):
    return synth.round_bf16(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("call", ["chunk_attn", "chunk_attn_static", "decode_attn"])
def test_graph_replays_equal_eager(call):
    import torch
    say("graph", call)
    rng = np.random.default_rng(3)
    nb, hq, hkv, d, w, n = 4, 16, 2, 128, 512, 8
    tw = Twin(1, nb, hq, hkv, d, w, n, True)
    tw.reset(0, [2**24 + 11 * b for b in range(nb)], [(29 * b) % w for b in range(nb)])
    for _ in range(w // n + 5):
        tw.append(0, 0, draw(rng, (nb, n, hkv, d)), draw(rng, (nb, n, hkv, d)))
    nq = 1 if call == "decode_attn" else n
    shape = (nb, hq, d) if nq == 1 else (nb, nq, hq, d)
    q = draw(rng, shape)
    qd = to_device(q, True)

    def run(out):
        if call == "decode_attn":
            tw.gpu.decode_attn(0, 0, nb, qd, out)
        else:
            getattr(tw.gpu, call)(0, 0, nb, nq, qd, out)

    eager = empty_out(shape, True)
    run(eager)                                   # also looks up the static array's address
    torch.cuda.synchronize()
    exp = tw.ora.decode(0, 0, q) if nq == 1 else tw.ora.chunk(0, 0, q)
    assert float(np.max(np.abs(to_host_f64(eager, True) - exp))) <= tw.tol

    captured = empty_out(shape, True)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    home = torch.cuda.current_stream().cuda_stream
    with torch.cuda.graph(graph, stream=side):
        tw.gpu.set_stream(side.cuda_stream)
        run(captured)
    tw.gpu.set_stream(home)
    torch.cuda.synchronize()
    for rep in range(4):
        captured.fill_(0)
        graph.replay()
        other = empty_out(shape, True)
        run(other)                               # eager work between the replays
        torch.cuda.synchronize()
        assert bool((captured == eager).all()), (call, rep)
        assert bool((other == eager).all()), (call, rep)
    tw.close()

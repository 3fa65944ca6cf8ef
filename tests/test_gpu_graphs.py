"""Entry points captured in a HIP graph (torch.cuda.graph) and replayed.

The library allocates nothing and clears its counters with kernels (no
memset nodes), so every entry point that does not read results back to the
host can be captured.  Each case: the call once eagerly (the reference), a
warm-up on a side stream, the capture, then three replays; before each
replay eager work overwrites the captured outputs (NaN, or -7 for integer
outputs), and after it every output must equal the eager result bit for bit
(every path here is deterministic).  The padded flow (sca_forward_rebatch)
reads the segment bounds back to the host and is not capturable.  Every
call goes through the C ABI (via the ctypes binding)."""
import pytest
import torch

from gpu_util import announce, dev, host
from test_gpu_streams import CASES

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")

CAPTURABLE = [c for c in CASES if c[0] != "sca_forward_rebatch"]


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _tensors(r):
    return list(r) if isinstance(r, tuple) else [r]


@pytest.mark.parametrize("case", CAPTURABLE, ids=[c[0] for c in CAPTURABLE])
def test_graph_replays_match_eager(case):
    _, make, call = case
    inputs = {k: dev(v) for k, v in make().items()}
    ref = [host(t) for t in _tensors(call(inputs, None))]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(inputs, None)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _tensors(call(inputs, None))
    for replay in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else -7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in outs]
        assert len(got) == len(ref)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert a.shape == b.shape and a.dtype == b.dtype, (replay, i)
            assert a.tobytes() == b.tobytes(), f"replay {replay}: output {i} differs from the eager result"
    del graph

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


def test_whole_sca_layer_in_one_graph():
    """One spatial cross-attention layer as a single graph: sampling offsets
    and logits from the query, the value projection into the head-pair
    layout, the compaction, the gather with its camera mean, and the output
    projection with the residual and layer norm.  Every intermediate and the
    layer output must equal the eager run bit for bit on every replay."""
    import numpy as np

    import workloads as W
    from test_gpu_parity import _rand_sca

    B, Ncam, Nq, nH, P, D, C = 2, 3, 400, 8, 4, 4, 256
    w = _rand_sca(77, B, Ncam, Nq, ((12, 20), (6, 10)), nH, P, D, 0.3)
    L, Nv = w["L"], w["Nv"]
    g = np.random.default_rng(78)
    bf = lambda a: W.bf16_bits_trunc(a.astype(np.float32))
    t = {k: dev(v) for k, v in {
        "feats": bf(g.normal(size=(B * Ncam * Nv, C))), "w_v": bf(g.normal(0, 1 / 16, (C, C))),
        "b_v": g.normal(size=C).astype(np.float32),
        "query": g.normal(size=(B * Nq, C)).astype(np.float32), "pos": g.normal(size=(B * Nq, C)).astype(np.float32),
        "w_off": bf(g.normal(0, 1 / 16, (nH * L * P * 2, C))), "b_off": g.normal(size=nH * L * P * 2).astype(np.float32),
        "w_att": bf(g.normal(0, 1 / 16, (nH * L * P, C))), "b_att": g.normal(size=nH * L * P).astype(np.float32),
        "w_o": bf(g.normal(0, 1 / 16, (C, C))), "b_o": g.normal(size=C).astype(np.float32),
        "gamma": g.uniform(0.5, 1.5, C).astype(np.float32), "beta": g.normal(size=C).astype(np.float32),
        "ss": w["spatial_shapes"], "starts": w["level_start_index"], "rho": w["reference_points_cam"],
        "mask": w["bev_mask"]}.items()}
    dv = t["query"].device
    o = {"off": torch.empty((B * Nq, nH * L * P * 2), dtype=torch.float32, device=dv),
         "logits": torch.empty((B * Nq, nH * L * P), dtype=torch.float32, device=dv),
         "value": torch.empty((B * Ncam, nH, Nv, 2, 32), dtype=torch.bfloat16, device=dv),
         "ws": torch.empty(msda.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device=dv),
         "slots": torch.empty((B, Nq, C), dtype=torch.float32, device=dv),
         "y": torch.empty((B * Nq, C), dtype=torch.float32, device=dv)}

    def layer():
        msda.msda_query_proj_bf16(t["query"], t["w_off"], t["b_off"], t["w_att"], t["b_att"], query_pos=t["pos"],
                                  offsets=o["off"], logits=o["logits"])
        msda.msda_value_proj_pairs_bf16(t["feats"], t["w_v"], t["b_v"], Nv, out=o["value"])
        msda.sca_compact(t["mask"], t["rho"], o["ws"])
        msda.sca_gather(o["value"].view(B, Ncam, nH, Nv, 2, 32), t["ss"], t["starts"], t["rho"],
                        o["off"].view(B, Nq, nH, L, P, 2), o["logits"].view(B, Nq, nH, L * P), o["ws"],
                        slots=o["slots"])
        msda.msda_output_proj_bf16(o["slots"].view(B * Nq, C), t["w_o"], t["b_o"], residual=t["query"],
                                   gamma=t["gamma"], beta=t["beta"], out=o["y"])

    checked = ("off", "logits", "value", "slots", "y")
    layer()
    torch.cuda.synchronize()
    ref = {k: host(o[k]) for k in checked}
    assert np.isfinite(ref["y"]).all() and np.abs(ref["slots"]).max() > 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    for replay in range(3):
        for k in checked + ("ws",):
            o[k].fill_(float("nan") if o[k].is_floating_point() else 0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in checked:
            assert ref[k].tobytes() == host(o[k]).tobytes(), f"replay {replay}: {k} differs from the eager result"
    del graph

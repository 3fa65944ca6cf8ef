"""Every entry point runs on the stream it is given.

On a fresh torch stream (torch's pool streams do not synchronise with the
null stream) a spin kernel is queued, then the copies that fill the inputs,
then the call: a launch on any other stream would read the inputs before
their copies land (they hold zeros until then).  Both ways of giving the
stream are covered: made current (`with torch.cuda.stream(s)`), and passed
as `stream=s` while the default stream stays current.  Each result is
compared, bit for bit, with the same call on the default stream: every path
here is deterministic, the value gradients included (the transpose gather
sums in a fixed order).  The oracle parity of these calls is in the other
GPU tests.  Every call goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import announce, dev, host
from test_gpu_pairs import pairs_host
from test_gpu_parity import _rand_msda, _rand_sca

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")

SPIN = 20_000_000  # clock cycles of torch's spin kernel, queued ahead of the input copies


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _msda_inputs():
    w = _rand_msda(71, 2, 300, ((16, 24), (8, 12)), 8, 4)
    g = np.random.default_rng(72).normal(size=(2, 300, 256)).astype(np.float32)
    return {"value": w["value"], "ss": w["spatial_shapes"], "starts": w["level_start_index"],
            "loc": w["sampling_locations"], "logits": w["attention_weights"], "gout": g}


def _frames_inputs():
    g = np.random.default_rng(73)
    B, F, Nq, nH, P = 2, 2, 150, 8, 4
    ss, starts, Nv = W.level_table(((12, 20), (6, 10)))
    return {"value": g.normal(size=(B, F, Nv, nH, 32)).astype(np.float32), "ss": ss, "starts": starts,
            "loc": g.uniform(-0.2, 1.2, (B, F, Nq, nH, 2, P, 2)).astype(np.float32),
            "logits": g.normal(size=(B, F, Nq, nH, 2 * P)).astype(np.float32),
            "gout": g.normal(size=(B, Nq, nH * 32)).astype(np.float32)}


def _sca_inputs():
    w = _rand_sca(74, 2, 6, 400, ((12, 20), (6, 10)), 8, 4, 4, 0.3)
    g = np.random.default_rng(75).normal(size=(2, 400, 256)).astype(np.float32)
    return {"value": w["value"], "ss": w["spatial_shapes"], "starts": w["level_start_index"],
            "rho": w["reference_points_cam"], "mask": w["bev_mask"], "off": w["sampling_offsets"],
            "logits": w["attention_logits"], "gout": g}


def _proj_inputs():
    g = np.random.default_rng(76)
    M, K, N = 1000, 256, 256
    bf = lambda a: W.bf16_bits_trunc(a.astype(np.float32))
    return {"x": bf(g.normal(size=(M, K))), "q": g.normal(size=(M, K)).astype(np.float32),
            "pos": g.normal(size=(M, K)).astype(np.float32), "w": bf(g.normal(0, 1 / 16, (N, K))),
            "w_off": bf(g.normal(0, 1 / 16, (512, K))), "w_att": bf(g.normal(0, 1 / 16, (N, K))),
            "bias": g.normal(size=N).astype(np.float32), "b_off": g.normal(size=512).astype(np.float32),
            "res": g.normal(size=(M, N)).astype(np.float32), "gamma": g.uniform(0.5, 1.5, N).astype(np.float32),
            "beta": g.normal(size=N).astype(np.float32)}


def _msda_forward(t, stream):
    return msda.msda_forward(t["value"], t["ss"], t["starts"], t["loc"], t["logits"], stream=stream)


def _msda_backward(t, stream):
    return msda.msda_backward(t["value"], t["ss"], t["starts"], t["loc"], t["logits"], t["gout"], stream=stream)


def _frames_forward(t, stream):
    return msda.msda_forward_frames(t["value"], t["ss"], t["starts"], t["loc"], t["logits"], stream=stream)


def _frames_backward(t, stream):
    return msda.msda_backward_frames(t["value"], t["ss"], t["starts"], t["loc"], t["logits"], t["gout"],
                                     stream=stream)


def _msda_planned(t, stream):
    """plan from the first sampling location of each query, then the planned
    gather (only the result is compared: the order inside a tile varies)"""
    B, Nq = t["loc"].shape[:2]
    row = t["loc"][0, 0].numel()
    plan = msda.msda_plan(t["loc"], B, Nq, Nq * row, row, stream=stream)
    return msda.msda_gather(t["value"], t["ss"], t["starts"], t["loc"], t["logits"], plan, stream=stream)


def _frames_planned(t, stream):
    B, F, Nq = t["loc"].shape[:3]
    row = t["loc"][0, 0, 0].numel()
    plan = msda.msda_plan(t["loc"], B, Nq, F * Nq * row, row, stream=stream)
    return msda.msda_gather(t["value"], t["ss"], t["starts"], t["loc"], t["logits"], plan, stream=stream)


def _sca_forward_noalloc(t, stream):
    B, Nq = t["gout"].shape[:2]
    Ncam = t["mask"].shape[0]
    dv = t["value"].device
    hit = torch.full((B, Nq), -7, dtype=torch.int32, device=dv)
    offs = torch.full((B * Ncam + 1,), -7, dtype=torch.int32, device=dv)
    pq = torch.full((B * Ncam * Nq,), -7, dtype=torch.int32, device=dv)
    slots = torch.empty((B, Nq, t["value"].shape[3] * 32), dtype=torch.float32, device=dv)
    msda.sca_forward_noalloc(t["value"], t["ss"], t["starts"], t["rho"], t["mask"], t["off"], t["logits"], slots,
                             hit_count=hit, pair_offsets=offs, pair_q=pq, stream=stream)
    return slots, hit, offs, pq


def _sca_forward(t, stream):
    B, Nq = t["gout"].shape[:2]
    Ncam = t["mask"].shape[0]
    dv = t["value"].device
    # pair_q is written up to the pair count: fill it so that its tail compares too
    hit = torch.full((B, Nq), -7, dtype=torch.int32, device=dv)
    offs = torch.full((B * Ncam + 1,), -7, dtype=torch.int32, device=dv)
    pq = torch.full((B * Ncam * Nq,), -7, dtype=torch.int32, device=dv)
    slots = msda.sca_forward(t["value"], t["ss"], t["starts"], t["rho"], t["mask"], t["off"], t["logits"],
                             hit_count=hit, pair_offsets=offs, pair_q=pq, stream=stream)
    return slots, hit, offs, pq


def _sca_two_stage(t, stream):
    B, Nq = t["gout"].shape[:2]
    Ncam = t["mask"].shape[0]
    ws = torch.empty(msda.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device=t["value"].device)
    msda.sca_compact(t["mask"], t["rho"], ws, stream=stream)
    return msda.sca_gather(t["value"], t["ss"], t["starts"], t["rho"], t["off"], t["logits"], ws, stream=stream)


def _sca_backward(t, stream):
    B, Nq = t["gout"].shape[:2]
    Ncam = t["mask"].shape[0]
    ws = torch.empty(msda.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device=t["value"].device)
    msda.sca_compact(t["mask"], t["rho"], ws, stream=stream)
    return msda.sca_backward(t["value"], t["ss"], t["starts"], t["rho"], t["off"], t["logits"], t["gout"], ws,
                             stream=stream)


def _sca_rebatch(t, stream):
    slots, _ = msda.sca_forward_rebatch(t["value"], t["ss"], t["starts"], t["rho"], t["mask"], t["off"],
                                        t["logits"], stream=stream)
    return slots


def _pairs_inputs():
    t = _sca_inputs()
    t["value_bits"] = W.bf16_bits_trunc(t["value"])
    t["pairs"] = pairs_host(t["value_bits"])
    return t


def _pack_pairs(t, stream):
    return msda.msda_pack_pairs_bf16(t["value_bits"], stream=stream)


def _sca_forward_pairs(t, stream):
    return _sca_forward({**t, "value": t["pairs"]}, stream)


def _value_proj_pairs(t, stream):
    return msda.msda_value_proj_pairs_bf16(t["x"], t["w"], t["bias"], 100, stream=stream)  # 10 images of 100 rows


def _gemm(t, stream):
    return (msda.msda_gemm_bf16(t["x"], t["w"], t["bias"], stream=stream),
            msda.msda_gemm_bf16(t["x"], t["w"], None, y_dtype=torch.float32, stream=stream))


def _query_proj(t, stream):
    return msda.msda_query_proj_bf16(t["q"], t["w_off"], t["b_off"], t["w_att"], t["bias"], query_pos=t["pos"],
                                     stream=stream)


def _output_proj(t, stream):
    return msda.msda_output_proj_bf16(t["q"], t["w"], t["bias"], residual=t["res"], gamma=t["gamma"],
                                      beta=t["beta"], stream=stream)


CASES = [
    ("msda_forward", _msda_inputs, _msda_forward),
    ("msda_backward", _msda_inputs, _msda_backward),
    ("msda_forward_frames", _frames_inputs, _frames_forward),
    ("msda_plan_then_gather", _msda_inputs, _msda_planned),
    ("msda_plan_then_gather_frames", _frames_inputs, _frames_planned),
    ("sca_forward_noalloc", _sca_inputs, _sca_forward_noalloc),
    ("msda_backward_frames", _frames_inputs, _frames_backward),
    ("sca_forward", _sca_inputs, _sca_forward),
    ("sca_compact_then_gather", _sca_inputs, _sca_two_stage),
    ("sca_backward", _sca_inputs, _sca_backward),
    ("sca_forward_rebatch", _sca_inputs, _sca_rebatch),
    ("msda_gemm_bf16", _proj_inputs, _gemm),
    ("msda_value_proj_pairs_bf16", _proj_inputs, _value_proj_pairs),
    ("msda_pack_pairs_bf16", _pairs_inputs, _pack_pairs),
    ("sca_forward_head_pairs", _pairs_inputs, _sca_forward_pairs),
    ("msda_query_proj_bf16", _proj_inputs, _query_proj),
    ("msda_output_proj_bf16", _proj_inputs, _output_proj),
]


def test_raw_handles_and_the_null_stream():
    """stream= also takes a raw hipStream_t handle, 0 being the null stream
    (torch's default stream)."""
    make, call = CASES[0][1], CASES[0][2]
    src = {k: dev(v) for k, v in make().items()}
    ref = [host(t) for t in _tensors_of(call(src, None))]
    s = torch.cuda.Stream()
    for handle in (0, s.cuda_stream):
        got = _tensors_of(call(src, handle))
        torch.cuda.synchronize()
        assert all(a.tobytes() == host(b).tobytes() for a, b in zip(ref, got)), handle


def _tensors_of(r):
    return r if isinstance(r, tuple) else (r,)


def _outputs(r):
    ts = r if isinstance(r, tuple) else (r,)
    return [host(x) for x in ts]


@pytest.mark.skipif(not hasattr(torch.cuda, "_sleep"), reason="torch has no spin kernel to queue")
@pytest.mark.parametrize("given", ["current", "argument"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_runs_on_the_given_stream(case, given):
    _, make, call = case
    src = {k: dev(v) for k, v in make().items()}
    ref = _outputs(call(src, None))
    torch.cuda.synchronize()

    filled = {k: torch.zeros_like(v) for k, v in src.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN)
        for k in src:
            filled[k].copy_(src[k])
        if given == "current":
            got = call(filled, None)
    if given == "argument":
        got = call(filled, s)
    s.synchronize()
    got = _outputs(got)
    assert len(got) == len(ref)
    for i, (a, b) in enumerate(zip(ref, got)):
        assert a.shape == b.shape and a.dtype == b.dtype, (i, a.shape, b.shape)
        assert a.tobytes() == b.tobytes(), f"output {i} differs from the default-stream result"

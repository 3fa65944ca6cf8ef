"""The padded rebatch form of SCA (an A/B baseline for the fused path),
against the oracle: the note's flow -- segment lists, locations materialised
as float32 tensors for every padded row, the MSDA operator over all B*Ncam
segments, scatter-add per camera and divide by the hit count.  Every call
goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_fp32_close, dev, host

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def rebatch_reference(w):
    """The oracle's run of the note's flow: (locations, logits, slots
    [B*Nq, C], max_len)."""
    r = oracle.sca_rebatch(*[w[k] for k in ("value", "spatial_shapes", "level_start_index", "reference_points_cam",
                                            "bev_mask", "sampling_offsets", "attention_logits")])
    return r["sampling_locations"], r["logits"], r["slots"], r["max_len"]


def run_rebatch(w):
    d = {k: dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "reference_points_cam", "bev_mask",
                                "sampling_offsets", "attention_logits")}
    slots, max_len = msda.sca_forward_rebatch(d["value"], d["spatial_shapes"], d["level_start_index"],
                                              d["reference_points_cam"], d["bev_mask"], d["sampling_offsets"],
                                              d["attention_logits"])
    return host(slots).reshape(-1, w["nH"] * w["Dh"]), max_len, d


def test_rebatch_bevformer_sca_full():
    """The BEVFormer-base SCA workload through the padded flow: max_len equals the longest segment,
    the materialised locations and logits are bit-identical to the float32
    definition, and the slots match the oracle's run of the same flow."""
    w = W.bevformer_sca()
    loc_ref, lg_ref, slots_ref, max_len_ref = rebatch_reference(w)
    got, max_len, d = run_rebatch(w)
    assert max_len == max_len_ref
    B, Ncam, Nq = w["B"], w["Ncam"], w["Nq"]
    hit = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device="cuda")
    pq = torch.empty(B * Ncam * Nq, dtype=torch.int32, device="cuda")
    ws = torch.empty(msda.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device="cuda")
    msda.sca_compact(d["bev_mask"], d["reference_points_cam"], ws, hit_count=hit, pair_offsets=offs, pair_q=pq)
    loc, lg = msda.sca_rebatch(offs, pq, d["reference_points_cam"], d["sampling_offsets"], d["attention_logits"],
                               d["spatial_shapes"], max_len)
    assert np.array_equal(host(loc), loc_ref), "rebatched locations differ from the float32 definition"
    assert np.array_equal(host(lg), lg_ref), "rebatched logits differ"
    assert_fp32_close(got, slots_ref, "rebatch flow slots")


REBATCH_EDGE = [
    # id, B, Ncam, bev, shapes, P, D
    ("two_items_masks_differ", 2, 6, 12, ((8, 12), (4, 6)), 4, 2),
    ("one_camera", 1, 1, 9, ((6, 7),), 4, 4),
    ("many_cameras_D1", 2, 9, 8, ((5, 5), (3, 3)), 3, 1),
]


@pytest.mark.parametrize("case", REBATCH_EDGE, ids=[c[0] for c in REBATCH_EDGE])
def test_rebatch_edge_cases(case):
    _, B, Ncam, bev, shapes, P, D = case
    w = W.bevformer_sca(cfg=40 + B + Ncam, B=B, Ncam=Ncam, bev=bev, shapes=shapes, P=P, D=D)
    _, _, slots_ref, max_len_ref = rebatch_reference(w)
    got, max_len, _ = run_rebatch(w)
    assert max_len == max_len_ref
    assert_fp32_close(got, slots_ref, "rebatch flow slots")


def test_rebatch_no_camera_sees_anything():
    """Empty segments everywhere: max_len = 0, nothing is gathered and the
    slots are zero."""
    w = W.bevformer_sca(cfg=47, B=2, Ncam=3, bev=6, shapes=((4, 4),), P=4, D=2)
    w["bev_mask"][:] = 0
    got, max_len, _ = run_rebatch(w)
    assert max_len == 0
    assert not got.any()

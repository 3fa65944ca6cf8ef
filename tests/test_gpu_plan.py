"""The operator in a locality order (msda_plan + msda_gather) and the
frame mean's two staging paths (all frames in one pass, or frame by frame),
against msda_forward / msda_forward_frames bit for bit and against the CPU
oracle.  Every call goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_abs_close, assert_fp32_close, dev, host

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def morton_bins(points):
    """Host form of the plan's tile index: 32 x 32 tiles of the clamped unit
    square, the bits of the row tile above those of the column tile."""
    t = np.minimum((np.clip(points.astype(np.float32), 0, 1) * np.float32(32)).astype(np.int64), 31)
    code = np.zeros(t.shape[:-1], np.int64)
    for bit in range(5):
        code |= ((t[..., 0] >> bit) & 1) << (2 * bit) | ((t[..., 1] >> bit) & 1) << (2 * bit + 1)
    return code


def check_plan(plan, points, B, Nq):
    """Each batch item's entries are its queries, each once, in tile order."""
    plan = plan[:B * Nq].reshape(B, Nq).astype(np.int64)
    bins = morton_bins(points.reshape(B * Nq, 2)).reshape(-1)
    for b in range(B):
        assert np.array_equal(np.sort(plan[b]), b * Nq + np.arange(Nq)), f"batch item {b}: not a permutation"
        assert np.all(np.diff(bins[plan[b]]) >= 0), f"batch item {b}: not in tile order"


def first_samples(loc, B, F, Nq):
    """The point standing for each query: its first sampling location (head 0,
    level 0, point 0; frame 0)."""
    return loc.reshape(B, F, Nq, -1)[:, 0, :, :2]


def test_plan_detr_encoder_full():
    w = W.detr_encoder_msda()
    B, Nq = w["B"], w["Nq"]
    loc = w["sampling_locations"]
    row = loc[0, 0].size
    d = [dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                             "attention_weights")]
    plan = msda.msda_plan(d[3], B, Nq, Nq * row, row)
    check_plan(host(msda.plan_order(plan, B, Nq)), first_samples(loc, B, 1, Nq), B, Nq)
    got = host(msda.msda_gather(*d, plan))
    ref = host(msda.msda_forward(*d))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "planned and unplanned results differ"
    assert_fp32_close(got.reshape(B * Nq, -1), oracle.msda(*[w[k] for k in (
        "value", "spatial_shapes", "level_start_index", "sampling_locations", "attention_weights")], True),
        "DETR encoder, planned, all 19947 queries")


def test_plan_temporal_frames_full():
    w = W.temporal_frames()
    B, F, Nq = w["B"], w["F"], w["Nq"]
    loc = w["sampling_locations"]
    row = loc[0, 0, 0].size
    d = [dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                             "attention_weights")]
    plan = msda.msda_plan(d[3], B, Nq, F * Nq * row, row)
    check_plan(host(msda.plan_order(plan, B, Nq)), first_samples(loc, B, F, Nq), B, Nq)
    got = host(msda.msda_gather(*d, plan))
    ref = host(msda.msda_forward_frames(*d))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "planned and unplanned results differ"


@pytest.mark.parametrize("B,Nq", [(3, 1000), (2, 1), (1, 70001)])
def test_plan_from_reference_points(B, Nq):
    """A plan built from reference points [B, Nq, 2] (some outside the unit
    square: clamped to its edge tiles) orders each batch item on its own."""
    g = np.random.default_rng(np.random.SeedSequence([77, B, Nq]))
    ref_pts = g.uniform(-0.3, 1.3, (B, Nq, 2)).astype(np.float32)
    plan = msda.msda_plan(dev(ref_pts), B, Nq, Nq * 2, 2)
    check_plan(host(msda.plan_order(plan, B, Nq)), ref_pts, B, Nq)
    if Nq <= 1000:
        w = {"value": g.normal(size=(B, 60, 8, 32)).astype(np.float32)}
        ss, st, Nv = W.level_table(((6, 8), (3, 4)))
        assert Nv == 60
        loc = (ref_pts[:, :, None, None, None, :] + g.normal(0, 0.05, (B, Nq, 8, 2, 4, 2))).astype(np.float32)
        lg = g.normal(size=(B, Nq, 8, 8)).astype(np.float32)
        d = [dev(w["value"]), dev(ss), dev(st), dev(loc), dev(lg)]
        got = host(msda.msda_gather(*d, plan))
        ref = host(msda.msda_forward(*d))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "planned and unplanned results differ"


def test_plan_empty_query_set():
    pts = torch.zeros((1, 2), device="cuda")
    plan = torch.full((msda.msda_plan_size(1, 0),), 7, dtype=torch.uint8, device="cuda")
    msda.msda_plan(pts, 1, 0, 0, 2, plan=plan)
    assert (host(plan) == 7).all()


def test_plan_reused_by_a_second_plan_call_and_other_sizes():
    """A plan buffer holding another call's counters is refilled correctly
    (the counters are cleared by the call itself), also for a smaller
    problem in a larger buffer."""
    g = np.random.default_rng(5)
    big = g.random((2, 5000, 2), dtype=np.float32)
    small = g.random((1, 333, 2), dtype=np.float32)
    buf = torch.empty(msda.msda_plan_size(2, 5000), dtype=torch.uint8, device="cuda")
    for pts, B, Nq in ((big, 2, 5000), (small, 1, 333), (big, 2, 5000)):
        msda.msda_plan(dev(pts), B, Nq, Nq * 2, 2, plan=buf)
        check_plan(host(msda.plan_order(buf, B, Nq)), pts, B, Nq)


def _frames_case(seed, B, F, Nq, shapes, nH, P, bf16=False):
    ss, starts, Nv = W.level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    value = g.normal(size=(B, F, Nv, nH, 32)).astype(np.float32)
    if bf16:
        value = W.bf16_bits_trunc(value)
    loc = g.uniform(-0.2, 1.2, (B, F, Nq, nH, L, P, 2)).astype(np.float32)
    w = g.normal(size=(B, F, Nq, nH, L * P)).astype(np.float32)
    return value, ss, starts, loc, w


# (id, seed, B, F, Nq, shapes, nH, P): F*L*P <= 32 and <= 64 stage every frame
# at once (one buffer over the F images); beyond 64 frame by frame
FRAMES = [
    ("flat_F3_LP8", 1, 2, 3, 45, ((6, 7), (3, 4)), 8, 4),
    ("flat_F4_LP12_wide_staging", 2, 1, 4, 33, ((5, 5), (4, 2), (2, 2)), 8, 4),
    ("flat_F64_one_point_each", 3, 1, 64, 17, ((4, 4),), 4, 1),
    ("flat_F5_odd_heads", 4, 2, 5, 19, ((3, 9),), 12, 1),
    ("per_frame_F3_LP32", 5, 1, 3, 29, ((8, 8), (4, 4), (2, 2), (1, 1)), 8, 8),
    ("per_frame_F2_LP64", 6, 2, 2, 13, ((8, 8), (4, 4), (2, 2), (1, 1)), 8, 16),
]


@pytest.mark.parametrize("case", FRAMES, ids=[c[0] for c in FRAMES])
def test_frames_staging_paths(case):
    _, seed, B, F, Nq, shapes, nH, P = case
    for bf16 in (False, True):
        value, ss, st, loc, w = _frames_case(seed, B, F, Nq, shapes, nH, P, bf16)
        for logits in (True, False):
            mode = msda.MSDA_WEIGHTS_LOGITS if logits else msda.MSDA_WEIGHTS_PROB
            out = msda.msda_forward_frames(dev(value), dev(ss), dev(st), dev(loc), dev(w), weight_mode=mode)
            ref = oracle.msda_frames(value, ss, st, loc, w, logits)
            assert_fp32_close(host(out).reshape(B * Nq, -1), ref, f"{case[0]} bf16={bf16} logits={logits}")

"""Backward pass of the MSDA operator and of SCA against the oracle's
gradients, element by element, on the same seeded inputs (workloads at full
size and the forward tests' edge cases).  Every call goes through the C ABI
(via the ctypes binding).

Tolerance: the float32 bar of the forward tests (1e-5 relative plus 1e-5 of
the output's rms) for the location / offset and weight / logit gradients.
The value gradient sums each row's contributions from every sample that
touches it (up to ~10^3 in the BEVFormer-base SCA workload's coarse levels)
in float32 -- in a fixed order by the transpose gather (the default), in no
fixed order with atomics -- so its bar is 1e-5 of the sum of the
contributions' magnitudes plus 1e-5 of that sum's rms over the elements
(gpu_util explains the rms term); the oracle gives the sum exactly:
contributions are alpha * w * g with alpha, w >= 0, so the oracle's value
gradient for |g| is that sum."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_fp32_close, assert_sum_close, dev, host
from test_gpu_parity import MSDA_EDGE, SCA_EDGE, _rand_msda, _rand_sca

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _grad_out(seed, B, Nq, C):
    return np.random.default_rng(seed).normal(size=(B, Nq, C)).astype(np.float32)


def check_msda_backward(w, gout, logits, what, atomic=False):
    mode = msda.MSDA_WEIGHTS_LOGITS if logits else msda.MSDA_WEIGHTS_PROB
    gv, gl, gw = msda.msda_backward(dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                                    dev(w["sampling_locations"]), dev(w["attention_weights"]), dev(gout),
                                    weight_mode=mode, atomic=atomic)
    rv, rl, rw = oracle.msda_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                      w["sampling_locations"], w["attention_weights"], gout, weights_are_logits=logits)
    mag, _, _ = oracle.msda_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                     w["sampling_locations"], w["attention_weights"], np.abs(gout),
                                     weights_are_logits=logits)
    if not logits:  # probabilities may be negative: the magnitude needs |alpha|
        mag, _, _ = oracle.msda_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                         w["sampling_locations"], np.abs(w["attention_weights"]), np.abs(gout),
                                         weights_are_logits=False)
    assert_sum_close(host(gv), rv, mag, what + ": grad value")
    assert_fp32_close(host(gl), rl, what + ": grad locations")
    assert_fp32_close(host(gw), rw, what + ": grad weights")


def test_tiny_msda_backward_all_modes():
    w = W.tiny_msda()
    gout = _grad_out(1, w["B"], w["Nq"], 256)
    check_msda_backward(w, gout, True, "logits")
    probs = np.random.default_rng(2).uniform(0, 0.2, w["attention_weights"].shape).astype(np.float32)
    check_msda_backward(dict(w, attention_weights=probs), gout, False, "probabilities")
    wb = dict(w, value=W.bf16_bits_trunc(w["value"]))
    check_msda_backward(wb, gout, True, "bf16 value")


def test_detr_encoder_msda_backward_full():
    """The DETR-encoder workload at full size: all 19947 queries, 4 levels."""
    w = W.detr_encoder_msda()
    gout = W.upstream_gradient(2, (w["B"], w["Nq"], 256))
    check_msda_backward(w, gout, True, "DETR encoder")


def test_detr_encoder_msda_backward_atomic():
    """The same with the value gradient accumulated by float32 atomics."""
    w = W.detr_encoder_msda()
    gout = W.upstream_gradient(2, (w["B"], w["Nq"], 256))
    check_msda_backward(w, gout, True, "DETR encoder, atomics", atomic=True)


@pytest.mark.parametrize("case", MSDA_EDGE, ids=[c[0] for c in MSDA_EDGE])
def test_msda_backward_edge_cases(case):
    _, seed, B, Nq, shapes, nH, P = case
    w = _rand_msda(seed, B, Nq, shapes, nH, P)
    gout = _grad_out(seed + 100, B, Nq, nH * 32)
    check_msda_backward(w, gout, True, case[0])
    probs = np.abs(w["attention_weights"]) / 8
    check_msda_backward(dict(w, attention_weights=probs), gout, False, case[0] + " probabilities")


@pytest.mark.parametrize("atomic", [False, True], ids=["gather", "atomic"])
def test_msda_backward_empty_query_set(atomic):
    """No queries: the value gradient is zero (overwritten), nothing else is touched."""
    w = _rand_msda(5, 1, 0, ((4, 4),), 8, 4)
    gv = torch.full((1, w["Nv"], 8, 32), float("nan"), device="cuda")
    empty = torch.empty(0, device="cuda")
    gv, _, _ = msda.msda_backward(dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                                  dev(w["sampling_locations"]), dev(w["attention_weights"]), empty.view(1, 0, 256),
                                  grad_value=gv, atomic=atomic)
    assert not host(gv).any()


def test_msda_backward_repeatable():
    """With the transpose gather every output, the value gradient included, is
    the same bit for bit over two runs (one of them into a workspace full of
    stale records from a different call); with atomics the locations and
    weights gradients still are, and the value gradient agrees to the float32
    bar."""
    w = _rand_msda(6, 2, 300, ((16, 24), (8, 12)), 8, 4)
    gout = _grad_out(7, 2, 300, 256)
    args = (dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]), dev(w["sampling_locations"]),
            dev(w["attention_weights"]), dev(gout))
    ws = torch.empty(msda.msda_backward_workspace_size(2, w["Nv"], 300, 8, 2, 4), dtype=torch.uint8, device="cuda")
    a = [host(t) for t in msda.msda_backward(*args, grad_workspace=ws)]
    other = _rand_msda(16, 2, 300, ((16, 24), (8, 12)), 8, 4)
    msda.msda_backward(dev(other["value"]), *args[1:3], dev(other["sampling_locations"]),
                       dev(other["attention_weights"]), args[5], grad_workspace=ws)
    b = [host(t) for t in msda.msda_backward(*args, grad_workspace=ws)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = [host(t) for t in msda.msda_backward(*args, atomic=True)]
    d = [host(t) for t in msda.msda_backward(*args, atomic=True)]
    assert np.array_equal(c[1], d[1]) and np.array_equal(c[2], d[2])
    assert np.array_equal(a[1], c[1]) and np.array_equal(a[2], c[2])
    mag, _, _ = oracle.msda_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                     w["sampling_locations"], w["attention_weights"], np.abs(gout),
                                     weights_are_logits=True)
    assert_sum_close(c[0], d[0], 2 * mag, "value gradient with atomics, two runs")
    assert_sum_close(a[0], c[0], 2 * mag, "value gradient, gather against atomics")


# ---------------------------------------------------------------------------
# SCA
# ---------------------------------------------------------------------------

def run_sca_backward(w, gout, **kw):
    B, Ncam, Nq = w["B"], w["Ncam"], w["Nq"]
    ws = torch.empty(msda.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device="cuda")
    msda.sca_compact(dev(w["bev_mask"]), dev(w["reference_points_cam"]), ws)
    go = torch.full((B, Nq, w["nH"], w["L"], w["P"], 2), float("nan"), device="cuda")
    gl = torch.full((B, Nq, w["nH"], w["L"] * w["P"]), float("nan"), device="cuda")
    gv, go, gl = msda.sca_backward(dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                                   dev(w["reference_points_cam"]), dev(w["sampling_offsets"]),
                                   dev(w["attention_logits"]), dev(gout), ws, grad_offsets=go, grad_logits=gl, **kw)
    return host(gv), host(go), host(gl)


def check_sca_backward(w, gout, what, **kw):
    gv, go, gl = run_sca_backward(w, gout, **kw)
    rv, ro, rl = oracle.sca_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                     w["reference_points_cam"], w["bev_mask"], w["sampling_offsets"],
                                     w["attention_logits"], gout)
    mag, _, _ = oracle.sca_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                    w["reference_points_cam"], w["bev_mask"], w["sampling_offsets"],
                                    w["attention_logits"], np.abs(gout))
    assert_sum_close(gv, rv, mag, what + ": grad value")
    assert_fp32_close(go, ro, what + ": grad offsets")
    assert_fp32_close(gl, rl, what + ": grad logits")


def check_frames_backward(w, gout, what, logits=True, atomic=False):
    mode = msda.MSDA_WEIGHTS_LOGITS if logits else msda.MSDA_WEIGHTS_PROB
    args = (w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"], w["attention_weights"])
    gv, gl, gw = (host(t) for t in msda.msda_backward_frames(*(dev(x) for x in args), dev(gout), weight_mode=mode,
                                                              atomic=atomic))
    rv, rl, rw = oracle.msda_frames_backward(*args, gout, weights_are_logits=logits)
    wmag = w["attention_weights"] if logits else np.abs(w["attention_weights"])
    mag = oracle.msda_frames_backward(*args[:4], wmag, np.abs(gout), weights_are_logits=logits)[0]
    assert_sum_close(gv, rv, mag, what + ": grad value")
    assert_fp32_close(gl, rl, what + ": grad locations")
    assert_fp32_close(gw, rw, what + ": grad weights")
    return gv


def test_temporal_frames_backward_full():
    """The frame mean's backward on the temporal workload at full size: two
    stacked 200x200 BEV maps, all 40000 queries, both value-gradient paths."""
    w = W.temporal_frames()
    gout = W.upstream_gradient(4, (w["B"], w["Nq"], 256))
    check_frames_backward(w, gout, "two stacked BEV maps")
    check_frames_backward(w, gout, "two stacked BEV maps, atomics", atomic=True)


def test_msda_frames_backward_three_frames():
    """Three frames (the division is not by a power of two), batch 2, two
    levels: logits, probabilities and a bf16 value map."""
    g = np.random.default_rng(43)
    B, F, Nq, nH, P = 2, 3, 37, 4, 3
    shapes = ((5, 7), (3, 2))
    ss, starts, Nv = W.level_table(shapes)
    w = {"value": g.normal(size=(B, F, Nv, nH, 32)).astype(np.float32), "spatial_shapes": ss,
         "level_start_index": starts,
         "sampling_locations": g.uniform(-0.2, 1.2, (B, F, Nq, nH, 2, P, 2)).astype(np.float32),
         "attention_weights": g.normal(size=(B, F, Nq, nH, 2 * P)).astype(np.float32)}
    gout = _grad_out(243, B, Nq, nH * 32)
    check_frames_backward(w, gout, "three frames")
    check_frames_backward(dict(w, attention_weights=g.uniform(0, 0.3, w["attention_weights"].shape)
                               .astype(np.float32)), gout, "three frames, probabilities", logits=False)
    check_frames_backward(dict(w, value=W.bf16_bits_trunc(w["value"])), gout, "three frames, bf16 value")


def test_bevformer_sca_backward_full():
    """The BEVFormer-base SCA workload at full size: 40000 queries, 6 cameras."""
    w = W.bevformer_sca()
    gout = W.upstream_gradient(3, (w["B"], w["Nq"], 256))
    check_sca_backward(w, gout, "BEVFormer-base SCA")


def test_bevformer_sca_backward_bf16_value():
    """The BEVFormer-base SCA workload's shapes with a bf16 value map, batch 2 at 100x100 queries."""
    w = W.bevformer_sca(cfg=33, B=2, bev=100, value_bf16=True)
    gout = W.upstream_gradient(33, (w["B"], w["Nq"], 256))
    check_sca_backward(w, gout, "bf16 value")


@pytest.mark.parametrize("case", SCA_EDGE, ids=[c[0] for c in SCA_EDGE])
def test_sca_backward_edge_cases(case):
    _, seed, B, Ncam, Nq, shapes, nH, P, D, pm = case
    w = _rand_sca(seed, B, Ncam, Nq, shapes, nH, P, D, pm)
    gout = _grad_out(seed + 200, B, Nq, nH * 32)
    check_sca_backward(w, gout, case[0])


def test_sca_backward_many_uneven_segments():
    """The value gradient's records are kept per (image, head): 4 x 8 cameras x
    16 heads = 512 segments (more than one block of the setup handles at a
    time), of unequal sizes -- camera 0 sees every query (two sort tiles per
    head), camera 7 none (empty segments), the others about a third."""
    w = _rand_sca(41, 4, 8, 300, ((6, 10), (3, 5)), 16, 4, 2, 0.2)
    w["bev_mask"][0] = 1
    w["bev_mask"][7] = 0
    gout = _grad_out(241, 4, 300, 16 * 32)
    check_sca_backward(w, gout, "512 uneven segments")


def test_msda_backward_many_segments():
    """40 batch items x 8 heads = 320 segments of one sort tile each."""
    w = _rand_msda(42, 40, 50, ((4, 4),), 8, 2)
    gout = _grad_out(242, 40, 50, 256)
    check_msda_backward(w, gout, True, "320 segments")


def test_bevformer_sca_backward_atomic():
    """The full-size SCA workload with the value gradient accumulated by float32 atomics."""
    w = W.bevformer_sca()
    gout = W.upstream_gradient(3, (w["B"], w["Nq"], 256))
    check_sca_backward(w, gout, "BEVFormer-base SCA, atomics", atomic=True)


def _pair_count(w):
    return int(w["bev_mask"].any(-1).sum())


def test_sca_backward_repeatable_and_exact_capacity():
    """A gradient workspace sized for exactly the pairs the compaction finds
    gives the same bits as one sized for every camera seeing every query, and
    two runs agree bit for bit."""
    w = _rand_sca(61, 2, 6, 300, ((12, 20), (6, 10)), 8, 8, 4, 0.6)
    gout = _grad_out(62, 2, 300, 256)
    n = _pair_count(w)
    a = run_sca_backward(w, gout)
    b = run_sca_backward(w, gout, max_pairs=n)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    check_sca_backward(w, gout, "exact capacity", max_pairs=n)


def test_sca_backward_too_few_pairs_gives_nan():
    """A gradient workspace for fewer pairs than the compaction finds: the
    value gradient is all NaN (the other outputs do not depend on it)."""
    w = _rand_sca(63, 1, 6, 200, ((12, 20), (6, 10)), 8, 8, 4, 0.6)
    gout = _grad_out(64, 1, 200, 256)
    n = _pair_count(w)
    assert n > 1
    gv, go, gl = run_sca_backward(w, gout, max_pairs=n - 1)
    assert np.isnan(gv).all()
    _, ro, rl = run_sca_backward(w, gout)
    assert np.array_equal(go, ro) and np.array_equal(gl, rl)


def _msda_with_levels(seed, Nq, shapes, starts, Nv, nH=8, P=4):
    g = np.random.default_rng(seed)
    ss = np.asarray(shapes, np.int64).reshape(-1, 2)
    L = len(ss)
    return {"value": g.normal(size=(1, Nv, nH, 32)).astype(np.float32), "spatial_shapes": ss,
            "level_start_index": np.asarray(starts, np.int64),
            "sampling_locations": g.uniform(-0.2, 1.2, (1, Nq, nH, L, P, 2)).astype(np.float32),
            "attention_weights": g.normal(size=(1, Nq, nH, L * P)).astype(np.float32),
            "B": 1, "Nq": Nq, "Nv": Nv, "nH": nH, "Dh": 32, "L": L, "P": P}


def test_msda_backward_overlapping_levels():
    """Levels whose rows overlap (level 1 reuses rows 4..7 of level 0): a value
    row's gradient sums the samples of every level that reads it."""
    w = _msda_with_levels(71, 60, ((4, 4), (2, 2)), (0, 4), 16)
    gout = _grad_out(72, 1, 60, 256)
    check_msda_backward(w, gout, True, "overlapping levels")


def test_msda_backward_level_table_beyond_key_range():
    """Four 2x2 levels on the same 4 rows: their cell corners (4 x 9) exceed the
    2 Nv + 2 L keys the gradient workspace provides, so the transpose gather
    fills grad_value with NaN; the atomic path and the other gradients are
    unaffected."""
    w = _msda_with_levels(73, 30, ((2, 2),) * 4, (0, 0, 0, 0), 4)
    gout = _grad_out(74, 1, 30, 256)
    args = (dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]), dev(w["sampling_locations"]),
            dev(w["attention_weights"]), dev(gout))
    gv, gl, gw = (host(t) for t in msda.msda_backward(*args))
    assert np.isnan(gv).all()
    _, rl, rw = oracle.msda_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                     w["sampling_locations"], w["attention_weights"], gout, weights_are_logits=True)
    assert_fp32_close(gl, rl, "grad locations")
    assert_fp32_close(gw, rw, "grad weights")
    check_msda_backward(w, gout, True, "shared 2x2 levels, atomics", atomic=True)

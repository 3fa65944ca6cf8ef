"""HIP path against the CPU oracle, element by element, on the same seeded
inputs: the five workloads at full size and edge cases at small sizes.
Every call goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (announce, assert_abs_close, assert_bf16_ulp_close, assert_fp32_close, bf16_bits_to_f64, dev,
                      host, oracle_by_rows)

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _softmax(x):
    e = np.exp(x.astype(np.float64) - x.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def run_msda(w, mode=msda.MSDA_WEIGHTS_LOGITS, weights=None):
    weights = w["attention_weights"] if weights is None else weights
    out = msda.msda_forward(dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                            dev(w["sampling_locations"]), dev(weights), weight_mode=mode)
    return host(out).reshape(-1, w["nH"] * w["Dh"])


def oracle_msda(w, logits=True, weights=None, rows=None):
    weights = w["attention_weights"] if weights is None else weights
    return oracle.msda(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"], weights,
                       weights_are_logits=logits, rows=rows)


def run_sca(w, value=None, want_compaction=True):
    value = w["value"] if value is None else value
    B, Ncam, Nq = w["B"], w["Ncam"], w["Nq"]
    hit = torch.full((B, Nq), -7, dtype=torch.int32, device="cuda")
    offs = torch.full((B * Ncam + 1,), -7, dtype=torch.int32, device="cuda")
    pq = torch.full((max(1, B * Ncam * Nq),), -7, dtype=torch.int32, device="cuda")
    slots = torch.full((B, Nq, w["nH"] * w["Dh"]), float("nan"), dtype=torch.float32, device="cuda")
    vt = value if isinstance(value, torch.Tensor) else dev(value)
    msda.sca_forward(vt, dev(w["spatial_shapes"]), dev(w["level_start_index"]), dev(w["reference_points_cam"]),
                     dev(w["bev_mask"]), dev(w["sampling_offsets"]), dev(w["attention_logits"]), slots=slots,
                     hit_count=hit if want_compaction else None, pair_offsets=offs if want_compaction else None,
                     pair_q=pq if want_compaction else None)
    res = {"slots": host(slots).reshape(B * Nq, w["nH"] * w["Dh"])}
    if want_compaction:
        res["hit_count"] = host(hit)
        res["pair_offsets"] = host(offs)
        n = int(res["pair_offsets"][-1])
        res["pair_q"] = host(pq)[:n]
    return res


def oracle_sca(w, value=None, rows=None):
    value = w["value"] if value is None else value
    return oracle.sca(value, w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"], w["bev_mask"],
                      w["sampling_offsets"], w["attention_logits"], rows=rows)


def check_compaction(got, ref, what):
    assert np.array_equal(got["hit_count"], ref["hit_count"]), f"{what}: hit counts differ"
    assert np.array_equal(got["pair_offsets"], ref["pair_offsets"]), f"{what}: pair offsets differ"
    assert np.array_equal(got["pair_q"], ref["pair_q"]), f"{what}: pair lists differ"


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_tiny_msda_fp32_logits_and_probabilities():
    w = W.tiny_msda()
    assert_fp32_close(run_msda(w), oracle_msda(w), "tiny MSDA, logits")
    p = _softmax(w["attention_weights"])
    assert_fp32_close(run_msda(w, msda.MSDA_WEIGHTS_PROB, p), oracle_msda(w, False, p), "tiny MSDA, probabilities")


def test_tiny_msda_bf16_value():
    w = W.msda_workload(1, 1, 256, ((32, 32),), P=4, value_bf16=True)
    assert_abs_close(run_msda(w), oracle_msda(w), 1e-2, "tiny MSDA, bf16 value")
    # tighter than the bf16 bar: the bf16 values are decoded exactly, only fp32 accumulation differs
    assert_fp32_close(run_msda(w), oracle_msda(w), "tiny MSDA, bf16 value (exact decode)")


def test_detr_encoder_msda_full():
    w = W.detr_encoder_msda()
    got = run_msda(w)
    assert_fp32_close(got, oracle_msda(w), "DETR encoder, all 19947 queries")


def test_temporal_frames_full():
    w = W.temporal_frames()
    out = msda.msda_forward_frames(dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                                   dev(w["sampling_locations"]), dev(w["attention_weights"]))
    ref = oracle.msda_frames(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                             w["attention_weights"], True)
    assert_fp32_close(host(out).reshape(-1, 256), ref, "two stacked BEV maps, all 40000 queries")


def test_bevformer_sca_full():
    w = W.bevformer_sca()
    got = run_sca(w)
    ref = oracle_sca(w)
    check_compaction(got, ref, "BEVFormer-base SCA")
    assert ref["pair_offsets"][-1] > 40000  # queries seen by two cameras exist
    assert_fp32_close(got["slots"], ref["slots"], "BEVFormer-base SCA, all 40000 queries")


def test_bevformer_sca_bf16_layer_with_projections():
    """The batch-4 bf16 layer workload: value projection (bf16 GEMM) -> SCA on bf16 value -> output
    projection (bf16 GEMM from fp32 slots).  The oracle runs its own chain:
    fp64 projection rounded to bf16, SCA on that, fp64 projection of the
    bf16-rounded slots.  Every row of every stage is compared."""
    w = W.bevformer_sca_bf16(bias=True)
    B, Ncam, Nq, Nv = w["B"], w["Ncam"], w["Nq"], w["Nv"]
    C = 256
    feat = w["feat"].reshape(-1, C)
    M = feat.shape[0]
    v = msda.msda_gemm_bf16(dev(feat), dev(w["W_v"]), dev(w["b_v"]), y_dtype=torch.bfloat16)
    v_host = host(v)
    # every one of the 739,800 rows against the float64-matmul form of the
    # oracle's projection, and sampled rows against its plain-loop form
    proj = oracle.linear_bf16_blas(feat, w["W_v"], w["b_v"])
    assert_bf16_ulp_close(v_host, proj, f"value projection, all {M} rows")
    rows_v = W.sample_rows(5, M, 2048)
    assert_bf16_ulp_close(v_host[rows_v], oracle.linear_bf16(feat[rows_v], w["W_v"], w["b_v"]),
                          "value projection (sampled rows, loop form)")

    # oracle value: its own projection, rounded to bf16, for every row
    ref_value = oracle.round_to_bf16(proj).reshape(B, Ncam, Nv, 8, 32)
    del proj
    value_gpu = v.view(B, Ncam, Nv, 8, 32)
    got = run_sca(w, value=value_gpu)
    ref = oracle.sca(ref_value, w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"],
                     w["bev_mask"], w["sampling_offsets"], w["attention_logits"], want_slots=False)
    check_compaction(got, ref, "batch-4 bf16 layer")
    ref_slots = oracle_by_rows(lambda r: oracle_sca(w, value=ref_value, rows=r)["slots"], np.arange(B * Nq))
    assert_abs_close(got["slots"], ref_slots, 1e-2, f"batch-4 bf16 layer SCA slots, all {B * Nq} queries")

    slots_gpu = torch.from_numpy(got["slots"]).cuda()
    o = msda.msda_gemm_bf16(slots_gpu, dev(w["W_o"]), dev(w["b_o"]), y_dtype=torch.float32)
    ref_o = oracle.linear_bf16_blas(oracle.round_to_bf16(ref_slots), w["W_o"], w["b_o"])
    assert_abs_close(host(o), ref_o, 1e-2, f"batch-4 bf16 layer output projection, all {B * Nq} rows")


# ---------------------------------------------------------------------------
# edge cases: MSDA operator
# ---------------------------------------------------------------------------

def _rand_msda(seed, B, Nq, shapes, nH, P, lo=-0.2, hi=1.2, bf16=False):
    ss, starts, Nv = W.level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    value = g.normal(size=(B, Nv, nH, 32)).astype(np.float32)
    if bf16:
        value = W.bf16_bits_trunc(value)
    loc = g.uniform(lo, hi, (B, Nq, nH, L, P, 2)).astype(np.float32)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    return {"value": value, "spatial_shapes": ss, "level_start_index": starts, "sampling_locations": loc,
            "attention_weights": logits, "B": B, "Nq": Nq, "Nv": Nv, "nH": nH, "Dh": 32, "L": L, "P": P}


MSDA_EDGE = [
    # id, seed, B, Nq, shapes, nH, P
    ("ragged_queries_nH4", 1, 2, 37, ((5, 7), (3, 2)), 4, 3),
    ("two_head_passes_nH12_odd_LP", 2, 3, 19, ((6, 4),), 12, 5),
    ("one_head_one_point", 3, 1, 9, ((4, 4),), 1, 1),
    ("max_points_LP64", 4, 1, 33, ((8, 8), (4, 4), (2, 2), (1, 1)), 8, 16),
    ("unit_levels_and_wide", 5, 2, 21, ((1, 1), (1, 40), (17, 1)), 8, 4),
    ("single_query", 6, 1, 1, ((9, 13),), 8, 2),
    ("many_heads_nH64", 7, 1, 5, ((3, 5),), 64, 2),
]


@pytest.mark.parametrize("case", MSDA_EDGE, ids=[c[0] for c in MSDA_EDGE])
def test_msda_edge_cases(case):
    _, seed, B, Nq, shapes, nH, P = case
    w = _rand_msda(seed, B, Nq, shapes, nH, P)
    assert_fp32_close(run_msda(w), oracle_msda(w), case[0])
    wb = _rand_msda(seed, B, Nq, shapes, nH, P, bf16=True)
    assert_fp32_close(run_msda(wb), oracle_msda(wb), case[0] + " bf16")


def test_msda_locations_on_borders_and_far_outside():
    w = _rand_msda(11, 1, 64, ((6, 10), (3, 5)), 8, 4)
    loc = w["sampling_locations"]
    g = np.random.default_rng(12)
    special = np.array([0.0, 1.0, -0.0, 0.5, 1e-8, 1 - 1e-7, -0.05, 1.05, 1e6, -1e6, 3e38, -3e38, 2.0, -1.0],
                       np.float32)
    idx = g.integers(0, len(special), loc.shape)
    mix = g.random(loc.shape) < 0.5
    loc[mix] = special[idx[mix]]
    # exact pixel centres and pixel edges of level 0
    loc[0, :8, :, 0, :, 0] = (np.arange(8)[:, None, None] % 10 + 0.5) / 10
    loc[0, 8:16, :, 0, :, 0] = (np.arange(8)[:, None, None] % 10) / 10
    assert_fp32_close(run_msda(w), oracle_msda(w), "borders and far outside")


def test_msda_probabilities_not_normalised():
    """Probability mode uses the weights as given (the operator's contract)."""
    w = _rand_msda(13, 2, 40, ((7, 9), (4, 5)), 8, 4)
    p = np.random.default_rng(14).uniform(-1, 2, w["attention_weights"].shape).astype(np.float32)
    assert_fp32_close(run_msda(w, msda.MSDA_WEIGHTS_PROB, p), oracle_msda(w, False, p), "raw weights")


def test_msda_inconsistent_level_table_reads_zero_outside():
    """A level whose pixels run past Nv reads zero for those rows and never
    faults: the start of level 1 points into the middle of level 0 (legal
    rows) and level 2 runs beyond the end (rows >= Nv read zero)."""
    w = _rand_msda(15, 1, 30, ((4, 6), (2, 3), (3, 3)), 8, 4, lo=0.0, hi=1.0)
    w["level_start_index"] = np.array([0, 10, 35], np.int64)  # Nv = 24 + 6 + 9 = 39; 35 + 9 > 39
    got = run_msda(w)
    # oracle refuses such tables; compare with a value tensor extended by
    # zero rows so that the oracle's table is consistent
    ext = dict(w)
    ext["value"] = np.concatenate([w["value"], np.zeros((1, 10, 8, 32), np.float32)], axis=1)
    assert_fp32_close(got, oracle_msda(ext), "inconsistent level table")


def test_msda_empty_query_set():
    w = _rand_msda(16, 1, 0, ((4, 4),), 8, 4)
    out = torch.full((1, 0, 256), 3.0, device="cuda")
    msda.msda_forward(dev(w["value"]), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                      dev(w["sampling_locations"]), dev(w["attention_weights"]), out=out)
    assert out.numel() == 0


def test_sca_empty_query_set():
    w = _rand_sca(34, 2, 3, 0, ((4, 4),), 8, 4, 4)
    slots = run_sca(w, want_compaction=False)["slots"]
    assert slots.size == 0


def test_msda_deterministic():
    w = W.detr_encoder_msda()
    a = run_msda(w)
    b = run_msda(w)
    assert np.array_equal(a, b), "two runs differ bitwise"


def test_frames_identical_frames_equal_single():
    w = _rand_msda(17, 2, 50, ((8, 8),), 8, 4)
    st = lambda x: np.ascontiguousarray(np.stack([x, x], axis=1))
    out = msda.msda_forward_frames(dev(st(w["value"])), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                                   dev(st(w["sampling_locations"])), dev(st(w["attention_weights"])))
    assert_fp32_close(host(out).reshape(-1, 256), oracle_msda(w), "identical frames")
    f3 = lambda x: np.ascontiguousarray(np.stack([x, x * 0.5, -x], axis=1))
    out3 = msda.msda_forward_frames(dev(f3(w["value"])), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                                    dev(st(w["sampling_locations"])[:, [0, 1, 0]].copy()),
                                    dev(st(w["attention_weights"])[:, [0, 1, 0]].copy()))
    ref3 = oracle.msda_frames(f3(w["value"]), w["spatial_shapes"], w["level_start_index"],
                              st(w["sampling_locations"])[:, [0, 1, 0]].copy(),
                              st(w["attention_weights"])[:, [0, 1, 0]].copy(), True)
    assert_fp32_close(host(out3).reshape(-1, 256), ref3, "three frames")


# ---------------------------------------------------------------------------
# edge cases: SCA
# ---------------------------------------------------------------------------

def _rand_sca(seed, B, Ncam, Nq, shapes, nH, P, D, p_mark=0.3, bf16=False):
    ss, starts, Nv = W.level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    value = g.normal(size=(B, Ncam, Nv, nH, 32)).astype(np.float32)
    if bf16:
        value = W.bf16_bits_trunc(value)
    mask = (g.random((Ncam, B, Nq, D)) < p_mark).astype(np.uint8)
    rho = g.uniform(-0.1, 1.1, (Ncam, B, Nq, D, 2)).astype(np.float32)
    off = g.normal(0, 2.0, (B, Nq, nH, L, P, 2)).astype(np.float32)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    return {"value": value, "spatial_shapes": ss, "level_start_index": starts, "reference_points_cam": rho,
            "bev_mask": mask, "sampling_offsets": off, "attention_logits": logits, "B": B, "Ncam": Ncam,
            "Nq": Nq, "Nv": Nv, "nH": nH, "Dh": 32, "L": L, "P": P, "D": D}


SCA_EDGE = [
    # id, seed, B, Ncam, Nq, shapes, nH, P, D, p_mark
    ("batch_masks_differ", 21, 3, 3, 50, ((6, 9), (3, 4)), 8, 4, 2, 0.3),
    ("multi_tile_ragged", 22, 2, 6, 700, ((8, 12), (4, 6)), 8, 8, 4, 0.15),
    ("one_camera", 23, 2, 1, 33, ((5, 5),), 8, 4, 4, 0.5),
    ("thirty_two_cameras", 24, 1, 32, 40, ((4, 6),), 8, 2, 1, 0.2),
    # every tile's queries start in many cameras: the compaction scans many segments per tile
    ("thirty_two_cameras_multi_tile", 31, 2, 32, 600, ((4, 6),), 8, 2, 1, 0.04),
    # many batch items: 240 segments, die shares per item, pair offsets across items
    ("forty_batch_items", 32, 40, 6, 60, ((5, 7), (3, 4)), 8, 4, 2, 0.3),
    ("anchor_per_point_D1_P3", 25, 1, 4, 30, ((5, 7), (2, 3)), 8, 3, 1, 0.4),
    ("half_heads_nH4", 26, 2, 3, 45, ((6, 6),), 4, 4, 2, 0.3),
    ("two_passes_nH16", 27, 1, 3, 25, ((6, 6),), 16, 4, 4, 0.3),
    ("nobody_sees_anything", 28, 2, 3, 20, ((4, 4),), 8, 4, 4, 0.0),
    ("everybody_sees_everything", 29, 1, 5, 20, ((4, 4), (2, 2)), 8, 4, 4, 1.0),
    ("max_points_LP64", 30, 1, 2, 24, ((8, 8), (4, 4)), 8, 32, 8, 0.4),
]


@pytest.mark.parametrize("case", SCA_EDGE, ids=[c[0] for c in SCA_EDGE])
def test_sca_edge_cases(case):
    _, seed, B, Ncam, Nq, shapes, nH, P, D, pm = case
    w = _rand_sca(seed, B, Ncam, Nq, shapes, nH, P, D, pm)
    got = run_sca(w)
    ref = oracle_sca(w)
    check_compaction(got, ref, case[0])
    assert_fp32_close(got["slots"], ref["slots"], case[0])
    wb = _rand_sca(seed, B, Ncam, Nq, shapes, nH, P, D, pm, bf16=True)
    gb = run_sca(wb, want_compaction=False)
    assert_fp32_close(gb["slots"], oracle_sca(wb)["slots"], case[0] + " bf16")


def test_sca_stages_and_compaction_reuse():
    """sca_compact once, sca_gather twice (two layers sharing one mask and
    anchors) equals sca_forward; the pair lists can live in the workspace
    only."""
    w = _rand_sca(31, 2, 6, 300, ((8, 12), (4, 6)), 8, 8, 4, 0.2)
    ws = torch.empty(msda.sca_workspace_size(2, 6, 300), dtype=torch.uint8, device="cuda")
    msda.sca_compact(dev(w["bev_mask"]), dev(w["reference_points_cam"]), ws)
    args = (dev(w["spatial_shapes"]), dev(w["level_start_index"]), dev(w["reference_points_cam"]),
            dev(w["sampling_offsets"]), dev(w["attention_logits"]), ws)
    s1 = host(msda.sca_gather(dev(w["value"]), *args)).reshape(600, -1)
    v2 = np.ascontiguousarray(w["value"][:, ::-1])
    s2 = host(msda.sca_gather(dev(v2), *args)).reshape(600, -1)
    assert_fp32_close(s1, oracle_sca(w)["slots"], "stage path, layer 1")
    assert_fp32_close(s2, oracle_sca(w, value=v2)["slots"], "stage path, layer 2")
    # the gather only reads the workspace, so the compaction serves any
    # number of launches: later launches into NaN-filled outputs still write
    # every row, with the same bits
    for k in range(4):
        out = torch.full((2, 300, 256), float("nan"), dtype=torch.float32, device="cuda")
        msda.sca_gather(dev(w["value"]), *args, slots=out)
        assert np.array_equal(host(out).reshape(600, -1), s1), f"stage path, repeat {k}"


def test_sca_deterministic():
    w = _rand_sca(32, 1, 6, 2000, ((16, 24), (8, 12)), 8, 8, 4, 0.2)
    a = run_sca(w)
    b = run_sca(w)
    assert np.array_equal(a["slots"], b["slots"]), "two runs differ bitwise"


def test_sca_rejects_bad_shapes_with_status():
    w = _rand_sca(33, 1, 2, 10, ((4, 4),), 8, 6, 4, 0.3)  # P % D != 0
    with pytest.raises(msda.MsdaError) as e:
        run_sca(w)
    assert e.value.code == 3  # MSDA_ERR_SHAPE

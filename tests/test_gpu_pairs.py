"""The head-pair layout of a bf16 value (MSDA_BF16_PAIRS: per image
[nH][Nv][2][32], line (h, p) = pixel p of head h, then pixel p + 1).

- msda_value_proj_pairs_bf16 and msda_pack_pairs_bf16 against a host
  re-indexing of the plain layout (bit for bit), and the projection against
  the oracle's;
- SCA on a value in pairs against the CPU oracle on the plain value: every
  row of the batch-4 bf16 layer workload, the SCA edge cases, levels so
  small that most corner pairs straddle a border, the stage path and the
  allocation-free entry point;
- the operator and its frame mean on a value in pairs: the DETR encoder and
  temporal workloads on every query (planned and unplanned, bit for bit),
  the operator's edge cases, both frame-staging paths, row ends.
Every call goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_abs_close, assert_bf16_ulp_close, assert_fp32_close, dev, host, oracle_by_rows

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def pairs_host(bits):
    """Host re-indexing of bf16 bits [..., Nv, nH, 32] into the head-pair
    layout [..., nH, Nv, 2, 32]: line (h, p) = pixel p, then pixel p + 1;
    zeros after the last pixel."""
    t = np.moveaxis(bits, -3, -2)
    out = np.zeros(t.shape[:-1] + (2, 32), bits.dtype)
    out[..., 0, :] = t
    out[..., :-1, 1, :] = t[..., 1:, :]
    return out


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


# ---------------------------------------------------------------------------
# the layout's producers
# ---------------------------------------------------------------------------

PROJ = [
    # id, n_images, Nv, K, N, bias, x_f32
    ("one_image_seven_pixels", 1, 7, 64, 96, True, True),
    ("single_pixel_images", 3, 1, 32, 32, False, False),
    ("ragged_tiles", 3, 100, 256, 256, True, True),
    ("two_column_blocks", 2, 63, 128, 512, True, False),
]


@pytest.mark.parametrize("case", PROJ, ids=[c[0] for c in PROJ])
def test_value_proj_pairs_small(case):
    _, n_img, Nv, K, N, use_bias, x_f32 = case
    g = np.random.default_rng(n_img * 1000 + Nv)
    M = n_img * Nv
    X = g.normal(size=(M, K)).astype(np.float32)
    if not x_f32:
        X = W.bf16_bits_trunc(X)
    Wt = W.bf16_bits_trunc(g.normal(size=(N, K)).astype(np.float32) / np.sqrt(K))
    bias = g.normal(size=N).astype(np.float32) if use_bias else None
    pr = msda.msda_value_proj_pairs_bf16(dev(X), dev(Wt), None if bias is None else dev(bias), Nv)
    plain = msda.msda_gemm_bf16(dev(X), dev(Wt), None if bias is None else dev(bias), y_dtype=torch.bfloat16)
    assert tuple(pr.shape) == (n_img, N // 32, Nv, 2, 32)
    ref_bits = pairs_host(_bits(plain).reshape(n_img, Nv, N // 32, 32))
    assert np.array_equal(_bits(pr), ref_bits), "pairs != plain projection re-indexed"
    proj = oracle.linear_bf16(X, Wt, bias)  # X: float32, or bf16 bits
    left = host(pr)[:, :, :, 0, :].transpose(0, 2, 1, 3).reshape(M, N)  # bf16 bits
    assert_bf16_ulp_close(left, proj, "pairs projection against the oracle")


def test_pack_pairs_keeps_every_bit():
    """A pure copy: random bit patterns (NaN and infinity encodings
    included) come out where the layout puts them."""
    g = np.random.default_rng(41)
    for shape in [(2, 3, 5, 8, 32), (1, 1, 1, 1, 32), (4, 1000, 16, 32), (7, 3, 32)]:
        bits = g.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        bits[..., :2] = np.array([0x7FC1, 0xFF80], np.uint16)  # a NaN and -inf in every row
        got = msda.msda_pack_pairs_bf16(dev(bits))
        assert np.array_equal(_bits(got), pairs_host(bits.view(np.int16))), shape
    empty = torch.empty((0, 5, 8, 32), dtype=torch.bfloat16, device="cuda")
    assert msda.msda_pack_pairs_bf16(empty).numel() == 0


# ---------------------------------------------------------------------------
# SCA on a value in pairs
# ---------------------------------------------------------------------------

def run_sca_pairs(w, value_pairs, **kw):
    B, Ncam, Nq = w["B"], w["Ncam"], w["Nq"]
    slots = torch.full((B, Nq, w["nH"] * 32), float("nan"), dtype=torch.float32, device="cuda")
    msda.sca_forward(value_pairs, dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                     dev(w["reference_points_cam"]), dev(w["bev_mask"]), dev(w["sampling_offsets"]),
                     dev(w["attention_logits"]), slots=slots, **kw)
    return host(slots).reshape(B * Nq, -1)


def oracle_slots(w, value, rows=None):
    return oracle.sca(value, w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"], w["bev_mask"],
                      w["sampling_offsets"], w["attention_logits"], rows=rows)["slots"]


def test_bevformer_sca_bf16_layer_in_pairs():
    """The batch-4 bf16 layer workload with the value projection written in
    pairs: the projection against the plain one re-indexed (bit for bit) and
    the slots of every query against the oracle's SCA on its own bf16
    projection, 1e-2 absolute on the unit-scale result."""
    w = W.bevformer_sca_bf16(bias=True)
    B, Ncam, Nq, Nv = w["B"], w["Ncam"], w["Nq"], w["Nv"]
    feat = w["feat"].reshape(-1, 256)
    pr = msda.msda_value_proj_pairs_bf16(dev(feat), dev(w["W_v"]), dev(w["b_v"]), Nv)
    plain = msda.msda_gemm_bf16(dev(feat), dev(w["W_v"]), dev(w["b_v"]), y_dtype=torch.bfloat16)
    plain_bits = _bits(plain).reshape(B * Ncam, Nv, 8, 32)
    assert np.array_equal(_bits(pr).reshape(B * Ncam, 8, Nv, 2, 32), pairs_host(plain_bits)), \
        "pairs projection != plain projection re-indexed"
    del plain_bits
    got = run_sca_pairs(w, pr.view(B, Ncam, 8, Nv, 2, 32))
    ref_value = oracle.round_to_bf16(oracle.linear_bf16_blas(feat, w["W_v"], w["b_v"])).reshape(B, Ncam, Nv, 8, 32)
    ref = oracle_by_rows(lambda r: oracle_slots(w, ref_value, rows=r), np.arange(B * Nq))
    assert_abs_close(got, ref, 1e-2, f"SCA on the pairs layout, all {B * Nq} queries")
    # against the plain bf16 layout on the same value: the same sums in another order
    plain_slots = host(msda.sca_forward(plain.view(B, Ncam, Nv, 8, 32), dev(w["spatial_shapes"]),
                                        dev(w["level_start_index"]), dev(w["reference_points_cam"]),
                                        dev(w["bev_mask"]), dev(w["sampling_offsets"]),
                                        dev(w["attention_logits"]))).reshape(B * Nq, -1)
    assert_fp32_close(got, plain_slots, "pairs against plain bf16 layout")


def _rand_sca(seed, B, Ncam, Nq, shapes, nH, P, D, p_mark, rho_lo=-0.1, rho_hi=1.1, off_px=2.0):
    ss, starts, Nv = W.level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    value = W.bf16_bits_trunc(g.normal(size=(B, Ncam, Nv, nH, 32)).astype(np.float32))
    return {"value": value, "spatial_shapes": ss, "level_start_index": starts,
            "reference_points_cam": g.uniform(rho_lo, rho_hi, (Ncam, B, Nq, D, 2)).astype(np.float32),
            "bev_mask": (g.random((Ncam, B, Nq, D)) < p_mark).astype(np.uint8),
            "sampling_offsets": g.normal(0, off_px, (B, Nq, nH, L, P, 2)).astype(np.float32),
            "attention_logits": g.normal(size=(B, Nq, nH, L * P)).astype(np.float32), "B": B, "Ncam": Ncam,
            "Nq": Nq, "Nv": Nv, "nH": nH, "L": L, "P": P, "D": D}


SCA_EDGE = [
    # id, seed, B, Ncam, Nq, shapes, nH, P, D, p_mark
    ("batch_masks_differ", 21, 3, 3, 50, ((6, 9), (3, 4)), 8, 4, 2, 0.3),
    ("multi_tile_ragged", 22, 2, 6, 700, ((8, 12), (4, 6)), 8, 8, 4, 0.15),
    ("one_camera", 23, 2, 1, 33, ((5, 5),), 8, 4, 4, 0.5),
    ("thirty_two_cameras", 24, 1, 32, 40, ((4, 6),), 8, 2, 1, 0.2),
    ("anchor_per_point_D1_P3", 25, 1, 4, 30, ((5, 7), (2, 3)), 8, 3, 1, 0.4),
    ("half_heads_nH4", 26, 2, 3, 45, ((6, 6),), 4, 4, 2, 0.3),
    ("two_passes_nH16", 27, 1, 3, 25, ((6, 6),), 16, 4, 4, 0.3),
    ("one_head", 34, 1, 2, 30, ((5, 6),), 1, 4, 2, 0.5),
    ("nobody_sees_anything", 28, 2, 3, 20, ((4, 4),), 8, 4, 4, 0.0),
    ("everybody_sees_everything", 29, 1, 5, 20, ((4, 4), (2, 2)), 8, 4, 4, 1.0),
    ("max_points_LP64", 30, 1, 2, 24, ((8, 8), (4, 4)), 8, 32, 8, 0.4),
    # one- and two-pixel-wide levels: nearly every x pair has a corner
    # outside, and row ends meet the next row or level in memory
    ("thin_levels", 35, 2, 3, 60, ((1, 1), (1, 3), (3, 1), (2, 2)), 8, 4, 2, 0.6),
]


@pytest.mark.parametrize("case", SCA_EDGE, ids=[c[0] for c in SCA_EDGE])
def test_sca_pairs_edge_cases(case):
    _, seed, B, Ncam, Nq, shapes, nH, P, D, pm = case
    w = _rand_sca(seed, B, Ncam, Nq, shapes, nH, P, D, pm)
    got = run_sca_pairs(w, dev(pairs_host(w["value"])))
    assert_fp32_close(got, oracle_slots(w, w["value"]), case[0])


def test_sca_pairs_border_pairs_read_no_neighbour():
    """A corner outside its level is never read, not even as the other half
    of a line: the right half of every row's last line holds the next row's
    (or level's) first pixel, which no sample may take from there.  With
    NaN in exactly those halves (and after the last pixel) the slots stay
    finite and equal the oracle's on the plain value."""
    shapes = ((4, 5), (2, 3), (1, 1))
    w = _rand_sca(36, 1, 2, 120, shapes, 8, 4, 2, 0.7, rho_lo=-0.3, rho_hi=1.3, off_px=1.5)
    ss, starts = w["spatial_shapes"], w["level_start_index"]
    pairs = pairs_host(w["value"])
    for (H, Wd), s0 in zip(ss, starts):
        row_ends = s0 + np.arange(H) * Wd + Wd - 1
        pairs[:, :, :, row_ends, 1, :] = np.uint16(0x7FC0)
    got = run_sca_pairs(w, dev(pairs))
    assert np.isfinite(got).all(), "a row end's right half was read"
    assert_fp32_close(got, oracle_slots(w, w["value"]), "border pairs")


def test_sca_pairs_stage_path_and_noalloc():
    """sca_compact + sca_gather and sca_forward_noalloc on a value in pairs
    give sca_forward's bits."""
    w = _rand_sca(37, 2, 6, 300, ((8, 12), (4, 6)), 8, 8, 4, 0.2)
    vp = dev(pairs_host(w["value"]))
    ref = run_sca_pairs(w, vp)
    args = (dev(w["spatial_shapes"]), dev(w["level_start_index"]), dev(w["reference_points_cam"]))
    ws = torch.empty(msda.sca_workspace_size(2, 6, 300), dtype=torch.uint8, device="cuda")
    msda.sca_compact(dev(w["bev_mask"]), dev(w["reference_points_cam"]), ws)
    s = msda.sca_gather(vp, *args, dev(w["sampling_offsets"]), dev(w["attention_logits"]), ws)
    assert np.array_equal(host(s).reshape(600, -1), ref), "stage path"
    out = torch.full((2, 300, 256), float("nan"), dtype=torch.float32, device="cuda")
    msda.sca_forward_noalloc(vp, *args[:2], dev(w["reference_points_cam"]), dev(w["bev_mask"]),
                             dev(w["sampling_offsets"]), dev(w["attention_logits"]), out)
    assert np.array_equal(host(out).reshape(600, -1), ref), "allocation-free entry point"
    assert_fp32_close(ref, oracle_slots(w, w["value"]), "pairs, stage test inputs")


# ---------------------------------------------------------------------------
# the operator (and its frame mean) on a value in pairs
# ---------------------------------------------------------------------------

def _bf16_value(w):
    """The workload with its value quantised to bf16 bits (the oracle reads
    those bits exactly)."""
    return {**w, "value": W.bf16_bits_trunc(w["value"])}


def run_op_pairs(w, frames=False, plan=False):
    args = (dev(pairs_host(w["value"])), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
            dev(w["sampling_locations"]), dev(w["attention_weights"]))
    if plan:
        B, Nq = w["B"], w["Nq"]
        F = w["value"].shape[1] if frames else 1
        loc = args[3]
        r = loc[0, 0, 0].numel() if frames else loc[0, 0].numel()  # one query's locations
        p = msda.msda_plan(loc, B, Nq, F * Nq * r, r)
        out = msda.msda_gather(*args, p)
    else:
        out = (msda.msda_forward_frames if frames else msda.msda_forward)(*args)
    return host(out).reshape(w["B"] * w["Nq"], -1)


def test_detr_encoder_in_pairs():
    """The DETR encoder workload on a bf16 value in pairs: every query
    against the oracle, and the planned gather bit for bit against the
    unplanned one."""
    w = _bf16_value(W.detr_encoder_msda())
    got = run_op_pairs(w)
    ref = oracle_by_rows(lambda r: oracle.msda(w["value"], w["spatial_shapes"], w["level_start_index"],
                                               w["sampling_locations"], w["attention_weights"],
                                               weights_are_logits=True, rows=r), np.arange(w["B"] * w["Nq"]))
    assert_fp32_close(got, ref, f"DETR encoder in pairs, all {w['Nq']} queries")
    assert np.array_equal(run_op_pairs(w, plan=True), got), "planned != unplanned"


def test_temporal_frames_in_pairs():
    """Two stacked BEV maps in pairs ([B,F,nH,Nv,2,32]): the frame mean of
    every query against the oracle, planned and unplanned."""
    w = _bf16_value(W.temporal_frames())
    got = run_op_pairs(w, frames=True)
    ref = oracle_by_rows(lambda r: oracle.msda_frames(w["value"], w["spatial_shapes"], w["level_start_index"],
                                                      w["sampling_locations"], w["attention_weights"], rows=r),
                         np.arange(w["B"] * w["Nq"]))
    assert_fp32_close(got, ref, "temporal frames in pairs, all queries")
    assert np.array_equal(run_op_pairs(w, frames=True, plan=True), got), "planned != unplanned"


OP_EDGE = [
    # id, seed, B, Nq, shapes, nH, P
    ("ragged_queries_nH4", 1, 2, 37, ((5, 7), (3, 2)), 4, 3),
    ("two_head_passes_nH12_odd_LP", 2, 3, 19, ((6, 4),), 12, 5),
    ("one_head_one_point", 3, 1, 9, ((4, 4),), 1, 1),
    ("max_points_LP64", 4, 1, 33, ((8, 8), (4, 4), (2, 2), (1, 1)), 8, 16),
    ("unit_levels_and_wide", 5, 2, 21, ((1, 1), (1, 40), (17, 1)), 8, 4),
    ("many_heads_nH64", 7, 1, 5, ((3, 5),), 64, 2),
]


def _rand_op(seed, B, Nq, shapes, nH, P, F=None):
    ss, starts, Nv = W.level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    lead = (B,) if F is None else (B, F)
    return {"value": W.bf16_bits_trunc(g.normal(size=lead + (Nv, nH, 32)).astype(np.float32)),
            "spatial_shapes": ss, "level_start_index": starts,
            "sampling_locations": g.uniform(-0.2, 1.2, lead + (Nq, nH, L, P, 2)).astype(np.float32),
            "attention_weights": g.normal(size=lead + (Nq, nH, L * P)).astype(np.float32), "B": B, "Nq": Nq}


@pytest.mark.parametrize("case", OP_EDGE, ids=[c[0] for c in OP_EDGE])
def test_operator_pairs_edge_cases(case):
    _, seed, B, Nq, shapes, nH, P = case
    w = _rand_op(seed, B, Nq, shapes, nH, P)
    ref = oracle.msda(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                      w["attention_weights"], weights_are_logits=True)
    assert_fp32_close(run_op_pairs(w), ref, case[0])


@pytest.mark.parametrize("F,shapes,P", [(3, ((6, 9), (3, 4)), 4), (3, ((6, 9), (3, 4)), 12)],
                         ids=["frames_in_one_pass", "frame_by_frame_FLP72"])
def test_frames_pairs_both_staging_paths(F, shapes, P):
    """F * L * P <= 64 stages all frames at once; 72 goes frame by frame."""
    w = _rand_op(40 + P, 2, 50, shapes, 8, P, F=F)
    ref = oracle.msda_frames(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                             w["attention_weights"])
    assert_fp32_close(run_op_pairs(w, frames=True), ref, f"frames in pairs, F={F}, P={P}")


def test_operator_pairs_row_ends_never_read():
    """As for the SCA: NaN in every row end's right half never reaches a
    result of the operator."""
    w = _rand_op(45, 2, 120, ((4, 5), (2, 3), (1, 1)), 8, 4)
    pairs = pairs_host(w["value"])
    for (H, Wd), s0 in zip(w["spatial_shapes"], w["level_start_index"]):
        row_ends = s0 + np.arange(H) * Wd + Wd - 1
        pairs[:, :, row_ends, 1, :] = np.uint16(0x7FC0)
    out = host(msda.msda_forward(dev(pairs), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                                 dev(w["sampling_locations"]), dev(w["attention_weights"]))).reshape(240, -1)
    assert np.isfinite(out).all(), "a row end's right half was read"
    ref = oracle.msda(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                      w["attention_weights"], weights_are_logits=True)
    assert_fp32_close(out, ref, "operator border pairs")
